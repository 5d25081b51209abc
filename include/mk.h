/*
 * mk.h -- C ABI of the persistent-kernel forward pass of a hybrid Gated-DeltaNet +
 * full-attention decoder on AMD Instinct MI355X (gfx950).
 *
 * What the library computes follows the launch page "OS Megakernel that match M5
 * Max Tok/w at 2x the Throughput on RTX 3090":
 *   - section "Why nobody had done this yet?": a decoder whose layers alternate
 *     DeltaNet layers (linear attention with a learned recurrence) and full
 *     attention layers;
 *   - section "We wrote a single CUDA kernel that runs the entire forward pass in
 *     one dispatch": one launch per forward pass, BF16 weights with FP32
 *     accumulation, the recurrence held in FP32, attention fused from the QKV
 *     projection through RoPE and causal softmax to the output projection, and a
 *     grid-wide synchronisation in place of per-op launches;
 *   - section "Results on the same RTX 3090": the workload is a prompt (pp)
 *     followed by one-token greedy decode steps (tg), with no host round trip
 *     between layers.
 * A verify call that runs several tokens in one forward and keeps only the
 * accepted prefix follows the speculative-decoding description on the page
 * "업데이트: 단일 RTX 3090에서 Qwen 3.8 27B를 140 tok/s로 구동" (greedy output equals the
 * main model's greedy choice; several draft tokens are checked per pass).  Its
 * loader rule, that every tensor's type is checked, is the error convention of
 * mk_load_weights.
 *
 * Conventions
 *   - Every function returns an int status: MK_OK (0) or a negative MK_E* code.
 *     Nothing aborts and no C++ exception crosses this boundary.
 *   - Argument validation happens before anything is enqueued, so a rejected call
 *     leaves the model and the stream untouched.
 *   - Pointers named d_* are device pointers (HIP device memory on the device that
 *     was current at mk_load_weights); all other pointers are host pointers.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     device work of a call is enqueued on that stream and is asynchronous unless
 *     stated otherwise; a call returns once its work is enqueued.
 *   - A model is not thread-safe; calls on one model must be serialised by the
 *     caller, and every call of one model must use streams of one device.
 *   - The caller owns every device buffer, including the arena.  The library
 *     never allocates device memory: it lays its weights, state and scratch out
 *     inside the caller's arena.
 */
#ifndef MK_H_
#define MK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status codes */
enum {
  MK_OK = 0,
  MK_EINVAL = -1,  /* null pointer, bad config value, n_tokens out of range, bad arena  */
  MK_EDTYPE = -2,  /* a weight tensor is not BF16                                        */
  MK_ESHAPE = -3,  /* a weight tensor is missing, duplicated, unknown or mis-shaped      */
  MK_ECTX = -4,    /* position + n_tokens would exceed max_ctx                           */
  MK_ESTATE = -5,  /* call on a model that was not loaded (or was freed)                 */
  MK_ELAUNCH = -6, /* the device cannot host the persistent grid (wrong GPU, occupancy)  */
  MK_EHIP = -7,    /* a HIP runtime call failed; mk_last_error() has the HIP message     */
  MK_EHANG = -8,   /* a device-side wait timed out (watchdog); results of that call void */
  MK_ETOKEN = -9,  /* a device token id was outside [0, vocab)                           */
  MK_ENAN = -10    /* non-finite logits met by the greedy argmax                         */
};

enum { MK_LAYER_DELTANET = 0, MK_LAYER_ATTENTION = 1 };
enum { MK_DTYPE_BF16 = 1, MK_DTYPE_F16 = 2, MK_DTYPE_F32 = 3 };

/* ---------------------------------------------------------------- model config
 * Shapes of the decoder.  The supported family (checked by every call that takes
 * a config): hidden % 256 == 0; dn_dk == dn_dv in {64, 128}; dn_heads <= 8;
 * conv_k == 4; at_head_dim in {64, 128}; at_q_heads <= 8 and a multiple of
 * at_kv_heads; ffn % 64 == 0; max_ctx a multiple of 64; prefill_chunk == 64;
 * 1 <= max_verify <= 5; tied_embedding == 1.                                      */
typedef struct mk_config {
  int32_t n_layers;
  const uint8_t *layer_kind; /* host array [n_layers] of MK_LAYER_*                  */
  int32_t hidden, vocab, ffn;
  int32_t dn_heads, dn_dk, dn_dv, conv_k;
  int32_t at_q_heads, at_kv_heads, at_head_dim;
  float rope_theta, rms_eps, l2_eps;
  int32_t tied_embedding, max_ctx, prefill_chunk, max_verify;
} mk_config;

/* One weight tensor in host memory.  Names and shapes ([out, in] for matrices):
 *   embed [vocab, hidden]; lnf [hidden]
 *   layers.{i}.ln1 [hidden], layers.{i}.ln2 [hidden]
 *   DeltaNet layer i: layers.{i}.dn.wq / .wk [dn_heads*dn_dk, hidden],
 *     .wv / .wz [dn_heads*dn_dv, hidden], .wa / .wb [dn_heads, hidden],
 *     .conv [2*dn_heads*dn_dk + dn_heads*dn_dv, conv_k], .gnorm [dn_dv],
 *     .wo [hidden, dn_heads*dn_dv]
 *   attention layer i: layers.{i}.attn.wq [at_q_heads*at_head_dim, hidden],
 *     .wk / .wv [at_kv_heads*at_head_dim, hidden], .wo [hidden, at_q_heads*at_head_dim]
 *   every layer: layers.{i}.ffn.wg / .wu [ffn, hidden], .wd [hidden, ffn]
 * All must be MK_DTYPE_BF16, row-major and contiguous.                             */
typedef struct mk_tensor {
  const char *name;
  int32_t dtype;
  int32_t ndim;
  int64_t shape[4];
  const void *data; /* host pointer; only read during mk_load_weights             */
} mk_tensor;

typedef struct mk_model mk_model; /* opaque */

/* Size in bytes of the device arena mk_load_weights needs for `cfg`.              */
int mk_required_bytes(const mk_config *cfg, size_t *arena_bytes);

/* Validate cfg and every tensor (type first, then shape), lay weights, recurrent
 * state, KV cache and scratch out in the caller's arena (d_arena, 256-byte
 * aligned, at least mk_required_bytes), copy and re-tile the weights, clear the
 * state, and return a new model in *out.  The stream is synchronised before
 * returning, so the host tensors may be freed afterwards.  The arena must stay
 * allocated until mk_free.                                                        */
int mk_load_weights(const mk_config *cfg, const mk_tensor *tensors, int32_t n_tensors,
                    void *d_arena, size_t arena_bytes, void *stream, mk_model **out);

/* Clear the recurrent state: DeltaNet states and conv history to zero, KV length
 * and position to zero, pending verify updates dropped, device error word cleared. */
int mk_reset_state(mk_model *m, void *stream);

/* Prefill: append d_tokens[0..n_tokens) (device int32) at the current position,
 * leave the state ready for decode, write the greedy token after the last prompt
 * token to d_next_token[0] (device int32) and, if d_last_logits is not NULL, that
 * position's logits to d_last_logits[0..vocab) (device float).  The prompt runs in
 * passes of up to 1024 tokens, each a stream-ordered sequence of kernels (MFMA
 * projections, the delta rule in chunks of 64); nothing returns to the host
 * between them.  Pending verify updates are applied first.                        */
int mk_prefill(mk_model *m, const int32_t *d_tokens, int32_t n_tokens, int32_t *d_next_token,
               float *d_last_logits, void *stream);

/* Decode step (n_tokens == 1) or verify forward (2 <= n_tokens <= max_verify), one
 * launch.  d_tokens[0] is the last accepted token; for verify d_tokens[1..] are
 * draft tokens.  Writes the greedy token after each position to d_argmax[0..n)
 * and, if d_logits is not NULL, the logits to d_logits[n][vocab].  For verify,
 * n_accepted = 1 + the length of the longest draft prefix that equals the greedy
 * choices is written to d_n_accepted[0] (if not NULL), and the state is left after
 * exactly the accepted tokens, so the next call starts from d_argmax[n_accepted-1].
 * d_tokens may alias the previous call's d_argmax (greedy decode then chains on
 * the device with no host round trip).                                            */
int mk_decode_step(mk_model *m, const int32_t *d_tokens, int32_t n_tokens, int32_t *d_argmax,
                   float *d_logits, int32_t *d_n_accepted, void *stream);

/* Synchronise `stream`, then report the device-side status of the work done so
 * far (MK_OK, MK_EHANG, MK_ETOKEN or MK_ENAN) and, if pos is not NULL, the number
 * of tokens the state holds.  A device error stays set until mk_reset_state.      */
int mk_sync_status(mk_model *m, void *stream, int32_t *pos);

/* Release the host-side model object (the arena stays the caller's).             */
void mk_free(mk_model *m);

/* Static description of a status code.                                            */
const char *mk_status_string(int status);

/* Message of the last failing call on this thread (HIP error text or the
 * validation failure), valid until the next call on this thread.                 */
const char *mk_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MK_H_ */
