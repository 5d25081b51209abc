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
 * 1 <= max_verify <= 5; tied_embedding == 1; kv_quant in {0, 1}; 0 <= n_seq <= 5.
 *
 * kv_quant selects the KV-cache format (the launch page of the 8-bit cache: "8-bit KV cache"
 * limits of the Korean write-up, and the RTX 3090 tag page).  0: rows stored as bf16.  1: every
 * cached row (one position, one KV head, K or V) stored as hd int8 codes q plus one int8 exponent
 * e, standing for q * 2^e: e is the smallest integer with max|x| <= 127 * 2^e (at least -126),
 * q = round-half-even(x * 2^-e).  Each q * 2^e is exactly a bf16 number, so the attention
 * arithmetic after the cache is the same in both formats; the cache takes half the bytes.      */
typedef struct mk_config {
  int32_t n_layers;
  const uint8_t *layer_kind; /* host array [n_layers] of MK_LAYER_*                  */
  int32_t hidden, vocab, ffn;
  int32_t dn_heads, dn_dk, dn_dv, conv_k;
  int32_t at_q_heads, at_kv_heads, at_head_dim;
  float rope_theta, rms_eps, l2_eps;
  int32_t tied_embedding, max_ctx, prefill_chunk, max_verify;
  int32_t kv_quant;          /* 0: bf16 KV cache; 1: 8-bit codes with a power-of-two scale per row */
  int32_t n_seq;             /* sequences held at once, 1..5 (0 means 1); see mk_decode_batch     */
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
  const void *data; /* only read during mk_load_weights                            */
  int32_t on_device; /* 0: data is host memory; 1: device memory of the current device
                        (copied to the host for re-tiling, after the stream is synchronised) */
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

/* Clear the recurrent state of every sequence: DeltaNet states and conv history to
 * zero, KV length and position to zero, pending verify updates dropped, device error
 * words cleared.  The selected sequence stays selected.                            */
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

/* Row blocks of a prefill pass (launch page "OS Megakernel that match M5 Max Tok/w at 2x the
 * Throughput on RTX 3090": one prompt, every layer, no host round trip).  max_blocks 2 (the
 * default): a pass of at least 256 tokens is split at a 64-token boundary near its middle and
 * the second block's kernels run on a side stream of the model (created on the first prefill,
 * default priority, destroyed by mk_free), one step behind the first block: its layer waits only
 * for the first block's state of that layer (delta-rule state and conv history, or keys and
 * values), so the two blocks' kernels overlap.  The side stream starts after everything enqueued
 * on `stream` before the call, and `stream` continues only after the side stream's last kernel,
 * so ordering for the caller is that of one stream.  Results are bit-identical to max_blocks 1
 * (one block on `stream`).  Returns MK_EINVAL for other values, MK_ESTATE for a freed model.  */
int mk_set_prefill_blocks(mk_model *m, int32_t max_blocks);

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

/* Size of the static exchange-slot array of mk_decode_step_static (one per device).        */
enum { MK_STATIC_SCRATCH_BYTES = 16 << 20 };

/* mk_decode_step for callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation.  Same
 * arguments, results and errors as mk_decode_step, but the launch's exchange slots (the
 * tagged partial results the workgroups hand each other) live in a static device array of
 * MK_STATIC_SCRATCH_BYTES per device, held until the process ends, instead of the model's
 * arena.  The slots of one launch take n_layers * n * 8 * (r_in_max + x_o_len + xm_len +
 * 4 * hidden) * 8 + n * 4096 bytes, with n = 1 for a decode step and n = 5 for a verify
 * forward (r_in_max, x_o_len, xm_len: the exchange row lengths, for the 24-layer hidden-1024
 * model 544, 4160 and 448, so a decode step needs 14.2 MiB); a call whose slots do not fit is
 * rejected with MK_EINVAL before anything is enqueued.  Calls no allocating routine.  All
 * calls on one device share the array: calls that overlap in time on one device (any models,
 * streams or threads) race and their results are undefined; calls ordered one after another
 * are independent (each launch tags its slots with a device-wide sequence number, so nothing
 * needs clearing between calls).                                                          */
int mk_decode_step_static(mk_model *m, const int32_t *d_tokens, int32_t n_tokens, int32_t *d_argmax,
                          float *d_logits, int32_t *d_n_accepted, void *stream);

/* Sequences.  A model holds mk_config.n_seq sequences, each with its own DeltaNet states, conv
 * history, KV cache, position and error word; the weights are shared.  mk_prefill, mk_decode_step,
 * mk_decode_step_static, mk_generate_lookup, mk_sync_status (position) act on the selected
 * sequence, 0 after loading.  mk_select_seq changes it (host-side only, nothing is enqueued); it
 * fails with MK_EINVAL for seq outside [0, n_seq).  All sequences of a model share its prefill
 * scratch and exchange slots: calls on one model, whatever the sequence, are ordered on one stream. */
int mk_select_seq(mk_model *m, int32_t seq);

/* Batch decode (B sequences share one weight pass; concurrency section of the RTX 3090 tag page's
 * Dflash2 item): one greedy decode step for each of the n distinct sequences seqs[0..n) (host
 * array, 1 <= n <= n_seq), in one launch.  d_tokens[c] (device int32) is the last token of
 * sequence seqs[c]; the greedy next token goes to d_argmax[c] and, if d_logits is not NULL, the
 * logits to d_logits[c][vocab].  Each sequence's results equal those of mk_decode_step on that
 * sequence alone, bit for bit; each position advances by one.  Rejected with MK_EINVAL (before
 * anything is enqueued) for a bad or repeated sequence index, a model with kv_quant = 1, or a
 * sequence whose last forward was a verify (a decode step or prefill on it applies its pending
 * updates first); MK_ECTX if a sequence is at max_ctx.  Device errors are reported by the next
 * mk_sync_status.                                                                            */
int mk_decode_batch(mk_model *m, const int32_t *seqs, int32_t n, const int32_t *d_tokens, int32_t *d_argmax,
                    float *d_logits, void *stream);

/* Weight-free draft tokens for speculative decoding ("lookup-augmented draft" on the RTX 3090 tag
 * page; several drafts checked per weight pass with greedy output unchanged, speed section of the
 * Korean update page): the longest suffix of history[0..n_history) of length g, for g from ngram_max
 * down to ngram_min, that also occurs earlier in the history; at its most recent earlier occurrence
 * the tokens that followed it (at most max_draft, fewer where the history ends) are copied to
 * out_draft.  Returns the number of draft tokens (0 when no such suffix recurs), or MK_EINVAL
 * (NULL pointer with a non-empty request, 1 <= ngram_min <= ngram_max violated, max_draft < 0).
 * Host memory only; no model or GPU involved.                                                     */
int mk_lookup_draft(const int32_t *history, int32_t n_history, int32_t ngram_min, int32_t ngram_max,
                    int32_t max_draft, int32_t *out_draft);

/* Counters of one mk_generate_lookup call.                                                         */
typedef struct mk_lookup_stats {
  int32_t forwards;   /* launches (decode steps and verify forwards)                              */
  int32_t drafted;    /* draft tokens sent to verify forwards                                     */
  int32_t accepted;   /* draft tokens accepted (committed without a launch of their own)          */
} mk_lookup_stats;

/* Greedy generation driven by lookup drafts.  The state holds history[0..n_history) (host; the
 * prompt and whatever was appended since) and last_token is the greedy token after it (as
 * mk_prefill or the last decode step returned it, not yet appended).  Generates n_generate tokens
 * into out_tokens[0..n_generate) (host): each launch takes last_token plus the drafts
 * mk_lookup_draft finds in history + generated tokens (at most max_verify - 1, and never more than
 * the tokens still to generate), as a verify forward, or as a decode step when there are none;
 * the accepted drafts and the greedy token after them are committed.  The result equals
 * n_generate chained mk_decode_step calls token for token (verify is bit-identical to decode), in
 * fewer launches when drafts are accepted.  The state is left after last_token and
 * out_tokens[0..n_generate - 1), with out_tokens[n_generate - 1] the next last_token.  stats may
 * be NULL.  Synchronises `stream` after every launch (the next drafts depend on the accepted
 * tokens); device-side errors (MK_EHANG, MK_ETOKEN, MK_ENAN) end the call with that status and the
 * tokens generated so far.  Its small device buffers live in the model's arena.                   */
int mk_generate_lookup(mk_model *m, const int32_t *history, int32_t n_history, int32_t last_token,
                       int32_t n_generate, int32_t ngram_min, int32_t ngram_max, int32_t *out_tokens,
                       mk_lookup_stats *stats, void *stream);

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
