// mk_layout.h -- device-side layout of one loaded model: shared by the host code that
// builds the arena and by the persistent kernels that read it.
//
// Work mapping of the persistent grid on MI355X: 256 workgroups, one per compute
// unit, 512 threads (8 wave64) each, so every XCD hosts exactly 32 of them.  The
// dispatcher places them round-robin over the 8 XCDs from a starting XCD that can
// differ between launches; a workgroup reads its XCD x from the hardware and is
// workgroup x + 8 * (blockIdx.x / 8) of the grid's partition.  Each XCD ("group" x) owns one DeltaNet head / one query head and one
// slice of the FFN intermediate dimension, so most hand-offs stay inside one XCD
// and go through its L2; only the residual-stream reductions cross XCDs.  Inside an
// XCD, workgroups b >> 3 < MK_NG run the token mixers and the others the FFNs.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MK_NX 8                      // XCDs = head groups
#define MK_NL 32                     // workgroups per XCD
#define MK_NG 16                     // workgroups per XCD in each of the two roles (token mixer, FFN)
#define MK_NWG (MK_NX * MK_NL)       // persistent grid size
#define MK_THREADS 512               // threads per workgroup
#define MK_WAVES (MK_THREADS / 64)   // wave64 per workgroup
#define MK_MAXCOL 5                  // tokens per verify forward
#define MK_PAGE 64                   // KV-cache page (tokens)
#define MK_RING 8                    // conv history ring (positions), >= conv_k - 1 + MK_MAXCOL
#define MK_KBLK 32                   // keys per attention block in decode
#define MK_LDS_BYTES (96 * 1024)     // dynamic LDS per workgroup (also forces 1 workgroup per CU)

// control words (int32) at the start of the control block
enum {
  MK_CTL_POS = 0,      // tokens held by the state
  MK_CTL_PEND = 1,     // pending DeltaNet updates to apply before the next use of S
  MK_CTL_PAR = 2,      // which pending buffer holds them
  MK_CTL_ERR = 3,      // device error bits (MK_DERR_*)
  MK_CTL_WHERE = 4,    // first watchdog expiry: site (step<<16 | layer<<8 | phase), block<<16|thread, seen tag, wanted tag
  MK_CTL_WORDS = 16
};
enum { MK_DERR_HANG = 1, MK_DERR_TOKEN = 2, MK_DERR_NAN = 4, MK_DERR_XCD = 8 };

// A tile-format matrix [rows][K] (bf16): row groups of 64/G rows; within a group,
// load i of lane l (16 bytes) holds row (l / G), elements [(i*G + l%G)*8, +8).
// Memory order is (group, i, lane), so every wave load is 1 KiB contiguous.
// G is the largest power of two <= 64 dividing K/8; L = K/8/G loads per lane.
struct MkTile {
  const uint16_t *w;
  int32_t rows, K, G, L;
};

// Pending delta-rule updates of a verify forward, per (parity, head, column): the key as 64 lane
// quads (k[l], k[64 + l], 0, 0) (MK_PEND_K floats; dk <= 128), then one quad per value row
// (v_r, alpha, beta, 0).  Every part is a 16-byte load per lane for the kernels that replay them.
#define MK_PEND_K 256
__host__ __device__ static inline int mk_pend_stride(int dv) { return MK_PEND_K + 4 * dv; }

struct MkLayerDev {
  int32_t kind;                       // 0 DeltaNet, 1 attention
  int32_t idx;                        // index among layers of the same kind
  const float *ln1, *ln2;             // RMSNorm gains [H]
  // DeltaNet
  const uint16_t *dn_in;              // [nh] tiles [r_in][H]: rows q(dk) k(dk) v(dv) z(dv) a b
  const float *dn_conv;               // [C][4]
  const float *dn_gnorm;              // [dv]
  const uint16_t *dn_out;             // [nh] tiles [H][dv]   (columns of head h of W_out)
  float *S;                           // [nh][dv][dk]
  float *ring;                        // [MK_RING][C] pre-conv inputs by position % MK_RING
  float *pend;                        // [2][nh][MK_MAXCOL][mk_pend_stride(dv)] pending updates (layout below)
  // attention
  const uint16_t *at_q;               // [nq] tiles [hd][H]
  const uint16_t *at_k, *at_v;        // [nkv] tiles [hd][H]
  const uint16_t *at_o;               // [nq] tiles [H][hd]   (columns of head i of W_o)
  void *kc, *vc;                      // [pages][nkv][MK_PAGE][hd] bf16, or int8 codes with kv_quant
  int8_t *kve;                        // kv_quant: [pages][nkv][MK_PAGE][2] exponents e of the K, V row
  // FFN (XCD x owns intermediate rows [x*J, (x+1)*J))
  const uint16_t *ffn_gu;             // [8] tiles [2J][H]: rows g_j, u_j interleaved
  const uint16_t *ffn_dn;             // [8] tiles [H][J]
};

// Tagged exchange slots (uint2 {float bits, tag}) of one launch with n columns: per layer, in this
// order,
//   x_in  [8][n][r_in_max]   XCD-local (in-projection / QKV rows)
//   x_o   [8][n][x_o_len]    XCD-local (DeltaNet o and o g silu(z) rows / attention partials)
//   x_mix [n][8][H]          grid      (mixer split-K partials)
//   x_r1  [8][n][H]          XCD-local (residual after the mixer)
//   x_m   [8][n][xm_len]     XCD-local (SwiGLU activations)
//   x_ffn [n][8][H]          grid      (down-projection partials)
//   x_r2  [8][n][H]          XCD-local (residual after the FFN)
// then, after the last layer, the argmax candidates: uint4 {value, index, tag, nan} [n][256].
// Every length is a multiple of 32 slots, so with a 256-byte aligned base no 256-byte block holds
// two XCDs' slots.  The layout depends on n: decode (n = 1) and verify (n = 5) launches place the
// same value at different slots, which is harmless because every launch has tags of its own.
__host__ __device__ static inline size_t mk_xch_layer_slots(int n, int H, int r_in_max, int x_o_len, int xm_len) {
  return (size_t)n * 8 * (size_t)(r_in_max + x_o_len + xm_len + 4 * H);
}
__host__ __device__ static inline size_t mk_xch_bytes(int n, int n_layers, int H, int r_in_max, int x_o_len, int xm_len) {
  return (size_t)n_layers * mk_xch_layer_slots(n, H, r_in_max, x_o_len, xm_len) * 8 + (size_t)n * MK_NWG * 16;
}

struct MkDev {
  int32_t n_layers, H, V, I, J;
  int32_t nh, dk, dv, C, r_in;        // r_in = 2dk + 2dv + 2
  int32_t nq, nkv, hd;
  int32_t r_in_max, x_o_len, xm_len;  // exchange row lengths (slots), multiples of 32: 256-byte blocks
  int32_t max_ctx, max_pages;
  int32_t kv_quant;                   // 0: bf16 cache; 1: int8 codes q, row value q * 2^e (e per row)
  float rms_eps, l2_eps;
  const uint16_t *embed;              // [V][H] (tile format with L == 1 or G == 64: row-major)
  const float *lnf;                   // [H]
  const float *rope;                  // [max_ctx][hd/2][2] cos, sin
  const int32_t *page_table;          // [max_pages] logical -> physical page
  const MkLayerDev *layers;           // [n_layers]
  int32_t *ctl;                       // [MK_CTL_WORDS]
};

// Arguments of one persistent-kernel launch.
struct MkLaunch {
  MkDev m;
  const int32_t *tokens;  // device: [n]
  int32_t n;              // columns: 1 (decode) or 2..MK_MAXCOL (verify)
  uint32_t tag0;          // exchange tag of the first forward pass of this launch
  int32_t *argmax;        // device: [n]
  float *logits;          // device, nullable: [n][V]
  int32_t *n_acc;         // device, nullable
  uint2 *xch;             // device: exchange slots of this launch (mk_xch_bytes(n_template, ...) bytes, 256-byte aligned)
  // batch launches (MK_BATCH): column c is one decode step of its own sequence, whose state
  // (DeltaNet S, conv ring, KV cache) the layer table seq_layers[c] points at and whose position
  // is seq_ctl[c][MK_CTL_POS]; m.layers / m.ctl are those of column 0's sequence
  const MkLayerDev *seq_layers[MK_MAXCOL];
  int32_t *seq_ctl[MK_MAXCOL];
};

// Instantiations of the persistent kernel: MK_SHAPE_H1024 has every dimension of the hidden-1024
// model as a compile-time constant; MK_SHAPE_ANY reads them from MkDev.  MK_KV_Q8 is or-ed in for
// a model whose KV cache holds 8-bit codes, MK_BATCH for a batch launch (MK_MAXCOL columns, one
// sequence each; bf16 cache).
enum { MK_SHAPE_ANY = 0, MK_SHAPE_H1024 = 1, MK_KV_Q8 = 2, MK_N_VARIANTS = 4, MK_BATCH = 4 };
static inline int mk_shape_of(const MkDev &d) {
  const bool h1024 = d.H == 1024 && d.nh == 8 && d.dk == 128 && d.dv == 128 && d.nq == 8 && d.nkv == 2 &&
                     d.hd == 128 && d.J == 448 && d.r_in == 514 && d.C == 3072 && d.r_in_max == 544 &&
                     d.x_o_len == 2080 && d.xm_len == 448;
  return h1024 ? MK_SHAPE_H1024 : MK_SHAPE_ANY;
}
static inline int mk_variant_of(const MkDev &d) { return mk_shape_of(d) | (d.kv_quant ? MK_KV_Q8 : 0); }

// 8-bit KV cache row: the exponent e of a row whose largest magnitude is a (FP32): the smallest
// integer with a <= 127 * 2^e, but at least -126 (every nonzero q * 2^e is then a normal number).
// The codes are round-half-even(x * 2^-e) in [-127, 127].
__host__ __device__ static inline int mk_q8_exp(float a) {
  union { float f; uint32_t u; } c;
  c.f = a;
  const int e = (int)(c.u >> 23) - 133 + ((c.u & 0x7fffffu) > 0x7e0000u ? 1 : 0);
  return e < -126 ? -126 : e;
}

__host__ __device__ static inline int mk_tile_G(int K) {
  int c = K / 8, g = 64;
  while (g > 1 && (c % g) != 0) g >>= 1;
  return g;
}

// ------------------------------------------------------------------------------ chunked prefill
// A prompt is processed in passes of up to MK_PT tokens by a stream-ordered sequence of
// kernels (projections as MFMA GEMMs, the delta rule in chunks of MK_CHUNK tokens).  Scratch
// for one pass lives in the arena.
#define MK_PT 1024                   // tokens per prefill pass (multiple of MK_CHUNK)
#define MK_CHUNK 64                  // delta-rule chunk

// Prefill copies of one layer's projection weights, each a matrix [N][K] in the GEMM operand
// block layout (1 KiB blocks of 16 rows x 32 k; rows padded with zeros to a multiple of 16), read
// only by the prefill GEMMs so that every weight block they load is 1 KiB of contiguous memory.
struct MkPfW {
  const uint16_t *in;                 // DeltaNet in-projection, rows of head h: q k v z a b  [nh r_in][H]
  const uint16_t *out;                // DeltaNet out-projection [H][nh dv]
  const uint16_t *qkv;                // attention q | k | v [(nq + 2 nkv) hd][H]
  const uint16_t *o;                  // attention o-projection [H][nq hd]
  const uint16_t *gu;                 // FFN gate and up rows interleaved (g_i row 2 i, u_i row 2 i + 1) [2 I][H]
  const uint16_t *dn;                 // FFN down-projection [H][I]
};

struct MkPf {
  float *X;                           // [PT][H] residual stream (FP32)
  uint16_t *a1h, *a1l;                // [PT][K1] GEMM operand as bf16 hi + lo, K1 = max(H, nh dv, nq hd)
  uint16_t *a2h, *a2l;                // [PT][I]  SwiGLU activations as bf16 hi + lo
  float *P;                           // [PT][NP] projection outputs, NP = max(nh r_in, (nq + 2 nkv) hd)
  float *cW, *cQ, *cU, *cO;           // [nh][PT/CHUNK][CHUNK][dk|dv] chunk terms W, Q~, U', O' of the delta rule
  float *cKt;                         // [nh][PT/CHUNK][dk][CHUNK] the chunk's keys, transposed
  float *cg, *cd;                     // [nh][PT/CHUNK][CHUNK] exp(G_i), exp(G_last - G_i)
  float *snap;                        // [nh][PT/CHUNK][dv][dk] delta-rule state entering each chunk
  float *aq;                          // [PT][nq hd] queries after RoPE
  unsigned long long *lmbest;         // [MK_NWG] packed (ordered value, ~index) candidates
  float *part;                        // [4][PT][H] split-K partial sums
  int32_t K1, NP;
};
