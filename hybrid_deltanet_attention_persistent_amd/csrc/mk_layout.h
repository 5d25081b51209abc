// mk_layout.h -- device-side layout of one loaded model: shared by the host code that
// builds the arena and by the persistent kernels that read it.
//
// Work mapping of the persistent grid on MI355X: 256 workgroups, one per compute
// unit, 512 threads (8 wave64) each.  Workgroup b runs on XCD b % 8 (the hardware
// dispatches workgroups to the 8 XCDs round-robin; the kernel checks this at
// start).  Each XCD ("group" x) owns one DeltaNet head / one query head and one
// slice of the FFN intermediate dimension, so most hand-offs stay inside one XCD
// and go through its L2; only the residual-stream reductions cross XCDs.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MK_NX 8                      // XCDs = head groups
#define MK_NL 32                     // workgroups per XCD
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
  float *pend;                        // [2][nh][MK_MAXCOL][dk + dv + 2]: k | v | alpha beta
  // attention
  const uint16_t *at_q;               // [nq] tiles [hd][H]
  const uint16_t *at_k, *at_v;        // [nkv] tiles [hd][H]
  const uint16_t *at_o;               // [nq] tiles [H][hd]   (columns of head i of W_o)
  uint16_t *kc, *vc;                  // [pages][nkv][MK_PAGE][hd] bf16
  // FFN (XCD x owns intermediate rows [x*J, (x+1)*J))
  const uint16_t *ffn_gu;             // [8] tiles [2J][H]: rows g_j, u_j interleaved
  const uint16_t *ffn_dn;             // [8] tiles [H][J]
  // tagged exchange buffers: uint2 {float bits, tag}
  uint2 *x_in;                        // [8][MAXCOL][r_in_max]   XCD-local
  uint2 *x_o;                         // [8][MAXCOL][x_o_len]    XCD-local (o rows / attention partials)
  uint2 *x_mix;                       // [MAXCOL][8][H]          grid (mixer split-K partials)
  uint2 *x_r1;                        // [8][MAXCOL][H]          XCD-local (residual after mixer)
  uint2 *x_m;                         // [8][MAXCOL][J]          XCD-local (SwiGLU activations)
  uint2 *x_ffn;                       // [MAXCOL][8][H]          grid (down-projection partials)
  uint2 *x_r2;                        // [8][MAXCOL][H]          XCD-local (residual after FFN)
};

struct MkDev {
  int32_t n_layers, H, V, I, J;
  int32_t nh, dk, dv, C, r_in;        // r_in = 2dk + 2dv + 2
  int32_t nq, nkv, hd;
  int32_t r_in_max, x_o_len, xm_len;  // exchange row lengths (slots), multiples of 32: 256-byte blocks
  int32_t max_ctx, max_pages;
  float rms_eps, l2_eps;
  const uint16_t *embed;              // [V][H] (tile format with L == 1 or G == 64: row-major)
  const float *lnf;                   // [H]
  const float *rope;                  // [max_ctx][hd/2][2] cos, sin
  const int32_t *page_table;          // [max_pages] logical -> physical page
  const MkLayerDev *layers;           // [n_layers]
  int32_t *ctl;                       // [MK_CTL_WORDS]
  uint4 *x_arg;                       // [MAXCOL][256] {value, index, tag, 0}  grid
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
};

// Instantiations of the persistent kernel: MK_SHAPE_H1024 has every dimension of the hidden-1024
// model as a compile-time constant; MK_SHAPE_ANY reads them from MkDev.
enum { MK_SHAPE_ANY = 0, MK_SHAPE_H1024 = 1 };
static inline int mk_shape_of(const MkDev &d) {
  const bool h1024 = d.H == 1024 && d.nh == 8 && d.dk == 128 && d.dv == 128 && d.nq == 8 && d.nkv == 2 &&
                     d.hd == 128 && d.J == 448 && d.r_in == 514 && d.C == 3072 && d.r_in_max == 544 &&
                     d.x_o_len == 4160 && d.xm_len == 448;
  return h1024 ? MK_SHAPE_H1024 : MK_SHAPE_ANY;
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

struct MkPf {
  float *X;                           // [PT][H] residual stream (FP32)
  uint16_t *a1h, *a1l;                // [PT][K1] GEMM operand as bf16 hi + lo, K1 = max(H, nh dv, nq hd)
  uint16_t *a2h, *a2l;                // [PT][I]  SwiGLU activations as bf16 hi + lo
  float *P;                           // [PT][NP] projection outputs, NP = max(nh r_in, (nq + 2 nkv) hd)
  float *cW, *cQ, *cU, *cO;           // [nh][PT/CHUNK][CHUNK][dk|dv] chunk terms W, Q~, U', O' of the delta rule
  float *cKt;                         // [nh][PT/CHUNK][dk][CHUNK] the chunk's keys, transposed
  float *cg, *cd;                     // [nh][PT/CHUNK][CHUNK] exp(G_i), exp(G_last - G_i)
  float *o;                           // [PT][nh dv] delta-rule output
  float *aq;                          // [PT][nq hd] queries after RoPE
  unsigned long long *lmbest;         // [MK_NWG] packed (ordered value, ~index) candidates
  float *part;                        // [4][PT][H] split-K partial sums
  int32_t K1, NP;
};
