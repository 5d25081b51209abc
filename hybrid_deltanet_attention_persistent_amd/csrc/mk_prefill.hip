// mk_prefill.hip -- chunked prefill of the hybrid Gated-DeltaNet + attention decoder on
// MI355X (gfx950).
//
// A prompt is processed in passes of up to MK_PT tokens.  Each pass is a stream-ordered
// sequence of kernels per layer (launch page "OS Megakernel that match M5 Max Tok/w at 2x the
// Throughput on RTX 3090", section "We wrote a single CUDA kernel ...": prefill turns the
// projections into dense products over all prompt rows):
//
//   RMSNorm -> MFMA GEMM (in-projection / QKV) -> chunked delta rule (per chunk and head in
//   parallel: conv + SiLU + L2 norm + gates and every term that does not depend on the state;
//   then one sequential scan over the chunks per block of state rows) -> gated RMSNorm ->
//   MFMA GEMM (out-projection, + residual) -> RMSNorm -> MFMA GEMM (gate/up, SwiGLU epilogue)
//   -> MFMA GEMM (down, + residual)
//
// and for attention layers RoPE + KV append and causal attention over the cache.
//
// Precision.  Weights are BF16 and activations FP32 (the contract of the decode kernel).  A
// GEMM operand a (FP32) enters the bf16 MFMA as two terms, hi = bf16(a) and lo = bf16(a - hi),
// both multiplied by the exact bf16 weight and accumulated in FP32: the operand keeps 16
// significant bits (relative error below 2^-17).  Attention multiplies on the matrix cores the
// same way (Q and the softmax weights as hi + lo, K and V exactly bf16), softmax in FP32.  The
// delta rule runs in full FP32: its products on the FP32 matrix cores (v_mfma_f32_16x16x4f32),
// conv and norms on the vector ALUs.
//
// The chunked delta rule follows from unrolling the recurrence S_i = alpha_i S_{i-1} +
// u_i k_i^T, u_i = beta_i (v_i - alpha_i S_{i-1} k_i) over a chunk that starts from S0.  With
// G_i the in-chunk prefix sum of log alpha and gamma_i = exp(G_i):
//   (I + A) U = B,  A_ij = beta_i exp(G_i - G_j) k_i.k_j (j < i),  B_i = beta_i (v_i - gamma_i S0 k_i)
//   o_i = gamma_i S0 q_i + sum_{j <= i} exp(G_i - G_j) (k_j.q_i) u_j
//   S_end = gamma_last S0 + sum_j exp(G_last - G_j) u_j k_j^T
// Everything but S0 is computed for all chunks in parallel, arranged so that S0 enters only
// through products with it (see pf_dn_chunk_prep); the scan carries S0 through the chunks, one
// block of 16 state rows per workgroup (rows of S evolve independently).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "mk_layout.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

namespace {

constexpr int PF_THREADS = 256;

__device__ __forceinline__ uint32_t f2bf(float f) {  // round to nearest even
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ void split_store(float v, uint16_t *hi, uint16_t *lo) {
  const uint32_t h = f2bf(v);
  *hi = (uint16_t)h;
  *lo = (uint16_t)f2bf(v - bf2f(h));
}
// four consecutive elements (8-byte aligned) as hi and lo bf16 in one 8-byte store each
__device__ __forceinline__ void split_store4(float4 v, uint16_t *hi, uint16_t *lo) {
  const uint32_t h0 = f2bf(v.x), h1 = f2bf(v.y), h2 = f2bf(v.z), h3 = f2bf(v.w);
  const uint32_t l0 = f2bf(v.x - bf2f(h0)), l1 = f2bf(v.y - bf2f(h1)), l2 = f2bf(v.z - bf2f(h2)), l3 = f2bf(v.w - bf2f(h3));
  *reinterpret_cast<uint2 *>(hi) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
  *reinterpret_cast<uint2 *>(lo) = make_uint2(l0 | (l1 << 16), l2 | (l3 << 16));
}
// GEMM operand layout (the A operand of every prefill projection): a [rows][Kc] bf16 matrix (Kc a
// multiple of 32) as 16 x 32 blocks of 1 KiB, block (rows 16 rb .., columns 32 kb ..) at element
// (rb Kc / 32 + kb) 512; within a block, row r's 8-element group q (columns 8 q ..) at 16-byte slot
// 4 r + (q ^ ((r >> 1) & 3)).  Rows are padded to a multiple of 16 (pad rows are never used).
__device__ __forceinline__ size_t ablk(int t, int k, int Kc) {
  const int r = t & 15, q = (k >> 3) & 3;
  return ((size_t)(t >> 4) * (Kc >> 5) + (k >> 5)) * 512 + (r * 4 + (q ^ ((r >> 1) & 3))) * 8 + (k & 7);
}
__device__ __forceinline__ float sigmoidf_(float x) {
  if (x >= 0.f) return 1.f / (1.f + expf(-x));
  const float e = expf(x);
  return e / (1.f + e);
}
__device__ __forceinline__ float siluf_(float x) { return x * sigmoidf_(x); }
// SiLU with the hardware exponential and reciprocal (a few ulp): x / (1 + e^-x)
__device__ __forceinline__ float silu_fast(float x) { return __fdividef(x, 1.f + __expf(-x)); }
__device__ __forceinline__ float softplusf_(float x) { return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))); }

// Max / sum over each 16-lane row with DPP (xor 1, xor 2, half-row mirror, row mirror): every lane
// of the row gets the result.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));
  v = fmaxf(v, dpp_mov<0x4E>(v));
  v = fmaxf(v, dpp_mov<0x141>(v));
  return fmaxf(v, dpp_mov<0x140>(v));
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  return v + dpp_mov<0x140>(v);
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// sum over the 256-thread workgroup; red: >= 4 floats of LDS
__device__ __forceinline__ float block_sum(float v, float *red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float s = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return s;
}

// Copy a [rows][cols] FP32 matrix (source row stride sstride) into LDS (row stride dstride; both
// multiples of 4 floats).  Rows >= nvalid read as zero.  Every thread of the workgroup calls it;
// each issues NB 16-byte loads before storing any, so the loads overlap instead of each paying
// the full memory latency.
template <int NB, int NT = PF_THREADS>
__device__ __forceinline__ void g2l(float *dst, int dstride, const float *src, size_t sstride, int rows, int cols,
                                    int nvalid) {
  const int c4 = cols >> 2, total = rows * c4;
  for (int base = 0; base < total; base += NB * NT) {
    float4 v[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int e = base + b * NT + (int)threadIdx.x;
      const int r = e / c4, c = e - r * c4;
      v[b] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e < total && r < nvalid) v[b] = *reinterpret_cast<const float4 *>(src + (size_t)r * sstride + c * 4);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int e = base + b * NT + (int)threadIdx.x;
      const int r = e / c4, c = e - r * c4;
      if (e < total) *reinterpret_cast<float4 *>(dst + r * dstride + c * 4) = v[b];
    }
  }
}
// The two halves of g2l for one batch of NB float4 per thread, so that a batch can be loaded
// into registers well before it is stored (software prefetch).
template <int NB, int NT = PF_THREADS>
__device__ __forceinline__ void g2r(float4 (&v)[NB], const float *src, size_t sstride, int rows, int cols, int nvalid) {
  const int c4 = cols >> 2, total = rows * c4;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int e = b * NT + (int)threadIdx.x;
    const int r = e / c4, c = e - r * c4;
    v[b] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (e < total && r < nvalid) v[b] = *reinterpret_cast<const float4 *>(src + (size_t)r * sstride + c * 4);
  }
}
template <int NB, int NT = PF_THREADS>
__device__ __forceinline__ void r2l(const float4 (&v)[NB], float *dst, int dstride, int rows, int cols) {
  const int c4 = cols >> 2, total = rows * c4;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int e = b * NT + (int)threadIdx.x;
    const int r = e / c4, c = e - r * c4;
    if (e < total) *reinterpret_cast<float4 *>(dst + r * dstride + c * 4) = v[b];
  }
}
__device__ __forceinline__ float dot4(const float4 a, const float4 b, float s) {
  s = fmaf(a.x, b.x, s); s = fmaf(a.y, b.y, s); s = fmaf(a.z, b.z, s); return fmaf(a.w, b.w, s);
}
__device__ __forceinline__ float4 ld4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
// Workgroup barrier that orders LDS only.  __syncthreads also waits for the wave's outstanding
// global stores, and with them (one in-order counter) for every load issued before them, which
// would drain a prefetch at each barrier; where waves exchange data through LDS only, this one
// keeps the prefetch in flight.
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ------------------------------------------------------------------------------ row kernels
__global__ void __launch_bounds__(PF_THREADS) pf_embed(const uint16_t *embed, const int32_t *tok, int H, int V,
                                                       float *X, int32_t *ctl) {
  const int t = blockIdx.x;
  int id = tok[t];
  if (id < 0 || id >= V) {
    if (threadIdx.x == 0) __hip_atomic_fetch_or(ctl + MK_CTL_ERR, MK_DERR_TOKEN, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    id = 0;
  }
  for (int i = threadIdx.x; i < H; i += PF_THREADS) X[(size_t)t * H + i] = bf2f(embed[(size_t)id * H + i]);
}

// h = x / sqrt(mean(x^2) + eps) * g, written as a bf16 hi + lo pair in the operand block layout (Kc = H)
__global__ void __launch_bounds__(PF_THREADS) pf_norm_split(const float *X, const float *g, int H, float eps,
                                                            uint16_t *oh, uint16_t *ol) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const float *x = X + (size_t)t * H;
  float s = 0.f;
  for (int i = threadIdx.x; i < H; i += PF_THREADS) s = fmaf(x[i], x[i], s);
  const float den = sqrtf(block_sum(s, red) / (float)H + eps);
  for (int i = threadIdx.x; i < H; i += PF_THREADS)
    split_store(x[i] / den * g[i], oh + ablk(t, i, H), ol + ablk(t, i, H));
}

// ------------------------------------------------------------------------------ MFMA GEMM
// C[M][N] = A[M][K] . W[N][K]^T with A given as bf16 hi + lo and W as bf16, both in the operand
// block layout (W: the prefill weight copies of mk_layout.h).  One wave computes MT x NT 16x16 blocks with
// v_mfma_f32_16x16x32_bf16 (lane l: A row l%16 and B column l%16 with k = 8 (l/16) .. +8;
// result rows 4 (l/16) .. +4 of column l%16).
struct PfGemm {
  const uint16_t *ah, *al;            // A as bf16 hi + lo in the GEMM operand block layout (Kc = K)
  int M, N, K;
  const uint16_t *w;                  // W [N][K] in the operand block layout (rows padded to a multiple of 16)
  float *c;
  int ldc;
  uint16_t *oh, *ol;                  // EPI_SWIGLU: output in the operand block layout, Kc = ldo
  int ldo;
  int kper;            // K columns per split; == K without split-K
  float *part;         // EPI_PART: split z writes part[z][row][ldc]
  size_t part_stride;  // elements per split
  int tn, tm, tz;      // tiles along N, along M, and K splits (the grid is their product)
};
enum { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_PART = 3 };


// Workgroup tile BM x BN (BM = WGM*MT*16, BN = WGN*NT*16, WGM*WGN waves), K in stages of 32.
// Each stage of A (hi and lo) and W is copied into LDS by direct-to-LDS loads
// (global_load_lds_dwordx4: lane l of a wave writes 16 bytes at LDS base + 16 l), in 1 KiB blocks of
// 16 rows x 32 k, in a ring of NS stages: the loads of stage st + NS are issued while stage st + 1
// is read, so NS - 1 stages are in flight and no register holds a load in flight.  Within a block,
// row r's 8-element group q sits at slot 4 r + (q ^ ((r >> 1) & 3)): the fragment reads (lane l:
// row l % 16, group l / 16) of each 8 consecutive lanes then cover all 32 banks once.  A arrives in
// that block layout already (written so by the kernels producing GEMM operands), W from the prefill
// weight copies in the same layout: every block load is 1 KiB of contiguous memory.
constexpr int GBK = 32;

template <int EPI, int MT, int NT, int WGM, int WGN, int NS>
__global__ void __launch_bounds__(WGM * WGN * 64) pf_gemm(PfGemm g) {
  constexpr int NW = WGM * WGN, BM = WGM * MT * 16, BN = WGN * NT * 16;
  constexpr int NBA = BM / 16, NBB = BN / 16, NBLK = 2 * NBA + NBB;   // 1 KiB blocks per stage
  static_assert(NBLK % NW == 0, "every wave issues the same number of block loads");
  constexpr int DPW = NBLK / NW;
  extern __shared__ __attribute__((aligned(1024))) unsigned char gsm[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w / WGN, wn = w % WGN;
  // Workgroup b runs on XCD b % 8.  XCD x takes a contiguous block of the tiles ordered (split,
  // N tile, M tile), so that each weight slice (and, with split-K, each activation slab) is pulled
  // into one XCD's L2 only.
  const int ntile = g.tn * g.tm * g.tz, xcd = blockIdx.x & 7, q8 = ntile >> 3, r8 = ntile & 7;
  const int tile = xcd * q8 + min(xcd, r8) + (int)(blockIdx.x >> 3);
  const int tmi = tile % g.tm, tni = (tile / g.tm) % g.tn, tzi = tile / (g.tm * g.tn);
  const int bm0 = tmi * BM, bn0 = tni * BN;
  const int kbeg = tzi * g.kper, nst = g.kper / GBK, kb0 = kbeg / GBK, kbn = g.K / GBK;
  // this lane's loads: block b = w + i NW of a stage (A hi blocks, A lo blocks, then W blocks; W
  // blocks past the last row block of N are clamped to it, their products never stored)
  const uint16_t *src[DPW];
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    const int b = w + i * NW;
    if (b < 2 * NBA) {
      const int hl = b / NBA, rb = b % NBA;
      src[i] = (hl ? g.al : g.ah) + ((size_t)(bm0 / 16 + rb) * kbn + kb0) * 512 + lane * 8;
    } else {
      const int nb = min(bn0 / 16 + (b - 2 * NBA), (g.N + 15) / 16 - 1);
      src[i] = g.w + ((size_t)nb * kbn + kb0) * 512 + lane * 8;
    }
  }
  auto issue = [&](int st) {
    const int buf = st % NS, sa = min(st, nst - 1);
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      const int b = w + i * NW;
      __builtin_amdgcn_global_load_lds((const void *)(src[i] + (size_t)sa * 512),
                                       (__attribute__((address_space(3))) void *)(gsm + (buf * NBLK + b) * 1024), 16, 0, 0);
    }
  };
  f32x4 acc[MT][NT], acl[MT][NT];   // hi and lo products in separate accumulators (no MFMA waits on its neighbour)
#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int ni = 0; ni < NT; ++ni) acc[mi][ni] = acl[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int fpos = ((lane & 15) * 4 + ((lane >> 4) ^ (((lane & 15) >> 1) & 3))) * 16;
  typedef bf16x8 FragM[MT];
  typedef bf16x8 FragN[NT];
  // Per stage, in this order with nothing moved across: the next stage's fragment reads one at a
  // time, each followed by MPR of the current stage's MFMAs (the loads of a later stage after the
  // second read), so that no wave queues all its LDS reads ahead of its first MFMA.
  constexpr int NRD = 2 * MT + NT, NMF = 2 * MT * NT, MPR = NMF / NRD;
  auto step = [&](int stn, int sti, FragM &fan, FragM &fln, FragN &fbn, const FragM &fa, const FragM &fl, const FragN &fb) {
    const unsigned char *sb = gsm + (stn % NS) * NBLK * 1024 + fpos;
    int mf = 0;
#pragma unroll
    for (int j = 0; j < NRD; ++j) {
      if (j < MT) fan[j] = *reinterpret_cast<const bf16x8 *>(sb + (wm * MT + j) * 1024);
      else if (j < 2 * MT) fln[j - MT] = *reinterpret_cast<const bf16x8 *>(sb + (NBA + wm * MT + j - MT) * 1024);
      else fbn[j - 2 * MT] = *reinterpret_cast<const bf16x8 *>(sb + (2 * NBA + wn * NT + j - 2 * MT) * 1024);
      if (j == 1) issue(sti);
      const int mend = (j == NRD - 1) ? NMF : mf + MPR;
#pragma unroll
      for (; mf < mend; ++mf) {
        const int lo = mf >= MT * NT, q = lo ? mf - MT * NT : mf, mi = q / NT, ni = q % NT;
        if (lo) acl[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fl[mi], fb[ni], acl[mi][ni], 0, 0, 0);
        else acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // vmcnt(n) with lgkmcnt(0): the encoding is vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
  constexpr int WPRO = (NS - 1) * DPW, WLOOP = (NS - 2) * DPW;
  constexpr int ENC_PRO = 0x0070 | (WPRO & 15) | ((WPRO >> 4) << 14);
  constexpr int ENC_LOOP = 0x0070 | (WLOOP & 15) | ((WLOOP >> 4) << 14);
  static_assert(WPRO < 64, "vmcnt range");
#pragma unroll
  for (int s = 0; s < NS; ++s) issue(s);
  __builtin_amdgcn_s_waitcnt(ENC_PRO);
  __builtin_amdgcn_s_barrier();
  FragM a0, l0, a1, l1;
  FragN b0, b1;
  {
    const unsigned char *sb = gsm + fpos;
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      a0[j] = *reinterpret_cast<const bf16x8 *>(sb + (wm * MT + j) * 1024);
      l0[j] = *reinterpret_cast<const bf16x8 *>(sb + (NBA + wm * MT + j) * 1024);
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) b0[j] = *reinterpret_cast<const bf16x8 *>(sb + (2 * NBA + wn * NT + j) * 1024);
  }
  // Iteration st: wait until stage st + 1 has landed (every wave's loads: vmcnt, then the barrier)
  // and every wave holds stage st in registers (lgkmcnt(0) before the barrier); read stage st + 1,
  // refill stage st's buffer with stage st + NS, multiply stage st.  Loads past the last stage
  // re-read it and are never used.
  for (int st = 0; st < nst; st += 2) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(ENC_LOOP);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    step(st + 1, st + NS, a1, l1, b1, a0, l0, b0);
    if (st + 1 >= nst) break;
    __builtin_amdgcn_s_waitcnt(ENC_LOOP);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    step(st + 2, st + NS + 1, a0, l0, b0, a1, l1, b1);
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): no load into LDS may outlive the workgroup
  // epilogue
  const int m0 = bm0 + wm * MT * 16, n0 = bn0 + wn * NT * 16;
#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int ni = 0; ni < NT; ++ni)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m0 + mi * 16 + (lane >> 4) * 4 + i;
        const int col = n0 + ni * 16 + (lane & 15);
        const float v = acc[mi][ni][i] + acl[mi][ni][i];
        if (EPI == EPI_SWIGLU) {
          // columns 2j (gate) and 2j+1 (up) of one intermediate index sit in lanes l, l^1 (DPP swap)
          const float u = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
          if ((lane & 1) == 0 && row < g.M && col < g.N) {
            const size_t o = ablk(row, col >> 1, g.ldo);
            split_store(__fdividef(v, 1.f + __expf(-v)) * u, g.oh + o, g.ol + o);   // SiLU(gate) * up
          }
        } else if (row < g.M && col < g.N) {
          if (EPI == EPI_PART) {
            g.part[tzi * g.part_stride + (size_t)row * g.ldc + col] = v;
          } else {
            float *cp = g.c + (size_t)row * g.ldc + col;
            if (EPI == EPI_RESID) *cp = *cp + v;
            else *cp = v;
          }
        }
      }
}

// X += sum of the split-K partials (split order), then, when g is given, the RMSNorm of the new row
// as a bf16 hi + lo pair in the operand block layout (Kc = H, the operand of the next projection):
// one pass over the row instead of a reduction kernel and a norm kernel.  One workgroup per row,
// float4 per thread (H <= 1024).
__global__ void __launch_bounds__(PF_THREADS) pf_reduce_norm(float *X, const float *part, int nsplit, size_t stride,
                                                             int H, const float *g, float eps, uint16_t *oh,
                                                             uint16_t *ol) {
  __shared__ float red[4];
  const int row = blockIdx.x, n4 = threadIdx.x;
  const bool on = n4 < H / 4;
  float4 xv = make_float4(0.f, 0.f, 0.f, 0.f);
  if (on) {   // (nsplit <= 4: all loads issued before the first add)
    float4 p[4];
#pragma unroll
    for (int z = 0; z < 4; ++z)
      p[z] = reinterpret_cast<const float4 *>(part + min(z, nsplit - 1) * stride + (size_t)row * H)[n4];
    float4 *xp = reinterpret_cast<float4 *>(X + (size_t)row * H) + n4;
    const float4 x0 = *xp;
    float4 acc = p[0];
#pragma unroll
    for (int z = 1; z < 4; ++z)
      if (z < nsplit) { acc.x += p[z].x; acc.y += p[z].y; acc.z += p[z].z; acc.w += p[z].w; }
    xv = make_float4(x0.x + acc.x, x0.y + acc.y, x0.z + acc.z, x0.w + acc.w);
    *xp = xv;
  }
  if (!g) return;   // uniform over the grid
  float sq = fmaf(xv.x, xv.x, 0.f);
  sq = fmaf(xv.y, xv.y, sq); sq = fmaf(xv.z, xv.z, sq); sq = fmaf(xv.w, xv.w, sq);
  const float den = sqrtf(block_sum(sq, red) / (float)H + eps);
  if (on) {
    const float4 gv = reinterpret_cast<const float4 *>(g)[n4];
    const size_t o = ablk(row, n4 * 4, H);
    split_store4(make_float4(xv.x / den * gv.x, xv.y / den * gv.y, xv.z / den * gv.z, xv.w / den * gv.w), oh + o, ol + o);
  }
}

// ------------------------------------------------------------------------------ DeltaNet
// v_mfma_f32_16x16x4f32: D += A B with A 16 x 4, B 4 x 16 (full FP32).  Lane l supplies
// A[l % 16][l / 16] and B[l / 16][l % 16]; register v of lane l holds D[4 (l / 16) + v][l % 16].
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

constexpr int PREP_TB = 16;   // tokens per run of the conv (and per workgroup of pf_dn_out)

struct PfChunk {
  const float *P;                     // [T][NP] in-projection outputs; per head x: [q | k | v | z | a | b]
  int NP, r_in, C, nh;                // C: conv channels (q of all heads, then k, then v)
  const float *conv;                  // [C][4] taps
  const float *ring;                  // [MK_RING][C] pre-conv inputs of earlier positions
  const int32_t *ctl;
  float l2_eps;
  int pofs;                           // position of row 0 = control-block position + pofs
  float *cW, *cQ, *cU, *cO, *cKt;     // per (head, chunk), CHUNK x dk each, in the fragment orders below
  float *cg, *cd;                     // [nh][PT/CHUNK][CHUNK] exp(G_i), exp(G_last - G_i)
  int T;
};

// Per (chunk, head), everything of the chunk that does not depend on the state entering it
// (the chunked form of the gated delta rule, rewritten so that the state enters only through
// products with it).  With G_i the in-chunk prefix sums of log alpha, gamma_i = e^{G_i},
// A_ij = beta_i e^{G_i - G_j} k_i.k_j (j < i), T = (I + A)^-1, M_ij = e^{G_i - G_j} q_i.k_j (j <= i):
//   W  = T diag(beta gamma) K,   U' = T diag(beta) V,
//   Q~ = diag(gamma) Q - M W,    O' = M U'
// so that, for the state S entering the chunk (rows = value dims):
//   U = U' - W S^T,   O = Q~ S^T + O',   S_next = gamma_last S + (diag(d) U)^T K,  d_i = e^{G_last - G_i}
// which is the recurrence token by token (U_i = beta_i (v_i - S_{i-1} k_i) scaled into the chunk).
// Q~ and O' use M T, computed once.  The products run on FP32 MFMA.
constexpr int CS = MK_CHUNK + 4;   // padded row stride of the chunk matrices in LDS
// The chunk terms are stored in the order in which the scan's MFMA fragments read them, so that
// each 16-byte load of a wave covers 1 KB of contiguous memory.  W, Q~, U', O' (token t, column
// n): 16 x 16 block (t / 16, n / 16), then column quad (n % 16) / 4, token t % 16, n % 4.
// K^T (dim d, token t): block (d / 16, t / 16), then token quad (t % 16) / 4, dim d % 16, t % 4.
template <int DK>
__device__ __forceinline__ int frag_tn(int t, int n) {
  return ((((t >> 4) * (DK / 16) + (n >> 4)) * 4 + ((n & 15) >> 2)) * 16 + (t & 15)) * 4 + (n & 3);
}
__device__ __forceinline__ int frag_kt(int d, int t) {
  return ((((d >> 4) * 4 + (t >> 4)) * 4 + ((t & 15) >> 2)) * 16 + (d & 15)) * 4 + (t & 3);
}
constexpr int CP_THREADS = 512, CP_WAVES = CP_THREADS / 64;
template <int DK>
__global__ void __launch_bounds__(CP_THREADS) pf_dn_chunk_prep(PfChunk c) {
  extern __shared__ float sm[];
  constexpr int KS = DK + 4;                   // padded rows keep float4 reads conflict-free
  // workgroup (head h, chunk ch) runs on XCD h % 8, like the scan workgroups of head h, which
  // then read what it writes from their own L2
  const int h = blockIdx.x, ch = blockIdx.y, nch = MK_PT / MK_CHUNK;
  const int t0 = ch * MK_CHUNK, Cn = min(MK_CHUNK, c.T - t0);
  float *Ks = sm, *Qs = Ks + MK_CHUNK * KS, *Vs = Qs + MK_CHUNK * KS;
  float *A = Vs + MK_CHUNK * KS;               // [64][CS] A (transposed), later M T
  float *X = A + MK_CHUNK * CS;                // [64][CS] (I + A)^-1
  float *Mm = X + MK_CHUNK * CS;               // [64][CS] M
  float *R = Mm + MK_CHUNK * CS;               // [3][16][17] partial sums of the inverse
  float *Gs = R + 3 * 16 * 17, *bs = Gs + MK_CHUNK, *gam = bs + MK_CHUNK, *bgam = gam + MK_CHUNK;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  {  // the causal conv (taps over positions p-3 .. p) + SiLU of the head's q, k and v channels
     // into Qs, Ks, Vs (rows past the chunk's end: zero).  Item = (channel, run of PREP_TB tokens):
     // lanes take consecutive channels, so each of its PREP_TB + 3 loads is a coalesced row
     // segment; all of them are issued before any is used.  Positions before the pass come from
     // the ring (the conv inputs of earlier positions).
    constexpr int NCH = 3 * DK, NRUN = MK_CHUNK / PREP_TB;
    const int p0 = c.ctl[MK_CTL_POS] + c.pofs;
#pragma unroll 1
    for (int it = tid; it < NCH * NRUN; it += CP_THREADS) {
      const int chn = it % NCH, run = it / NCH, seg = chn / DK, i = chn - seg * DK;
      const int col = h * c.r_in + chn, cch = seg * c.nh * DK + h * DK + i, tb = t0 + run * PREP_TB;
      const float4 wt = ld4(c.conv + cch * 4);
      float x[PREP_TB + 3];
#pragma unroll
      for (int u = 0; u < PREP_TB + 3; ++u) {   // branch-free: every load issued, invalid ones zeroed
        const int tt = tb + u - 3;              // pass token
        const bool ok = tt >= 0 ? tt < c.T : p0 + tt >= 0;
        const float *src = tt >= 0 ? c.P + (size_t)min(tt, c.T - 1) * c.NP + col
                                   : c.ring + ((p0 + tt) & (MK_RING - 1)) * c.C + cch;
        const float v = *src;
        x[u] = ok ? v : 0.f;
      }
      float *dst = (seg == 0 ? Qs : seg == 1 ? Ks : Vs) + (run * PREP_TB) * KS + i;
#pragma unroll
      for (int j = 0; j < PREP_TB; ++j) {
        float a = fmaf(wt.x, x[j], 0.f);
        a = fmaf(wt.y, x[j + 1], a);
        a = fmaf(wt.z, x[j + 2], a);
        a = fmaf(wt.w, x[j + 3], a);
        dst[j * KS] = (run * PREP_TB + j < Cn) ? silu_fast(a) : 0.f;
      }
    }
  }
  __syncthreads();
  {  // L2 norms of the q and k rows, in place: 16 lanes per row (token j, Qs or Ks), DK / 16
     // elements per lane, summed with DPP
    constexpr int EPL = DK / 16, RPW = 4, NR = 2 * MK_CHUNK;
#pragma unroll 1
    for (int r = w * RPW + (lane >> 4); r < NR; r += CP_WAVES * RPW) {
      float *row = ((r & 1) ? Ks : Qs) + (r >> 1) * KS + (lane & 15) * EPL;
      float v[EPL];
#pragma unroll
      for (int q = 0; q < EPL; q += 4) {
        const float4 x4 = ld4(row + q);
        v[q] = x4.x; v[q + 1] = x4.y; v[q + 2] = x4.z; v[q + 3] = x4.w;
      }
      float sq = 0.f;
#pragma unroll
      for (int q = 0; q < EPL; ++q) sq = fmaf(v[q], v[q], sq);
      const float nrm = sqrtf(row_sum16(sq) + c.l2_eps);
#pragma unroll
      for (int q = 0; q < EPL; q += 4)
        *reinterpret_cast<float4 *>(row + q) = make_float4(v[q] / nrm, v[q + 1] / nrm, v[q + 2] / nrm, v[q + 3] / nrm);
    }
  }
  if (tid < 64) {  // in-chunk prefix sums of log alpha (one wave, Hillis-Steele), the decays
    // gates of token t0 + tid: log alpha = -softplus(a), beta = sigmoid(b)
    const bool ok = tid < Cn;
    const float *pa = c.P + (size_t)(t0 + (ok ? tid : 0)) * c.NP + h * c.r_in + 4 * DK;   // a, b
    const float pa0 = pa[0], pa1 = pa[1];
    float G = ok ? -softplusf_(pa0) : 0.f;
    const float b = ok ? sigmoidf_(pa1) : 0.f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(G, o, 64);
      if (tid >= o) G += y;
    }
    Gs[tid] = G;
    bs[tid] = b;
    gam[tid] = ok ? expf(G) : 0.f;
    bgam[tid] = b * gam[tid];
  }
  __syncthreads();
  // the 10 16 x 16 tiles (ti, tj) with ti >= tj of a 64 x 64 lower triangular matrix
  auto tile = [](int tt, int &ti, int &tj) { ti = tt < 1 ? 0 : tt < 3 ? 1 : tt < 6 ? 2 : 3; tj = tt - ti * (ti + 1) / 2; };
  {  // k_i.k_j and q_i.k_j on the lower tiles (FP32 MFMA; in the i-th group of four k steps lane
     // group g takes the dims 16 i + 4 g ..); tiles above are never read
#pragma unroll 1
    for (int tt = w; tt < 10; tt += CP_WAVES) {
      int ti, tj;
      tile(tt, ti, tj);
      f32x4 kk = {0.f, 0.f, 0.f, 0.f}, qk = kk;
      const float *ka = Ks + (16 * ti + c16) * KS + 4 * g, *qa = Qs + (16 * ti + c16) * KS + 4 * g;
      const float *kb = Ks + (16 * tj + c16) * KS + 4 * g;
#pragma unroll 4
      for (int i = 0; i < DK / 16; ++i) {
        const float4 a = ld4(ka + 16 * i), q = ld4(qa + 16 * i), b = ld4(kb + 16 * i);
        kk = mfma4(a.x, b.x, kk); qk = mfma4(q.x, b.x, qk);
        kk = mfma4(a.y, b.y, kk); qk = mfma4(q.y, b.y, qk);
        kk = mfma4(a.z, b.z, kk); qk = mfma4(q.z, b.z, qk);
        kk = mfma4(a.w, b.w, kk); qk = mfma4(q.w, b.w, qk);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = 16 * ti + 4 * g + v, j = 16 * tj + c16;
        const bool lower = j <= i && i < Cn;
        const float dec = lower ? expf(Gs[i] - Gs[j]) : 0.f;
        A[j * CS + i] = (lower && j < i) ? bs[i] * dec * kk[v] : 0.f;   // transposed: A[j][i] holds A_ij
        Mm[i * CS + j] = dec * qk[v];
      }
    }
  }
  __syncthreads();
  // X = (I + A)^-1 (unit lower triangular), by blocks of 16: the four diagonal blocks
  // X_qq = (I + A_qq)^-1 by forward substitution, one wave each (lane c < 16 owns column c in
  // registers); then block row by block row X_ij = -X_ii sum_{k=j}^{i-1} A_ik X_kj, each 16 x 16
  // product on 256 threads, the two halves of the workgroup taking alternate blocks j.
  // Blocks above the diagonal are zero.
  {
    constexpr int NB = 16, NBK = MK_CHUNK / NB;
    for (int e = tid; e < MK_CHUNK * MK_CHUNK; e += CP_THREADS) {
      const int i = e / MK_CHUNK, jx = e % MK_CHUNK;
      if (jx / NB > i / NB) X[i * CS + jx] = 0.f;
    }
    if (w < NBK && lane < NB) {
      const int b0 = w * NB, jj = lane;
      float col[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) col[i] = (i == jj) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < NB - 1; ++m) {
        const float xm = col[m];
        const float *am = A + (b0 + m) * CS + b0;   // A[b0+m][b0+i] = A_{b0+i, b0+m}
#pragma unroll
        for (int i = m + 1; i < NB; ++i) col[i] = fmaf(-am[i], xm, col[i]);
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) X[(b0 + i) * CS + b0 + jj] = col[i];
    }
    __syncthreads();
    constexpr int RS = NB + 1;   // R: [NBK - 1][NB][RS] partial sums of one block row
    const int half = tid >> 8, ri = (tid >> 4) & 15, rj = tid & 15;   // element of a 16 x 16 block
    for (int bi = 1; bi < NBK; ++bi) {
      // R_bj = sum_{k=j}^{bi-1} A_{bi,k} X_{k,j} for every block j < bi
      for (int bj = half; bj < bi; bj += 2) {
        float acc = 0.f;
        for (int bk = bj; bk < bi; ++bk)
#pragma unroll
          for (int t = 0; t < NB; ++t)   // A_{bi*16+ri, bk*16+t} X_{bk*16+t, bj*16+rj}
            acc = fmaf(A[(bk * NB + t) * CS + bi * NB + ri], X[(bk * NB + t) * CS + bj * NB + rj], acc);
        R[(bj * NB + ri) * RS + rj] = acc;
      }
      __syncthreads();
      // X_{bi,j} = -X_{bi,bi} R_bj (X_bi,bi lower triangular)
      for (int bj = half; bj < bi; bj += 2) {
        float acc = 0.f;
#pragma unroll
        for (int t = 0; t < NB; ++t)
          if (t <= ri) acc = fmaf(X[(bi * NB + ri) * CS + bi * NB + t], R[(bj * NB + t) * RS + rj], acc);
        X[(bi * NB + ri) * CS + bj * NB + rj] = -acc;
      }
      __syncthreads();
    }
  }
  {  // M T into A (both lower triangular), by lower tiles: MT_{ti,tj} = sum_{kb=tj}^{ti} M_{ti,kb} T_{kb,tj}
#pragma unroll 1
    for (int tt = w; tt < 10; tt += CP_WAVES) {
      int ti, tj;
      tile(tt, ti, tj);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int kb = tj; kb <= ti; ++kb)
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          const int m = 16 * kb + 4 * k4 + g;
          acc = mfma4(Mm[(16 * ti + c16) * CS + m], X[m * CS + 16 * tj + c16], acc);
        }
#pragma unroll
      for (int v = 0; v < 4; ++v) A[(16 * ti + 4 * g + v) * CS + 16 * tj + c16] = acc[v];
    }
  }
  __syncthreads();
  const size_t cb = (size_t)h * nch + ch, mo = cb * MK_CHUNK * DK;
  {  // W, U', Q~, O' by 16 x 16 blocks (token block rb, column block nt), computed transposed
     // (A operand from K or V, B operand from T or M T) so that each lane ends with four
     // consecutive columns of one token: one 16-byte store in fragment order.  The k range of
     // token block rb ends at its diagonal.
    // With two workgroups per (head, chunk) (blockIdx.z, for DK == 128) each takes half of the
    // column blocks nt, and each wave two units whose k ranges add up to 5 blocks: token blocks 0
    // and 3, or 1 and 2 (the work of unit (rb, nt) grows with rb).  One workgroup: every unit.
    const bool split = DK == 128 && gridDim.z == 2;
    const int nunit = split ? 2 : (DK / 16) * 4 / CP_WAVES;
#pragma unroll 1
    for (int ui = 0; ui < nunit; ++ui) {
      const int u = w + ui * CP_WAVES;
      const int nt = split ? (int)blockIdx.z * 4 + (w & 3) : u % (DK / 16);
      const int rb = split ? ((w >> 2) ? (ui ? 2 : 1) : (ui ? 3 : 0)) : u / (DK / 16);
      const int d = 16 * nt + c16;
      f32x4 aw = {0.f, 0.f, 0.f, 0.f}, aq = aw, au = aw, ao = aw;
      for (int kb = 0; kb <= rb; ++kb) {
        float x[4], mt[4], bk[4], bv[4];
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          const int j = 16 * kb + 4 * k4 + g;
          x[k4] = X[(16 * rb + c16) * CS + j];
          mt[k4] = A[(16 * rb + c16) * CS + j];
          bk[k4] = Ks[j * KS + d] * bgam[j];
          bv[k4] = Vs[j * KS + d] * bs[j];
        }
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          aw = mfma4(bk[k4], x[k4], aw);
          aq = mfma4(bk[k4], mt[k4], aq);
          au = mfma4(bv[k4], x[k4], au);
          ao = mfma4(bv[k4], mt[k4], ao);
        }
      }
      // lane (g, c16), register v: token t = 16 rb + c16, column 16 nt + 4 g + v
      const int t = 16 * rb + c16, n0 = 16 * nt + 4 * g;
      const size_t o = mo + frag_tn<DK>(t, n0);
      const float4 q4 = ld4(Qs + t * KS + n0);
      const float gt = gam[t];
      *reinterpret_cast<float4 *>(c.cW + o) = make_float4(aw[0], aw[1], aw[2], aw[3]);
      *reinterpret_cast<float4 *>(c.cQ + o) = make_float4(gt * q4.x - aq[0], gt * q4.y - aq[1], gt * q4.z - aq[2], gt * q4.w - aq[3]);
      *reinterpret_cast<float4 *>(c.cU + o) = make_float4(au[0], au[1], au[2], au[3]);
      *reinterpret_cast<float4 *>(c.cO + o) = make_float4(ao[0], ao[1], ao[2], ao[3]);
    }
  }
  if (blockIdx.z != 0) return;   // the rest is written once per (head, chunk)
  for (int e = tid; e < DK * MK_CHUNK; e += CP_THREADS) {   // K^T in fragment order:
    // e = (((db * 4 + tb) * 4 + tq) * 16 + dl) * 4 + te
    const int te = e & 3, dl = (e >> 2) & 15, tq = (e >> 6) & 3, tb = (e >> 8) & 3, db = e >> 10;
    const int d = 16 * db + dl, t = 16 * tb + 4 * tq + te;
    c.cKt[mo + e] = Ks[t * KS + d];
  }
  if (tid < MK_CHUNK) {
    const int i = tid;
    const size_t o = cb * MK_CHUNK + i;
    c.cg[o] = gam[i];
    c.cd[o] = i < Cn ? expf(Gs[Cn - 1] - Gs[i]) : 0.f;
  }
}

struct PfScan {
  float *S;                        // [nh][dv][dk] layer state
  const float *pend;               // [2][nh][MAXCOL][mk_pend_stride(dv)] pending updates (mk_layout.h)
  const int32_t *ctl;
  const float *cW, *cU, *cKt, *cg, *cd;
  float *snap;                     // [nh][PT/CHUNK][dv][dk] the state entering each chunk
  int T, nh;
  const float *P;                  // [T][NP] in-projection outputs (conv inputs of the pass)
  int NP, r_in, C;
  float *ring;                     // [MK_RING][C] conv inputs by position, for the decode kernel
  int pofs;                        // position of row 0 = control-block position + pofs
  int replay;                      // 1: apply the pending updates of a verify forward first (the
                                   // first row block of a pass; a later block finds them applied)
};

// Carry 16 rows of one head's state through every chunk of the pass.  Per chunk, with S the
// state entering it (first stored as the chunk's snapshot for the outputs): P = S W^T (16 x 64
// on FP32 MFMA: wave w takes token block w % 4 over half w / 4 of the key dims, the halves
// summed through LDS), U = U' - P^T; then S <- gamma_last S + (diag(d) U)^T K (wave w takes the
// 16 state columns of block w).  The outputs O = Q~ S^T + O' need only the snapshots and are
// computed afterwards for all chunks at once (pf_dn_out), off this sequential path.  The state
// moves between the two MFMA layouts through LDS; the next chunk's operands are loaded into
// registers while the current one is computed.
constexpr int SCAN_THREADS = 512;
template <int DK>
__global__ void __launch_bounds__(SCAN_THREADS) pf_dn_scan(PfScan s) {
  constexpr int SR = 16;              // state rows per workgroup
  // MFMA k order: in the i-th group of four k steps, lane group g takes the four dims (or tokens)
  // 16 i + 4 g .. 16 i + 4 g + 3, so that one 16-byte load per lane reads 64 contiguous bytes per row
  constexpr int SL = DK + 4, DL = MK_CHUNK + 4;
  extern __shared__ float sm[];
  float *Sl = sm;                     // [SR][SL] the state rows, row-major
  float *Dl = Sl + SR * SL;           // [SR][DL] diag(d) U, transposed: [row][token]
  float *Pl = Dl + SR * DL;           // [4][64][4] second halves of the P tiles, per (token block, lane)
  const int h = blockIdx.x, r0 = blockIdx.y * SR;   // head h on XCD h % 8 (see the chunk terms)
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int nch = MK_PT / MK_CHUNK, nchunk = (s.T + MK_CHUNK - 1) / MK_CHUNK;
  const bool upd = w < DK / 16, lo = w < 4;
  const int pt = w & 3, kh = w >> 2;  // token block and key-dim half of the P tile
  float *Sg = s.S + ((size_t)h * DK + r0) * DK;
  if (blockIdx.y == 0) {  // the head's conv inputs of the pass's last positions into the ring
    // (the conv of this pass has read the earlier positions it needs from it already)
    const int n = min(s.T, MK_RING), p0 = s.ctl[MK_CTL_POS] + s.pofs;
    for (int e = tid; e < n * 3 * DK; e += SCAN_THREADS) {
      const int t = s.T - n + e / (3 * DK), q = e % (3 * DK), seg = q / DK;
      s.ring[((p0 + t) & (MK_RING - 1)) * s.C + seg * s.nh * DK + h * DK + (q - seg * DK)] =
          s.P[(size_t)t * s.NP + h * s.r_in + q];
    }
  }
  for (int e = tid; e < SR * DK / 4; e += SCAN_THREADS) {
    const int r = e / (DK / 4), c4 = e - r * (DK / 4);
    *reinterpret_cast<float4 *>(Sl + r * SL + c4 * 4) = ld4(Sg + r * DK + c4 * 4);
  }
  __syncthreads();
  // pending updates left by a verify forward (same arithmetic as the decode kernel's step)
  const int pend_n = s.replay ? s.ctl[MK_CTL_PEND] : 0, par = s.ctl[MK_CTL_PAR];
  for (int jp = 0; jp < pend_n; ++jp) {
    const float *pk = s.pend + (((size_t)par * s.nh + h) * MK_MAXCOL + jp) * mk_pend_stride(DK);
    const float *pv = pk + MK_PEND_K;   // (v_r, alpha, beta, 0) per value row
    const float a = pv[1], b = pv[2];
    for (int r = w; r < SR; r += SCAN_THREADS / 64) {
      float p = 0.f;
      for (int e = lane; e < DK; e += 64) p = fmaf(Sl[r * SL + e], pk[4 * (e & 63) + (e >> 6)], p);
      const float sk = wave_sum(p);
      const float u = b * (pv[4 * (r0 + r)] - a * sk);
      for (int e = lane; e < DK; e += 64) Sl[r * SL + e] = fmaf(u, pk[4 * (e & 63) + (e >> 6)], a * Sl[r * SL + e]);
    }
  }
  __syncthreads();
  // the state in the MFMA result layout: S[4 g + v][16 w + c16] (waves with a column block)
  f32x4 sc = {0.f, 0.f, 0.f, 0.f};
  if (upd) {
#pragma unroll
    for (int v = 0; v < 4; ++v) sc[v] = Sl[(4 * g + v) * SL + 16 * w + c16];
  }
  // operands of one chunk, per lane: the P tile's B fragments (W row 16 pt + c16, the lane's half
  // of the dims), the K^T fragments of the column block (dim 16 w + c16), U' (token 16 pt + c16,
  // rows 4 g ..) and d of that token
  constexpr int NBP = DK / 32;
  struct Ops { float4 bp[NBP]; float4 bk[4]; float4 uo; float dd, gl; };
  // Every wave issues the same loads for every chunk index (clamped to the last chunk), so the
  // number of loads in flight never depends on the path taken and the compiler's waits stay exact.
  auto fetch = [&](Ops &op, int c) {
    c = min(c, nchunk - 1);
    const size_t cb = (size_t)h * nch + c, mo = cb * MK_CHUNK * DK;
    const float *P = s.cW + mo + frag_tn<DK>(16 * pt + c16, 4 * g);
#pragma unroll
    for (int i = 0; i < NBP; ++i) op.bp[i] = ld4(P + 256 * (kh * NBP + i));
    const float *K = s.cKt + mo + frag_kt(16 * min(w, DK / 16 - 1) + c16, 4 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) op.bk[i] = ld4(K + 256 * i);
    op.uo = ld4(s.cU + mo + frag_tn<DK>(16 * pt + c16, r0 + 4 * g));
    op.dd = s.cd[cb * MK_CHUNK + 16 * pt + c16];
    op.gl = s.cg[cb * MK_CHUNK + min(MK_CHUNK, s.T - c * MK_CHUNK) - 1];   // gamma of the chunk's last token
  };
  // one chunk: operands in `cur`, while the operands of chunk c + 2 are loaded into `pre`.  A step
  // past the last chunk (the loop runs in threes) leaves the state as it is: d = 0, gamma = 1.
  auto step = [&](const Ops &cur, Ops &pre, int c) {
    const bool act = c < nchunk;
    const float dd = act ? cur.dd : 0.f, gl = act ? cur.gl : 1.f;
    if (act) {   // snapshot of the state entering chunk c (uniform branch)
      float *sn = s.snap + (((size_t)h * nch + c) * DK + r0) * DK;
      for (int e = tid; e < SR * DK / 4; e += SCAN_THREADS) {
        const int r = e / (DK / 4), c4 = e - r * (DK / 4);
        *reinterpret_cast<float4 *>(sn + r * DK + c4 * 4) = ld4(Sl + r * SL + c4 * 4);
      }
    }
    fetch(pre, c + 2);
    // P tile half: rows 4 g + v, token 16 pt + c16, dims of half kh; two chains of MFMAs
    f32x4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = p0;
    {
      const float *sr = Sl + c16 * SL + 4 * g + kh * (DK / 2);
#pragma unroll
      for (int i = 0; i < NBP; i += 2) {
        const float4 a = ld4(sr + 16 * i), b = cur.bp[i];
        const float4 a2 = ld4(sr + 16 * (i + 1)), b2 = cur.bp[i + 1];
        p0 = mfma4(a.x, b.x, p0); p1 = mfma4(a2.x, b2.x, p1);
        p0 = mfma4(a.y, b.y, p0); p1 = mfma4(a2.y, b2.y, p1);
        p0 = mfma4(a.z, b.z, p0); p1 = mfma4(a2.z, b2.z, p1);
        p0 = mfma4(a.w, b.w, p0); p1 = mfma4(a2.w, b2.w, p1);
      }
    }
    const f32x4 p = p0 + p1;
    if (!lo) *reinterpret_cast<f32x4 *>(Pl + (pt * 64 + lane) * 4) = p;
    lds_barrier();
    if (lo) {
      const f32x4 q = *reinterpret_cast<const f32x4 *>(Pl + (pt * 64 + lane) * 4);
      const int tok = 16 * pt + c16;
      Dl[(4 * g + 0) * DL + tok] = dd * (cur.uo.x - (p[0] + q[0]));
      Dl[(4 * g + 1) * DL + tok] = dd * (cur.uo.y - (p[1] + q[1]));
      Dl[(4 * g + 2) * DL + tok] = dd * (cur.uo.z - (p[2] + q[2]));
      Dl[(4 * g + 3) * DL + tok] = dd * (cur.uo.w - (p[3] + q[3]));
    }
    lds_barrier();
    if (upd) {  // S <- gamma_last S + D K on the column block 16 w ..
      f32x4 acc = {gl * sc[0], gl * sc[1], gl * sc[2], gl * sc[3]};
      const float *dr = Dl + c16 * DL + 4 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 a = ld4(dr + 16 * i), b = cur.bk[i];
        acc = mfma4(a.x, b.x, acc); acc = mfma4(a.y, b.y, acc); acc = mfma4(a.z, b.z, acc); acc = mfma4(a.w, b.w, acc);
      }
      sc = acc;
#pragma unroll
      for (int v = 0; v < 4; ++v) Sl[(4 * g + v) * SL + 16 * w + c16] = sc[v];
    }
    lds_barrier();
  };
  // three operand sets in rotation (no register copies, so that nothing waits on a load in
  // flight before its chunk): each chunk's operands are loaded two chunks ahead
  Ops o0, o1, o2;
  fetch(o0, 0);
  fetch(o1, 1);
  // wait for the first two chunks' operands here: with loads still pending on the way into the
  // loop, the compiler's waits at the loop head would also wait for the prefetch issued in it
  wait_loads();
  for (int c = 0; c < nchunk; c += 3) {
    step(o0, o2, c);
    step(o1, o0, c + 1);
    step(o2, o1, c + 2);
  }
  if (upd) {
#pragma unroll
    for (int v = 0; v < 4; ++v) Sg[(size_t)(4 * g + v) * DK + 16 * w + c16] = sc[v];
  }
}

// Outputs of the delta rule for 16 tokens of one head, from the snapshot S of the state entering
// their chunk: O = Q~ S^T + O' (FP32 MFMA, wave w: value columns 16 w ..), then the gated RMSNorm
// y = O / sqrt(mean(O^2) + eps) * g * SiLU(z) per token, written as bf16 hi + lo in the operand
// block layout (Kc = nh dv) for the out-projection.  z of head h, token t: P[t NP + h r_in + 2 dk + dv + i].
struct PfOut {
  const float *cQ, *cO, *snap;
  const float *P;
  int NP, r_in;
  const float *gn;
  int nh;
  float eps;
  uint16_t *oh, *ol;
  int T;
};
template <int DK>
__global__ void __launch_bounds__(DK * 4) pf_dn_out(PfOut o) {
  constexpr int NWV = DK / 16;
  __shared__ float red[NWV][16];
  const int h = blockIdx.y, t0 = blockIdx.x * 16, c = t0 / MK_CHUNK, nch = MK_PT / MK_CHUNK;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const size_t cb = (size_t)h * nch + c, mo = cb * MK_CHUNK * DK;
  const int tc = t0 - c * MK_CHUNK;   // token offset inside the chunk
  const float *qa = o.cQ + mo + frag_tn<DK>(tc + c16, 4 * g);
  const float *sb = o.snap + (cb * DK + 16 * w + c16) * DK + 4 * g;
  float4 qf[DK / 16], sf[DK / 16];
#pragma unroll
  for (int i = 0; i < DK / 16; ++i) { qf[i] = ld4(qa + 256 * i); sf[i] = ld4(sb + 16 * i); }
  float op[4], zv[4];
  const int n = 16 * w + c16;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    op[v] = o.cO[mo + frag_tn<DK>(tc + 4 * g + v, n)];
    zv[v] = o.P[(size_t)min(t0 + 4 * g + v, o.T - 1) * o.NP + h * o.r_in + 3 * DK + n];
  }
  const float gnv = o.gn[n];
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
#pragma unroll
  for (int i = 0; i < DK / 16; i += 2) {
    a0 = mfma4(qf[i].x, sf[i].x, a0); a1 = mfma4(qf[i + 1].x, sf[i + 1].x, a1);
    a0 = mfma4(qf[i].y, sf[i].y, a0); a1 = mfma4(qf[i + 1].y, sf[i + 1].y, a1);
    a0 = mfma4(qf[i].z, sf[i].z, a0); a1 = mfma4(qf[i + 1].z, sf[i + 1].z, a1);
    a0 = mfma4(qf[i].w, sf[i].w, a0); a1 = mfma4(qf[i + 1].w, sf[i + 1].w, a1);
  }
  // lane (g, c16), register v: token t0 + 4 g + v, value column 16 w + c16
  float ov[4], sq[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    ov[v] = a0[v] + a1[v] + op[v];
    sq[v] = row_sum16(ov[v] * ov[v]);
  }
  if (c16 == 0) {
#pragma unroll
    for (int v = 0; v < 4; ++v) red[w][4 * g + v] = sq[v];
  }
  __syncthreads();
  const int Kc = o.nh * DK;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int tl = 4 * g + v, t = t0 + tl;
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < NWV; ++q) ss += red[q][tl];
    if (t < o.T) {
      const float den = sqrtf(ss / (float)DK + o.eps);
      const size_t off = ablk(t, h * DK + n, Kc);
      split_store(ov[v] / den * gnv * siluf_(zv[v]), o.oh + off, o.ol + off);
    }
  }
}

// ------------------------------------------------------------------------------ attention
// 8 int8 codes (lowest byte first) times 2^e as 8 bf16 (exact: a code needs 7 significant bits and
// e is in [-126, 127], so each value is a normal bf16 number or zero)
__device__ __forceinline__ uint4 deq8_bf16(uint2 q, int e) {
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = i < 2 ? q.x : q.y, sh = 16 * (i & 1);
    const float lo = ldexpf((float)(int8_t)(w >> sh), e), hi = ldexpf((float)(int8_t)(w >> (sh + 8)), e);
    o[i] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

struct PfAtt {
  const float *P;             // [T][NP]: q (nq hd) | k (nkv hd) | v (nkv hd)
  int NP, T;
  const float *rope;          // [max_ctx][hd/2][2]
  const int32_t *page_table;
  const int32_t *ctl;
  void *kc, *vc;              // [pages][nkv][PAGE][hd] bf16, or int8 codes with kvq
  int8_t *kve;                // kvq: [pages][nkv][PAGE][2] exponents of the K, V rows
  int kvq;                    // 8-bit cache
  float *aq;                  // [PT][nq hd]
  int nq, nkv, hd;
  uint16_t *oh, *ol;          // output, operand block layout with Kc = nq hd
  int pofs;                   // position of row 0 = control-block position + pofs
};

__device__ __forceinline__ size_t kv_off(const PfAtt &a, int p, int kvh) {
  return (((size_t)a.page_table[p / MK_PAGE] * a.nkv + kvh) * MK_PAGE + (p % MK_PAGE)) * a.hd;
}

// RoPE on q and k at position p0 + t; K and V appended to the cache as bf16, or (8-bit cache) as
// codes q and an exponent e per row, q = round-half-even(x 2^-e) with e the smallest integer
// (>= -126) that keeps |q| <= 127
__global__ void __launch_bounds__(PF_THREADS) pf_att_rope(PfAtt a) {
  __shared__ float kv8[2 * MK_NX * 128];   // 8-bit cache: the rows to quantise [K|V][kv head][hd]
  const int t = blockIdx.x, p = a.ctl[MK_CTL_POS] + a.pofs + t, half = a.hd / 2;
  const float *row = a.P + (size_t)t * a.NP;
  uint16_t *kc = static_cast<uint16_t *>(a.kc), *vc = static_cast<uint16_t *>(a.vc);
  for (int e = threadIdx.x; e < (a.nq + a.nkv) * half; e += PF_THREADS) {
    const int hh = e / half, d = e % half;
    const float cs = a.rope[((size_t)p * half + d) * 2 + 0], sn = a.rope[((size_t)p * half + d) * 2 + 1];
    if (hh < a.nq) {
      const float q1 = row[hh * a.hd + d], q2 = row[hh * a.hd + d + half];
      a.aq[(size_t)t * a.nq * a.hd + hh * a.hd + d] = q1 * cs - q2 * sn;
      a.aq[(size_t)t * a.nq * a.hd + hh * a.hd + d + half] = q2 * cs + q1 * sn;
    } else {
      const int kvh = hh - a.nq;
      const float *kr = row + a.nq * a.hd + kvh * a.hd;
      const float k1 = kr[d], k2 = kr[d + half];
      if (a.kvq) {
        kv8[kvh * a.hd + d] = k1 * cs - k2 * sn;
        kv8[kvh * a.hd + d + half] = k2 * cs + k1 * sn;
      } else {
        const size_t o = kv_off(a, p, kvh);
        kc[o + d] = (uint16_t)f2bf(k1 * cs - k2 * sn);
        kc[o + d + half] = (uint16_t)f2bf(k2 * cs + k1 * sn);
      }
    }
  }
  if (!a.kvq) {
    for (int e = threadIdx.x; e < a.nkv * a.hd; e += PF_THREADS) {
      const int kvh = e / a.hd, d = e % a.hd;
      vc[kv_off(a, p, kvh) + d] = (uint16_t)f2bf(row[(a.nq + a.nkv) * a.hd + e]);
    }
    return;
  }
  for (int e = threadIdx.x; e < a.nkv * a.hd; e += PF_THREADS) kv8[MK_NX * 128 + e] = row[(a.nq + a.nkv) * a.hd + e];
  __syncthreads();
  // one wave per row: K rows of every kv head, then V rows
  const int lane = threadIdx.x & 63;
  for (int r = threadIdx.x >> 6; r < 2 * a.nkv; r += PF_THREADS / 64) {
    const int isv = r / a.nkv, kvh = r % a.nkv;
    const float *x = kv8 + isv * MK_NX * 128 + kvh * a.hd;
    const float x0 = lane < a.hd ? x[lane] : 0.f, x1 = lane + 64 < a.hd ? x[lane + 64] : 0.f;
    float am = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
    const int ex = mk_q8_exp(am);
    const size_t rix = kv_off(a, p, kvh) / a.hd;
    int8_t *dst = static_cast<int8_t *>(isv ? a.vc : a.kc) + rix * a.hd;
    if (lane < a.hd) dst[lane] = (int8_t)(int)rintf(ldexpf(x0, -ex));
    if (lane + 64 < a.hd) dst[lane + 64] = (int8_t)(int)rintf(ldexpf(x1, -ex));
    if (lane == 0) a.kve[rix * 2 + isv] = (int8_t)ex;
  }
}

// Causal attention on the matrix cores, computed transposed so that each lane owns one query:
// S^T = K Q^T and O^T += V^T P^T with v_mfma_f32_16x16x32_bf16 (result layout: lane l holds rows
// 4 (l / 16) + i of column l % 16, i.e. four keys / four dims of query l % 16).  Workgroup = 4
// waves x 16 queries of one head; key blocks of 64 positions come from the paged bf16 cache into
// LDS (row-major K and V), shared by the 4 waves.  V fragments are read with the transposing LDS
// load (ds_read_b64_tr_b16: in each 16-lane group, lanes 4r .. 4r+3 supply the 16 elements of row
// r and lane i receives column i of the four rows).  Q (FP32) and P enter as bf16 hi + lo, K
// and V are exactly bf16; the online softmax runs in FP32 per lane, with the column reductions
// over the four lane groups done by permlane swaps, and P moves from the result layout to the
// operand layout by two permlane swaps, without LDS.
constexpr int AKB = 64;                  // keys per block

// v[0..3] of two 16-key result tiles X (keys 0..15 of a 32-key step) and Y (16..31), each lane
// group g holding keys 4 g .. 4 g + 3 of its query -> the operand layout of that step: lane group
// g gets keys 8 g .. 8 g + 7 (first four in lo[], last four in hi[]).
__device__ __forceinline__ void p_to_operand(const f32x4 &X, const f32x4 &Y, float (&lo)[4], float (&hi)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x2 a = __builtin_amdgcn_permlane32_swap(__float_as_uint(X[i]), __float_as_uint(Y[i]), false, false);
    const u32x2 b = __builtin_amdgcn_permlane16_swap(a.x, a.y, false, false);
    lo[i] = __uint_as_float(b.x);
    hi[i] = __uint_as_float(b.y);
  }
}
// max / sum over the four lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48): every lane gets the result
__device__ __forceinline__ float group4_max(float v) {
  u32x2 p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(p.x), __uint_as_float(p.y));
  p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p.x), __uint_as_float(p.y));
}
__device__ __forceinline__ float group4_sum(float v) {
  u32x2 p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(p.x) + __uint_as_float(p.y);
  p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p.x) + __uint_as_float(p.y);
}
// 8 FP32 values as the bf16 hi and lo operands
__device__ __forceinline__ void split8(const float (&f)[8], bf16x8 &h, bf16x8 &l) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = (__bf16)f[e];
    l[e] = (__bf16)(f[e] - (float)h[e]);
  }
}

template <int HD, bool KVQ>
__global__ void __launch_bounds__(PF_THREADS) pf_att_mfma(PfAtt a) {
  constexpr int KS = HD / 32;            // 32-wide dim steps of K Q^T
  constexpr int NDB = HD / 16;           // 16-dim blocks of O^T
  constexpr int NCB = AKB / 16;          // 16-key tiles of S^T
  constexpr int KLD = HD + 8, VLD = HD + 16;   // padded LDS rows (bf16 elements)
  __shared__ uint16_t Ks[AKB * KLD];     // [key][dim]
  __shared__ uint16_t Vs[AKB * VLD];     // [key][dim]
  __shared__ int pages[10240 / MK_PAGE];  // the page table of every cached position (checked on the host)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hq = blockIdx.y, kvh = hq * a.nkv / a.nq;
  const int p0 = a.ctl[MK_CTL_POS] + a.pofs;
  const int t0 = blockIdx.x * 64, tw = t0 + w * 16;          // first query row of the workgroup / wave
  const int nq_wg = min(64, a.T - t0);
  const int last = p0 + t0 + nq_wg - 1;                      // largest query position of the workgroup
  const int wlast = p0 + min(tw + 15, a.T - 1);              // ... of this wave
  const bool wlive = tw < a.T;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int qrow = tw + r16, qp = p0 + qrow;                 // this lane's query
  const bool qok = qrow < a.T;
  const float sl2 = 1.4426950408889634f / sqrtf((float)HD);  // softmax in base 2: scale * log2(e)
  // Q operand of this wave: query r16, dims 32 s + 8 g4 .. +8, as hi and lo
  bf16x8 qh[KS], ql[KS];
  {
    const float *qr = a.aq + (size_t)qrow * a.nq * HD + hq * HD;
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = 0.f;
      if (qok) {
        const float4 x0 = *reinterpret_cast<const float4 *>(qr + s2 * 32 + g4 * 8);
        const float4 x1 = *reinterpret_cast<const float4 *>(qr + s2 * 32 + g4 * 8 + 4);
        f[0] = x0.x; f[1] = x0.y; f[2] = x0.z; f[3] = x0.w; f[4] = x1.x; f[5] = x1.y; f[6] = x1.z; f[7] = x1.w;
      }
      split8(f, qh[s2], ql[s2]);
    }
  }
  f32x4 o[NDB];                           // O^T: dims 16 d + 4 g4 + i of this lane's query
#pragma unroll
  for (int d = 0; d < NDB; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow = -INFINITY, lrow = 0.f;     // running max (base 2) and sum of this lane's query
  constexpr int CPR = HD / 8;                            // 16-byte chunks per key row
  constexpr int NCH = AKB * CPR / PF_THREADS;            // chunks per thread and tile
  const int nkb = last / AKB + 1;
  for (int i = tid; i <= last / MK_PAGE; i += PF_THREADS) pages[i] = a.page_table[i];
  __syncthreads();
  // K and V rows of block kb into registers (positions past `last` read as zeros); the next
  // block's loads are in flight while the current block is multiplied
  uint4 kr[NCH], vr[NCH];
  auto load_kv = [&](int kb) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int e = c * PF_THREADS + tid, r = e % AKB, cc = e / AKB, pp = kb * AKB + r;
      kr[c] = make_uint4(0u, 0u, 0u, 0u);
      vr[c] = make_uint4(0u, 0u, 0u, 0u);
      if (pp <= last) {
        const size_t rix = ((size_t)pages[pp / MK_PAGE] * a.nkv + kvh) * MK_PAGE + (pp % MK_PAGE), off = rix * HD + cc * 8;
        if constexpr (KVQ) {   // 8 codes and the row's exponent -> 8 bf16 (exactly: |code| <= 127)
          const uint2 kq = *reinterpret_cast<const uint2 *>(static_cast<const int8_t *>(a.kc) + off);
          const uint2 vq = *reinterpret_cast<const uint2 *>(static_cast<const int8_t *>(a.vc) + off);
          const char2 ex = *reinterpret_cast<const char2 *>(a.kve + rix * 2);
          kr[c] = deq8_bf16(kq, ex.x);
          vr[c] = deq8_bf16(vq, ex.y);
        } else {
          kr[c] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.kc) + off);
          vr[c] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.vc) + off);
        }
      }
    }
  };
  load_kv(0);
  for (int kb = 0; kb < nkb; ++kb) {
    const int k0 = kb * AKB;
    __syncthreads();   // every wave is done with the previous tiles
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int e = c * PF_THREADS + tid, r = e % AKB, cc = e / AKB;
      *reinterpret_cast<uint4 *>(Ks + r * KLD + cc * 8) = kr[c];
      *reinterpret_cast<uint4 *>(Vs + r * VLD + cc * 8) = vr[c];
    }
    __syncthreads();
    if (kb + 1 < nkb) load_kv(kb + 1);
    if (!wlive || k0 > wlast) continue;                  // wave-uniform: no key of this block is visible
    // S^T = K Q^T: tile cb holds keys k0 + 16 cb + 4 g4 + i of query r16
    f32x4 sc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) sc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      bf16x8 kf[NCB];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) kf[cb] = *reinterpret_cast<const bf16x8 *>(Ks + (cb * 16 + r16) * KLD + s2 * 32 + g4 * 8);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) sc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[cb], qh[s2], sc[cb], 0, 0, 0);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) sc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[cb], ql[s2], sc[cb], 0, 0, 0);
    }
    // online softmax of this lane's query over its 4 NCB keys, then over the lane groups
    float mx = -INFINITY;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kp = k0 + cb * 16 + 4 * g4 + i;
        sc[cb][i] = (qok && kp <= qp) ? sc[cb][i] * sl2 : -INFINITY;
        mx = fmaxf(mx, sc[cb][i]);
      }
    mx = group4_max(mx);
    const float mn = fmaxf(mrow, mx);
    const float al = (mn == -INFINITY) ? 1.f : exp2f(mrow - mn);
    float rs = 0.f;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sc[cb][i] = (sc[cb][i] == -INFINITY) ? 0.f : exp2f(sc[cb][i] - mn);
        rs += sc[cb][i];
      }
    rs = group4_sum(rs);
    lrow = lrow * al + rs;
    mrow = mn;
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[d][i] *= al;
    // O^T += V^T P^T, 32 keys per step
#pragma unroll
    for (int h = 0; h < AKB / 32; ++h) {
      float plo[4], phi[4];
      p_to_operand(sc[2 * h], sc[2 * h + 1], plo, phi);
      const float pf[8] = {plo[0], plo[1], plo[2], plo[3], phi[0], phi[1], phi[2], phi[3]};
      bf16x8 pah, pal;
      split8(pf, pah, pal);
#pragma unroll
      for (int d = 0; d < NDB; ++d) {
        // keys h 32 + 8 g4 .. +8 of dim 16 d + r16: rows r16 / 4 and 4 + r16 / 4 of the lane group's
        // eight keys, columns 4 (r16 % 4) .. +4
        const uint16_t *vp = Vs + (h * 32 + g4 * 8 + (r16 >> 2)) * VLD + d * 16 + (r16 & 3) * 4;
        const v4i16 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)vp);
        const v4i16 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)(vp + 4 * VLD));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, v8i16{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
        o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pah, o[d], 0, 0, 0);
        o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pal, o[d], 0, 0, 0);
      }
    }
  }
  // O / l, as hi + lo: query qrow, dims 16 d + 4 g4 + i
  if (qok) {
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const size_t off = ablk(qrow, hq * HD + d * 16 + 4 * g4 + i, a.nq * HD);
        split_store(o[d][i] / lrow, a.oh + off, a.ol + off);
      }
  }
}

// ------------------------------------------------------------------------------ LM head
__device__ __forceinline__ unsigned long long pack_best(float v, int idx) {
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // order-preserving
  return ((unsigned long long)u << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)idx);
}

// logits of the last row (final RMSNorm + tied embedding) and each workgroup's best
__global__ void __launch_bounds__(PF_THREADS) pf_lm(const float *X, int row, const float *lnf, float eps,
                                                    const uint16_t *embed, int V, int H, float *logits,
                                                    unsigned long long *best, int32_t *ctl) {
  __shared__ float hn[1024];
  __shared__ float red[4];
  __shared__ unsigned long long wb[4];
  const float *x = X + (size_t)row * H;
  float s = 0.f;
  for (int i = threadIdx.x; i < H; i += PF_THREADS) s = fmaf(x[i], x[i], s);
  const float den = sqrtf(block_sum(s, red) / (float)H + eps);
  for (int i = threadIdx.x; i < H; i += PF_THREADS) hn[i] = x[i] / den * lnf[i];
  __syncthreads();
  const int b = blockIdx.x, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r0 = (int)((long long)b * V / gridDim.x), r1 = (int)((long long)(b + 1) * V / gridDim.x);
  unsigned long long mybest = 0;
  int bad = 0;
  // Each wave streams batches of RBATCH rows, the next batch's loads in flight while the current
  // one is reduced.  Every load is issued (rows past the range and lanes past H read valid memory
  // and are masked), so the compiler's waits stay exact.
  constexpr int RBATCH = 8;
  const int stride = (PF_THREADS / 64) * RBATCH;
  auto load = [&](uint4 (&wv)[RBATCH][2], int rb) {
#pragma unroll
    for (int q = 0; q < RBATCH; ++q)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int i = lane * 8 + h2 * 512;
        wv[q][h2] = *reinterpret_cast<const uint4 *>(embed + (size_t)min(rb + q, r1 - 1) * H + (i < H ? i : 0));
      }
  };
  // a lane multiplies the same 16 hidden elements in every row: kept in registers
  float hr[2][8];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int i = lane * 8 + h2 * 512;
#pragma unroll
    for (int e = 0; e < 8; ++e) hr[h2][e] = i < H ? hn[i + e] : 0.f;
  }
  auto reduce = [&](const uint4 (&wv)[RBATCH][2], int rb) {
#pragma unroll
    for (int q = 0; q < RBATCH; ++q) {
      float p = 0.f;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int i = lane * 8 + h2 * 512;
        if (i < H) {
          const uint32_t ww[4] = {wv[q][h2].x, wv[q][h2].y, wv[q][h2].z, wv[q][h2].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            p = fmaf(__uint_as_float(ww[e] << 16), hr[h2][2 * e], p);
            p = fmaf(__uint_as_float(ww[e] & 0xffff0000u), hr[h2][2 * e + 1], p);
          }
        }
      }
      const float tot = wave_sum(p);
      const int r = rb + q;
      if (lane == 0 && r < r1) {
        if (logits) logits[r] = tot;
        if (!(tot == tot) || isinf(tot)) bad = 1;
        const unsigned long long kk = pack_best(tot, r);
        if (kk > mybest) mybest = kk;
      }
    }
  };
  uint4 wa[RBATCH][2], wc[RBATCH][2];
  int rb = r0 + w * RBATCH;
  load(wa, rb);
  for (; rb < r1; rb += 2 * stride) {
    load(wc, rb + stride);
    reduce(wa, rb);
    load(wa, rb + 2 * stride);
    reduce(wc, rb + stride);
  }
  if (lane == 0) wb[w] = mybest;
  if (bad) __hip_atomic_fetch_or(ctl + MK_CTL_ERR, MK_DERR_NAN, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long m = wb[0];
    for (int i = 1; i < 4; ++i) m = wb[i] > m ? wb[i] : m;
    best[b] = m;
  }
}

// end of a pass: the greedy token (last pass), the position, pending updates consumed
// (one wave: each lane takes every 64th candidate, then a butterfly maximum over the lanes)
__global__ void pf_finish(const unsigned long long *best, int nbest, int32_t *argmax, int32_t *ctl, int T) {
  const int lane = threadIdx.x;
  if (argmax) {
    unsigned long long m = 0;
    for (int i = lane; i < nbest; i += 64) m = best[i] > m ? best[i] : m;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const unsigned long long y = __shfl_xor(m, o, 64);
      m = y > m ? y : m;
    }
    if (lane == 0) argmax[0] = (int32_t)(0xFFFFFFFFu - (uint32_t)(m & 0xFFFFFFFFu));
  }
  if (lane == 0) {
    ctl[MK_CTL_POS] += T;
    ctl[MK_CTL_PEND] = 0;
  }
}

}  // namespace

// ------------------------------------------------------------------------------ host driver
struct MkPfHost {
  const MkDev *d;
  const MkLayerDev *layers;   // host copy of the layer table
  MkPf pf;
};

template <int EPI, int MT, int NT, int WGM, int WGN, int NS>
static hipError_t launch_gemm_t(PfGemm g, int nsplit, hipStream_t st) {
  constexpr int BM = WGM * MT * 16, BN = WGN * NT * 16;
  g.tn = (g.N + BN - 1) / BN;
  g.tm = (g.M + BM - 1) / BM;
  g.tz = nsplit;
  const size_t lds = (size_t)NS * (2 * BM / 16 + BN / 16) * 1024;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void *)pf_gemm<EPI, MT, NT, WGM, WGN, NS>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL((pf_gemm<EPI, MT, NT, WGM, WGN, NS>), dim3(g.tn * g.tm * g.tz), dim3(WGM * WGN * 64), lds, st, g);
  return hipGetLastError();
}
// Tiles (measured at 520 rows, then per row block): outputs wider than 2048 columns take 64 x 256
// workgroup tiles (8 waves of 32 x 64, 96 KiB of LDS, one workgroup per CU; 64 x 128 for row blocks
// of at most 384 rows); narrower ones 64 x 64 tiles (4 waves
// of 32 x 32) so that the grid still fills the chip.  The 1024-wide outputs that add into the
// residual stream use 64 x 128 tiles (8 waves of 32 x 32) with split-K (partials reduced in split
// order), so that the grid fills the chip and each K stream is short.
// The RMSNorm that follows a projection adding into the residual stream, fused into the split-K
// reduction when there is one (gain g; output as hi + lo in the operand block layout, Kc = N).
struct PfNext {
  const float *g;
  float eps;
  uint16_t *oh, *ol;
};
static hipError_t launch_gemm(int epi, PfGemm g, float *part, hipStream_t st, const PfNext *next = nullptr) {
  if (g.K % GBK != 0) return hipErrorInvalidValue;
  g.kper = g.K;
  // outputs wider than 2048 columns: 64 x 256 tiles, or 64 x 128 for a row block of at most 384
  // rows (measured: pp520 in two blocks 3.05 -> 3.00 ms; a 512-row block is faster with 64 x 256)
  const bool wide = g.N > 2048, few = g.M <= 384;
  if (epi == EPI_STORE)
    return !wide ? launch_gemm_t<EPI_STORE, 2, 2, 2, 2, 4>(g, 1, st)
                 : few ? launch_gemm_t<EPI_STORE, 2, 2, 2, 4, 4>(g, 1, st) : launch_gemm_t<EPI_STORE, 2, 4, 2, 4, 4>(g, 1, st);
  if (epi == EPI_SWIGLU)
    return !wide ? launch_gemm_t<EPI_SWIGLU, 2, 2, 2, 2, 4>(g, 1, st)
                 : few ? launch_gemm_t<EPI_SWIGLU, 2, 2, 2, 4, 4>(g, 1, st) : launch_gemm_t<EPI_SWIGLU, 2, 4, 2, 4, 4>(g, 1, st);
  const int ns = g.K / GBK;
  const int nsplit = (ns % 4 == 0 && ns >= 16) ? 4 : (ns % 2 == 0 && ns >= 8) ? 2 : 1;
  if (nsplit == 1 || !part || g.N > 4 * PF_THREADS || g.N % 4 != 0) {
    hipError_t e = launch_gemm_t<EPI_RESID, 2, 2, 2, 2, 4>(g, 1, st);
    if (e != hipSuccess || !next) return e;
    hipLaunchKernelGGL(pf_norm_split, dim3(g.M), dim3(PF_THREADS), 0, st, (const float *)g.c, next->g, g.N, next->eps,
                       next->oh, next->ol);
    return hipGetLastError();
  }
  g.kper = g.K / nsplit;
  g.part = part;
  g.part_stride = (size_t)MK_PT * g.ldc;
  hipError_t e = launch_gemm_t<EPI_PART, 2, 2, 2, 4, 4>(g, nsplit, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pf_reduce_norm, dim3(g.M), dim3(PF_THREADS), 0, st, g.c, (const float *)part, nsplit, g.part_stride,
                     g.N, next ? next->g : (const float *)nullptr, next ? next->eps : 0.f,
                     next ? next->oh : (uint16_t *)nullptr, next ? next->ol : (uint16_t *)nullptr);
  return hipGetLastError();
}

static size_t chunk_prep_lds(int dk) { return (size_t)(3 * MK_CHUNK * (dk + 4) + 3 * MK_CHUNK * CS + 3 * 16 * 17 + 4 * MK_CHUNK) * 4; }
static size_t scan_lds(int dk) { return (size_t)(16 * (dk + 4) + 16 * (MK_CHUNK + 4) + 4 * 64 * 4) * 4; }

// One pass of a prompt is enqueued as row blocks: block b holds pass rows [r0, r0 + T) and its
// kernels see pointers into the pass buffers offset to row r0 and positions offset by r0.  With
// two blocks the second runs on a side stream one step behind the first: its layer l waits only
// for the first block's state of layer l (after the delta-rule scan: the state S and the conv
// inputs in the ring; after the KV append: the keys and values of the earlier rows), so the two
// blocks' kernels overlap.  Every buffer of a pass is indexed by row (or by chunk, or in 16-row
// operand blocks), so the blocks touch disjoint parts of it; r0 is a multiple of the delta-rule
// chunk, which keeps the chunk boundaries, and with them every result, those of one block.
struct PfBlk {
  int r0, T;
  bool first;   // the pass's first block (replays the pending updates of a verify forward)
};
enum { PF_NONE = 0, PF_RECORD = 1, PF_WAIT = 2 };

static hipError_t enqueue_layer(const MkDev *d, const MkLayerDev &L, const MkPfW &PW, const MkLayerDev *next,
                                const MkPf *pf, const PfBlk &b, hipStream_t st, int sync, hipEvent_t ev) {
  const int H = d->H, nh = d->nh, dk = d->dk, dv = d->dv, nq = d->nq, nkv = d->nkv, hd = d->hd, I = d->I;
  const int r0 = b.r0, T = b.T;
  const size_t rH = (size_t)r0 * H, rK = (size_t)r0 * pf->K1;
  uint16_t *a1h = pf->a1h + rK, *a1l = pf->a1l + rK;   // operand blocks of width H, nh dv or nq hd (<= K1)
  float *P = pf->P + (size_t)r0 * pf->NP, *X = pf->X + rH, *part = pf->part + rH;
  // the norm after the mixer (FFN input) and after the FFN (next layer's input) run inside the
  // split-K reductions of the projections that add into the residual stream
  const PfNext n2{L.ln2, d->rms_eps, a1h, a1l};
  const PfNext n1{next ? next->ln1 : nullptr, d->rms_eps, a1h, a1l};
  PfGemm g{};
  g.ah = a1h; g.al = a1l; g.M = T;
  hipError_t e;
  if (L.kind == 0) {
    g.N = nh * d->r_in; g.K = H;
    g.c = P; g.ldc = pf->NP; g.w = PW.in;
    if ((e = launch_gemm(EPI_STORE, g, nullptr, st)) != hipSuccess) return e;
    if (sync == PF_WAIT && (e = hipStreamWaitEvent(st, ev, 0)) != hipSuccess) return e;
    const int nchunk = (T + MK_CHUNK - 1) / MK_CHUNK;
    const size_t rc = (size_t)r0 * dk;   // chunk terms: (r0 / CHUNK) chunks of CHUNK x dk
    // dk == dv in {64, 128} (checked when the model is loaded).  The conv (in the chunk kernel)
    // reads the ring (conv inputs of earlier positions) before the scan overwrites it with this
    // block's last ones.
    PfChunk ck{P, pf->NP, d->r_in, d->C, nh, L.dn_conv, L.ring, d->ctl, d->l2_eps, r0,
               pf->cW + rc, pf->cQ + rc, pf->cU + rc, pf->cO + rc, pf->cKt + rc, pf->cg + r0, pf->cd + r0, T};
    PfScan sc{L.S, L.pend, d->ctl, pf->cW + rc, pf->cU + rc, pf->cKt + rc, pf->cg + r0, pf->cd + r0,
              pf->snap + (size_t)(r0 / MK_CHUNK) * dv * dk, T, nh, P, pf->NP, d->r_in, d->C, L.ring, r0, b.first ? 1 : 0};
    PfOut po{pf->cQ + rc, pf->cO + rc, pf->snap + (size_t)(r0 / MK_CHUNK) * dv * dk, P, pf->NP, d->r_in, L.dn_gnorm, nh,
             d->rms_eps, a1h, a1l, T};
    const dim3 gtok((T + PREP_TB - 1) / PREP_TB, nh);
    if (dk == 128) {
      hipLaunchKernelGGL(pf_dn_chunk_prep<128>, dim3(nh, nchunk, 2), dim3(CP_THREADS), chunk_prep_lds(128), st, ck);
      hipLaunchKernelGGL(pf_dn_scan<128>, dim3(nh, 128 / 16), dim3(SCAN_THREADS), scan_lds(128), st, sc);
    } else {
      hipLaunchKernelGGL(pf_dn_chunk_prep<64>, dim3(nh, nchunk), dim3(CP_THREADS), chunk_prep_lds(64), st, ck);
      hipLaunchKernelGGL(pf_dn_scan<64>, dim3(nh, 64 / 16), dim3(SCAN_THREADS), scan_lds(64), st, sc);
    }
    if (sync == PF_RECORD && (e = hipEventRecord(ev, st)) != hipSuccess) return e;
    if (dk == 128) hipLaunchKernelGGL(pf_dn_out<128>, gtok, dim3(128 * 4), 0, st, po);
    else hipLaunchKernelGGL(pf_dn_out<64>, gtok, dim3(64 * 4), 0, st, po);
    PfGemm go{};
    go.ah = a1h; go.al = a1l; go.M = T; go.N = H; go.K = nh * dv;
    go.c = X; go.ldc = H; go.w = PW.out;
    if ((e = launch_gemm(EPI_RESID, go, part, st, &n2)) != hipSuccess) return e;
  } else {
    g.N = (nq + 2 * nkv) * hd; g.K = H;
    g.c = P; g.ldc = pf->NP; g.w = PW.qkv;
    if ((e = launch_gemm(EPI_STORE, g, nullptr, st)) != hipSuccess) return e;
    PfAtt at{};
    at.P = P; at.NP = pf->NP; at.T = T; at.rope = d->rope; at.page_table = d->page_table; at.ctl = d->ctl;
    at.kc = L.kc; at.vc = L.vc; at.kve = L.kve; at.kvq = d->kv_quant;
    at.aq = pf->aq + (size_t)r0 * nq * hd; at.nq = nq; at.nkv = nkv; at.hd = hd;
    at.oh = a1h; at.ol = a1l; at.pofs = r0;
    hipLaunchKernelGGL(pf_att_rope, dim3(T), dim3(PF_THREADS), 0, st, at);
    if (sync == PF_RECORD && (e = hipEventRecord(ev, st)) != hipSuccess) return e;
    if (sync == PF_WAIT && (e = hipStreamWaitEvent(st, ev, 0)) != hipSuccess) return e;
    const dim3 ga((T + 63) / 64, nq);
    if (hd == 128 && !at.kvq) hipLaunchKernelGGL((pf_att_mfma<128, false>), ga, dim3(PF_THREADS), 0, st, at);
    else if (hd == 128) hipLaunchKernelGGL((pf_att_mfma<128, true>), ga, dim3(PF_THREADS), 0, st, at);
    else if (hd == 64 && !at.kvq) hipLaunchKernelGGL((pf_att_mfma<64, false>), ga, dim3(PF_THREADS), 0, st, at);
    else if (hd == 64) hipLaunchKernelGGL((pf_att_mfma<64, true>), ga, dim3(PF_THREADS), 0, st, at);
    else return hipErrorInvalidValue;   // head_dim is 64 or 128 (checked at load)
    PfGemm go{};
    go.ah = a1h; go.al = a1l; go.M = T; go.N = H; go.K = nq * hd;
    go.c = X; go.ldc = H; go.w = PW.o;
    if ((e = launch_gemm(EPI_RESID, go, part, st, &n2)) != hipSuccess) return e;
  }
  PfGemm gu{};
  gu.ah = a1h; gu.al = a1l; gu.M = T; gu.N = 2 * I; gu.K = H;
  gu.w = PW.gu;
  gu.oh = pf->a2h + (size_t)r0 * I; gu.ol = pf->a2l + (size_t)r0 * I; gu.ldo = I;
  if ((e = launch_gemm(EPI_SWIGLU, gu, nullptr, st)) != hipSuccess) return e;
  PfGemm gd{};
  gd.ah = gu.oh; gd.al = gu.ol; gd.M = T; gd.N = H; gd.K = I;
  gd.w = PW.dn;
  gd.c = X; gd.ldc = H;
  return launch_gemm(EPI_RESID, gd, part, st, n1.g ? &n1 : nullptr);
}

// Enqueue the prefill of n tokens (device buffer) on the stream.  layers_host: the layer table;
// pfw: per layer, the prefill copies of its projection weights.
// side / ev (nullable): a second stream and d->n_layers + 2 events for the two-block form; a
// pass of fewer than PF_SPLIT_MIN rows, or max_blocks 1, runs as one block on st.
constexpr int PF_SPLIT_MIN = 256;
extern "C" hipError_t mk_prefill_enqueue(const MkDev *d, const MkLayerDev *layers_host, const MkPf *pf,
                                         const int32_t *tokens, int n, int32_t *argmax, float *logits,
                                         hipStream_t st, hipStream_t side, hipEvent_t *ev, int max_blocks,
                                         const MkPfW *pfw) {
  static bool attr_done = false;
  if (!attr_done) {
    hipError_t e;
    if ((e = hipFuncSetAttribute((const void *)pf_dn_chunk_prep<64>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)chunk_prep_lds(64))) != hipSuccess) return e;
    if ((e = hipFuncSetAttribute((const void *)pf_dn_chunk_prep<128>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)chunk_prep_lds(128))) != hipSuccess) return e;
    if ((e = hipFuncSetAttribute((const void *)pf_dn_scan<64>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)scan_lds(64))) != hipSuccess) return e;
    if ((e = hipFuncSetAttribute((const void *)pf_dn_scan<128>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)scan_lds(128))) != hipSuccess) return e;
    attr_done = true;
  }
  const int H = d->H, NL = d->n_layers;
  for (int s0 = 0; s0 < n; s0 += MK_PT) {
    const int T = n - s0 < MK_PT ? n - s0 : MK_PT;
    const bool last = s0 + T == n;
    const bool two = side && ev && max_blocks >= 2 && T >= PF_SPLIT_MIN;
    // split at a chunk boundary near the middle (both blocks >= 128 rows)
    const int r1 = two ? (T / 2) / MK_CHUNK * MK_CHUNK : T;
    PfBlk blk[2] = {{0, r1, true}, {r1, T - r1, false}};
    const int nb = two ? 2 : 1;
    hipError_t e;
    if (two) {   // the side stream starts after everything enqueued on st before this pass
      if ((e = hipEventRecord(ev[NL], st)) != hipSuccess) return e;
      if ((e = hipStreamWaitEvent(side, ev[NL], 0)) != hipSuccess) return e;
    }
    for (int bi = 0; bi < nb; ++bi) {
      const PfBlk &b = blk[bi];
      hipStream_t sb = bi ? side : st;
      hipLaunchKernelGGL(pf_embed, dim3(b.T), dim3(PF_THREADS), 0, sb, d->embed, tokens + s0 + b.r0, H, d->V,
                         pf->X + (size_t)b.r0 * H, d->ctl);
      hipLaunchKernelGGL(pf_norm_split, dim3(b.T), dim3(PF_THREADS), 0, sb, (const float *)pf->X + (size_t)b.r0 * H,
                         layers_host[0].ln1, H, d->rms_eps, pf->a1h + (size_t)b.r0 * pf->K1,
                         pf->a1l + (size_t)b.r0 * pf->K1);
    }
    for (int li = 0; li < NL; ++li) {
      const MkLayerDev *next = li + 1 < NL ? &layers_host[li + 1] : nullptr;
      for (int bi = 0; bi < nb; ++bi) {
        const int sync = !two ? PF_NONE : bi == 0 ? PF_RECORD : PF_WAIT;
        if ((e = enqueue_layer(d, layers_host[li], pfw[li], next, pf, blk[bi], bi ? side : st, sync,
                               two ? ev[li] : nullptr)) != hipSuccess)
          return e;
      }
    }
    if (two) {   // st continues after the side stream's last layer
      if ((e = hipEventRecord(ev[NL + 1], side)) != hipSuccess) return e;
      if ((e = hipStreamWaitEvent(st, ev[NL + 1], 0)) != hipSuccess) return e;
    }
    if (last) {
      hipLaunchKernelGGL(pf_lm, dim3(MK_NWG), dim3(PF_THREADS), 0, st, (const float *)pf->X, T - 1, d->lnf, d->rms_eps,
                         d->embed, d->V, H, logits, pf->lmbest, d->ctl);
      hipLaunchKernelGGL(pf_finish, dim3(1), dim3(64), 0, st, (const unsigned long long *)pf->lmbest, MK_NWG, argmax,
                         d->ctl, T);
    } else {
      hipLaunchKernelGGL(pf_finish, dim3(1), dim3(64), 0, st, (const unsigned long long *)pf->lmbest, 0,
                         (int32_t *)nullptr, d->ctl, T);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}
