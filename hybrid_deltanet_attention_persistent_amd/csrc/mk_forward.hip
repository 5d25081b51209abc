// mk_forward.hip -- persistent single-launch forward pass of the hybrid Gated-DeltaNet +
// attention decoder on MI355X (gfx950): one decode step, one multi-token verify
// forward, or a prompt processed token by token, each in one cooperative launch.
//
// What it computes: the launch page "OS Megakernel that match M5 Max Tok/w at 2x
// the Throughput on RTX 3090" (section "We wrote a single CUDA kernel that runs
// the entire forward pass in one dispatch": every layer in one dispatch, BF16
// weights with FP32 accumulation, the DeltaNet recurrence in FP32 registers,
// attention fused from QKV through RoPE and causal softmax to the output
// projection, grid-wide synchronisation instead of launches).
//
// How (MI355X-first, not the page's design):
//   * 256 workgroups x 512 threads, one per CU; workgroup b lives on XCD b % 8.
//   * No grid barrier.  Every hand-off is a tagged exchange slot {value, tag}
//     written once per forward; a consumer polls the slots it needs until every
//     tag equals the forward's tag.  Slots are written and read with
//     device-coherent (sc1) 64-bit stores and loads.
//   * XCD x owns DeltaNet head x / query head x and FFN intermediate slice x, so
//     in-projection -> conv -> delta rule -> gated norm -> out-projection stay
//     inside one XCD; the out-projection and the FFN down-projection are split
//     over XCDs along their input dimension, and the residual stream is rebuilt
//     by a reduce-scatter (over XCDs) + all-gather (inside the XCD) per sublayer.
//   * Weights are streamed once per forward in a tile layout that makes every
//     wave load a contiguous 1 KiB (see mk_layout.h).
//   * Decode and verify use the same per-column arithmetic in the same order, so
//     a verify forward's logits are bit-identical to sequential decode steps.
#include <hip/hip_runtime.h>
#include <math.h>
#include "mk_layout.h"

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define MK_WAIT_TICKS 20000000ull   // watchdog: 0.2 s of the 100 MHz device wall clock
// Hand-offs inside one XCD use the same device-coherent (sc1) loads as those between XCDs:
// polling through the XCD's L2 alone (sc0) did not observe peers' stores reliably here.
#define AUX_L2 16
#define AUX_DEV 16                  // sc1: device-coherent
#define RSRC_W3 0x00020000

// ------------------------------------------------------------------------------ helpers
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

__device__ __forceinline__ uint32_t f2bf(float f) {  // round to nearest even
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float rbf(float f) { return __uint_as_float(f2bf(f) << 16); }
__device__ __forceinline__ float bfv(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ void unpack8(const u32x4 &w, float f[8]) {
  f[0] = __uint_as_float(w.x << 16); f[1] = __uint_as_float(w.x & 0xffff0000u);
  f[2] = __uint_as_float(w.y << 16); f[3] = __uint_as_float(w.y & 0xffff0000u);
  f[4] = __uint_as_float(w.z << 16); f[5] = __uint_as_float(w.z & 0xffff0000u);
  f[6] = __uint_as_float(w.w << 16); f[7] = __uint_as_float(w.w & 0xffff0000u);
}

__device__ __forceinline__ float sigmoidf_(float x) {
  if (x >= 0.f) return 1.f / (1.f + expf(-x));
  const float e = expf(x);
  return e / (1.f + e);
}
__device__ __forceinline__ float siluf_(float x) { return x * sigmoidf_(x); }
__device__ __forceinline__ float softplusf_(float x) { return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ float group_sum(float v, int G) {  // butterfly over aligned groups of G lanes
  for (int off = G >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
// Sum of one value per thread over the workgroup, fixed order; red: >= MK_WAVES floats of LDS.
__device__ __forceinline__ float block_sum(float v, float *red) {
  v = wave_sum(v);
  if (lane_id() == 0) red[wave_id()] = v;
  __syncthreads();
  float s = red[0];
#pragma unroll
  for (int w = 1; w < MK_WAVES; ++w) s += red[w];
  __syncthreads();
  return s;
}

// tagged exchange slot: 8 bytes {float bits, tag}, written with one device-coherent 64-bit store
__device__ __forceinline__ void pub_l2(uint2 *p, float v, uint32_t tag) {
  __hip_atomic_store(reinterpret_cast<unsigned long long *>(p), ((unsigned long long)tag << 32) | __float_as_uint(v),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void pub_dev(uint2 *p, float v, uint32_t tag) {
  __hip_atomic_store(reinterpret_cast<unsigned long long *>(p),
                     ((unsigned long long)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// Gather a [nrow][ncol] block of tagged slots (row stride `stride` slots, ncol even)
// into dst[nrow][ncol] (LDS), polling until every tag equals `tag`.  All threads
// call it; ends with a barrier.  Returns false on watchdog expiry.
template <int AUX>
__device__ bool gather2d(const uint2 *src, int nrow, int ncol, int stride, uint32_t tag, float *dst,
                         int *fail, int32_t *ctl, int site) {
  const int half = ncol >> 1;
  const int nchunk = nrow * half;
  const uint32_t bytes = (uint32_t)(((nrow - 1) * stride + ncol) * 8);
  __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)src, 0, bytes, RSRC_W3);
  const int tid = threadIdx.x;
  uint32_t pend = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (tid + j * MK_THREADS < nchunk) pend |= 1u << j;
  if (pend) {
    const unsigned long long deadline = wall_clock64() + MK_WAIT_TICKS;
    while (true) {
      u32x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (pend & (1u << j)) {
          const int c = tid + j * MK_THREADS;
          const int r = c / half, q = c - r * half;
          v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, (r * stride + 2 * q) * 8, 0, AUX);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if ((pend & (1u << j)) && v[j].y == tag && v[j].w == tag) {
          const int c = tid + j * MK_THREADS;
          const int r = c / half, q = c - r * half;
          dst[r * ncol + 2 * q] = __uint_as_float(v[j].x);
          dst[r * ncol + 2 * q + 1] = __uint_as_float(v[j].z);
          pend &= ~(1u << j);
        }
      }
      if (!pend) break;
      if (wall_clock64() > deadline) {
        *fail = 1;
        // record the first expiry on the device: where, who, and the tag still found there
        uint32_t seen = 0;
#pragma unroll
        for (int j = 7; j >= 0; --j)
          if (pend & (1u << j)) seen = v[j].y;
        int expect = 0;
        if (__hip_atomic_compare_exchange_strong(ctl + MK_CTL_WHERE, &expect, site | (1 << 30), __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
          __hip_atomic_store(ctl + MK_CTL_WHERE + 1, (int)(blockIdx.x * 65536 + threadIdx.x), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(ctl + MK_CTL_WHERE + 2, (int)seen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(ctl + MK_CTL_WHERE + 3, (int)tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
  return *fail == 0;
}

// ------------------------------------------------------------------------------ GEMV on tiles
template <int LMAX>
__device__ __forceinline__ void rg_load(const uint16_t *tile, int rg, int L, u32x4 (&w)[LMAX]) {
  const u32x4 *p = reinterpret_cast<const u32x4 *>(tile) + (size_t)rg * L * 64 + lane_id();
#pragma unroll
  for (int i = 0; i < LMAX; ++i)
    if (i < L) w[i] = __builtin_nontemporal_load(p + i * 64);
}

// Dot products of one row group with NCOL activation vectors act[c*astride + k];
// returns each lane's row result (valid in every lane of the row's G-lane segment).
template <int NCOL, int LMAX>
__device__ __forceinline__ void rg_dot(const u32x4 (&w)[LMAX], int L, int G, const float *act, int astride,
                                       int n, float (&out)[NCOL]) {
  const int kl = (lane_id() & (G - 1)) * 8;
#pragma unroll
  for (int c = 0; c < NCOL; ++c) out[c] = 0.f;
#pragma unroll
  for (int i = 0; i < LMAX; ++i) {
    if (i < L) {
      float f[8];
      unpack8(w[i], f);
      const int k0 = i * G * 8 + kl;
#pragma unroll
      for (int c = 0; c < NCOL; ++c) {
        if (c < n) {
          const float4 a0 = *reinterpret_cast<const float4 *>(act + c * astride + k0);
          const float4 a1 = *reinterpret_cast<const float4 *>(act + c * astride + k0 + 4);
          float s = out[c];
          s = fmaf(f[0], a0.x, s); s = fmaf(f[1], a0.y, s); s = fmaf(f[2], a0.z, s); s = fmaf(f[3], a0.w, s);
          s = fmaf(f[4], a1.x, s); s = fmaf(f[5], a1.y, s); s = fmaf(f[6], a1.z, s); s = fmaf(f[7], a1.w, s);
          out[c] = s;
        }
      }
    }
  }
#pragma unroll
  for (int c = 0; c < NCOL; ++c) out[c] = group_sum(out[c], G);
}

// RMSNorm of src[c][H] into dst[c][H] with gain g.
template <int NCOL>
__device__ void rmsnorm_cols(const float *src, float *dst, const float *g, int H, float eps, int n, float *red) {
  for (int c = 0; c < NCOL; ++c) {
    if (c >= n) break;
    float s = 0.f;
    for (int k = threadIdx.x; k < H; k += MK_THREADS) s = fmaf(src[c * H + k], src[c * H + k], s);
    const float tot = block_sum(s, red);
    const float den = sqrtf(tot / (float)H + eps);
    for (int k = threadIdx.x; k < H; k += MK_THREADS) {
      dst[c * H + k] = src[c * H + k] / den * g[k];
    }
  }
  __syncthreads();
}

// loop over the live columns with compile-time indices (register arrays stay in registers)
#define FOR_COL(c) _Pragma("unroll") for (int c = 0; c < NCOL; ++c) if (c < ncol)

// ------------------------------------------------------------------------------ shared memory map
struct Lds {
  float *xres, *hn, *work, *red;
  int *flag;
};

// ------------------------------------------------------------------------------ the kernel
// On a watchdog expiry the whole workgroup records the error and leaves; the other
// workgroups then time out on its missing outputs and leave too.
#define MK_BAIL()                                                                                   \
  do {                                                                                              \
    if (tid == 0)                                                                                   \
      __hip_atomic_fetch_or(m.ctl + MK_CTL_ERR, MK_DERR_HANG, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); \
    return;                                                                                         \
  } while (0)

template <int NCOL, bool PROMPT>
__global__ void __launch_bounds__(MK_THREADS, 1) mk_forward(MkLaunch a) {
  extern __shared__ float lds_raw[];
  const MkDev &m = a.m;
  const int b = blockIdx.x, x = b & (MK_NX - 1), lw = b >> 3;
  const int w8 = wave_id(), lane = lane_id(), tid = threadIdx.x;
  const int wx = lw * MK_WAVES + w8;  // wave index inside the XCD, 0..255
  const int H = m.H;

  Lds L;
  L.xres = lds_raw;
  L.hn = L.xres + NCOL * H;
  L.work = L.hn + NCOL * H;
  L.red = L.work + 8192;
  L.flag = reinterpret_cast<int *>(L.red + 64);
  if (tid == 0) {
    L.flag[0] = 0;
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    if ((int)(xcc & 7) != x) __hip_atomic_fetch_or(m.ctl + MK_CTL_ERR, MK_DERR_XCD, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();

  const int ctl_pos = __hip_atomic_load(m.ctl + MK_CTL_POS, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  int pend_n = __hip_atomic_load(m.ctl + MK_CTL_PEND, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int par = __hip_atomic_load(m.ctl + MK_CTL_PAR, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const bool verify = !a.prefill && a.n > 1;
  const int nsteps = a.prefill ? a.n : 1;
  const int ncol = a.prefill ? 1 : a.n;
  // prompts written in this launch are read back by other XCDs in later steps of it
  const bool kv_live = a.prefill != 0;
  const int G_h = mk_tile_G(H), L_h = H / 8 / G_h, RG_h = 64 / G_h;
  const int SL = H / MK_NL;  // residual slice per workgroup in the reductions

  for (int step = 0; step < nsteps; ++step) {
    const uint32_t tag = a.tag0 + step;
    const int pos0 = ctl_pos + step;       // position of column 0
    const bool last_step = step == nsteps - 1;

    // ---- embedding rows
    for (int c = 0; c < ncol; ++c) {
      int t = a.tokens[a.prefill ? step : c];
      if (t < 0 || t >= m.V) {
        if (tid == 0) __hip_atomic_fetch_or(m.ctl + MK_CTL_ERR, MK_DERR_TOKEN, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        t = 0;
      }
      const uint16_t *row = m.embed + (size_t)t * H;
      for (int k = tid; k < H; k += MK_THREADS) L.xres[c * H + k] = bfv(row[k]);
    }
    __syncthreads();

    for (int li = 0; li < m.n_layers; ++li) {
      // the layer table is read-only: reading it through the constant address space gives
      // scalar loads, so every pointer below is known to be wave-uniform
      typedef const __attribute__((address_space(4))) MkLayerDev ConstLayer;
      ConstLayer &ly = ((ConstLayer *)(uintptr_t)m.layers)[li];
      const uint32_t tg = tag;
      // ================================================================ mixer
      rmsnorm_cols<NCOL>(L.xres, L.hn, ly.ln1, H, m.rms_eps, ncol, L.red);
      if (ly.kind == 0) {
        // ------------------------------------------------ D1: in-projection rows of head x
        const int nh = m.nh, dk = m.dk, dv = m.dv, r_in = m.r_in;
        uint2 *xin = ly.x_in + (size_t)x * MK_MAXCOL * m.r_in_max;
        if (x < nh) {
          const uint16_t *tile = ly.dn_in + (size_t)x * r_in * H;
          const int nrg = r_in / RG_h;
          for (int rg = wx; rg < nrg; rg += MK_NL * MK_WAVES) {
            u32x4 wr[2];
            rg_load<2>(tile, rg, L_h, wr);
            float o[NCOL];
            rg_dot<NCOL, 2>(wr, L_h, G_h, L.hn, H, ncol, o);
            if ((lane & (G_h - 1)) == 0) {
              const int row = rg * RG_h + lane / G_h;
              FOR_COL(c) pub_l2(xin + c * m.r_in_max + row, o[c], tg);
            }
          }
        }
        // ------------------------------------------------ D2: conv, norms, gates, delta rule
        const int RW = dv / MK_NL, r0 = lw * RW;
        const int HPR = dk / 64;  // waves per state row
        float *qk = L.work;                       // [NCOL][2dk]
        float *vr = qk + NCOL * 2 * dk;           // [NCOL][RWp]
        const int RWp = RW < 2 ? 2 : RW;
        float *ab = vr + NCOL * RWp;              // [NCOL][2]
        float *nrm = ab + NCOL * 2;               // [NCOL][2] 1/den of q, k
        float *gts = nrm + NCOL * 2;              // [NCOL][2] alpha, beta
        float *ored = gts + NCOL * 2;             // [16] row-partial exchange
        if (x < nh) {
          for (int c = 0; c < ncol; ++c) {
            if (!gather2d<AUX_L2>(xin + c * m.r_in_max, 1, 2 * dk, 0, tg, qk + c * 2 * dk, L.flag, m.ctl, (step << 16) | (li << 8) | 1)) MK_BAIL();
            if (!gather2d<AUX_L2>(xin + c * m.r_in_max + 2 * dk + r0, 1, RWp, 0, tg, vr + c * RWp, L.flag, m.ctl, (step << 16) | (li << 8) | 2)) MK_BAIL();
            if (!gather2d<AUX_L2>(xin + c * m.r_in_max + 2 * dk + 2 * dv, 1, 2, 0, tg, ab + c * 2, L.flag, m.ctl, (step << 16) | (li << 8) | 3)) MK_BAIL();
          }
          // conv + SiLU: threads [0, 2dk) are q/k channels of head x, [2dk, 2dk+RW) my v channels
          {
            const int nch = 2 * dk + RW;
            if (tid < nch) {
              int ch;
              float *cur;  // column stride cstride
              int cstride;
              if (tid < 2 * dk) {
                ch = (tid < dk) ? x * dk + tid : nh * dk + x * dk + (tid - dk);
                cur = qk + tid;
                cstride = 2 * dk;
              } else {
                ch = 2 * nh * dk + x * dv + r0 + (tid - 2 * dk);
                cur = vr + (tid - 2 * dk);
                cstride = RWp;
              }
              const float w0 = ly.dn_conv[ch * 4 + 0], w1 = ly.dn_conv[ch * 4 + 1];
              const float w2 = ly.dn_conv[ch * 4 + 2], w3 = ly.dn_conv[ch * 4 + 3];
              float raw[NCOL];
#pragma unroll
              for (int c = 0; c < NCOL; ++c) raw[c] = (c < ncol) ? cur[c * cstride] : 0.f;
              float hist[3];
              {
                __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(ly.ring, 0, MK_RING * m.C * 4, RSRC_W3);
#pragma unroll
                for (int i = 0; i < 3; ++i) {
                  const int pp = pos0 - 3 + i;
                  hist[i] = (pp >= 0) ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                                            rr, ((pp & (MK_RING - 1)) * m.C + ch) * 4, 0, AUX_L2))
                                      : 0.f;
                }
              }
              const float wt[4] = {w0, w1, w2, w3};
              FOR_COL(c) {
                float s = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const int back = 3 - i;              // tap i meets the token `back` steps before column c
                  const int cc = c - back;
                  const float v = (cc >= 0) ? raw[cc < 0 ? 0 : cc] : hist[cc + 3 < 0 ? 0 : cc + 3];
                  s = fmaf(wt[i], v, s);
                }
                cur[c * cstride] = siluf_(s);
              }
              if (tid >= 2 * dk || lw == 0)
                FOR_COL(c) ly.ring[((pos0 + c) & (MK_RING - 1)) * m.C + ch] = raw[c];
            }
          }
          __syncthreads();
          // L2 norms of q and k (wave w handles ranges w, w+8, ...), gates
          for (int r = w8; r < 2 * ncol; r += MK_WAVES) {
            const int c = r >> 1, which = r & 1;
            const float *p = qk + c * 2 * dk + which * dk;
            float s = 0.f;
            for (int i = lane; i < dk; i += 64) s = fmaf(p[i], p[i], s);
            s = wave_sum(s);
            if (lane == 0) nrm[c * 2 + which] = sqrtf(s + m.l2_eps);
          }
          if (tid < ncol) {
            gts[tid * 2 + 0] = expf(-softplusf_(ab[tid * 2 + 0]));
            gts[tid * 2 + 1] = sigmoidf_(ab[tid * 2 + 1]);
          }
          __syncthreads();
          for (int i = tid; i < ncol * 2 * dk; i += MK_THREADS) qk[i] = qk[i] / nrm[(i / (2 * dk)) * 2 + ((i % (2 * dk)) >= dk)];
          __syncthreads();

          // delta rule on my RW rows: wave w -> row w / HPR, lanes -> element (w % HPR)*64 + lane
          const int rr = w8 / HPR, e = (w8 % HPR) * 64 + lane;
          const bool act = rr < RW;
          float *Srow = ly.S + ((size_t)x * dv + r0 + (act ? rr : 0)) * dk;
          float s = act ? Srow[e] : 0.f;
          const float *pk_base = ly.pend + (size_t)par * nh * MK_MAXCOL * (dk + dv + 2) + (size_t)x * MK_MAXCOL * (dk + dv + 2);
          auto rowsum = [&](float v) -> float {
            v = wave_sum(v);
            if (lane == 0) ored[w8] = v;
            __syncthreads();
            float t = 0.f;
            if (act) {
              t = ored[rr * HPR];
              for (int hh = 1; hh < HPR; ++hh) t += ored[rr * HPR + hh];
            }
            __syncthreads();
            return t;
          };
          // pending updates left by a verify forward: replay the accepted ones
          for (int j = 0; j < pend_n; ++j) {
            const float *pk = pk_base + j * (dk + dv + 2);
            const float kj = pk[e < dk ? e : 0];
            const float vj = pk[dk + r0 + (act ? rr : 0)];
            const float aj = pk[dk + dv], bj = pk[dk + dv + 1];
            const float sk = rowsum(act ? s * kj : 0.f);
            const float u = bj * (vj - aj * sk);
            s = fmaf(u, kj, aj * s);
          }
          if (verify && act) Srow[e] = s;  // S after the accepted tokens; this forward's tokens become pending
          float *outo = L.work + 4096;     // [NCOL][RWp] o rows
          for (int c = 0; c < ncol; ++c) {
            const float kc = qk[c * 2 * dk + dk + (e < dk ? e : 0)];
            const float qc = qk[c * 2 * dk + (e < dk ? e : 0)];
            const float al = gts[c * 2 + 0], be = gts[c * 2 + 1];
            const float vv = act ? vr[c * RWp + rr] : 0.f;
            const float sk = rowsum(act ? s * kc : 0.f);
            const float u = be * (vv - al * sk);
            s = fmaf(u, kc, al * s);
            const float o = rowsum(act ? s * qc : 0.f);
            if (act && (w8 % HPR) == 0 && lane == 0) outo[c * RWp + rr] = o;
          }
          if (!verify && act) Srow[e] = s;
          if (verify) {  // this forward's (k, v, alpha, beta) become the pending updates
            float *pw = ly.pend + (size_t)(par ^ 1) * nh * MK_MAXCOL * (dk + dv + 2) + (size_t)x * MK_MAXCOL * (dk + dv + 2);
            for (int c = 0; c < ncol; ++c) {
              float *pc = pw + c * (dk + dv + 2);
              if (lw == 0) {
                for (int i = tid; i < dk; i += MK_THREADS) pc[i] = qk[c * 2 * dk + dk + i];
                if (tid == 0) { pc[dk + dv] = gts[c * 2]; pc[dk + dv + 1] = gts[c * 2 + 1]; }
              }
              if (tid < RW) pc[dk + r0 + tid] = vr[c * RWp + tid];
            }
          }
          __syncthreads();
          wait_stores();
          {
            uint2 *xo = ly.x_o + (size_t)x * MK_MAXCOL * m.x_o_len;
            if (tid < ncol * RW) {
              const int c = tid / RW, r = tid % RW;
              pub_l2(xo + c * m.x_o_len + r0 + r, outo[c * RWp + r], tg);
            }
          }
        }
        // ------------------------------------------------ D3: gated RMSNorm + out-projection slice
        {
          uint2 *xmix = ly.x_mix;
          const int G_o = mk_tile_G(dv), L_o = dv / 8 / G_o, RG_o = 64 / G_o;
          if (x < nh) {
            float *o = L.work;              // [NCOL][dv]
            float *z = o + NCOL * dv;       // [NCOL][dv]
            uint2 *xo = ly.x_o + (size_t)x * MK_MAXCOL * m.x_o_len;
            for (int c = 0; c < ncol; ++c) {
              if (!gather2d<AUX_L2>(xo + c * m.x_o_len, 1, dv, 0, tg, o + c * dv, L.flag, m.ctl, (step << 16) | (li << 8) | 4)) MK_BAIL();
              if (!gather2d<AUX_L2>(xin + c * m.r_in_max + 2 * dk + dv, 1, dv, 0, tg, z + c * dv, L.flag, m.ctl, (step << 16) | (li << 8) | 5)) MK_BAIL();
            }
            for (int c = 0; c < ncol; ++c) {
              float sq = 0.f;
              for (int i = tid; i < dv; i += MK_THREADS) sq = fmaf(o[c * dv + i], o[c * dv + i], sq);
              const float den = sqrtf(block_sum(sq, L.red) / (float)dv + m.rms_eps);
              for (int i = tid; i < dv; i += MK_THREADS) {
                o[c * dv + i] = o[c * dv + i] / den * ly.dn_gnorm[i] * siluf_(z[c * dv + i]);
              }
            }
            __syncthreads();
            const uint16_t *tile = ly.dn_out + (size_t)x * H * dv;
            const int nrg = H / RG_o;
            for (int rg = wx; rg < nrg; rg += MK_NL * MK_WAVES) {
              u32x4 wr[2];
              rg_load<2>(tile, rg, L_o, wr);
              float oo[NCOL];
              rg_dot<NCOL, 2>(wr, L_o, G_o, o, dv, ncol, oo);
              if ((lane & (G_o - 1)) == 0) {
                const int row = rg * RG_o + lane / G_o;
                FOR_COL(c) pub_dev(xmix + ((size_t)c * MK_NX + x) * H + row, oo[c], tg);
              }
            }
          } else {
            for (int i = tid + lw * MK_THREADS; i < H; i += MK_NL * MK_THREADS)
              for (int c = 0; c < ncol; ++c) pub_dev(xmix + ((size_t)c * MK_NX + x) * H + i, 0.f, tg);
          }
        }
      } else {
        // ================================================ attention layer
        const int nq = m.nq, nkv = m.nkv, hd = m.hd;
        const int kvh = x * nkv / (nq > 0 ? nq : 1);
        uint2 *xin = ly.x_in + (size_t)x * MK_MAXCOL * m.r_in_max;
        uint2 *xo = ly.x_o + (size_t)x * MK_MAXCOL * m.x_o_len;
        uint2 *xmix = ly.x_mix;
        if (x < nq) {
          // ------------------------------------------------ A1: q rows of head x, k/v rows of its kv head
          const int per = hd / RG_h;
          const int nunits = 3 * per;
          for (int u = wx; u < nunits; u += MK_NL * MK_WAVES) {
            const int t = u / per, rg = u - t * per;
            const uint16_t *tile = (t == 0) ? ly.at_q + (size_t)x * hd * H
                                 : (t == 1) ? ly.at_k + (size_t)kvh * hd * H
                                            : ly.at_v + (size_t)kvh * hd * H;
            u32x4 wr[2];
            rg_load<2>(tile, rg, L_h, wr);
            float o[NCOL];
            rg_dot<NCOL, 2>(wr, L_h, G_h, L.hn, H, ncol, o);
            if ((lane & (G_h - 1)) == 0) {
              const int row = t * hd + rg * RG_h + lane / G_h;
              FOR_COL(c) pub_l2(xin + c * m.r_in_max + row, o[c], tg);
            }
          }
          // ------------------------------------------------ A2: RoPE, KV append, split-KV partials
          float *qkv = L.work;                    // [NCOL][3hd]
          for (int c = 0; c < ncol; ++c)
            if (!gather2d<AUX_L2>(xin + c * m.r_in_max, 1, 3 * hd, 0, tg, qkv + c * 3 * hd, L.flag, m.ctl, (step << 16) | (li << 8) | 6)) MK_BAIL();
          {
            const int half = hd / 2;
            for (int i = tid; i < ncol * half; i += MK_THREADS) {
              const int c = i / half, d = i - c * half;
              const float cs = m.rope[((size_t)(pos0 + c) * half + d) * 2 + 0];
              const float sn = m.rope[((size_t)(pos0 + c) * half + d) * 2 + 1];
              float *q = qkv + c * 3 * hd, *k = q + hd, *v = k + hd;
              const float q1 = q[d], q2 = q[d + half], k1 = k[d], k2 = k[d + half];
              q[d] = q1 * cs - q2 * sn;
              q[d + half] = q2 * cs + q1 * sn;
              k[d] = rbf(k1 * cs - k2 * sn); k[d + half] = rbf(k2 * cs + k1 * sn);
              v[d] = rbf(v[d]); v[d + half] = rbf(v[d + half]);
            }
          }
          __syncthreads();
          if (lw == 0 && (x * nkv) % nq == 0) {   // first query head of the kv group appends K, V
            const __amdgpu_buffer_rsrc_t kst = __builtin_amdgcn_make_buffer_rsrc(ly.kc, 0, 0x7fffffff, RSRC_W3);
            const __amdgpu_buffer_rsrc_t vst = __builtin_amdgcn_make_buffer_rsrc(ly.vc, 0, 0x7fffffff, RSRC_W3);
            for (int i = tid; i < ncol * hd; i += MK_THREADS) {
              const int c = i / hd, d = i - c * hd;
              const int p = pos0 + c;
              const size_t off = (((size_t)m.page_table[p / MK_PAGE] * nkv + kvh) * MK_PAGE + (p % MK_PAGE)) * hd + d;
              const uint16_t kb = (uint16_t)(__float_as_uint(qkv[c * 3 * hd + hd + d]) >> 16);
              const uint16_t vb = (uint16_t)(__float_as_uint(qkv[c * 3 * hd + 2 * hd + d]) >> 16);
              __builtin_amdgcn_raw_buffer_store_b16(kb, kst, (uint32_t)(off * 2), 0, AUX_DEV);
              __builtin_amdgcn_raw_buffer_store_b16(vb, vst, (uint32_t)(off * 2), 0, AUX_DEV);
            }
            wait_stores();
          }
          {
            float *sc = L.work + NCOL * 3 * hd;   // scores of my keys [<= 320]
            float *pv = sc + 320;                  // [MK_WAVES][hd] partial P.V per wave
            float *mx = pv + MK_WAVES * hd;        // [2]: max, sum
            const float scale = 1.f / sqrtf((float)hd);
            const int lpk = hd / 8;                // lanes per key
            const int kpw = 64 / lpk;              // keys per wave step
            const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(ly.kc, 0, 0x7fffffff, RSRC_W3);
            const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(ly.vc, 0, 0x7fffffff, RSRC_W3);
            const int kaux = kv_live ? AUX_DEV : 0;
            for (int c = 0; c < ncol; ++c) {
              const int P = pos0 + c;             // query position; keys 0..P
              const int nblk = P / MK_KBLK + 1;
              const int myblk = (nblk > lw) ? (nblk - lw + MK_NL - 1) / MK_NL : 0;
              const int nk = (myblk == 0) ? 0 : (myblk - 1) * MK_KBLK + min(MK_KBLK, P + 1 - (lw + (myblk - 1) * MK_NL) * MK_KBLK);
              const float *q = qkv + c * 3 * hd;
              // scores: key slot ks -> block lw + (ks / 32) * 32, offset ks % 32
              for (int base = w8 * kpw; base < nk; base += MK_WAVES * kpw) {
                const int ks = base + lane / lpk;
                float sdot = 0.f;
                if (ks < nk) {
                  const int tpos = (lw + (ks / MK_KBLK) * MK_NL) * MK_KBLK + (ks % MK_KBLK);
                  const int d0 = (lane % lpk) * 8;
                  float kf[8];
                  if (tpos < pos0) {
                    const uint32_t off = (uint32_t)((((size_t)m.page_table[tpos / MK_PAGE] * nkv + kvh) * MK_PAGE + (tpos % MK_PAGE)) * hd + d0) * 2;
                    u32x4 kw = (kaux == AUX_DEV) ? __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, AUX_DEV)
                                                 : __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0);
                    unpack8(kw, kf);
                  } else {
                    const float *kk = qkv + (tpos - pos0) * 3 * hd + hd + d0;
#pragma unroll
                    for (int i = 0; i < 8; ++i) kf[i] = kk[i];
                  }
#pragma unroll
                  for (int i = 0; i < 8; ++i) sdot = fmaf(q[d0 + i], kf[i], sdot);
                }
                sdot = group_sum(sdot, lpk);
                if (ks < nk && (lane % lpk) == 0) sc[ks] = sdot * scale;
              }
              __syncthreads();
              if (w8 == 0) {
                float mv = -INFINITY;
                for (int i = lane; i < nk; i += 64) mv = fmaxf(mv, sc[i]);
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) mv = fmaxf(mv, __shfl_xor(mv, off, 64));
                if (lane == 0) mx[0] = mv;
              }
              __syncthreads();
              if (w8 == 0) {
                const float mv = mx[0];
                float ls = 0.f;
                for (int i = lane; i < nk; i += 64) {
                  const float p = expf(sc[i] - mv);
                  sc[i] = p;
                  ls += p;
                }
                ls = wave_sum(ls);
                if (lane == 0) mx[1] = ls;
              }
              __syncthreads();
              // P.V: wave w takes keys w, w+8, ...; lanes take dims
              for (int d = lane; d < hd; d += 64) {
                float acc = 0.f;
                for (int ks = w8; ks < nk; ks += MK_WAVES) {
                  const int tpos = (lw + (ks / MK_KBLK) * MK_NL) * MK_KBLK + (ks % MK_KBLK);
                  float vvv;
                  if (tpos < pos0) {
                    const uint32_t off = (uint32_t)((((size_t)m.page_table[tpos / MK_PAGE] * nkv + kvh) * MK_PAGE + (tpos % MK_PAGE)) * hd + d) * 2;
                    const uint32_t raw = (kaux == AUX_DEV) ? __builtin_amdgcn_raw_buffer_load_b16(vrs, off, 0, AUX_DEV)
                                                           : __builtin_amdgcn_raw_buffer_load_b16(vrs, off, 0, 0);
                    vvv = __uint_as_float(raw << 16);
                  } else {
                    vvv = qkv[(tpos - pos0) * 3 * hd + 2 * hd + d];
                  }
                  acc = fmaf(sc[ks], vvv, acc);
                }
                pv[w8 * hd + d] = acc;
              }
              __syncthreads();
              const int plen = hd + 2;
              uint2 *dst = xo + c * m.x_o_len + lw * plen;
              for (int d = tid; d < hd; d += MK_THREADS) {
                float acc = pv[d];
                for (int ww = 1; ww < MK_WAVES; ++ww) acc += pv[ww * hd + d];
                pub_l2(dst + 2 + d, acc, tg);
              }
              if (tid == 0) {
                pub_l2(dst + 0, nk > 0 ? mx[0] : -INFINITY, tg);
                pub_l2(dst + 1, nk > 0 ? mx[1] : 0.f, tg);
              }
              __syncthreads();
            }
          }
          // ------------------------------------------------ A3: merge partials + o-projection slice
          {
            const int plen = hd + 2;
            float *part = L.work + 2048;           // [32][plen]
            float *ov = L.work;                    // [NCOL][hd]
            for (int c = 0; c < ncol; ++c) {
              if (!gather2d<AUX_L2>(xo + c * m.x_o_len, 1, MK_NL * plen, 0, tg, part, L.flag, m.ctl, (step << 16) | (li << 8) | 7)) MK_BAIL();
              for (int d = tid; d < hd; d += MK_THREADS) {
                float M = -INFINITY;
                for (int ww = 0; ww < MK_NL; ++ww)
                  if (part[ww * plen + 1] > 0.f) M = fmaxf(M, part[ww * plen]);
                float Ls = 0.f, acc = 0.f;
                for (int ww = 0; ww < MK_NL; ++ww) {
                  if (part[ww * plen + 1] > 0.f) {
                    const float sc = expf(part[ww * plen] - M);
                    Ls = fmaf(part[ww * plen + 1], sc, Ls);
                    acc = fmaf(part[ww * plen + 2 + d], sc, acc);
                  }
                }
                ov[c * hd + d] = acc / Ls;
              }
              __syncthreads();
            }
            const int G_o = mk_tile_G(hd), L_o = hd / 8 / G_o, RG_o = 64 / G_o;
            const uint16_t *tile = ly.at_o + (size_t)x * H * hd;
            const int nrg = H / RG_o;
            for (int rg = wx; rg < nrg; rg += MK_NL * MK_WAVES) {
              u32x4 wr[2];
              rg_load<2>(tile, rg, L_o, wr);
              float oo[NCOL];
              rg_dot<NCOL, 2>(wr, L_o, G_o, ov, hd, ncol, oo);
              if ((lane & (G_o - 1)) == 0) {
                const int row = rg * RG_o + lane / G_o;
                FOR_COL(c) pub_dev(xmix + ((size_t)c * MK_NX + x) * H + row, oo[c], tg);
              }
            }
          }
        } else {
          for (int i = tid + lw * MK_THREADS; i < H; i += MK_NL * MK_THREADS)
            for (int c = 0; c < ncol; ++c) pub_dev(xmix + ((size_t)c * MK_NX + x) * H + i, 0.f, tg);
        }
      }
      // ---------------------------------------------------- R1: residual += sum of the 8 mixer slices
      {
        float *tmp = L.work;  // [NCOL*8][SL]
        if (!gather2d<AUX_DEV>(ly.x_mix + lw * SL, ncol * MK_NX, SL, H, tg, tmp, L.flag, m.ctl, (step << 16) | (li << 8) | 8)) MK_BAIL();
        uint2 *xr = ly.x_r1 + (size_t)x * MK_MAXCOL * H;
        for (int i = tid; i < ncol * SL; i += MK_THREADS) {
          const int c = i / SL, k = i - c * SL;
          float s = tmp[(c * MK_NX) * SL + k];
#pragma unroll
          for (int g = 1; g < MK_NX; ++g) s += tmp[(c * MK_NX + g) * SL + k];
          pub_l2(xr + c * H + lw * SL + k, L.xres[c * H + lw * SL + k] + s, tg);
        }
        if (!gather2d<AUX_L2>(xr, ncol, H, H, tg, L.xres, L.flag, m.ctl, (step << 16) | (li << 8) | 9)) MK_BAIL();
      }
      // ================================================================ FFN
      rmsnorm_cols<NCOL>(L.xres, L.hn, ly.ln2, H, m.rms_eps, ncol, L.red);
      {
        const int J = m.J;
        uint2 *xm = ly.x_m + (size_t)x * MK_MAXCOL * J;
        const uint16_t *gu = ly.ffn_gu + (size_t)x * 2 * J * H;
        // F1: gate/up pairs j -> m_j = SiLU(g_j) * u_j
        for (int j = wx; j < J; j += MK_NL * MK_WAVES) {
          float g[NCOL], u[NCOL];
          if (RG_h == 1) {
            u32x4 wg[2], wu[2];
            rg_load<2>(gu, 2 * j, L_h, wg);
            rg_load<2>(gu, 2 * j + 1, L_h, wu);
            rg_dot<NCOL, 2>(wg, L_h, G_h, L.hn, H, ncol, g);
            rg_dot<NCOL, 2>(wu, L_h, G_h, L.hn, H, ncol, u);
          } else {  // RG_h == 2: lanes [0,32) compute g_j, lanes [32,64) u_j
            u32x4 wr[2];
            rg_load<2>(gu, j, L_h, wr);
            rg_dot<NCOL, 2>(wr, L_h, G_h, L.hn, H, ncol, g);
#pragma unroll
            for (int c = 0; c < NCOL; ++c) u[c] = __shfl_xor(g[c], 32, 64);
          }
          if (lane == 0)
            FOR_COL(c) {
              pub_l2(xm + c * J + j, siluf_(g[c]) * u[c], tg);
            }
        }
        // F2: down-projection slice (columns x*J .. x*J+J of W_d)
        float *mv = L.work;  // [NCOL][J]
        if (!gather2d<AUX_L2>(xm, ncol, J, J, tg, mv, L.flag, m.ctl, (step << 16) | (li << 8) | 11)) MK_BAIL();
        const int G_d = mk_tile_G(J), L_d = J / 8 / G_d, RG_d = 64 / G_d;
        const uint16_t *tile = ly.ffn_dn + (size_t)x * H * J;
        const int nrg = H / RG_d;
        for (int rg = wx; rg < nrg; rg += MK_NL * MK_WAVES) {
          u32x4 wr[8];
          rg_load<8>(tile, rg, L_d, wr);
          float oo[NCOL];
          rg_dot<NCOL, 8>(wr, L_d, G_d, mv, J, ncol, oo);
          if ((lane & (G_d - 1)) == 0) {
            const int row = rg * RG_d + lane / G_d;
            FOR_COL(c) pub_dev(ly.x_ffn + ((size_t)c * MK_NX + x) * H + row, oo[c], tg);
          }
        }
      }
      // ---------------------------------------------------- R2: residual += sum of the 8 FFN slices
      {
        float *tmp = L.work;
        if (!gather2d<AUX_DEV>(ly.x_ffn + lw * SL, ncol * MK_NX, SL, H, tg, tmp, L.flag, m.ctl, (step << 16) | (li << 8) | 12)) MK_BAIL();
        uint2 *xr = ly.x_r2 + (size_t)x * MK_MAXCOL * H;
        for (int i = tid; i < ncol * SL; i += MK_THREADS) {
          const int c = i / SL, k = i - c * SL;
          float s = tmp[(c * MK_NX) * SL + k];
#pragma unroll
          for (int g = 1; g < MK_NX; ++g) s += tmp[(c * MK_NX + g) * SL + k];
          pub_l2(xr + c * H + lw * SL + k, L.xres[c * H + lw * SL + k] + s, tg);
        }
        if (!gather2d<AUX_L2>(xr, ncol, H, H, tg, L.xres, L.flag, m.ctl, (step << 16) | (li << 8) | 9)) MK_BAIL();
      }
    }  // layers

    if (!last_step) {
      pend_n = 0;   // the pending updates were applied (and stored) during this token
      continue;
    }
    // ================================================================ LM head + greedy argmax
    rmsnorm_cols<NCOL>(L.xres, L.hn, m.lnf, H, m.rms_eps, ncol, L.red);
    {
      const int nrg_all = m.V / RG_h;
      const int g0 = (int)((long long)b * nrg_all / MK_NWG), g1 = (int)((long long)(b + 1) * nrg_all / MK_NWG);
      const int cnt = g1 - g0;
      const int wg0 = g0 + w8 * cnt / MK_WAVES, wg1 = g0 + (w8 + 1) * cnt / MK_WAVES;
      float best[NCOL];
      int bidx[NCOL];
      int nanf = 0;
#pragma unroll
      for (int c = 0; c < NCOL; ++c) { best[c] = -INFINITY; bidx[c] = 0x7fffffff; }
      for (int rg = wg0; rg < wg1; ++rg) {
        u32x4 wr[2];
        rg_load<2>(m.embed, rg, L_h, wr);
        float o[NCOL];
        rg_dot<NCOL, 2>(wr, L_h, G_h, L.hn, H, ncol, o);
        if ((lane & (G_h - 1)) == 0) {
          const int row = rg * RG_h + lane / G_h;
#pragma unroll
          for (int c = 0; c < NCOL; ++c) {
            if (c < ncol) {
              if (a.logits) a.logits[(size_t)c * m.V + row] = o[c];
              if (!(o[c] == o[c]) || isinf(o[c])) nanf = 1;
              if (o[c] > best[c] || (o[c] == best[c] && row < bidx[c])) { best[c] = o[c]; bidx[c] = row; }
            }
          }
        }
      }
      // wave reduce (value desc, index asc), then across waves
      float *rv = L.work;                  // [NCOL][8]
      int *ri = reinterpret_cast<int *>(L.work + 64);
      int *rn = reinterpret_cast<int *>(L.work + 128);
#pragma unroll
      for (int c = 0; c < NCOL; ++c) {
        float bv = best[c];
        int bi = bidx[c];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
          const float ov = __shfl_xor(bv, off, 64);
          const int oi = __shfl_xor(bi, off, 64);
          if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
        }
        if (lane == 0) { rv[c * 8 + w8] = bv; ri[c * 8 + w8] = bi; }
      }
      int anynan = __any(nanf) ? 1 : 0;
      if (lane == 0) rn[w8] = anynan;
      __syncthreads();
      if (tid < ncol) {
        const int c = tid;
        float bv = rv[c * 8];
        int bi = ri[c * 8];
        int nn = 0;
        for (int ww = 0; ww < MK_WAVES; ++ww) {
          nn |= rn[ww];
          if (rv[c * 8 + ww] > bv || (rv[c * 8 + ww] == bv && ri[c * 8 + ww] < bi)) { bv = rv[c * 8 + ww]; bi = ri[c * 8 + ww]; }
        }
        uint4 rec = make_uint4(__float_as_uint(bv), (uint32_t)bi, tag, (uint32_t)nn);
        __hip_atomic_store(reinterpret_cast<unsigned long long *>(m.x_arg + c * MK_NWG + b),
                           ((unsigned long long)rec.y << 32) | rec.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        wait_stores();
        __hip_atomic_store(reinterpret_cast<unsigned long long *>(m.x_arg + c * MK_NWG + b) + 1,
                           ((unsigned long long)rec.w << 32) | rec.z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();  // the candidate above was read from the scratch the final gather reuses
    if (b == 0) {
      // final argmax over the 256 workgroup candidates; the tag word is written after the
      // value/index word by the same thread, so a matching tag implies the record is complete
      float *cv = L.work;                         // [NCOL][256]
      int *ci = reinterpret_cast<int *>(L.work + NCOL * MK_NWG);
      int *cn = reinterpret_cast<int *>(L.work + 2 * NCOL * MK_NWG);
      __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(m.x_arg, 0, MK_MAXCOL * MK_NWG * 16, RSRC_W3);
      for (int i = tid; i < ncol * MK_NWG; i += MK_THREADS) {
        const unsigned long long deadline = wall_clock64() + MK_WAIT_TICKS;
        while (true) {
          const uint32_t tw = __builtin_amdgcn_raw_buffer_load_b32(rs, i * 16 + 8, 0, AUX_DEV);
          if (tw == tag) break;
          if (wall_clock64() > deadline) { L.flag[0] = 1; break; }
          __builtin_amdgcn_s_sleep(1);
        }
        u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, i * 16, 0, AUX_DEV);
        cv[i] = __uint_as_float(v.x);
        ci[i] = (int)v.y;
        cn[i] = (int)v.w;
      }
      __syncthreads();
      if (L.flag[0]) MK_BAIL();
      if (w8 == 0) {
        int gsel[MK_MAXCOL];
        int anynan = 0;
#pragma unroll
        for (int c = 0; c < MK_MAXCOL; ++c) {
          gsel[c] = 0;
          if (c >= ncol) continue;
          float bv = -INFINITY;
          int bi = 0x7fffffff, nn = 0;
          for (int i = lane; i < MK_NWG; i += 64) {
            const float v = cv[c * MK_NWG + i];
            const int ix = ci[c * MK_NWG + i];
            nn |= cn[c * MK_NWG + i];
            if (v > bv || (v == bv && ix < bi)) { bv = v; bi = ix; }
          }
#pragma unroll
          for (int off = 32; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off, 64);
            const int oi = __shfl_xor(bi, off, 64);
            if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
          }
          anynan |= __any(nn) ? 1 : 0;
          gsel[c] = (bi == 0x7fffffff) ? 0 : bi;
        }
        if (lane == 0) {
          int nacc = ncol;
          if (verify) {
            nacc = 1;
            bool run = true;
#pragma unroll
            for (int c = 1; c < MK_MAXCOL; ++c)
              if (run && c < ncol && a.tokens[c] == gsel[c - 1]) ++nacc;
              else run = false;
          }
#pragma unroll
          for (int c = 0; c < MK_MAXCOL; ++c)
            if (c < ncol) a.argmax[c] = gsel[c];
          if (a.n_acc) a.n_acc[0] = nacc;
          if (anynan) __hip_atomic_fetch_or(m.ctl + MK_CTL_ERR, MK_DERR_NAN, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const int consumed = a.prefill ? a.n : (verify ? nacc : 1);
          __hip_atomic_store(m.ctl + MK_CTL_POS, ctl_pos + consumed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(m.ctl + MK_CTL_PEND, verify ? nacc : 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(m.ctl + MK_CTL_PAR, verify ? (par ^ 1) : par, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }  // steps
}

// ------------------------------------------------------------------------------ host-side launchers
// Instantiations: one decode column, up to MK_MAXCOL verify columns, and the prompt
// processed token by token (a distinct kernel so that profiles separate it).
static const void *forward_fn(int ncol_template, int prompt) {
  if (prompt) return (const void *)mk_forward<1, true>;
  return (ncol_template == 1) ? (const void *)mk_forward<1, false> : (const void *)mk_forward<MK_MAXCOL, false>;
}

extern "C" hipError_t mk_launch_forward(const MkLaunch *a, int ncol_template, hipStream_t stream) {
  void *args[] = {const_cast<MkLaunch *>(a)};
  return hipLaunchCooperativeKernel(forward_fn(ncol_template, a->prefill), dim3(MK_NWG), dim3(MK_THREADS), args,
                                    MK_LDS_BYTES, stream);
}

extern "C" hipError_t mk_forward_occupancy(int ncol_template, int *blocks_per_cu) {
  const void *fn = forward_fn(ncol_template, ncol_template == 0);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, MK_LDS_BYTES);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, MK_THREADS, MK_LDS_BYTES);
}
