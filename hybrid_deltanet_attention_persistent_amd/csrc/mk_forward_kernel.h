// mk_forward_kernel.h -- persistent single-launch forward pass of the hybrid Gated-DeltaNet +
// attention decoder on MI355X (gfx950): one decode step or one multi-token verify
// forward, each in one launch (prompts go through mk_prefill.hip).
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
//     tag equals the forward's tag.  Slots are read with device-coherent (sc1)
//     loads, which skip the per-CU L1; a slot read by other XCDs is written through
//     to memory, a slot read only inside the writer's XCD stops in that XCD's L2.
//   * XCD x owns DeltaNet head x / query head x and FFN intermediate slice x, so
//     in-projection -> conv -> delta rule -> gated norm -> out-projection stay
//     inside one XCD; the out-projection and the FFN down-projection are split
//     over XCDs along their input dimension, and the residual stream is rebuilt
//     by a reduce-scatter (over XCDs) + all-gather (inside the XCD) per sublayer.
//   * Weights stream once per forward in a tile layout that makes every wave load
//     a contiguous 1 KiB (mk_layout.h), and each phase's weight rows are loaded
//     into registers one phase ahead, so HBM latency overlaps the hand-off wait:
//     in decode, waves 0-6 hold the weight loads and wave 7 alone polls (a poll
//     waits for every older load of its wave), and workgroup barriers fence LDS
//     only (a full fence would drain the weight loads at every barrier).
//   * Decode and verify use the same per-column arithmetic in the same order, so
//     a verify forward's logits are bit-identical to sequential decode steps.
//
// The kernel template is instantiated in two translation units, mk_forward.hip (one decode
// column) and mk_verify.hip (MK_MAXCOL verify columns), so that each is compiled on its own.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include "mk_layout.h"

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define MK_WAIT_TICKS 20000000ull   // watchdog: 0.2 s of the 100 MHz device wall clock
#define AUX_DEV 16                  // sc1: device-coherent
#define RSRC_W3 0x00020000

// per-wave register budgets of the prefetched weight rows (checked against the model on the host)
#define NRG_IN 3   // in-projection / QKV row groups per wave
#define NPAIR 2    // gate/up row pairs per wave
#define LMAX_D 8   // loads per lane of one down-projection row group
#define LM_BATCH(NCOL) ((NCOL) == 1 ? 8 : 4)

// ------------------------------------------------------------------------------ helpers
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Workgroup barrier that orders LDS only.  A full barrier also waits for the wave's outstanding
// global stores, and with them (one in-order counter) for every weight load issued before them;
// no global data is handed between the waves of a workgroup, so an LDS-scope fence is enough and
// prefetched weights stay in flight across the barrier.
// Compiler-only memory barrier: keeps prefetch loads where they are issued.  The LDS-scope
// barriers do not order global loads, so without it the compiler may sink a prefetch down to
// its use and nothing is in flight during the hand-offs.
__device__ __forceinline__ void keep_issued() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ void lbar() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

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

// Cross-lane sums with DPP (no LDS traffic).  Within a 16-lane row: xor 1 and xor 2 (quad
// permutes), then the half-row and row mirrors pair up 4- and 8-lane groups; every lane of the
// group ends with the same value (a + b == b + a).  Across rows the four row totals are added in
// a fixed order.
#define DPP_XOR1 0xB1       // quad_perm [1,0,3,2]
#define DPP_XOR2 0x4E       // quad_perm [2,3,0,1]
#define DPP_HALF_MIRROR 0x141
#define DPP_MIRROR 0x140
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_sum16(float v) {
  v = dpp_add<DPP_XOR1>(v);
  v = dpp_add<DPP_XOR2>(v);
  v = dpp_add<DPP_HALF_MIRROR>(v);
  return dpp_add<DPP_MIRROR>(v);
}
// Sum over the 64 lanes in a fixed order: lane pairs (l, l ^ 32) through a permlane32 swap, then
// (l, l ^ 16) through a permlane16 swap, then the 16-lane row tree above.  Every lane gets the
// total.  Each swap returns {low half, high half} operands, so every add is (lower lane) + (upper).
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float swap_add32(float a, float b) {  // lanes < 32: a[l] + a[l+32]; >= 32: b[l-32] + b[l]
  const u32x2 p = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(p.x) + __uint_as_float(p.y);
}
__device__ __forceinline__ float swap_add16(float a, float b) {  // rows {0,1,2,3} <- a r0+r1, b r0+r1, a r2+r3, b r2+r3
  const u32x2 p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(p.x) + __uint_as_float(p.y);
}
__device__ __forceinline__ float wave_sum(float v) {
  v = swap_add32(v, v);
  v = swap_add16(v, v);
  return row_sum16(v);
}
// Four wave sums at once, each with exactly wave_sum's additions: lanes [0,16) get the total of a,
// [16,32) of c, [32,48) of b, [48,64) of d.
__device__ __forceinline__ float wave_sum4(float a, float b, float c, float d) {
  return row_sum16(swap_add16(swap_add32(a, b), swap_add32(c, d)));
}
__device__ __forceinline__ float group_sum(float v, int G) {  // sum over aligned groups of G lanes
  if (G == 64) return wave_sum(v);
  if (G >= 2) v = dpp_add<DPP_XOR1>(v);
  if (G >= 4) v = dpp_add<DPP_XOR2>(v);
  if (G >= 8) v = dpp_add<DPP_HALF_MIRROR>(v);
  if (G >= 16) v = dpp_add<DPP_MIRROR>(v);
  if (G == 32) v += __shfl_xor(v, 16, 64);
  return v;
}
// Sum of one value per thread over the workgroup, fixed order; red: >= MK_WAVES floats of LDS.
__device__ __forceinline__ float block_sum(float v, float *red) {
  v = wave_sum(v);
  if (lane_id() == 0) red[wave_id()] = v;
  lbar();
  float s = red[0];
#pragma unroll
  for (int w = 1; w < MK_WAVES; ++w) s += red[w];
  lbar();
  return s;
}

// tagged exchange slot: 8 bytes {float bits, tag}, written with one device-coherent 64-bit store
// (written through to memory, where the other XCDs' polls see it)
__device__ __forceinline__ void pub(uint2 *p, float v, uint32_t tag) {
  __hip_atomic_store(reinterpret_cast<unsigned long long *>(p), ((unsigned long long)tag << 32) | __float_as_uint(v),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A slot read only by workgroups of the writer's own XCD: the 64-bit store stops in that XCD's
// L2, which the consumers' device-coherent loads (they skip the per-CU L1) read directly.  The
// round trip is about half that of a store written through to memory.  Every such slot region is
// owned by one XCD and padded to whole 256-byte blocks, so no cache line holds two XCDs' slots.
__device__ __forceinline__ void pub_xcd(uint2 *p, float v, uint32_t tag) {
  __hip_atomic_store(reinterpret_cast<unsigned long long *>(p), ((unsigned long long)tag << 32) | __float_as_uint(v),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Watchdog expiry inside a gather: flag the workgroup and record the first failing site.
__device__ __noinline__ void gather_timeout(int *fail, int32_t *ctl, int site, int tid, uint32_t seen, uint32_t tag) {
  *fail = 1;
  int expect = 0;
  if (__hip_atomic_compare_exchange_strong(ctl + MK_CTL_WHERE, &expect, site | (1 << 30), __ATOMIC_RELAXED,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
    __hip_atomic_store(ctl + MK_CTL_WHERE + 1, (int)(blockIdx.x * 65536 + tid), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(ctl + MK_CTL_WHERE + 2, (int)seen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(ctl + MK_CTL_WHERE + 3, (int)tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Poll up to MAXC 16-byte chunks per lane (two tagged slots each) until both tags equal `tag`,
// then store the two values to LDS.  Polls follow each other without a sleep: each round waits
// for its own loads, which paces it (measured: a sleep between rounds only delays detection).
// Returns false on watchdog expiry.
template <int MAXC>
__device__ __forceinline__ bool poll_chunks(__amdgpu_buffer_rsrc_t rs, const uint32_t (&off)[MAXC], float *const (&dp)[MAXC],
                                            uint32_t pend, uint32_t tag, int *fail, int32_t *ctl, int site, int tid) {
  if (!pend) return true;
  const unsigned long long deadline = wall_clock64() + MK_WAIT_TICKS;
  while (true) {
    u32x4 v[MAXC];
#pragma unroll
    for (int j = 0; j < MAXC; ++j)
      if (pend & (1u << j)) v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, off[j], 0, AUX_DEV);
#pragma unroll
    for (int j = 0; j < MAXC; ++j) {
      if ((pend & (1u << j)) && v[j].y == tag && v[j].w == tag) {
        dp[j][0] = __uint_as_float(v[j].x);
        dp[j][1] = __uint_as_float(v[j].z);
        pend &= ~(1u << j);
      }
    }
    if (!pend) return true;
    if (wall_clock64() > deadline) {
      uint32_t seen = 0;
#pragma unroll
      for (int j = MAXC - 1; j >= 0; --j)
        if (pend & (1u << j)) seen = v[j].y;
      gather_timeout(fail, ctl, site, tid, seen, tag);
      return false;
    }
  }
}

// Gather a [nrow][ncol] block of tagged slots (row stride `stride` slots, ncol even) into
// dst[nrow][ncol] (LDS), polling until every tag equals `tag`.  Only the last NPW waves poll, in
// rounds of MAXC chunks per lane: a wave that polls waits for every older load of its own, so the
// waves that keep weight loads in flight stay out of it.  Every thread calls it; it ends with a
// barrier.  On watchdog expiry records the first failing site in the control block and returns false.
template <int MAXC, int NPW>
__device__ bool poll2d(const uint2 *src, int nrow, int ncol, int stride, uint32_t tag, float *dst, int *fail,
                       int32_t *ctl, int site, int tid) {
  const int half = ncol >> 1;
  const int nchunk = nrow * half;
  const int pt = tid - (MK_WAVES - NPW) * 64;   // index among the polling threads
  if (pt >= 0 && *fail == 0) {   // (after a watchdog expiry in this workgroup: go straight to the barrier)
    const uint32_t bytes = (uint32_t)(((nrow - 1) * stride + ncol) * 8);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)src, 0, bytes, RSRC_W3);
    for (int base = 0; base < nchunk; base += MAXC * NPW * 64) {
      uint32_t off[MAXC];
      float *dp[MAXC];
      uint32_t pend = 0;
#pragma unroll
      for (int j = 0; j < MAXC; ++j) {
        const int c = base + pt + j * NPW * 64;
        const int r = c / half, q = c - r * half;
        off[j] = (uint32_t)((r * stride + 2 * q) * 8);
        dp[j] = dst + r * ncol + 2 * q;
        if (c < nchunk) pend |= 1u << j;
      }
      if (!poll_chunks<MAXC>(rs, off, dp, pend, tag, fail, ctl, site, tid)) break;
    }
  }
  return *fail == 0;
}
template <int MAXC, int NPW>
__device__ bool gather2d(const uint2 *src, int nrow, int ncol, int stride, uint32_t tag, float *dst, int *fail,
                         int32_t *ctl, int site, int tid) {
  poll2d<MAXC, NPW>(src, nrow, ncol, stride, tag, dst, fail, ctl, site, tid);
  lbar();
  return *fail == 0;
}

// One segment of a multi-segment gather: nrow rows of ncol (even) slots starting `off` slots
// after the common base, row stride `stride` slots, into dst[nrow][ncol].
struct GSeg {
  int off, nrow, ncol, stride;
  float *dst;
};

// Gather several blocks (all addressed from one base) in one polling loop and one barrier.
// MK_SEG_INLINE is empty in the decode unit and __forceinline__ in the verify unit: inlined, the
// segment table stays in registers (the out-of-line call passes it through scratch memory), while
// the decode kernel measured faster with the compiler's own choice.
#ifndef MK_SEG_INLINE
#define MK_SEG_INLINE
#endif
template <int MAXC, int NPW, int NSEG>
__device__ MK_SEG_INLINE bool poll_segs(const uint2 *base, const GSeg (&sg)[NSEG], uint32_t tag, int *fail, int32_t *ctl,
                            int site, int tid) {
  int total = 0;
#pragma unroll
  for (int s = 0; s < NSEG; ++s) total += sg[s].nrow * (sg[s].ncol >> 1);
  const int pt = tid - (MK_WAVES - NPW) * 64;
  if (pt >= 0 && *fail == 0) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, 0x7fffffff, RSRC_W3);
    for (int b0 = 0; b0 < total; b0 += MAXC * NPW * 64) {
      uint32_t off[MAXC];
      float *dp[MAXC];
      uint32_t pend = 0;
#pragma unroll
      for (int j = 0; j < MAXC; ++j) {
        int c = b0 + pt + j * NPW * 64;
        off[j] = 0;
        dp[j] = nullptr;
        if (c < total) {
          pend |= 1u << j;
#pragma unroll
          for (int s = 0; s < NSEG; ++s) {
            const int half = sg[s].ncol >> 1, n = sg[s].nrow * half;
            if (c >= 0 && c < n) {
              const int r = c / half, q = c - r * half;
              off[j] = (uint32_t)((sg[s].off + r * sg[s].stride + 2 * q) * 8);
              dp[j] = sg[s].dst + r * sg[s].ncol + 2 * q;
            }
            c -= n;
          }
        }
      }
      if (!poll_chunks<MAXC>(rs, off, dp, pend, tag, fail, ctl, site, tid)) break;
    }
  }
  return *fail == 0;
}
template <int MAXC, int NPW, int NSEG>
__device__ MK_SEG_INLINE bool gather_segs(const uint2 *base, const GSeg (&sg)[NSEG], uint32_t tag, int *fail, int32_t *ctl,
                            int site, int tid) {
  poll_segs<MAXC, NPW, NSEG>(base, sg, tag, fail, ctl, site, tid);
  lbar();
  return *fail == 0;
}

// ------------------------------------------------------------------------------ GEMV on tiles
#define AUX_NT 2                    // non-temporal: weights are streamed once per token
#define OOB_OFF 0x80000000u         // a buffer offset beyond every tile: the load reads zeros, touches no memory

// Buffer descriptor of a weight tile of `bytes` bytes (0: every load reads zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, RSRC_W3);
}

// Element i of a float vector of n elements, branch-free (0 for i >= n).
__device__ __forceinline__ float ld_gain(const float *p, int n, int i) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(tile_rsrc(p, (uint32_t)(n * 4)), (uint32_t)(i * 4), 0, 0));
}

// Prefetch up to NRG row groups rg = first + r*stride (valid below `end`) of a tile, L (<= LMAX)
// 16-byte loads per lane each.  Branch-free: every slot issues one load, an invalid slot with an
// out-of-range offset.  Straight-line loads let the compiler count exactly how many younger loads
// may stay in flight when one is consumed; a branch around a load makes it wait for all of them.
template <int NRG, int LMAX>
__device__ __forceinline__ void rg_issue(__amdgpu_buffer_rsrc_t rs, int first, int stride, int end, int L,
                                         u32x4 (&w)[NRG][LMAX]) {
  const int lane = lane_id();
#pragma unroll
  for (int r = 0; r < NRG; ++r) {
    const int rg = first + r * stride;
#pragma unroll
    for (int i = 0; i < LMAX; ++i) {
      const bool ok = rg < end && i < L;
      const uint32_t off = ok ? (uint32_t)(((rg * L + i) * 64 + lane) * 16) : OOB_OFF;
      w[r][i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, AUX_NT);
    }
  }
}

// Dot products of one loaded row group with NCOL activation vectors act[c*astride + k]; returns each
// lane's row result (valid in every lane of the row's G-lane segment).
template <int NCOL, int LMAX>
__device__ __forceinline__ void rg_dot(const u32x4 (&w)[LMAX], int L, int G, const float *act, int astride, int n,
                                       float (&out)[NCOL]) {
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

// rg_dot for the down projection (up to 8 loads per lane): every activation load of a column is
// issued before its products, and the products alternate between two accumulators, so the loads
// overlap and the dependent chain is half as long.  Decode and verify both use it (same order).
template <int NCOL, int LMAX>
__device__ __forceinline__ void rg_dot_dn(const u32x4 (&w)[LMAX], int L, int G, const float *act, int astride, int n,
                                          float (&out)[NCOL]) {
  const int kl = (lane_id() & (G - 1)) * 8;
#pragma unroll
  for (int c = 0; c < NCOL; ++c) {
    out[c] = 0.f;
    if (c < n) {
      float4 a[LMAX][2];
#pragma unroll
      for (int i = 0; i < LMAX; ++i) {   // (past L: a valid re-read, unused)
        const int k0 = (i < L ? i : 0) * G * 8 + kl;
        a[i][0] = *reinterpret_cast<const float4 *>(act + c * astride + k0);
        a[i][1] = *reinterpret_cast<const float4 *>(act + c * astride + k0 + 4);
      }
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int i = 0; i < LMAX; ++i) {
        if (i < L) {
          float f[8];
          unpack8(w[i], f);
          s0 = fmaf(f[0], a[i][0].x, s0); s1 = fmaf(f[1], a[i][0].y, s1);
          s0 = fmaf(f[2], a[i][0].z, s0); s1 = fmaf(f[3], a[i][0].w, s1);
          s0 = fmaf(f[4], a[i][1].x, s0); s1 = fmaf(f[5], a[i][1].y, s1);
          s0 = fmaf(f[6], a[i][1].z, s0); s1 = fmaf(f[7], a[i][1].w, s1);
        }
      }
      out[c] = s0 + s1;
    }
  }
#pragma unroll
  for (int c = 0; c < NCOL; ++c) out[c] = group_sum(out[c], G);
}

// Per-lane partial dot of 16 bf16 weights (two 16-byte loads) with 16 cached activations.
__device__ __forceinline__ float dot16(const u32x4 &w0, const u32x4 &w1, const float (&a)[16]) {
  float f[8], s = 0.f;
  unpack8(w0, f);
#pragma unroll
  for (int e = 0; e < 8; ++e) s = fmaf(f[e], a[e], s);
  unpack8(w1, f);
#pragma unroll
  for (int e = 0; e < 8; ++e) s = fmaf(f[e], a[8 + e], s);
  return s;
}

// Decode: dot product of one loaded row group with the activations in registers (rmsnorm_regs
// layout), summed over each row's G lanes: the same products, order and tree as rg_dot.
__device__ __forceinline__ float rg_dot_regs(const u32x4 &w0, const u32x4 &w1, int G, const float (&a)[16]) {
  return group_sum(dot16(w0, w1, a), G);
}

// Sum each of 8 per-lane partials over the 64 lanes: a transposing butterfly that moves half of
// the partials at each of the first three steps.  Returns, in lane l, the total of partial l >> 3.
__device__ __forceinline__ float reduce8(const float (&p)[8]) {
  const int lane = lane_id();
  const bool hi32 = lane & 32, hi16 = lane & 16, hi8 = lane & 8;
  float q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // offset 32: the upper half keeps partials 4..7, the lower half 0..3
    const float send = hi32 ? p[i] : p[i + 4];
    const float keep = hi32 ? p[i + 4] : p[i];
    q[i] = keep + __shfl_xor(send, 32, 64);
  }
  float r[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {  // offset 16
    const float send = hi16 ? q[i] : q[i + 2];
    const float keep = hi16 ? q[i + 2] : q[i];
    r[i] = keep + __shfl_xor(send, 16, 64);
  }
  const float send = hi8 ? r[0] : r[1];  // offset 8
  float t = (hi8 ? r[1] : r[0]) + __shfl_xor(send, 8, 64);
  t = dpp_add<DPP_XOR1>(t);
  t = dpp_add<DPP_XOR2>(t);
  return dpp_add<DPP_HALF_MIRROR>(t);
}

// The same sum as reduce8 for a single partial: identical additions in identical order
// (offsets 32, 16, 8, then 1, 2 and the half-row mirror), so decode and verify agree bit for bit.
__device__ __forceinline__ float wave_sum_lm(float t) {
  t += __shfl_xor(t, 32, 64);
  t += __shfl_xor(t, 16, 64);
  t += __shfl_xor(t, 8, 64);
  t = dpp_add<DPP_XOR1>(t);
  t = dpp_add<DPP_XOR2>(t);
  return dpp_add<DPP_HALF_MIRROR>(t);
}

// RMSNorm.  The sum of squares of a hidden vector x[H] is taken the way the GEMV lanes hold the
// vector: lane l owns elements (i G + l % G) 8 + e (i < L, e < 8; G, L: the tile layout of a
// row of H), summed in that order, then over G lanes.  Every wave computes it itself, so the
// norm needs no exchange between waves; decode and verify use this one order.
__device__ __forceinline__ float col_sumsq(const float *x, int G, int L) {
  const int kl = (lane_id() & (G - 1)) * 8;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (i < L) {
      const float4 a0 = *reinterpret_cast<const float4 *>(x + i * G * 8 + kl);
      const float4 a1 = *reinterpret_cast<const float4 *>(x + i * G * 8 + kl + 4);
      ss = fmaf(a0.x, a0.x, ss); ss = fmaf(a0.y, a0.y, ss); ss = fmaf(a0.z, a0.z, ss); ss = fmaf(a0.w, a0.w, ss);
      ss = fmaf(a1.x, a1.x, ss); ss = fmaf(a1.y, a1.y, ss); ss = fmaf(a1.z, a1.z, ss); ss = fmaf(a1.w, a1.w, ss);
    }
  }
  return group_sum(ss, G);
}
__device__ __forceinline__ float rms_scale(float sumsq, int H, float eps) { return 1.f / sqrtf(sumsq / (float)H + eps); }

// RMSNorm of src[c][H] into dst[c][H] (LDS); thread t scales elements t and t + 512 (H <= 1024)
// with the gains g0, g1 it holds.  Ends with a barrier.
template <int NCOL>
__device__ void rmsnorm_cols_r(const float *src, float *dst, float g0, float g1, int H, int G, int L, float eps,
                               int n, int tid) {
  for (int c = 0; c < NCOL; ++c) {
    if (c >= n) break;
    const float r = rms_scale(col_sumsq(src + c * H, G, L), H, eps);
    if (tid < H) dst[c * H + tid] = src[c * H + tid] * r * g0;
    if (tid + MK_THREADS < H) dst[c * H + tid + MK_THREADS] = src[c * H + tid + MK_THREADS] * r * g1;
  }
  lbar();
}

// Decode: this lane's normalised activations of a hidden vector, in registers: element
// (i G + l % G) 8 + e goes to a[i * 8 + e] (the operand layout of a tile row), with the gains the
// lane holds in the same layout.  The same values as rmsnorm_cols_r, without LDS or barriers.
__device__ __forceinline__ void rmsnorm_regs(const float *x, const float (&g)[16], int H, int G, int L, float eps,
                                             float (&a)[16]) {
  const float r = rms_scale(col_sumsq(x, G, L), H, eps);
  const int kl = (lane_id() & (G - 1)) * 8;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) a[i * 8 + e] = (i < L) ? x[i * G * 8 + kl + e] * r * g[i * 8 + e] : 0.f;
}
// The gains of one RMSNorm in the operand layout of rmsnorm_regs (zeros past L), four 16-byte loads.
// Branch-free: a wave that needs none passes live = false.
__device__ __forceinline__ void ld_gain16(const float *p, int H, int G, bool live, float (&g)[16]) {
  const __amdgpu_buffer_rsrc_t rs = tile_rsrc(p, live ? (uint32_t)(H * 4) : 0u);   // not live: zeros, no traffic
  const int kl = (lane_id() & (G - 1)) * 8;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)((i * G * 8 + kl + h * 4) * 4), 0, 0);
      g[i * 8 + h * 4 + 0] = __uint_as_float(v.x);
      g[i * 8 + h * 4 + 1] = __uint_as_float(v.y);
      g[i * 8 + h * 4 + 2] = __uint_as_float(v.z);
      g[i * 8 + h * 4 + 3] = __uint_as_float(v.w);
    }
}

// loop over the live columns with compile-time indices (register arrays stay in registers)
#define FOR_COL(c) _Pragma("unroll") for (int c = 0; c < NCOL; ++c) if (c < ncol)

// On a watchdog expiry the whole workgroup records the error and leaves; the other
// workgroups then time out on its missing outputs and leave too.
#define MK_BAIL()                                                                                   \
  do {                                                                                              \
    if (tid == 0)                                                                                   \
      __hip_atomic_fetch_or(m.ctl + MK_CTL_ERR, MK_DERR_HANG, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); \
    return;                                                                                         \
  } while (0)
#define SITE(ph) ((step << 16) | (li << 8) | (ph))

typedef const __attribute__((address_space(4))) MkLayerDev ConstLayer;

// ------------------------------------------------------------------------------ the kernel
template <int NCOL, int SH>
__global__ void __launch_bounds__(MK_THREADS, 1) mk_forward(MkLaunch a) {
  extern __shared__ float lds_raw[];
  const MkDev &m = a.m;
  const int b = blockIdx.x, x = b & (MK_NX - 1), lw = b >> 3;
  // the wave index is wave-uniform: read it into a scalar register so that every row-group
  // index derived from it is scalar too
  const int w8 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id(), tid = threadIdx.x, tid0 = threadIdx.x;
  // Decode: waves 0..6 stream weight rows, wave 7 polls the hand-offs (it holds no
  // weight loads, so its polls never wait behind them).  Verify: all 8 waves do both.
  constexpr int CW = (NCOL == 1) ? MK_WAVES - 1 : MK_WAVES;   // weight-streaming waves
  constexpr int NPW = (CW < MK_WAVES) ? MK_WAVES - CW : MK_WAVES;   // polling waves
  constexpr int NRG_O = (CW < MK_WAVES) ? 2 : 1;               // out-projection row groups per wave
  const int wx = (w8 < CW) ? lw * CW + w8 : (1 << 24);        // streaming-wave index inside the XCD
  const int XW = MK_NL * CW;                                   // streaming waves per XCD
  // SH == MK_SHAPE_H1024 fixes every dimension of the hidden-1024 model (8 DeltaNet heads with
  // d_k = d_v = 128, 8 query and 2 KV heads of 128, FFN 3584) at compile time: tile strides,
  // row-group counts and reduction widths fold into straight-line code.  SH == MK_SHAPE_ANY reads
  // them from the launch arguments.
  constexpr bool FX = SH == MK_SHAPE_H1024;
  const int H = FX ? 1024 : m.H;
  // the layer table is read-only: reading it through the constant address space gives
  // scalar loads, so every pointer taken from it is known to be wave-uniform
  ConstLayer *const layers = (ConstLayer *)(uintptr_t)m.layers;

  float *xres = lds_raw;                        // [NCOL][H] residual stream
  float *hn = xres + NCOL * H;                  // [NCOL][H] normalised activations
  float *work = hn + NCOL * H;                  // [8192] phase scratch
  float *red = work + 8192;                     // [64] reductions
  int *flag = reinterpret_cast<int *>(red + 64);
  // physical pages of this workgroup's attention key blocks lw, lw + 32, ... (32 keys each, two
  // blocks per page), read once per launch: block j of the workgroup lies in page pgs[j]
  int *pgs = flag + 16;                         // [16] (10240 positions / 32 / 32 = 10 blocks)
  // RoPE cos / sin of this launch's positions [NCOL][hd / 2][2] (hd <= 128), loaded with the
  // embedding rows so that no attention layer waits for them
  float *rl = reinterpret_cast<float *>(pgs + 16);
  if (tid < 16) {
    const int pi = (lw + tid * MK_NL) * MK_KBLK / MK_PAGE;
    pgs[tid] = (pi < m.max_pages) ? m.page_table[pi] : 0;
  }
  if (tid == 0) {
    flag[0] = 0;
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    if ((int)(xcc & 7) != x) __hip_atomic_fetch_or(m.ctl + MK_CTL_ERR, MK_DERR_XCD, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  lbar();

  const int ctl_pos = __hip_atomic_load(m.ctl + MK_CTL_POS, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  int pend_n = __hip_atomic_load(m.ctl + MK_CTL_PEND, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int par = __hip_atomic_load(m.ctl + MK_CTL_PAR, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const bool verify = a.n > 1;
  const int ncol = a.n;
  const int G_h = mk_tile_G(H), L_h = H / 8 / G_h, RG_h = 64 / G_h;
  const int SL = H / MK_NL;  // residual slice per workgroup in the reductions
  const int nh = FX ? 8 : m.nh, dk = FX ? 128 : m.dk, dv = FX ? 128 : m.dv;
  const int nq = FX ? 8 : m.nq, nkv = FX ? 2 : m.nkv, hd = FX ? 128 : m.hd, J = FX ? 448 : m.J;
  const int r_in = FX ? 514 : m.r_in, nconv = FX ? 3072 : m.C;
  const int r_in_max = FX ? 544 : m.r_in_max, x_o_len = FX ? 4160 : m.x_o_len, xm_len = FX ? 448 : m.xm_len;
  const int G_o = mk_tile_G(dv), RG_o = 64 / G_o;        // out-projection columns of one head: L == 1
  const int G_a = mk_tile_G(hd), RG_a = 64 / G_a;        // o-projection columns of one head: L == 1
  const int G_d = mk_tile_G(J), L_d = J / 8 / G_d, RG_d = 64 / G_d;
  constexpr int MCS = (NPW == 1) ? 4 : (NCOL == 1 ? 1 : 2);   // polled chunks per lane and round: small gathers
  constexpr int MCL = (NPW == 1) ? 8 : NCOL;                  // ... gathers of whole hidden vectors

  // prefetched weight rows (registers), one phase ahead of their use
  u32x4 w_in[NRG_IN][2];      // D1 / A1
  u32x4 w_out[NRG_O][1];      // D3 / A3
  u32x4 w_gu[NPAIR][4];       // F1 (gate and up rows of up to NPAIR pairs)
  u32x4 w_dn[1][LMAX_D];      // F2

  // in-projection (DeltaNet) or QKV (attention) rows of layer li for this wave, branch-free: the
  // tile of each slot is selected with scalar selects and absent rows read as zeros
  auto issue_in = [&](int li) {   // li == n_layers: nothing to load (every slot reads zeros)
    const bool live = li < m.n_layers;
    ConstLayer &ly = layers[live ? li : 0];
    const bool dn = ly.kind == 0;
    const int per = hd / RG_h;                     // row groups of one attention head
    const int nrg = !live ? 0 : dn ? ((x < nh) ? r_in / RG_h : 0) : ((x < nq) ? 3 * per : 0);
#pragma unroll
    for (int r = 0; r < NRG_IN; ++r) {
      const int u = wx + r * XW;
      const int t = dn ? 0 : min(u / per, 2), rg = dn ? u : u - t * per;
      const uint16_t *tile = dn ? ly.dn_in + (size_t)x * r_in * H
                           : (t == 0) ? ly.at_q + (size_t)x * hd * H
                           : (t == 1) ? ly.at_k + (size_t)(x * nkv / nq) * hd * H
                                      : ly.at_v + (size_t)(x * nkv / nq) * hd * H;
      const __amdgpu_buffer_rsrc_t rs = tile_rsrc(tile, (u < nrg) ? (uint32_t)((rg + 1) * L_h * 1024) : 0u);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const bool ok = u < nrg && i < L_h;
        const uint32_t off = ok ? (uint32_t)(((rg * L_h + i) * 64 + lane) * 16) : OOB_OFF;
        w_in[r][i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, AUX_NT);
      }
    }
    keep_issued();
  };
  // gate/up rows of FFN slice x for this wave: pair j = rows 2j, 2j+1, contiguous in the tile
  // (two row groups when a row group is one row, one when it is two), 2 L_h / RG_h loads
  auto issue_gu = [&](ConstLayer &ly) {
    const int nl = 2 * L_h / RG_h;
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(ly.ffn_gu + (size_t)x * 2 * J * H, (uint32_t)(2 * J * H * 2));
#pragma unroll
    for (int pr = 0; pr < NPAIR; ++pr) {
      const int j = wx + pr * XW;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = j < J && i < nl;
        const uint32_t off = ok ? (uint32_t)(((j * nl + i) * 64 + lane) * 16) : OOB_OFF;
        w_gu[pr][i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, AUX_NT);
      }
    }
    keep_issued();
  };

  // Residual slice lw of every column: xres slice + the 8 XCD partials of `part` (layout
  // [col][8][H]), published to the XCD's residual slots `xr`.  With one polling wave (decode) that
  // wave gathers, sums and publishes on its own, without a barrier (its own LDS writes are seen by
  // its later reads); otherwise every wave takes part after the gather's barrier.  A watchdog
  // expiry is reported through `flag` and acted on after the next gather.
  auto reduce_slices = [&](const uint2 *part, uint2 *xr, float *tmp, int site) {
    if constexpr (NPW == 1) {
      if (w8 == MK_WAVES - 1 && poll2d<MCS, NPW>(part + lw * SL, ncol * MK_NX, SL, H, a.tag0, tmp, flag, m.ctl, site, tid0)) {
        for (int i = lane; i < ncol * SL; i += 64) {
          const int c = i / SL, k = i - c * SL;
          float sm = tmp[(c * MK_NX) * SL + k];
#pragma unroll
          for (int g = 1; g < MK_NX; ++g) sm += tmp[(c * MK_NX + g) * SL + k];
          pub_xcd(xr + c * H + lw * SL + k, xres[c * H + lw * SL + k] + sm, a.tag0);
        }
      }
    } else {
      gather2d<MCS, NPW>(part + lw * SL, ncol * MK_NX, SL, H, a.tag0, tmp, flag, m.ctl, site, tid0);
      if (*flag == 0) {
        for (int i = tid0; i < ncol * SL; i += MK_THREADS) {
          const int c = i / SL, k = i - c * SL;
          float sm = tmp[(c * MK_NX) * SL + k];
#pragma unroll
          for (int g = 1; g < MK_NX; ++g) sm += tmp[(c * MK_NX + g) * SL + k];
          pub_xcd(xr + c * H + lw * SL + k, xres[c * H + lw * SL + k] + sm, a.tag0);
        }
      }
    }
  };

  {
    const int step = 0;                    // (the watchdog's site code keeps a step field)
    const uint32_t tg = a.tag0;
    const int pos0 = ctl_pos;              // position of column 0
    int li = 0;

    // gains of the next RMSNorm: decode's weight-streaming lanes hold them in the operand layout of
    // their tile rows (rmsnorm_regs), verify's threads hold elements t and t + 512
    float g1v[16], g1a = 0.f, g1b = 0.f;
    if constexpr (NCOL == 1) {
      ld_gain16(layers[0].ln1, H, G_h, w8 < CW, g1v);
    } else {
      g1a = ld_gain(layers[0].ln1, H, tid);
      g1b = ld_gain(layers[0].ln1, H, tid + MK_THREADS);
    }
    issue_in(0);
    // ---- embedding rows
    for (int c = 0; c < ncol; ++c) {
      int t = a.tokens[c];
      if (t < 0 || t >= m.V) {
        if (tid == 0) __hip_atomic_fetch_or(m.ctl + MK_CTL_ERR, MK_DERR_TOKEN, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        t = 0;
      }
      const uint16_t *row = m.embed + (size_t)t * H;
      for (int k = tid; k < H; k += MK_THREADS) xres[c * H + k] = bfv(row[k]);
    }
    if (m.nq > 0) {
      const int half = hd / 2;
      for (int i = tid; i < ncol * half; i += MK_THREADS) {
        const int c = i / half, d = i - c * half;
        const float2 r = *reinterpret_cast<const float2 *>(m.rope + ((size_t)(pos0 + c) * half + d) * 2);
        rl[i * 2 + 0] = r.x;
        rl[i * 2 + 1] = r.y;
      }
    }
    lbar();

    for (li = 0; li < m.n_layers; ++li) {
      ConstLayer &ly = layers[li];
      // A per-layer copy of the thread index the compiler cannot see through: address
      // arithmetic derived from it stays inside the layer loop instead of being hoisted out
      // (and spilled) for the whole loop.
      int tid = tid0;
      asm volatile("" : "+v"(tid));
      const int lane = tid & 63;
      // gains of this layer's gated RMSNorm (DeltaNet), held by the last wave, which applies it in
      // D3: elements lane and lane + 64
      const int gnn = (ly.kind == 0 && w8 == MK_WAVES - 1) ? dv : 0;
      const float gnv0 = ld_gain(ly.dn_gnorm, gnn, lane), gnv1 = ld_gain(ly.dn_gnorm, gnn, lane + 64);
      // gains of this layer's FFN norm, needed after the mixer
      float g2v[16], g2a = 0.f, g2b = 0.f;
      if constexpr (NCOL == 1) {
        ld_gain16(ly.ln2, H, G_h, w8 < CW, g2v);
      } else {
        g2a = ld_gain(ly.ln2, H, tid);
        g2b = ld_gain(ly.ln2, H, tid + MK_THREADS);
      }
      // decode: each weight-streaming wave normalises the residual into registers itself (no LDS
      // pass, no barrier); verify: into hn
      float av[16];
      if constexpr (NCOL == 1) {
        if (w8 < CW) rmsnorm_regs(xres, g1v, H, G_h, L_h, m.rms_eps, av);
      } else {
        rmsnorm_cols_r<NCOL>(xres, hn, g1a, g1b, H, G_h, L_h, m.rms_eps, ncol, tid);
      }
      if (ly.kind == 0) {
        // ================================================ DeltaNet layer
        uint2 *xin = ly.x_in + (size_t)x * MK_MAXCOL * r_in_max;
        uint2 *xo = ly.x_o + (size_t)x * MK_MAXCOL * x_o_len;
        const int RW = dv / MK_NL, r0 = lw * RW;
        // ---- D1: in-projection rows of head x (weights already in flight)
        if (x < nh) {
          const int nrg = r_in / RG_h;
          if constexpr (NCOL == 1) {
            if (G_h == 64) {  // one row per row group: the three rows of this wave reduced together
              const float t = wave_sum4(dot16(w_in[0][0], w_in[0][1], av), dot16(w_in[1][0], w_in[1][1], av),
                                        dot16(w_in[2][0], w_in[2][1], av), 0.f);
              const int r = (lane == 0) ? 0 : (lane == 32) ? 1 : (lane == 16) ? 2 : NRG_IN;   // lanes holding row r
              if (r < NRG_IN && wx + r * XW < nrg) pub_xcd(xin + (wx + r * XW), t, tg);
            } else {
#pragma unroll
              for (int r = 0; r < NRG_IN; ++r) {
                const int rg = wx + r * XW;
                const float o = rg_dot_regs(w_in[r][0], w_in[r][1], G_h, av);
                if (rg < nrg && (lane & (G_h - 1)) == 0) pub_xcd(xin + rg * RG_h + lane / G_h, o, tg);
              }
            }
          } else {
#pragma unroll
            for (int r = 0; r < NRG_IN; ++r) {
              const int rg = wx + r * XW;
              if (rg < nrg) {
                float o[NCOL];
                rg_dot<NCOL, 2>(w_in[r], L_h, G_h, hn, H, ncol, o);
                if ((lane & (G_h - 1)) == 0) {
                  const int row = rg * RG_h + lane / G_h;
                  FOR_COL(c) pub_xcd(xin + c * r_in_max + row, o[c], tg);
                }
              }
            }
          }
          // prefetch: the out-projection rows (D3)
          rg_issue<NRG_O, 1>(tile_rsrc(ly.dn_out + (size_t)x * H * dv, (uint32_t)(H * dv * 2)), wx, XW, H / RG_o, 1, w_out);
          keep_issued();
        }
        // ---- D2: conv, norms, gates, delta rule on my RW rows of S
        float *qk = work;                         // [NCOL][2dk]
        float *vr = qk + NCOL * 2 * dk;           // [NCOL][RW] (RW even)
        float *ab = vr + NCOL * RW;               // [NCOL][2]
        float *nrm = ab + NCOL * 2;               // [NCOL][2]
        float *gts = nrm + NCOL * 2;              // [NCOL][2] alpha, beta
        float *outo = gts + NCOL * 2;             // [NCOL][RW]
        if (x < nh) {
          // this wave's row of S (wave w < RW owns row r0 + w; lane holds elements lane + 64 j)
          const bool act = w8 < RW;
          float *Srow = ly.S + ((size_t)x * dv + r0 + (act ? w8 : 0)) * dk;
          float s[2] = {0.f, 0.f};
          if (act) {
            s[0] = Srow[lane];
            if (dk > 64) s[1] = Srow[64 + lane];
          }
          // conv history of my channels (positions pos0-3 .. pos0-1), loaded before the waits
          const int nch = 2 * dk + RW;
          int ch = 0;
          if (tid < 2 * dk) ch = (tid < dk) ? x * dk + tid : nh * dk + x * dk + (tid - dk);
          else if (tid < nch) ch = 2 * nh * dk + x * dv + r0 + (tid - 2 * dk);
          float hist[3] = {0.f, 0.f, 0.f};
          float4 wt = make_float4(0.f, 0.f, 0.f, 0.f);
          if (tid < nch) {
            wt = *reinterpret_cast<const float4 *>(ly.dn_conv + ch * 4);
            const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(ly.ring, 0, MK_RING * nconv * 4, RSRC_W3);
#pragma unroll
            for (int i = 0; i < 3; ++i) {
              const int pp = pos0 - 3 + i;
              if (pp >= 0)
                hist[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rr, ((pp & (MK_RING - 1)) * nconv + ch) * 4, 0, AUX_DEV));
            }
          }
          {
            const GSeg sg[3] = {{0, ncol, 2 * dk, r_in_max, qk},                 // q, k pre-conv
                                {2 * dk + r0, ncol, RW, r_in_max, vr},           // my v rows
                                {2 * dk + 2 * dv, ncol, 2, r_in_max, ab}};       // a, b
            if (!gather_segs<MCS, NPW, 3>(xin, sg, tg, flag, m.ctl, SITE(1), tid)) MK_BAIL();
          }
          // conv + SiLU: threads [0, 2dk) are the q/k channels of head x, [2dk, 2dk+RW) my v channels
          {
            if (tid < nch) {
              int cstride;
              float *cur;
              if (tid < 2 * dk) {
                cur = qk + tid;
                cstride = 2 * dk;
              } else {
                cur = vr + (tid - 2 * dk);
                cstride = RW;
              }
              float raw[NCOL];
#pragma unroll
              for (int c = 0; c < NCOL; ++c) raw[c] = (c < ncol) ? cur[c * cstride] : 0.f;
              const float wv[4] = {wt.x, wt.y, wt.z, wt.w};
              FOR_COL(c) {
                float sacc = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const int cc = c - (3 - i);              // tap i meets the token 3 - i steps before column c
                  const float v = (cc >= 0) ? raw[cc < 0 ? 0 : cc] : hist[cc + 3 < 0 ? 0 : cc + 3];
                  sacc = fmaf(wv[i], v, sacc);
                }
                cur[c * cstride] = siluf_(sacc);
              }
              if (tid >= 2 * dk || lw == 0)
                FOR_COL(c) ly.ring[((pos0 + c) & (MK_RING - 1)) * nconv + ch] = raw[c];
            }
          }
          lbar();
          // L2 norms of q and k (wave w handles ranges w, w+8, ...), gates
          for (int r = w8; r < 2 * ncol; r += MK_WAVES) {
            const int c = r >> 1, which = r & 1;
            const float *p = qk + c * 2 * dk + which * dk;
            float sq = 0.f;
            for (int i = lane; i < dk; i += 64) sq = fmaf(p[i], p[i], sq);
            sq = wave_sum(sq);
            if (lane == 0) nrm[c * 2 + which] = sqrtf(sq + m.l2_eps);
          }
          if (tid < ncol) {
            gts[tid * 2 + 0] = expf(-softplusf_(ab[tid * 2 + 0]));
            gts[tid * 2 + 1] = sigmoidf_(ab[tid * 2 + 1]);
          }
          lbar();
          for (int i = tid; i < ncol * 2 * dk; i += MK_THREADS)
            qk[i] = qk[i] / nrm[(i / (2 * dk)) * 2 + ((i % (2 * dk)) >= dk)];
          lbar();
          // delta rule: S_r <- alpha S_r + beta (v_r - alpha S_r.k) k ; o_r = S_r.q (rows are independent)
          if (act) {
            const int J2 = dk / 64;
            auto rowdot = [&](const float *vec) {  // S_r . vec (vec: dk values)
              float p = fmaf(s[0], vec[lane], 0.f);
              if (J2 > 1) p = fmaf(s[1], vec[64 + lane], p);
              return wave_sum(p);
            };
            const float *pk_base = ly.pend + ((size_t)par * nh + x) * MK_MAXCOL * (dk + dv + 2);
            for (int j = 0; j < pend_n; ++j) {  // pending updates left by a verify forward
              const float *pk = pk_base + j * (dk + dv + 2);
              const float aj = pk[dk + dv], bj = pk[dk + dv + 1], vj = pk[dk + r0 + w8];
              const float sk = rowdot(pk);
              const float u = bj * (vj - aj * sk);
              s[0] = fmaf(u, pk[lane], aj * s[0]);
              if (J2 > 1) s[1] = fmaf(u, pk[64 + lane], aj * s[1]);
            }
            if (verify) {  // S after the accepted tokens; this forward's tokens become pending
              Srow[lane] = s[0];
              if (J2 > 1) Srow[64 + lane] = s[1];
            }
            FOR_COL(c) {
              const float *kc = qk + c * 2 * dk + dk, *qc = qk + c * 2 * dk;
              const float al = gts[c * 2 + 0], be = gts[c * 2 + 1];
              const float sk = rowdot(kc);
              const float u = be * (vr[c * RW + w8] - al * sk);
              s[0] = fmaf(u, kc[lane], al * s[0]);
              if (J2 > 1) s[1] = fmaf(u, kc[64 + lane], al * s[1]);
              const float o = rowdot(qc);
              if (lane == 0) outo[c * RW + w8] = o;
            }
            if (!verify) {
              Srow[lane] = s[0];
              if (J2 > 1) Srow[64 + lane] = s[1];
            }
          }
          if (verify) {  // this forward's (k, v, alpha, beta) become the pending updates
            float *pw = ly.pend + ((size_t)(par ^ 1) * nh + x) * MK_MAXCOL * (dk + dv + 2);
            for (int c = 0; c < ncol; ++c) {
              float *pc = pw + c * (dk + dv + 2);
              if (lw == 0) {
                for (int i = tid; i < dk; i += MK_THREADS) pc[i] = qk[c * 2 * dk + dk + i];
                if (tid == 0) { pc[dk + dv] = gts[c * 2]; pc[dk + dv + 1] = gts[c * 2 + 1]; }
              }
              if (tid < RW) pc[dk + r0 + tid] = vr[c * RW + tid];
            }
          }
          lbar();   // (the ring, S and pending updates written here are read by the next launch only)
          if (tid < ncol * RW) {
            const int c = tid / RW, r = tid - (tid / RW) * RW;
            pub_xcd(xo + c * x_o_len + r0 + r, outo[c * RW + r], tg);
          }
        }
        // ---- D3: gated RMSNorm + out-projection columns of head x
        if (x < nh) {
          float *o = work;                 // [NCOL][dv]
          float *z = o + NCOL * dv;        // [NCOL][dv]
          {
            const GSeg sg[2] = {{(int)(xo - xin), ncol, dv, x_o_len, o},       // o rows of the head
                                {2 * dk + dv, ncol, dv, r_in_max, z}};         // z of the head
            // with one polling wave, that wave gathers and normalises before the barrier
            if constexpr (NPW == 1) poll_segs<MCS, NPW, 2>(xin, sg, tg, flag, m.ctl, SITE(4), tid);
            else gather_segs<MCS, NPW, 2>(xin, sg, tg, flag, m.ctl, SITE(4), tid);
          }
          // gated RMSNorm of each column, by the last wave (lane: elements lane, lane + 64)
          if (w8 == MK_WAVES - 1 && *flag == 0) {
            FOR_COL(c) {
              const float a0 = o[c * dv + lane], a1 = (dv > 64) ? o[c * dv + 64 + lane] : 0.f;
              const float sq = fmaf(a1, a1, fmaf(a0, a0, 0.f));
              const float den = sqrtf(wave_sum(sq) / (float)dv + m.rms_eps);
              o[c * dv + lane] = a0 / den * gnv0 * siluf_(z[c * dv + lane]);
              if (dv > 64) o[c * dv + 64 + lane] = a1 / den * gnv1 * siluf_(z[c * dv + 64 + lane]);
            }
          }
          lbar();
          if (*flag) MK_BAIL();
#pragma unroll
          for (int r = 0; r < NRG_O; ++r) {
            const int rg = wx + r * XW;
            if (rg < H / RG_o) {
              float oo[NCOL];
              rg_dot<NCOL, 1>(w_out[r], 1, G_o, o, dv, ncol, oo);
              if ((lane & (G_o - 1)) == 0) {
                const int row = rg * RG_o + lane / G_o;
                FOR_COL(c) pub(ly.x_mix + ((size_t)c * MK_NX + x) * H + row, oo[c], tg);
              }
            }
          }
        } else {
          for (int i = tid + lw * MK_THREADS; i < H; i += MK_NL * MK_THREADS)
            for (int c = 0; c < ncol; ++c) pub(ly.x_mix + ((size_t)c * MK_NX + x) * H + i, 0.f, tg);
        }
      } else {
        // ================================================ attention layer
        const int kvh = x * nkv / nq;
        uint2 *xin = ly.x_in + (size_t)x * MK_MAXCOL * r_in_max;
        uint2 *xo = ly.x_o + (size_t)x * MK_MAXCOL * x_o_len;
        if (x < nq) {
          // ---- A1: q rows of head x, k/v rows of its kv head (weights already in flight)
          const int per = hd / RG_h;
          if constexpr (NCOL == 1) {
            if (G_h == 64) {  // as D1: three rows reduced together (row group u is row u)
              const float tt = wave_sum4(dot16(w_in[0][0], w_in[0][1], av), dot16(w_in[1][0], w_in[1][1], av),
                                         dot16(w_in[2][0], w_in[2][1], av), 0.f);
              const int r = (lane == 0) ? 0 : (lane == 32) ? 1 : (lane == 16) ? 2 : NRG_IN;
              const int u = wx + r * XW;
              if (r < NRG_IN && u < 3 * per) pub_xcd(xin + u, tt, tg);   // row t hd + rg == u when per == hd
            } else {
#pragma unroll
              for (int r = 0; r < NRG_IN; ++r) {
                const int u = wx + r * XW;
                const float o = rg_dot_regs(w_in[r][0], w_in[r][1], G_h, av);
                if (u < 3 * per && (lane & (G_h - 1)) == 0) {
                  const int t = u / per, rg = u - t * per;
                  pub_xcd(xin + t * hd + rg * RG_h + lane / G_h, o, tg);
                }
              }
            }
          } else {
#pragma unroll
            for (int r = 0; r < NRG_IN; ++r) {
              const int u = wx + r * XW;
              if (u < 3 * per) {
                const int t = u / per, rg = u - t * per;
                float o[NCOL];
                rg_dot<NCOL, 2>(w_in[r], L_h, G_h, hn, H, ncol, o);
                if ((lane & (G_h - 1)) == 0) {
                  const int row = t * hd + rg * RG_h + lane / G_h;
                  FOR_COL(c) pub_xcd(xin + c * r_in_max + row, o[c], tg);
                }
              }
            }
          }
          rg_issue<NRG_O, 1>(tile_rsrc(ly.at_o + (size_t)x * H * hd, (uint32_t)(H * hd * 2)), wx, XW, H / RG_a, 1, w_out);
          keep_issued();
          // ---- A2: RoPE, KV append, split-KV partials
          float *qkv = work;                    // [NCOL][3hd]
          if (!gather2d<MCS, NPW>(xin, ncol, 3 * hd, r_in_max, tg, qkv, flag, m.ctl, SITE(6), tid)) MK_BAIL();
          {
            const int half = hd / 2;
            for (int i = tid; i < ncol * half; i += MK_THREADS) {
              const int c = i / half, d = i - c * half;
              const float cs = rl[i * 2 + 0], sn = rl[i * 2 + 1];
              float *q = qkv + c * 3 * hd, *k = q + hd, *v = k + hd;
              const float q1 = q[d], q2 = q[d + half], k1 = k[d], k2 = k[d + half];
              q[d] = q1 * cs - q2 * sn;
              q[d + half] = q2 * cs + q1 * sn;
              k[d] = rbf(k1 * cs - k2 * sn); k[d + half] = rbf(k2 * cs + k1 * sn);
              v[d] = rbf(v[d]); v[d + half] = rbf(v[d + half]);
            }
          }
          lbar();
          // first query head of the kv group appends K, V; with a polling wave, that wave does it
          // (its wait for the stores then waits for no weight loads)
          if (lw == 0 && (x * nkv) % nq == 0 && w8 >= MK_WAVES - NPW) {
            const __amdgpu_buffer_rsrc_t kst = __builtin_amdgcn_make_buffer_rsrc(ly.kc, 0, 0x7fffffff, RSRC_W3);
            const __amdgpu_buffer_rsrc_t vst = __builtin_amdgcn_make_buffer_rsrc(ly.vc, 0, 0x7fffffff, RSRC_W3);
            for (int i = tid - (MK_WAVES - NPW) * 64; i < ncol * hd; i += NPW * 64) {
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
            float *sc = work + NCOL * 3 * hd;      // scores of my keys [<= 320]
            float *pv = sc + 320;                  // [MK_WAVES][hd] partial P.V per wave
            float *mx = pv + MK_WAVES * hd;        // [2]: max, sum
            const float scale = 1.f / sqrtf((float)hd);
            const int lpk = hd / 8;                // lanes per key
            const int kpw = 64 / lpk;              // keys per wave step
            const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(ly.kc, 0, 0x7fffffff, RSRC_W3);
            const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(ly.vc, 0, 0x7fffffff, RSRC_W3);
#pragma unroll 1
            for (int c = 0; c < ncol; ++c) {
              const int P = pos0 + c;             // query position; keys 0..P
              const int nblk = P / MK_KBLK + 1;
              const int myblk = (nblk > lw) ? (nblk - lw + MK_NL - 1) / MK_NL : 0;
              const int nk = (myblk == 0) ? 0 : (myblk - 1) * MK_KBLK + min(MK_KBLK, P + 1 - (lw + (myblk - 1) * MK_NL) * MK_KBLK);
              const float *q = qkv + c * 3 * hd;
              // scores: key slot ks -> block lw + (ks / 32) * 32, offset ks % 32.  Cached keys come
              // through branch-free buffer loads (absent ones with an out-of-range offset), so the
              // loads of several steps can be in flight together; this step's keys come from LDS.
#pragma unroll 2
              for (int base = w8 * kpw; base < nk; base += MK_WAVES * kpw) {
                const int ks = base + lane / lpk, j = ks / MK_KBLK;
                const int tpos = (lw + j * MK_NL) * MK_KBLK + (ks % MK_KBLK);
                const int d0 = (lane % lpk) * 8;
                const bool cached = ks < nk && tpos < pos0;
                const uint32_t off = cached ? (uint32_t)((((pgs[j] * nkv + kvh) * MK_PAGE + (tpos % MK_PAGE)) * hd + d0) * 2) : OOB_OFF;
                float kf[8];
                unpack8(__builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0), kf);
                // this step's keys: read from LDS for every slot (row 0 where unused) and selected,
                // so the loop body stays one block and the loads of several steps issue together
                const bool cur = ks < nk && !cached;
                const float *kk = qkv + (cur ? tpos - pos0 : 0) * 3 * hd + hd + d0;
#pragma unroll
                for (int i = 0; i < 8; ++i) kf[i] = cur ? kk[i] : kf[i];
                float sdot = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) sdot = fmaf(q[d0 + i], kf[i], sdot);
                sdot = group_sum(sdot, lpk);
                if (ks < nk && (lane % lpk) == 0) sc[ks] = sdot * scale;
              }
              lbar();
              if (w8 == 0) {
                float mv = -INFINITY;
                for (int i = lane; i < nk; i += 64) mv = fmaxf(mv, sc[i]);
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) mv = fmaxf(mv, __shfl_xor(mv, off, 64));
                float ls = 0.f;
                for (int i = lane; i < nk; i += 64) {
                  const float p = expf(sc[i] - mv);
                  sc[i] = p;
                  ls += p;
                }
                ls = wave_sum(ls);
                if (lane == 0) { mx[0] = mv; mx[1] = ls; }
              }
              lbar();
              // P.V: wave w takes keys w, w+8, ...; lane l takes dims l dpl .. +dpl (one 2- or 4-byte
              // load per key, branch-free as above)
              {
                const int dpl = hd / 64;   // 1 or 2
                float acc[2] = {0.f, 0.f};
#pragma unroll 4
                for (int ks = w8; ks < nk; ks += MK_WAVES) {
                  const int j = ks / MK_KBLK, tpos = (lw + j * MK_NL) * MK_KBLK + (ks % MK_KBLK);
                  const bool cached = tpos < pos0;
                  const uint32_t off = cached ? (uint32_t)((((pgs[j] * nkv + kvh) * MK_PAGE + (tpos % MK_PAGE)) * hd + lane * dpl) * 2) : OOB_OFF;
                  float v0, v1;
                  if (dpl == 2) {
                    const uint32_t raw = __builtin_amdgcn_raw_buffer_load_b32(vrs, off, 0, 0);
                    v0 = __uint_as_float(raw << 16);
                    v1 = __uint_as_float(raw & 0xffff0000u);
                  } else {
                    v0 = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(vrs, off, 0, 0) << 16);
                    v1 = 0.f;
                  }
                  const float *vv = qkv + (cached ? 0 : tpos - pos0) * 3 * hd + 2 * hd + lane * dpl;
                  const float l0 = vv[0], l1 = (dpl == 2) ? vv[1] : 0.f;
                  v0 = cached ? v0 : l0;
                  v1 = cached ? v1 : l1;
                  const float p = sc[ks];
                  acc[0] = fmaf(p, v0, acc[0]);
                  acc[1] = fmaf(p, v1, acc[1]);
                }
                pv[w8 * hd + lane * dpl] = acc[0];
                if (dpl == 2) pv[w8 * hd + lane * dpl + 1] = acc[1];
              }
              lbar();
              const int plen = hd + 2;
              uint2 *dst = xo + c * x_o_len + lw * plen;
              for (int d = tid; d < hd; d += MK_THREADS) {
                float acc = pv[d];
#pragma unroll 1
                for (int ww = 1; ww < MK_WAVES; ++ww) acc += pv[ww * hd + d];
                pub_xcd(dst + 2 + d, acc, tg);
              }
              if (tid == 0) {
                pub_xcd(dst + 0, nk > 0 ? mx[0] : -INFINITY, tg);
                pub_xcd(dst + 1, nk > 0 ? mx[1] : 0.f, tg);
              }
              lbar();
            }
          }
          // ---- A3: merge the 32 partials + o-projection columns of head x
          {
            const int plen = hd + 2;
            float *part = work + 2048;             // [32][plen]
            float *ov = work;                      // [NCOL][hd]
            for (int c = 0; c < ncol; ++c) {
              if (!gather2d<5, MK_WAVES>(xo + c * x_o_len, 1, MK_NL * plen, 0, tg, part, flag, m.ctl, SITE(7), tid)) MK_BAIL();
              // per-partial scale exp(m_w - M) (0 for workgroups without keys), once, in wave 0
              float *scl = part + MK_NL * plen;     // [32] scales, [32] = sum of l_w * scale
              if (w8 == 0) {
                const bool has = lane < MK_NL && part[lane * plen + 1] > 0.f;
                float M = has ? part[lane * plen] : -INFINITY;
#pragma unroll
                for (int off = 16; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
                const float sv = has ? expf(part[lane * plen] - M) : 0.f;
                if (lane < MK_NL) scl[lane] = sv;
                if (lane == 0) {  // (LDS writes of one wave are seen by its later reads)
                  float Ls = 0.f;
                  for (int ww = 0; ww < MK_NL; ++ww) Ls = fmaf(part[ww * plen + 1], scl[ww], Ls);
                  scl[MK_NL] = Ls;
                }
              }
              lbar();
              for (int d = tid; d < hd; d += MK_THREADS) {
                float acc = 0.f;
#pragma unroll 8
                for (int ww = 0; ww < MK_NL; ++ww) acc = fmaf(part[ww * plen + 2 + d], scl[ww], acc);
                ov[c * hd + d] = acc / scl[MK_NL];
              }
              lbar();
            }
#pragma unroll
            for (int r = 0; r < NRG_O; ++r) {
              const int rg = wx + r * XW;
              if (rg < H / RG_a) {
                float oo[NCOL];
                rg_dot<NCOL, 1>(w_out[r], 1, G_a, ov, hd, ncol, oo);
                if ((lane & (G_a - 1)) == 0) {
                  const int row = rg * RG_a + lane / G_a;
                  FOR_COL(c) pub(ly.x_mix + ((size_t)c * MK_NX + x) * H + row, oo[c], tg);
                }
              }
            }
          }
        } else {
          for (int i = tid + lw * MK_THREADS; i < H; i += MK_NL * MK_THREADS)
            for (int c = 0; c < ncol; ++c) pub(ly.x_mix + ((size_t)c * MK_NX + x) * H + i, 0.f, tg);
        }
      }
      // prefetch: gate/up rows of FFN slice x (F1), in flight during the residual reduction
      issue_gu(ly);
      // ---- R1: residual += sum of the 8 mixer slices (reduce-scatter over XCDs, all-gather in the XCD)
      {
        // [NCOL*8][SL], apart from everything the mixer phases read: the polling wave fills it
        // while the other waves may still be reading the out-projection operand
        float *tmp = work + 6400;
        uint2 *xr = ly.x_r1 + (size_t)x * MK_MAXCOL * H;
        reduce_slices(ly.x_mix, xr, tmp, SITE(8));
        if (!gather2d<MCL, NPW>(xr, ncol, H, H, tg, xres, flag, m.ctl, SITE(9), tid)) MK_BAIL();
      }
      // ================================================================ FFN
      if constexpr (NCOL == 1) {
        if (w8 < CW) rmsnorm_regs(xres, g2v, H, G_h, L_h, m.rms_eps, av);
      } else {
        rmsnorm_cols_r<NCOL>(xres, hn, g2a, g2b, H, G_h, L_h, m.rms_eps, ncol, tid);
      }
      {
        uint2 *xm = ly.x_m + (size_t)x * MK_MAXCOL * xm_len;
        // ---- F1: gate/up pairs j -> m_j = SiLU(g_j) * u_j (weights already in flight)
        if constexpr (NCOL == 1) {
          if (RG_h == 1 && L_h == 2) {
            // both pairs at once: lanes [0,16) gate 0, [16,32) gate 1, [32,48) up 0, [48,64) up 1;
            // the permlane32 swap then puts gate and up of pair 0 in lane 0 and of pair 1 in lane 16
            const float t = wave_sum4(dot16(w_gu[0][0], w_gu[0][1], av), dot16(w_gu[0][2], w_gu[0][3], av),
                                      dot16(w_gu[1][0], w_gu[1][1], av), dot16(w_gu[1][2], w_gu[1][3], av));
            const u32x2 gu = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
            const int j = wx + (lane >> 4) * XW;
            if ((lane == 0 || lane == 16) && j < J) pub_xcd(xm + j, siluf_(__uint_as_float(gu.x)) * __uint_as_float(gu.y), tg);
          } else {
#pragma unroll
            for (int pr = 0; pr < NPAIR; ++pr) {
              const int j = wx + pr * XW;
              float g, u;
              if (RG_h == 1) {  // gate = loads [0, L_h), up = loads [L_h, 2 L_h)
                g = rg_dot_regs(w_gu[pr][0], L_h == 2 ? w_gu[pr][1] : u32x4{0u, 0u, 0u, 0u}, G_h, av);
                u = rg_dot_regs(L_h == 2 ? w_gu[pr][2] : w_gu[pr][1], L_h == 2 ? w_gu[pr][3] : u32x4{0u, 0u, 0u, 0u}, G_h, av);
              } else {  // one row group holds the pair: lanes [0,32) compute g_j, lanes [32,64) u_j
                g = rg_dot_regs(w_gu[pr][0], w_gu[pr][1], G_h, av);
                u = __shfl_xor(g, 32, 64);
              }
              if (lane == 0 && j < J) pub_xcd(xm + j, siluf_(g) * u, tg);
            }
          }
        } else {
#pragma unroll
          for (int pr = 0; pr < NPAIR; ++pr) {
            const int j = wx + pr * XW;
            if (j < J) {
              float g[NCOL], u[NCOL];
              if (RG_h == 1) {  // gate = loads [0, L_h), up = loads [L_h, 2 L_h)
                const u32x4 wg[2] = {w_gu[pr][0], w_gu[pr][1]};
                const u32x4 wu[2] = {L_h == 2 ? w_gu[pr][2] : w_gu[pr][1], w_gu[pr][3]};
                rg_dot<NCOL, 2>(wg, L_h, G_h, hn, H, ncol, g);
                rg_dot<NCOL, 2>(wu, L_h, G_h, hn, H, ncol, u);
              } else {  // one row group holds the pair: lanes [0,32) compute g_j, lanes [32,64) u_j
                const u32x4 wg[2] = {w_gu[pr][0], w_gu[pr][1]};
                rg_dot<NCOL, 2>(wg, L_h, G_h, hn, H, ncol, g);
#pragma unroll
                for (int c = 0; c < NCOL; ++c) u[c] = __shfl_xor(g[c], 32, 64);
              }
              if (lane == 0) FOR_COL(c) pub_xcd(xm + c * xm_len + j, siluf_(g[c]) * u[c], tg);
            }
          }
        }
        // prefetch: down-projection rows (F2), in flight during the m hand-off
        const uint16_t *tile = ly.ffn_dn + (size_t)x * H * J;
        const int nrg = H / RG_d;
        rg_issue<1, LMAX_D>(tile_rsrc(tile, (uint32_t)(H * J * 2)), wx, XW, nrg, L_d, w_dn);
        keep_issued();
        // ---- F2: down-projection columns of slice x
        float *mv = work;  // [NCOL][J]
        if (!gather2d<MCS, NPW>(xm, ncol, J, xm_len, tg, mv, flag, m.ctl, SITE(11), tid)) MK_BAIL();
        if (wx < nrg) {
          float oo[NCOL];
          rg_dot_dn<NCOL, LMAX_D>(w_dn[0], L_d, G_d, mv, J, ncol, oo);
          if ((lane & (G_d - 1)) == 0) {
            const int row = wx * RG_d + lane / G_d;
            FOR_COL(c) pub(ly.x_ffn + ((size_t)c * MK_NX + x) * H + row, oo[c], tg);
          }
        }
      }
      // prefetch: the next layer's in-projection / QKV rows, in flight during the reduction
      // (gains first: the in-order wait for them at the next norm then excludes the weights)
      {
        const bool more = li + 1 < m.n_layers;
        const float *gsrc = more ? layers[li + 1].ln1 : m.lnf;   // else the final norm's gains
        if constexpr (NCOL == 1) {
          ld_gain16(gsrc, H, G_h, w8 < CW || !more, g1v);   // every wave takes part in the LM head
        } else {
          g1a = ld_gain(gsrc, H, tid);
          g1b = ld_gain(gsrc, H, tid + MK_THREADS);
        }
        issue_in(li + 1);
      }
      // ---- R2: residual += sum of the 8 FFN slices
      {
        float *tmp = work + 6400;  // [NCOL*8][SL], apart from the down-projection operand mv
        uint2 *xr = ly.x_r2 + (size_t)x * MK_MAXCOL * H;
        reduce_slices(ly.x_ffn, xr, tmp, SITE(12));
        if (!gather2d<MCL, NPW>(xr, ncol, H, H, tg, xres, flag, m.ctl, SITE(13), tid)) MK_BAIL();
      }
    }  // layers

    // ================================================================ LM head + greedy argmax
    float avf[16];   // decode: the final norm in registers (every wave)
    if constexpr (NCOL == 1) rmsnorm_regs(xres, g1v, H, G_h, L_h, m.rms_eps, avf);
    else rmsnorm_cols_r<NCOL>(xres, hn, g1a, g1b, H, G_h, L_h, m.rms_eps, ncol, tid0);
    {
      const int nrg_all = m.V / RG_h;
      const int g0 = (int)((long long)b * nrg_all / MK_NWG), g1 = (int)((long long)(b + 1) * nrg_all / MK_NWG);
      const int cnt = g1 - g0;
      const int wg0 = g0 + w8 * cnt / MK_WAVES, wg1 = g0 + (w8 + 1) * cnt / MK_WAVES;
      constexpr int B = LM_BATCH(NCOL);
      float best[NCOL];
      int bidx[NCOL];
      int nanf = 0;
#pragma unroll
      for (int c = 0; c < NCOL; ++c) { best[c] = -INFINITY; bidx[c] = 0x7fffffff; }
      // this lane's activations: elements (i*G_h + lane % G_h)*8 + e of load i (L_h <= 2)
      float av[NCOL][16];
      {
        const int kl = (lane & (G_h - 1)) * 8;
#pragma unroll
        for (int c = 0; c < NCOL; ++c)
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e)
              av[c][i * 8 + e] = (NCOL == 1) ? avf[i * 8 + e] : (c < ncol && i < L_h) ? hn[c * H + i * G_h * 8 + kl + e] : 0.f;
      }
      // embedding rows stream through two register batches: the next batch's loads are issued
      // before the current one is multiplied (branch-free: rows past this wave's range read zeros)
      const __amdgpu_buffer_rsrc_t ers = tile_rsrc(m.embed, (uint32_t)((size_t)m.V * H * 2));
      auto lm_load = [&](int rb, u32x4 (&wr)[B][2]) {
#pragma unroll
        for (int r = 0; r < B; ++r) {
          const bool ok = rb + r < wg1;
          const uint32_t o0 = ok ? (uint32_t)(((size_t)(rb + r) * L_h * 64 + lane) * 16) : OOB_OFF;
          wr[r][0] = __builtin_amdgcn_raw_buffer_load_b128(ers, o0, 0, AUX_NT);
          wr[r][1] = (L_h > 1) ? __builtin_amdgcn_raw_buffer_load_b128(ers, ok ? o0 + 1024u : OOB_OFF, 0, AUX_NT)
                               : u32x4{0u, 0u, 0u, 0u};
        }
      };
      auto lm_compute = [&](int rb, const u32x4 (&wr)[B][2]) {
#pragma unroll
        for (int c = 0; c < NCOL; ++c) {
          if (c >= ncol) break;
          if (G_h == 64 && B == 8) {
            float part[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) part[r] = dot16(wr[r][0], wr[r][1], av[c]);
            const float tot = reduce8(part);           // lane l: row rb + (l >> 3)
            const int row = rb + (lane >> 3);
            if ((lane & 7) == 0 && row < wg1) {
              if (a.logits) a.logits[(size_t)c * m.V + row] = tot;
              if (!(tot == tot) || isinf(tot)) nanf = 1;
              if (tot > best[c] || (tot == best[c] && row < bidx[c])) { best[c] = tot; bidx[c] = row; }
            }
          } else {
#pragma unroll
            for (int r = 0; r < B; ++r) {
              const int rg = rb + r;
              const float pl = dot16(wr[r][0], wr[r][1], av[c]);
              const float tot = (G_h == 64) ? wave_sum_lm(pl) : group_sum(pl, G_h);
              const int row = rg * RG_h + lane / G_h;
              if ((lane & (G_h - 1)) == 0 && rg < wg1) {
                if (a.logits) a.logits[(size_t)c * m.V + row] = tot;
                if (!(tot == tot) || isinf(tot)) nanf = 1;
                if (tot > best[c] || (tot == best[c] && row < bidx[c])) { best[c] = tot; bidx[c] = row; }
              }
            }
          }
        }
      };
      u32x4 wa[B][2], wb[B][2];
      lm_load(wg0, wa);
      for (int rb = wg0; rb < wg1; rb += 2 * B) {
        lm_load(rb + B, wb);
        lm_compute(rb, wa);
        lm_load(rb + 2 * B, wa);
        lm_compute(rb + B, wb);
      }
      // wave reduce (value desc, index asc), then across waves
      float *rv = work;                  // [NCOL][8]
      int *ri = reinterpret_cast<int *>(work + 64);
      int *rn = reinterpret_cast<int *>(work + 128);
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
      const int anynan = __any(nanf) ? 1 : 0;
      if (lane == 0) rn[w8] = anynan;
      lbar();
      if (tid < ncol) {
        const int c = tid;
        float bv = rv[c * 8];
        int bi = ri[c * 8];
        int nn = 0;
        for (int ww = 0; ww < MK_WAVES; ++ww) {
          nn |= rn[ww];
          if (rv[c * 8 + ww] > bv || (rv[c * 8 + ww] == bv && ri[c * 8 + ww] < bi)) { bv = rv[c * 8 + ww]; bi = ri[c * 8 + ww]; }
        }
        unsigned long long *rec = reinterpret_cast<unsigned long long *>(m.x_arg + c * MK_NWG + b);
        __hip_atomic_store(rec, ((unsigned long long)(uint32_t)bi << 32) | __float_as_uint(bv), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        wait_stores();  // value and index land before the tag word
        __hip_atomic_store(rec + 1, ((unsigned long long)(uint32_t)nn << 32) | tg, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    lbar();  // the candidate above was read from the scratch the final gather reuses
    if (b == 0) {
      // final argmax over the 256 workgroup candidates; the tag word is written after the
      // value/index word by the same thread, so a matching tag implies the record is complete
      float *cv = work;                         // [NCOL][256]
      int *ci = reinterpret_cast<int *>(work + NCOL * MK_NWG);
      int *cn = reinterpret_cast<int *>(work + 2 * NCOL * MK_NWG);
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(m.x_arg, 0, MK_MAXCOL * MK_NWG * 16, RSRC_W3);
      for (int i = tid; i < ncol * MK_NWG; i += MK_THREADS) {
        const unsigned long long deadline = wall_clock64() + MK_WAIT_TICKS;
        while (true) {
          const uint32_t tw = __builtin_amdgcn_raw_buffer_load_b32(rs, i * 16 + 8, 0, AUX_DEV);
          if (tw == tg) break;
          if (wall_clock64() > deadline) { flag[0] = 1; break; }
          __builtin_amdgcn_s_sleep(1);
        }
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, i * 16, 0, AUX_DEV);
        cv[i] = __uint_as_float(v.x);
        ci[i] = (int)v.y;
        cn[i] = (int)v.w;
      }
      lbar();
      if (flag[0]) MK_BAIL();
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
          const int consumed = verify ? nacc : 1;
          __hip_atomic_store(m.ctl + MK_CTL_POS, ctl_pos + consumed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(m.ctl + MK_CTL_PEND, verify ? nacc : 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(m.ctl + MK_CTL_PAR, verify ? (par ^ 1) : par, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }
}
