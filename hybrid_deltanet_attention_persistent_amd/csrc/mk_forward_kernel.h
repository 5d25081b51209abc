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
//   * Two roles per XCD: 16 workgroups run the token mixer (DeltaNet or attention) of
//     every layer, the other 16 the FFN.  A role loads the weight rows of its next phase
//     into registers at the end of its current one, so they stream from HBM while the
//     other role computes; when a role's phase starts its weights are in registers and
//     nothing is queued in front of its polls (a CU's loads return in order, so a poll
//     issued behind a burst of weight loads waits for the whole burst).
//   * No grid barrier.  Every hand-off is a tagged exchange slot {value, tag} written
//     once per forward; a consumer polls the slots it needs until every tag equals the
//     forward's tag.  Slots are read with device-coherent (sc1) loads, which skip the
//     per-CU L1; a slot read by other XCDs is written with device scope, a slot read only
//     inside the writer's XCD stops in that XCD's L2.
//   * XCD x owns DeltaNet head x / query head x and FFN intermediate slice x, so
//     in-projection -> conv -> delta rule -> gated norm -> out-projection stay inside one
//     XCD; the out-projection and the FFN down-projection are split over XCDs along their
//     input dimension.  The role that produced the split-K partials sums them (a
//     reduce-scatter over the XCDs: each workgroup one slice of the residual) and the
//     other role gathers the slices inside the XCD at the start of its phase.
//   * Weights stream once per forward in a tile layout that makes every wave load a
//     contiguous 1 KiB (mk_layout.h).
//   * Decode and verify use the same per-column arithmetic in the same order, so a
//     verify forward's logits are bit-identical to sequential decode steps.
//
// The kernel template is instantiated in two translation units, mk_forward.hip (one decode
// column) and mk_verify.hip (MK_MAXCOL verify columns), so that each is compiled on its own.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <type_traits>
#include "mk_layout.h"

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define MK_WAIT_TICKS 20000000ull   // watchdog: 0.2 s of the 100 MHz device wall clock
#define AUX_DEV 16                  // sc1: device-coherent
#define RSRC_W3 0x00020000

// per-wave register budgets of the prefetched weight rows (checked against the model on the host)
#define NRG_IN 5   // mixer role: in-projection / QKV row groups per wave (two loads each)
#define NRG_O 2    // mixer role: out- / o-projection row groups per wave (one load each)
#define NPAIR 4    // FFN role: gate/up row pairs per wave (four loads each)
#define LMAX_D 8   // FFN role: loads per lane of one down-projection row group
#define NWR 24     // registers (u32x4) of the larger role: 4 NPAIR + LMAX_D >= 2 NRG_IN + NRG_O
#define NKV_PRE 6  // mixer role: attention key steps whose cached K and V rows are prefetched (2 NKV_PRE spare registers)
#define KV_GRP 4   // later key steps whose loads are issued together
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

// Gates and activations with the hardware exponential (v_exp_f32) and a fast divide: a few ulp,
// far inside the parity bar, and a fraction of the instructions of the correctly rounded forms.
__device__ __forceinline__ float sigmoid_f(float x) { return __fdividef(1.f, 1.f + __expf(-x)); }
__device__ __forceinline__ float silu_f(float x) { return __fdividef(x, 1.f + __expf(-x)); }
// exp(-softplus(a)) == 1 / (1 + e^a)
__device__ __forceinline__ float decay_f(float a) { return __fdividef(1.f, 1.f + __expf(a)); }

// Cross-lane sums with DPP (no LDS traffic).  Within a 16-lane row: xor 1 and xor 2 (quad
// permutes), then the half-row and row mirrors pair up 4- and 8-lane groups; every lane of the
// group ends with the same value (a + b == b + a).  Across rows the four row totals are added in
// a fixed order.
#define DPP_XOR1 0xB1       // quad_perm [1,0,3,2]
#define DPP_XOR2 0x4E       // quad_perm [2,3,0,1]
#define DPP_HALF_MIRROR 0x141
#define DPP_MIRROR 0x140
#define DPP_ROR8 0x128      // row_ror:8
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
  // the watchdog clock is read every 64 rounds only (a clock read is a scalar memory round trip
  // that would otherwise lengthen every round)
  unsigned long long deadline = 0;
  uint32_t rounds = 0;
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
    if ((++rounds & 63) != 0) continue;
    const unsigned long long now = wall_clock64();
    if (deadline == 0) deadline = now + MK_WAIT_TICKS;
    else if (now > deadline) {
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
// dst[nrow][ncol] (LDS), polling until every tag equals `tag`.  The last NPW waves poll, in rounds
// of MAXC chunks per lane (a wave that polls waits for every older load of its own).  Every thread
// calls it; it ends with a barrier.  On watchdog expiry records the first failing site in the
// control block and returns false.
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
__device__ __forceinline__ float rms_scale(float sumsq, int H, float eps) { return rsqrtf(sumsq / (float)H + eps); }

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
// loop over the live columns at run time, for bodies that index no register array by column: one
// copy of the body.  (Measured: 8 KB of code that never runs made decode 4 % slower, so the
// multi-column kernels keep one copy of each GEMV phase instead of NCOL.)
#define FOR_COL_R(c) _Pragma("unroll 1") for (int c = 0; c < NCOL && c < ncol; ++c)

// On a watchdog expiry the whole workgroup records the error and leaves; the other
// workgroups then time out on its missing outputs and leave too.
#define MK_BAIL()                                                                                   \
  do {                                                                                              \
    if (tid == 0)                                                                                   \
      __hip_atomic_fetch_or(m.ctl + MK_CTL_ERR, MK_DERR_HANG, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); \
    return;                                                                                         \
  } while (0)
#define SITE(ph) ((step << 16) | (li << 8) | (ph))

// Timestamp hook at phase boundaries (empty unless a tracing build defines it).
#ifndef MK_TRACE_POINT
#define MK_TRACE_POINT(li, ev)
#endif

typedef const __attribute__((address_space(4))) MkLayerDev ConstLayer;

// Byte offset of elements [d, d + 8) of the cached key or value row of position k, kv head kvh,
// in the paged cache [page][kv head][MK_PAGE][hd] (page table in LDS).
__device__ __forceinline__ uint32_t kv_off(const int *ptl, int k, int kvh, int nkv, int hd, int d) {
  return (uint32_t)((((ptl[k / MK_PAGE] * nkv + kvh) * MK_PAGE + (k % MK_PAGE)) * hd + d) * 2);
}

// 8-bit cache: byte offset of codes [d, d + 16) of a cached row, and of the row's exponent pair
// (K exponent, V exponent) in [page][kv head][MK_PAGE][2].
__device__ __forceinline__ uint32_t kv8_off(const int *ptl, int k, int kvh, int nkv, int hd, int d) {
  return (uint32_t)(((ptl[k / MK_PAGE] * nkv + kvh) * MK_PAGE + (k % MK_PAGE)) * hd + d);
}
__device__ __forceinline__ uint32_t kve_off(const int *ptl, int k, int kvh, int nkv) {
  return (uint32_t)(((ptl[k / MK_PAGE] * nkv + kvh) * MK_PAGE + (k % MK_PAGE)) * 2);
}
// A cached row's dims [d0, d0 + DPL) as FP32: 8 bf16 values (DPL 8), or 16 int8 codes (DPL 16,
// two's complement, lowest byte first; one sign-extending convert each), whose row scale 2^e the
// caller applies once per dot product / per probability.  (The codes are converted where used:
// hoisted out of the column loop, every prefetched row's would be live at once.)
template <int DPL>
__device__ __forceinline__ void kv_unpack(const u32x4 &w, float (&f)[DPL]) {
  if constexpr (DPL == 16) {
    u32x4 v = w;
    asm volatile("" : "+v"(v));
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) f[4 * i + j] = (float)(int)(int8_t)(u[i] >> (8 * j));
  } else {
    unpack8(w, f);
  }
}
// 2^e as FP32 for an 8-bit cache exponent e in [-126, 127] (given as its byte)
__device__ __forceinline__ float q8_scale(uint32_t eb) { return __uint_as_float((uint32_t)((int)(int8_t)eb + 127) << 23); }

// ------------------------------------------------------------------------------ the kernel
template <int NCOL, int SH>
__global__ void __launch_bounds__(MK_THREADS, 1) mk_forward(MkLaunch a) {
  extern __shared__ float lds_raw[];
  const MkDev &m = a.m;
  // Placement: the dispatcher puts workgroup blockIdx.x on XCD (blockIdx.x + r) mod 8, round-robin
  // from a starting XCD r that work on other hardware queues moves (measured on the device: r = 0
  // when only one queue has run kernels, other values after kernels on a second stream).  So the
  // XCD is read from the hardware and the index inside the XCD is blockIdx.x / 8, which names each
  // (XCD, index) pair once for any r and keeps which compute units take which role; b is the
  // logical workgroup index used for every partition of the work.  The final gather checks that
  // every workgroup saw the same r.
  const int lw = (int)(blockIdx.x >> 3);
  int x, rot;
  {
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    x = (int)(xcc & (MK_NX - 1));
    rot = (x - (int)blockIdx.x) & (MK_NX - 1);
  }
  const int b = x + MK_NX * lw;
  // role of this workgroup: the first MK_NG workgroups of an XCD run the token mixer (DeltaNet
  // or attention) of every layer, the other MK_NG the FFN; lg is the index inside the role
  const bool mixer = lw < MK_NG;
  const int lg = lw & (MK_NG - 1);
  // the wave index is wave-uniform: read it into a scalar register so that every row-group
  // index derived from it is scalar too
  const int w8 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id(), tid0 = threadIdx.x;
  constexpr int XW = MK_NG * MK_WAVES;                        // weight-streaming waves per role and XCD
  const int wx = lg * MK_WAVES + w8;                          // this wave's index among them
  // SH == MK_SHAPE_H1024 fixes every dimension of the hidden-1024 model (8 DeltaNet heads with
  // d_k = d_v = 128, 8 query and 2 KV heads of 128, FFN 3584) at compile time: tile strides,
  // row-group counts and reduction widths fold into straight-line code.  SH == MK_SHAPE_ANY reads
  // them from the launch arguments.
  constexpr bool FX = (SH & MK_SHAPE_H1024) != 0;
  // MK_KV_Q8: the KV cache holds int8 codes with one exponent per row; a lane then takes 16
  // dimensions of a cached row per 16-byte load instead of 8
  constexpr bool KVQ = (SH & MK_KV_Q8) != 0;
  constexpr int DPL = KVQ ? 16 : 8;
  // MK_BATCH: column c is a decode step of its own sequence (state and KV cache through
  // a.seq_layers[c], position a.seq_ctl[c][MK_CTL_POS]); no verify semantics, no pending updates
  constexpr bool BAT = (SH & MK_BATCH) != 0;
  static_assert(!BAT || (NCOL == MK_MAXCOL && !KVQ), "batch launches: MK_MAXCOL columns, bf16 cache");
  // attention key steps prefetched with the weights (batch: the first two steps of every column,
  // from its own cache: step 0 in slots 2c, 2c + 1 of the prefetch registers, loaded with the
  // weights; step 1 in registers 2c, 2c + 1, loaded at the start of A2)
  constexpr int NPRE = BAT ? 2 : KVQ ? 3 : NKV_PRE;
  const int H = FX ? 1024 : m.H;
  // the layer table is read-only: reading it through the constant address space gives
  // scalar loads, so every pointer taken from it is known to be wave-uniform
  ConstLayer *const layers = (ConstLayer *)(uintptr_t)m.layers;

  float *xres = lds_raw;                        // [NCOL][H] residual stream
  constexpr int WORK = NCOL == 1 ? 8192 : 12288;  // phase scratch (verify: the merge of all columns' partials)
  float *work = xres + NCOL * H;                // [WORK] phase scratch
  float *red = work + WORK;                     // [64] reductions
  int *flag = reinterpret_cast<int *>(red + 64);
  // batch: the columns' sequence positions, for loops whose column index is not a compile-time
  // constant (written at start, first read after many barriers)
  int *bposl = flag + 8;                        // [NCOL] (flag[8 .. 8 + NCOL))
  // the page table of the KV cache (logical page -> physical page), read once per launch
  int *ptl = flag + 16;                         // [160] (10240 positions / 64)
  // RoPE cos / sin of this launch's positions [NCOL][hd / 2][2] (hd <= 128), loaded with the
  // embedding rows so that no attention layer waits for them
  float *rl = reinterpret_cast<float *>(ptl + 160);
  for (int i = tid0; i < m.max_pages; i += MK_THREADS) ptl[i] = m.page_table[i];
  if (BAT && tid0 < NCOL)
    bposl[tid0] = tid0 < a.n ? __hip_atomic_load(a.seq_ctl[tid0] + MK_CTL_POS, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
  if (tid0 == 0) flag[0] = flag[1] = 0;

  const int ctl_pos = BAT ? 0 : __hip_atomic_load(m.ctl + MK_CTL_POS, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int pend_n = BAT ? 0 : __hip_atomic_load(m.ctl + MK_CTL_PEND, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int par = BAT ? 0 : __hip_atomic_load(m.ctl + MK_CTL_PAR, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const bool verify = !BAT && a.n > 1;
  // batch: every column's sequence position (wave-uniform); bsel picks column c's entry of a
  // per-column array for a c that is not a compile-time constant, without indexing registers
  int bpos[NCOL];
#pragma unroll
  for (int c = 0; c < NCOL; ++c)
    bpos[c] = (BAT && c < a.n) ? __builtin_amdgcn_readfirstlane(
                                     __hip_atomic_load(a.seq_ctl[c] + MK_CTL_POS, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                               : 0;

  const int ncol = a.n;
  const int G_h = mk_tile_G(H), L_h = H / 8 / G_h, RG_h = 64 / G_h;
  const int SL = H / MK_NG;  // residual slice per workgroup in the reductions
  const int nh = FX ? 8 : m.nh, dk = FX ? 128 : m.dk, dv = FX ? 128 : m.dv;
  const int nq = FX ? 8 : m.nq, nkv = FX ? 2 : m.nkv, hd = FX ? 128 : m.hd, J = FX ? 448 : m.J;
  const int r_in = FX ? 514 : m.r_in, nconv = FX ? 3072 : m.C;
  const int r_in_max = FX ? 544 : m.r_in_max, x_o_len = FX ? 2080 : m.x_o_len, xm_len = FX ? 448 : m.xm_len;
  const int G_o = mk_tile_G(dv), RG_o = 64 / G_o;        // out-projection columns of one head: L == 1
  const int G_a = mk_tile_G(hd), RG_a = 64 / G_a;        // o-projection columns of one head: L == 1
  const int G_d = mk_tile_G(J), L_d = J / 8 / G_d, RG_d = 64 / G_d;
  const int RW = dv / MK_NG, r0 = lg * RW;               // DeltaNet: rows of S owned by this workgroup
  const int CPW = 2 * dk / MK_WAVES;                     // DeltaNet: q/k conv channels per wave
  constexpr int MCS = NCOL;                              // polled chunks per lane and round
  const int step = 0;                                    // (the watchdog's site code keeps a step field)
  const uint32_t tg = a.tag0;
  const int pos0 = ctl_pos;                              // position of column 0
  int li = 0;

  // Weight rows in registers, loaded one phase of the other role ahead: the mixer role keeps its
  // in-projection / QKV row groups in wr[0, 2 NRG_IN) and its out- / o-projection row groups in
  // wr[2 NRG_IN, 2 NRG_IN + NRG_O); the FFN role its gate/up pairs in wr[0, 4 NPAIR) and its
  // down-projection row group in wr[4 NPAIR, 4 NPAIR + LMAX_D).
  u32x4 wr[NWR];
  // batch: column c's prefetched K (KV false) or V (KV true) row, for a c that is not a
  // compile-time constant.  (Each candidate passes an empty asm first: a select between loads of
  // the register array could otherwise be folded into one load at a computed index, which would
  // move the whole array to scratch memory.)
  // Step 0 sits in the prefetch slots, step 1 in the slots of the in-projection rows (free once
  // A1 has used them).
  auto wsel = [&](int c, auto kvc, auto stc) {
    constexpr int kv = decltype(kvc)::value, base = decltype(stc)::value == 0 ? 2 * NRG_IN + NRG_O : 0;
    u32x4 v = wr[base + kv];
    asm volatile("" : "+v"(v));
#pragma unroll
    for (int j = 1; j < NCOL; ++j) {
      u32x4 t = wr[base + 2 * j + kv];
      asm volatile("" : "+v"(t));
      v = (c == j) ? t : v;
    }
    return v;
  };
  float gv[16];                                          // gains of the role's RMSNorm (operand layout)
  // DeltaNet state of this wave for the next mixer phase, loaded with its weights
  float srow[2] = {0.f, 0.f}, hist[3] = {0.f, 0.f, 0.f}, grow = 0.f;
  float4 cwt = make_float4(0.f, 0.f, 0.f, 0.f);
  // A lane's conv channel in D2: q/k channel w8 CPW + lane (lane < CPW) or, in lane 63, the v
  // channel of the wave's row of S.  (Computed where used from a lane index the compiler cannot
  // see through, so that nothing derived from it is hoisted out of the layer loop.)
  auto conv_channel = [&](int ln) {
    const int cq = w8 * CPW + ln;
    return (ln < CPW) ? ((cq < dk) ? x * dk + cq : nh * dk + x * dk + (cq - dk)) : 2 * nh * dk + x * dv + r0 + w8;
  };

  // (each issue computes its per-lane offsets from a lane index the compiler cannot see through,
  // so they are not hoisted out of the layer loop and kept live -- and spilled -- across it)
  auto issue_mixer = [&](int l) {   // l == n_layers: nothing to load (every slot reads zeros)
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const bool live = l < m.n_layers;
    // (read through readfirstlane: the layer index stays in a scalar register, so the table is
    // read with scalar loads and every tile descriptor is wave-uniform)
    ConstLayer &ly = layers[__builtin_amdgcn_readfirstlane(live ? l : 0)];
    const bool dn = ly.kind == 0;
    const int per = hd / RG_h;                     // row groups of one attention head
    const int nrg = !live ? 0 : dn ? ((x < nh) ? r_in / RG_h : 0) : ((x < nq) ? 3 * per : 0);
    const int kvh = x * nkv / nq;
#pragma unroll
    for (int r = 0; r < NRG_IN; ++r) {
      const int u = wx + r * XW;
      const int t = dn ? 0 : min(u / per, 2), rg = dn ? u : u - t * per;
      const uint16_t *tile = dn ? ly.dn_in + (size_t)x * r_in * H
                           : (t == 0) ? ly.at_q + (size_t)x * hd * H
                           : (t == 1) ? ly.at_k + (size_t)kvh * hd * H
                                      : ly.at_v + (size_t)kvh * hd * H;
      const __amdgpu_buffer_rsrc_t rs = tile_rsrc(tile, (u < nrg) ? (uint32_t)((rg + 1) * L_h * 1024) : 0u);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const bool ok = u < nrg && i < L_h;
        const uint32_t off = ok ? (uint32_t)(((rg * L_h + i) * 64 + lane) * 16) : OOB_OFF;
        wr[r * 2 + i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, AUX_NT);
      }
    }
    // out-projection (DeltaNet) or o-projection (attention) columns of head x: one load per row group
    const bool has = live && (dn ? x < nh : x < nq);
    const int K = dn ? dv : hd, ngo = H / (dn ? RG_o : RG_a);
    const __amdgpu_buffer_rsrc_t ro =
        tile_rsrc(dn ? ly.dn_out + (size_t)x * H * dv : ly.at_o + (size_t)x * H * hd, has ? (uint32_t)(H * K * 2) : 0u);
#pragma unroll
    for (int r = 0; r < NRG_O; ++r) {
      const int rg = wx + r * XW;
      wr[2 * NRG_IN + r] = __builtin_amdgcn_raw_buffer_load_b128(ro, rg < ngo ? (uint32_t)((rg * 64 + lane) * 16) : OOB_OFF, 0, AUX_NT);
    }
    // attention: this lane's cached K and V rows of the first NKV_PRE key steps (keys lg + 16 ks,
    // slot ks = step * MK_WAVES * kpw + w8 * kpw + lane / lpk; 16 bytes of one row per lane).
    // DeltaNet: the same registers take the pending updates left by a verify forward, update j in
    // slots 2 j (v, alpha, beta of this wave's row) and 2 j + 1 (this lane's key quad), so that
    // D2 replays them without a memory round trip per update.
    if constexpr (!BAT) {
      const bool at = live && !dn && x < nq;
      const bool pdn = live && dn && x < nh && pend_n > 0;
      const int lpk = hd / DPL, kpw = 64 / lpk, pks = mk_pend_stride(dv);
      const __amdgpu_buffer_rsrc_t krs = tile_rsrc(ly.kc, at ? 0x7fffffffu : 0u);
      const __amdgpu_buffer_rsrc_t vrs = tile_rsrc(ly.vc, at ? 0x7fffffffu : 0u);
      const __amdgpu_buffer_rsrc_t prs =
          tile_rsrc(ly.pend + ((size_t)par * nh + (pdn ? x : 0)) * MK_MAXCOL * pks, pdn ? (uint32_t)(MK_MAXCOL * pks * 4) : 0u);
      const int prow = (w8 < RW) ? r0 + w8 : -1;
#pragma unroll
      for (int st = 0; st < NKV_PRE; ++st) {
        const int ks = st * MK_WAVES * kpw + w8 * kpw + lane / lpk, k = lg + MK_NG * ks;
        const uint32_t off = (k >= pos0 || st >= NPRE) ? OOB_OFF
                             : KVQ ? kv8_off(ptl, k, kvh, nkv, hd, (lane % lpk) * DPL) : kv_off(ptl, k, kvh, nkv, hd, (lane % lpk) * 8);
        const bool pj = st < pend_n;
        const uint32_t pv = (pj && prow >= 0) ? (uint32_t)((st * pks + MK_PEND_K + 4 * prow) * 4) : OOB_OFF;
        const uint32_t pk = pj ? (uint32_t)((st * pks + 4 * lane) * 4) : OOB_OFF;
        wr[2 * NRG_IN + NRG_O + 2 * st] = __builtin_amdgcn_raw_buffer_load_b128(dn ? prs : krs, dn ? pv : off, 0, 0);
        wr[2 * NRG_IN + NRG_O + 2 * st + 1] = __builtin_amdgcn_raw_buffer_load_b128(dn ? prs : vrs, dn ? pk : off, 0, 0);
      }
    }
    if constexpr (BAT) {
      // batch: per column c, in slots 2c and 2c + 1 of the prefetch registers, that column's own
      // sequence's DeltaNet state (S row of this wave: x, y; conv history of this lane's channel:
      // z, w and the second slot's x) or its cached K and V rows of the first key step
      const bool sdn = live && dn && x < nh, at = live && !dn && x < nq;
      const bool chl = lane < CPW || (lane == 63 && w8 < RW);
      const int conv_ch = conv_channel(lane);
      const int lpk = hd / DPL, kpw = 64 / lpk, k = lg + MK_NG * (w8 * kpw + lane / lpk);
#pragma unroll
      for (int j = 0; j < NCOL; ++j) {
        const bool lj = j < ncol;
        ConstLayer &lyj = ((ConstLayer *)(uintptr_t)a.seq_layers[lj ? j : 0])[__builtin_amdgcn_readfirstlane(live ? l : 0)];
        u32x4 &s0 = wr[2 * NRG_IN + NRG_O + 2 * j];
        u32x4 &s1 = wr[2 * NRG_IN + NRG_O + 2 * j + 1];
        if (dn) {
          const bool ow = sdn && lj && w8 < RW;
          const __amdgpu_buffer_rsrc_t rs = tile_rsrc(lyj.S + ((size_t)x * dv + r0 + (ow ? w8 : 0)) * dk, ow ? (uint32_t)(dk * 4) : 0u);
          const __amdgpu_buffer_rsrc_t rr = tile_rsrc(lyj.ring, (sdn && lj) ? (uint32_t)(MK_RING * nconv * 4) : 0u);
          uint32_t h[3];
#pragma unroll
          for (int i = 0; i < 3; ++i) {
            const int pp = bpos[j] - 3 + i;
            h[i] = __builtin_amdgcn_raw_buffer_load_b32(
                rr, (chl && pp >= 0) ? (uint32_t)(((pp & (MK_RING - 1)) * nconv + conv_ch) * 4) : OOB_OFF, 0, AUX_DEV);
          }
          s0 = u32x4{__builtin_amdgcn_raw_buffer_load_b32(rs, lane * 4, 0, AUX_DEV),
                     __builtin_amdgcn_raw_buffer_load_b32(rs, (64 + lane) * 4, 0, AUX_DEV), h[0], h[1]};
          s1 = u32x4{h[2], 0u, 0u, 0u};
        } else {
          const __amdgpu_buffer_rsrc_t krs = tile_rsrc(lyj.kc, (at && lj) ? 0x7fffffffu : 0u);
          const __amdgpu_buffer_rsrc_t vrs = tile_rsrc(lyj.vc, (at && lj) ? 0x7fffffffu : 0u);
          const uint32_t off = (k < bpos[j]) ? kv_off(ptl, k, kvh, nkv, hd, (lane % lpk) * 8) : OOB_OFF;
          s0 = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0);
          s1 = __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0);
        }
      }
    }
    // this wave's DeltaNet state: its row of S, the conv taps and history of its lane's channel,
    // the gated-norm gain of its row (batch: the conv taps and the gain; each column's S row and
    // history are its own sequence's, loaded in D2)
    const bool sdn = live && dn && x < nh;
    const bool own = sdn && w8 < RW && !BAT;
    const __amdgpu_buffer_rsrc_t rsS = tile_rsrc(ly.S + ((size_t)x * dv + r0 + (own ? w8 : 0)) * dk, own ? (uint32_t)(dk * 4) : 0u);
    srow[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsS, lane * 4, 0, AUX_DEV));
    srow[1] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsS, (64 + lane) * 4, 0, AUX_DEV));
    // (the descriptors are wave-uniform; a lane without a channel reads zeros through an
    // out-of-range offset)
    const bool chl = lane < CPW || (lane == 63 && w8 < RW);
    const int conv_ch = conv_channel(lane);
    const __amdgpu_buffer_rsrc_t rc = tile_rsrc(ly.dn_conv, sdn ? (uint32_t)(nconv * 16) : 0u);
    const u32x4 wt = __builtin_amdgcn_raw_buffer_load_b128(rc, chl ? (uint32_t)(conv_ch * 16) : OOB_OFF, 0, 0);
    cwt = make_float4(__uint_as_float(wt.x), __uint_as_float(wt.y), __uint_as_float(wt.z), __uint_as_float(wt.w));
    const __amdgpu_buffer_rsrc_t rr = tile_rsrc(ly.ring, (sdn && !BAT) ? (uint32_t)(MK_RING * nconv * 4) : 0u);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int pp = pos0 - 3 + i;
      hist[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          rr, (chl && pp >= 0) ? (uint32_t)(((pp & (MK_RING - 1)) * nconv + conv_ch) * 4) : OOB_OFF, 0, AUX_DEV));
    }
    grow = ld_gain(ly.dn_gnorm, (sdn && w8 < RW) ? dv : 0, r0 + w8);
    ld_gain16(ly.ln1, H, G_h, live, gv);
    keep_issued();
  };
  auto issue_ffn = [&](int l) {
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const bool live = l < m.n_layers;
    // (read through readfirstlane: the layer index stays in a scalar register, so the table is
    // read with scalar loads and every tile descriptor is wave-uniform)
    ConstLayer &ly = layers[__builtin_amdgcn_readfirstlane(live ? l : 0)];
    // gate/up pairs j = wx + pr XW of FFN slice x: rows 2j, 2j + 1 of the slice's tile, contiguous
    // (two row groups when a row group is one row, one when it is two): nl loads per lane
    const int nl = 2 * L_h / RG_h;
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(ly.ffn_gu + (size_t)x * 2 * J * H, live ? (uint32_t)(2 * J * H * 2) : 0u);
#pragma unroll
    for (int pr = 0; pr < NPAIR; ++pr) {
      const int j = wx + pr * XW;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = j < J && i < nl;
        wr[pr * 4 + i] = __builtin_amdgcn_raw_buffer_load_b128(rs, ok ? (uint32_t)(((j * nl + i) * 64 + lane) * 16) : OOB_OFF, 0, AUX_NT);
      }
    }
    // down-projection row group wx of slice x
    const int nrg = H / RG_d;
    const __amdgpu_buffer_rsrc_t rd = tile_rsrc(ly.ffn_dn + (size_t)x * H * J, live ? (uint32_t)(H * J * 2) : 0u);
#pragma unroll
    for (int i = 0; i < LMAX_D; ++i) {
      const bool ok = wx < nrg && i < L_d;
      wr[4 * NPAIR + i] = __builtin_amdgcn_raw_buffer_load_b128(rd, ok ? (uint32_t)(((wx * L_d + i) * 64 + lane) * 16) : OOB_OFF, 0, AUX_NT);
    }
    ld_gain16(ly.ln2, H, G_h, live, gv);
    keep_issued();
  };

  // Reduce-scatter of one sublayer's split-K partials part[col][XCD][H] over the XCDs: this
  // workgroup sums slice lg (SL elements) of every column in a fixed order, adds the residual
  // and publishes the new residual slice to the XCD's slots xr[col][H].  Ends after its gather's
  // barrier; returns false on a watchdog expiry.
  auto reduce_slices = [&](const uint2 *part, uint2 *xr, int site, int tid) {
    float *tmp = work + 4352;   // [NCOL * 8][SL], apart from every buffer a phase may still be reading
    if (!gather2d<MCS, MK_WAVES>(part + lg * SL, ncol * MK_NX, SL, H, tg, tmp, flag, m.ctl, site, tid)) return false;
    for (int i = tid; i < ncol * SL; i += MK_THREADS) {
      const int c = i / SL, k = i - c * SL;
      float sm = tmp[(c * MK_NX) * SL + k];
#pragma unroll
      for (int g = 1; g < MK_NX; ++g) sm += tmp[(c * MK_NX + g) * SL + k];
      pub_xcd(xr + c * H + lg * SL + k, xres[c * H + lg * SL + k] + sm, tg);
    }
    return true;
  };

  // ---- embedding rows (every workgroup) and this launch's RoPE rows
  for (int c = 0; c < ncol; ++c) {
    int t = a.tokens[c];
    if (t < 0 || t >= m.V) {
      if (tid0 == 0) __hip_atomic_fetch_or(m.ctl + MK_CTL_ERR, MK_DERR_TOKEN, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      t = 0;
    }
    const uint16_t *row = m.embed + (size_t)t * H;
    for (int k = tid0; k < H; k += MK_THREADS) xres[c * H + k] = bfv(row[k]);
  }
  if (m.nq > 0) {
    const int half = hd / 2;
    for (int i = tid0; i < ncol * half; i += MK_THREADS) {
      const int c = i / half, d = i - c * half;
      const int pc = BAT ? __hip_atomic_load(a.seq_ctl[c] + MK_CTL_POS, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : pos0 + c;
      const float2 r = *reinterpret_cast<const float2 *>(m.rope + ((size_t)pc * half + d) * 2);
      rl[i * 2 + 0] = r.x;
      rl[i * 2 + 1] = r.y;
    }
  }
  lbar();   // (the first mixer issue reads the page table from LDS)
  if (mixer) issue_mixer(0);
  else issue_ffn(0);

  for (li = 0; li < m.n_layers; ++li) {
    li = __builtin_amdgcn_readfirstlane(li);   // keep the layer index (and all derived from it) scalar
    ConstLayer &ly = layers[li];
    // A per-layer copy of the thread index the compiler cannot see through: address
    // arithmetic derived from it stays inside the layer loop instead of being hoisted out
    // (and spilled) for the whole loop.
    int tid = tid0;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    // this layer's exchange slots (layout in mk_layout.h)
    uint2 *const x_in_l = a.xch + (size_t)li * mk_xch_layer_slots(NCOL, H, r_in_max, x_o_len, xm_len);
    uint2 *const x_o_l = x_in_l + NCOL * MK_NX * r_in_max;
    uint2 *const x_mix_l = x_o_l + NCOL * MK_NX * x_o_len;
    uint2 *const x_r1_l = x_mix_l + NCOL * MK_NX * H;
    uint2 *const x_m_l = x_r1_l + NCOL * MK_NX * H;
    uint2 *const x_ffn_l = x_m_l + NCOL * MK_NX * xm_len;
    if (mixer) {
      // ============================================================ token mixer of layer li
      MK_TRACE_POINT(li, 0);
      if (li > 0) {   // residual after the previous layer's FFN, published slice by slice by the FFN role
        uint2 *const x_r2_p = x_in_l - mk_xch_layer_slots(NCOL, H, r_in_max, x_o_len, xm_len) +
                              (size_t)NCOL * MK_NX * (r_in_max + x_o_len + xm_len + 3 * H);
        if (!gather2d<MCS, MK_WAVES>(x_r2_p + (size_t)x * NCOL * H, ncol, H, H, tg, xres, flag, m.ctl, SITE(13), tid)) MK_BAIL();
      }
      MK_TRACE_POINT(li, 1);
      uint2 *xin = x_in_l + (size_t)x * NCOL * r_in_max;
      uint2 *xo = x_o_l + (size_t)x * NCOL * x_o_len;
      if (ly.kind == 0) {
        // ------------------------------------------------ DeltaNet
        // ---- D1: in-projection rows u = wx + r XW of head x (weights already in registers)
        if (x < nh) {
          const int nrg = r_in / RG_h;
          FOR_COL_R(c) {
            float av[16];
            rmsnorm_regs(xres + c * H, gv, H, G_h, L_h, m.rms_eps, av);
            if (G_h == 64) {  // one row per row group: rows 0-3 of this wave reduced together, then row 4
              const float t = wave_sum4(dot16(wr[0], wr[1], av), dot16(wr[2], wr[3], av), dot16(wr[4], wr[5], av),
                                        dot16(wr[6], wr[7], av));
              const int r = (lane == 0) ? 0 : (lane == 32) ? 1 : (lane == 16) ? 2 : (lane == 48) ? 3 : NRG_IN;
              if (r < NRG_IN && wx + r * XW < nrg) pub_xcd(xin + c * r_in_max + wx + r * XW, t, tg);
              if (wx + 4 * XW < nrg) {
                const float t4 = wave_sum(dot16(wr[8], wr[9], av));
                if (lane == 0) pub_xcd(xin + c * r_in_max + wx + 4 * XW, t4, tg);
              }
            } else {
#pragma unroll
              for (int r = 0; r < NRG_IN; ++r) {
                const int rg = wx + r * XW;
                const float o = rg_dot_regs(wr[2 * r], wr[2 * r + 1], G_h, av);
                if (rg < nrg && (lane & (G_h - 1)) == 0) pub_xcd(xin + c * r_in_max + rg * RG_h + lane / G_h, o, tg);
              }
            }
          }
        }
        MK_TRACE_POINT(li, 2);
        // ---- D2: conv, norms, gates, delta rule; wave w8 < RW owns row r0 + w8 of S
        if (x < nh) {
          float *gqk = work;                      // [NCOL][2dk]  q, k before the conv
          float *gvv = gqk + NCOL * 2 * dk;       // [NCOL][RW]   my v rows before the conv
          float *gz = gvv + NCOL * RW;            // [NCOL][RW]   my z rows
          float *gab = gz + NCOL * RW;            // [NCOL][2]    a, b
          float *qkc = gab + NCOL * 2;            // [NCOL][2dk]  q, k after conv + SiLU
          float *rsq = qkc + NCOL * 2 * dk;       // [NCOL][8]    per-wave sums of squares
          // batch: each column's conv history (this lane's channel) and S row (this wave's row)
          // come from its own sequence's state; loaded here, in flight during the gather
          // (prefetched with the layer's weights, slots 2c and 2c + 1)
          float hb[NCOL][3], sb[NCOL][2];
          if constexpr (BAT) {
#pragma unroll
            for (int c = 0; c < NCOL; ++c) {
              const u32x4 s0 = wr[2 * NRG_IN + NRG_O + 2 * c], s1 = wr[2 * NRG_IN + NRG_O + 2 * c + 1];
              sb[c][0] = __uint_as_float(s0.x);
              sb[c][1] = __uint_as_float(s0.y);
              hb[c][0] = __uint_as_float(s0.z);
              hb[c][1] = __uint_as_float(s0.w);
              hb[c][2] = __uint_as_float(s1.x);
            }
          }
          {
            const GSeg sg[4] = {{0, ncol, 2 * dk, r_in_max, gqk},
                                {2 * dk + r0, ncol, RW, r_in_max, gvv},
                                {2 * dk + dv + r0, ncol, RW, r_in_max, gz},
                                {2 * dk + 2 * dv, ncol, 2, r_in_max, gab}};
            if (!gather_segs<MCS, MK_WAVES, 4>(xin, sg, tg, flag, m.ctl, SITE(1), tid)) MK_BAIL();
          }
          MK_TRACE_POINT(li, 3);
          // conv + SiLU of this lane's channel for every column: tap i meets the token 3 - i steps
          // before the column (earlier columns of this forward, else the history)
          const bool qkl = lane < CPW, vl = lane == 63 && w8 < RW;
          const int chq = w8 * CPW + lane, conv_ch = conv_channel(lane);
          float raw[NCOL], cv[NCOL];
#pragma unroll
          for (int c = 0; c < NCOL; ++c) raw[c] = (c < ncol) ? (qkl ? gqk[c * 2 * dk + chq] : vl ? gvv[c * RW + w8] : 0.f) : 0.f;
          {
            const float wv[4] = {cwt.x, cwt.y, cwt.z, cwt.w};
#pragma unroll
            for (int c = 0; c < NCOL; ++c) {
              float sacc = 0.f;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int cc = c - (3 - i);
                // (batch: every column is the newest token of its own sequence, as in decode)
                const float v = BAT ? (i < 3 ? hb[c][i < 3 ? i : 0] : raw[c])
                                    : (cc >= 0) ? raw[cc < 0 ? 0 : cc] : hist[cc + 3 < 0 ? 0 : cc + 3];
                sacc = fmaf(wv[i], v, sacc);
              }
              cv[c] = silu_f(sacc);
            }
          }
          // q/k channels to LDS with each wave's sum of squares (waves [0, 4) hold q, [4, 8) k)
          FOR_COL(c) {
            if (qkl) qkc[c * 2 * dk + chq] = cv[c];
            const float sq = wave_sum(qkl ? fmaf(cv[c], cv[c], 0.f) : 0.f);
            if (lane == 0) rsq[c * MK_WAVES + w8] = sq;
          }
          // this forward's pre-conv inputs into the ring (q/k by workgroup 0 of the role, v by the owner)
          if ((qkl && lg == 0) || vl) {
            if constexpr (BAT) {
              FOR_COL(c) ((ConstLayer *)(uintptr_t)a.seq_layers[c])[li].ring[(bpos[c] & (MK_RING - 1)) * nconv + conv_ch] = raw[c];
            } else {
              FOR_COL(c) ly.ring[((pos0 + c) & (MK_RING - 1)) * nconv + conv_ch] = raw[c];
            }
          }
          lbar();
          if (w8 < RW) {
            // delta rule on row r0 + w8: S_r <- alpha S_r + beta (v_r - alpha S_r.k) k ; o_r = S_r.q
            const int J2 = dk / 64;
            auto rowdot = [&](float e0, float e1) {  // S_r . vec, lane holds vec[lane], vec[64 + lane]
              float p = fmaf(srow[0], e0, 0.f);
              if (J2 > 1) p = fmaf(srow[1], e1, p);
              return wave_sum(p);
            };
#pragma unroll
            for (int j = 0; j < MK_MAXCOL; ++j) {  // pending updates left by a verify forward (in registers)
              if (j >= pend_n) break;
              const u32x4 pvj = wr[2 * NRG_IN + NRG_O + 2 * j], pkj = wr[2 * NRG_IN + NRG_O + 2 * j + 1];
              const float vj = __uint_as_float(pvj.x), aj = __uint_as_float(pvj.y), bj = __uint_as_float(pvj.z);
              const float k0 = __uint_as_float(pkj.x), k1 = (J2 > 1) ? __uint_as_float(pkj.y) : 0.f;
              const float u = bj * (vj - aj * rowdot(k0, k1));
              srow[0] = fmaf(u, k0, aj * srow[0]);
              if (J2 > 1) srow[1] = fmaf(u, k1, aj * srow[1]);
            }
            float *Srow = ly.S + ((size_t)x * dv + r0 + w8) * dk;
            if (verify) {  // S after the accepted tokens; this forward's tokens become pending
              Srow[lane] = srow[0];
              if (J2 > 1) Srow[64 + lane] = srow[1];
            }
            float *pw = ly.pend + ((size_t)(par ^ 1) * nh + x) * MK_MAXCOL * mk_pend_stride(dv);
            // several columns: lane c computes column c's norm scales of k and q, its gates and its
            // SiLU(z) (the same operations on the same values as the column's own lanes would) into
            // this wave's LDS table, so each column's chain below reads them in one LDS round trip
            // (written and read by this wave only: no barrier; apart from D3's gather buffer)
            float *csc = work + 4096 + w8 * (MK_MAXCOL * 8);   // [NCOL][8]: k scale, q scale, alpha, beta, SiLU(z)
            if constexpr (NCOL > 1) {
              if (lane < NCOL) {
                const float *rc = rsq + lane * 8;
                const float ka = rc[4], kb = rc[5], kc = rc[6], kd = rc[7], qa = rc[0], qb = rc[1], qc = rc[2], qd = rc[3];
                const float ga = gab[lane * 2 + 0], gb = gab[lane * 2 + 1], zz = gz[lane * RW + w8];
                *reinterpret_cast<float4 *>(csc + lane * 8) =
                    make_float4(rsqrtf(((ka + kb) + kc) + kd + m.l2_eps), rsqrtf(((qa + qb) + qc) + qd + m.l2_eps), decay_f(ga),
                                sigmoid_f(gb));
                csc[lane * 8 + 4] = silu_f(zz);
              }
            }
            // the readout o = S q of column c from its updated state row, and o's gated numerator
            auto readout = [&](int c, float s0, float s1) {
              const float qr = NCOL > 1 ? csc[c * 8 + 1]
                                        : rsqrtf(((rsq[c * 8 + 0] + rsq[c * 8 + 1]) + rsq[c * 8 + 2]) + rsq[c * 8 + 3] + m.l2_eps);
              const float *qc = qkc + c * 2 * dk;
              const float q0 = qc[lane] * qr, q1 = (J2 > 1) ? qc[64 + lane] * qr : 0.f;
              float p = fmaf(s0, q0, 0.f);   // o = S_c . q (rowdot on the column's state row)
              if (J2 > 1) p = fmaf(s1, q1, p);
              const float o = wave_sum(p);
              // the gated norm's numerator o g silu(z); D3 divides by the RMS of the head's o
              const float uo = o * grow * (NCOL > 1 ? csc[c * 8 + 4] : silu_f(gz[c * RW + w8]));
              if (lane == 0) {
                pub_xcd(xo + c * x_o_len + r0 + w8, o, tg);
                pub_xcd(xo + c * x_o_len + dv + r0 + w8, uo, tg);
              }
            };
            FOR_COL(c) {
              if constexpr (BAT) {   // this column's sequence's row of S
                srow[0] = sb[c][0];
                srow[1] = sb[c][1];
              }
              const float kr = NCOL > 1 ? csc[c * 8 + 0]
                                        : rsqrtf(((rsq[c * 8 + 4] + rsq[c * 8 + 5]) + rsq[c * 8 + 6]) + rsq[c * 8 + 7] + m.l2_eps);
              const float *qc = qkc + c * 2 * dk;
              const float k0 = qc[dk + lane] * kr, k1 = (J2 > 1) ? qc[dk + 64 + lane] * kr : 0.f;
              const float vr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cv[c]), 63));
              const float al = NCOL > 1 ? csc[c * 8 + 2] : decay_f(gab[c * 2 + 0]);
              const float be = NCOL > 1 ? csc[c * 8 + 3] : sigmoid_f(gab[c * 2 + 1]);
              const float u = be * (vr - al * rowdot(k0, k1));
              srow[0] = fmaf(u, k0, al * srow[0]);
              if (J2 > 1) srow[1] = fmaf(u, k1, al * srow[1]);
              readout(c, srow[0], srow[1]);
              if (verify) {  // (k, v, alpha, beta) of this column become a pending update
                float *pc = pw + c * mk_pend_stride(dv);
                if (lg == 0 && w8 == 0) *reinterpret_cast<float4 *>(pc + 4 * lane) = make_float4(k0, k1, 0.f, 0.f);
                if (lane == 0) *reinterpret_cast<float4 *>(pc + MK_PEND_K + 4 * (r0 + w8)) = make_float4(vr, al, be, 0.f);
              }
              if constexpr (BAT) {
                float *Sc = ((ConstLayer *)(uintptr_t)a.seq_layers[c])[li].S + ((size_t)x * dv + r0 + w8) * dk;
                Sc[lane] = srow[0];
                if (J2 > 1) Sc[64 + lane] = srow[1];
              }
            }
            if (!verify && !BAT) {
              Srow[lane] = srow[0];
              if (J2 > 1) Srow[64 + lane] = srow[1];
            }
          }
        }
        MK_TRACE_POINT(li, 4);
        // ---- D3: out-projection columns of head x: (W u) / RMS(o)
        if (x < nh) {
          float *d3 = work + 2816;           // [NCOL][2dv]: o | o g silu(z)  (apart from D2's buffers)
          if (!gather2d<MCS, MK_WAVES>(xo, ncol, 2 * dv, x_o_len, tg, d3, flag, m.ctl, SITE(4), tid)) MK_BAIL();
          MK_TRACE_POINT(li, 5);
          const int kl = (lane & (G_o - 1)) * 8;
          FOR_COL_R(c) {
            float ss = 0.f, uu[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float ov = d3[c * 2 * dv + kl + e];
              ss = fmaf(ov, ov, ss);
              uu[e] = d3[c * 2 * dv + dv + kl + e];
            }
            const float rinv = rsqrtf(group_sum(ss, G_o) / (float)dv + m.rms_eps);
#pragma unroll
            for (int r = 0; r < NRG_O; ++r) {
              const int rg = wx + r * XW;
              float f[8], s = 0.f;
              unpack8(wr[2 * NRG_IN + r], f);
#pragma unroll
              for (int e = 0; e < 8; ++e) s = fmaf(f[e], uu[e], s);
              s = group_sum(s, G_o);
              if (rg < H / RG_o && (lane & (G_o - 1)) == 0)
                pub(x_mix_l + ((size_t)c * MK_NX + x) * H + rg * RG_o + lane / G_o, s * rinv, tg);
            }
          }
        } else {
          for (int i = tid + lg * MK_THREADS; i < H; i += MK_NG * MK_THREADS)
            for (int c = 0; c < ncol; ++c) pub(x_mix_l + ((size_t)c * MK_NX + x) * H + i, 0.f, tg);
        }
      } else {
        // ------------------------------------------------ attention
        const int kvh = x * nkv / nq;
        if (x < nq) {
          // ---- A1: q rows of head x, k / v rows of its kv head (weights already in registers)
          const int per = hd / RG_h;
          FOR_COL_R(c) {
            float av[16];
            rmsnorm_regs(xres + c * H, gv, H, G_h, L_h, m.rms_eps, av);
            if (G_h == 64) {  // row group u is row u (t hd + rg == u)
              const float t = wave_sum4(dot16(wr[0], wr[1], av), dot16(wr[2], wr[3], av), dot16(wr[4], wr[5], av),
                                        dot16(wr[6], wr[7], av));
              const int r = (lane == 0) ? 0 : (lane == 32) ? 1 : (lane == 16) ? 2 : (lane == 48) ? 3 : NRG_IN;
              if (r < NRG_IN && wx + r * XW < 3 * per) pub_xcd(xin + c * r_in_max + wx + r * XW, t, tg);
              if (wx + 4 * XW < 3 * per) {
                const float t4 = wave_sum(dot16(wr[8], wr[9], av));
                if (lane == 0) pub_xcd(xin + c * r_in_max + wx + 4 * XW, t4, tg);
              }
            } else {
#pragma unroll
              for (int r = 0; r < NRG_IN; ++r) {
                const int u = wx + r * XW;
                const float o = rg_dot_regs(wr[2 * r], wr[2 * r + 1], G_h, av);
                if (u < 3 * per && (lane & (G_h - 1)) == 0) {
                  const int t = u / per, rg = u - t * per;
                  pub_xcd(xin + c * r_in_max + t * hd + rg * RG_h + lane / G_h, o, tg);
                }
              }
            }
          }
          MK_TRACE_POINT(li, 2);
          // ---- A2: RoPE, KV append, split-KV partials
          // 8-bit cache: the exponent pairs of the prefetched rows, loaded here (not with the rows:
          // held across the layer they would not fit in registers) and in flight during the gather
          uint32_t kvx[NPRE > 0 ? NPRE : 1];
          if constexpr (KVQ) {
            const int lpk = hd / DPL, kpw = 64 / lpk;
            const __amdgpu_buffer_rsrc_t ers = __builtin_amdgcn_make_buffer_rsrc(ly.kve, 0, 0x7fffffff, RSRC_W3);
#pragma unroll
            for (int st = 0; st < NPRE; ++st) {
              const int k = lg + MK_NG * (st * MK_WAVES * kpw + w8 * kpw + lane / lpk);
              kvx[st] = __builtin_amdgcn_raw_buffer_load_b16(ers, (k < pos0) ? kve_off(ptl, k, kvh, nkv) : OOB_OFF, 0, 0);
            }
          }
          float *qkv = work;                    // [NCOL][3hd]
          // 8-bit cache: scales 2^e of this forward's K, V rows [NCOL][2] (past the split-KV buffers below)
          float *kvs = work + NCOL * 3 * hd + 640 + MK_WAVES * hd + 2;
          if (!gather2d<MCS, MK_WAVES>(xin, ncol, 3 * hd, r_in_max, tg, qkv, flag, m.ctl, SITE(6), tid)) MK_BAIL();
          if constexpr (BAT) {
            // every column's cached K and V rows of key step 1 (see NPRE), issued after the gather (a
            // wave's loads complete in order: issued before it, they would delay its polls)
            const int lpk = hd / DPL, kpw = 64 / lpk;
            const int k = lg + MK_NG * (MK_WAVES * kpw + w8 * kpw + lane / lpk);
#pragma unroll
            for (int j = 0; j < NCOL; ++j) {
              const bool lj = j < ncol;
              ConstLayer &lyj = ((ConstLayer *)(uintptr_t)a.seq_layers[lj ? j : 0])[li];
              const __amdgpu_buffer_rsrc_t krs = tile_rsrc(lyj.kc, lj ? 0x7fffffffu : 0u);
              const __amdgpu_buffer_rsrc_t vrs = tile_rsrc(lyj.vc, lj ? 0x7fffffffu : 0u);
              const uint32_t off = (k < bpos[j]) ? kv_off(ptl, k, kvh, nkv, hd, (lane % lpk) * 8) : OOB_OFF;
              wr[2 * j] = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0);
              wr[2 * j + 1] = __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0);
            }
          }
          MK_TRACE_POINT(li, 3);
          {
            const int half = hd / 2;
            for (int i = tid; i < ncol * half; i += MK_THREADS) {
              const int c = i / half, d = i - c * half;
              const float cs = rl[i * 2 + 0], sn = rl[i * 2 + 1];
              float *q = qkv + c * 3 * hd, *k = q + hd, *v = k + hd;
              const float q1 = q[d], q2 = q[d + half], k1 = k[d], k2 = k[d + half];
              q[d] = q1 * cs - q2 * sn;
              q[d + half] = q2 * cs + q1 * sn;
              if constexpr (KVQ) {
                k[d] = k1 * cs - k2 * sn; k[d + half] = k2 * cs + k1 * sn;
              } else {
                k[d] = rbf(k1 * cs - k2 * sn); k[d + half] = rbf(k2 * cs + k1 * sn);
                v[d] = rbf(v[d]); v[d + half] = rbf(v[d + half]);
              }
            }
          }
          lbar();
          if constexpr (KVQ) {
            // 8-bit cache: each K and V row of this forward (one wave per row) becomes codes and an
            // exponent; LDS keeps the codes (as FP32) and the row scales 2^e, in the form later
            // forwards read them from the cache.  The first query head of the kv group appends the rows.
            const bool app = lg == 0 && (x * nkv) % nq == 0;
            const __amdgpu_buffer_rsrc_t cst = __builtin_amdgcn_make_buffer_rsrc(ly.kc, 0, 0x7fffffff, RSRC_W3);
            const __amdgpu_buffer_rsrc_t vst = __builtin_amdgcn_make_buffer_rsrc(ly.vc, 0, 0x7fffffff, RSRC_W3);
            const __amdgpu_buffer_rsrc_t est = __builtin_amdgcn_make_buffer_rsrc(ly.kve, 0, 0x7fffffff, RSRC_W3);
            for (int r = w8; r < 2 * ncol; r += MK_WAVES) {
              const int c = r >> 1, isv = r & 1;
              float *row = qkv + c * 3 * hd + (1 + isv) * hd;
              const float x0 = lane < hd ? row[lane] : 0.f, x1 = lane + 64 < hd ? row[lane + 64] : 0.f;
              float am = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
              for (int o = 32; o > 0; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
              const int e = mk_q8_exp(am);
              // (through int: a code of zero is +0, as the cache's byte converts)
              const float q0 = (float)(int)rintf(ldexpf(x0, -e)), q1 = (float)(int)rintf(ldexpf(x1, -e));
              const int p = pos0 + c;
              const uint32_t rix = ((uint32_t)ptl[p / MK_PAGE] * nkv + kvh) * MK_PAGE + (p % MK_PAGE);
              if (lane == 0) kvs[r] = q8_scale((uint32_t)e);
              if (lane < hd) {
                row[lane] = q0;
                if (app) __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(int)q0, isv ? vst : cst, rix * hd + lane, 0, AUX_DEV);
              }
              if (lane + 64 < hd) {
                row[lane + 64] = q1;
                if (app) __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(int)q1, isv ? vst : cst, rix * hd + lane + 64, 0, AUX_DEV);
              }
              if (app && lane == 0) __builtin_amdgcn_raw_buffer_store_b8((uint8_t)e, est, rix * 2 + isv, 0, AUX_DEV);
            }
            lbar();
          } else if (lg == 0 && (x * nkv) % nq == 0) {
            // the first query head of the kv group appends K, V (read by later launches only: this
            // launch takes its own positions' keys and values from LDS)
            if constexpr (BAT) {   // column c into its own sequence's cache, at its position
              FOR_COL(c) {
                ConstLayer &cl = ((ConstLayer *)(uintptr_t)a.seq_layers[c])[li];
                const __amdgpu_buffer_rsrc_t kst = __builtin_amdgcn_make_buffer_rsrc(cl.kc, 0, 0x7fffffff, RSRC_W3);
                const __amdgpu_buffer_rsrc_t vst = __builtin_amdgcn_make_buffer_rsrc(cl.vc, 0, 0x7fffffff, RSRC_W3);
                const int p = bpos[c];
                for (int d = tid; d < hd; d += MK_THREADS) {
                  const size_t off = (((size_t)ptl[p / MK_PAGE] * nkv + kvh) * MK_PAGE + (p % MK_PAGE)) * hd + d;
                  const uint16_t kb = (uint16_t)(__float_as_uint(qkv[c * 3 * hd + hd + d]) >> 16);
                  const uint16_t vb = (uint16_t)(__float_as_uint(qkv[c * 3 * hd + 2 * hd + d]) >> 16);
                  __builtin_amdgcn_raw_buffer_store_b16(kb, kst, (uint32_t)(off * 2), 0, AUX_DEV);
                  __builtin_amdgcn_raw_buffer_store_b16(vb, vst, (uint32_t)(off * 2), 0, AUX_DEV);
                }
              }
            } else {
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
            }
          }
          {
            // Split-KV partials: this workgroup takes keys lg, lg + 16, lg + 32, ... of each query
            // position (balanced over the 16 workgroups).  Key slot ks is key lg + 16 ks; a step of
            // the workgroup covers MK_WAVES * kpw slots, kpw per wave, lpk lanes per key with 8
            // dimensions each.  Cached keys and values of the first NKV_PRE steps are in registers
            // (loaded with this layer's weights), later steps load them here.  This forward's own
            // positions (at most one per column in this workgroup, as ncol < 16) come from LDS.
            float *sc = work + NCOL * 3 * hd;      // scores of my keys [<= 640]
            float *pv = sc + 640;                  // [MK_WAVES][hd] partial P.V per wave
            float *mx = pv + MK_WAVES * hd;        // [2]: max, sum
            const float scale = 1.f / sqrtf((float)hd);
            const int lpk = hd / DPL, kpw = 64 / lpk, spw = MK_WAVES * kpw;
            const int d0 = (lane % lpk) * DPL, kslot = w8 * kpw + lane / lpk;
            const __amdgpu_buffer_rsrc_t krs0 = __builtin_amdgcn_make_buffer_rsrc(ly.kc, 0, 0x7fffffff, RSRC_W3);
            const __amdgpu_buffer_rsrc_t vrs0 = __builtin_amdgcn_make_buffer_rsrc(ly.vc, 0, 0x7fffffff, RSRC_W3);
            const __amdgpu_buffer_rsrc_t ers = __builtin_amdgcn_make_buffer_rsrc(KVQ ? (void *)ly.kve : nullptr, 0, KVQ ? 0x7fffffff : 0, RSRC_W3);
            // byte offset of this lane's part of cached row ks (a slot below ncache), and of its exponents
            auto row_off = [&](int ks) {
              return KVQ ? kv8_off(ptl, lg + MK_NG * ks, kvh, nkv, hd, d0) : kv_off(ptl, lg + MK_NG * ks, kvh, nkv, hd, d0);
            };
if constexpr (NCOL > 1 && !BAT && !KVQ) {
              // Verify: every column reads the same cached keys and values (the sequence's, below
              // pos0), so each cached row is converted once and used for all columns, and the phase
              // has four barriers instead of four per column.  Per column the products, sums and their
              // order are those of the one-column loop below, so the results equal decode's bit for
              // bit.  Column c: scores at scv + 640 c, P.V partials at pvv + MK_WAVES hd c, max and sum
              // at mxv[2 c], mxv[2 c + 1].
              float *scv = sc;                                 // [NCOL][640]
              float *pvv = scv + NCOL * 640;                   // [NCOL][MK_WAVES][hd]
              float *mxv = pvv + NCOL * MK_WAVES * hd;         // [NCOL][2]
              const int ncache = (pos0 > lg) ? (pos0 - 1 - lg) / MK_NG + 1 : 0;
              const int nstc = (ncache + spw - 1) / spw;
              // keys of this workgroup up to column c's position, and its own key (at most one)
              auto nkc = [&](int c) { const int P = pos0 + c; return (P >= lg) ? (P - lg) / MK_NG + 1 : 0; };
              float qv[NCOL][DPL];   // (columns past ncol: zeros, computed and never stored)
#pragma unroll
              for (int c = 0; c < NCOL; ++c)
#pragma unroll
                for (int i = 0; i < DPL; ++i) qv[c][i] = (c < ncol) ? qkv[c * 3 * hd + d0 + i] : 0.f;
              auto score_all = [&](int ks, const float (&kf)[DPL]) {
#pragma unroll
                for (int c = 0; c < NCOL; ++c) {
                  float sdot = 0.f;
#pragma unroll
                  for (int i = 0; i < DPL; ++i) sdot = fmaf(qv[c][i], kf[i], sdot);
                  sdot = group_sum(sdot, lpk);
                  if (c < ncol && ks < ncache && (lane % lpk) == 0) scv[c * 640 + ks] = sdot * scale;
                }
              };
#pragma unroll
              for (int st = 0; st < NPRE; ++st) {
                if (st < nstc) {
                  float kf[DPL];
                  kv_unpack<DPL>(wr[2 * NRG_IN + NRG_O + 2 * st], kf);
                  score_all(st * spw + kslot, kf);
                }
              }
#pragma unroll 1
              for (int st = NPRE; st < nstc; st += KV_GRP) {
                u32x4 kr[KV_GRP];
#pragma unroll
                for (int u = 0; u < KV_GRP; ++u) {
                  const int ks = (st + u) * spw + kslot;
                  kr[u] = __builtin_amdgcn_raw_buffer_load_b128(krs0, ks < ncache ? row_off(ks) : OOB_OFF, 0, 0);
                }
#pragma unroll
                for (int u = 0; u < KV_GRP; ++u) {
                  if (st + u < nstc) {
                    float kf[DPL];
                    kv_unpack<DPL>(kr[u], kf);
                    score_all((st + u) * spw + kslot, kf);
                  }
                }
              }
              if (w8 == 0 && lane < lpk) {   // this forward's keys: from LDS
#pragma unroll
                for (int c = 0; c < NCOL; ++c) {
                  const int nk = nkc(c), kc_ = lg + MK_NG * (nk - 1);
                  if (c < ncol && nk > 0 && kc_ >= pos0) {
                    const float *kk = qkv + (kc_ - pos0) * 3 * hd + hd + d0;
                    float sdot = 0.f;
#pragma unroll
                    for (int i = 0; i < DPL; ++i) sdot = fmaf(qv[c][i], kk[i], sdot);
                    sdot = group_sum(sdot, lpk);
                    if (lane == 0) scv[c * 640 + nk - 1] = sdot * scale;
                  }
                }
              }
              lbar();
              if (w8 < ncol) {   // softmax of column w8
                const int c = w8, nk = nkc(c);
                float *scc = scv + c * 640;
                float mv = -INFINITY;
                for (int i = lane; i < nk; i += 64) mv = fmaxf(mv, scc[i]);
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) mv = fmaxf(mv, __shfl_xor(mv, off, 64));
                float ls = 0.f;
                for (int i = lane; i < nk; i += 64) {
                  const float pe = __expf(scc[i] - mv);
                  scc[i] = pe;
                  ls += pe;
                }
                ls = wave_sum(ls);
                if (lane == 0) { mxv[2 * c] = mv; mxv[2 * c + 1] = ls; }
              }
              lbar();
              float acc[NCOL][DPL];
#pragma unroll
              for (int c = 0; c < NCOL; ++c)
#pragma unroll
                for (int i = 0; i < DPL; ++i) acc[c][i] = 0.f;
              auto pvacc_all = [&](int ks, const float (&vf)[DPL]) {
#pragma unroll
                for (int c = 0; c < NCOL; ++c) {
                  const float pe = (ks < ncache) ? scv[c * 640 + (ks < ncache ? ks : 0)] : 0.f;
#pragma unroll
                  for (int i = 0; i < DPL; ++i) acc[c][i] = fmaf(pe, vf[i], acc[c][i]);
                }
              };
#pragma unroll
              for (int st = 0; st < NPRE; ++st) {
                if (st < nstc) {
                  float vf[DPL];
                  kv_unpack<DPL>(wr[2 * NRG_IN + NRG_O + 2 * st + 1], vf);
                  pvacc_all(st * spw + kslot, vf);
                }
              }
#pragma unroll 1
              for (int st = NPRE; st < nstc; st += KV_GRP) {
                u32x4 vr[KV_GRP];
#pragma unroll
                for (int u = 0; u < KV_GRP; ++u) {
                  const int ks = (st + u) * spw + kslot;
                  vr[u] = __builtin_amdgcn_raw_buffer_load_b128(vrs0, ks < ncache ? row_off(ks) : OOB_OFF, 0, 0);
                }
#pragma unroll
                for (int u = 0; u < KV_GRP; ++u) {
                  if (st + u < nstc) {
                    float vf[DPL];
                    kv_unpack<DPL>(vr[u], vf);
                    pvacc_all((st + u) * spw + kslot, vf);
                  }
                }
              }
#pragma unroll
              for (int c = 0; c < NCOL; ++c) {
                // this forward's value, added by the lanes that own its slot in the step order
                const int nk = nkc(c), kc_ = lg + MK_NG * (nk - 1), kcs = (nk - 1) % spw;
                if (c < ncol && nk > 0 && kc_ >= pos0 && w8 == kcs / kpw && lane / lpk == kcs % kpw) {
                  const float pe = scv[c * 640 + nk - 1];
                  const float *vv = qkv + (kc_ - pos0) * 3 * hd + 2 * hd + d0;
#pragma unroll
                  for (int i = 0; i < DPL; ++i) acc[c][i] = fmaf(pe, vv[i], acc[c][i]);
                }
                // sum over the kpw key groups of the wave, as in the one-column loop
#pragma unroll
                for (int i = 0; i < DPL; ++i) {
                  float v = acc[c][i];
                  if (lpk == 16) {
                    v = swap_add32(v, v);
                    v = swap_add16(v, v);
                  } else {
                    for (int o = lpk; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
                  }
                  acc[c][i] = v;
                }
                if (c < ncol && lane < lpk) {
#pragma unroll
                  for (int i = 0; i < DPL; ++i) pvv[(c * MK_WAVES + w8) * hd + d0 + i] = acc[c][i];
                }
              }
              lbar();
              const int plen = hd + 2;
              for (int i = tid; i < ncol * hd; i += MK_THREADS) {
                const int c = i / hd, d = i - c * hd;
                const float *pc = pvv + c * MK_WAVES * hd;
                float a2 = pc[d];
#pragma unroll 1
                for (int ww = 1; ww < MK_WAVES; ++ww) a2 += pc[ww * hd + d];
                pub_xcd(xo + c * x_o_len + lg * plen + 2 + d, a2, tg);
              }
              if (tid < ncol) {
                const int c = tid, nk = nkc(c);
                uint2 *dst = xo + c * x_o_len + lg * plen;
                pub_xcd(dst + 0, nk > 0 ? mxv[2 * c] : -INFINITY, tg);
                pub_xcd(dst + 1, nk > 0 ? mxv[2 * c + 1] : 0.f, tg);
              }
              lbar();
            } else if constexpr (BAT) {
              // Batch: each column reads its own sequence's cache; the columns' scores, softmaxes and
              // P.V partials are each one pass over the columns (four barriers per attention layer
              // instead of four per column), each column with decode's arithmetic and order.
              float *scv = sc;                                 // [NCOL][640]
              float *pvv = scv + NCOL * 640;                   // [NCOL][MK_WAVES][hd]
              float *mxv = pvv + NCOL * MK_WAVES * hd;         // [NCOL][2]
              auto ncache_of = [&](int P) { return (P > lg) ? (P - 1 - lg) / MK_NG + 1 : 0; };
              auto nk_of = [&](int P) { return (P >= lg) ? (P - lg) / MK_NG + 1 : 0; };
#pragma unroll 1
              for (int c = 0; c < ncol; ++c) {   // scores
                const int P = bposl[c], ncache = ncache_of(P), nstc = (ncache + spw - 1) / spw, nk = nk_of(P);
                const int kc_ = lg + MK_NG * (nk - 1);
                ConstLayer &cl = ((ConstLayer *)(uintptr_t)a.seq_layers[c])[li];
                const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(cl.kc, 0, 0x7fffffff, RSRC_W3);
                float *scc = scv + c * 640;
                float qv[DPL];
#pragma unroll
                for (int i = 0; i < DPL; ++i) qv[i] = qkv[c * 3 * hd + d0 + i];
                auto score = [&](int ks, const float (&kf)[DPL]) {
                  float sdot = 0.f;
#pragma unroll
                  for (int i = 0; i < DPL; ++i) sdot = fmaf(qv[i], kf[i], sdot);
                  sdot = group_sum(sdot, lpk);
                  if (ks < ncache && (lane % lpk) == 0) scc[ks] = sdot * scale;
                };
                if (nstc > 0) {
                  float kf[DPL];
                  kv_unpack<DPL>(wsel(c, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}), kf);
                  score(kslot, kf);
                }
                if (nstc > 1) {
                  float kf[DPL];
                  kv_unpack<DPL>(wsel(c, std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{}), kf);
                  score(spw + kslot, kf);
                }
#pragma unroll 1
                for (int st = NPRE; st < nstc; st += KV_GRP) {
                  u32x4 kr[KV_GRP];
#pragma unroll
                  for (int u = 0; u < KV_GRP; ++u) {
                    const int ks = (st + u) * spw + kslot;
                    kr[u] = __builtin_amdgcn_raw_buffer_load_b128(krs, ks < ncache ? row_off(ks) : OOB_OFF, 0, 0);
                  }
#pragma unroll
                  for (int u = 0; u < KV_GRP; ++u) {
                    if (st + u < nstc) {
                      float kf[DPL];
                      kv_unpack<DPL>(kr[u], kf);
                      score((st + u) * spw + kslot, kf);
                    }
                  }
                }
                if (nk > 0 && kc_ >= P && w8 == 0 && lane < lpk) {   // the column's own key: from LDS
                  const float *kk = qkv + c * 3 * hd + hd + d0;
                  float sdot = 0.f;
#pragma unroll
                  for (int i = 0; i < DPL; ++i) sdot = fmaf(qv[i], kk[i], sdot);
                  sdot = group_sum(sdot, lpk);
                  if (lane == 0) scc[nk - 1] = sdot * scale;
                }
              }
              lbar();
              if (w8 < ncol) {   // softmax of column w8
                const int c = w8, nk = nk_of(bposl[c]);
                float *scc = scv + c * 640;
                float mv = -INFINITY;
                for (int i = lane; i < nk; i += 64) mv = fmaxf(mv, scc[i]);
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) mv = fmaxf(mv, __shfl_xor(mv, off, 64));
                float ls = 0.f;
                for (int i = lane; i < nk; i += 64) {
                  const float pe = __expf(scc[i] - mv);
                  scc[i] = pe;
                  ls += pe;
                }
                ls = wave_sum(ls);
                if (lane == 0) { mxv[2 * c] = mv; mxv[2 * c + 1] = ls; }
              }
              lbar();
#pragma unroll 1
              for (int c = 0; c < ncol; ++c) {   // P.V
                const int P = bposl[c], ncache = ncache_of(P), nstc = (ncache + spw - 1) / spw, nk = nk_of(P);
                const int kc_ = lg + MK_NG * (nk - 1);
                ConstLayer &cl = ((ConstLayer *)(uintptr_t)a.seq_layers[c])[li];
                const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(cl.vc, 0, 0x7fffffff, RSRC_W3);
                const float *scc = scv + c * 640;
                float acc[DPL];
#pragma unroll
                for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
                auto pvacc = [&](int ks, const float (&vf)[DPL]) {
                  const float pe = (ks < ncache) ? scc[ks < ncache ? ks : 0] : 0.f;
#pragma unroll
                  for (int i = 0; i < DPL; ++i) acc[i] = fmaf(pe, vf[i], acc[i]);
                };
                if (nstc > 0) {
                  float vf[DPL];
                  kv_unpack<DPL>(wsel(c, std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{}), vf);
                  pvacc(kslot, vf);
                }
                if (nstc > 1) {
                  float vf[DPL];
                  kv_unpack<DPL>(wsel(c, std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{}), vf);
                  pvacc(spw + kslot, vf);
                }
#pragma unroll 1
                for (int st = NPRE; st < nstc; st += KV_GRP) {
                  u32x4 vr[KV_GRP];
#pragma unroll
                  for (int u = 0; u < KV_GRP; ++u) {
                    const int ks = (st + u) * spw + kslot;
                    vr[u] = __builtin_amdgcn_raw_buffer_load_b128(vrs, ks < ncache ? row_off(ks) : OOB_OFF, 0, 0);
                  }
#pragma unroll
                  for (int u = 0; u < KV_GRP; ++u) {
                    if (st + u < nstc) {
                      float vf[DPL];
                      kv_unpack<DPL>(vr[u], vf);
                      pvacc((st + u) * spw + kslot, vf);
                    }
                  }
                }
                const int kcs = (nk - 1) % spw;
                if (nk > 0 && kc_ >= P && w8 == kcs / kpw && lane / lpk == kcs % kpw) {   // own value, in step order
                  const float pe = scc[nk - 1];
                  const float *vv = qkv + c * 3 * hd + 2 * hd + d0;
#pragma unroll
                  for (int i = 0; i < DPL; ++i) acc[i] = fmaf(pe, vv[i], acc[i]);
                }
#pragma unroll
                for (int i = 0; i < DPL; ++i) {
                  float v = acc[i];
                  if (lpk == 16) {
                    v = swap_add32(v, v);
                    v = swap_add16(v, v);
                  } else {
                    for (int o = lpk; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
                  }
                  acc[i] = v;
                }
                if (lane < lpk) {
#pragma unroll
                  for (int i = 0; i < DPL; ++i) pvv[(c * MK_WAVES + w8) * hd + d0 + i] = acc[i];
                }
              }
              lbar();
              const int plen = hd + 2;
              for (int i = tid; i < ncol * hd; i += MK_THREADS) {
                const int c = i / hd, d = i - c * hd;
                const float *pc = pvv + c * MK_WAVES * hd;
                float a2 = pc[d];
#pragma unroll 1
                for (int ww = 1; ww < MK_WAVES; ++ww) a2 += pc[ww * hd + d];
                pub_xcd(xo + c * x_o_len + lg * plen + 2 + d, a2, tg);
              }
              if (tid < ncol) {
                const int c = tid, nk = nk_of(bposl[c]);
                uint2 *dst = xo + c * x_o_len + lg * plen;
                pub_xcd(dst + 0, nk > 0 ? mxv[2 * c] : -INFINITY, tg);
                pub_xcd(dst + 1, nk > 0 ? mxv[2 * c + 1] : 0.f, tg);
              }
              lbar();
            } else {
#pragma unroll 1
              for (int c = 0; c < ncol; ++c) {
                // first position of this forward in column c's sequence: cached keys are below it
                const int base = BAT ? bposl[c] : pos0;
                const int P = BAT ? base : pos0 + c;  // query position; keys 0..P
                // cached keys of this workgroup: slots [0, ncache)
                const int ncache = (base > lg) ? (base - 1 - lg) / MK_NG + 1 : 0;
                const int nstc = (ncache + spw - 1) / spw;
                // (batch: column c's own cache, its sequence's K and V of this layer)
                ConstLayer &cl = ((ConstLayer *)(uintptr_t)a.seq_layers[BAT ? c : 0])[li];
                const __amdgpu_buffer_rsrc_t krs = BAT ? __builtin_amdgcn_make_buffer_rsrc(cl.kc, 0, 0x7fffffff, RSRC_W3) : krs0;
                const __amdgpu_buffer_rsrc_t vrs = BAT ? __builtin_amdgcn_make_buffer_rsrc(cl.vc, 0, 0x7fffffff, RSRC_W3) : vrs0;
                const int nk = (P >= lg) ? (P - lg) / MK_NG + 1 : 0;
                // this forward's key of this workgroup, if any: position kc_ in [base, P], slot nk - 1
                const int kc_ = lg + MK_NG * (nk - 1);
                const bool hascur = nk > 0 && kc_ >= base;
                const int crow = BAT ? c : kc_ - pos0;   // its row of this forward's K, V in LDS
                float qv[DPL];
  #pragma unroll
                for (int i = 0; i < DPL; ++i) qv[i] = qkv[c * 3 * hd + d0 + i];
                auto score = [&](int ks, const float (&kf)[DPL], float ksc) {
                  float sdot = 0.f;
  #pragma unroll
                  for (int i = 0; i < DPL; ++i) sdot = fmaf(qv[i], kf[i], sdot);
                  if constexpr (KVQ) sdot *= ksc;
                  sdot = group_sum(sdot, lpk);
                  if (ks < ncache && (lane % lpk) == 0) sc[ks] = sdot * scale;
                };
  #pragma unroll
                for (int st = 0; st < NPRE; ++st) {
                  if (st < nstc) {
                    float kf[DPL];
                    kv_unpack<DPL>(!BAT ? wr[2 * NRG_IN + NRG_O + 2 * st]
                                   : st == 0 ? wsel(c, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{})
                                             : wsel(c, std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{}), kf);
                    score(st * spw + kslot, kf, KVQ ? q8_scale(kvx[st] & 0xffu) : 1.f);
                  }
                }
                // later steps: KV_GRP steps' loads issued together, then used in step order
  #pragma unroll 1
                for (int st = NPRE; st < nstc; st += KV_GRP) {
                  u32x4 kr[KV_GRP];
                  uint32_t ke[KV_GRP];
  #pragma unroll
                  for (int u = 0; u < KV_GRP; ++u) {
                    const int ks = (st + u) * spw + kslot;
                    kr[u] = __builtin_amdgcn_raw_buffer_load_b128(krs, ks < ncache ? row_off(ks) : OOB_OFF, 0, 0);
                    if constexpr (KVQ) ke[u] = __builtin_amdgcn_raw_buffer_load_b8(ers, ks < ncache ? kve_off(ptl, lg + MK_NG * ks, kvh, nkv) : OOB_OFF, 0, 0);
                    else ke[u] = 0;
                  }
  #pragma unroll
                  for (int u = 0; u < KV_GRP; ++u) {
                    if (st + u < nstc) {
                      float kf[DPL];
                      kv_unpack<DPL>(kr[u], kf);
                      score((st + u) * spw + kslot, kf, KVQ ? q8_scale(ke[u]) : 1.f);
                    }
                  }
                }
                if (hascur && w8 == 0 && lane < lpk) {   // this forward's key: from LDS
                  const float *kk = qkv + crow * 3 * hd + hd + d0;
                  float sdot = 0.f;
  #pragma unroll
                  for (int i = 0; i < DPL; ++i) sdot = fmaf(qv[i], kk[i], sdot);
                  if constexpr (KVQ) sdot *= kvs[crow * 2];
                  sdot = group_sum(sdot, lpk);
                  if (lane == 0) sc[nk - 1] = sdot * scale;
                }
                lbar();
                if (w8 == 0) {
                  float mv = -INFINITY;
                  for (int i = lane; i < nk; i += 64) mv = fmaxf(mv, sc[i]);
  #pragma unroll
                  for (int off = 32; off > 0; off >>= 1) mv = fmaxf(mv, __shfl_xor(mv, off, 64));
                  float ls = 0.f;
                  for (int i = lane; i < nk; i += 64) {
                    const float pe = __expf(sc[i] - mv);
                    sc[i] = pe;
                    ls += pe;
                  }
                  ls = wave_sum(ls);
                  if (lane == 0) { mx[0] = mv; mx[1] = ls; }
                }
                lbar();
                // P.V over the same slots: each lane accumulates its 8 dimensions
                float acc[DPL];
  #pragma unroll
                for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
                auto pvacc = [&](int ks, const float (&vf)[DPL], float vsc) {
                  float pe = (ks < ncache) ? sc[ks < ncache ? ks : 0] : 0.f;
                  if constexpr (KVQ) pe *= vsc;
  #pragma unroll
                  for (int i = 0; i < DPL; ++i) acc[i] = fmaf(pe, vf[i], acc[i]);
                };
  #pragma unroll
                for (int st = 0; st < NPRE; ++st) {
                  if (st < nstc) {
                    float vf[DPL];
                    kv_unpack<DPL>(!BAT ? wr[2 * NRG_IN + NRG_O + 2 * st + 1]
                                   : st == 0 ? wsel(c, std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{})
                                             : wsel(c, std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{}), vf);
                    pvacc(st * spw + kslot, vf, KVQ ? q8_scale(kvx[st] >> 8) : 1.f);
                  }
                }
  #pragma unroll 1
                for (int st = NPRE; st < nstc; st += KV_GRP) {
                  u32x4 vr[KV_GRP];
                  uint32_t ve[KV_GRP];
  #pragma unroll
                  for (int u = 0; u < KV_GRP; ++u) {
                    const int ks = (st + u) * spw + kslot;
                    vr[u] = __builtin_amdgcn_raw_buffer_load_b128(vrs, ks < ncache ? row_off(ks) : OOB_OFF, 0, 0);
                    if constexpr (KVQ) ve[u] = __builtin_amdgcn_raw_buffer_load_b8(ers, ks < ncache ? kve_off(ptl, lg + MK_NG * ks, kvh, nkv) + 1 : OOB_OFF, 0, 0);
                    else ve[u] = 0;
                  }
  #pragma unroll
                  for (int u = 0; u < KV_GRP; ++u) {
                    if (st + u < nstc) {
                      float vf[DPL];
                      kv_unpack<DPL>(vr[u], vf);
                      pvacc((st + u) * spw + kslot, vf, KVQ ? q8_scale(ve[u]) : 1.f);
                    }
                  }
                }
                // this forward's value, from LDS, added by the lanes that own its slot in the step order
                // (as a cached key of a later decode step it is accumulated there: same additions, same
                // order, so verify and sequential decode agree bit for bit)
                const int kcs = (nk - 1) % spw;
                if (hascur && w8 == kcs / kpw && lane / lpk == kcs % kpw) {
                  float pe = sc[nk - 1];
                  if constexpr (KVQ) pe *= kvs[crow * 2 + 1];
                  const float *vv = qkv + crow * 3 * hd + 2 * hd + d0;
  #pragma unroll
                  for (int i = 0; i < DPL; ++i) acc[i] = fmaf(pe, vv[i], acc[i]);
                }
                // sum over the kpw key groups of the wave (lanes l, l + lpk, ...), then over the waves
  #pragma unroll
                for (int i = 0; i < DPL; ++i) {
                  float v = acc[i];
                  if (lpk == 16) {
                    v = swap_add32(v, v);
                    v = swap_add16(v, v);
                  } else if (lpk == 8) {
                    v = dpp_add<DPP_ROR8>(v);   // (l, l ^ 8) within each row of 16 lanes
                    v = swap_add32(v, v);
                    v = swap_add16(v, v);
                  } else {
                    for (int o = lpk; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
                  }
                  acc[i] = v;
                }
                if (lane < lpk) {
  #pragma unroll
                  for (int i = 0; i < DPL; ++i) pv[w8 * hd + d0 + i] = acc[i];
                }
                lbar();
                const int plen = hd + 2;
                uint2 *dst = xo + c * x_o_len + lg * plen;
                for (int d = tid; d < hd; d += MK_THREADS) {
                  float a2 = pv[d];
  #pragma unroll 1
                  for (int ww = 1; ww < MK_WAVES; ++ww) a2 += pv[ww * hd + d];
                  pub_xcd(dst + 2 + d, a2, tg);
                }
                if (tid == 0) {
                  pub_xcd(dst + 0, nk > 0 ? mx[0] : -INFINITY, tg);
                  pub_xcd(dst + 1, nk > 0 ? mx[1] : 0.f, tg);
                }
                lbar();
              }
            }
          }
          MK_TRACE_POINT(li, 4);
          // ---- A3: merge the 16 partials + o-projection columns of head x
          {
            // every column's partials in one gather; the scales of column c in wave c; then the
            // merged outputs of all columns (per column the same arithmetic as one column alone)
            const int plen = hd + 2;
            float *ov = work;                        // [NCOL][hd]
            float *part = work + NCOL * hd;          // [NCOL][16][plen]
            float *scl = part + NCOL * MK_NG * plen; // [NCOL][17]: per-partial scales, [16] = sum of l_w * scale
            constexpr int A3C = NCOL == 1 ? 3 : 6;
            if (!gather2d<A3C, MK_WAVES>(xo, ncol, MK_NG * plen, x_o_len, tg, part, flag, m.ctl, SITE(7), tid)) MK_BAIL();
            // per-partial scale exp(m_w - M) (0 for workgroups without keys)
            if (w8 < ncol) {
              const float *pc = part + w8 * MK_NG * plen;
              float *sc = scl + w8 * (MK_NG + 1);
              const bool has = lane < MK_NG && pc[lane * plen + 1] > 0.f;
              float M = has ? pc[lane * plen] : -INFINITY;
#pragma unroll
              for (int off = MK_NG / 2; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
              const float sv = has ? __expf(pc[lane * plen] - M) : 0.f;
              if (lane < MK_NG) sc[lane] = sv;
              if (lane == 0) {  // (LDS writes of one wave are seen by its later reads)
                float Ls = 0.f;
                for (int ww = 0; ww < MK_NG; ++ww) Ls = fmaf(pc[ww * plen + 1], sc[ww], Ls);
                sc[MK_NG] = Ls;
              }
            }
            lbar();
            for (int i = tid; i < ncol * hd; i += MK_THREADS) {
              const int c = i / hd, d = i - c * hd;
              const float *pc = part + c * MK_NG * plen;
              const float *sc = scl + c * (MK_NG + 1);
              float acc = 0.f;
#pragma unroll 8
              for (int ww = 0; ww < MK_NG; ++ww) acc = fmaf(pc[ww * plen + 2 + d], sc[ww], acc);
              ov[c * hd + d] = acc / sc[MK_NG];
            }
            lbar();
            MK_TRACE_POINT(li, 5);
            const int kl = (lane & (G_a - 1)) * 8;
            FOR_COL_R(c) {
#pragma unroll
              for (int r = 0; r < NRG_O; ++r) {
                const int rg = wx + r * XW;
                float f[8], s = 0.f;
                unpack8(wr[2 * NRG_IN + r], f);
#pragma unroll
                for (int e = 0; e < 8; ++e) s = fmaf(f[e], ov[c * hd + kl + e], s);
                s = group_sum(s, G_a);
                if (rg < H / RG_a && (lane & (G_a - 1)) == 0)
                  pub(x_mix_l + ((size_t)c * MK_NX + x) * H + rg * RG_a + lane / G_a, s, tg);
              }
            }
          }
        } else {
          for (int i = tid + lg * MK_THREADS; i < H; i += MK_NG * MK_THREADS)
            for (int c = 0; c < ncol; ++c) pub(x_mix_l + ((size_t)c * MK_NX + x) * H + i, 0.f, tg);
        }
      }
      MK_TRACE_POINT(li, 6);
      // ---- R1: residual after the mixer (reduce-scatter over the XCDs), for the FFN role
      if (!reduce_slices(x_mix_l, x_r1_l + (size_t)x * NCOL * H, SITE(8), tid)) MK_BAIL();
      MK_TRACE_POINT(li, 7);
      // the next layer's mixer weights and state, in flight while the FFN role works (after the
      // last layer: the final norm's gains)
      if (li + 1 < m.n_layers) issue_mixer(li + 1);
      else ld_gain16(m.lnf, H, G_h, true, gv);
    } else {
      // ============================================================ FFN of layer li
      MK_TRACE_POINT(li, 8);
      if (!gather2d<MCS, MK_WAVES>(x_r1_l + (size_t)x * NCOL * H, ncol, H, H, tg, xres, flag, m.ctl, SITE(9), tid)) MK_BAIL();
      MK_TRACE_POINT(li, 9);
      uint2 *xm = x_m_l + (size_t)x * NCOL * xm_len;
      // ---- F1: gate/up pairs j = wx + pr XW -> m_j = SiLU(g_j) u_j (weights already in registers)
      FOR_COL_R(c) {
        float av[16];
        rmsnorm_regs(xres + c * H, gv, H, G_h, L_h, m.rms_eps, av);
        if (RG_h == 1 && L_h == 2) {
          // two pairs at once: lanes [0,16) gate p, [16,32) gate p+1, [32,48) up p, [48,64) up p+1;
          // the permlane32 swap then puts gate and up of pair p in lane 0 and of pair p+1 in lane 16
#pragma unroll
          for (int pp = 0; pp < NPAIR; pp += 2) {
            const float t = wave_sum4(dot16(wr[pp * 4 + 0], wr[pp * 4 + 1], av), dot16(wr[pp * 4 + 2], wr[pp * 4 + 3], av),
                                      dot16(wr[pp * 4 + 4], wr[pp * 4 + 5], av), dot16(wr[pp * 4 + 6], wr[pp * 4 + 7], av));
            const u32x2 gu = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
            const int j = wx + (pp + (lane >> 4)) * XW;
            if ((lane == 0 || lane == 16) && j < J)
              pub_xcd(xm + c * xm_len + j, silu_f(__uint_as_float(gu.x)) * __uint_as_float(gu.y), tg);
          }
        } else {
#pragma unroll
          for (int pr = 0; pr < NPAIR; ++pr) {
            const int j = wx + pr * XW;
            float g, u;
            if (RG_h == 1) {  // gate = loads [0, L_h), up = loads [L_h, 2 L_h)
              g = rg_dot_regs(wr[pr * 4 + 0], L_h == 2 ? wr[pr * 4 + 1] : u32x4{0u, 0u, 0u, 0u}, G_h, av);
              u = rg_dot_regs(L_h == 2 ? wr[pr * 4 + 2] : wr[pr * 4 + 1], L_h == 2 ? wr[pr * 4 + 3] : u32x4{0u, 0u, 0u, 0u}, G_h, av);
            } else {  // one row group holds the pair: lanes [0,32) compute g_j, lanes [32,64) u_j
              g = rg_dot_regs(wr[pr * 4 + 0], wr[pr * 4 + 1], G_h, av);
              u = __shfl_xor(g, 32, 64);
            }
            if (lane == 0 && j < J) pub_xcd(xm + c * xm_len + j, silu_f(g) * u, tg);
          }
        }
      }
      MK_TRACE_POINT(li, 10);
      // ---- F2: down-projection columns of slice x
      {
        float *mv = work;  // [NCOL][J]
        if (!gather2d<MCS, MK_WAVES>(xm, ncol, J, xm_len, tg, mv, flag, m.ctl, SITE(11), tid)) MK_BAIL();
        MK_TRACE_POINT(li, 11);
        if (wx < H / RG_d) {
          const int kl = (lane & (G_d - 1)) * 8;
          FOR_COL_R(c) {
            // every activation load of the column first, then the products alternating between two
            // accumulators (the loads overlap, the dependent chain is half as long)
            float4 av[LMAX_D][2];
#pragma unroll
            for (int i = 0; i < LMAX_D; ++i) {   // (past L_d: a valid re-read, unused)
              const int k0 = (i < L_d ? i : 0) * G_d * 8 + kl;
              av[i][0] = *reinterpret_cast<const float4 *>(mv + c * J + k0);
              av[i][1] = *reinterpret_cast<const float4 *>(mv + c * J + k0 + 4);
            }
            float s0 = 0.f, s1 = 0.f;
#pragma unroll
            for (int i = 0; i < LMAX_D; ++i) {
              if (i < L_d) {
                float f[8];
                unpack8(wr[4 * NPAIR + i], f);
                s0 = fmaf(f[0], av[i][0].x, s0); s1 = fmaf(f[1], av[i][0].y, s1);
                s0 = fmaf(f[2], av[i][0].z, s0); s1 = fmaf(f[3], av[i][0].w, s1);
                s0 = fmaf(f[4], av[i][1].x, s0); s1 = fmaf(f[5], av[i][1].y, s1);
                s0 = fmaf(f[6], av[i][1].z, s0); s1 = fmaf(f[7], av[i][1].w, s1);
              }
            }
            const float oo = group_sum(s0 + s1, G_d);
            if ((lane & (G_d - 1)) == 0) pub(x_ffn_l + ((size_t)c * MK_NX + x) * H + wx * RG_d + lane / G_d, oo, tg);
          }
        }
      }
      MK_TRACE_POINT(li, 12);
      // ---- R2: residual after the FFN, for the mixer role of the next layer (and the LM head)
      uint2 *const x_r2_l = x_ffn_l + NCOL * MK_NX * H;
      if (!reduce_slices(x_ffn_l, x_r2_l + (size_t)x * NCOL * H, SITE(12), tid)) MK_BAIL();
      MK_TRACE_POINT(li, 13);
      if (li + 1 < m.n_layers) issue_ffn(li + 1);
      else ld_gain16(m.lnf, H, G_h, true, gv);
    }
  }  // layers

  // ================================================================ final residual, LM head, argmax
  {
    const int tid = tid0;
    uint2 *const x_r2_last = a.xch + (size_t)m.n_layers * mk_xch_layer_slots(NCOL, H, r_in_max, x_o_len, xm_len) -
                             (size_t)NCOL * MK_NX * H;
    li = m.n_layers;
    if (!gather2d<MCS, MK_WAVES>(x_r2_last + (size_t)x * NCOL * H, ncol, H, H, tg, xres, flag, m.ctl, SITE(13), tid)) MK_BAIL();
  }
  MK_TRACE_POINT(li, 0);
  uint4 *const x_arg = reinterpret_cast<uint4 *>(a.xch + (size_t)m.n_layers * mk_xch_layer_slots(NCOL, H, r_in_max, x_o_len, xm_len));
  {
    const int tid = tid0;
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
    // this lane's activations of every column: RMSNorm(x) * g in the operand layout
    float av[NCOL][16];
#pragma unroll
    for (int c = 0; c < NCOL; ++c) {
      if (c < ncol) rmsnorm_regs(xres + c * H, gv, H, G_h, L_h, m.rms_eps, av[c]);
      else {
#pragma unroll
        for (int e = 0; e < 16; ++e) av[c][e] = 0.f;
      }
    }
    // embedding rows stream through two register batches: the next batch's loads are issued
    // before the current one is multiplied (branch-free: rows past this wave's range read zeros)
    const __amdgpu_buffer_rsrc_t ers = tile_rsrc(m.embed, (uint32_t)((size_t)m.V * H * 2));
    auto lm_load = [&](int rb, u32x4 (&wb)[B][2]) {
#pragma unroll
      for (int r = 0; r < B; ++r) {
        const bool ok = rb + r < wg1;
        const uint32_t o0 = ok ? (uint32_t)(((size_t)(rb + r) * L_h * 64 + lane) * 16) : OOB_OFF;
        wb[r][0] = __builtin_amdgcn_raw_buffer_load_b128(ers, o0, 0, AUX_NT);
        wb[r][1] = (L_h > 1) ? __builtin_amdgcn_raw_buffer_load_b128(ers, ok ? o0 + 1024u : OOB_OFF, 0, AUX_NT)
                             : u32x4{0u, 0u, 0u, 0u};
      }
    };
    auto lm_compute = [&](int rb, const u32x4 (&wb)[B][2]) {
#pragma unroll
      for (int c = 0; c < NCOL; ++c) {
        if (c >= ncol) break;
        if (G_h == 64 && B == 8) {
          float part[8];
#pragma unroll
          for (int r = 0; r < 8; ++r) part[r] = dot16(wb[r][0], wb[r][1], av[c]);
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
            const float pl = dot16(wb[r][0], wb[r][1], av[c]);
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
    MK_TRACE_POINT(li, 1);
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
      unsigned long long *rec = reinterpret_cast<unsigned long long *>(x_arg + c * MK_NWG + b);
      __hip_atomic_store(rec, ((unsigned long long)(uint32_t)bi << 32) | __float_as_uint(bv), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      wait_stores();  // value and index land before the tag word
      __hip_atomic_store(rec + 1, ((unsigned long long)(uint32_t)(nn | rot << 8) << 32) | tg, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  lbar();  // the candidate above was read from the scratch the final gather reuses
  if (b == 0) {
    const int tid = tid0;
    // final argmax over the 256 workgroup candidates; the tag word is written after the
    // value/index word by the same thread, so a matching tag implies the record is complete
    float *cv = work;                         // [NCOL][256]
    int *ci = reinterpret_cast<int *>(work + NCOL * MK_NWG);
    int *cn = reinterpret_cast<int *>(work + 2 * NCOL * MK_NWG);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(x_arg, 0, NCOL * MK_NWG * 16, RSRC_W3);
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
      cn[i] = (int)(v.w & 0xffu);
      if ((int)(v.w >> 8) != rot) flag[1] = 1;   // placement rotation of workgroup i % 256
    }
    lbar();
    if (flag[0]) MK_BAIL();
    MK_TRACE_POINT(li, 2);
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
        if (flag[1]) __hip_atomic_fetch_or(m.ctl + MK_CTL_ERR, MK_DERR_XCD, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if constexpr (BAT) {   // every sequence of the batch advances by its one token
#pragma unroll
          for (int c = 0; c < NCOL; ++c)
            if (c < ncol) __hip_atomic_store(a.seq_ctl[c] + MK_CTL_POS, bpos[c] + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          const int consumed = verify ? nacc : 1;
          __hip_atomic_store(m.ctl + MK_CTL_POS, ctl_pos + consumed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(m.ctl + MK_CTL_PEND, verify ? nacc : 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(m.ctl + MK_CTL_PAR, verify ? (par ^ 1) : par, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }
}
