// mk_forward.hip -- decode instantiations of the persistent forward kernel (one column per
// launch) and the host-side launch entry points for both decode and verify.
#include <mutex>

#include "mk.h"
#include "mk_forward_kernel.h"

// ------------------------------------------------------------------------------ static exchange slots
// The exchange slots of mk_decode_step_static, for callers that cannot allocate: one array per
// device (each device holds its own copy of the code object's globals), kept until the process
// ends.  Zero at load, so every slot starts with tag 0, which no launch uses.  Host code must not
// pass `scratch` itself to a kernel (on the host it names a stand-in, not device memory): it takes
// the device address from mk_static_scratch and passes that.
static __device__ __align__(256) unsigned char scratch[MK_STATIC_SCRATCH_BYTES];

// Device address of `scratch` on the current device, looked up once per device (the library's
// load call does it with the model's device current).
extern "C" hipError_t mk_static_scratch(void **ptr) {
  static std::mutex mu;
  static void *addr[256] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 256) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || ((uintptr_t)p & 255) != 0) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

// ------------------------------------------------------------------------------ host-side launchers
// Instantiations: one decode column (here) or up to MK_MAXCOL verify columns (mk_verify.hip), each
// for the generic and the hidden-1024 shape, with a bf16 or an 8-bit KV cache.
const void *mk_verify_kernel(int variant);

static const void *forward_fn(int ncol_template, int variant) {
  if (ncol_template != 1) return mk_verify_kernel(variant);
  switch (variant) {
    case MK_SHAPE_H1024: return (const void *)mk_forward<1, MK_SHAPE_H1024>;
    case MK_SHAPE_ANY | MK_KV_Q8: return (const void *)mk_forward<1, MK_SHAPE_ANY | MK_KV_Q8>;
    case MK_SHAPE_H1024 | MK_KV_Q8: return (const void *)mk_forward<1, MK_SHAPE_H1024 | MK_KV_Q8>;
    default: return (const void *)mk_forward<1, MK_SHAPE_ANY>;
  }
}

// The workgroups wait for each other's data, so all 256 must be resident at once.  The launch does
// not need the cooperative-launch path for that (measured: it costs about 16 us per launch): the
// grid is one workgroup per CU (the LDS request admits one per CU, the host checks the occupancy
// and the CU count at load), launches on one stream run one after the other, and every wait is
// bounded -- if another process's kernel held CUs so that some workgroups could not start, the
// resident ones report MK_EHANG after the watchdog instead of waiting forever.
extern "C" hipError_t mk_launch_forward(const MkLaunch *a, int ncol_template, int variant, hipStream_t stream) {
  void *args[] = {const_cast<MkLaunch *>(a)};
  return hipLaunchKernel(forward_fn(ncol_template, variant), dim3(MK_NWG), dim3(MK_THREADS), args, MK_LDS_BYTES, stream);
}

extern "C" hipError_t mk_forward_occupancy(int ncol_template, int variant, int *blocks_per_cu) {
  const void *fn = forward_fn(ncol_template, variant);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, MK_LDS_BYTES);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, MK_THREADS, MK_LDS_BYTES);
}
