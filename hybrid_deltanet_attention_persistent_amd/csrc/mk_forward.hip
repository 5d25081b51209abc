// mk_forward.hip -- decode instantiations of the persistent forward kernel (one column per
// launch) and the host-side launch entry points for both decode and verify.
#include "mk_forward_kernel.h"

// ------------------------------------------------------------------------------ host-side launchers
// Instantiations: one decode column (here) or up to MK_MAXCOL verify columns (mk_verify.hip), each
// for the generic and the hidden-1024 shape.
const void *mk_verify_kernel(int shape);

static const void *forward_fn(int ncol_template, int shape) {
  if (ncol_template != 1) return mk_verify_kernel(shape);
  return (shape == MK_SHAPE_H1024) ? (const void *)mk_forward<1, MK_SHAPE_H1024> : (const void *)mk_forward<1, MK_SHAPE_ANY>;
}

// The workgroups wait for each other's data, so all 256 must be resident at once.  The launch does
// not need the cooperative-launch path for that (measured: it costs about 16 us per launch): the
// grid is one workgroup per CU (the LDS request admits one per CU, the host checks the occupancy
// and the CU count at load), launches on one stream run one after the other, and every wait is
// bounded -- if another process's kernel held CUs so that some workgroups could not start, the
// resident ones report MK_EHANG after the watchdog instead of waiting forever.
extern "C" hipError_t mk_launch_forward(const MkLaunch *a, int ncol_template, int shape, hipStream_t stream) {
  void *args[] = {const_cast<MkLaunch *>(a)};
  return hipLaunchKernel(forward_fn(ncol_template, shape), dim3(MK_NWG), dim3(MK_THREADS), args, MK_LDS_BYTES, stream);
}

extern "C" hipError_t mk_forward_occupancy(int ncol_template, int shape, int *blocks_per_cu) {
  const void *fn = forward_fn(ncol_template, shape);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, MK_LDS_BYTES);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, MK_THREADS, MK_LDS_BYTES);
}
