// mk_verify.hip -- verify instantiations of the persistent forward kernel (up to MK_MAXCOL
// columns per launch).  Compiled apart from the decode unit, with the block-gather helpers
// always inlined.
#define MK_SEG_INLINE __forceinline__
#include "mk_forward_kernel.h"

const void *mk_verify_kernel(int shape) {
  return (shape == MK_SHAPE_H1024) ? (const void *)mk_forward<MK_MAXCOL, MK_SHAPE_H1024>
                                   : (const void *)mk_forward<MK_MAXCOL, MK_SHAPE_ANY>;
}
