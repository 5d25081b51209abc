// mk_verify.hip -- verify and batch instantiations of the persistent forward kernel (up to
// MK_MAXCOL columns per launch).  Compiled apart from the decode unit, with the block-gather helpers
// always inlined.
#define MK_SEG_INLINE __forceinline__
#include "mk_forward_kernel.h"

const void *mk_verify_kernel(int variant) {
  switch (variant) {
    case MK_SHAPE_H1024: return (const void *)mk_forward<MK_MAXCOL, MK_SHAPE_H1024>;
    case MK_SHAPE_ANY | MK_KV_Q8: return (const void *)mk_forward<MK_MAXCOL, MK_SHAPE_ANY | MK_KV_Q8>;
    case MK_SHAPE_H1024 | MK_KV_Q8: return (const void *)mk_forward<MK_MAXCOL, MK_SHAPE_H1024 | MK_KV_Q8>;
    case MK_SHAPE_ANY | MK_BATCH: return (const void *)mk_forward<MK_MAXCOL, MK_SHAPE_ANY | MK_BATCH>;
    case MK_SHAPE_H1024 | MK_BATCH: return (const void *)mk_forward<MK_MAXCOL, MK_SHAPE_H1024 | MK_BATCH>;
    default: return (const void *)mk_forward<MK_MAXCOL, MK_SHAPE_ANY>;
  }
}
