// Tables of kernel instances by (op, protocol, form) for one element type,
// shared by the translation units that instantiate them.  The eager kernels
// and the captured ones (stream capture) are compiled in translation units of
// their own: built in one module with the captured instances, the eager
// Simple kernel came out with 128 VGPRs and a spill under its 128-register
// bound instead of 123 and none.
#pragma once

#include "ring_kernel_impl.h"

namespace ringar {

// The ring kernels of one collective (kAllReduce, kReduceScatter or
// kAllGather); LL128 has no small-slice form.
template <class E, int COLL, int OP, bool CAP>
const void* ring_instance(int proto, bool small) {
  if constexpr (CAP) {
    if (proto == kLL) return small ? (const void*)&ring_kernel_lines_captured<E, OP, kLL, true, COLL>
                                   : (const void*)&ring_kernel_lines_captured<E, OP, kLL, false, COLL>;
    if (proto == kLL128) return (const void*)&ring_kernel_lines_captured<E, OP, kLL128, false, COLL>;
  }
  if (proto == kLL) return small ? (const void*)&ring_kernel_lines<E, OP, kLL, true, COLL>
                                 : (const void*)&ring_kernel_lines<E, OP, kLL, false, COLL>;
  if (proto == kLL128) return (const void*)&ring_kernel_lines<E, OP, kLL128, false, COLL>;
  return small ? (const void*)&ring_kernel<E, OP, kSimple, true, COLL, CAP>
               : (const void*)&ring_kernel<E, OP, kSimple, false, COLL, CAP>;
}

template <class E, int COLL, bool CAP>
const void* ring_instance_by_op(int op, int proto, bool small) {
  switch (op) {
    case 0: return ring_instance<E, COLL, 0, CAP>(proto, small);
    case 1: return ring_instance<E, COLL, 1, CAP>(proto, small);
    case 2: return ring_instance<E, COLL, 2, CAP>(proto, small);
    case 3: return ring_instance<E, COLL, 3, CAP>(proto, small);
    default: return ring_instance<E, COLL, 4, CAP>(proto, small);
  }
}

template <class E, int OP, bool CAP>
const void* tree_instance(int proto, bool small) {
  if (proto == kSimpleSplitTree) {
    if constexpr (CAP) return nullptr;   // the captured form is never split
    else return (const void*)&tree_kernel_split<E, OP>;
  }
  if (proto == kLL) return small ? (const void*)&tree_kernel<E, OP, kLL, true, CAP>
                                 : (const void*)&tree_kernel<E, OP, kLL, false, CAP>;
  if (proto == kLL128) return (const void*)&tree_kernel<E, OP, kLL128, false, CAP>;
  return small ? (const void*)&tree_kernel_simple<E, OP, kSimple, true, CAP>
               : (const void*)&tree_kernel_simple<E, OP, kSimple, false, CAP>;
}

template <class E, bool CAP>
const void* tree_instance_by_op(int op, int proto, bool small) {
  switch (op) {
    case 0: return tree_instance<E, 0, CAP>(proto, small);
    case 1: return tree_instance<E, 1, CAP>(proto, small);
    case 2: return tree_instance<E, 2, CAP>(proto, small);
    case 3: return tree_instance<E, 3, CAP>(proto, small);
    default: return tree_instance<E, 4, CAP>(proto, small);
  }
}

}  // namespace ringar
