// Top-k kernel for unsigned 8-bit integer keys (one translation unit per key type, so
// that the library builds in parallel).
#include "topk_plain_kernel.h"

namespace segtopk_impl {
template hipError_t launch_topk_plain<SEGTOPK_KEY_U8>(const Params &, bool, uint32_t, size_t,
                                                        hipStream_t);
}  // namespace segtopk_impl
