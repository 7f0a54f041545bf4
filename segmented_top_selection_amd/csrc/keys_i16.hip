// Top-k kernels for signed 16-bit integer keys (one translation unit per key type, so
// that the library builds in parallel).
#include "topk_kernel.h"

namespace segtopk_impl {
template hipError_t launch_topk<SEGTOPK_KEY_I16>(const Params &, bool, int, uint32_t, size_t, hipStream_t);
template int topk_per_cu<SEGTOPK_KEY_I16>(bool, size_t);
}  // namespace segtopk_impl
