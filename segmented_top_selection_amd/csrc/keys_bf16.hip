// Top-k kernels for bfloat16 keys (one translation unit per key type, so
// that the library builds in parallel).
#include "topk_kernel.h"

namespace segtopk_impl {
template hipError_t launch_topk<SEGTOPK_KEY_BF16>(const Params &, bool, int, uint32_t, size_t, hipStream_t);
template int topk_per_cu<SEGTOPK_KEY_BF16>(bool, size_t);
}  // namespace segtopk_impl
