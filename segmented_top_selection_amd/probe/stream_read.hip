// stream_read.hip -- measurement aid for the benchmark, not part of the top-k
// library: a plain streaming read of a device buffer with 16-byte
// non-temporal loads (the load the top-k kernels stream their keys with),
// eight loads per thread in flight, so that the benchmark can state each
// kernel's bandwidth against what a read-only stream reaches on the same
// device.  Each thread folds what it read into one word so that the loads
// are not dropped; one word per thread is written.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *src, uint64_t nvec,
                                                         uint32_t *sink) {
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    const v4u *p = reinterpret_cast<const v4u *>(src);
    const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    uint32_t acc = 0;
    uint64_t i = tid;
    for (; i + 7 * stride < nvec; i += 8 * stride) {
        v4u v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < nvec; i += stride) {
        const v4u v = __builtin_nontemporal_load(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    sink[tid] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16) from `src` with `workgroups` workgroups of
// 256 threads; `sink` must hold workgroups * 256 words.  Returns a hipError_t.
extern "C" int segtopk_probe_stream_read(const void *src, uint64_t bytes, uint32_t workgroups,
                                         uint32_t *sink, hipStream_t stream) {
    if (!src || !sink || workgroups == 0 || (bytes & 15)) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(256), 0, stream,
                       static_cast<const uint4 *>(src), bytes / 16, sink);
    return (int)hipGetLastError();
}
