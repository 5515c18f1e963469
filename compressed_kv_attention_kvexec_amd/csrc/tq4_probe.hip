// tq4_probe.hip -- streaming-read bandwidth probe (tq4_probe.h): a plain grid-stride read
// with four 16-byte loads in flight per thread, 256 threads per workgroup.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq4_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void tq4_probe_read_kernel(const u32x4 *p, size_t n64, uint32_t *sink) {
    // thread t reads 16-byte words t, t + S, t + 2 S, ... (S = threads in the grid), four per
    // iteration, so each load instruction of a wavefront covers one contiguous KiB
    const size_t stride = static_cast<size_t>(gridDim.x) * kProbeThreads;
    const size_t tid = static_cast<size_t>(blockIdx.x) * kProbeThreads + threadIdx.x;
    const size_t n = n64 * 4;  // 16-byte words
    uint32_t acc = 0;
    size_t i = tid;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const u32x4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n; i += stride) {
        const u32x4 a = p[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    sink[tid] = acc;
}

}  // namespace

extern "C" {

size_t tq4_probe_sink_words(int32_t workgroups) {
    if (workgroups < 1 || workgroups > 65535) return 0;
    return static_cast<size_t>(workgroups) * kProbeThreads;
}

int tq4_probe_stream_read(const void *src, size_t bytes, void *sink, int32_t workgroups, void *stream) {
    if (src == nullptr || sink == nullptr || bytes == 0 || bytes % 64 != 0) return -1;
    if ((reinterpret_cast<uintptr_t>(src) & 15) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3) != 0) return -1;
    if (workgroups < 1 || workgroups > 65535) return -1;
    hipLaunchKernelGGL(tq4_probe_read_kernel, dim3(static_cast<unsigned>(workgroups)), dim3(kProbeThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(src), bytes / 64,
                       static_cast<uint32_t *>(sink));
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
