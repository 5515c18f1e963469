// tq4_probe.hip -- streaming-read bandwidth probe (tq4_probe.h).
//
// The buffer is cut into blocks of kProbeThreads * U 16-byte words; workgroup w reads blocks
// w, w + W, w + 2 W, ... (W workgroups).  Inside a block, thread t loads words t + kProbeThreads k
// for k < U, all U loads issued before any is used, so every load instruction of a wavefront covers
// one contiguous KiB and a workgroup has kProbeThreads * U * 16 bytes in flight.  The loaded words
// are folded with XOR into one word per thread, so no load can be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq4_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kProbeThreads = 512;

template <int U>
__global__ __launch_bounds__(kProbeThreads) void tq4_probe_read_kernel(const u32x4 *p, size_t n16, uint32_t *sink) {
    constexpr size_t kBlock = static_cast<size_t>(kProbeThreads) * U;  // 16-byte words per block
    const size_t n_full = n16 / kBlock;
    const size_t t = threadIdx.x;
    uint32_t acc = 0;
    for (size_t blk = blockIdx.x; blk < n_full; blk += gridDim.x) {
        const u32x4 *b = p + blk * kBlock + t;
        u32x4 v[U];
#pragma unroll
        for (int k = 0; k < U; ++k) v[k] = b[static_cast<size_t>(k) * kProbeThreads];
#pragma unroll
        for (int k = 0; k < U; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
    // the words past the last full block, one load per thread and step
    const size_t stride = static_cast<size_t>(gridDim.x) * kProbeThreads;
    for (size_t i = n_full * kBlock + static_cast<size_t>(blockIdx.x) * kProbeThreads + t; i < n16; i += stride) {
        const u32x4 a = p[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    sink[static_cast<size_t>(blockIdx.x) * kProbeThreads + t] = acc;
}

}  // namespace

extern "C" {

size_t tq4_probe_sink_words(int32_t workgroups) {
    if (workgroups < 1 || workgroups > 65535) return 0;
    return static_cast<size_t>(workgroups) * kProbeThreads;
}

int tq4_probe_stream_read(const void *src, size_t bytes, void *sink, int32_t workgroups, int32_t loads_in_flight,
                          void *stream) {
    if (src == nullptr || sink == nullptr || bytes == 0 || bytes % 16 != 0) return -1;
    if ((reinterpret_cast<uintptr_t>(src) & 15) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3) != 0) return -1;
    if (workgroups < 1 || workgroups > 65535) return -1;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const u32x4 *p = static_cast<const u32x4 *>(src);
    uint32_t *out = static_cast<uint32_t *>(sink);
    const dim3 grid(static_cast<unsigned>(workgroups)), block(kProbeThreads);
    switch (loads_in_flight) {
        case 4: hipLaunchKernelGGL(tq4_probe_read_kernel<4>, grid, block, 0, s, p, bytes / 16, out); break;
        case 8: hipLaunchKernelGGL(tq4_probe_read_kernel<8>, grid, block, 0, s, p, bytes / 16, out); break;
        case 16: hipLaunchKernelGGL(tq4_probe_read_kernel<16>, grid, block, 0, s, p, bytes / 16, out); break;
        default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
