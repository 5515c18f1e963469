// tq4_encode.hip -- TQ4 encoder for gfx950: one wavefront per 256-dim vector.
//
// Record format and the decode steps it must invert: "Fitting a 27B-Parameter
// LLM into 24 GiB of Laptop Memory", section "KVExec: Fused Reconstruction
// with Layer-Scoped Lifetime" (32 u32 words of eight 4-bit indices plus one
// fp16 norm; centroid lookup, inverse Hadamard rotation, norm restore).
//
// The per-vector algorithm (fixed so every implementation gets the same bits) is in
// tq4_encode_wave.h.
#pragma clang fp contract(off)

#include "tq4_device.h"
#include "tq4_encode_wave.h"
#include "tq4_launch.h"

namespace tq4 {

struct EncodeArgs {
    EncodeParams p;
    float thr[15];
};

__global__ __launch_bounds__(256) void tq4_encode_kernel(EncodeArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t vec = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int64_t per_half = static_cast<int64_t>(a.p.n_tokens) * a.p.n_kv;
    // vectors are ordered [half][token][kv head]; halves with no source are not launched
    int half;
    int64_t rem;
    if (a.p.src[0] != nullptr) {
        half = vec < per_half ? 0 : 1;
        rem = vec - half * per_half;
    } else {
        half = 1;
        rem = vec;
    }
    if (rem >= per_half || a.p.src[half] == nullptr) return;
    const int token = static_cast<int>(rem / a.p.n_kv);
    const int head = static_cast<int>(rem % a.p.n_kv);
    const int slot = a.p.slots[token];
    if (slot < 0 || slot >= a.p.num_slots) return;
    const int page = slot / a.p.page_size;
    const int off = slot - page * a.p.page_size;
    const int64_t rec = (static_cast<int64_t>(page) * a.p.n_kv + head) * a.p.page_size + off;
    const size_t esize = a.p.src_bf16 ? 2 : 4;
    encode_vector_wave(static_cast<const char *>(a.p.src[half]) + rem * kDim * esize, a.p.src_bf16 != 0, a.thr,
                       a.p.words[half] + rec * kWords, a.p.norms[half] + rec, lane);
}

hipError_t launch_encode(const EncodeParams &p, hipStream_t stream) {
    EncodeArgs a;
    a.p = p;
    const Codebook &cb = codebook();
    for (int i = 0; i < 15; ++i) a.thr[i] = cb.threshold[i];
    const int halves = (p.src[0] != nullptr) + (p.src[1] != nullptr);
    const int64_t vectors = static_cast<int64_t>(halves) * p.n_tokens * p.n_kv;
    if (vectors == 0) return hipSuccess;
    const int64_t blocks = (vectors + 3) / 4;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(tq4_encode_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace tq4
