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

constexpr int kEncWaves = 4;               // wavefronts per workgroup
constexpr int64_t kEncMaxWorkgroups = 2048;  // 8 per CU (all resident): each wavefront loops over vectors
constexpr int kEncDropOffset = 0x40000000;   // a buffer offset past any record: the store is dropped
constexpr int kBufferFlags = 0x00020000;     // raw 32-bit buffer resource word 3

// Each wavefront encodes vectors wave0, wave0 + stride, ... ([half][token][kv head] order).  The
// loop body has no branches: the next vector's source and slot are requested (index clamped)
// before the current vector is encoded, and the record is written through buffer resources that
// cover exactly the record (or nothing, for a slot outside the pool), so lanes that must not
// store and invalid slots are dropped by the hardware.  With no branch around loads or stores
// the compiler's wait counts stay exact: each iteration waits only for its own source.
template <bool BF16>
__global__ __launch_bounds__(kEncWaves * kWave) void tq4_encode_kernel(EncodeArgs a) {
    const int lane = threadIdx.x & 63;
    // vector indices fit in 31 bits (the launch checks it)
    const int wave0 = static_cast<int>(blockIdx.x) * kEncWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int stride = static_cast<int>(gridDim.x) * kEncWaves;
    const int per_half = a.p.n_tokens * a.p.n_kv;
    const int first_half = a.p.src[0] != nullptr ? 0 : 1;
    const int total = per_half * ((a.p.src[0] != nullptr) + (a.p.src[1] != nullptr));
    if (wave0 >= total) return;
    constexpr size_t esize = BF16 ? 2 : 4;
    auto half_of = [&](int vec) { return first_half + static_cast<int>(vec >= per_half); };
    auto rem_of = [&](int vec) { return vec - (vec >= per_half ? per_half : 0); };
    auto load = [&](int vec, float x[4], int &slot) {
        const int rem = rem_of(vec);
        encode_load(static_cast<const char *>(a.p.src[half_of(vec)]) + static_cast<int64_t>(rem) * kDim * esize, BF16,
                    lane, x);
        slot = a.p.slots[rem / a.p.n_kv];
    };
    const int word_off = (lane & 1) ? kEncDropOffset : (lane >> 1) * 4;
    const int norm_off = lane == 0 ? 0 : kEncDropOffset;

    // encode vector vec from x (slot = its page-table slot) and write its record; live == false
    // (a clamped repeat of a vector past the end) drops both stores
    auto encode_store = [&](int vec, const float x[4], int slot, bool live) {
        const int half = half_of(vec);
        const int head = rem_of(vec) % a.p.n_kv;
        const int s_u = __builtin_amdgcn_readfirstlane(slot);
        const bool valid = live && s_u >= 0 && s_u < a.p.num_slots;
        const int sl = valid ? s_u : 0;
        const int page = sl / a.p.page_size;
        const int64_t rec = (static_cast<int64_t>(page) * a.p.n_kv + head) * a.p.page_size + (sl - page * a.p.page_size);
        uint32_t word;
        const float n32 = encode_compute(x, a.thr, lane, word);
        const __amdgpu_buffer_rsrc_t wr =
            __builtin_amdgcn_make_buffer_rsrc(a.p.words[half] + rec * kWords, 0, valid ? kWords * 4 : 0, kBufferFlags);
        const __amdgpu_buffer_rsrc_t nr =
            __builtin_amdgcn_make_buffer_rsrc(a.p.norms[half] + rec, 0, valid ? 2 : 0, kBufferFlags);
        __builtin_amdgcn_raw_buffer_store_b32(word, wr, word_off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b16(f32_to_f16_bits(n32), nr, norm_off, 0, 0);
    };

    // two register sets used in turn (no copies between iterations)
    float x0[4], x1[4];
    int slot0, slot1;
    load(wave0, x0, slot0);
    {   // two dropped stores: the loop is entered with the same pending operations as its back edge
        const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(a.p.words[half_of(wave0)], 0, 0, kBufferFlags);
        __builtin_amdgcn_raw_buffer_store_b32(0u, none, word_off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(0), none, norm_off, 0, 0);
    }
    for (int vec = wave0; vec < total; vec += 2 * stride) {
        const bool live1 = vec < total - stride;
        const int v1 = live1 ? vec + stride : vec;
        load(v1, x1, slot1);
        __builtin_amdgcn_sched_barrier(0);  // requested before this vector's work
        encode_store(vec, x0, slot0, true);
        const int v2 = vec < total - 2 * stride ? vec + 2 * stride : vec;
        load(v2, x0, slot0);
        __builtin_amdgcn_sched_barrier(0);
        encode_store(v1, x1, slot1, live1);
    }
}

hipError_t launch_encode(const EncodeParams &p, hipStream_t stream) {
    EncodeArgs a;
    a.p = p;
    const Codebook &cb = codebook();
    for (int i = 0; i < 15; ++i) a.thr[i] = cb.threshold[i];
    const int halves = (p.src[0] != nullptr) + (p.src[1] != nullptr);
    const int64_t vectors = static_cast<int64_t>(halves) * p.n_tokens * p.n_kv;
    if (vectors == 0) return hipSuccess;
    if (vectors > 0x7fffffff - 2 * kEncMaxWorkgroups * kEncWaves) return hipErrorInvalidValue;
    int64_t blocks = (vectors + kEncWaves - 1) / kEncWaves;
    if (blocks > kEncMaxWorkgroups) blocks = kEncMaxWorkgroups;
    if (p.src_bf16)
        hipLaunchKernelGGL(tq4_encode_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(kEncWaves * kWave), 0, stream, a);
    else
        hipLaunchKernelGGL(tq4_encode_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(kEncWaves * kWave), 0, stream, a);
    return hipGetLastError();
}

}  // namespace tq4
