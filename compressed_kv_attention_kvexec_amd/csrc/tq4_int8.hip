// tq4_int8.hip -- the uniform INT8 KV arm on gfx950: encoder, and decode attention over INT8 pages
// for one query token per request or its last n_queries tokens (the packed verifier) ("Fitting a
// 27B-Parameter LLM into 24 GiB of Laptop Memory", section "Reasoning at 200K: 29 of 30 AIME
// Problems": a uniform INT8 KV cache is the comparison arm of the TQ4 run).
//
// Record (the page fixes no format; this is the plain per-vector reading): 256 signed codes q_d in
// [-127, 127] and one fp16 scale s; the vector is q * s in the natural domain (no rotation).
// Encoding, fp32 with round to nearest even: s = fp16(max_d |x_d| / 127), q_d = clamp(rint(x_d / s),
// -127, 127), every code 0 when s == 0.
//
// Attention keeps the work decomposition of the TQ4 decode kernel: grid (split, KV head, request);
// the query rows of a KV head (G heads x n_queries tokens) are MFMA columns, 16 per block; a
// wavefront owns one block and every NS-th 32-key tile of its split (decode: one block, 8
// wavefronts, two per SIMD).  Per tile and wavefront:
//   S^T[32 keys][16] = C_K . Q^T       codes -> fp16 exactly     16 x v_mfma_f32_16x16x32_f16
//   x_j = S_j s_k,j, online softmax in base 2 (lazy rescale as in the TQ4 kernel)
//   O^T[256][16] += (C_V s_v)^T . P^T  each value code * scale rounded once to fp16, 16 MFMAs
// A code becomes fp16 with one v_cvt_f16_i16 reading the byte with sign extension (SDWA), so no
// table and no shift or pack instructions sit between the loads and the MFMAs.  The splits are
// merged by the shared combine kernel in the natural domain (o = O / L).
//
// Lane layout (lane = 16 gq + n):
//   K: M-tile mt, K-step ks: lane holds key 16 mt + n, dims 64 (ks / 2) + 16 gq + 8 (ks % 2) .. +7,
//      from one 16-byte load per (mt, ks / 2); the query operand uses the same dims per column n.
//   scores: lane holds column n, keys sigma(j) = j < 4 ? 4 gq + j : 16 + 4 gq + j - 4.
//   V: lane loads dims 16 n .. 16 n + 15 of keys sigma(0..7); M-tile e (0..15) takes byte e of
//      each key, so its row n is dim 16 n + e and lane (gq, n) accumulates dims 16 (4 gq + r) + e.
#pragma clang fp contract(off)

#include <cfloat>

#include "tq4_device.h"
#include "tq4_encode_wave.h"
#include "tq4_launch.h"
#include "tq4_tile.h"

namespace tq4 {

// ---------------------------------------------------------------- encoder

constexpr int kI8EncWaves = 4;
constexpr int64_t kI8EncMaxWorkgroups = 2048;
constexpr int kI8DropOffset = 0x40000000;  // a buffer offset past any record: the store is dropped
constexpr int kI8BufferFlags = 0x00020000;

struct Int8EncodeArgs {
    Int8EncodeParams p;
    FastDiv by_kv;    // n_kv
    FastDiv by_page;  // page_size
};

__device__ __forceinline__ float wave_max_abs(const float x[4]) {
    float m = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
    return wave_max_f32(m, static_cast<int>(threadIdx.x) & (kWave - 1));
}

// One code: clamp(rint(x / s), -127, 127) as a byte (s > 0), correctly rounded division.
__device__ __forceinline__ uint32_t int8_code(float x, float s) {
    const float q = fminf(fmaxf(__builtin_rintf(x / s), -127.0f), 127.0f);
    return static_cast<uint32_t>(static_cast<int32_t>(q)) & 0xffu;
}

// One vector held by a wavefront (lane l: dims 4 l .. 4 l + 3): returns the lane's four codes as
// one word (dim 4 l in the low byte) and sets the record's scale (fp16 bits).
__device__ __forceinline__ uint32_t int8_encode_lane(const float x[4], uint16_t &s16) {
    s16 = f32_to_f16_bits(wave_max_abs(x) / 127.0f);
    const float s = f16_bits_to_f32(s16);
    if (!(s > 0.0f)) return 0u;
    return int8_code(x[0], s) | (int8_code(x[1], s) << 8) | (int8_code(x[2], s) << 16) | (int8_code(x[3], s) << 24);
}

// Each wavefront encodes vectors wave0, wave0 + stride, ... ([half][token][kv head] order); lane l
// holds dims 4 l .. 4 l + 3 and stores their four codes as one word; lane 0 stores the scale.  The
// next vector is requested before the current one is encoded; stores go through buffer resources
// that cover the record exactly, or nothing for a slot outside the pool.
template <bool BF16>
__global__ __launch_bounds__(kI8EncWaves * kWave) void tq4_int8_encode_kernel(Int8EncodeArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave0 = static_cast<int>(blockIdx.x) * kI8EncWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int stride = static_cast<int>(gridDim.x) * kI8EncWaves;
    const int per_half = a.p.n_tokens * a.p.n_kv;
    const int first_half = a.p.src[0] != nullptr ? 0 : 1;
    const int total = per_half * ((a.p.src[0] != nullptr) + (a.p.src[1] != nullptr));
    if (wave0 >= total) return;
    // the two halves' pointers, read once (an index into the argument array would be a scalar
    // load and wait at every use)
    const char *const src0 = static_cast<const char *>(a.p.src[0]), *const src1 = static_cast<const char *>(a.p.src[1]);
    int8_t *const codes0 = a.p.codes[0], *const codes1 = a.p.codes[1];
    uint16_t *const scales0 = a.p.scales[0], *const scales1 = a.p.scales[1];
    constexpr size_t esize = BF16 ? 2 : 4;
    auto half_of = [&](int vec) { return first_half + static_cast<int>(vec >= per_half); };
    auto rem_of = [&](int vec) { return vec - (vec >= per_half ? per_half : 0); };
    auto load = [&](int vec, float x[4], int &slot) {
        const int rem = rem_of(vec);
        encode_load((half_of(vec) ? src1 : src0) + static_cast<int64_t>(rem) * kDim * esize, BF16, lane, x);
        slot = a.p.slots[fast_div(rem, a.by_kv)];
    };
    const int scale_off = lane == 0 ? 0 : kI8DropOffset;
    auto encode_store = [&](int vec, const float x[4], int slot, bool live) {
        const int half = half_of(vec);
        const int rv = rem_of(vec);
        const int head = rv - fast_div(rv, a.by_kv) * a.p.n_kv;
        const int s_u = __builtin_amdgcn_readfirstlane(slot);
        const bool valid = live && s_u >= 0 && s_u < a.p.num_slots;
        const int sl = valid ? s_u : 0;
        const int page = fast_div(sl, a.by_page);
        const int64_t rec = (static_cast<int64_t>(page) * a.p.n_kv + head) * a.p.page_size + (sl - page * a.p.page_size);
        uint16_t s16;
        const uint32_t word = int8_encode_lane(x, s16);
        const __amdgpu_buffer_rsrc_t cr =
            __builtin_amdgcn_make_buffer_rsrc((half ? codes1 : codes0) + rec * kDim, 0, valid ? kDim : 0, kI8BufferFlags);
        const __amdgpu_buffer_rsrc_t sr =
            __builtin_amdgcn_make_buffer_rsrc((half ? scales1 : scales0) + rec, 0, valid ? 2 : 0, kI8BufferFlags);
        __builtin_amdgcn_raw_buffer_store_b32(word, cr, 4 * lane, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b16(s16, sr, scale_off, 0, 0);
    };
    float x0[4], x1[4];
    int slot0, slot1;
    load(wave0, x0, slot0);
    for (int vec = wave0; vec < total; vec += 2 * stride) {
        const bool live1 = vec < total - stride;
        const int v1 = live1 ? vec + stride : vec;
        load(v1, x1, slot1);
        __builtin_amdgcn_sched_barrier(0);
        encode_store(vec, x0, slot0, true);
        const int v2 = vec < total - 2 * stride ? vec + 2 * stride : vec;
        load(v2, x0, slot0);
        __builtin_amdgcn_sched_barrier(0);
        encode_store(v1, x1, slot1, live1);
    }
}

hipError_t launch_int8_encode(const Int8EncodeParams &p, hipStream_t stream) {
    Int8EncodeArgs a;
    a.p = p;
    a.by_kv = make_fast_div(static_cast<uint32_t>(p.n_kv));
    a.by_page = make_fast_div(static_cast<uint32_t>(p.page_size));
    const int halves = (p.src[0] != nullptr) + (p.src[1] != nullptr);
    const int64_t vectors = static_cast<int64_t>(halves) * p.n_tokens * p.n_kv;
    if (vectors == 0) return hipSuccess;
    if (vectors > 0x7fffffff - 2 * kI8EncMaxWorkgroups * kI8EncWaves) return hipErrorInvalidValue;
    int64_t blocks = (vectors + kI8EncWaves - 1) / kI8EncWaves;
    if (blocks > kI8EncMaxWorkgroups) blocks = kI8EncMaxWorkgroups;
    const dim3 grid(static_cast<unsigned>(blocks)), block(kI8EncWaves * kWave);
    if (p.src_bf16)
        hipLaunchKernelGGL(tq4_int8_encode_kernel<true>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(tq4_int8_encode_kernel<false>, grid, block, 0, stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------- decode attention

constexpr float kI8RescaleSlack = 8.0f;  // log2 headroom before the running maximum is moved

struct Int8DecodeArgs {
    Int8DecodeParams p;
    int32_t group;
    int32_t n_queries;  // query tokens per request (1: decode)
    int32_t rows;       // n_queries * group
    int32_t n_splits;
    int32_t split_tiles;
    int32_t partial_floats;
    uint64_t parts_off;  // byte offset of the partials inside the workspace
};

// Two signed bytes -> packed fp16 (exact): byte SA of a in the low half, byte SB of b in the high
// half, each by one v_cvt_f16_i16 whose source operand selects the byte and sign-extends it.
#define TQ4_I8X2_ASM(SA, SB)                                                                       \
    asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_" #SA \
        "\n\tv_cvt_f16_i16_sdwa %0, sext(%2) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_" #SB \
        : "=&v"(r)                                                                                 \
        : "v"(a), "v"(b))
template <int SA, int SB>
__device__ __forceinline__ uint32_t i8x2_to_f16x2(uint32_t a, uint32_t b) {
    uint32_t r;
    if constexpr (SA == 0 && SB == 1) TQ4_I8X2_ASM(0, 1);
    else if constexpr (SA == 2 && SB == 3) TQ4_I8X2_ASM(2, 3);
    else if constexpr (SA == 0 && SB == 0) TQ4_I8X2_ASM(0, 0);
    else if constexpr (SA == 1 && SB == 1) TQ4_I8X2_ASM(1, 1);
    else if constexpr (SA == 2 && SB == 2) TQ4_I8X2_ASM(2, 2);
    else {
        static_assert(SA == 3 && SB == 3, "byte pair not instantiated");
        TQ4_I8X2_ASM(3, 3);
    }
    return r;
}
#undef TQ4_I8X2_ASM

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t mul_f16x2(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, a) * __builtin_bit_cast(half2v, b));
}

// Byte e of keys sigma(0..7) (dims 16 n + e), times their value scales: the A operand of V M-tile e.
template <int E>
__device__ __forceinline__ half8 v_operand(const u32x4 v[8], const u32x2 vn[2]) {
    constexpr int W = E >> 2, C = E & 3;
    u32x4 r;
    r.x = mul_f16x2(i8x2_to_f16x2<C, C>(v[0][W], v[1][W]), vn[0].x);
    r.y = mul_f16x2(i8x2_to_f16x2<C, C>(v[2][W], v[3][W]), vn[0].y);
    r.z = mul_f16x2(i8x2_to_f16x2<C, C>(v[4][W], v[5][W]), vn[1].x);
    r.w = mul_f16x2(i8x2_to_f16x2<C, C>(v[6][W], v[7][W]), vn[1].y);
    return __builtin_bit_cast(half8, r);
}

template <int E, int ITER_END>
struct VSteps {
    __device__ __forceinline__ static void run(const u32x4 v[8], const u32x2 vn[2], half8 pop, float4v oacc[16]) {
        oacc[E] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v_operand<E>(v, vn), pop, oacc[E], 0, 0, 0);
        VSteps<E + 1, ITER_END>::run(v, vn, pop, oacc);
    }
};
template <int ITER_END>
struct VSteps<ITER_END, ITER_END> {
    __device__ __forceinline__ static void run(const u32x4 *, const u32x2 *, half8, float4v *) {}
};

struct I8KRegs {
    u32x4 k[2][4];  // [M-tile][h]: bytes 64 h + 16 gq .. +15 of key 16 mt + n
    u32x2 kn[2];    // K scales of keys sigma(0..3) and sigma(4..7)
};
struct I8VRegs {
    u32x4 v[8];     // bytes 16 n .. 16 n + 15 of key sigma(j)
    u32x2 vn[2];    // V scales of the same keys
};

struct I8LaneOffsets {
    uint32_t k;    // key n, byte 16 gq
    uint32_t v;    // key 4 gq, byte 16 n
    uint32_t nrm;  // scale of key 4 gq
};

__device__ __forceinline__ I8LaneOffsets i8_lane_offsets(int lane) {
    const uint32_t n = lane & 15, gq = lane >> 4;
    return {n * 256u + gq * 16u, gq * 1024u + n * 16u, gq * 8u};
}

__device__ __forceinline__ void i8_load_k(const Int8DecodeParams &p, int64_t rec0, const I8LaneOffsets &o, I8KRegs &t) {
    const char *cb = reinterpret_cast<const char *>(p.k_codes) + rec0 * kDim;
    const char *sb = reinterpret_cast<const char *>(p.k_scales) + rec0 * 2;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int h = 0; h < 4; ++h) t.k[mt][h] = *reinterpret_cast<const u32x4 *>(cb + o.k + (4096u * mt + 64u * h));
#pragma unroll
    for (int h = 0; h < 2; ++h) t.kn[h] = *reinterpret_cast<const u32x2 *>(sb + o.nrm + 32u * h);
}

__device__ __forceinline__ void i8_load_v(const Int8DecodeParams &p, int64_t rec0, const I8LaneOffsets &o, I8VRegs &t) {
    const char *cb = reinterpret_cast<const char *>(p.v_codes) + rec0 * kDim;
    const char *sb = reinterpret_cast<const char *>(p.v_scales) + rec0 * 2;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t koff = (j < 4) ? 256u * j : 4096u + 256u * (j - 4);
        t.v[j] = *reinterpret_cast<const u32x4 *>(cb + o.v + koff);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) t.vn[h] = *reinterpret_cast<const u32x2 *>(sb + o.nrm + 32u * h);
}

// The query rows of one (request, KV head) -- row r = i G + h for query token i of n_queries and
// head h of the group -- fill NB blocks of 16 MFMA columns; wavefront w = blk NS + slot owns
// column block blk and every NS-th tile from its slot, so the NB wavefronts of a slot read the
// same tiles (the caches serve all but the first).  Decode is NB = 1, NS = 8; the multi-query
// verifier uses NB = 2, NS = 4 and NB = 3, NS = 2.  Column r of query token i sees positions
// 0 .. L - KQ + i.
template <int NB, int NS>
__global__ __launch_bounds__(NB * NS * kWave) void tq4_int8_split_kernel(Int8DecodeArgs a) {
    constexpr int NW = NB * NS;
    constexpr int NT = NW * kWave;
    constexpr int NCOL = 16 * NB;
    constexpr int kTreeBlocks = 8 / NS;  // blocks merged per round: [blocks][NS / 2][16][64] rows
    __shared__ __align__(16) half8 qop_sh[NB][8][kWave];  // query operand per block, K-step, lane
    __shared__ __align__(16) float4v tree[kTreeBlocks][NS / 2][16][kWave];
    __shared__ float stat_m[NW][16];
    __shared__ float stat_l[NW][16];
    __shared__ float row_f[NCOL];
    __shared__ float resL[NCOL];
    __shared__ float resM[NCOL];
    __shared__ int32_t progress[NW];

    const Int8DecodeParams &p = a.p;
    const int G = a.group;
    const int KQ = a.n_queries;
    const int ROWS = a.rows;  // KQ * G <= NCOL
    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, gq = lane >> 4;

    const int L_req = p.seq_lens[b];
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int slot = wave_u % NS, blk = wave_u / NS;
    const int split_keys = a.split_tiles * kTile;
    const int key_begin = s * split_keys;
    const int32_t *pt_row = p.page_table + static_cast<int64_t>(b) * p.table_stride;
    const bool append_mode = p.k_new != nullptr || p.v_new != nullptr;
    // element offset of query row r (token i, head h) in q and out: [request][token][q head][256]
    auto row_off = [&](int r) -> int64_t {
        const int i = r / G, h = r - i * G;
        return ((static_cast<int64_t>(b) * KQ + i) * p.n_q + static_cast<int64_t>(g) * G + h) * kDim;
    };

    int pid_vec = 0;
    auto fetch_pids = [&](int chunk) {
        const int tile = slot + (chunk * kWave + lane) * NS;
        pid_vec = pt_row[min((key_begin + tile * kTile) / p.page_size, p.table_stride - 1)];
    };
    auto pid_of = [&](int j) -> int { return __builtin_amdgcn_readlane(pid_vec, j & (kWave - 1)); };

    const I8LaneOffsets lofs = i8_lane_offsets(lane);
    const I8LaneOffsets dead_ofs{0u, 0u, 0u};
    auto rec_of = [&](int t, int inext, bool &valid_d) -> int64_t {
        const int key0 = __builtin_amdgcn_readfirstlane(key_begin + t * kTile);
        return tile_rec0(p, g, key0, pid_of(inext), valid_d);
    };
    I8KRegs kr;
    I8VRegs vr;
    bool valid_t = false;
    auto issue = [&](int t, int inext, bool live) {
        const int64_t rec = rec_of(t, inext, valid_t);
        const int64_t r = live ? rec : 0;
        const I8LaneOffsets o = live ? lofs : dead_ofs;
        __builtin_amdgcn_sched_barrier(0);
        i8_load_k(p, r, o, kr);
        __builtin_amdgcn_sched_barrier(0);
        i8_load_v(p, r, o, vr);
        __builtin_amdgcn_sched_barrier(0);
    };

    // query row, page IDs and the first tile are requested before the length is known
    const u32x2 q_raw0 = *reinterpret_cast<const u32x2 *>(p.q + row_off(min(wave_u, ROWS - 1)) + 4 * lane);
    fetch_pids(0);
    issue(slot, 0, true);

    const int L = L_req < 0 ? 0 : (L_req > p.max_seq_len ? p.max_seq_len : L_req);
    const int n_active = (L + split_keys - 1) / split_keys;
    if (s >= n_active) {
        if (L == 0 && s == 0)
            for (int i = tid; i < ROWS * kDim; i += NT) p.out[row_off(i / kDim) + (i % kDim)] = 0;
        return;
    }
    const int key_end = min(key_begin + split_keys, L);
    const int n_tiles = (key_end - key_begin + kTile - 1) / kTile;
    const int n_mine = slot < n_tiles ? (n_tiles - slot + NS - 1) / NS : 0;

    // ---- query operand: column r (a query row) is written by wavefront r % NW; a power-of-two
    // scale puts max |q| in [2^13, 2^14) for the fp16 operand; padding columns are zeroed
    if (tid < NW) progress[tid] = 0;
    auto put_row = [&](int r, u32x2 raw) {
        const float y[4] = {__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xffff0000u),
                            __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xffff0000u)};
        const int e = q_exponent(wave_max_abs(y));
        const float qs = ldexpf(1.0f, e);
        if (lane == 0) row_f[r] = p.scale * 1.4426950408889634f * ldexpf(1.0f, -e);
        // dims 4 l .. 4 l + 3: K-step 2 (l / 16) + (l / 2) % 2, lane group (l / 4) % 4, bytes 8 (l % 2)
        const int ks = 2 * (lane >> 4) + ((lane >> 1) & 1);
        const int dst_lane = 16 * ((lane >> 2) & 3) + (r & 15);
        u32x2 hv;
        hv.x = pack_f16x2(y[0] * qs, y[1] * qs);
        hv.y = pack_f16x2(y[2] * qs, y[3] * qs);
        *reinterpret_cast<u32x2 *>(reinterpret_cast<char *>(&qop_sh[r >> 4][ks][dst_lane]) + 8 * (lane & 1)) = hv;
    };
    auto zero_column = [&](int r) {
        if (lane < 32)
            reinterpret_cast<u32x4 *>(&qop_sh[r >> 4][lane & 7][16 * (lane >> 3) + (r & 15)])[0] = u32x4{0u, 0u, 0u, 0u};
    };
    if (wave_u < ROWS)
        put_row(wave_u, q_raw0);
    else
        zero_column(wave_u);
    for (int r = wave_u + NW; r < NCOL; r += NW) {
        if (r < ROWS)
            put_row(r, *reinterpret_cast<const u32x2 *>(p.q + row_off(r) + 4 * lane));
        else
            zero_column(r);
    }
    __syncthreads();

    // ---- append (decode only): the wavefront that owns the request's last tile is the only one
    // that reads it, so it writes the new token's K and V records (position seq_len - 1) here,
    // with the encoder's arithmetic, before its loop; if the first tile it requested above is that
    // last tile, it requests the tile again once the stores are complete.
    if constexpr (NB == 1) {
        if (append_mode && s == n_active - 1 && n_tiles > 0 && slot == (n_tiles - 1) % NS) {
            const int slot_new = p.new_slots[b];
            if (slot_new >= 0 && slot_new < p.num_pages * p.page_size) {
                const int page = slot_new / p.page_size;
                const int64_t rec =
                    (static_cast<int64_t>(page) * p.n_kv + g) * p.page_size + (slot_new - page * p.page_size);
                const size_t off = (static_cast<size_t>(b) * p.n_kv + g) * kDim * (p.new_bf16 ? 2 : 4);
                float xk[4], xv[4];
                if (p.k_new != nullptr) encode_load(static_cast<const char *>(p.k_new) + off, p.new_bf16 != 0, lane, xk);
                if (p.v_new != nullptr) encode_load(static_cast<const char *>(p.v_new) + off, p.new_bf16 != 0, lane, xv);
                auto put = [&](const float x[4], const int8_t *codes, const uint16_t *scales) {
                    uint16_t s16;
                    const uint32_t word = int8_encode_lane(x, s16);
                    reinterpret_cast<uint32_t *>(const_cast<int8_t *>(codes) + rec * kDim)[lane] = word;
                    if (lane == 0) const_cast<uint16_t *>(scales)[rec] = s16;
                };
                if (p.k_new != nullptr) put(xk, p.k_codes, p.k_scales);
                if (p.v_new != nullptr) put(xv, p.v_codes, p.v_scales);
            }
            // vmcnt(0): the record stores (and the first tile) have completed before the
            // wavefront loads the last tile (vmcnt bits [3:0] and [15:14] zero, expcnt and
            // lgkmcnt left at max)
            __builtin_amdgcn_s_waitcnt(0x0F70);
            if (n_mine == 1) issue(slot, 0, true);
        }
    }

    // this lane's column r = 16 blk + n: score factor and causal limit (padding columns see every
    // key and are never written)
    const int col = 16 * blk + n;
    const bool live_col = col < ROWS;
    const float fcol = live_col ? row_f[col] : 1.f;
    const int lim_col = live_col ? L - KQ + col / G + 1 : L;
    const half8 *qop = &qop_sh[blk][0][lane];

    float4v oacc[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) oacc[t] = float4v{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    // Issue priority of the pair of wavefronts on one SIMD (w and w ^ 4), as in the TQ4 kernel:
    // the younger takes the higher priority while not ahead of its partner, the older only while
    // behind.  Tile assignment is static, so results do not depend on timing.
    constexpr bool kPaired = NW == 8;
    const int partner = wave_u ^ (NW / 2);
    const bool younger = wave_u >= NW / 2;
    auto step = [&](int t, int inext, bool live, int done) {
        int other = 0;
        if constexpr (kPaired) {
            if (lane == 0) progress[wave_u] = done;
            other = __builtin_amdgcn_readfirstlane(progress[partner]);
        }
        const int key0 = key_begin + t * kTile;
        const bool valid = valid_t;
        float4v sacc[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            sacc[mt] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const u32x4 kw = kr.k[mt][ks >> 1];
                const uint32_t w0 = (ks & 1) ? kw.z : kw.x;
                const uint32_t w1 = (ks & 1) ? kw.w : kw.y;
                u32x4 c;
                c.x = i8x2_to_f16x2<0, 1>(w0, w0);
                c.y = i8x2_to_f16x2<2, 3>(w0, w0);
                c.z = i8x2_to_f16x2<0, 1>(w1, w1);
                c.w = i8x2_to_f16x2<2, 3>(w1, w1);
                sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, c), qop[ks * kWave], sacc[mt], 0, 0, 0);
            }
        }
        float ksc[8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            ksc[4 * h + 0] = f16lo(kr.kn[h].x);
            ksc[4 * h + 1] = f16hi(kr.kn[h].x);
            ksc[4 * h + 2] = f16lo(kr.kn[h].y);
            ksc[4 * h + 3] = f16hi(kr.kn[h].y);
        }
        float xs[8];
        const int lim = valid ? (min(key_end, lim_col) - key0) : 0;  // keys at offset >= lim are masked
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int r = 0; r < 4; ++r) xs[4 * h + r] = sacc[h][r] * ksc[4 * h + r];
        const int64_t rec = rec_of(t + NS, inext, valid_t);
        const int64_t rec_pf = live ? rec : 0;
        const I8LaneOffsets ofs_pf = live ? lofs : dead_ofs;
        __builtin_amdgcn_sched_barrier(0);
        i8_load_k(p, rec_pf, ofs_pf, kr);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kPaired) {
            if (younger ? (done <= other) : (done < other))
                __builtin_amdgcn_s_setprio(1);
            else
                if constexpr (kPaired) __builtin_amdgcn_s_setprio(0);
        }
        // value scales of the tile's keys as fp16 pairs (keys sigma(2i), sigma(2i + 1))
        u32x2 vn[2] = {vr.vn[0], vr.vn[1]};
        // Masking, only in a tile that is not visible in full (in place, so the common path has no
        // copies).  A key outside this lane's column's limit gets score -inf (so P = 0).  A key past
        // the request's length (or on an invalid page) also gets value scale 0: its record may
        // hold any bits, and code * scale must be an exact 0.  The value operand is shared by every
        // column, so only that column-independent limit may touch it.
        if (!__all(lim >= kTile)) {
            const int lim_v = valid ? (key_end - key0) : 0;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k0 = 16 * h + 4 * gq;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (k0 + r >= lim) xs[4 * h + r] = -INFINITY;
                vn[h].x &= (k0 < lim_v ? 0xffffu : 0u) | (k0 + 1 < lim_v ? 0xffff0000u : 0u);
                vn[h].y &= (k0 + 2 < lim_v ? 0xffffu : 0u) | (k0 + 3 < lim_v ? 0xffff0000u : 0u);
            }
        }
        float mx = xs[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mx = fmaxf(mx, xs[j]);
        float lo, hi;
        lane_pair<16>(mx, lo, hi);
        mx = fmaxf(lo, hi);
        lane_pair<32>(mx, lo, hi);
        mx = fmaxf(lo, hi) * fcol;
        if (__any(mx > m_run + kI8RescaleSlack)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = (m_new > m_run) ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
            l_run *= alpha;
#pragma unroll
            for (int tt = 0; tt < 16; ++tt) oacc[tt] *= alpha;
            m_run = m_new;
        }
        const float neg_m = -fmaxf(m_run, -FLT_MAX);
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            pv[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(xs[j], fcol, neg_m));
            l_run += pv[j];
        }
        u32x4 pr;
        pr.x = pack_f16x2(pv[0], pv[1]);
        pr.y = pack_f16x2(pv[2], pv[3]);
        pr.z = pack_f16x2(pv[4], pv[5]);
        pr.w = pack_f16x2(pv[6], pv[7]);
        VSteps<0, 16>::run(vr.v, vn, __builtin_bit_cast(half8, pr), oacc);
        __builtin_amdgcn_sched_barrier(0);
        i8_load_v(p, rec_pf, ofs_pf, vr);
        __builtin_amdgcn_sched_barrier(0);
    };

    for (int c0 = 0; c0 < n_mine; c0 += kWave) {
        const int cn = min(kWave, n_mine - c0);
        const int tc = slot + c0 * NS;
        if (c0 > 0) {
            fetch_pids(c0 / kWave);
            issue(tc, 0, true);
        }
        for (int i = 0; i < cn; ++i) step(tc + i * NS, i + 1, i + 1 < cn, c0 + i);
    }
    if constexpr (kPaired) __builtin_amdgcn_s_setprio(0);

    // ---- merge the wavefronts of each block: rescale to the block maximum, then a fixed-order
    // tree in LDS, kTreeBlocks blocks at a time (only query-row lanes take part)
    float l_tot = l_run + lane_xor<16>(l_run, lane);
    l_tot = l_tot + lane_xor<32>(l_tot, lane);
    if (gq == 0) {
        stat_m[wave_u][n] = m_run;
        stat_l[wave_u][n] = l_tot;
    }
    __syncthreads();
    {
        float M = -INFINITY;
#pragma unroll
        for (int j = 0; j < NS; ++j) M = fmaxf(M, stat_m[blk * NS + j][n]);
        const float f = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
#pragma unroll
        for (int tt = 0; tt < 16; ++tt) oacc[tt] *= f;
    }
    if (tid < NCOL) {
        const int cb = tid >> 4, cn = tid & 15;
        float M = -INFINITY;
        for (int j = 0; j < NS; ++j) M = fmaxf(M, stat_m[cb * NS + j][cn]);
        float Ls = 0.f;
        for (int j = 0; j < NS; ++j) {
            const float mj = stat_m[cb * NS + j][cn];
            Ls += (mj == -INFINITY) ? 0.f : stat_l[cb * NS + j][cn] * __builtin_amdgcn_exp2f(mj - M);
        }
        resM[tid] = M;
        resL[tid] = Ls;
    }
#pragma unroll
    for (int b0 = 0; b0 < NB; b0 += kTreeBlocks) {
        const bool mine = blk >= b0 && blk < b0 + kTreeBlocks && live_col;
#pragma unroll
        for (int half = NS / 2; half >= 1; half >>= 1) {
            if (mine && slot >= half && slot < 2 * half) {
#pragma unroll
                for (int tt = 0; tt < 16; ++tt) tree[blk - b0][slot - half][tt][lane] = oacc[tt];
            }
            __syncthreads();
            if (mine && slot < half) {
#pragma unroll
                for (int tt = 0; tt < 16; ++tt) oacc[tt] += tree[blk - b0][slot][tt][lane];
            }
            __syncthreads();
        }
    }
    if (slot != 0 || !live_col) return;

    // lane (gq, n), register r of M-tile e: dim 16 (4 gq + r) + e of column col
    if (n_active > 1) {
        const size_t bg = static_cast<size_t>(b) * p.n_kv + g;
        float *dst = reinterpret_cast<float *>(static_cast<char *>(p.workspace) + a.parts_off) +
                     (bg * a.n_splits + s) * static_cast<size_t>(a.partial_floats);
        if (gq == 0) {
            dst[col] = resM[col];
            dst[kSplitStatPad + col] = resL[col];
        }
        float *row = dst + 2 * kSplitStatPad + col * kDim;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float *d = row + 16 * (4 * gq + r);
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4)
                *reinterpret_cast<float4 *>(d + 4 * e4) =
                    make_float4(oacc[4 * e4][r], oacc[4 * e4 + 1][r], oacc[4 * e4 + 2][r], oacc[4 * e4 + 3][r]);
        }
        return;
    }
    // single split: o = O / L straight to the output
    const float Lh = resL[col];
    const float f = Lh > 0.f ? 1.0f / Lh : 0.f;
    uint16_t *orow = p.out + row_off(col);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        u32x4 o0, o1;
        o0.x = pack_bf16x2(oacc[0][r] * f, oacc[1][r] * f);
        o0.y = pack_bf16x2(oacc[2][r] * f, oacc[3][r] * f);
        o0.z = pack_bf16x2(oacc[4][r] * f, oacc[5][r] * f);
        o0.w = pack_bf16x2(oacc[6][r] * f, oacc[7][r] * f);
        o1.x = pack_bf16x2(oacc[8][r] * f, oacc[9][r] * f);
        o1.y = pack_bf16x2(oacc[10][r] * f, oacc[11][r] * f);
        o1.z = pack_bf16x2(oacc[12][r] * f, oacc[13][r] * f);
        o1.w = pack_bf16x2(oacc[14][r] * f, oacc[15][r] * f);
        u32x4 *d = reinterpret_cast<u32x4 *>(orow + 16 * (4 * gq + r));
        d[0] = o0;
        d[1] = o1;
    }
}

hipError_t launch_int8_decode(const Int8DecodeParams &p, const DecodePlan &plan, hipStream_t stream) {
    Int8DecodeArgs a;
    a.p = p;
    a.group = plan.group;
    a.n_queries = plan.n_queries;
    a.rows = plan.rows;
    a.n_splits = plan.n_splits;
    a.split_tiles = plan.split_tiles;
    a.partial_floats = static_cast<int32_t>(plan.partial_floats);
    a.parts_off = plan.counters_bytes;
    const dim3 grid(plan.n_splits, p.n_kv, p.batch);
    switch (plan.col_blocks) {
        case 1:
            hipLaunchKernelGGL((tq4_int8_split_kernel<1, 8>), grid, dim3(8 * kWave), 0, stream, a);
            break;
        case 2:
            hipLaunchKernelGGL((tq4_int8_split_kernel<2, 4>), grid, dim3(8 * kWave), 0, stream, a);
            break;
        case 3:  // 12 wavefronts would leave 168 registers each and spill; 6 fit without
            hipLaunchKernelGGL((tq4_int8_split_kernel<3, 2>), grid, dim3(6 * kWave), 0, stream, a);
            break;
        default:
            return hipErrorInvalidValue;
    }
    if (plan.n_splits > 1) {
        CombineArgs c;
        c.parts = reinterpret_cast<const float *>(static_cast<const char *>(p.workspace) + plan.counters_bytes);
        c.seq_lens = p.seq_lens;
        c.out = p.out;
        c.max_seq_len = p.max_seq_len;
        c.split_tiles = plan.split_tiles;
        c.n_splits = plan.n_splits;
        c.partial_floats = static_cast<int32_t>(plan.partial_floats);
        c.rows = plan.rows;
        c.group = plan.group;
        c.n_queries = plan.n_queries;
        c.n_q = p.n_q;
        c.n_kv = p.n_kv;
        c.batch = p.batch;
        return launch_split_combine(c, false, stream);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------- chunked prefill
//
// Causal attention of a chunk of query tokens over INT8 pages: the TQ4 prefill's decomposition
// (grid (key split, 128-row block, KV head), 8 wavefronts of 16 rows, a double-buffered LDS image
// of each 32-key tile's fp16 MFMA operands that the wavefronts fill together, one barrier per
// tile) with the byte conversion in place of the table, the natural domain (no rotation), value
// operands pre-scaled (code * scale, one fp16 rounding) and key scales in the scores.  Three
// kernels per call: query rows to fp16 operands with a power-of-two scale; attend; the shared
// prefill combine without the inverse rotation.

constexpr int kI8PfWaves = 8;
constexpr int kI8PfRowsPerWg = kI8PfWaves * 16;  // must equal the plan's rows per block
constexpr int kI8PfAhead = 4;
constexpr float kI8PfRescaleSlack = 8.0f;

struct Int8PrefillArgs {
    Int8PrefillParams p;
    int32_t group;
    int32_t rows;        // chunk_len * group (per KV head)
    int32_t n_splits;
    int32_t split_tiles;
    uint64_t qop_off;    // fp16 [chunk_len * n_q][256], natural dim order
    uint64_t frow_off;   // float [chunk_len * n_q]
    uint64_t parts_off;  // float [n_kv][rows][n_splits][kPfPartial]
};

__global__ __launch_bounds__(256) void tq4_int8_prefill_query_kernel(Int8PrefillArgs a) {
    const Int8PrefillParams &p = a.p;
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);  // t * n_q + qh
    if (row >= static_cast<int64_t>(p.chunk_len) * p.n_q) return;
    const u32x2 raw = *reinterpret_cast<const u32x2 *>(p.q + row * kDim + 4 * lane);
    const float y[4] = {__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xffff0000u),
                        __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xffff0000u)};
    const int e = q_exponent(wave_max_abs(y));
    const float qs = ldexpf(1.0f, e);
    char *ws = static_cast<char *>(p.workspace);
    u32x2 hv;
    hv.x = pack_f16x2(y[0] * qs, y[1] * qs);
    hv.y = pack_f16x2(y[2] * qs, y[3] * qs);
    *reinterpret_cast<u32x2 *>(ws + a.qop_off + row * (kDim * 2) + 8 * lane) = hv;
    if (lane == 0) reinterpret_cast<float *>(ws + a.frow_off)[row] = p.scale * 1.4426950408889634f * ldexpf(1.0f, -e);
}

// Tile image: entry mt * 8 + ks is the K operand of M-tile mt, K-step ks; entry 16 + e the
// (pre-scaled) V operand of M-tile e; ksc the 32 key scales.
struct I8PfTileImage {
    half8 op[32][kWave];
    float ksc[32];
};

__global__ __launch_bounds__(kI8PfWaves * kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
void tq4_int8_prefill_kernel(Int8PrefillArgs a) {
    constexpr int NW = kI8PfWaves;
    __shared__ __align__(16) I8PfTileImage img[2];
    const Int8PrefillParams &p = a.p;
    const int G = a.group;
    const int s = blockIdx.x, rb = blockIdx.y, g = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, gq = lane >> 4;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    char *ws = static_cast<char *>(p.workspace);

    const int row0 = rb * kI8PfRowsPerWg + wave_u * 16;  // this wave's rows: row0 + n
    const int wg_last_row = min(rb * kI8PfRowsPerWg + kI8PfRowsPerWg, a.rows) - 1;
    const int wg_kmax = p.prior_len + wg_last_row / G + 1;  // keys any row of the workgroup sees
    const int total_keys = p.prior_len + p.chunk_len;
    const int split_keys = a.split_tiles * kTile;
    const int key_begin = s * split_keys;
    const int key_end = min(key_begin + split_keys, wg_kmax);
    const int n_tiles = key_end > key_begin ? (key_end - key_begin + kTile - 1) / kTile : 0;

    // ---- this wave's share of each tile: K operands e0, e0 + 1 and V operands 16 + e0, 16 + e0 + 1
    // (e0 = 2 wave).  The K pair is bytes 64 (ks / 2) + 16 gq .. + 15 of key 16 mt + n (one 16-byte
    // load; mt = e0 / 8, ks = e0 % 8).  The V pair takes bytes e0 and e0 + 1 of dims 16 n .. of keys
    // sigma(0..7): one word per key (bytes 4 (e0 / 4) ..), shifted so the pair sits in bytes 0, 1.
    const int e0 = 2 * wave_u;
    const int mt_w = e0 >> 3, ks_w = e0 & 7;
    const uint32_t k_lane_off = (16u * mt_w + n) * 256u + 64u * (ks_w >> 1) + 16u * gq;
    const uint32_t v_lane_off = gq * 1024u + n * 16u + 4u * (e0 >> 2);
    const uint32_t v_shift = 8u * (e0 & 3);  // 0 or 16
    const int32_t *pt = p.page_table;
    const int pt_last = (total_keys - 1) / p.page_size;
    struct Staging {
        u32x4 k;
        uint32_t v[8];
        u32x2 vs[2];
        uint32_t ks;
        int key0;
        bool valid;
    };
    auto load_share = [&](Staging &st, int t) {
        const int key0 = key_begin + t * kTile;  // t is clamped by the caller to a tile of this split
        const int pid = pt[min(key0 / p.page_size, pt_last)];
        const int64_t rec = tile_rec0(p, g, key0, pid, st.valid);
        st.key0 = key0;
        const char *kb = reinterpret_cast<const char *>(p.k_codes) + rec * kDim;
        const char *vb = reinterpret_cast<const char *>(p.v_codes) + rec * kDim;
        st.k = *reinterpret_cast<const u32x4 *>(kb + k_lane_off);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t koff = (j < 4) ? 256u * j : 4096u + 256u * (j - 4);
            st.v[j] = *reinterpret_cast<const uint32_t *>(vb + v_lane_off + koff);
        }
        const char *vsb = reinterpret_cast<const char *>(p.v_scales) + rec * 2 + gq * 8u;
#pragma unroll
        for (int h = 0; h < 2; ++h) st.vs[h] = *reinterpret_cast<const u32x2 *>(vsb + 32u * h);
        st.ks = p.k_scales[rec + (lane & 31)];
    };
    auto decode_share = [&](const Staging &st, I8PfTileImage &im) {
        // value scales of keys past the cached length (or on an invalid page) become 0: their
        // records may hold any bits, and the value operand is shared by every row
        const int lim_v = st.valid ? total_keys - st.key0 : 0;
        u32x2 vs[2] = {st.vs[0], st.vs[1]};
        if (!__all(lim_v >= kTile)) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k0 = 16 * h + 4 * gq;
                vs[h].x &= (k0 < lim_v ? 0xffffu : 0u) | (k0 + 1 < lim_v ? 0xffff0000u : 0u);
                vs[h].y &= (k0 + 2 < lim_v ? 0xffffu : 0u) | (k0 + 3 < lim_v ? 0xffff0000u : 0u);
            }
        }
        u32x4 k0v, k1v;
        k0v.x = i8x2_to_f16x2<0, 1>(st.k.x, st.k.x);
        k0v.y = i8x2_to_f16x2<2, 3>(st.k.x, st.k.x);
        k0v.z = i8x2_to_f16x2<0, 1>(st.k.y, st.k.y);
        k0v.w = i8x2_to_f16x2<2, 3>(st.k.y, st.k.y);
        k1v.x = i8x2_to_f16x2<0, 1>(st.k.z, st.k.z);
        k1v.y = i8x2_to_f16x2<2, 3>(st.k.z, st.k.z);
        k1v.z = i8x2_to_f16x2<0, 1>(st.k.w, st.k.w);
        k1v.w = i8x2_to_f16x2<2, 3>(st.k.w, st.k.w);
        uint32_t w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = st.v[j] >> v_shift;
        u32x4 v0, v1;
        v0.x = mul_f16x2(i8x2_to_f16x2<0, 0>(w[0], w[1]), vs[0].x);
        v0.y = mul_f16x2(i8x2_to_f16x2<0, 0>(w[2], w[3]), vs[0].y);
        v0.z = mul_f16x2(i8x2_to_f16x2<0, 0>(w[4], w[5]), vs[1].x);
        v0.w = mul_f16x2(i8x2_to_f16x2<0, 0>(w[6], w[7]), vs[1].y);
        v1.x = mul_f16x2(i8x2_to_f16x2<1, 1>(w[0], w[1]), vs[0].x);
        v1.y = mul_f16x2(i8x2_to_f16x2<1, 1>(w[2], w[3]), vs[0].y);
        v1.z = mul_f16x2(i8x2_to_f16x2<1, 1>(w[4], w[5]), vs[1].x);
        v1.w = mul_f16x2(i8x2_to_f16x2<1, 1>(w[6], w[7]), vs[1].y);
        im.op[e0][lane] = __builtin_bit_cast(half8, k0v);
        im.op[e0 + 1][lane] = __builtin_bit_cast(half8, k1v);
        im.op[16 + e0][lane] = __builtin_bit_cast(half8, v0);
        im.op[16 + e0 + 1][lane] = __builtin_bit_cast(half8, v1);
        if (lane < 32) im.ksc[lane] = f16_bits_to_f32(static_cast<uint16_t>(st.ks));  // every wave: same values
    };

    Staging sa, sb;
    load_share(sa, 0);

    // ---- row data: causal limit, score factor, query operand (rows past the chunk see no key and
    // are never written).  K-step ks takes dims 64 (ks / 2) + 16 gq + 8 (ks % 2) .. + 7.
    const int row = row0 + n;
    const bool live = row < a.rows;
    const int tq = live ? row / G : 0;
    const int qrow = tq * p.n_q + g * G + (live ? row - tq * G : 0);
    const int lim_row = live ? p.prior_len + tq + 1 : 0;
    const float fcol = live ? reinterpret_cast<const float *>(ws + a.frow_off)[qrow] : 1.f;
    half8 qop[8];
    {
        const char *qr = ws + a.qop_off + static_cast<int64_t>(qrow) * (kDim * 2);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            u32x4 v = *reinterpret_cast<const u32x4 *>(qr + 2 * (64 * (ks >> 1) + 16 * gq + 8 * (ks & 1)));
            if (!live) v = u32x4{0u, 0u, 0u, 0u};
            qop[ks] = __builtin_bit_cast(half8, v);
        }
    }
    const int t_last = max(n_tiles - 1, 0);
    decode_share(sa, img[0]);
    bool valid0 = sa.valid, valid1 = false;
    load_share(sb, min(1, t_last));
    load_share(sa, min(2, t_last));
    __syncthreads();

    float4v oacc[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) oacc[t] = float4v{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    auto compute = [&](const I8PfTileImage &im, int t, bool valid) {
        const int key0 = key_begin + t * kTile;
        float4v sacc[2] = {float4v{0.f, 0.f, 0.f, 0.f}, float4v{0.f, 0.f, 0.f, 0.f}};
        half8 opb[kI8PfAhead + 1];
#pragma unroll
        for (int e = 0; e < kI8PfAhead; ++e) opb[e] = im.op[e][lane];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            if (e + kI8PfAhead < 16) opb[(e + kI8PfAhead) % (kI8PfAhead + 1)] = im.op[e + kI8PfAhead][lane];
            sacc[e >> 3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(opb[e % (kI8PfAhead + 1)], qop[e & 7], sacc[e >> 3], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int e = 0; e < kI8PfAhead; ++e) opb[e] = im.op[16 + e][lane];
        // lane holds keys sigma(j): j < 4 -> 4 gq + j, else 16 + 4 gq + j - 4
        const float4 k0s = *reinterpret_cast<const float4 *>(&im.ksc[4 * gq]);
        const float4 k1s = *reinterpret_cast<const float4 *>(&im.ksc[16 + 4 * gq]);
        const float ksc[8] = {k0s.x, k0s.y, k0s.z, k0s.w, k1s.x, k1s.y, k1s.z, k1s.w};
        const int lim = valid ? min(key_end, lim_row) - key0 : 0;
        float xs[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) xs[q] = sacc[q >> 2][q & 3] * ksc[q];
        if (!__all(lim >= kTile)) {  // masked in place, so the common path has no copies
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int koff = (q < 4) ? (4 * gq + q) : (16 + 4 * gq + (q - 4));
                if (koff >= lim) xs[q] = -INFINITY;
            }
        }
        float mx = xs[0];
#pragma unroll
        for (int q = 1; q < 8; ++q) mx = fmaxf(mx, xs[q]);
        float lo, hi;
        lane_pair<16>(mx, lo, hi);
        mx = fmaxf(lo, hi);
        lane_pair<32>(mx, lo, hi);
        mx = fmaxf(lo, hi) * fcol;
        if (__any(mx > m_run + kI8PfRescaleSlack)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = (m_new > m_run) ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
            l_run *= alpha;
#pragma unroll
            for (int tt = 0; tt < 16; ++tt) {
                oacc[tt] *= alpha;
                __builtin_amdgcn_sched_barrier(0);
            }
            m_run = m_new;
        }
        const float neg_m = -fmaxf(m_run, -FLT_MAX);
        float pv[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            pv[q] = __builtin_amdgcn_exp2f(__builtin_fmaf(xs[q], fcol, neg_m));
            l_run += pv[q];
        }
        u32x4 pr;
        pr.x = pack_f16x2(pv[0], pv[1]);
        pr.y = pack_f16x2(pv[2], pv[3]);
        pr.z = pack_f16x2(pv[4], pv[5]);
        pr.w = pack_f16x2(pv[6], pv[7]);
        const half8 pop = __builtin_bit_cast(half8, pr);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            if (e + kI8PfAhead < 16) opb[(e + kI8PfAhead) % (kI8PfAhead + 1)] = im.op[16 + e + kI8PfAhead][lane];
            oacc[e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(opb[e % (kI8PfAhead + 1)], pop, oacc[e], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // the two wavefronts of a SIMD take each step's halves in opposite orders, as in the TQ4
    // prefill (the barrier only separates the two image buffers)
    const bool late = wave_u >= kI8PfWaves / 2;
    for (int t = 0; t < n_tiles; t += 2) {
        if (!late) {
            decode_share(sb, img[1]);
            valid1 = sb.valid;
            load_share(sb, min(t + 3, t_last));
        }
        compute(img[0], t, valid0);
        if (late) {
            decode_share(sb, img[1]);
            valid1 = sb.valid;
            load_share(sb, min(t + 3, t_last));
        }
        __syncthreads();
        if (!late) {
            decode_share(sa, img[0]);
            valid0 = sa.valid;
            load_share(sa, min(t + 4, t_last));
        }
        compute(img[1], t + 1, valid1 && t + 1 < n_tiles);
        if (late) {
            decode_share(sa, img[0]);
            valid0 = sa.valid;
            load_share(sa, min(t + 4, t_last));
        }
        __syncthreads();
    }

    // ---- partial: lane (gq, n) holds row n, dims 16 (4 gq + r) + e in oacc[e][r]
    float l_tot = l_run + lane_xor<16>(l_run, lane);
    l_tot = l_tot + lane_xor<32>(l_tot, lane);
    if (!live) return;
    float *dst = reinterpret_cast<float *>(ws + a.parts_off) +
                 ((static_cast<int64_t>(g) * a.rows + row) * a.n_splits + s) * kPfPartial;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float *d = dst + 16 * (4 * gq + r);
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4)
            *reinterpret_cast<float4 *>(d + 4 * e4) =
                make_float4(oacc[4 * e4][r], oacc[4 * e4 + 1][r], oacc[4 * e4 + 2][r], oacc[4 * e4 + 3][r]);
    }
    if (gq == 0) {
        dst[kDim] = m_run;
        dst[kDim + 1] = l_tot;
    }
}

hipError_t launch_int8_prefill(const Int8PrefillParams &p, const PrefillPlan &plan, hipStream_t stream) {
    if (plan.q_tokens_per_block != kI8PfRowsPerWg) return hipErrorInvalidValue;
    Int8PrefillArgs a;
    a.p = p;
    a.group = plan.group;
    a.rows = p.chunk_len * plan.group;
    a.n_splits = plan.n_splits;
    a.split_tiles = plan.split_tiles;
    const size_t qrows = static_cast<size_t>(p.chunk_len) * p.n_q;
    a.qop_off = 0;
    a.frow_off = ((qrows * kDim * 2 + 255) / 256) * 256;
    a.parts_off = plan.counters_bytes;
    const int64_t q_blocks = (static_cast<int64_t>(qrows) + 3) / 4;
    if (q_blocks > 0x7fffffff || plan.n_qblocks > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL(tq4_int8_prefill_query_kernel, dim3(static_cast<unsigned>(q_blocks)), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(tq4_int8_prefill_kernel, dim3(plan.n_splits, plan.n_qblocks, p.n_kv), dim3(kI8PfWaves * kWave), 0,
                       stream, a);
    PrefillCombineArgs c;
    c.parts = reinterpret_cast<const float *>(static_cast<const char *>(p.workspace) + a.parts_off);
    c.out = p.out;
    c.rows = a.rows;
    c.group = a.group;
    c.n_splits = a.n_splits;
    c.n_kv = p.n_kv;
    c.n_q = p.n_q;
    return launch_prefill_combine(c, false, stream);
}

}  // namespace tq4
