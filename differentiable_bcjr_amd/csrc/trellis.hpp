// trellis.hpp -- geometry of the bitshift trellis as laid out on gfx950, and the wave/block primitives the three
// kernels share.  GPU path only (the CPU oracle has its own code).
//
// Trellis (BCJR-QAT, arXiv 2605.10655; the pages fix neither L nor k, the bitshift rule is the reading taken):
// L-bit state, k = 2 bits shifted in per step at the low end.  With G = 2^(L-2) "groups":
//   * the 4 predecessors of s' are s' >> 2 | a << (L-2), a = 0..3: they depend only on u = s' >> 2, so the
//     forward message collapses to one value per group, R_t(u) = logsumexp_a alpha_{t-1}(u | a << (L-2)), and
//     alpha_t(s') = theta_t(s') + R_t(s' >> 2);
//   * the 4 successors of s are (s << 2 | b) & (2^L-1): they depend only on s & (G-1), so the backward message is
//     one value per group too, beta_t(s) = B_t(s & (G-1)).
// Work is handed out in "quads": quad j (0 <= j < Q = 2^(L-4)) owns the 16 states s = a << (L-2) | j << 2 | i,
// i, a in [0,4).  In the forward direction these are the 4 predecessor sets of the groups 4j..4j+3 (which read
// R_t(j + Q a)); in the backward direction they are the successor sets of the groups j + Q a (which read
// B_{t+1}(4j + i)).  The same 16 states serve both directions, so a thread keeps their codebook values in registers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bcjr {

// Log-domain "minus infinity": finite, so all-masked groups never produce inf - inf; 2^(x - max) underflows to 0.
constexpr float kNeg = -1.0e30f;

// Threads per sequence, quads per thread, sequences per block, for state bits L (k = 2).
template <int L_>
struct Geo {
    static constexpr int L = L_;
    static constexpr int S = 1 << L;          // states
    static constexpr int G = 1 << (L - 2);    // groups
    static constexpr int Q = 1 << (L - 4);    // quads
    static constexpr int QPT = L >= 14 ? (1 << (L - 14)) : 1;
    static constexpr int TPS = Q / QPT;       // threads per sequence (<= 1024)
    static constexpr int NT = TPS >= 64 ? TPS : 64;
    static constexpr int SPB = NT / TPS;      // sequences per block
    static constexpr int WPS = TPS >= 64 ? TPS / 64 : 1;  // waves per sequence
    static constexpr int SEG = TPS < 64 ? TPS : 64;       // lanes of one sequence inside one wave
    static_assert(L >= 4 && L <= 16, "4 <= L <= 16");
};

// The same numbers for a runtime L (host-side planning).
struct GeoRT {
    int G, Q, QPT, TPS, NT, SPB, WPS;
};
__host__ __device__ constexpr GeoRT geo_rt(int L) {
    const int G = 1 << (L - 2), Q = 1 << (L - 4);
    const int QPT = L >= 14 ? (1 << (L - 14)) : 1;
    const int TPS = Q / QPT;
    const int NT = TPS >= 64 ? TPS : 64;
    return GeoRT{G, Q, QPT, TPS, NT, NT / TPS, TPS >= 64 ? TPS / 64 : 1};
}

// Blocks per CU the launch plans for (bounds the grid, hence the workspace): one block fills a CU at L >= 15.  The
// host multiplies this by the device's CU count.
__host__ __device__ constexpr int blocks_per_cu(int L) { return L >= 15 ? 1 : (L == 14 ? 2 : 8); }

// ---------------------------------------------------------------------------------------------------------------
// fast math (hardware transcendental units; inputs here are always in range)

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }
// The per-step offsets that keep the expectation messages centred are rounded to multiples of 2^-6.  Any offset
// serves (the true message is the stored one plus the sum of the offsets applied), and on this grid every running
// sum of offsets, and every difference of two such sums, is exact in float32 while it stays below 2^18 in
// magnitude; E[F | s_t = s] - E[F] then carries only roundings at the size of the centred messages, not at the size
// of F itself.
__device__ __forceinline__ float grid_offset(float x) { return __builtin_rintf(x * 64.f) * 0.015625f; }
// Maxima over finite values use the IEEE-2019 maximum (v_maximum3_f32).  fmaxf must quiet signalling NaNs, so the
// compiler re-canonicalises every operand it cannot prove canonical (a DPP or LDS result, one that left an asm ordering
// point) with an extra half-rate v_max per use; the maximum has no such requirement, and the two agree on the finite
// values and sentinels used here.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float max4(float a, float b, float c, float d) { return vmax(vmax(a, b), vmax(c, d)); }
__device__ __forceinline__ float run_max(float acc, float x) { return vmax(acc, x); }

// Keeps the compiler from deferring the accumulation of these values past this point (which would keep every
// group's temporaries alive at once): an empty volatile asm that claims to read and rewrite them.
__device__ __forceinline__ void pin_order(float& a, float& b, float& c) { asm volatile("" : "+v"(a), "+v"(b), "+v"(c)); }
__device__ __forceinline__ void pin_order(float& a, float& b) { asm volatile("" : "+v"(a), "+v"(b)); }

// ---------------------------------------------------------------------------------------------------------------
// barriers that order LDS traffic only: global loads and stores stay in flight across them

__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------------------------------------------------------
// reductions over the SEG lanes of one sequence inside a wave (butterfly, result in every lane)

template <int SEG>
__device__ __forceinline__ float seg_max(float x) {
#pragma unroll
    for (int o = 1; o < SEG; o <<= 1) x = vmax(x, __shfl_xor(x, o));
    return x;
}

template <int SEG>
__device__ __forceinline__ float seg_sum(float x) {
#pragma unroll
    for (int o = 1; o < SEG; o <<= 1) x += __shfl_xor(x, o);
    return x;
}

// Lexicographic (value, index) minimum: smaller value, then smaller index.
__device__ __forceinline__ void argmin_merge(float& v, uint32_t& i, float v2, uint32_t i2) {
    bool take = (v2 < v) || (v2 == v && i2 < i);
    v = take ? v2 : v;
    i = take ? i2 : i;
}

template <int SEG>
__device__ __forceinline__ void seg_argmin(float& v, uint32_t& i) {
#pragma unroll
    for (int o = 1; o < SEG; o <<= 1) {
        float v2 = __shfl_xor(v, o);
        uint32_t i2 = (uint32_t)__shfl_xor((int)i, o);
        argmin_merge(v, i, v2, i2);
    }
}

// ---------------------------------------------------------------------------------------------------------------
// full-wave (64-lane) reductions with DPP row operations and 4 readlanes; the result is wave-uniform

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_max64(float x) {
    x = vmax(x, dpp<0xB1>(x));    // quad_perm [1,0,3,2]
    x = vmax(x, dpp<0x4E>(x));    // quad_perm [2,3,0,1]
    x = vmax(x, dpp<0x141>(x));   // row_half_mirror
    x = vmax(x, dpp<0x140>(x));   // row_mirror: every lane of a row holds the row max
    const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
    const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
    const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
    const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
    return max4(a, b, c, d);
}

__device__ __forceinline__ float wave_sum64(float x) {
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    x += dpp<0x140>(x);
    const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
    const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
    const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
    const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
    return (a + b) + (c + d);
}

// Segment reductions: DPP for whole waves, butterfly shuffles for sub-wave segments.
template <int SEG>
__device__ __forceinline__ float seg_max_fast(float x) {
    if constexpr (SEG == 64) return wave_max64(x);
    else return seg_max<SEG>(x);
}
template <int SEG>
__device__ __forceinline__ float seg_sum_fast(float x) {
    if constexpr (SEG == 64) return wave_sum64(x);
    else return seg_sum<SEG>(x);
}

// Combine the per-wave slots of one sequence (at most 16): each lane reads slot (lane & 15), lanes past the last
// slot hold the neutral value, and a DPP tree inside each 16-lane row leaves the result in every lane.  All four
// rows read the same slots, so the result is wave-uniform.  Max and first-max are exact, so they match a serial
// scan over the slots; a sum is added in tree order.
__device__ __forceinline__ float row16_max(float x) {
    x = vmax(x, dpp<0xB1>(x));
    x = vmax(x, dpp<0x4E>(x));
    x = vmax(x, dpp<0x141>(x));
    return vmax(x, dpp<0x140>(x));
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    return x + dpp<0x140>(x);
}
// (max of v over the row, q of the lowest lane of the row attaining it)
__device__ __forceinline__ void row16_argmax_payload(float& v, float& q) {
    const float m = row16_max(v);
    const uint64_t hit = __ballot(v == m) & 0xFFFFull;
    const int src = hit ? __builtin_ctzll(hit) : 0;
    q = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, q), src));
    v = m;
}

// (max of v, q of the lowest lane attaining it) over the SEG lanes of one sequence inside a wave.
template <int SEG>
__device__ __forceinline__ void seg_argmax_payload(float& v, float& q) {
    if constexpr (SEG == 64) {
        const float m = wave_max64(v);
        const uint64_t hit = __ballot(v == m);
        const int src = __builtin_ctzll(hit);
        q = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, q), src));
        v = m;
    } else {
        int lane = (int)(threadIdx.x & 63);
#pragma unroll
        for (int o = 1; o < SEG; o <<= 1) {
            const float v2 = __shfl_xor(v, o);
            const float q2 = __shfl_xor(q, o);
            const int l2 = __shfl_xor(lane, o);
            const bool take = (v2 > v) || (v2 == v && l2 < lane);
            v = take ? v2 : v;
            q = take ? q2 : q;
            lane = take ? l2 : lane;
        }
    }
}

// Wave-uniform value into a scalar register (only valid when every lane holds the same value).
__device__ __forceinline__ float uniform_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// ---------------------------------------------------------------------------------------------------------------
// raw buffer access: SGPR base + 32-bit VGPR offset + SGPR offset, so per-lane 64-bit addresses are never kept

using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // gfx9 raw buffer, 32-bit data format

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ float buf_ld(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ float4 buf_ld4(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ float2 buf_ld2(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
__device__ __forceinline__ void buf_st2(float2 v, rsrc_t r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned int, v), r,
                                          voff, soff, 0);
}
__device__ __forceinline__ void buf_st(float v, rsrc_t r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, voff, soff, 0);
}
// A store wider than 8 bytes reads its data VGPRs after issue, so a VALU write to them in the next cycle can reach
// memory instead of the stored value (seen here as the first dword of a 16-byte tape store changing from run to
// run while the store queue was full).  The compiler inserts the required wait state only for stores whose SGPR
// offset field is not a register, so the whole offset goes through the VGPR and the SGPR offset stays literal 0.
__device__ __forceinline__ void buf_st4(float4 v, rsrc_t r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v), r,
                                           voff + soff, 0, 0);
}

// The forward tapes are written once and read once, a full pass later: their accesses carry the non-temporal
// policy so the stream does not evict what is reused from L2 (the codebook).
constexpr int kStreamPolicy = 2;   // nt on gfx950
__device__ __forceinline__ float buf_ld_nt(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kStreamPolicy));
}
__device__ __forceinline__ float2 buf_ld2_nt(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kStreamPolicy));
}
// Same store form as buf_st4 (whole offset in the VGPR, so the compiler adds the wait state after it).
__device__ __forceinline__ void buf_st4_nt(float4 v, rsrc_t r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v), r,
                                           voff + soff, 0, kStreamPolicy);
}

// Tape rows of the forward messages.  Without checkpoints row t sits at t * row_bytes.  With checkpoint interval c,
// rows t = 0, c, 2c, .. (n / c + 1 of them) come first, then c - 1 rows for the steps inside one segment: row t at
// segment position t mod c - 1.  The forward pass stores the checkpoints and row n - 1 (which the sigma end reads);
// the backward pass recomputes each segment's other rows from its checkpoint.
struct TapeRows {
    int c, n;
    uint32_t row_bytes, seg_base;
    __device__ __forceinline__ uint32_t off(int t) const {
        if (c == 0) return (uint32_t)t * row_bytes;
        const int r = t % c;
        return r == 0 ? (uint32_t)(t / c) * row_bytes : seg_base + (uint32_t)(r - 1) * row_bytes;
    }
    __device__ __forceinline__ bool stored(int t) const { return c == 0 || t % c == 0 || t == n - 1; }
    __host__ __device__ static constexpr size_t rows(int c, int n) { return c == 0 ? (size_t)n + 1 : (size_t)(n / c + c); }
};

// Per-slot workspace layout (bytes), shared by the host planner and the kernels.
__host__ __device__ constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace bcjr
