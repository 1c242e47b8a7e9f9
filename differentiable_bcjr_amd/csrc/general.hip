// general.hip -- soft codeword, exact gradient and Viterbi hard code for a general bitshift trellis on gfx950:
// k bits shifted in per step (2^k predecessors and 2^k successors per state), V weights emitted per step.
//
// The method is that of the k = 2 kernels (BCJR-QAT, arXiv 2605.10655: gist.science Technical Summary, "Core
// Mechanism" and "Key Technical Innovations"; the abstract for the T -> 0 limit).  The pages fix neither k nor V.
// Here a state emits a V-vector c(s) (codebook [2^L][V]), step t consumes the weights w[t V .. t V + V - 1], and the
// log weight of a state is -|w_t - c(s)|^2 / T.
//
// Grouped messages.  All states with the same u = s >> k share their 2^k predecessors u | a << (L-k), so the forward
// pass carries one value per group, R_t(u) = logsumexp_a alpha_{t-1}(u | a << (L-k)).  All states with the same
// s & (G-1) share their successors, so the backward pass carries B_t(s & (G-1)).  That is G = 2^(L-k) values per step
// in each direction.
//
// Blocks.  With P = 2^k and J = 2^(L-2k), block j (0 <= j < J) holds the P^2 states s(j, a, i) = a << (L-k) | j << k | i
// for a, i < P.  These are the predecessor sets of the forward groups u = j P + i, which read R_t(j + J a).  They are
// also the successor sets of the backward groups v = j + J a, which read B_{t+1}(j P + i).  So a thread that owns the
// states of a block serves both directions from the same codebook values.
//
// A thread owns SPT = 64 states (SPT = 2^L below L = 6):
//   * k <= 3: 64 / P^2 whole blocks;
//   * k = 4:  4 forward groups of one block, and the 4 lanes of a quad share the block's backward groups, combining
//             them with DPP.
// The 2^k-way log-sum-exps run over tiles of at most 4 x 4 states.  A tile's terms are exponentiated against the tile's
// own maximum, and tiles merge with one exponential, so registers stay bounded at every k.
//
// Codebook: in VGPRs when a thread's SPT V values fit in 64 registers, else read through L1/L2 at each use; a tile row
// is contiguous, 4 V floats.
//
// LDS holds the messages: G floats per buffer, double-buffered when two buffers fit.  Otherwise one buffer is used,
// and each step reads its inputs into registers and passes a barrier before it writes its outputs.  The gradient
// always keeps R and its expectation message Q in one buffer each.
//
// L is a run-time argument: one sequence per workgroup of 2^L / SPT threads, persistent over the batch.  k, V and SPT
// are compile-time.  The forward tapes, normalisers and per-wave partial sums use the workspace layout of the k = 2
// kernels.
#include <type_traits>

#include "kernel_args.hpp"
#include "trellis.hpp"

#ifndef GEN_NO_SCHED
#define GEN_SCHED_BARRIER() __builtin_amdgcn_sched_barrier(0)
#else
#define GEN_SCHED_BARRIER() ((void)0)
#endif

namespace bcjr {

namespace {

template <int K_, int V_, int SPT_>
struct GG {
    static constexpr int K = K_, V = V_, SPT = SPT_;
    static constexpr int P = 1 << K;
    static constexpr int P2 = P * P;
    static constexpr int C = P2 > SPT ? P2 / SPT : 1;      // threads sharing one block
    static constexpr int I = P / C;                         // forward groups of a block per thread
    static constexpr int BPT = P2 > SPT ? 1 : SPT / P2;     // blocks per thread
    static constexpr int TA = P < 4 ? P : 4;                // predecessor rows per tile
    static constexpr int TI = I < 4 ? I : 4;                // groups per tile
    static constexpr int NA = P / TA, NI = I / TI;
    static constexpr int ROW = TI * V;                      // codebook floats of one tile row
    static_assert(C == 1 || C == 4, "a block is shared by at most the 4 lanes of a quad");
    static_assert(C == 1 || NI == 1, "a shared block gives each lane one tile of groups");
    static_assert(V >= 1 && V <= 2, "V = 1 or 2");
};

// N floats from a raw buffer at a byte offset aligned to the load width.
template <int N>
__device__ __forceinline__ void ld_floats(rsrc_t r, uint32_t off, float* out) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            const float4 v = buf_ld4(r, off + 4u * i, 0);
            out[i] = v.x;
            out[i + 1] = v.y;
            out[i + 2] = v.z;
            out[i + 3] = v.w;
        }
    } else if constexpr (N == 2) {
        const float2 v = buf_ld2(r, off, 0);
        out[0] = v.x;
        out[1] = v.y;
    } else {
        static_assert(N == 1, "1, 2 or a multiple of 4 floats");
        out[0] = buf_ld(r, off, 0);
    }
}

// N floats to a raw buffer at a byte offset (the whole offset in the VGPR: see buf_st4).
template <int N>
__device__ __forceinline__ void st_row(const float* v, rsrc_t r, uint32_t off) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 4) buf_st4(make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]), r, off + 4u * i, 0u);
    } else if constexpr (N == 2) {
        buf_st2(make_float2(v[0], v[1]), r, off, 0u);
    } else {
        static_assert(N == 1, "1, 2 or a multiple of 4 floats");
        buf_st(v[0], r, off, 0u);
    }
}

// N floats to LDS and (when `store`) to the tape at one element offset (N = 1, 2 or 4, aligned to N floats).
template <int N>
__device__ __forceinline__ void st_floats(const float* v, float* lds, int idx, rsrc_t tape, uint32_t voff,
                                          uint32_t soff, bool store = true) {
    if constexpr (N == 4) {
        const float4 x = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(lds + idx) = x;
        if (store) buf_st4_nt(x, tape, voff, soff);
    } else if constexpr (N == 2) {
        const float2 x = make_float2(v[0], v[1]);
        *reinterpret_cast<float2*>(lds + idx) = x;
        if (store) buf_st2(x, tape, voff, soff);
    } else {
        lds[idx] = v[0];
        if (store) buf_st(v[0], tape, voff, soff);
    }
}

// N floats (1, 2 or 4) to LDS at an N-aligned element offset, as one store.
template <int N>
__device__ __forceinline__ void lds_st(float* lds, int idx, const float* v) {
    if constexpr (N == 4) {
        *reinterpret_cast<float4*>(lds + idx) = make_float4(v[0], v[1], v[2], v[3]);
    } else if constexpr (N == 2) {
        *reinterpret_cast<float2*>(lds + idx) = make_float2(v[0], v[1]);
    } else {
        static_assert(N == 1, "1, 2 or 4 floats");
        lds[idx] = v[0];
    }
}

// N floats from the tape at one element offset into LDS (restoring a checkpoint row).
template <int N>
__device__ __forceinline__ void ld_to_lds(float* lds, int idx, rsrc_t tape, uint32_t voff, uint32_t soff) {
    float v[N];
    ld_floats<N>(tape, voff + soff, v);
#pragma unroll
    for (int i = 0; i < N; ++i) lds[idx + i] = v[i];
}

// Maximum and sum over the SEG lanes of one sequence (SEG = 64, or the whole sub-wave block).
__device__ __forceinline__ float gseq_max(float x, int seg) {
    if (seg == 64) return wave_max64(x);
    for (int o = 1; o < seg; o <<= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float gseq_sum(float x, int seg) {
    if (seg == 64) return wave_sum64(x);
    for (int o = 1; o < seg; o <<= 1) x += __shfl_xor(x, o);
    return x;
}
__device__ __forceinline__ void gseq_argmin(float& v, uint32_t& i, int seg) {
    for (int o = 1; o < seg; o <<= 1) {
        const float v2 = __shfl_xor(v, o);
        const uint32_t i2 = (uint32_t)__shfl_xor((int)i, o);
        argmin_merge(v, i, v2, i2);
    }
}
// (max of v, q of the lowest lane attaining it) over the SEG lanes of one sequence.
__device__ __forceinline__ void gseq_argmax_payload(float& v, float& q, int seg) {
    if (seg == 64) {
        seg_argmax_payload<64>(v, q);
        return;
    }
    int lane = (int)(threadIdx.x & 63);
    for (int o = 1; o < seg; o <<= 1) {
        const float v2 = __shfl_xor(v, o);
        const float q2 = __shfl_xor(q, o);
        const int l2 = __shfl_xor(lane, o);
        const bool take = (v2 > v) || (v2 == v && l2 < lane);
        v = take ? v2 : v;
        q = take ? q2 : q;
        lane = take ? l2 : lane;
    }
}

__device__ __forceinline__ void pin_one(float& a) { asm volatile("" : "+v"(a)); }

// Quad reductions (the 4 lanes sharing a block at k = 4).
__device__ __forceinline__ float quad_max(float x) {
    x = fmaxf(x, dpp<0xB1>(x));
    return fmaxf(x, dpp<0x4E>(x));
}
__device__ __forceinline__ float quad_sum(float x) {
    x += dpp<0xB1>(x);
    return x + dpp<0x4E>(x);
}

// Merge the log-sum-exp of one tile (maximum cm, sum of 2^(x - cm) cs, and optionally sum of 2^(x - cm) z, cz) into a
// running one (mx, s, sz): the side with the smaller maximum is scaled by 2^(-|mx - cm|), one exponential.
__device__ __forceinline__ void lse_merge(float& mx, float& s, float cm, float cs) {
    const bool keep = mx >= cm;
    const float e = ex2(fminf(mx, cm) - fmaxf(mx, cm));
    s = keep ? fmaf(cs, e, s) : fmaf(s, e, cs);
    mx = keep ? mx : cm;
}
__device__ __forceinline__ void lse_merge(float& mx, float& s, float& sz, float cm, float cs, float cz) {
    const bool keep = mx >= cm;
    const float e = ex2(fminf(mx, cm) - fmaxf(mx, cm));
    s = keep ? fmaf(cs, e, s) : fmaf(s, e, cs);
    sz = keep ? fmaf(cz, e, sz) : fmaf(sz, e, cz);
    mx = keep ? mx : cm;
}

// IEEE float32 squared distance plus the incoming metric, in a fixed order without fused multiply-add:
// e = fl(d_0 d_0), e = fl(e + fl(d_v d_v)) for v = 1.., then fl(e + vin), d_v = fl(w_v - c_v).
template <int V>
__device__ __forceinline__ float vmetric(const float* wt, const float* c, float vin) {
#pragma clang fp contract(off)
    const float d0 = wt[0] - c[0];
    float e = d0 * d0;
#pragma unroll
    for (int v = 1; v < V; ++v) {
        const float dv = wt[v] - c[v];
        const float ev = dv * dv;
        e = e + ev;
    }
    return e + vin;
}

// LDS position of message group u.  At k = 3 a thread reads and writes its block's 8 consecutive groups as two 16-byte
// accesses 32 bytes apart across the lanes, which puts lanes 4 apart on the same banks.  Flipping bit 2 of u in every
// 32-group row of odd index (bit 5 set) spreads them over distinct banks; a 16-byte access keeps its 4 groups together
// (they share bit 5), and the lane-contiguous accesses of the other direction stay conflict-free.  It is a
// permutation inside each 64 groups.  It is applied where the J = 2^(L-2k) blocks number at least 64 (L >= 12), so
// that j + J a has the bits 2 and 5 of j and the position of j + J a is that of j plus J a.  Other k: the identity.
template <int K>
__device__ __forceinline__ int mpos(int u, int J) {
    if constexpr (K == 3) return J >= 64 ? u ^ ((u >> 3) & 4) : u;
    else return u;
}

// Per-thread view of the trellis: which blocks and groups it owns, and its codebook values.
template <int K, int V, int SPT, bool REG>
struct Owner {
    using Gm = GG<K, V, SPT>;
    static constexpr int P = Gm::P, I = Gm::I, BPT = Gm::BPT, C = Gm::C, TI = Gm::TI, NI = Gm::NI, ROW = Gm::ROW;
    int L, tau, TPS, cl, i0;
    rsrc_t cbs;
    float cbr[REG ? BPT : 1][REG ? P : 1][REG ? I * V : 1];

    __device__ __forceinline__ int j(int m) const { return C == 1 ? tau + TPS * m : tau / C; }
    // first forward group of tile q of block m
    __device__ __forceinline__ int fgroup(int m, int q) const { return (j(m) << K) + i0 + TI * q; }
    // state of (block m, row a, group i0 + TI q + ii)
    __device__ __forceinline__ uint32_t state(int m, int a, int q, int ii) const {
        return ((uint32_t)a << (L - K)) | (uint32_t)fgroup(m, q) + (uint32_t)ii;
    }
    __device__ __forceinline__ uint32_t row_bytes(int m, int a, int q) const {
        return 4u * (uint32_t)V * state(m, a, q, 0);
    }
    // Position of group u in a tape row (G groups).  It is the identity, except where a thread owns several tiles of
    // one block's groups (k = 3).  There the row is tile-major, tile 0 of every block first and then tile 1, so each
    // 16-byte store of a step is contiguous across lanes rather than half of every 32-byte stride.
    __device__ __forceinline__ uint32_t tpos(uint32_t u, uint32_t G) const {
        if constexpr (NI > 1) {
            static_assert(TI == 4 && (P / 4) % NI == 0, "tile index = (u >> 2) mod NI");
            return ((u >> 2) & (uint32_t)(NI - 1)) * (G / NI) + (u >> K) * TI + (u & (uint32_t)(TI - 1));
        } else {
            return u;
        }
    }

    __device__ __forceinline__ void init(const float* cb, int L_, int TPS_) {
        L = L_;
        TPS = TPS_;
        tau = threadIdx.x;
        cl = C == 1 ? 0 : (tau & (C - 1));
        i0 = cl * I;
        cbs = make_rsrc(cb, (uint32_t)V * (4u << L));
        if constexpr (REG) {
#pragma unroll
            for (int m = 0; m < BPT; ++m)
#pragma unroll
                for (int a = 0; a < P; ++a)
#pragma unroll
                    for (int q = 0; q < NI; ++q) ld_floats<ROW>(cbs, row_bytes(m, a, q), &cbr[m][a][ROW * q]);
        }
    }
    // codebook values of tile row (m, a, q): ROW floats, group-major then component
    __device__ __forceinline__ void row(int m, int a, int q, float* out) const {
        if constexpr (REG) {
#pragma unroll
            for (int x = 0; x < ROW; ++x) out[x] = cbr[m][a][ROW * q + x];
        } else {
            ld_floats<ROW>(cbs, row_bytes(m, a, q), out);
        }
    }
    // The rows in the order a step visits them, fetched ahead when they come from memory: forward order (m, q, a)
    // and backward order (m, a, q).  Row idx + 1 after the last is the next step's first.
    static constexpr int NROW = BPT * NI * P;
    __device__ __forceinline__ void fwd_next(int idx, float* nx) const {
        if constexpr (!REG) {
            const int x = (idx + 1) % NROW;
            row(x / (NI * P), x % P, (x / P) % NI, nx);
        }
    }
    __device__ __forceinline__ void bwd_next(int idx, float* nx) const {
        if constexpr (!REG) {
            const int x = (idx + 1) % NROW;
            row(x / (NI * P), (x / NI) % P, x % NI, nx);
        }
    }
    // Rows in flight from memory: two cover the L2 latency for the gradient (k = 3: 82.9 -> 78.6 ms); three cost it
    // registers.  The forward and backward orders differ from the second row on, so a change of direction primes the
    // ring again.
    static constexpr int PFD = 2;
    using Ring = float[REG ? 1 : PFD][REG ? 1 : ROW];
    __device__ __forceinline__ void fwd_prime(Ring& nx) const {
        if constexpr (!REG) {
#pragma unroll
            for (int d = 0; d < PFD; ++d) fwd_next(d - 1, nx[d]);
        }
    }
    __device__ __forceinline__ void bwd_prime(Ring& nx) const {
        if constexpr (!REG) {
#pragma unroll
            for (int d = 0; d < PFD; ++d) bwd_next(d - 1, nx[d]);
        }
    }
    // this row: from registers, or the oldest prefetched copy (then the row PFD ahead is fetched into the ring)
    __device__ __forceinline__ void take_fwd(int m, int a, int q, float* c, Ring& nx) const {
        if constexpr (REG) {
            row(m, a, q, c);
        } else {
#pragma unroll
            for (int x = 0; x < ROW; ++x) c[x] = nx[0][x];
#pragma unroll
            for (int d = 0; d + 1 < PFD; ++d)
#pragma unroll
                for (int x = 0; x < ROW; ++x) nx[d][x] = nx[d + 1][x];
            fwd_next((m * NI + q) * P + a + PFD - 1, nx[PFD - 1]);
        }
    }
    __device__ __forceinline__ void take_bwd(int m, int a, int q, float* c, Ring& nx) const {
        if constexpr (REG) {
            row(m, a, q, c);
        } else {
#pragma unroll
            for (int x = 0; x < ROW; ++x) c[x] = nx[0][x];
#pragma unroll
            for (int d = 0; d + 1 < PFD; ++d)
#pragma unroll
                for (int x = 0; x < ROW; ++x) nx[d][x] = nx[d + 1][x];
            bwd_next((m * P + a) * NI + q + PFD - 1, nx[PFD - 1]);
        }
    }
};

}  // namespace

// ------------------------------------------------------------------------------------------------------------------
// soft codeword (and ln Z)

template <int K, int V, int SPT, int LT>
__global__ void __launch_bounds__(1024) gen_soft_kernel(GenArgs args) {
    using Gm = GG<K, V, SPT>;
    constexpr int P = Gm::P, I = Gm::I, BPT = Gm::BPT, C = Gm::C, TA = Gm::TA, TI = Gm::TI, NA = Gm::NA,
                  NI = Gm::NI, ROW = Gm::ROW;
    // codebook in VGPRs only where it leaves room: k = 1 holds 32 inputs per step, k = 4 16 rows of tape loads
    constexpr bool REG = SPT * V <= 64 && (SPT < 64 || (K == 2 || K == 3));
    extern __shared__ float lds[];
    __shared__ float redmax[2][16];
    __shared__ float redsum[2][16];

    const int L = LT ? LT : args.L, n = args.n, TPS = LT ? (1 << LT) / SPT : (int)blockDim.x, tau = threadIdx.x;
    const int lane = tau & 63, wv = tau >> 6;
    const int G = 1 << (L - K), J = 1 << (L - 2 * K);
    const int WPS = TPS >= 64 ? TPS >> 6 : 1, SEG = TPS >= 64 ? 64 : TPS;
    const float scale = args.scale, inv_scale = 1.0f / scale;
    float* msg0 = lds;
    float* msg1 = args.dbl ? lds + G : lds;

    Owner<K, V, SPT, REG> own;
    own.init(args.cb, L, TPS);

    // tape of the block's sequence: the R~ rows (TapeRows), [n] normalisers, the per-wave (S0, S1[V]) of every step,
    // then (checkpoint mode) each thread's share of the backward message while a segment is recomputed
    const uint32_t slot_bytes = (uint32_t)args.slot_bytes;
    const rsrc_t tape = make_rsrc(args.ws + (size_t)blockIdx.x * args.slot_bytes, slot_bytes);
    const uint32_t row_bytes = (uint32_t)G * 4u;
    const int ck = args.ckpt;
    const TapeRows rows{ck, n, row_bytes, ck ? (uint32_t)(n / ck + 1) * row_bytes : 0u};
    const uint32_t nrm_base = (uint32_t)align256(TapeRows::rows(ck, n) * G * 4);
    const uint32_t part_base = nrm_base + (uint32_t)align256((size_t)n * 4);
    const uint32_t save_base = part_base + (WPS > 1 ? (uint32_t)align256((size_t)n * WPS * (1 + V) * 4) : 0u);
    const uint32_t v_j0 = 4u * (uint32_t)own.j(0);   // lane part of a backward group's tape offset
    // tape offset of backward group j(m) + J a: a lane part (VGPR) and a uniform part, or all of it in the VGPR when
    // the row is tile-major
    auto grp_voff = [&](int m, int a) -> uint32_t {
        if constexpr (NI > 1) return 4u * own.tpos((uint32_t)(own.j(m) + J * a), (uint32_t)G);
        else return v_j0;
    };
    auto grp_soff = [&](int m, int a) -> uint32_t {
        if constexpr (NI > 1) return 0u;
        else return 4u * (uint32_t)(own.j(m) - own.j(0) + J * a);
    };
    typename Owner<K, V, SPT, REG>::Ring cnx;          // the next codebook rows (read from memory)
    own.fwd_prime(cnx);

    for (int64_t b = blockIdx.x; b < args.B; b += gridDim.x) {
        if (b != blockIdx.x) own.fwd_prime(cnx);   // the backward pass left the ring in its own order
        const int64_t row = args.sigma_enum ? (b >> L) : b;   // the weights' row (sigma enumeration: v >> L)
        const float* wb = args.w + row * (int64_t)n * V;
        const bool has_sigma = args.sigma_enum || args.sigma != nullptr;
        const uint32_t sig = args.sigma_enum ? (uint32_t)(b & ((1 << L) - 1))
                                             : has_sigma ? ((uint32_t)args.sigma[b] & ((1u << L) - 1u)) : 0u;

        // ------------------------------------------------------------------ forward
#pragma unroll
        for (int m = 0; m < BPT; ++m)
#pragma unroll
            for (int q = 0; q < NI; ++q) {
                float r[TI];
                const int u0 = own.fgroup(m, q);
#pragma unroll
                for (int ii = 0; ii < TI; ++ii)
                    r[ii] = (!has_sigma || (uint32_t)(u0 + ii) == (sig & (uint32_t)(G - 1))) ? 0.f : kNeg;
                st_floats<TI>(r, msg0, mpos<K>(u0, J), tape, 4u * own.tpos(u0, G), 0u);
            }
        lds_barrier();

        // One forward step: R~_{t+1} = logsumexp over the predecessors minus Nt, from mc into mn (the same buffer when
        // single-buffered: every input is read before a barrier), and into the tape at row_soff when `store`.  Returns
        // this thread's maximum of the outputs.  The checkpoint recompute runs it again with the stored normalisers,
        // so the recomputed rows are bit-identical to the first pass's.
        auto fwd_step = [&](const float* wt, float Nt, const float* mc, float* mn, uint32_t row_soff, bool store) {
            float rin[BPT][P];
#pragma unroll
            for (int m = 0; m < BPT; ++m)
#pragma unroll
                for (int a = 0; a < P; ++a) rin[m][a] = mc[mpos<K>(own.j(m), J) + J * a];
            if (!args.dbl) lds_barrier();   // every input read before any output overwrites it
            float lmax = -3.0e38f;
#pragma unroll
            for (int m = 0; m < BPT; ++m)
#pragma unroll
                for (int q = 0; q < NI; ++q) {
                    float mx[TI], s[TI];
#pragma unroll
                    for (int r = 0; r < NA; ++r) {
                        float x[TA][TI];
#pragma unroll
                        for (int aa = 0; aa < TA; ++aa) {
                            const int a = r * TA + aa;
                            float c[ROW];
                            own.take_fwd(m, a, q, c, cnx);
#pragma unroll
                            for (int ii = 0; ii < TI; ++ii) {
                                float acc = rin[m][a];
#pragma unroll
                                for (int v = 0; v < V; ++v) {
                                    const float d = fmaf(c[ii * V + v], scale, -wt[v]);
                                    acc = fmaf(-d, d, acc);
                                }
                                x[aa][ii] = acc;
                            }
                        }
#pragma unroll
                        for (int ii = 0; ii < TI; ++ii) {
                            float cm = x[0][ii];
#pragma unroll
                            for (int aa = 1; aa < TA; ++aa) cm = fmaxf(cm, x[aa][ii]);
                            float cs = 0.f;
#pragma unroll
                            for (int aa = 0; aa < TA; ++aa) cs += ex2(x[aa][ii] - cm);
                            if (r == 0) {
                                mx[ii] = cm;
                                s[ii] = cs;
                            } else {
                                lse_merge(mx[ii], s[ii], cm, cs);
                            }
                        }
                        GEN_SCHED_BARRIER();
                    }
                    float o[TI];
#pragma unroll
                    for (int ii = 0; ii < TI; ++ii) {
                        o[ii] = (mx[ii] - Nt) + lg2(s[ii]);
                        lmax = run_max(lmax, o[ii]);
                    }
                    const int u0 = own.fgroup(m, q);
                    st_floats<TI>(o, mn, mpos<K>(u0, J), tape, 4u * own.tpos(u0, G), row_soff, store);
                }
            return lmax;
        };

        float N = 0.f, N_last = 0.f;
        double A = 0.0;
        float w_nx[V];
#pragma unroll
        for (int v = 0; v < V; ++v) w_nx[v] = wb[v];
        for (int t = 0; t < n; ++t) {
            const float* mc = args.dbl && (t & 1) ? msg1 : msg0;
            float* mn = args.dbl ? ((t & 1) ? msg0 : msg1) : msg0;
            float wt[V];
#pragma unroll
            for (int v = 0; v < V; ++v) wt[v] = w_nx[v] * scale;
            if (t + 1 < n) {
#pragma unroll
                for (int v = 0; v < V; ++v) w_nx[v] = wb[(t + 1) * V + v];
            }
            const float lmax_t = fwd_step(wt, N, mc, mn, rows.off(t + 1), rows.stored(t + 1));
            float lmax = lmax_t;
            if (tau == 0) buf_st(N, tape, 0u, nrm_base + 4u * t);
            lmax = gseq_max(lmax, SEG);
            if (WPS > 1 && lane == 0) redmax[t & 1][wv] = lmax;
            lds_barrier();
            if (WPS > 1) lmax = row16_max((lane & 15) < WPS ? redmax[t & 1][lane & 15] : -3.0e38f);
            lmax = uniform_f(lmax);
            A += (double)N;
            N_last = N;
            N = lmax;
        }
        // rz = log2 Z - A_n
        float rz;
        if (!has_sigma) {
            const float* mf = args.dbl && (n & 1) ? msg1 : msg0;
            float part = 0.f;
#pragma unroll
            for (int m = 0; m < BPT; ++m)
#pragma unroll
                for (int q = 0; q < NI; ++q)
#pragma unroll
                    for (int ii = 0; ii < TI; ++ii) part += ex2(mf[mpos<K>(own.fgroup(m, q), J) + ii] - N);
            part = gseq_sum(part, SEG);
            if (WPS > 1 && lane == 0) redsum[n & 1][wv] = part;
            lds_barrier();
            if (WPS > 1) {
                part = 0.f;
                for (int q = 0; q < WPS; ++q) part += redsum[n & 1][q];
            }
            rz = N + lg2(part);
            __syncthreads();
        } else {
            __syncthreads();   // the tape rows of the forward pass, written by other threads
            const float r = buf_ld_nt(tape, 0u, rows.off(n - 1) + 4u * own.tpos(sig >> K, G));
            float x = r;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const float d = fmaf(args.cb[sig * V + v], scale, -(wb[(n - 1) * V + v] * scale));
                x = fmaf(-d, d, x);
            }
            rz = (r < 0.5f * kNeg) ? kNeg : x - N_last;
        }
        const bool valid = rz > 0.5f * kNeg;
        if (tau == 0 && args.log_z)
            args.log_z[b] = valid ? (float)((A + (double)rz) * 0.6931471805599453) : -__builtin_inff();

        // ------------------------------------------------------------------ backward + posterior
        float Nb = 0.f, C_ = 0.f, D = 0.f;
        int t = n - 1;
        if (!has_sigma) {
            float* mi = args.dbl && ((n - 1) & 1) ? msg1 : msg0;
#pragma unroll
            for (int m = 0; m < BPT; ++m)
#pragma unroll
                for (int q = 0; q < NI; ++q)
#pragma unroll
                    for (int ii = 0; ii < TI; ++ii) mi[mpos<K>(own.fgroup(m, q), J) + ii] = 0.f;
        } else {
            // s_n = sigma: the posterior at n-1 is the indicator of sigma; the one finite message left is
            // B_{n-2}(sigma >> k) = theta_{n-1}(sigma).  It goes into the offset C_ and the message starts at 0, so
            // the next step's branch terms are not rounded at theta's magnitude (a hundred or more in log2 units)
            float* mi = args.dbl && ((n - 2) & 1) ? msg1 : msg0;
            float th = 0.f;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const float d = fmaf(args.cb[sig * V + v], scale, -(wb[(n - 1) * V + v] * scale));
                th = fmaf(-d, d, th);
            }
            if (n > 1) {
#pragma unroll
                for (int m = 0; m < BPT; ++m)
#pragma unroll
                    for (int q = 0; q < NI; ++q)
#pragma unroll
                        for (int ii = 0; ii < TI; ++ii) {
                            const uint32_t u = (uint32_t)(own.fgroup(m, q) + ii);
                            mi[mpos<K>((int)u, J)] = (u == (sig >> K)) ? 0.f : kNeg;
                        }
            }
            if (tau == 0) {
#pragma unroll
                for (int v = 0; v < V; ++v)
                    args.w_soft[(b * n + n - 1) * V + v] = valid ? args.cb[sig * V + v] : __builtin_nanf("");
            }
            D = N_last;
            C_ = th;
            t = n - 2;
        }
        lds_barrier();

        const int t_out = t;
        float N_nx = 0.f, rq_nx = 0.f;
        if (t >= 0) {
#pragma unroll
            for (int v = 0; v < V; ++v) w_nx[v] = wb[t * V + v];
            N_nx = buf_ld_nt(tape, 0u, nrm_base + 4u * t);
            rq_nx = buf_ld_nt(tape, grp_voff(0, 0), rows.off(t) + grp_soff(0, 0));
        }
        own.bwd_prime(cnx);
        while (t >= 0) {
        const int t0 = ck ? (t / ck) * ck : 0;   // first step of this segment
        if (ck) {
            // checkpoint mode: keep this thread's share of the backward message in the workspace, rebuild
            // R~_{t0+1..t} from checkpoint t0 with the stored normalisers, then restore the message
#pragma unroll
            for (int m = 0; m < BPT; ++m)
#pragma unroll
                for (int q = 0; q < NI; ++q) st_row<TI>(msg0 + mpos<K>(own.fgroup(m, q), J), tape, save_base + 4u * own.fgroup(m, q));
            lds_barrier();   // every share read before the recompute overwrites the buffer
#pragma unroll
            for (int m = 0; m < BPT; ++m)
#pragma unroll
                for (int q = 0; q < NI; ++q)
                    ld_to_lds<TI>(msg0, mpos<K>(own.fgroup(m, q), J), tape, 4u * own.tpos(own.fgroup(m, q), G), rows.off(t0));
            lds_barrier();
            own.fwd_prime(cnx);
            for (int tt = t0; tt < t; ++tt) {
                float wr[V];
#pragma unroll
                for (int v = 0; v < V; ++v) wr[v] = wb[tt * V + v] * scale;
                const float Nr = uniform_f(buf_ld(tape, 0u, nrm_base + 4u * tt));
                fwd_step(wr, Nr, msg0, msg0, rows.off(tt + 1), true);
                lds_barrier();
            }
            own.bwd_prime(cnx);
            __syncthreads();   // the recomputed rows, written by other threads, before the backward reads them
#pragma unroll
            for (int m = 0; m < BPT; ++m)
#pragma unroll
                for (int q = 0; q < NI; ++q)
                    ld_to_lds<TI>(msg0, mpos<K>(own.fgroup(m, q), J), tape, save_base + 4u * own.fgroup(m, q), 0u);
            lds_barrier();
            rq_nx = buf_ld_nt(tape, grp_voff(0, 0), rows.off(t) + grp_soff(0, 0));
        }
        for (; t >= t0; --t) {
            const float* mc = args.dbl && (t & 1) ? msg1 : msg0;
            float* mn = args.dbl ? ((t & 1) ? msg0 : msg1) : msg0;
            float wt[V];
#pragma unroll
            for (int v = 0; v < V; ++v) wt[v] = w_nx[v] * scale;
            const float Nt = uniform_f(N_nx);
            if (t > 0) {
#pragma unroll
                for (int v = 0; v < V; ++v) w_nx[v] = wb[(t - 1) * V + v];
                N_nx = buf_ld_nt(tape, 0u, nrm_base + 4u * (t - 1));
            }
            float bin[BPT][I];
#pragma unroll
            for (int m = 0; m < BPT; ++m)
#pragma unroll
                for (int q = 0; q < NI; ++q)
#pragma unroll
                    for (int ii = 0; ii < TI; ++ii) bin[m][TI * q + ii] = mc[mpos<K>(own.fgroup(m, q), J) + ii];
            if (!args.dbl) lds_barrier();
            D += Nt;
            const float ref = (rz + D) - C_;
            float lmax = -3.0e38f, S0 = 0.f, S1[V];
#pragma unroll
            for (int v = 0; v < V; ++v) S1[v] = 0.f;
#pragma unroll
            for (int m = 0; m < BPT; ++m)
#pragma unroll
                for (int a = 0; a < P; ++a) {
                    const int vg = own.j(m) + J * a;   // backward group of row a
                    // R~_t of this group, and the next group's (or the next step's first) one row ahead
                    const float rq = rq_nx;
                    if (m * P + a + 1 < BPT * P) {
                        const int m2 = (m * P + a + 1) / P, a2 = (m * P + a + 1) % P;
                        rq_nx = buf_ld_nt(tape, grp_voff(m2, a2), rows.off(t) + grp_soff(m2, a2));
                    } else {   // the next step's first (a harmless re-read of row 0 at t = 0; in checkpoint mode
                               // re-read after the next segment is rebuilt)
                        rq_nx = buf_ld_nt(tape, grp_voff(0, 0), rows.off(t > 0 ? t - 1 : 0) + grp_soff(0, 0));
                    }
                    float mx = 0.f, s = 0.f;
#pragma unroll
                    for (int q = 0; q < NI; ++q) {
                        float c[ROW], y[TI], d[TI][V];
                        own.take_bwd(m, a, q, c, cnx);
#pragma unroll
                        for (int ii = 0; ii < TI; ++ii) {
                            float acc = bin[m][TI * q + ii];
#pragma unroll
                            for (int v = 0; v < V; ++v) {
                                d[ii][v] = fmaf(c[ii * V + v], scale, -wt[v]);
                                acc = fmaf(-d[ii][v], d[ii][v], acc);
                            }
                            y[ii] = acc;
                        }
                        float cm = y[0];
#pragma unroll
                        for (int ii = 1; ii < TI; ++ii) cm = fmaxf(cm, y[ii]);
                        if constexpr (C > 1) cm = quad_max(cm);
                        float e[TI], cs = 0.f;
#pragma unroll
                        for (int ii = 0; ii < TI; ++ii) {
                            e[ii] = ex2(y[ii] - cm);
                            cs += e[ii];
                        }
                        const float f = ex2((cm + rq) - ref);
                        S0 = fmaf(f, cs, S0);
#pragma unroll
                        for (int v = 0; v < V; ++v) {
                            float ed = 0.f;
#pragma unroll
                            for (int ii = 0; ii < TI; ++ii) ed = fmaf(e[ii], d[ii][v], ed);
                            S1[v] = fmaf(f, ed, S1[v]);
                        }
                        if constexpr (C > 1) cs = quad_sum(cs);
                        if (q == 0) {
                            mx = cm;
                            s = cs;
                        } else {
                            lse_merge(mx, s, cm, cs);
                        }
                    }
                    const float out = (mx - Nb) + lg2(s);
                    lmax = run_max(lmax, out);
                    mn[mpos<K>(own.j(m), J) + J * a] = out;   // the lanes of a quad store the same value; at t = 0 nobody reads it
                    pin_order(S0, lmax);
#pragma unroll
                    for (int v = 0; v < V; ++v) pin_one(S1[v]);
                    GEN_SCHED_BARRIER();
                }
            lmax = gseq_max(lmax, SEG);
            S0 = gseq_sum(S0, SEG);
#pragma unroll
            for (int v = 0; v < V; ++v) S1[v] = gseq_sum(S1[v], SEG);
            if (WPS > 1) {
                if (lane == 0) {
                    redmax[t & 1][wv] = lmax;
                    const uint32_t po = part_base + 4u * (uint32_t)((t * WPS + wv) * (1 + V));
                    buf_st(S0, tape, 0u, po);
#pragma unroll
                    for (int v = 0; v < V; ++v) buf_st(S1[v], tape, 0u, po + 4u * (1 + v));
                }
            } else if (tau == 0) {
#pragma unroll
                for (int v = 0; v < V; ++v)
                    args.w_soft[(b * n + t) * V + v] = valid ? fmaf(S1[v] / S0, inv_scale, wb[t * V + v])
                                                             : __builtin_nanf("");
            }
            lds_barrier();
            if (WPS > 1) lmax = row16_max((lane & 15) < WPS ? redmax[t & 1][lane & 15] : -3.0e38f);
            lmax = uniform_f(lmax);
            C_ += Nb;
            Nb = lmax;
        }
        }   // segments
        if (WPS > 1) {
            __syncthreads();   // the per-wave partial sums, written by other waves
            for (int tt = tau; tt <= t_out; tt += TPS) {
                float S0 = 0.f, S1[V];
#pragma unroll
                for (int v = 0; v < V; ++v) S1[v] = 0.f;
                for (int q = 0; q < WPS; ++q) {
                    const uint32_t po = part_base + 4u * (uint32_t)((tt * WPS + q) * (1 + V));
                    S0 += buf_ld(tape, 0u, po);
#pragma unroll
                    for (int v = 0; v < V; ++v) S1[v] += buf_ld(tape, 0u, po + 4u * (1 + v));
                }
#pragma unroll
                for (int v = 0; v < V; ++v)
                    args.w_soft[(b * n + tt) * V + v] = valid ? fmaf(S1[v] / S0, inv_scale, wb[tt * V + v])
                                                              : __builtin_nanf("");
            }
        }
        __syncthreads();   // the next sequence reuses the tape and LDS
    }
}

// ------------------------------------------------------------------------------------------------------------------
// Viterbi hard code

// NSQ = 2: the workgroup decodes two sequences in lockstep, so every codebook row it reads from memory serves both
// (where the codebook does not fit in registers, its stream through L1 otherwise takes most of a step).  Lanes 0..NSQ-1
// trace the sequences back, so a workgroup needs at least NSQ threads (the host pairs sequences only at L >= 12).
template <int K, int V, int SPT, int LT, int NSQ>
__global__ void __launch_bounds__(1024) gen_viterbi_kernel(GenArgs args) {
    using Gm = GG<K, V, SPT>;
    constexpr int P = Gm::P, I = Gm::I, BPT = Gm::BPT, C = Gm::C, TI = Gm::TI, NI = Gm::NI, ROW = Gm::ROW;
    constexpr bool REG = SPT * V <= 64;
    constexpr float kInf = __builtin_huge_valf();
    extern __shared__ float lds[];
    __shared__ float redv[NSQ][16];
    __shared__ uint32_t redi[NSQ][16];

    const int L = LT ? LT : args.L, n = args.n, TPS = LT ? (1 << LT) / SPT : (int)blockDim.x, tau = threadIdx.x;
    const int lane = tau & 63, wv = tau >> 6;
    const int G = 1 << (L - K), J = 1 << (L - 2 * K);
    const int WPS = TPS >= 64 ? TPS >> 6 : 1, SEG = TPS >= 64 ? 64 : TPS;
    const int MB = args.dbl ? 2 * G : G;   // floats of one sequence's message buffers (sequence z at lds + z MB)

    Owner<K, V, SPT, REG> own;
    own.init(args.cb, L, TPS);

    // back-pointer tape: 2 parities (by round) x NSQ sequences of [n][TPS] words.  A thread's word of step t holds,
    // for each of its forward groups g = m I + ii, the k-bit row a of the best predecessor in bits [g k, g k + k).
    const uint32_t slot_bytes = (uint32_t)args.slot_bytes;
    const rsrc_t tape = make_rsrc(args.ws + (size_t)blockIdx.x * args.slot_bytes, slot_bytes);
    const uint32_t buf_bytes = (uint32_t)n * TPS * 4u;
    typename Owner<K, V, SPT, REG>::Ring cnx;   // the next codebook rows (read from memory)
    own.fwd_prime(cnx);

    // the word and bit field of forward group u at any step
    auto bp_loc = [&](uint32_t u, uint32_t& word_idx, uint32_t& bit) {
        const uint32_t jj = u >> K, i = u & (uint32_t)(P - 1);
        if constexpr (C == 1) {
            word_idx = jj % (uint32_t)TPS;
            bit = ((jj / (uint32_t)TPS) * I + i) * K;
        } else {
            word_idx = jj * C + i / I;
            bit = (i % I) * K;
        }
    };

    const bool trace = args.states != nullptr;   // else costs only: no traceback (the back pointers are still kept)
    // pending traceback: lane z (tau == z) traces back the previous round's sequence z, one step per forward step
    int64_t pend_b = -1;
    int pend_t = 0;
    uint32_t pend_s = 0, pend_word = 0, pend_buf = 0;
    auto pend_fetch = [&]() {   // the word that decides s_{pend_t - 1}
        uint32_t wi, bit;
        bp_loc(pend_s >> K, wi, bit);
        pend_word = __builtin_bit_cast(uint32_t, buf_ld(tape, 0u, pend_buf + (uint32_t)(pend_t - 1) * (TPS * 4u) +
                                                                          4u * wi));
    };
    auto pend_step = [&]() {
        uint32_t wi, bit;
        const uint32_t u = pend_s >> K;
        bp_loc(u, wi, bit);
        const uint32_t a = (pend_word >> bit) & (uint32_t)(P - 1);
        pend_s = (a << (L - K)) | u;
        --pend_t;
        args.states[pend_b * args.n + pend_t] = (int32_t)pend_s;
        if (pend_t >= 1) pend_fetch();
    };
    // codewords of a finished round's sequences (their states are complete)
    auto gather = [&](int64_t rr) {
#pragma unroll
        for (int z = 0; z < NSQ; ++z) {
            const int64_t pb = rr * NSQ + z;
            if (pb >= args.B) continue;
            for (int x = tau; x < n * V; x += TPS) {
                const int tt = x / V, v = x - tt * V;
                args.w_hard[pb * n * V + x] = args.cb[(size_t)args.states[pb * n + tt] * V + v];
            }
        }
    };

    const int64_t rounds = (args.B + NSQ - 1) / NSQ;
    const bool has_sigma = args.sigma_enum || args.sigma != nullptr;
    int64_t iter = 0;
    for (int64_t r = blockIdx.x; r < rounds; r += gridDim.x, ++iter) {
        const uint32_t par = (uint32_t)(iter & 1);
        int64_t bz[NSQ];
        const float* wb[NSQ];
        uint32_t sig[NSQ];
#pragma unroll
        for (int z = 0; z < NSQ; ++z) {
            bz[z] = r * NSQ + z;
            const int64_t bb = bz[z] < args.B ? bz[z] : args.B - 1;   // a missing second sequence repeats the last
            const int64_t row = args.sigma_enum ? (bb >> L) : bb;      // the weights' row (sigma enumeration: v >> L)
            wb[z] = args.w + row * (int64_t)n * V;
            sig[z] = args.sigma_enum ? (uint32_t)(bb & ((1 << L) - 1))
                                     : has_sigma ? ((uint32_t)args.sigma[bb] & ((1u << L) - 1u)) : 0u;
        }

#pragma unroll
        for (int z = 0; z < NSQ; ++z)
#pragma unroll
            for (int m = 0; m < BPT; ++m)
#pragma unroll
                for (int q = 0; q < NI; ++q)
#pragma unroll
                    for (int ii = 0; ii < TI; ++ii) {
                        const int u = own.fgroup(m, q) + ii;
                        lds[z * MB + mpos<K>(u, J)] = (!has_sigma || (uint32_t)u == (sig[z] & (uint32_t)(G - 1))) ? 0.f : kInf;
                    }
        lds_barrier();

        for (int t = 0; t + 1 < n; ++t) {
            const int oc = args.dbl && (t & 1) ? G : 0, on = args.dbl ? ((t & 1) ? 0 : G) : 0;
            float wt[NSQ][V];
#pragma unroll
            for (int z = 0; z < NSQ; ++z)
#pragma unroll
                for (int v = 0; v < V; ++v) wt[z][v] = wb[z][t * V + v];
            float vin[NSQ][BPT][P];
#pragma unroll
            for (int z = 0; z < NSQ; ++z)
#pragma unroll
                for (int m = 0; m < BPT; ++m)
#pragma unroll
                    for (int a = 0; a < P; ++a) vin[z][m][a] = lds[z * MB + oc + mpos<K>(own.j(m), J) + J * a];
            if (!args.dbl) lds_barrier();
            uint32_t word[NSQ];
#pragma unroll
            for (int z = 0; z < NSQ; ++z) word[z] = 0;
#pragma unroll
            for (int m = 0; m < BPT; ++m)
#pragma unroll
                for (int q = 0; q < NI; ++q) {
                    float best[NSQ][TI];
                    uint32_t arg[NSQ][TI];
#pragma unroll
                    for (int z = 0; z < NSQ; ++z)
#pragma unroll
                        for (int ii = 0; ii < TI; ++ii) {
                            best[z][ii] = kInf;
                            arg[z][ii] = 0;
                        }
#pragma unroll
                    for (int a = 0; a < P; ++a) {
                        float c[ROW];
                        own.take_fwd(m, a, q, c, cnx);
#pragma unroll
                        for (int z = 0; z < NSQ; ++z)
#pragma unroll
                            for (int ii = 0; ii < TI; ++ii) {
                                const float M = vmetric<V>(wt[z], &c[ii * V], vin[z][m][a]);
                                const bool take = M < best[z][ii];   // strict: the smallest a wins ties
                                best[z][ii] = take ? M : best[z][ii];
                                arg[z][ii] = take ? (uint32_t)a : arg[z][ii];
                            }
                        if constexpr (NSQ > 1) GEN_SCHED_BARRIER();   // one row at a time: bounds the live values
                    }
#pragma unroll
                    for (int z = 0; z < NSQ; ++z) {
#pragma unroll
                        for (int ii = 0; ii < TI; ++ii) word[z] |= arg[z][ii] << ((m * I + TI * q + ii) * K);
                        // the tile's metrics as one 16-byte (8-byte at k = 1) store: the position is TI-aligned
                        lds_st<TI>(lds + z * MB + on, mpos<K>(own.fgroup(m, q), J), best[z]);
                    }
                    GEN_SCHED_BARRIER();
                }
#pragma unroll
            for (int z = 0; z < NSQ; ++z)
                buf_st(__builtin_bit_cast(float, word[z]), tape, 4u * tau,
                       (par * NSQ + z) * buf_bytes + (uint32_t)t * (TPS * 4u));
            if (tau < NSQ && pend_b >= 0 && pend_t >= 1) pend_step();
            lds_barrier();
        }

        // last step: M_{n-1}(s) of every state and the end state (the smallest s attaining the minimum), or sigma
        const int ol = args.dbl && ((n - 1) & 1) ? G : 0;
        float wl[NSQ][V];
#pragma unroll
        for (int z = 0; z < NSQ; ++z)
#pragma unroll
            for (int v = 0; v < V; ++v) wl[z][v] = wb[z][(n - 1) * V + v];
        float best[NSQ];
        uint32_t bidx[NSQ];
#pragma unroll
        for (int z = 0; z < NSQ; ++z) {
            best[z] = kInf;
            bidx[z] = 0xffffffffu;
        }
        if (!has_sigma) {
#pragma unroll
            for (int m = 0; m < BPT; ++m)
#pragma unroll
                for (int a = 0; a < P; ++a) {
                    float vl[NSQ];
#pragma unroll
                    for (int z = 0; z < NSQ; ++z) vl[z] = lds[z * MB + ol + mpos<K>(own.j(m), J) + J * a];
#pragma unroll
                    for (int q = 0; q < NI; ++q) {
                        float c[ROW];
                        own.row(m, a, q, c);
#pragma unroll
                        for (int z = 0; z < NSQ; ++z)
#pragma unroll
                            for (int ii = 0; ii < TI; ++ii)
                                argmin_merge(best[z], bidx[z], vmetric<V>(wl[z], &c[ii * V], vl[z]),
                                             own.state(m, a, q, ii));
                    }
                }
#pragma unroll
            for (int z = 0; z < NSQ; ++z) {
                gseq_argmin(best[z], bidx[z], SEG);
                if (WPS > 1 && lane == 0) {
                    redv[z][wv] = best[z];
                    redi[z][wv] = bidx[z];
                }
            }
            __syncthreads();   // also publishes this round's back pointers to the traceback lanes
            if (WPS > 1) {
#pragma unroll
                for (int z = 0; z < NSQ; ++z)
                    for (int q = 0; q < WPS; ++q) argmin_merge(best[z], bidx[z], redv[z][q], redi[z][q]);
            }
        } else {
            __syncthreads();
#pragma unroll
            for (int z = 0; z < NSQ; ++z) {
                bidx[z] = sig[z];
                best[z] = vmetric<V>(wl[z], args.cb + (size_t)sig[z] * V, lds[z * MB + ol + mpos<K>((int)(sig[z] >> K), J)]);
            }
        }
        if (tau == 0 && args.cost) {
#pragma unroll
            for (int z = 0; z < NSQ; ++z)
                if (bz[z] < args.B) args.cost[bz[z]] = best[z];
        }

        // finish the previous round's tracebacks and gather its codewords
        if (tau < NSQ && pend_b >= 0) {
            while (pend_t >= 1) pend_step();
        }
        __syncthreads();
        if (args.w_hard && iter > 0) gather(r - gridDim.x);
        if (tau < NSQ && trace) {
            pend_b = -1;
#pragma unroll
            for (int z = 0; z < NSQ; ++z) {
                if (z == tau && bz[z] < args.B) {   // lane z takes this round's sequence z
                    pend_b = bz[z];
                    pend_buf = (par * NSQ + z) * buf_bytes;
                    pend_s = bidx[z];
                    pend_t = n - 1;
                    args.states[bz[z] * n + n - 1] = (int32_t)bidx[z];
                    if (n > 1) pend_fetch();
                }
            }
        }
        __syncthreads();   // LDS and the other parity's back-pointer buffers are reused next
    }

    if (tau < NSQ && pend_b >= 0) {
        while (pend_t >= 1) pend_step();
    }
    __syncthreads();
    if (args.w_hard && iter > 0) gather(blockIdx.x + (iter - 1) * (int64_t)gridDim.x);
}

// ------------------------------------------------------------------------------------------------------------------
// exact gradient with respect to the weights (and the soft codeword; with GC, the codebook values too)
//
// As in the k = 2 gradient kernel: grad_{u,v} = (2/T) Cov_p(c(s_u, v), F) with F = sum_t <g_t, c(s_t) - w_t>, and
// E[F | s_t] is split into a forward expectation message Q (weighted by the forward softmax over a) and a backward one
// P (weighted by the backward softmax over i).  Both are re-centred every step by a constant the covariance ignores:
// Q by its value at the most likely group, P by kappa_{t+1} = <g_{t+1}, w_soft_{t+1} - w_{t+1}>.  The constants are
// carried as one per-step offset, so E[F | s] - E[F] is formed from small numbers only.
//
// GC adds the codebook gradient, as in the k = 2 kernel.  For every state s, component v and step t of the backward
// pass it adds p_t(s) [g_{t,v} + (2/T) (w_{t,v} - c(s, v)) (E[F | s_t = s] - E[F])] to a per-slot float accumulator
// [2^L][V] at the end of the slot.  Each thread reads and writes only its own states' entries.  Each step's posterior
// is normalised by the previous step's exact total, with the running normaliser sums in double.  A later reduction
// sums the slots in a fixed order.

// QG: the expectation message Q^ lives in the workspace (served from L2) instead of LDS, for trellises whose two
// message arrays exceed LDS (k = 1 at L = 16: 2 x 128 KiB); the step barriers then fence global memory as well.
template <int K, int V, int SPT, int LT, bool GC, bool CK, bool QG>
__global__ void __launch_bounds__(1024) gen_grad_kernel(GenArgs args) {
    using Gm = GG<K, V, SPT>;
    constexpr int P = Gm::P, I = Gm::I, BPT = Gm::BPT, C = Gm::C, TA = Gm::TA, TI = Gm::TI, NA = Gm::NA,
                  NI = Gm::NI, ROW = Gm::ROW;
    constexpr bool REG = SPT * V <= 32;
    constexpr int NS = 2 + 2 * V;   // S0, S1[V], S2, S3[V]
    extern __shared__ float lds[];
    __shared__ float redmax[2][16];
    __shared__ float redq[2][16];
    __shared__ float reds[2][16][2 + V];

    const int L = LT ? LT : args.L, n = args.n, TPS = LT ? (1 << LT) / SPT : (int)blockDim.x, tau = threadIdx.x;
    const int lane = tau & 63, wv = tau >> 6;
    const int G = 1 << (L - K), J = 1 << (L - 2 * K);
    const int WPS = TPS >= 64 ? TPS >> 6 : 1, SEG = TPS >= 64 ? 64 : TPS;
    const float scale = args.scale, inv_scale = 1.0f / scale;
    float* mr = lds;

    Owner<K, V, SPT, REG> own;
    own.init(args.cb, L, TPS);

    // tape: the R~ rows and the Q^ rows (TapeRows each), [n] normalisers N_t, [n] offsets K_{t-1} (true
    // Q_t = Q^_t + K_{t-1}), the per-wave (S0, S1[V], S2, S3[V]) of every step, the codebook accumulator (GC), then
    // (checkpoint mode) the [n] per-step Q input offsets and each thread's share of the two backward messages while a
    // segment is recomputed, then (QG) the Q^ message buffer
    const uint32_t slot_bytes = (uint32_t)args.slot_bytes;
    const rsrc_t tape = make_rsrc(args.ws + (size_t)blockIdx.x * args.slot_bytes, slot_bytes);
    const uint32_t row_bytes = (uint32_t)G * 4u;
    const int ck = CK ? args.ckpt : 0;   // a compile-time 0 keeps the full-tape kernels free of the recompute
    const TapeRows rows{ck, n, row_bytes, ck ? (uint32_t)(n / ck + 1) * row_bytes : 0u};
    const uint32_t q_base = (uint32_t)align256(TapeRows::rows(ck, n) * G * 4);
    const uint32_t nrm_base = 2u * q_base;
    const uint32_t kq_base = nrm_base + (uint32_t)align256((size_t)n * 4);
    const uint32_t part_base = kq_base + (uint32_t)align256((size_t)n * 4);
    const uint32_t v_j0 = 4u * (uint32_t)own.j(0);   // lane part of a backward group's tape offset
    // tape offset of backward group j(m) + J a: a lane part (VGPR) and a uniform part, or all of it in the VGPR when
    // the row is tile-major
    auto grp_voff = [&](int m, int a) -> uint32_t {
        if constexpr (NI > 1) return 4u * own.tpos((uint32_t)(own.j(m) + J * a), (uint32_t)G);
        else return v_j0;
    };
    auto grp_soff = [&](int m, int a) -> uint32_t {
        if constexpr (NI > 1) return 0u;
        else return 4u * (uint32_t)(own.j(m) - own.j(0) + J * a);
    };
    typename Owner<K, V, SPT, REG>::Ring cnx;          // the next codebook rows (read from memory)
    own.fwd_prime(cnx);
    // the codebook-gradient accumulator of the slot: c(s, v) at acc_base + 4 (s V + v), so a tile row's entries are
    // contiguous like its codebook values
    const uint32_t acc_base = part_base + (WPS > 1 ? (uint32_t)align256((size_t)n * WPS * NS * 4) : 0u);
    // and (boundary-state mode) each state's two pending contributions of the last step, P1 = f e [g + (2/T)(w - c)
    // (E[F | s] - E[F])] and P2 = f e (2/T)(c - w), folded in during the next step as (P1 + m2 P2) / S0: there the
    // posterior is nearly frozen, each step is divided by its own exact total (the forced steps near the boundary give
    // log-weights of a hundred or more, whose roundings differ between the two passes and would make the previous
    // step's total misweight the step by up to ~1e-5), and E[F | s] - E[F] is centred by its posterior mean m2 (zero
    // exactly; numerically the rounding its O(1) parts share, which dL/dc would multiply by (2/T)(w - c)), as the
    // weights' gradient is through its covariance
    const uint32_t pend_base = acc_base + (uint32_t)align256(((size_t)V * 4) << L);
    const uint32_t pend2_base = pend_base + (uint32_t)align256(((size_t)V * 4) << L);
    const uint32_t kin_base = acc_base + (GC ? 3u * (uint32_t)align256(((size_t)V * 4) << L) : 0u);
    const bool exact = GC && (args.sigma_enum || args.sigma != nullptr);
    const uint32_t save_base = kin_base + (uint32_t)align256((size_t)n * 4);
    float* mq;
    if constexpr (QG) {
        const uint32_t qmsg_base = ck ? save_base + (uint32_t)align256((size_t)2 * G * 4) : kin_base;
        mq = reinterpret_cast<float*>(args.ws + (size_t)blockIdx.x * args.slot_bytes + qmsg_base);
    } else {
        mq = lds + G;
    }
    auto bar = [&]() {   // a step barrier: LDS only, or global memory too when Q^ is in the workspace
        if constexpr (QG) __syncthreads();
        else lds_barrier();
    };
    using RT = typename std::conditional<GC, double, float>::type;   // running normaliser sums
    const float kap = args.two_over_T * inv_scale;   // (2/T) (w - c) = -kap d with d in scaled units
    if constexpr (GC) {
        float z[ROW];
#pragma unroll
        for (int x = 0; x < ROW; ++x) z[x] = 0.f;
#pragma unroll
        for (int m = 0; m < BPT; ++m)
#pragma unroll
            for (int a = 0; a < P; ++a)
#pragma unroll
                for (int q = 0; q < NI; ++q) {
                    st_row<ROW>(z, tape, acc_base + own.row_bytes(m, a, q));
                    if (exact) {
                        st_row<ROW>(z, tape, pend_base + own.row_bytes(m, a, q));
                        st_row<ROW>(z, tape, pend2_base + own.row_bytes(m, a, q));
                    }
                }
    }

    for (int64_t b = blockIdx.x; b < args.B; b += gridDim.x) {
        if (b != blockIdx.x) own.fwd_prime(cnx);   // the backward pass left the ring in its own order
        const int64_t row = args.sigma_enum ? (b >> L) : b;   // the weights' row (sigma enumeration: v >> L)
        const float* wb = args.w + row * (int64_t)n * V;
        const float* gb = args.g + row * (int64_t)n * V;
        const bool has_sigma = args.sigma_enum || args.sigma != nullptr;
        const uint32_t sig = args.sigma_enum ? (uint32_t)(b & ((1 << L) - 1))
                                             : has_sigma ? ((uint32_t)args.sigma[b] & ((1u << L) - 1u)) : 0u;

        // ------------------------------------------------------------------ forward: R~ and Q
#pragma unroll
        for (int m = 0; m < BPT; ++m)
#pragma unroll
            for (int q = 0; q < NI; ++q) {
                float r[TI], z[TI];
                const int u0 = own.fgroup(m, q);
#pragma unroll
                for (int ii = 0; ii < TI; ++ii) {
                    r[ii] = (!has_sigma || (uint32_t)(u0 + ii) == (sig & (uint32_t)(G - 1))) ? 0.f : kNeg;
                    z[ii] = 0.f;
                }
                st_floats<TI>(r, mr, mpos<K>(u0, J), tape, 4u * own.tpos(u0, G), 0u);
                st_floats<TI>(z, mq, mpos<K>(u0, J), tape, 4u * own.tpos(u0, G), q_base);
            }
        bar();

        // One forward step t: R~_{t+1} and Q^_{t+1} from R~_t and Q^_t - kqt, normalised by Nt, into LDS (inputs read
        // before a barrier, outputs written in place) and into the tape at row_soff when `store`.  Returns this
        // thread's maximum of R~_{t+1} and the Q^ of the group attaining it.  The checkpoint recompute runs it again
        // with the stored Nt and kqt, so the recomputed rows are bit-identical to the first pass's.
        auto fwd_step = [&](int tt, float Nt, float kqt, uint32_t row_soff, bool store, float& lmax, float& lq) {
            float rin[BPT][P], qin[BPT][P];
#pragma unroll
            for (int m = 0; m < BPT; ++m)
#pragma unroll
                for (int a = 0; a < P; ++a) {
                    rin[m][a] = mr[mpos<K>(own.j(m), J) + J * a];
                    qin[m][a] = mq[mpos<K>(own.j(m), J) + J * a] - kqt;
                }
            bar();   // every input read before any output overwrites it
            float wt[V], gt[V];
#pragma unroll
            for (int v = 0; v < V; ++v) {
                wt[v] = wb[tt * V + v] * scale;
                gt[v] = gb[tt * V + v] * inv_scale;
            }
            lmax = -3.0e38f;
            lq = 0.f;
#pragma unroll
            for (int m = 0; m < BPT; ++m)
#pragma unroll
                for (int q = 0; q < NI; ++q) {
                    float mx[TI], s[TI], sz[TI];
#pragma unroll
                    for (int r = 0; r < NA; ++r) {
                        float x[TA][TI], z[TA][TI];
#pragma unroll
                        for (int aa = 0; aa < TA; ++aa) {
                            const int a = r * TA + aa;
                            float c[ROW];
                            own.take_fwd(m, a, q, c, cnx);
#pragma unroll
                            for (int ii = 0; ii < TI; ++ii) {
                                float acc = rin[m][a], zz = qin[m][a];
#pragma unroll
                                for (int v = 0; v < V; ++v) {
                                    const float d = fmaf(c[ii * V + v], scale, -wt[v]);
                                    acc = fmaf(-d, d, acc);
                                    zz = fmaf(gt[v], d, zz);
                                }
                                x[aa][ii] = acc;
                                z[aa][ii] = zz;
                            }
                        }
#pragma unroll
                        for (int ii = 0; ii < TI; ++ii) {
                            float cm = x[0][ii];
#pragma unroll
                            for (int aa = 1; aa < TA; ++aa) cm = fmaxf(cm, x[aa][ii]);
                            float cs = 0.f, cz = 0.f;
#pragma unroll
                            for (int aa = 0; aa < TA; ++aa) {
                                const float e = ex2(x[aa][ii] - cm);
                                cs += e;
                                cz = fmaf(e, z[aa][ii], cz);
                            }
                            if (r == 0) {
                                mx[ii] = cm;
                                s[ii] = cs;
                                sz[ii] = cz;
                            } else {
                                lse_merge(mx[ii], s[ii], sz[ii], cm, cs, cz);
                            }
                        }
                        GEN_SCHED_BARRIER();
                    }
                    float ro[TI], qo[TI];
#pragma unroll
                    for (int ii = 0; ii < TI; ++ii) {
                        ro[ii] = (mx[ii] - Nt) + lg2(s[ii]);
                        qo[ii] = sz[ii] * rcp(s[ii]);
                        const bool up = ro[ii] > lmax;
                        lmax = up ? ro[ii] : lmax;
                        lq = up ? qo[ii] : lq;
                    }
                    const int u0 = own.fgroup(m, q);
                    st_floats<TI>(ro, mr, mpos<K>(u0, J), tape, 4u * own.tpos(u0, G), row_soff, store);
                    st_floats<TI>(qo, mq, mpos<K>(u0, J), tape, 4u * own.tpos(u0, G), q_base + row_soff, store);
                }
        };

        double A = 0.0;
        float N = 0.f, kq = 0.f, Kq = 0.f, N_last = 0.f, K_last = 0.f;
        for (int t = 0; t < n; ++t) {
            if (tau == 0) {
                buf_st(N, tape, 0u, nrm_base + 4u * t);
                buf_st(Kq, tape, 0u, kq_base + 4u * t);
                if (ck) buf_st(kq, tape, 0u, kin_base + 4u * t);
            }
            K_last = Kq;
            Kq += kq;
            float lmax, lq;
            fwd_step(t, N, kq, rows.off(t + 1), rows.stored(t + 1), lmax, lq);
            gseq_argmax_payload(lmax, lq, SEG);
            if (WPS > 1 && lane == 0) {
                redmax[t & 1][wv] = lmax;
                redq[t & 1][wv] = lq;
            }
            bar();
            if (WPS > 1) {
                const int qs = lane & 15;
                float bm = qs < WPS ? redmax[t & 1][qs] : -3.0e38f;
                float bq = qs < WPS ? redq[t & 1][qs] : 0.f;
                row16_argmax_payload(bm, bq);   // the first wave attaining the maximum
                lmax = bm;
                lq = bq;
            }
            lmax = uniform_f(lmax);
            lq = uniform_f(lq);
            A += (double)N;
            N_last = N;
            N = lmax;
            kq = grid_offset(lq);
        }
        // rz = log2 Z - A_n, and E[F], which centres the covariance of the backward pass
        float rz, EF, Kfin;   // E[F] = Kfin + EF: the offsets' exact sum, and the centred rest
        RT rzr;   // rz in the precision of the running sums
        if (!has_sigma) {
            float z0 = 0.f, z1 = 0.f;
#pragma unroll
            for (int m = 0; m < BPT; ++m)
#pragma unroll
                for (int q = 0; q < NI; ++q)
#pragma unroll
                    for (int ii = 0; ii < TI; ++ii) {
                        const int u = own.fgroup(m, q) + ii;
                        const float p = ex2(mr[mpos<K>(u, J)] - N);
                        z0 += p;
                        z1 = fmaf(p, mq[mpos<K>(u, J)], z1);
                    }
            z0 = gseq_sum(z0, SEG);
            z1 = gseq_sum(z1, SEG);
            if (WPS > 1 && lane == 0) {
                reds[n & 1][wv][0] = z0;
                reds[n & 1][wv][1] = z1;
            }
            bar();
            if (WPS > 1) {
                z0 = 0.f;
                z1 = 0.f;
                for (int q = 0; q < WPS; ++q) {
                    z0 += reds[n & 1][q][0];
                    z1 += reds[n & 1][q][1];
                }
            }
            rz = N + lg2(z0);
            rzr = (RT)N + (RT)lg2(z0);
            EF = z1 / z0;   // the final Q^_n carries the offset K_{n-1}
            Kfin = Kq;
            __syncthreads();
        } else {
            __syncthreads();   // R~_{n-1} and Q^_{n-1} are on the tape, written by other threads
            const float r = buf_ld_nt(tape, 0u, rows.off(n - 1) + 4u * own.tpos(sig >> K, G));
            const float qv = buf_ld_nt(tape, 0u, q_base + rows.off(n - 1) + 4u * own.tpos(sig >> K, G));
            float x = r;
            EF = qv;   // Q^_{n-1} carries the offset K_{n-2}
            Kfin = K_last;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const float d = fmaf(args.cb[sig * V + v], scale, -(wb[(n - 1) * V + v] * scale));
                x = fmaf(-d, d, x);
                EF = fmaf(gb[(n - 1) * V + v] * inv_scale, d, EF);
            }
            rz = (r < 0.5f * kNeg) ? kNeg : x - N_last;
            rzr = (r < 0.5f * kNeg) ? (RT)kNeg : (RT)x - (RT)N_last;
        }
        const bool valid = rz > 0.5f * kNeg;

        // ------------------------------------------------------------------ backward: B~ and P, covariance
        float Nb = 0.f;
        RT C_ = 0, D = 0;
        float lam = 1.f;  // 1 / (posterior total of the previous step), GC only
        float m2p = 0.f;  // E[E[F | s] - E[F]] of the previous step, boundary-state GC only
        float kb = 0.f;   // kappa_{t+1}, subtracted from the P inputs
        float H = 0.f;    // sum of the kappas of the steps after t
        int t = n - 1;
        if (!has_sigma) {
#pragma unroll
            for (int m = 0; m < BPT; ++m)
#pragma unroll
                for (int q = 0; q < NI; ++q)
#pragma unroll
                    for (int ii = 0; ii < TI; ++ii) {
                        const int u = own.fgroup(m, q) + ii;
                        mr[mpos<K>(u, J)] = 0.f;
                        mq[mpos<K>(u, J)] = 0.f;
                    }
        } else {
            // s_n = sigma: the posterior at n-1 is the indicator of sigma (grad_{n-1} = 0, w_soft_{n-1} = c(sigma));
            // the messages left are B_{n-2}(sigma >> k) = theta_{n-1}(sigma) and P_{n-2}(sigma >> k) = <g, c - w>,
            // which is kappa_{n-1} as well.  theta goes into the offset C_ and the message starts at 0, so the next
            // step's branch terms are not rounded at theta's magnitude (a hundred or more in log2 units)
            float th = 0.f, pz = 0.f;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const float d = fmaf(args.cb[sig * V + v], scale, -(wb[(n - 1) * V + v] * scale));
                th = fmaf(-d, d, th);
                pz = fmaf(gb[(n - 1) * V + v] * inv_scale, d, pz);
            }
#pragma unroll
            for (int m = 0; m < BPT; ++m)
#pragma unroll
                for (int q = 0; q < NI; ++q)
#pragma unroll
                    for (int ii = 0; ii < TI; ++ii) {
                        const uint32_t u = (uint32_t)(own.fgroup(m, q) + ii);
                        mr[mpos<K>((int)u, J)] = (u == (sig >> K)) ? 0.f : kNeg;
                        mq[mpos<K>((int)u, J)] = (u == (sig >> K)) ? pz : 0.f;
                    }
            if (tau == 0) {
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    if (!GC || args.grad) args.grad[(b * n + n - 1) * V + v] = valid ? 0.f : __builtin_nanf("");
                    if (args.w_soft)
                        args.w_soft[(b * n + n - 1) * V + v] = valid ? args.cb[sig * V + v] : __builtin_nanf("");
                }
            }
            if constexpr (GC) {
                // p_{n-1} is the indicator of sigma and E[F | s_{n-1}] = E[F]: dL/dc(sigma, v) += g_{n-1,v}, added by
                // the thread that owns sigma (it alone touches that entry)
                const uint32_t js = (sig >> K) & (uint32_t)(J - 1), is = sig & (uint32_t)(P - 1);
                const uint32_t owner = C == 1 ? js % (uint32_t)TPS : js * C + is / I;
                if (valid && (uint32_t)tau == owner) {
#pragma unroll
                    for (int v = 0; v < V; ++v) {
                        const uint32_t o = acc_base + 4u * (sig * V + v);
                        buf_st(buf_ld(tape, 0u, o) + gb[(n - 1) * V + v], tape, 0u, o);
                    }
                }
            }
            D = N_last;
            C_ = (RT)th;
            kb = grid_offset(pz);
            H = kb;
            t = n - 2;
        }
        bar();

        const int t_out = t;
        // the accumulator row of the next unit (GC), one unit ahead, wrapping to the next step's first
        float acn[GC ? ROW : 1], pen[GC ? ROW : 1], pfn[GC ? ROW : 1];
        auto acc_next = [&](int idx, float* nx, float* np, float* nf) {
            if constexpr (GC) {
                const int x = (idx + 1) % (BPT * P * NI);
                const uint32_t o = own.row_bytes(x / (NI * P), (x / NI) % P, x % NI);
                ld_floats<ROW>(tape, acc_base + o, nx);
                if (exact) {
                    ld_floats<ROW>(tape, pend_base + o, np);
                    ld_floats<ROW>(tape, pend2_base + o, nf);
                }
            }
        };
        acc_next(-1, acn, pen, pfn);
        float N_nx = 0.f, K_nx = 0.f, rt_nx = 0.f, qt_nx = 0.f;
        if (t >= 0) {
            N_nx = buf_ld_nt(tape, 0u, nrm_base + 4u * t);
            K_nx = buf_ld_nt(tape, 0u, kq_base + 4u * t);
            rt_nx = buf_ld_nt(tape, grp_voff(0, 0), rows.off(t) + grp_soff(0, 0));
            qt_nx = buf_ld_nt(tape, grp_voff(0, 0), q_base + rows.off(t) + grp_soff(0, 0));
        }
        own.bwd_prime(cnx);
        while (t >= 0) {
        const int t0 = ck ? (t / ck) * ck : 0;   // first step of this segment
        if (ck) {
            // checkpoint mode: keep this thread's share of both backward messages in the workspace, rebuild R~ and
            // Q^ of steps t0+1..t from checkpoint t0 with the stored normalisers and offsets, then restore them
#pragma unroll
            for (int m = 0; m < BPT; ++m)
#pragma unroll
                for (int q = 0; q < NI; ++q) {
                    const int u0 = own.fgroup(m, q);
                    st_row<TI>(mr + mpos<K>(u0, J), tape, save_base + 4u * u0);
                    st_row<TI>(mq + mpos<K>(u0, J), tape, save_base + row_bytes + 4u * u0);
                }
            bar();   // every share read before the recompute overwrites the buffers
#pragma unroll
            for (int m = 0; m < BPT; ++m)
#pragma unroll
                for (int q = 0; q < NI; ++q) {
                    const int u0 = own.fgroup(m, q);
                    ld_to_lds<TI>(mr, mpos<K>(u0, J), tape, 4u * own.tpos(u0, G), rows.off(t0));
                    ld_to_lds<TI>(mq, mpos<K>(u0, J), tape, 4u * own.tpos(u0, G), q_base + rows.off(t0));
                }
            bar();
            own.fwd_prime(cnx);
            for (int tt = t0; tt < t; ++tt) {
                const float Nr = uniform_f(buf_ld(tape, 0u, nrm_base + 4u * tt));
                const float kr = uniform_f(buf_ld(tape, 0u, kin_base + 4u * tt));
                float lm, lqr;
                fwd_step(tt, Nr, kr, rows.off(tt + 1), true, lm, lqr);
                bar();
            }
            own.bwd_prime(cnx);
            __syncthreads();   // the recomputed rows, written by other threads, before the backward reads them
#pragma unroll
            for (int m = 0; m < BPT; ++m)
#pragma unroll
                for (int q = 0; q < NI; ++q) {
                    const int u0 = own.fgroup(m, q);
                    ld_to_lds<TI>(mr, mpos<K>(u0, J), tape, save_base + 4u * u0, 0u);
                    ld_to_lds<TI>(mq, mpos<K>(u0, J), tape, save_base + row_bytes + 4u * u0, 0u);
                }
            bar();
            rt_nx = buf_ld_nt(tape, grp_voff(0, 0), rows.off(t) + grp_soff(0, 0));
            qt_nx = buf_ld_nt(tape, grp_voff(0, 0), q_base + rows.off(t) + grp_soff(0, 0));
        }
        for (; t >= t0; --t) {
            float bin[BPT][I], pin[BPT][I];
#pragma unroll
            for (int m = 0; m < BPT; ++m)
#pragma unroll
                for (int q = 0; q < NI; ++q)
#pragma unroll
                    for (int ii = 0; ii < TI; ++ii) {
                        const int u = mpos<K>(own.fgroup(m, q), J) + ii;
                        bin[m][TI * q + ii] = mr[u];
                        pin[m][TI * q + ii] = mq[u] - kb;
                    }
            bar();
            float wt[V], gt[V], gnat[V];
#pragma unroll
            for (int v = 0; v < V; ++v) {
                wt[v] = wb[t * V + v] * scale;
                gnat[v] = gb[t * V + v];
                gt[v] = gnat[v] * inv_scale;
            }
            const float Nt = uniform_f(N_nx), Kt = uniform_f(K_nx);
            if (t > 0) {
                N_nx = buf_ld_nt(tape, 0u, nrm_base + 4u * (t - 1));
                K_nx = buf_ld_nt(tape, 0u, kq_base + 4u * (t - 1));
            }
            const uint32_t row_t = rows.off(t), row_prev = rows.off(t > 0 ? t - 1 : 0);
            D += (RT)Nt;
            const float ref = (float)(((RT)rzr + D) - C_);
            // E[F | s_t = s] - E[F] = Q^_t(s >> k) + cst + <g_t, c(s) - w_t> + P''_t(s & (G-1)), cst per step
            const float brk = (Kt - Kfin) + H;   // exact (offsets on the 2^-6 grid)
            const float cst = brk - EF;
            float lmax = -3.0e38f, S0 = 0.f, S2 = 0.f, S1[V], S3[V];
#pragma unroll
            for (int v = 0; v < V; ++v) {
                S1[v] = 0.f;
                S3[v] = 0.f;
            }
#pragma unroll
            for (int m = 0; m < BPT; ++m)
#pragma unroll
                for (int a = 0; a < P; ++a) {
                    const int vg = own.j(m) + J * a;   // backward group of row a
                    // R~_t and Q^_t of this group; the next group's (or the next step's first) one row ahead
                    const float rt = rt_nx;
                    const float qt = qt_nx + cst;
                    const float qs = qt_nx - EF;   // GC: the small parts of E[F | s] - E[F]
                    if (m * P + a + 1 < BPT * P) {
                        const int m2 = (m * P + a + 1) / P, a2 = (m * P + a + 1) % P;
                        const uint32_t so = row_t + grp_soff(m2, a2);
                        rt_nx = buf_ld_nt(tape, grp_voff(m2, a2), so);
                        qt_nx = buf_ld_nt(tape, grp_voff(m2, a2), q_base + so);
                    } else {   // the next step's first (a harmless re-read of row 0 at t = 0; in checkpoint mode
                               // re-read after the next segment is rebuilt)
                        const uint32_t so = row_prev + grp_soff(0, 0);
                        rt_nx = buf_ld_nt(tape, grp_voff(0, 0), so);
                        qt_nx = buf_ld_nt(tape, grp_voff(0, 0), q_base + so);
                    }
                    float mx = 0.f, s = 0.f, sez = 0.f;
#pragma unroll
                    for (int q = 0; q < NI; ++q) {
                        float c[ROW], y[TI], z[TI], d[TI][V];
                        own.take_bwd(m, a, q, c, cnx);
#pragma unroll
                        for (int ii = 0; ii < TI; ++ii) {
                            float acc = bin[m][TI * q + ii], zz = pin[m][TI * q + ii];
#pragma unroll
                            for (int v = 0; v < V; ++v) {
                                d[ii][v] = fmaf(c[ii * V + v], scale, -wt[v]);
                                acc = fmaf(-d[ii][v], d[ii][v], acc);
                                zz = fmaf(gt[v], d[ii][v], zz);
                            }
                            y[ii] = acc;
                            z[ii] = zz;
                        }
                        float cm = y[0];
#pragma unroll
                        for (int ii = 1; ii < TI; ++ii) cm = fmaxf(cm, y[ii]);
                        if constexpr (C > 1) cm = quad_max(cm);
                        float cs = 0.f, ez = 0.f, er = 0.f, ed[V], edr[V], e[TI], r[TI];
#pragma unroll
                        for (int v = 0; v < V; ++v) {
                            ed[v] = 0.f;
                            edr[v] = 0.f;
                        }
#pragma unroll
                        for (int ii = 0; ii < TI; ++ii) {
                            e[ii] = ex2(y[ii] - cm);
                            // E[F | s] - E[F], formed before any product: its parts nearly cancel at the likely
                            // states, and multiplying them separately would keep their rounding
                            if constexpr (GC) {
                                // dL/dc weighs it by (2/T)(w - c) state by state, so at a frozen posterior the
                                // roundings of its O(1) parts (<g_t, c - w> at the likely state and the offsets'
                                // bracket, which cancel there) would survive: join them before any rounding (one
                                // fma; for V > 1 a float64 chain, exact for these products) and add the small parts
                                const float small = pin[m][TI * q + ii] + qs;
                                if constexpr (V == 1) {
                                    r[ii] = fmaf(gt[0], d[ii][0], brk) + small;
                                } else {
                                    double rr = (double)brk;
#pragma unroll
                                    for (int v = 0; v < V; ++v) rr = __builtin_fma((double)gt[v], (double)d[ii][v], rr);
                                    r[ii] = (float)(rr + (double)small);
                                }
                            } else {
                                r[ii] = z[ii] + qt;
                            }
                            cs += e[ii];
                            ez = fmaf(e[ii], z[ii], ez);
                            er = fmaf(e[ii], r[ii], er);
#pragma unroll
                            for (int v = 0; v < V; ++v) {
                                const float edv = e[ii] * d[ii][v];
                                ed[v] += edv;
                                edr[v] = fmaf(edv, r[ii], edr[v]);
                            }
                        }
                        const float f = ex2((cm + rt) - ref);
                        if constexpr (GC) {
                            // p_t(s) [g_{t,v} + (2/T)(w_{t,v} - c(s, v)) (E[F | s] - E[F])] with p_t(s) = lam f e
                            float ac[ROW], pe[ROW], pf[ROW];
#pragma unroll
                            for (int x = 0; x < ROW; ++x) {
                                ac[x] = acn[x];
                                pe[x] = pen[x];
                                pf[x] = pfn[x];
                            }
                            acc_next((m * P + a) * NI + q, acn, pen, pfn);
                            if (exact) {
                                // the previous step's pending sums join the accumulator, centred by that step's m2 and
                                // divided by its total (lam); this step's wait
                                const float ka = f * kap;
#pragma unroll
                                for (int ii = 0; ii < TI; ++ii)
#pragma unroll
                                    for (int v = 0; v < V; ++v) {
                                        const int x = ii * V + v;
                                        ac[x] = fmaf(lam, fmaf(m2p, pf[x], pe[x]), ac[x]);
                                        const float ed = e[ii] * d[ii][v];
                                        pe[x] = fmaf(f * gnat[v], e[ii], -ka * (ed * r[ii]));
                                        pf[x] = ka * ed;
                                    }
                                st_row<ROW>(ac, tape, acc_base + own.row_bytes(m, a, q));
                                st_row<ROW>(pe, tape, pend_base + own.row_bytes(m, a, q));
                                st_row<ROW>(pf, tape, pend2_base + own.row_bytes(m, a, q));
                            } else {
                                const float fa = lam * f, ka = fa * kap;
#pragma unroll
                                for (int ii = 0; ii < TI; ++ii)
#pragma unroll
                                    for (int v = 0; v < V; ++v)
                                        ac[ii * V + v] = fmaf(fa * gnat[v], e[ii],
                                                              fmaf(-ka, e[ii] * d[ii][v] * r[ii], ac[ii * V + v]));
                                st_row<ROW>(ac, tape, acc_base + own.row_bytes(m, a, q));
                            }
                        }
                        S0 = fmaf(f, cs, S0);
                        S2 = fmaf(f, er, S2);
#pragma unroll
                        for (int v = 0; v < V; ++v) {
                            S1[v] = fmaf(f, ed[v], S1[v]);
                            S3[v] = fmaf(f, edr[v], S3[v]);
                        }
                        if constexpr (C > 1) {
                            cs = quad_sum(cs);
                            ez = quad_sum(ez);
                        }
                        if (q == 0) {
                            mx = cm;
                            s = cs;
                            sez = ez;
                        } else {
                            lse_merge(mx, s, sez, cm, cs, ez);
                        }
                    }
                    const float out = (mx - Nb) + lg2(s);
                    lmax = run_max(lmax, out);
                    // the lanes of a quad store the same values; at t = 0 nobody reads them
                    mr[mpos<K>(own.j(m), J) + J * a] = out;
                    mq[mpos<K>(own.j(m), J) + J * a] = sez * rcp(s);
                    pin_order(S0, S2, lmax);
#pragma unroll
                    for (int v = 0; v < V; ++v) pin_order(S1[v], S3[v]);
                    GEN_SCHED_BARRIER();
                }
            lmax = gseq_max(lmax, SEG);
            float Sv[NS];
            Sv[0] = gseq_sum(S0, SEG);
            Sv[1 + V] = gseq_sum(S2, SEG);
#pragma unroll
            for (int v = 0; v < V; ++v) {
                Sv[1 + v] = gseq_sum(S1[v], SEG);
                Sv[2 + V + v] = gseq_sum(S3[v], SEG);
            }
            if (WPS > 1 && lane == 0) {
                redmax[t & 1][wv] = lmax;
#pragma unroll
                for (int x = 0; x <= V + 1; ++x) reds[t & 1][wv][x] = Sv[x];   // S0, S1[V], S2
                const uint32_t po = part_base + 4u * (uint32_t)((t * WPS + wv) * NS);
#pragma unroll
                for (int x = 0; x < NS; ++x) buf_st(Sv[x], tape, 0u, po + 4u * x);
            }
            bar();
            float m1[V];   // w_soft_t - w_t per component, in scaled codebook units
            if (WPS > 1) {
                const int qs = lane & 15;
                lmax = row16_max(qs < WPS ? redmax[t & 1][qs] : -3.0e38f);
                // only the P offset uses m1 here, and any value common to the sequence serves
                const float s0b = row16_sum(qs < WPS ? reds[t & 1][qs][0] : 0.f);
#pragma unroll
                for (int v = 0; v < V; ++v) m1[v] = row16_sum(qs < WPS ? reds[t & 1][qs][1 + v] : 0.f) * rcp(s0b);
                if constexpr (GC) lam = uniform_f(rcp(s0b));
                if constexpr (GC) m2p = uniform_f(row16_sum(qs < WPS ? reds[t & 1][qs][1 + V] : 0.f) * rcp(s0b));
            } else {
#pragma unroll
                for (int v = 0; v < V; ++v) m1[v] = Sv[1 + v] * (1.0f / Sv[0]);
                if constexpr (GC) lam = uniform_f(1.0f / Sv[0]);
                if constexpr (GC) m2p = uniform_f(Sv[1 + V] * (1.0f / Sv[0]));
                if (tau == 0) {
                    const float i0 = 1.0f / Sv[0];
                    const float m2 = Sv[1 + V] * i0;
#pragma unroll
                    for (int v = 0; v < V; ++v) {
                        const float cov = fmaf(-m1[v], m2, Sv[2 + V + v] * i0);
                        if (!GC || args.grad)
                            args.grad[(b * n + t) * V + v] = valid ? args.two_over_T * cov * inv_scale
                                                                   : __builtin_nanf("");
                        if (args.w_soft)
                            args.w_soft[(b * n + t) * V + v] = valid ? fmaf(m1[v], inv_scale, wb[t * V + v])
                                                                     : __builtin_nanf("");
                    }
                }
            }
            float kap = 0.f;
#pragma unroll
            for (int v = 0; v < V; ++v) kap = fmaf(gt[v], m1[v], kap);
            kb = grid_offset(uniform_f(kap));
            lmax = uniform_f(lmax);
            H += kb;
            C_ += (RT)Nb;
            Nb = lmax;
        }
        }   // segments
        if (WPS > 1) {
            __syncthreads();   // the per-wave partial sums, written by other waves
            for (int tt = tau; tt <= t_out; tt += TPS) {
                float Sv[NS];
#pragma unroll
                for (int x = 0; x < NS; ++x) Sv[x] = 0.f;
                for (int q = 0; q < WPS; ++q) {
                    const uint32_t po = part_base + 4u * (uint32_t)((tt * WPS + q) * NS);
#pragma unroll
                    for (int x = 0; x < NS; ++x) Sv[x] += buf_ld(tape, 0u, po + 4u * x);
                }
                const float i0 = 1.0f / Sv[0];
                const float m2 = Sv[1 + V] * i0;
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    const float m1 = Sv[1 + v] * i0;
                    const float cov = fmaf(-m1, m2, Sv[2 + V + v] * i0);
                    if (!GC || args.grad)
                        args.grad[(b * n + tt) * V + v] = valid ? args.two_over_T * cov * inv_scale
                                                                : __builtin_nanf("");
                    if (args.w_soft)
                        args.w_soft[(b * n + tt) * V + v] = valid ? fmaf(m1, inv_scale, wb[tt * V + v]) : __builtin_nanf("");
                }
            }
        }
        if constexpr (GC) {
            if (exact) {   // the last step's pending sums; the pending arrays left at zero
                float z[ROW];
#pragma unroll
                for (int i = 0; i < ROW; ++i) z[i] = 0.f;
#pragma unroll
                for (int m = 0; m < BPT; ++m)
#pragma unroll
                    for (int a = 0; a < P; ++a)
#pragma unroll
                        for (int q = 0; q < NI; ++q) {
                            const uint32_t o = own.row_bytes(m, a, q);
                            float ac[ROW], pe[ROW], pf[ROW];
                            ld_floats<ROW>(tape, acc_base + o, ac);
                            ld_floats<ROW>(tape, pend_base + o, pe);
                            ld_floats<ROW>(tape, pend2_base + o, pf);
#pragma unroll
                            for (int i = 0; i < ROW; ++i) ac[i] = fmaf(lam, fmaf(m2p, pf[i], pe[i]), ac[i]);
                            st_row<ROW>(ac, tape, acc_base + o);
                            st_row<ROW>(z, tape, pend_base + o);
                            st_row<ROW>(z, tape, pend2_base + o);
                        }
            }
            if (!valid) {   // no admissible path: the loss, hence its gradient, is undefined
                float x[ROW];
#pragma unroll
                for (int i = 0; i < ROW; ++i) x[i] = __builtin_nanf("");
#pragma unroll
                for (int m = 0; m < BPT; ++m)
#pragma unroll
                    for (int a = 0; a < P; ++a)
#pragma unroll
                        for (int q = 0; q < NI; ++q) st_row<ROW>(x, tape, acc_base + own.row_bytes(m, a, q));
            }
        }
        __syncthreads();   // the next sequence reuses the tape and LDS
    }
}

// ------------------------------------------------------------------------------------------------------------------
// host-side launch

namespace {

using GenKernel = void (*)(GenArgs);

template <int K, int V, int SPT, int LT>
GenKernel pick(int op, bool ck, int nsq, bool qg) {
    switch (op) {
        case 0: return gen_soft_kernel<K, V, SPT, LT>;
        case 1:
        case 3:
            if (qg) {   // Q^ in the workspace: instantiated where it is needed, k = 1 at L = 16
                if constexpr (K == 1 && LT == 16) {
                    if (op == 1) return ck ? gen_grad_kernel<K, V, SPT, LT, false, true, true>
                                           : gen_grad_kernel<K, V, SPT, LT, false, false, true>;
                    return ck ? gen_grad_kernel<K, V, SPT, LT, true, true, true>
                              : gen_grad_kernel<K, V, SPT, LT, true, false, true>;
                }
                return nullptr;
            }
            if (op == 1) return ck ? gen_grad_kernel<K, V, SPT, LT, false, true, false>
                                   : gen_grad_kernel<K, V, SPT, LT, false, false, false>;
            return ck ? gen_grad_kernel<K, V, SPT, LT, true, true, false>
                      : gen_grad_kernel<K, V, SPT, LT, true, false, false>;
        default:
            if constexpr (V == 2 && SPT == 64) {   // the codebook streams: two sequences per workgroup share it
                if (nsq == 2) return gen_viterbi_kernel<K, V, SPT, LT, 2>;
            }
            return nsq == 1 ? gen_viterbi_kernel<K, V, SPT, LT, 1> : nullptr;
    }
}

// L = 16 (the workloads' trellis) has its own instantiation, whose strides are compile-time; other L read it at run
// time.
template <int V, int SPT>
GenKernel pick_k(int op, bool ck, int nsq, bool qg, int k, int L) {
    if constexpr (SPT < 64) {
        switch (k) {
            case 1: return pick<1, V, SPT, 0>(op, ck, nsq, qg);
            case 2: return pick<2, V, SPT, 0>(op, ck, nsq, qg);
            default: return nullptr;
        }
    } else {
        switch (k) {
            case 1: return L == 16 ? pick<1, V, SPT, 16>(op, ck, nsq, qg) : pick<1, V, SPT, 0>(op, ck, nsq, qg);
            case 2: return L == 16 ? pick<2, V, SPT, 16>(op, ck, nsq, qg) : pick<2, V, SPT, 0>(op, ck, nsq, qg);
            case 3: return L == 16 ? pick<3, V, SPT, 16>(op, ck, nsq, qg) : pick<3, V, SPT, 0>(op, ck, nsq, qg);
            case 4: return L == 16 ? pick<4, V, SPT, 16>(op, ck, nsq, qg) : pick<4, V, SPT, 0>(op, ck, nsq, qg);
            default: return nullptr;
        }
    }
}

template <int V>
GenKernel pick_spt(int op, bool ck, int nsq, bool qg, int k, int L) {
    switch (L) {
        case 4: return pick_k<V, 16>(op, ck, nsq, qg, k, L);
        case 5: return pick_k<V, 32>(op, ck, nsq, qg, k, L);
        default: return pick_k<V, 64>(op, ck, nsq, qg, k, L);
    }
}

}  // namespace

// op: 0 soft, 1 gradient, 2 Viterbi, 3 gradient with the codebook accumulator (summed afterwards by
// launch_codebook_reduce).  The caller has checked 1 <= k <= 4, 2k <= L <= 16, V in {1, 2}.
hipError_t launch_general(int op, int k, int V, const GenArgs& a, int grid, int threads, size_t lds_bytes,
                          hipStream_t st) {
    const bool ck = a.ckpt != 0;
    const int nsq = a.nsq > 1 ? a.nsq : 1;
    const bool qg = a.qg != 0;
    const GenKernel f = V == 1 ? pick_spt<1>(op, ck, nsq, qg, k, a.L) : pick_spt<2>(op, ck, nsq, qg, k, a.L);
    if (f == nullptr) return hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(f), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds_bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(f, dim3(grid), dim3(threads), lds_bytes, st, a);
    return hipGetLastError();
}

}  // namespace bcjr
