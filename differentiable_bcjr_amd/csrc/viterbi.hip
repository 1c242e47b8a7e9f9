// viterbi.hip -- Viterbi hard code (minimum-energy trellis path) on gfx950.
//
// The Viterbi decision is the zero-temperature limit of the Boltzmann path measure that the soft codeword averages
// over (BCJR-QAT, arXiv 2605.10655: abstract; gist.science Technical Summary, "Core Mechanism"), i.e. the QTIP hard
// code.  The path metric is accumulated in IEEE float32 in a fixed order without fused multiply-add, so the decoded
// states are bit-identical to any implementation that follows the same order:
//   V_{t+1}(v) = min_a M_t(v | a << (L-2)),  M_t(s) = fl( fl(d*d) + V_t(s >> 2) ),  d = fl(w_t - c(s)),
// with back pointer bp_{t+1}(v) = the smallest a attaining the min; the end state is the smallest s attaining
// min_s M_{n-1}(s) (or sigma), and the path is traced back through the pointers.
//
// Layout: the same quads as the soft pass (64 states per thread at L = 16, raw codebook values in VGPRs), V messages
// double-buffered in LDS.  Each thread packs its 16 back pointers of a step into one 32-bit word (coalesced store to
// a per-sequence back-pointer tape).  The traceback of a sequence runs in one lane while the block decodes the next
// sequence, one dependent load per step, so its latency hides behind the next forward pass; the tape is
// double-buffered by sequence for that.  Codewords c(s_t) are gathered by the whole block once a path is complete.
//
// The tail-biting hard code with a decoder-chosen start state (s_0 = s_n) reuses this kernel: weights read rotated
// (rotate-and-decode), one virtual sequence per (row, sigma) for the exact choice, and a costs-only mode without
// traceback; tb_select_kernel and tb_rotate_sigma_kernel pick sigma between the passes.
#include "kernel_args.hpp"
#include "trellis.hpp"

namespace bcjr {

namespace {

// IEEE float32 operations that the compiler may not fuse or reorder.
__device__ __forceinline__ float emit_metric(float w, float c, float v) {
#pragma clang fp contract(off)
    const float d = w - c;
    const float e = d * d;
    return e + v;
}

}  // namespace

template <int L>
__global__ void __launch_bounds__(Geo<L>::NT) viterbi_kernel(ViterbiArgs args) {
    using Gm = Geo<L>;
    constexpr int G = Gm::G, Q = Gm::Q, QPT = Gm::QPT, TPS = Gm::TPS, SPB = Gm::SPB, WPS = Gm::WPS;
    constexpr int SEG = Gm::SEG;
    constexpr float kInf = __builtin_huge_valf();
    __shared__ float4 msg4[SPB][2][G / 4];
    __shared__ float redv[SPB][WPS];
    __shared__ uint32_t redi[SPB][WPS];

    const int tid = threadIdx.x;
    const int sq = tid / TPS;
    const int tau = tid % TPS;
    const int lane = tid & 63;
    const int wv = tau >> 6;
    float* msg0 = reinterpret_cast<float*>(&msg4[sq][0][0]);
    float* msg1 = reinterpret_cast<float*>(&msg4[sq][1][0]);
    const int n = args.n;

    float cb[QPT][4][4];
#pragma unroll
    for (int m = 0; m < QPT; ++m) {
        const int j = tau + TPS * m;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const float4 v = *reinterpret_cast<const float4*>(args.cb + (a << (L - 2)) + 4 * j);
            cb[m][a][0] = v.x;
            cb[m][a][1] = v.y;
            cb[m][a][2] = v.z;
            cb[m][a][3] = v.w;
        }
    }

    // back-pointer tape: per sequence slot, 2 buffers (by sequence parity) of [n][TPS] words
    const uint32_t slot_bytes = (uint32_t)args.slot_bytes;
    const rsrc_t tape = make_rsrc(args.ws + (size_t)blockIdx.x * SPB * args.slot_bytes, SPB * slot_bytes);
    const uint32_t buf_bytes = (uint32_t)n * TPS * 4u;
    const uint32_t v_word = sq * slot_bytes + 4u * tau;

    const bool trace = args.states != nullptr;   // costs only otherwise
    const int rot = args.rot;
    // pending traceback (run by the sequence's lane tau == 0)
    int32_t pend_b = -1;
    int pend_t = 0;
    uint32_t pend_s = 0, pend_word = 0, pend_par = 0;

    const int64_t ngroups = (args.B + SPB - 1) / SPB;
    int64_t iter = 0;
    for (int64_t gi = blockIdx.x; gi < ngroups; gi += gridDim.x, ++iter) {
        const int64_t b = gi * SPB + sq;
        const bool active = b < args.B;
        const int64_t bb = active ? b : args.B - 1;
        const float* wb = args.w + (args.sigma_enum ? (bb >> L) : bb) * n;
        const bool has_sigma = args.sigma_enum || args.sigma != nullptr;
        const uint32_t sig = args.sigma_enum ? (uint32_t)(bb & (Gm::S - 1))
                                             : has_sigma ? ((uint32_t)args.sigma[bb] & (uint32_t)(Gm::S - 1)) : 0u;
        const uint32_t par = (uint32_t)(iter & 1);

        // V_0: free start -> 0; sigma -> only the successors of sigma reachable
#pragma unroll
        for (int m = 0; m < QPT; ++m) {
            const int j = tau + TPS * m;
            float4 r;
            r.x = (!has_sigma || (uint32_t)(4 * j + 0) == (sig & (G - 1))) ? 0.f : kInf;
            r.y = (!has_sigma || (uint32_t)(4 * j + 1) == (sig & (G - 1))) ? 0.f : kInf;
            r.z = (!has_sigma || (uint32_t)(4 * j + 2) == (sig & (G - 1))) ? 0.f : kInf;
            r.w = (!has_sigma || (uint32_t)(4 * j + 3) == (sig & (G - 1))) ? 0.f : kInf;
            *reinterpret_cast<float4*>(msg0 + 4 * j) = r;
        }
        lds_barrier();

        for (int t = 0; t + 1 < n; ++t) {
            const float* mc = (t & 1) ? msg1 : msg0;
            float* mn = (t & 1) ? msg0 : msg1;
            const float wt = wb[t + rot < n ? t + rot : t + rot - n];
            uint32_t word = 0;
#pragma unroll
            for (int m = 0; m < QPT; ++m) {
                const int j = tau + TPS * m;
                float v[4];
#pragma unroll
                for (int a = 0; a < 4; ++a) v[a] = mc[j + Q * a];
                float o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float M[4];
#pragma unroll
                    for (int a = 0; a < 4; ++a) M[a] = emit_metric(wt, cb[m][a][i], v[a]);
                    const float mn4 = fminf(fminf(M[0], M[1]), fminf(M[2], M[3]));
                    const uint32_t arg = (M[0] == mn4) ? 0u : (M[1] == mn4) ? 1u : (M[2] == mn4) ? 2u : 3u;
                    word |= arg << (8 * m + 2 * i);
                    o[i] = mn4;
                }
                *reinterpret_cast<float4*>(mn + 4 * j) = make_float4(o[0], o[1], o[2], o[3]);
            }
            // bp_{t+1}: one word per thread
            if (trace) buf_st(__builtin_bit_cast(float, word), tape, v_word, par * buf_bytes + (uint32_t)(t + 1) * (TPS * 4u));

            // one step of the previous sequence's traceback
            if (tau == 0 && pend_b >= 0 && pend_t >= 1) {
                const uint32_t v = pend_s >> 2, j = v >> 2, i = v & 3u;
                const uint32_t a = (pend_word >> (8u * (j / TPS) + 2u * i)) & 3u;
                pend_s = v | (a << (L - 2));
                --pend_t;
                args.states[(int64_t)pend_b * n + pend_t] = (int32_t)pend_s;
                if (pend_t >= 1)
                    pend_word = __builtin_bit_cast(uint32_t, buf_ld(tape, sq * slot_bytes, pend_par * buf_bytes +
                                                                    (uint32_t)pend_t * (TPS * 4u) + 4u * ((pend_s >> 4) % TPS)));
            }
            lds_barrier();
        }

        // last step: M_{n-1}(s) for every state, then the end state
        const float* ml = ((n - 1) & 1) ? msg1 : msg0;
        const float wl = wb[n - 1 + rot < n ? n - 1 + rot : n - 1 + rot - n];
        float best = kInf;
        uint32_t bidx = 0xffffffffu;
        if (!has_sigma) {
#pragma unroll
            for (int m = 0; m < QPT; ++m) {
                const int j = tau + TPS * m;
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const float v = ml[j + Q * a];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float M = emit_metric(wl, cb[m][a][i], v);
                        const uint32_t s = ((uint32_t)a << (L - 2)) | ((uint32_t)j << 2) | (uint32_t)i;
                        argmin_merge(best, bidx, M, s);
                    }
                }
            }
            seg_argmin<SEG>(best, bidx);
            if constexpr (WPS > 1) {
                if (lane == 0) {
                    redv[sq][wv] = best;
                    redi[sq][wv] = bidx;
                }
            }
            __syncthreads();   // also publishes this sequence's back pointers to the traceback lane
            if constexpr (WPS > 1) {
#pragma unroll
                for (int q = 0; q < WPS; ++q) argmin_merge(best, bidx, redv[sq][q], redi[sq][q]);
            }
        } else {
            __syncthreads();
            bidx = sig;
            best = emit_metric(wl, args.cb[sig], ml[sig >> 2]);
        }
        if (tau == 0 && active && args.cost) args.cost[b] = best;

        // finish the previous sequence's traceback (at most a step or two remain) and gather its codewords
        if (tau == 0 && pend_b >= 0) {
            while (pend_t >= 1) {
                const uint32_t v = pend_s >> 2, j = v >> 2, i = v & 3u;
                const uint32_t a = (pend_word >> (8u * (j / TPS) + 2u * i)) & 3u;
                pend_s = v | (a << (L - 2));
                --pend_t;
                args.states[(int64_t)pend_b * n + pend_t] = (int32_t)pend_s;
                if (pend_t >= 1)
                    pend_word = __builtin_bit_cast(uint32_t, buf_ld(tape, sq * slot_bytes, pend_par * buf_bytes +
                                                                    (uint32_t)pend_t * (TPS * 4u) + 4u * ((pend_s >> 4) % TPS)));
            }
        }
        __syncthreads();
        if (args.w_hard) {
            // every sequence of the block had a pending traceback or none; gather for those that did
            const int64_t pb = (iter > 0) ? (gi - gridDim.x) * SPB + sq : -1;
            if (pb >= 0 && pb < args.B)
                for (int t = tau; t < n; t += TPS) args.w_hard[pb * n + t] = args.cb[args.states[pb * n + t]];
        }
        // this sequence becomes the pending traceback
        if (tau == 0 && trace) {
            pend_b = active ? (int32_t)b : -1;
            pend_par = par;
            pend_s = bidx;
            pend_t = n - 1;
            if (active) {
                args.states[b * n + n - 1] = (int32_t)bidx;
                if (n > 1)
                    pend_word = __builtin_bit_cast(uint32_t, buf_ld(tape, sq * slot_bytes, par * buf_bytes +
                                                                    (uint32_t)(n - 1) * (TPS * 4u) + 4u * ((bidx >> 4) % TPS)));
            }
        }
        __syncthreads();   // LDS buffers and the other back-pointer buffer are reused next
    }

    // drain the block's last traceback
    if (tau == 0 && pend_b >= 0) {
        while (pend_t >= 1) {
            const uint32_t v = pend_s >> 2, j = v >> 2, i = v & 3u;
            const uint32_t a = (pend_word >> (8u * (j / TPS) + 2u * i)) & 3u;
            pend_s = v | (a << (L - 2));
            --pend_t;
            args.states[(int64_t)pend_b * n + pend_t] = (int32_t)pend_s;
            if (pend_t >= 1)
                pend_word = __builtin_bit_cast(uint32_t, buf_ld(tape, sq * slot_bytes, pend_par * buf_bytes +
                                                                (uint32_t)pend_t * (TPS * 4u) + 4u * ((pend_s >> 4) % TPS)));
        }
    }
    __syncthreads();
    if (args.w_hard && iter > 0) {
        const int64_t gl = blockIdx.x + (iter - 1) * (int64_t)gridDim.x;
        const int64_t pb = gl * SPB + sq;
        if (pb < args.B)
            for (int t = tau; t < n; t += TPS) args.w_hard[pb * n + t] = args.cb[args.states[pb * n + t]];
    }
}

// Tail-biting start-state choice, exact: per row, the first sigma attaining the minimum of costs[row * S + sigma]
// (a NaN cost ranks below every number, as the first NaN is what a plain argmin returns).  One wave per row.
__global__ void __launch_bounds__(256) tb_select_kernel(const float* costs, int64_t rows, int S, int32_t* sigma,
                                                         int32_t* sigma_out) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;   // the whole wave leaves together
    float best = __builtin_huge_valf();
    uint32_t arg = 0xffffffffu;
    for (int s = lane; s < S; s += 64) {
        const float v = costs[row * S + s];
        argmin_merge(best, arg, __builtin_isnan(v) ? -__builtin_huge_valf() : v, (uint32_t)s);
    }
    seg_argmin<64>(best, arg);
    if (lane == 0) {
        sigma[row] = (int32_t)arg;
        if (sigma_out) sigma_out[row] = (int32_t)arg;
    }
}

// Tail-biting start-state choice, rotate-and-decode: sigma = the state of the rotated free decode at position pos.
__global__ void __launch_bounds__(256) tb_rotate_sigma_kernel(const int32_t* states_rot, int64_t rows, int n, int pos,
                                                               int32_t* sigma, int32_t* sigma_out) {
    const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (row >= rows) return;
    const int32_t s = states_rot[row * n + pos];
    sigma[row] = s;
    if (sigma_out) sigma_out[row] = s;
}

hipError_t launch_tb_select(const float* costs, int64_t rows, int S, int32_t* sigma, int32_t* sigma_out,
                            hipStream_t st) {
    hipLaunchKernelGGL(tb_select_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, costs, rows, S, sigma,
                       sigma_out);
    return hipGetLastError();
}

hipError_t launch_tb_rotate_sigma(const int32_t* states_rot, int64_t rows, int n, int pos, int32_t* sigma,
                                  int32_t* sigma_out, hipStream_t st) {
    hipLaunchKernelGGL(tb_rotate_sigma_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, states_rot,
                       rows, n, pos, sigma, sigma_out);
    return hipGetLastError();
}

template <int L>
static hipError_t launch_viterbi_L(const ViterbiArgs& a, int grid, hipStream_t st) {
    hipLaunchKernelGGL(viterbi_kernel<L>, dim3(grid), dim3(Geo<L>::NT), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_viterbi(int L, const ViterbiArgs& a, int grid, hipStream_t st) {
    switch (L) {
        case 4: return launch_viterbi_L<4>(a, grid, st);
        case 5: return launch_viterbi_L<5>(a, grid, st);
        case 6: return launch_viterbi_L<6>(a, grid, st);
        case 7: return launch_viterbi_L<7>(a, grid, st);
        case 8: return launch_viterbi_L<8>(a, grid, st);
        case 9: return launch_viterbi_L<9>(a, grid, st);
        case 10: return launch_viterbi_L<10>(a, grid, st);
        case 11: return launch_viterbi_L<11>(a, grid, st);
        case 12: return launch_viterbi_L<12>(a, grid, st);
        case 13: return launch_viterbi_L<13>(a, grid, st);
        case 14: return launch_viterbi_L<14>(a, grid, st);
        case 15: return launch_viterbi_L<15>(a, grid, st);
        case 16: return launch_viterbi_L<16>(a, grid, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace bcjr
