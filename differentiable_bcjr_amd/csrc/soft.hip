// soft.hip -- temperature-T BCJR forward-backward pass producing the soft codeword (and ln Z) on gfx950.
//
// The soft codeword is the Boltzmann expectation of the emitted codebook value over all trellis paths, computed by
// the BCJR sum-product recursion at temperature T (BCJR-QAT, arXiv 2605.10655: abstract; gist.science Technical
// Summary, "Core Mechanism" and "Key Technical Innovations", where gather, log-sum-exp and add are fused in one
// launch).  Here one launch runs both directions for every sequence:
//
//   forward   R~_{t+1}(v) = logsumexp_a[ theta_t(v | a << (L-2)) + R~_t(v >> 2 | a << (L-4)) ] - N_t
//   backward  B~_{t-1}(u) = logsumexp_b[ theta_t(4u + b)         + B~_t((4u + b) & (G-1)) ] - N'_t
//   posterior p_t(s) = 2^( theta_t(s) + R~_t(s >> 2) + B~_t(s & (G-1)) - ref_t ),  w_soft_t = sum_s c(s) p_t(s)
//
// All logs are base 2: theta_t(s) = -(c(s) k - w'_t)^2 with k = sqrt(log2 e / T), w' = w k, the difference formed by
// one fused multiply-add so that each state's log-weight carries a single rounding.
// N_t, N'_t are per-step normalisers (the max of the incoming message), so messages stay within one step's
// emission range of 0.  With A_t = sum_{tau<t} N_tau and C_t = sum_{tau>t} N'_tau, ref_t = log2 Z - A_t - C_t makes
// sum_s p_t(s) = 1 without a second pass; any error in ref_t cancels in the ratio that gives w_soft_t.
//
// Layout: 1024 threads per sequence at L = 16 (4 quads = 64 states per thread, their codebook values in VGPRs),
// messages double-buffered in LDS (2 x 64 KiB), one block per CU.  The forward messages R~_t of every step go to a
// per-block tape in the workspace ([n+1][G] float32 written as float4, then the per-step normalisers N_t) and are read
// back by the backward pass one quad ahead, through raw buffer instructions (SGPR base + one VGPR lane offset) with
// the non-temporal policy (written once, read once a pass later).  The next step's weight and normaliser are loaded
// one step ahead.  With several waves per sequence each wave's (S0, S1) of every step goes to the workspace and the
// soft codewords are formed after the backward pass, so the step loop carries no serial output reduction.
#include "kernel_args.hpp"
#include "trellis.hpp"

namespace bcjr {

// Groups of 4 states whose work the scheduler may interleave between two scheduling barriers (forward, backward).
#ifndef BCJR_SOFT_FWD_GROUPS
#define BCJR_SOFT_FWD_GROUPS 2
#endif
#ifndef BCJR_SOFT_BWD_GROUPS
#define BCJR_SOFT_BWD_GROUPS 2
#endif
constexpr int kSoftFwdGroups = BCJR_SOFT_FWD_GROUPS;
constexpr int kSoftBwdGroups = BCJR_SOFT_BWD_GROUPS;

// CK: the checkpoint mode.  The forward pass stores only rows t = 0, c, 2c, .. and row n - 1 (TapeRows); the
// backward pass walks the segments from the end and, before each, saves its message to the workspace, reloads the
// segment's checkpoint into LDS, reruns the forward steps of the segment with the stored normalisers (the same code
// and numbers as the first pass, so the rows come out bit-identical), and restores its message.  A compile-time flag,
// so the full-tape kernel carries none of it.
template <int L, bool CK>
__global__ void __launch_bounds__(Geo<L>::NT) soft_kernel(SoftArgs args) {
    using Gm = Geo<L>;
    constexpr int G = Gm::G, Q = Gm::Q, QPT = Gm::QPT, TPS = Gm::TPS, SPB = Gm::SPB, WPS = Gm::WPS;
    constexpr int SEG = Gm::SEG;
    __shared__ float4 msg4[SPB][2][G / 4];
    __shared__ float redmax[2][SPB][WPS];
    __shared__ float redsum[2][SPB][WPS];

    const int tid = threadIdx.x;
    const int sq = tid / TPS;
    const int tau = tid % TPS;
    const int lane = tid & 63;
    const int wv = tau >> 6;
    float* msg0 = reinterpret_cast<float*>(&msg4[sq][0][0]);
    float* msg1 = reinterpret_cast<float*>(&msg4[sq][1][0]);

    const int n = args.n;
    const float scale = args.scale;
    const float inv_scale = 1.0f / scale;

    // codebook c(s) for this thread's quads, s = a << (L-2) | j << 2 | i, unscaled: the scaled difference is formed
    // as fma(c, sqrt(log2 e / T), -w'), which rounds once per state instead of rounding c' first
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

    // tape of this block's sequences: slot sq at sq * slot_bytes; the message rows (TapeRows), then [n] normalisers
    const uint32_t slot_bytes = (uint32_t)args.slot_bytes;
    const rsrc_t tape = make_rsrc(args.ws + (size_t)blockIdx.x * SPB * args.slot_bytes, SPB * slot_bytes);
    const uint32_t v_quad = sq * slot_bytes + 16u * tau;   // float4 at group 4j, j = tau + TPS m
    const uint32_t v_grp = sq * slot_bytes + 4u * tau;     // float at group j + Q a
    const int ck = CK ? args.ckpt : 0;
    constexpr uint32_t row_bytes = G * 4u;
    const TapeRows rows{ck, n, row_bytes, ck ? (uint32_t)(n / ck + 1) * row_bytes : 0u};
    const uint32_t nrm_base = (uint32_t)align256(TapeRows::rows(ck, n) * row_bytes);
    // with several waves per sequence, each wave's (S0, S1) of every step goes here and the soft codeword is formed
    // after the backward pass, so no wave waits on a serial per-step reduction
    const uint32_t part_base = nrm_base + (uint32_t)align256((size_t)n * 4);
    // checkpoint mode: each thread's share of the backward message while a segment is rebuilt
    const uint32_t save_base = part_base + (WPS > 1 ? (uint32_t)align256((size_t)n * WPS * 8) : 0u);

    // One forward step: R~_{t+1} = logsumexp over the 4 predecessors of theta_t + R~_t (read from mc) minus the
    // normaliser N, written to mn and, when `store`, to the tape row at row_off.  Returns this thread's maximum of
    // the outputs.  The first pass and the checkpoint recompute both run it.
    auto fwd_step = [&](const float* mc, float* mn, float wt, float N, bool store, uint32_t row_off) -> float {
        float lmax = -3.0e38f;
#pragma unroll
        for (int m = 0; m < QPT; ++m) {
            const int j = tau + TPS * m;
            float r[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) r[a] = mc[j + Q * a];
            float o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float x[4];
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const float d = fmaf(cb[m][a][i], scale, -wt);
                    x[a] = fmaf(-d, d, r[a]);
                }
                const float mx = max4(x[0], x[1], x[2], x[3]);
                const float s = (ex2(x[0] - mx) + ex2(x[1] - mx)) + (ex2(x[2] - mx) + ex2(x[3] - mx));
                o[i] = (mx - N) + lg2(s);
                if ((i + 1) % kSoftFwdGroups == 0) __builtin_amdgcn_sched_barrier(0);
            }
            lmax = run_max(lmax, max4(o[0], o[1], o[2], o[3]));
            const float4 o4 = make_float4(o[0], o[1], o[2], o[3]);
            *reinterpret_cast<float4*>(mn + 4 * j) = o4;
            if (store) buf_st4_nt(o4, tape, v_quad, row_off + 16u * TPS * m);
        }
        return lmax;
    };

    const int64_t ngroups = (args.B + SPB - 1) / SPB;
    for (int64_t gi = blockIdx.x; gi < ngroups; gi += gridDim.x) {
        const int64_t b = gi * SPB + sq;
        const bool active = b < args.B;
        const int64_t bb = active ? b : args.B - 1;
        const int64_t row = args.sigma_enum ? (bb >> L) : bb;   // the weights' row (sigma enumeration: v >> L)
        const float* wb = args.w + row * n;
        const bool has_sigma = args.sigma_enum || args.sigma != nullptr;
        const uint32_t sig = args.sigma_enum ? (uint32_t)(bb & (Gm::S - 1))
                                             : has_sigma ? ((uint32_t)args.sigma[bb] & (uint32_t)(Gm::S - 1)) : 0u;

        // ------------------------------------------------------------------ forward
        // R~_0: free start -> 0 everywhere; sigma -> only the successors of sigma (group sigma & (G-1)) reachable
#pragma unroll
        for (int m = 0; m < QPT; ++m) {
            const int j = tau + TPS * m;
            float4 r;
            r.x = (!has_sigma || (uint32_t)(4 * j + 0) == (sig & (G - 1))) ? 0.f : kNeg;
            r.y = (!has_sigma || (uint32_t)(4 * j + 1) == (sig & (G - 1))) ? 0.f : kNeg;
            r.z = (!has_sigma || (uint32_t)(4 * j + 2) == (sig & (G - 1))) ? 0.f : kNeg;
            r.w = (!has_sigma || (uint32_t)(4 * j + 3) == (sig & (G - 1))) ? 0.f : kNeg;
            *reinterpret_cast<float4*>(msg0 + 4 * j) = r;
            buf_st4_nt(r, tape, v_quad, 16u * TPS * m);   // row 0
        }
        lds_barrier();

        float N = 0.f;        // normaliser subtracted at this step (max of R~_t)
        double A = 0.0;       // A_t: log2 offset of R~_t
        float N_last = 0.f;   // N_{n-1}
        float w_nx = wb[0];   // the next step's weight, loaded one step ahead
        for (int t = 0; t < n; ++t) {
            const float* mc = (t & 1) ? msg1 : msg0;
            float* mn = (t & 1) ? msg0 : msg1;
            const float wt = w_nx * scale;
            if (t + 1 < n) w_nx = wb[t + 1];
            // row n is a spare the full tape keeps; in checkpoint mode only the checkpoints and row n - 1 go out
            float lmax = fwd_step(mc, mn, wt, N, rows.stored(t + 1), rows.off(t + 1));
            if (tau == 0) buf_st(N, tape, sq * slot_bytes, nrm_base + 4u * t);
            lmax = seg_max_fast<SEG>(lmax);
            if constexpr (WPS > 1) {
                if (lane == 0) redmax[t & 1][sq][wv] = lmax;
            }
            lds_barrier();
            if constexpr (WPS > 1) {
                static_assert(WPS <= 16, "per-wave slots are combined inside one 16-lane row");
                lmax = row16_max((lane & 15) < WPS ? redmax[t & 1][sq][lane & 15] : -3.0e38f);
            }
            if constexpr (SPB == 1) lmax = uniform_f(lmax);
            A += (double)N;
            N_last = N;
            N = lmax;
        }
        // now: R~_n in msg[n & 1] with max N, and A = A_n;  R~_{n-1} in msg[(n-1) & 1]
        // rz = log2 Z - A_n
        float rz;
        if (!has_sigma) {
            const float* mf = (n & 1) ? msg1 : msg0;
            float part = 0.f;
#pragma unroll
            for (int m = 0; m < QPT; ++m) {
                const float4 o = *reinterpret_cast<const float4*>(mf + 4 * (tau + TPS * m));
                part += (ex2(o.x - N) + ex2(o.y - N)) + (ex2(o.z - N) + ex2(o.w - N));
            }
            part = seg_sum_fast<SEG>(part);
            if constexpr (WPS > 1) {
                if (lane == 0) redsum[n & 1][sq][wv] = part;
            }
            lds_barrier();
            if constexpr (WPS > 1) {
                part = 0.f;
#pragma unroll
                for (int q = 0; q < WPS; ++q) part += redsum[n & 1][sq][q];
            }
            rz = N + lg2(part);
        } else {
            const float* ml = ((n - 1) & 1) ? msg1 : msg0;
            const float d = fmaf(args.cb[sig], scale, -(wb[n - 1] * scale));
            const float r = ml[sig >> 2];
            lds_barrier();
            rz = (r < 0.5f * kNeg) ? kNeg : fmaf(-d, d, r) - N_last;
        }
        const bool valid = rz > 0.5f * kNeg;
        if (tau == 0 && active && args.log_z)
            args.log_z[b] = valid ? (float)((A + (double)rz) * 0.6931471805599453) : -__builtin_inff();

        // ------------------------------------------------------------------ backward + posterior
        __syncthreads();   // tape writes of the forward pass visible to every thread of the block
        float Nb = 0.f;    // normaliser for this step's outputs (max of B~_t)
        float C = 0.f;     // C_t: log2 offset of B~_t
        float D = 0.f;     // D_t = A_n - A_t
        int t = n - 1;
        if (!has_sigma) {
            // free end: beta_{n-1} = 0, i.e. B~_{n-1} = 0 in every group
            float* mi = ((n - 1) & 1) ? msg1 : msg0;
#pragma unroll
            for (int m = 0; m < QPT; ++m)
                *reinterpret_cast<float4*>(mi + 4 * (tau + TPS * m)) = make_float4(0.f, 0.f, 0.f, 0.f);
        } else {
            // s_n = sigma: the posterior at n-1 is the indicator of sigma, and the only finite message left is
            // B_{n-2}(sigma >> 2) = theta_{n-1}(sigma).  It goes into the offset C, and the message starts at 0:
            // theta can be a hundred or more in log2 units, and the next step's branch terms, added to it, would
            // keep only its absolute precision (each state's weight off by ~1e-5)
            float* mi = ((n - 2) & 1) ? msg1 : msg0;
            const float d = fmaf(args.cb[sig], scale, -(wb[n - 1] * scale));
            const float th = -d * d;
            if (n > 1) {
#pragma unroll
                for (int m = 0; m < QPT; ++m)
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        const uint32_t u = (uint32_t)(tau + TPS * m + Q * a);
                        mi[u] = (u == (sig >> 2)) ? 0.f : kNeg;
                    }
            }
            if (tau == 0 && active) args.w_soft[b * n + n - 1] = valid ? args.cb[sig] : __builtin_nanf("");
            D = N_last;
            C = th;
            t = n - 2;
        }
        lds_barrier();

        float rq[4], rn[4];
        if (t >= 0) {
#pragma unroll
            for (int a = 0; a < 4; ++a) rq[a] = buf_ld_nt(tape, v_grp, rows.off(t) + 4u * Q * a);
        }
        const int t_out = t;   // last step whose soft codeword the loop below produces
        float N_nx = 0.f;
        if (t >= 0) {
            w_nx = wb[t];
            N_nx = buf_ld_nt(tape, sq * slot_bytes, nrm_base + 4u * t);
        }
        while (t >= 0) {
            const int t0 = ck ? (t / ck) * ck : 0;   // first step of this segment
            if (CK && ck) {
                // keep this thread's share of the backward message (the quads it reads at step t), rebuild the
                // segment's rows t0+1..t from checkpoint t0 with the stored normalisers, then restore the message
                const float* mb = (t & 1) ? msg1 : msg0;
#pragma unroll
                for (int m = 0; m < QPT; ++m)
                    buf_st4(*reinterpret_cast<const float4*>(mb + 4 * (tau + TPS * m)), tape, v_quad,
                            save_base + 16u * TPS * m);
                lds_barrier();   // every share read before the recompute overwrites the buffers
                float* m0 = (t0 & 1) ? msg1 : msg0;
#pragma unroll
                for (int m = 0; m < QPT; ++m)
                    *reinterpret_cast<float4*>(m0 + 4 * (tau + TPS * m)) =
                        buf_ld4(tape, v_quad, rows.off(t0) + 16u * TPS * m);
                lds_barrier();
                for (int tt = t0; tt < t; ++tt) {
                    const float* mc = (tt & 1) ? msg1 : msg0;
                    float* mn = (tt & 1) ? msg0 : msg1;
                    float Nr = buf_ld(tape, sq * slot_bytes, nrm_base + 4u * tt);
                    if constexpr (SPB == 1) Nr = uniform_f(Nr);
                    fwd_step(mc, mn, wb[tt] * scale, Nr, true, rows.off(tt + 1));
                    lds_barrier();
                }
                __syncthreads();   // the rebuilt rows, written by other threads, before the backward reads them
                float* mr = (t & 1) ? msg1 : msg0;
#pragma unroll
                for (int m = 0; m < QPT; ++m)
                    *reinterpret_cast<float4*>(mr + 4 * (tau + TPS * m)) = buf_ld4(tape, v_quad, save_base + 16u * TPS * m);
                lds_barrier();
#pragma unroll
                for (int a = 0; a < 4; ++a) rq[a] = buf_ld_nt(tape, v_grp, rows.off(t) + 4u * Q * a);
            }
            for (; t >= t0; --t) {
                const float* mc = (t & 1) ? msg1 : msg0;
                float* mn = (t & 1) ? msg0 : msg1;
                const float wt = w_nx * scale;
                float Nt = N_nx;
                if (t > 0) {   // the next step's weight and forward normaliser, one step ahead
                    w_nx = wb[t - 1];
                    N_nx = buf_ld_nt(tape, sq * slot_bytes, nrm_base + 4u * (t - 1));
                }
                if constexpr (SPB == 1) Nt = uniform_f(Nt);
                D += Nt;
                const float ref = (rz + D) - C;
                float lmax = -3.0e38f, S0 = 0.f, S1 = 0.f;
#pragma unroll
                for (int m = 0; m < QPT; ++m) {
                    const int j = tau + TPS * m;
                    // prefetch the forward messages of the next quad (or of the next step's first quad; in
                    // checkpoint mode a row past the segment is read again once it has been rebuilt)
                    if (m + 1 < QPT) {
#pragma unroll
                        for (int a = 0; a < 4; ++a)
                            rn[a] = buf_ld_nt(tape, v_grp, rows.off(t) + 4u * (TPS * (m + 1) + Q * a));
                    } else if (t > 0) {
#pragma unroll
                        for (int a = 0; a < 4; ++a) rn[a] = buf_ld_nt(tape, v_grp, rows.off(t - 1) + 4u * Q * a);
                    }
                    const float4 bq = *reinterpret_cast<const float4*>(mc + 4 * j);
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        const float d0 = fmaf(cb[m][a][0], scale, -wt), d1 = fmaf(cb[m][a][1], scale, -wt);
                        const float d2 = fmaf(cb[m][a][2], scale, -wt), d3 = fmaf(cb[m][a][3], scale, -wt);
                        const float y0 = fmaf(-d0, d0, bq.x), y1 = fmaf(-d1, d1, bq.y);
                        const float y2 = fmaf(-d2, d2, bq.z), y3 = fmaf(-d3, d3, bq.w);
                        const float mx = max4(y0, y1, y2, y3);
                        const float e0 = ex2(y0 - mx), e1 = ex2(y1 - mx), e2 = ex2(y2 - mx), e3 = ex2(y3 - mx);
                        const float s = (e0 + e1) + (e2 + e3);
                        const float out = (mx - Nb) + lg2(s);
                        const float f = ex2((mx + rq[a]) - ref);
                        S0 = fmaf(f, s, S0);
                        S1 = fmaf(f, fmaf(e0, d0, fmaf(e1, d1, fmaf(e2, d2, e3 * d3))), S1);
                        lmax = run_max(lmax, out);
                        mn[j + Q * a] = out;   // at t = 0 this lands in a buffer nobody reads
                        if ((a + 1) % kSoftBwdGroups == 0) {
                            pin_order(S0, S1, lmax);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
#pragma unroll
                    for (int a = 0; a < 4; ++a) rq[a] = rn[a];
                }
                lmax = seg_max_fast<SEG>(lmax);
                S0 = seg_sum_fast<SEG>(S0);
                S1 = seg_sum_fast<SEG>(S1);
                if constexpr (WPS > 1) {
                    if (lane == 0) {
                        redmax[t & 1][sq][wv] = lmax;
                        buf_st2(make_float2(S0, S1), tape, sq * slot_bytes, part_base + 8u * (uint32_t)(t * WPS + wv));
                    }
                }
                lds_barrier();
                if constexpr (WPS > 1) {
                    lmax = row16_max((lane & 15) < WPS ? redmax[t & 1][sq][lane & 15] : -3.0e38f);
                } else {
                    if (tau == 0 && active)
                        args.w_soft[b * n + t] = valid ? fmaf(S1 / S0, inv_scale, wb[t]) : __builtin_nanf("");
                }
                if constexpr (SPB == 1) lmax = uniform_f(lmax);
                C += Nb;
                Nb = lmax;
            }
        }
        if constexpr (WPS > 1) {
            // soft codewords of steps 0..t_out from the per-wave partial sums, one step per thread, summed over the
            // waves in wave order
            __syncthreads();
            for (int tt = tau; tt <= t_out; tt += TPS) {
                float S0 = 0.f, S1 = 0.f;
#pragma unroll
                for (int q = 0; q < WPS; ++q) {
                    const float2 p = buf_ld2(tape, sq * slot_bytes, part_base + 8u * (uint32_t)(tt * WPS + q));
                    S0 += p.x;
                    S1 += p.y;
                }
                if (active) args.w_soft[b * n + tt] = valid ? fmaf(S1 / S0, inv_scale, wb[tt]) : __builtin_nanf("");
            }
        }
        // the next sequence reuses the tape and the LDS buffers
        __syncthreads();
    }
}

// ------------------------------------------------------------------------------------------------------------------
// host-side launch (called by the C-ABI after argument checks)

template <int L>
static hipError_t launch_soft_L(const SoftArgs& a, int grid, hipStream_t st) {
    if (a.ckpt) hipLaunchKernelGGL((soft_kernel<L, true>), dim3(grid), dim3(Geo<L>::NT), 0, st, a);
    else hipLaunchKernelGGL((soft_kernel<L, false>), dim3(grid), dim3(Geo<L>::NT), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_soft(int L, const SoftArgs& a, int grid, hipStream_t st) {
    switch (L) {
        case 4: return launch_soft_L<4>(a, grid, st);
        case 5: return launch_soft_L<5>(a, grid, st);
        case 6: return launch_soft_L<6>(a, grid, st);
        case 7: return launch_soft_L<7>(a, grid, st);
        case 8: return launch_soft_L<8>(a, grid, st);
        case 9: return launch_soft_L<9>(a, grid, st);
        case 10: return launch_soft_L<10>(a, grid, st);
        case 11: return launch_soft_L<11>(a, grid, st);
        case 12: return launch_soft_L<12>(a, grid, st);
        case 13: return launch_soft_L<13>(a, grid, st);
        case 14: return launch_soft_L<14>(a, grid, st);
        case 15: return launch_soft_L<15>(a, grid, st);
        case 16: return launch_soft_L<16>(a, grid, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace bcjr
