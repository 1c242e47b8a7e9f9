// grad.hip -- exact gradient of the soft codeword with respect to the weights (and the codebook values), on gfx950.
//
// The soft codeword is exactly differentiable in the weight pre-image (BCJR-QAT, arXiv 2605.10655: gist.science
// Technical Summary, "Core Mechanism"; "Key Technical Innovations").  Differentiating w_soft_t = E_p[c(s_t)] under
// p(path) ~ exp(-sum_t (w_t - c(s_t))^2 / T) gives d w_soft_t / d w_u = (2/T) Cov_p(c(s_t), c(s_u)), so for an
// upstream gradient g
//     grad_u = (2/T) Cov_p( c(s_u), F ),   F = sum_t g_t (c(s_t) - w_t)
// (subtracting the constant sum_t g_t w_t from F changes no covariance and keeps F small).  E[F | s_u] splits at u
// because the posterior is a Markov chain, and both halves are carried as one extra message per group alongside the
// log-sum-exp messages of the soft pass, weighted by the same softmax weights (the expectation semiring):
//   forward   Q_{t+1}(v) = sum_a pi_a  [ g_t (c(s_a) - w_t) + Q_t(v >> 2 | a << (L-4)) ],  pi = softmax over a
//   backward  P_{t-1}(u) = sum_b rho_b [ g_t (c(s_b) - w_t) + P_t((4u + b) & (G-1)) ],   rho = softmax over b
//   at step t, for state s: E[F | s_t = s] = g_t (c(s) - w_t) + Q_t(s >> 2) + P_t(s & (G-1))
// The covariance is reduced over the block per step from the posterior weights of the soft pass.  Float32 accuracy
// needs every per-state term of that reduction to stay O(1), so both expectation messages are re-centred each step
// by a per-step constant (Cov ignores constants): Q by its value at the forward pass's most likely group, P by
// g_t (w_soft_t - w_t), which turns P into E[sum_{tau>t} g_tau (c(s_tau) - w_soft_tau) | s_t], a zero-mean quantity.
// The constants are carried separately and recombined into one per-step offset, so E[F | s_t] - E[F] is formed
// from small numbers only.
//
// LDS holds the log-sum-exp message and the expectation message of one direction (2 x 64 KiB at L = 16) in a single
// buffer: each step loads its inputs into registers, barriers, then writes its outputs.  Both forward messages go to
// the workspace tape (non-temporal: written once, read once a pass later).  At L = 16 the codebook is read through
// L1/L2 each step (a thread has no registers left for it); at smaller L it stays in registers.  Memory latency is
// covered by issuing the backward's tape loads and codebook rows several groups ahead, the forward's codebook rows one
// quad ahead, and the next step's scalars (w, g, normaliser, Q offset) one step ahead.  With several waves per sequence only (S0, S1) is
// combined across waves inside the step loop; every wave's (S0..S3) goes to the workspace and the outputs are formed
// after the backward pass.
//
// The soft codeword is exactly differentiable in the codebook values as well (the trellis parameters, same passage).
// The GC instantiation adds, for every state s and step t of the backward pass,
//     p_t(s) [ g_t + (2/T) (w_t - c(s)) (E[F | s_t = s] - E[F]) ]
// to a per-slot float accumulator in the workspace; codebook_reduce_kernel then sums the slots in a fixed order.
#include <type_traits>

#include "kernel_args.hpp"
#include "trellis.hpp"

namespace bcjr {

// Groups of 4 states whose work the scheduler may interleave between two scheduling barriers (forward, backward).
#ifndef BCJR_GRAD_FWD_GROUPS
#define BCJR_GRAD_FWD_GROUPS 1
#endif
#ifndef BCJR_GRAD_BWD_GROUPS
#define BCJR_GRAD_BWD_GROUPS 2
#endif
// How many groups ahead the backward pass issues its tape loads (R~ and Q^ of one group) and its codebook rows (read
// through L1/L2 at L = 16), each a power of two; at most the groups of a step are used.  Vector-memory loads complete
// in issue order under one counter, so waiting for a codebook row also waits for every tape load issued before it:
// the codebook row of a group is issued before that group's tape loads, and a tape load's lead is then the smaller of
// the tape depth and the codebook depth plus one group.  Measured on the 1024x1024 workload (T = 0.1): tape/codebook
// depth 1/1 (codebook after the tape) 76.6 ms, 2/1 77.0, 4/2 76.2, 4/4 74.0, 8/4 75.0, 8/8 92.0 (the rings spill).
#ifndef BCJR_GRAD_TAPE_DEPTH
#define BCJR_GRAD_TAPE_DEPTH 4
#endif
#ifndef BCJR_GRAD_CB_DEPTH
#define BCJR_GRAD_CB_DEPTH 4
#endif
constexpr int kGradFwdGroups = BCJR_GRAD_FWD_GROUPS;
constexpr int kGradBwdGroups = BCJR_GRAD_BWD_GROUPS;

// Codebook row c(a << (L-2) | j << 2 | 0..3) of quad m (unscaled): from registers, or through L1/L2.
template <int L, int TPS, bool CB_REG, int M>
__device__ __forceinline__ float4 cb_row(const float (&cbr)[M][4][4], rsrc_t cbs, uint32_t v_cb, int m, int a) {
    if constexpr (CB_REG) {
        return make_float4(cbr[m][a][0], cbr[m][a][1], cbr[m][a][2], cbr[m][a][3]);
    } else {
        return buf_ld4(cbs, v_cb, 4u * ((uint32_t)a << (L - 2)) + 16u * TPS * m);
    }
}

// GCM = 1: also accumulate dL/dc per state of the trellis into this slot's accumulator (read-modify-write of
// [2^L] floats at the end of the slot, one float4 per group and step), normalising each step's posterior by the
// previous step's exact total, with the running normaliser sums in double.
// GCM = 2 (boundary-state mode): there the last ~L/2 steps are forced through far codewords, the posterior is nearly
// frozen, and two roundings that cancel in the weights' gradient survive in dL/dc:
//   * the messages carry log-weights of a hundred or more, whose roundings differ between the forward and the
//     backward pass, so consecutive steps' totals differ by up to ~1e-5 and the previous step's total misweights
//     the step; here every step is divided by its own exact total;
//   * E[F | s] - E[F] at the likely state, a small difference of O(1) expectation messages, carries their
//     roundings, which dL/dc multiplies by (2/T)(w - c); the weights' gradient is a covariance, centred by
//     m2 = E[E[F | s] - E[F]] (zero exactly, the step's common rounding numerically), and here dL/dc is centred
//     the same way: p(s) (2/T)(w - c(s)) (E[F | s] - E[F] - m2).
// Both need the step's totals, known after its loop, so each step's contribution is kept in two further [2^L]
// arrays, P1 = f e [g + (2/T)(w - c)(E[F | s] - E[F])] and P2 = f e (2/T)(c - w) (f the step's posterior factor),
// and folded in during the next step (and after the last) as A += (P1 + m2 P2) / S0: two more reads and writes per
// state and step in this mode.
// CK: the checkpoint mode.  The forward pass stores only rows t = 0, c, 2c, .. and row n - 1 of both messages
// (TapeRows), and each step's Q input offset; the backward pass walks the segments from the end and, before each,
// saves its two messages to the workspace, reloads the segment's checkpoint, reruns the forward steps of the segment
// with the stored normalisers and offsets (the same code and numbers as the first pass, so the rows come out
// bit-identical), and restores its messages.  A compile-time flag, so the full-tape kernels carry none of it.
template <int L, int GCM, bool CK>
__global__ void __launch_bounds__(Geo<L>::NT) grad_kernel(GradArgs args) {
    constexpr bool GC = GCM != 0, EXACT = GCM == 2;
    using Gm = Geo<L>;
    constexpr int G = Gm::G, Q = Gm::Q, QPT = Gm::QPT, TPS = Gm::TPS, SPB = Gm::SPB, WPS = Gm::WPS;
    constexpr int SEG = Gm::SEG;
    constexpr bool CB_REG = QPT <= 2;
    __shared__ float4 lds_r4[SPB][G / 4];
    __shared__ float4 lds_q4[SPB][G / 4];
    __shared__ float redmax[2][SPB][WPS];
    __shared__ float redq[2][SPB][WPS];
    __shared__ float4 redsum[2][SPB][WPS];
    __shared__ float4 redsum2[2][SPB][WPS];

    const int tid = threadIdx.x;
    const int sq = tid / TPS;
    const int tau = tid % TPS;
    const int lane = tid & 63;
    const int wv = tau >> 6;
    float* mr = reinterpret_cast<float*>(&lds_r4[sq][0]);
    float* mq = reinterpret_cast<float*>(&lds_q4[sq][0]);

    const int n = args.n;
    const float scale = args.scale;
    const float inv_scale = 1.0f / scale;

    const rsrc_t cbs = make_rsrc(args.cb, 4u << L);
    const uint32_t v_cb = 16u * tau;
    float cbr[CB_REG ? QPT : 1][4][4];
    if constexpr (CB_REG) {
#pragma unroll
        for (int m = 0; m < QPT; ++m)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const float4 v = buf_ld4(cbs, v_cb, 4u * ((uint32_t)a << (L - 2)) + 16u * TPS * m);
                cbr[m][a][0] = v.x;
                cbr[m][a][1] = v.y;
                cbr[m][a][2] = v.z;
                cbr[m][a][3] = v.w;
            }
    }

    // tape of this block's sequences: slot sq at sq * slot_bytes; the R~ rows and the Q^ rows (TapeRows each; with
    // the codebook gradient's full tape, one row of (R~, Q^) pairs per step instead), then per step the normaliser
    // N_t and the offset K_{t-1} of Q^_t (true Q_t = Q^_t + K_{t-1})
    const uint32_t slot_bytes = (uint32_t)args.slot_bytes;
    const rsrc_t tape = make_rsrc(args.ws + (size_t)blockIdx.x * SPB * args.slot_bytes, SPB * slot_bytes);
    const uint32_t v_quad = sq * slot_bytes + 16u * tau;
    const uint32_t v_grp = sq * slot_bytes + 4u * tau;
    const int ck = CK ? args.ckpt : 0;
    // The codebook gradient's full tape holds (R~, Q^) pairs, group u's two messages side by side, so its backward
    // reads both with one 8-byte load next to its accumulator traffic (measured 2-3% faster there, while in the
    // weights-only gradient the forward's extra register moves for the interleaved stores cost more than the loads
    // save).  Otherwise the R~ rows and the Q^ rows are two tapes, R~ first.  Both layouts span the same bytes.
    constexpr bool PAIR = GC && !CK;
    constexpr uint32_t row_bytes = G * (PAIR ? 8u : 4u);
    const TapeRows rows{ck, n, row_bytes, ck ? (uint32_t)(n / ck + 1) * row_bytes : 0u};
    const uint32_t q_base = (uint32_t)align256(TapeRows::rows(ck, n) * G * 4u);
    const uint32_t nrm_base = 2u * q_base;
    const uint32_t v_pair = sq * slot_bytes + 32u * tau;   // pair rows: the 4 pairs of groups 4j..4j+3
    const uint32_t v_grp2 = sq * slot_bytes + 8u * tau;    // pair rows: the pair of group j + Q a
    // stores the forward messages of quad j (groups 4j..4j+3) into the tape row at roff
    auto store_quad = [&](float4 r, float4 q, uint32_t roff, int m) {
        if constexpr (PAIR) {
            buf_st4_nt(make_float4(r.x, q.x, r.y, q.y), tape, v_pair, roff + 32u * TPS * m);
            buf_st4_nt(make_float4(r.z, q.z, r.w, q.w), tape, v_pair, roff + 32u * TPS * m + 16u);
        } else {
            buf_st4_nt(r, tape, v_quad, roff + 16u * TPS * m);
            buf_st4_nt(q, tape, v_quad, q_base + roff + 16u * TPS * m);
        }
    };
    // R~_t and Q^_t of group (m, a) of this thread from the tape row at roff
    auto load_group = [&](float& r, float& q, uint32_t roff, int m, int a) {
        if constexpr (PAIR) {
            const float2 v = buf_ld2_nt(tape, v_grp2, roff + 8u * (TPS * m + Q * a));
            r = v.x;
            q = v.y;
        } else {
            const uint32_t so = roff + 4u * (TPS * m + Q * a);
            r = buf_ld_nt(tape, v_grp, so);
            q = buf_ld_nt(tape, v_grp, q_base + so);
        }
    };
    const uint32_t kq_base = nrm_base + (uint32_t)align256((size_t)n * 4);
    // with several waves per sequence, each wave's (S0, S1, S2, S3) of every step goes here and the outputs are
    // formed after the backward pass; only (S0, S1) is reduced across waves inside the loop (for the P offset)
    const uint32_t part_base = kq_base + (uint32_t)align256((size_t)n * 4);
    // the codebook-gradient accumulator of the slot: state s at acc_base + 4 s, so the 4 states of group (m, a)
    // are the float4 at acc_base + 16 (a Q + j)
    const uint32_t acc_base = part_base + (WPS > 1 ? (uint32_t)align256((size_t)n * WPS * 16) : 0u);
    // checkpoint mode: each step's Q input offset, then each thread's share of the two backward messages while a
    // segment is rebuilt
    // GCM = 2: the pending contributions P1 and P2
    const uint32_t pend_base = acc_base + (uint32_t)align256((size_t)4 << L);
    const uint32_t pend2_base = pend_base + (uint32_t)align256((size_t)4 << L);
    const uint32_t kqi_base = acc_base + (GC ? 3u * (uint32_t)align256((size_t)4 << L) : 0u);
    const uint32_t save_base = kqi_base + (uint32_t)align256((size_t)n * 4);
    using RT = typename std::conditional<GC, double, float>::type;   // running normaliser sums
    const float kap = args.two_over_T * inv_scale;   // (2/T) (w - c) = -kap d with d in scaled units
    if constexpr (GC) {
#pragma unroll
        for (int m = 0; m < QPT; ++m)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                buf_st4(make_float4(0.f, 0.f, 0.f, 0.f), tape, v_quad, acc_base + 16u * (TPS * m + Q * a));
                if constexpr (EXACT) {
                    buf_st4(make_float4(0.f, 0.f, 0.f, 0.f), tape, v_quad, pend_base + 16u * (TPS * m + Q * a));
                    buf_st4(make_float4(0.f, 0.f, 0.f, 0.f), tape, v_quad, pend2_base + 16u * (TPS * m + Q * a));
                }
            }
    }

    const int64_t ngroups = (args.B + SPB - 1) / SPB;
    for (int64_t gi = blockIdx.x; gi < ngroups; gi += gridDim.x) {
        const int64_t b = gi * SPB + sq;
        const bool active = b < args.B;
        const int64_t bb = active ? b : args.B - 1;
        const int64_t row = args.sigma_enum ? (bb >> L) : bb;   // the weights' row (sigma enumeration: v >> L)
        const float* wb = args.w + row * n;
        const float* gb = args.g + row * n;
        const bool has_sigma = args.sigma_enum || args.sigma != nullptr;
        const uint32_t sig = args.sigma_enum ? (uint32_t)(bb & (Gm::S - 1))
                                             : has_sigma ? ((uint32_t)args.sigma[bb] & (uint32_t)(Gm::S - 1)) : 0u;

        // ------------------------------------------------------------------ forward: R~ and Q
#pragma unroll
        for (int m = 0; m < QPT; ++m) {
            const int j = tau + TPS * m;
            float4 r;
            r.x = (!has_sigma || (uint32_t)(4 * j + 0) == (sig & (G - 1))) ? 0.f : kNeg;
            r.y = (!has_sigma || (uint32_t)(4 * j + 1) == (sig & (G - 1))) ? 0.f : kNeg;
            r.z = (!has_sigma || (uint32_t)(4 * j + 2) == (sig & (G - 1))) ? 0.f : kNeg;
            r.w = (!has_sigma || (uint32_t)(4 * j + 3) == (sig & (G - 1))) ? 0.f : kNeg;
            const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
            *reinterpret_cast<float4*>(mr + 4 * j) = r;
            *reinterpret_cast<float4*>(mq + 4 * j) = z;
            store_quad(r, z, 0u, m);
        }
        lds_barrier();

        float4 fc[4];   // codebook rows of the next quad, when they come from memory
        // One forward step: R~_{t+1} and Q^_{t+1} from R~_t and Q^_t - kq (LDS, one buffer each: every input is read
        // before a barrier, then the outputs overwrite them), normaliser N subtracted; to LDS and, when `store`, to the
        // tape rows at roff.  lmax, lq: this thread's maximum of R~_{t+1} and the Q^ of the group attaining it.  The
        // first pass and the checkpoint recompute both run it; fc must hold the first quad's codebook rows.
        auto fwd_step = [&](int t, float N, float kq, bool store, uint32_t roff, float& lmax, float& lq) {
            float rin[QPT][4], qin[QPT][4];
#pragma unroll
            for (int m = 0; m < QPT; ++m)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    rin[m][a] = mr[tau + TPS * m + Q * a];
                    qin[m][a] = mq[tau + TPS * m + Q * a] - kq;
                }
            lds_barrier();   // every input read before any output overwrites it
            const float wt = wb[t] * scale;
            const float gt = gb[t] * inv_scale;
            lmax = -3.0e38f;
            lq = 0.f;
#pragma unroll
            for (int m = 0; m < QPT; ++m) {
                const int j = tau + TPS * m;
                float4 c0, c1, c2, c3;
                if constexpr (!CB_REG) {
                    c0 = fc[0]; c1 = fc[1]; c2 = fc[2]; c3 = fc[3];
                    const int m2 = (m + 1) % QPT;   // the last quad fetches the next step's first
#pragma unroll
                    for (int a = 0; a < 4; ++a) fc[a] = cb_row<L, TPS, CB_REG>(cbr, cbs, v_cb, m2, a);
                } else {
                    c0 = cb_row<L, TPS, CB_REG>(cbr, cbs, v_cb, m, 0);
                    c1 = cb_row<L, TPS, CB_REG>(cbr, cbs, v_cb, m, 1);
                    c2 = cb_row<L, TPS, CB_REG>(cbr, cbs, v_cb, m, 2);
                    c3 = cb_row<L, TPS, CB_REG>(cbr, cbs, v_cb, m, 3);
                }
                const float cv[4][4] = {{c0.x, c0.y, c0.z, c0.w}, {c1.x, c1.y, c1.z, c1.w},
                                        {c2.x, c2.y, c2.z, c2.w}, {c3.x, c3.y, c3.z, c3.w}};
                float ro[4], qo[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float x[4], z[4];
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        const float d = fmaf(cv[a][i], scale, -wt);
                        x[a] = fmaf(-d, d, rin[m][a]);
                        z[a] = fmaf(gt, d, qin[m][a]);
                    }
                    const float mx = max4(x[0], x[1], x[2], x[3]);
                    const float e0 = ex2(x[0] - mx), e1 = ex2(x[1] - mx), e2 = ex2(x[2] - mx), e3 = ex2(x[3] - mx);
                    const float s = (e0 + e1) + (e2 + e3);
                    ro[i] = (mx - N) + lg2(s);
                    qo[i] = fmaf(e0, z[0], fmaf(e1, z[1], fmaf(e2, z[2], e3 * z[3]))) * rcp(s);
                    const bool up = ro[i] > lmax;
                    lmax = up ? ro[i] : lmax;
                    lq = up ? qo[i] : lq;
                    if ((i + 1) % kGradFwdGroups == 0) {
                        pin_order(ro[i], qo[i]);
                        pin_order(lmax, lq);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                const float4 r4 = make_float4(ro[0], ro[1], ro[2], ro[3]);
                const float4 q4 = make_float4(qo[0], qo[1], qo[2], qo[3]);
                *reinterpret_cast<float4*>(mr + 4 * j) = r4;
                *reinterpret_cast<float4*>(mq + 4 * j) = q4;
                if (store) store_quad(r4, q4, roff, m);
            }
        };
        auto prime_fc = [&]() {
#pragma unroll
            for (int a = 0; a < 4; ++a)
                fc[a] = !CB_REG ? cb_row<L, TPS, CB_REG>(cbr, cbs, v_cb, 0, a) : make_float4(0.f, 0.f, 0.f, 0.f);
        };

        double A = 0.0;
        float N = 0.f;
        float kq = 0.f;       // kappa_t: Q^_t at the most likely group of R~_t, subtracted on input
        float K = 0.f;        // K_{t-1} = sum of the kappas applied so far
        float N_last = 0.f, K_last = 0.f;
        prime_fc();
        for (int t = 0; t < n; ++t) {
            if (tau == 0) {
                buf_st(N, tape, sq * slot_bytes, nrm_base + 4u * t);
                buf_st(K, tape, sq * slot_bytes, kq_base + 4u * t);
                if constexpr (CK) buf_st(kq, tape, sq * slot_bytes, kqi_base + 4u * t);
            }
            K_last = K;
            K += kq;
            float lmax, lq;
            fwd_step(t, N, kq, rows.stored(t + 1), rows.off(t + 1), lmax, lq);
            seg_argmax_payload<SEG>(lmax, lq);
            if constexpr (WPS > 1) {
                if (lane == 0) {
                    redmax[t & 1][sq][wv] = lmax;
                    redq[t & 1][sq][wv] = lq;
                }
            }
            lds_barrier();
            if constexpr (WPS > 1) {
                static_assert(WPS <= 16, "per-wave slots are combined inside one 16-lane row");
                const int qs = lane & 15;
                float bm = qs < WPS ? redmax[t & 1][sq][qs] : -3.0e38f;
                float bq = qs < WPS ? redq[t & 1][sq][qs] : 0.f;
                row16_argmax_payload(bm, bq);   // first wave attaining the max, as a serial scan would pick
                lmax = bm;
                lq = bq;
            }
            if constexpr (SPB == 1) {
                lmax = uniform_f(lmax);
                lq = uniform_f(lq);
            }
            A += (double)N;
            N_last = N;
            N = lmax;
            kq = grid_offset(lq);
        }
        // rz = log2 Z - A_n and E[F] (which centres the covariance of the backward pass)
        float rz, EF, Kfin;   // E[F] = Kfin + EF: the offsets' exact sum, and the centred rest
        RT rzr;   // rz in the precision of the running sums
        if (!has_sigma) {
            float z0 = 0.f, z1 = 0.f;
#pragma unroll
            for (int m = 0; m < QPT; ++m) {
                const int j = tau + TPS * m;
                const float4 o = *reinterpret_cast<const float4*>(mr + 4 * j);
                const float4 q = *reinterpret_cast<const float4*>(mq + 4 * j);
                const float p0 = ex2(o.x - N), p1 = ex2(o.y - N), p2 = ex2(o.z - N), p3 = ex2(o.w - N);
                z0 += (p0 + p1) + (p2 + p3);
                z1 += fmaf(p0, q.x, fmaf(p1, q.y, fmaf(p2, q.z, p3 * q.w)));
            }
            z0 = seg_sum_fast<SEG>(z0);
            z1 = seg_sum_fast<SEG>(z1);
            if constexpr (WPS > 1) {
                if (lane == 0) redsum[n & 1][sq][wv] = make_float4(z0, z1, 0.f, 0.f);
            }
            lds_barrier();
            if constexpr (WPS > 1) {
                z0 = 0.f;
                z1 = 0.f;
#pragma unroll
                for (int q = 0; q < WPS; ++q) {
                    z0 += redsum[n & 1][sq][q].x;
                    z1 += redsum[n & 1][sq][q].y;
                }
            }
            rz = N + lg2(z0);
            rzr = (RT)N + (RT)lg2(z0);
            EF = z1 / z0;   // the final outputs Q^_n carry the offset K_{n-1}
            Kfin = K;
            __syncthreads();   // tape writes of the forward pass visible to every thread of the block
        } else {
            // R~_{n-1}, Q_{n-1} are on the tape (the last step overwrote LDS), written by other threads
            __syncthreads();
            const float d = fmaf(args.cb[sig], scale, -(wb[n - 1] * scale));
            const float r = buf_ld_nt(tape, sq * slot_bytes, rows.off(n - 1) + (PAIR ? 8u : 4u) * (sig >> 2));
            const float q = PAIR ? buf_ld_nt(tape, sq * slot_bytes, rows.off(n - 1) + 8u * (sig >> 2) + 4u)
                                      : buf_ld_nt(tape, sq * slot_bytes, q_base + rows.off(n - 1) + 4u * (sig >> 2));
            rz = (r < 0.5f * kNeg) ? kNeg : fmaf(-d, d, r) - N_last;
            rzr = (r < 0.5f * kNeg) ? (RT)kNeg : (RT)fmaf(-d, d, r) - (RT)N_last;
            EF = fmaf(gb[n - 1] * inv_scale, d, q);   // Q^_{n-1} carries the offset K_{n-2}
            Kfin = K_last;
        }
        const bool valid = rz > 0.5f * kNeg;

        // ------------------------------------------------------------------ backward: B~ and P, covariance
        float Nb = 0.f;
        RT C = 0;
        RT D = 0;
        float lam = 1.f;   // 1 / (posterior total of the previous step), GC only
        float m2p = 0.f;   // E[E[F | s] - E[F]] of the previous step, GCM = 2
        float kb = 0.f;   // kappa_{t+1} = g_{t+1} (w_soft_{t+1} - w_{t+1}), subtracted from the P^ inputs
        float H = 0.f;    // sum of the kappas of the steps after t
        int t = n - 1;
        if (!has_sigma) {
#pragma unroll
            for (int m = 0; m < QPT; ++m) {
                const int j = tau + TPS * m;
                const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
                *reinterpret_cast<float4*>(mr + 4 * j) = z;
                *reinterpret_cast<float4*>(mq + 4 * j) = z;
            }
        } else {
            // s_n = sigma: posterior at n-1 is the indicator of sigma (so grad_{n-1} = 0, w_soft_{n-1} = c(sigma));
            // the messages left are B_{n-2}(sigma >> 2) = theta_{n-1}(sigma), P^_{n-2}(sigma >> 2) = g (c(sigma) - w),
            // and kappa_{n-1} = g (c(sigma) - w) as well.  theta goes into the offset C and the message starts at 0,
            // so the next step's branch terms are not rounded at theta's magnitude (a hundred or more in log2 units)
            const float d = fmaf(args.cb[sig], scale, -(wb[n - 1] * scale));
            const float th = -d * d;
            const float pz = gb[n - 1] * inv_scale * d;
#pragma unroll
            for (int m = 0; m < QPT; ++m)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const uint32_t u = (uint32_t)(tau + TPS * m + Q * a);
                    mr[u] = (u == (sig >> 2)) ? 0.f : kNeg;
                    mq[u] = (u == (sig >> 2)) ? pz : 0.f;
                }
            if (tau == 0 && active) {
                if (!GC || args.grad) args.grad[b * n + n - 1] = valid ? 0.f : __builtin_nanf("");
                if (args.w_soft) args.w_soft[b * n + n - 1] = valid ? args.cb[sig] : __builtin_nanf("");
            }
            D = N_last;
            C = (RT)th;
            kb = grid_offset(pz);
            H = kb;
            t = n - 2;
            if constexpr (GC) {   // p_{n-1} is the indicator of sigma and E[F | s_{n-1}] = E[F]: dL/dc(sigma) += g_{n-1}
                const uint32_t js = (sig >> 2) & (uint32_t)(Q - 1);
                if (active && valid && (uint32_t)tau == js % (uint32_t)TPS) {
                    const float acc = buf_ld(tape, sq * slot_bytes, acc_base + 4u * sig);
                    buf_st(acc + gb[n - 1], tape, sq * slot_bytes, acc_base + 4u * sig);
                }
            }
        }
        lds_barrier();

        // loads of later groups (forward messages R~, Q^ of this step, codebook rows) are issued ahead, in rings
        constexpr int NGS = 4 * QPT;   // groups per step
        constexpr int TD = BCJR_GRAD_TAPE_DEPTH < NGS ? BCJR_GRAD_TAPE_DEPTH : NGS;   // tape prefetch depth
        constexpr int CBD = BCJR_GRAD_CB_DEPTH < NGS ? BCJR_GRAD_CB_DEPTH : NGS;      // codebook prefetch depth
        static_assert(NGS % TD == 0 && NGS % CBD == 0, "the prefetch rings must divide the groups of a step");
        float rt_q[TD], qt_q[TD];   // R~_t and Q^_t of the next TD groups, group gi in slot gi % TD
        // the first TD groups of step tt into the ring
        auto prefetch_row = [&](int tt) {
#pragma unroll
            for (int q = 0; q < TD; ++q) load_group(rt_q[q], qt_q[q], rows.off(tt), q >> 2, q & 3);
        };
        float4 cr_q[CBD];   // codebook rows of the next CBD groups, group gi in slot gi % CBD
#pragma unroll
        for (int q = 0; q < CBD; ++q) cr_q[q] = make_float4(0.f, 0.f, 0.f, 0.f);
        float4 ac_n = make_float4(0.f, 0.f, 0.f, 0.f);   // the next group's accumulator (GC)
        float4 pe_n = make_float4(0.f, 0.f, 0.f, 0.f);   // and its pending contributions (GCM = 2)
        float4 pf_n = make_float4(0.f, 0.f, 0.f, 0.f);
        if (t >= 0) {
            prefetch_row(t);
            if constexpr (!CB_REG) {
#pragma unroll
                for (int q = 0; q < CBD; ++q) cr_q[q] = cb_row<L, TPS, CB_REG>(cbr, cbs, v_cb, q >> 2, q & 3);
            }
            if constexpr (GC) ac_n = buf_ld4(tape, v_quad, acc_base);
            if constexpr (EXACT) {
                pe_n = buf_ld4(tape, v_quad, pend_base);
                pf_n = buf_ld4(tape, v_quad, pend2_base);
            }
        }
        const int t_out = t;   // last step whose outputs the loop below produces
        float w_nx = 0.f, g_nx = 0.f, N_nx = 0.f, K_nx = 0.f;
        if (t >= 0) {
            w_nx = wb[t];
            g_nx = gb[t];
            N_nx = buf_ld_nt(tape, sq * slot_bytes, nrm_base + 4u * t);
            K_nx = buf_ld_nt(tape, sq * slot_bytes, kq_base + 4u * t);
        }
        while (t >= 0) {
        const int t0 = ck ? (t / ck) * ck : 0;   // first step of this segment
        if (CK && ck) {
            // keep this thread's share of both backward messages (the quads it reads at step t), rebuild the
            // segment's rows t0+1..t of R~ and Q^ from checkpoint t0 with the stored normalisers and offsets, then
            // restore the messages
#pragma unroll
            for (int m = 0; m < QPT; ++m) {
                const int j = tau + TPS * m;
                buf_st4(*reinterpret_cast<const float4*>(mr + 4 * j), tape, v_quad, save_base + 16u * TPS * m);
                buf_st4(*reinterpret_cast<const float4*>(mq + 4 * j), tape, v_quad, save_base + G * 4u + 16u * TPS * m);
            }
            lds_barrier();   // every share read before the recompute overwrites the buffers
#pragma unroll
            for (int m = 0; m < QPT; ++m) {
                const int j = tau + TPS * m;
                if constexpr (PAIR) {
                    const float4 p0 = buf_ld4(tape, v_pair, rows.off(t0) + 32u * TPS * m);
                    const float4 p1 = buf_ld4(tape, v_pair, rows.off(t0) + 32u * TPS * m + 16u);
                    *reinterpret_cast<float4*>(mr + 4 * j) = make_float4(p0.x, p0.z, p1.x, p1.z);
                    *reinterpret_cast<float4*>(mq + 4 * j) = make_float4(p0.y, p0.w, p1.y, p1.w);
                } else {
                    *reinterpret_cast<float4*>(mr + 4 * j) = buf_ld4(tape, v_quad, rows.off(t0) + 16u * TPS * m);
                    *reinterpret_cast<float4*>(mq + 4 * j) =
                        buf_ld4(tape, v_quad, q_base + rows.off(t0) + 16u * TPS * m);
                }
            }
            lds_barrier();
            prime_fc();
            for (int tt = t0; tt < t; ++tt) {
                float Nr = buf_ld(tape, sq * slot_bytes, nrm_base + 4u * tt);
                float kr = buf_ld(tape, sq * slot_bytes, kqi_base + 4u * tt);
                if constexpr (SPB == 1) {
                    Nr = uniform_f(Nr);
                    kr = uniform_f(kr);
                }
                float lm, lqr;
                fwd_step(tt, Nr, kr, true, rows.off(tt + 1), lm, lqr);
                lds_barrier();
            }
            __syncthreads();   // the rebuilt rows, written by other threads, before the backward reads them
#pragma unroll
            for (int m = 0; m < QPT; ++m) {
                const int j = tau + TPS * m;
                *reinterpret_cast<float4*>(mr + 4 * j) = buf_ld4(tape, v_quad, save_base + 16u * TPS * m);
                *reinterpret_cast<float4*>(mq + 4 * j) = buf_ld4(tape, v_quad, save_base + G * 4u + 16u * TPS * m);
            }
            lds_barrier();
            prefetch_row(t);
        }
        for (; t >= t0; --t) {
            float bin[QPT][4], pin[QPT][4];
#pragma unroll
            for (int m = 0; m < QPT; ++m) {
                const float4 v = *reinterpret_cast<const float4*>(mr + 4 * (tau + TPS * m));
                const float4 p = *reinterpret_cast<const float4*>(mq + 4 * (tau + TPS * m));
                bin[m][0] = v.x; bin[m][1] = v.y; bin[m][2] = v.z; bin[m][3] = v.w;
                pin[m][0] = p.x - kb; pin[m][1] = p.y - kb; pin[m][2] = p.z - kb; pin[m][3] = p.w - kb;
            }
            lds_barrier();
            const float wt = w_nx * scale;
            const float gt = g_nx * inv_scale;
            const float gnat = g_nx;
            float Nt = N_nx, Kt = K_nx;
            if (t > 0) {   // the next step's weight, upstream gradient and forward scalars, one step ahead
                w_nx = wb[t - 1];
                g_nx = gb[t - 1];
                N_nx = buf_ld_nt(tape, sq * slot_bytes, nrm_base + 4u * (t - 1));
                K_nx = buf_ld_nt(tape, sq * slot_bytes, kq_base + 4u * (t - 1));
            }
            if constexpr (SPB == 1) {
                Nt = uniform_f(Nt);
                Kt = uniform_f(Kt);
            }
            D += Nt;
            const float ref = (float)((rzr + D) - C);
            // E[F | s_t = s] - E[F] = Q^_t(s >> 2) + cst + g_t (c(s) - w_t) + P''_t(s & (G-1)), cst per step
            const float brk = (Kt - Kfin) + H;   // exact (offsets on the 2^-6 grid)
            const float cst = brk - EF;
            float lmax = -3.0e38f, S0 = 0.f, S1 = 0.f, S2 = 0.f, S3 = 0.f;
#pragma unroll
            for (int m = 0; m < QPT; ++m) {
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int gi = 4 * m + a, slot = gi % TD;
                    const float rt = rt_q[slot];
                    const float qt = qt_q[slot] + cst;
                    const float qs = qt_q[slot] - EF;   // GC: the small parts of E[F | s] - E[F]
                    float4 cr;
                    if constexpr (CB_REG) cr = cb_row<L, TPS, CB_REG>(cbr, cbs, v_cb, m, a);
                    else cr = cr_q[gi % CBD];
                    // before this group's math, issue the codebook row CBD groups ahead, then the tape loads of the
                    // group TD ahead (of the next step's groups once past this one's last); in checkpoint mode a row
                    // past the segment is read again once rebuilt
                    const bool last = (m == QPT - 1) && (a == 3);
                    const int m2 = (a == 3) ? m + 1 : m, a2 = (a + 1) & 3;
                    if constexpr (!CB_REG) {
                        const int gc = gi + CBD;
                        if (gc < NGS) cr_q[gi % CBD] = cb_row<L, TPS, CB_REG>(cbr, cbs, v_cb, gc >> 2, gc & 3);
                        else if (t > 0)
                            cr_q[gi % CBD] = cb_row<L, TPS, CB_REG>(cbr, cbs, v_cb, (gc - NGS) >> 2, (gc - NGS) & 3);
                    }
                    {
                        const int gn = gi + TD;
                        if (gn < NGS) {
                            load_group(rt_q[slot], qt_q[slot], rows.off(t), gn >> 2, gn & 3);
                        } else if (t > 0) {
                            const int g2 = gn - NGS;
                            load_group(rt_q[slot], qt_q[slot], rows.off(t - 1), g2 >> 2, g2 & 3);
                        }
                    }
                    float4 ac = ac_n, pe = pe_n, pf = pf_n;
                    if constexpr (GC) {
                        if (!last) ac_n = buf_ld4(tape, v_quad, acc_base + 16u * (TPS * m2 + Q * a2));
                        else if (t > 0) ac_n = buf_ld4(tape, v_quad, acc_base);
                    }
                    if constexpr (EXACT) {
                        if (!last) {
                            pe_n = buf_ld4(tape, v_quad, pend_base + 16u * (TPS * m2 + Q * a2));
                            pf_n = buf_ld4(tape, v_quad, pend2_base + 16u * (TPS * m2 + Q * a2));
                        } else if (t > 0) {
                            pe_n = buf_ld4(tape, v_quad, pend_base);
                            pf_n = buf_ld4(tape, v_quad, pend2_base);
                        }
                    }
                    const float d0 = fmaf(cr.x, scale, -wt), d1 = fmaf(cr.y, scale, -wt);
                    const float d2 = fmaf(cr.z, scale, -wt), d3 = fmaf(cr.w, scale, -wt);
                    const float y0 = fmaf(-d0, d0, bin[m][0]), y1 = fmaf(-d1, d1, bin[m][1]);
                    const float y2 = fmaf(-d2, d2, bin[m][2]), y3 = fmaf(-d3, d3, bin[m][3]);
                    const float z0 = fmaf(gt, d0, pin[m][0]), z1 = fmaf(gt, d1, pin[m][1]);
                    const float z2 = fmaf(gt, d2, pin[m][2]), z3 = fmaf(gt, d3, pin[m][3]);
                    const float mx = max4(y0, y1, y2, y3);
                    const float e0 = ex2(y0 - mx), e1 = ex2(y1 - mx), e2 = ex2(y2 - mx), e3 = ex2(y3 - mx);
                    const float s = (e0 + e1) + (e2 + e3);
                    const float ez = fmaf(e0, z0, fmaf(e1, z1, fmaf(e2, z2, e3 * z3)));
                    const float ed0 = e0 * d0, ed1 = e1 * d1, ed2 = e2 * d2, ed3 = e3 * d3;
                    const float ed = (ed0 + ed1) + (ed2 + ed3);
                    // E[F | s] - E[F] per state, formed before any product: its two parts nearly cancel at the
                    // likely states, and multiplying them separately would keep their rounding
                    float r0, r1, r2, r3;
                    if constexpr (GC) {
                        // dL/dc weighs it by (2/T)(w - c) state by state, so at a frozen posterior the roundings of
                        // its two O(1) parts (g_t (c - w) at the likely state and the offsets' bracket, which cancel
                        // there) would survive: join them inside one fma, exact before its single rounding, and add
                        // the small parts after
                        r0 = fmaf(gt, d0, brk) + (pin[m][0] + qs);
                        r1 = fmaf(gt, d1, brk) + (pin[m][1] + qs);
                        r2 = fmaf(gt, d2, brk) + (pin[m][2] + qs);
                        r3 = fmaf(gt, d3, brk) + (pin[m][3] + qs);
                    } else {
                        r0 = z0 + qt;
                        r1 = z1 + qt;
                        r2 = z2 + qt;
                        r3 = z3 + qt;
                    }
                    const float er = fmaf(e0, r0, fmaf(e1, r1, fmaf(e2, r2, e3 * r3)));
                    const float edr = fmaf(ed0, r0, fmaf(ed1, r1, fmaf(ed2, r2, ed3 * r3)));
                    const float out = (mx - Nb) + lg2(s);
                    const float f = ex2((mx + rt) - ref);
                    S0 = fmaf(f, s, S0);
                    S1 = fmaf(f, ed, S1);
                    S2 = fmaf(f, er, S2);
                    S3 = fmaf(f, edr, S3);
                    lmax = run_max(lmax, out);
                    if constexpr (GC) {
                        if constexpr (EXACT) {
                            // the previous step's pending contributions join the accumulator, centred by that step's
                            // m2 and divided by its total (lam); this step's wait
                            ac.x = fmaf(lam, fmaf(m2p, pf.x, pe.x), ac.x);
                            ac.y = fmaf(lam, fmaf(m2p, pf.y, pe.y), ac.y);
                            ac.z = fmaf(lam, fmaf(m2p, pf.z, pe.z), ac.z);
                            ac.w = fmaf(lam, fmaf(m2p, pf.w, pe.w), ac.w);
                            const float ga = f * gnat, ka = f * kap;
                            pe.x = fmaf(ga, e0, -ka * (ed0 * r0));
                            pe.y = fmaf(ga, e1, -ka * (ed1 * r1));
                            pe.z = fmaf(ga, e2, -ka * (ed2 * r2));
                            pe.w = fmaf(ga, e3, -ka * (ed3 * r3));
                            pf.x = ka * ed0;
                            pf.y = ka * ed1;
                            pf.z = ka * ed2;
                            pf.w = ka * ed3;
                            if (active) {
                                buf_st4(ac, tape, v_quad, acc_base + 16u * (TPS * m + Q * a));
                                buf_st4(pe, tape, v_quad, pend_base + 16u * (TPS * m + Q * a));
                                buf_st4(pf, tape, v_quad, pend2_base + 16u * (TPS * m + Q * a));
                            }
                        } else {
                            // p_t(s) [g_t + (2/T)(w_t - c(s))(E[F | s] - E[F])] with p_t(s) = lam f e_i
                            const float fa = lam * f;
                            const float ga = fa * gnat, ka = fa * kap;
                            ac.x = fmaf(ga, e0, fmaf(-ka, ed0 * r0, ac.x));
                            ac.y = fmaf(ga, e1, fmaf(-ka, ed1 * r1, ac.y));
                            ac.z = fmaf(ga, e2, fmaf(-ka, ed2 * r2, ac.z));
                            ac.w = fmaf(ga, e3, fmaf(-ka, ed3 * r3, ac.w));
                            if (active) buf_st4(ac, tape, v_quad, acc_base + 16u * (TPS * m + Q * a));
                        }
                    }
                    const uint32_t u = (uint32_t)(tau + TPS * m + Q * a);
                    mr[u] = out;            // at t = 0 these land in buffers nobody reads
                    mq[u] = ez * rcp(s);
                    if ((a + 1) % kGradBwdGroups == 0) {
                        pin_order(S0, S1, lmax);
                        pin_order(S2, S3);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
            lmax = seg_max_fast<SEG>(lmax);
            S0 = seg_sum_fast<SEG>(S0);
            S1 = seg_sum_fast<SEG>(S1);
            S2 = seg_sum_fast<SEG>(S2);
            S3 = seg_sum_fast<SEG>(S3);
            if constexpr (WPS > 1) {
                if (lane == 0) {
                    redsum2[t & 1][sq][wv] = make_float4(S0, S1, S2, 0.f);
                    redmax[t & 1][sq][wv] = lmax;
                    buf_st4(make_float4(S0, S1, S2, S3), tape, sq * slot_bytes,
                            part_base + 16u * (uint32_t)(t * WPS + wv));
                }
            }
            lds_barrier();
            float m1;   // w_soft_t - w_t in scaled codebook units
            if constexpr (WPS > 1) {
                const int qs = lane & 15;
                const float4 p = qs < WPS ? redsum2[t & 1][sq][qs] : make_float4(0.f, 0.f, 0.f, 0.f);
                lmax = row16_max(qs < WPS ? redmax[t & 1][sq][qs] : -3.0e38f);
                // only the P offset uses m1 here, and any value common to the block serves: the approximate
                // reciprocal keeps the division off the step's critical path
                const float s0b = row16_sum(p.x);
                m1 = row16_sum(p.y) * rcp(s0b);
                if constexpr (GC) lam = rcp(s0b);
                if constexpr (EXACT) m2p = row16_sum(p.z) * rcp(s0b);
            } else {
                m1 = S1 * (1.0f / S0);
                if constexpr (GC) lam = 1.0f / S0;
                if constexpr (EXACT) m2p = S2 * (1.0f / S0);
            }
            if constexpr (WPS == 1) {
                if (tau == 0 && active) {
                    const float i0 = 1.0f / S0;
                    const float m2 = S2 * i0;
                    const float cov = fmaf(-m1, m2, S3 * i0);   // Cov(c' - w', E[F | s] - E[F]), c' scaled
                    if (!GC || args.grad)
                        args.grad[b * n + t] = valid ? args.two_over_T * cov * inv_scale : __builtin_nanf("");
                    if (args.w_soft) args.w_soft[b * n + t] = valid ? fmaf(m1, inv_scale, wb[t]) : __builtin_nanf("");
                }
            }
            kb = grid_offset(gt * m1);
            if constexpr (SPB == 1) {
                lmax = uniform_f(lmax);
                kb = uniform_f(kb);
                if constexpr (GC) lam = uniform_f(lam);
                if constexpr (EXACT) m2p = uniform_f(m2p);
            }
            H += kb;
            C += Nb;
            Nb = lmax;
        }
        }   // segments
        if constexpr (WPS > 1) {
            // outputs of steps 0..t_out from the per-wave partial sums, one step per thread, summed over the waves
            // in wave order
            __syncthreads();
            for (int tt = tau; tt <= t_out; tt += TPS) {
                float S0 = 0.f, S1 = 0.f, S2 = 0.f, S3 = 0.f;
#pragma unroll
                for (int q = 0; q < WPS; ++q) {
                    const float4 p = buf_ld4(tape, sq * slot_bytes, part_base + 16u * (uint32_t)(tt * WPS + q));
                    S0 += p.x;
                    S1 += p.y;
                    S2 += p.z;
                    S3 += p.w;
                }
                const float i0 = 1.0f / S0;
                const float m1 = S1 * i0;
                const float m2 = S2 * i0;
                const float cov = fmaf(-m1, m2, S3 * i0);   // Cov(c' - w', E[F | s] - E[F]), c' in scaled units
                if (active) {
                    if (!GC || args.grad)
                        args.grad[b * n + tt] = valid ? args.two_over_T * cov * inv_scale : __builtin_nanf("");
                    if (args.w_soft) args.w_soft[b * n + tt] = valid ? fmaf(m1, inv_scale, wb[tt]) : __builtin_nanf("");
                }
            }
        }
        if constexpr (EXACT) {   // the last step's pending contributions; the arrays left at zero
            if (active) {
#pragma unroll
                for (int m = 0; m < QPT; ++m)
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        const uint32_t o = 16u * (TPS * m + Q * a);
                        float4 ac = buf_ld4(tape, v_quad, acc_base + o);
                        const float4 pe = buf_ld4(tape, v_quad, pend_base + o);
                        const float4 pf = buf_ld4(tape, v_quad, pend2_base + o);
                        ac.x = fmaf(lam, fmaf(m2p, pf.x, pe.x), ac.x);
                        ac.y = fmaf(lam, fmaf(m2p, pf.y, pe.y), ac.y);
                        ac.z = fmaf(lam, fmaf(m2p, pf.z, pe.z), ac.z);
                        ac.w = fmaf(lam, fmaf(m2p, pf.w, pe.w), ac.w);
                        buf_st4(ac, tape, v_quad, acc_base + o);
                        buf_st4(make_float4(0.f, 0.f, 0.f, 0.f), tape, v_quad, pend_base + o);
                        buf_st4(make_float4(0.f, 0.f, 0.f, 0.f), tape, v_quad, pend2_base + o);
                    }
            }
        }
        if constexpr (GC) {
            if (active && !valid) {   // no admissible path: the loss, hence its gradient, is undefined
                const float nan = __builtin_nanf("");
#pragma unroll
                for (int m = 0; m < QPT; ++m)
#pragma unroll
                    for (int a = 0; a < 4; ++a)
                        buf_st4(make_float4(nan, nan, nan, nan), tape, v_quad, acc_base + 16u * (TPS * m + Q * a));
            }
        }
        __syncthreads();
    }
    if constexpr (GC && SPB > 1) {
        // the block's sequence slots hold the same states: fold them into slot 0, in slot order (the __syncthreads
        // that ends the last sequence orders every thread's accumulator stores before these loads)
        if (sq == 0) {
#pragma unroll
            for (int m = 0; m < QPT; ++m)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const uint32_t o = acc_base + 16u * (TPS * m + Q * a) + 16u * tau;
                    float4 x = buf_ld4(tape, 0u, o);
                    for (int q = 1; q < SPB; ++q) {
                        const float4 y = buf_ld4(tape, (uint32_t)q * slot_bytes, o);
                        x.x += y.x; x.y += y.y; x.z += y.z; x.w += y.w;
                    }
                    buf_st4(x, tape, 0u, o);
                }
        }
    }
}

// dL/dc = the sum of the per-block accumulators (slot 0 of every block, `count` of them, `stride` bytes apart), in
// block order and in double.  A block of 256 threads covers W = min(2^L, 64) states with 256 / W interleaved runs of
// blocks each; the runs are added in run order, so the result does not depend on timing.
__global__ void __launch_bounds__(256) codebook_reduce_kernel(const unsigned char* ws, size_t stride, uint32_t acc_off,
                                                              int count, int S, float* out) {
    __shared__ double part[256];
    const int W = S < 64 ? S : 64;
    const int R = 256 / W;
    const int r = threadIdx.x / W, v = blockIdx.x * W + threadIdx.x % W;
    double acc = 0.0;
    const unsigned char* base = ws + acc_off + 4 * (size_t)v;
    for (int q = r; q < count; q += R) acc += (double)*reinterpret_cast<const float*>(base + (size_t)q * stride);
    part[threadIdx.x] = acc;
    __syncthreads();
    if (r == 0) {
        double x = part[threadIdx.x];
        for (int q = 1; q < R; ++q) x += part[q * W + threadIdx.x];
        out[v] = (float)x;
    }
}

template <int L, int GCM>
static hipError_t launch_grad_L(const GradArgs& a, int grid, hipStream_t st) {
    if (a.ckpt) hipLaunchKernelGGL((grad_kernel<L, GCM, true>), dim3(grid), dim3(Geo<L>::NT), 0, st, a);
    else hipLaunchKernelGGL((grad_kernel<L, GCM, false>), dim3(grid), dim3(Geo<L>::NT), 0, st, a);
    return hipGetLastError();
}

template <int GCM>
static hipError_t launch_grad_any(int L, const GradArgs& a, int grid, hipStream_t st) {
    switch (L) {
        case 4: return launch_grad_L<4, GCM>(a, grid, st);
        case 5: return launch_grad_L<5, GCM>(a, grid, st);
        case 6: return launch_grad_L<6, GCM>(a, grid, st);
        case 7: return launch_grad_L<7, GCM>(a, grid, st);
        case 8: return launch_grad_L<8, GCM>(a, grid, st);
        case 9: return launch_grad_L<9, GCM>(a, grid, st);
        case 10: return launch_grad_L<10, GCM>(a, grid, st);
        case 11: return launch_grad_L<11, GCM>(a, grid, st);
        case 12: return launch_grad_L<12, GCM>(a, grid, st);
        case 13: return launch_grad_L<13, GCM>(a, grid, st);
        case 14: return launch_grad_L<14, GCM>(a, grid, st);
        case 15: return launch_grad_L<15, GCM>(a, grid, st);
        case 16: return launch_grad_L<16, GCM>(a, grid, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_grad(int L, const GradArgs& a, int grid, hipStream_t st) {
    return launch_grad_any<0>(L, a, grid, st);
}

// dL/dc from `count` per-slot accumulators of S floats each, `stride` bytes apart starting at ws + acc_off.
hipError_t launch_codebook_reduce(const unsigned char* ws, size_t stride, uint32_t acc_off, int count, int S,
                                  float* out, hipStream_t st) {
    const int W = S < 64 ? S : 64;
    hipLaunchKernelGGL(codebook_reduce_kernel, dim3(S / W), dim3(256), 0, st, ws, stride, acc_off, count, S, out);
    return hipGetLastError();
}

hipError_t launch_grad_codebook(int L, const GradArgs& a, int grid, hipStream_t st, float* grad_codebook) {
    // boundary-state mode normalises each step by its own total (GCM = 2)
    const bool exact = a.sigma != nullptr || a.sigma_enum;
    const hipError_t e = exact ? launch_grad_any<2>(L, a, grid, st) : launch_grad_any<1>(L, a, grid, st);
    if (e != hipSuccess) return e;
    const GeoRT g = geo_rt(L);
    const int S = 1 << L;
    const int W = S < 64 ? S : 64;
    // the accumulator sits after the tape, the two scalar tracks and (several waves per sequence) the partial sums
    const size_t n = (size_t)a.n;
    const size_t acc_off = 2 * align256(TapeRows::rows(a.ckpt, (int)n) * (size_t)g.G * 4) + 2 * align256(n * 4) +
                           (g.WPS > 1 ? align256(n * (size_t)g.WPS * 16) : 0);
    hipLaunchKernelGGL(codebook_reduce_kernel, dim3(S / W), dim3(256), 0, st, a.ws, a.slot_bytes * g.SPB,
                       (uint32_t)acc_off, grid, S, grad_codebook);
    return hipGetLastError();
}

}  // namespace bcjr
