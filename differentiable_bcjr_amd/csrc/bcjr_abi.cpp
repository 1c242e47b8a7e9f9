// bcjr_abi.cpp -- the C-ABI of libbcjr.so (declared in include/bcjr.h): argument checks, workspace planning and
// kernel dispatch.  Every check runs on the host before any HIP call, so all error paths are testable without a GPU.
#include "bcjr.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <mutex>

#include "trellis.hpp"

namespace bcjr {

struct SoftArgs;
struct GradArgs;
struct ViterbiArgs;
hipError_t launch_soft(int L, const SoftArgs& a, int grid, hipStream_t st);
hipError_t launch_grad(int L, const GradArgs& a, int grid, hipStream_t st);
hipError_t launch_grad_codebook(int L, const GradArgs& a, int grid, hipStream_t st, float* grad_codebook);
hipError_t launch_viterbi(int L, const ViterbiArgs& a, int grid, hipStream_t st);
hipError_t launch_tb_soft_combine(const float* ws_all, const float* lz_all, int64_t rows, int n, int S,
                                  float* w_soft, float* log_z, hipStream_t st);
hipError_t launch_tb_grad_combine(const float* ws_all, const float* lz_all, const float* gr_all, const float* g,
                                  int64_t rows, int n, int S, float two_over_T, float* grad, float* w_soft,
                                  hipStream_t st);
hipError_t launch_tb_select(const float* costs, int64_t rows, int S, int32_t* sigma, int32_t* sigma_out,
                            hipStream_t st);
hipError_t launch_tb_rotate_sigma(const int32_t* states_rot, int64_t rows, int n, int pos, int32_t* sigma,
                                  int32_t* sigma_out, hipStream_t st);
hipError_t launch_tb_rotate_rows(const float* w, int64_t rows, int nv, int shift, float* out, hipStream_t st);
struct GenArgs;
hipError_t launch_general(int op, int k, int V, const GenArgs& a, int grid, int threads, size_t lds_bytes,
                          hipStream_t st);
hipError_t launch_codebook_reduce(const unsigned char* ws, size_t stride, uint32_t acc_off, int count, int S,
                                  float* out, hipStream_t st);

}  // namespace bcjr

#include "kernel_args.hpp"

namespace {

using namespace bcjr;

constexpr int64_t kMaxN = 4096;   // keeps every per-block workspace offset (two [n+1][2^14] float tapes) below 2^31
constexpr int64_t kMaxB = 2147483647LL;
constexpr float kMinT = 1e-12f;
constexpr int32_t kMaxTailBitingExactL = 10;   // the exact choice decodes every one of the 2^L start states

struct Plan {
    int grid;
    int slots;
    size_t slot_bytes;
    size_t total;
};

constexpr int32_t kMaxGenK = 4;   // the general trellis kernels: 1 <= k <= 4
constexpr int32_t kMaxGenV = 2;   // and V = 1 or 2 weights per step

// L >= 4 for every k: the k = 2 kernels hand out quads of 16 states, and the general kernels give a thread at least
// 16 states (a 64-lane wave covers the 2^L states of the smallest trellis several times over).
constexpr int32_t kMinL = 4;

int check_dims(int64_t B, int64_t n, int32_t L, int32_t k, int32_t V) {
    if (B < 1 || B > kMaxB || n < 1 || n > kMaxN || k < 1 || L < 2 * k || L < kMinL || L > 16 || V < 1)
        return BCJR_ERR_SHAPE;
    return BCJR_OK;
}

// Compute units of the current device, asked of the runtime once per device.  The persistent grids are sized from
// it (one or more workgroups per CU), and so are the workspaces.  With no device visible (a host that only plans
// workspaces) it is 256, an MI355X's count.
constexpr int kMaxDevices = 64;
constexpr int kDefaultCUs = 256;

int device_cus() {
    static std::atomic<int> cache[kMaxDevices];   // 0 until asked
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return kDefaultCUs;
    int cus = cache[dev].load(std::memory_order_relaxed);
    if (cus > 0) return cus;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        cus = kDefaultCUs;
    cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

// Soft codeword, gradient and Viterbi: the k = 2, V = 1 kernels, or the general ones.
int check_shape_v(int64_t B, int64_t n, int32_t L, int32_t k, int32_t V) {
    const int rc = check_dims(B, n, L, k, V);
    if (rc) return rc;
    if (k > kMaxGenK || V > kMaxGenV) return BCJR_ERR_UNSUPPORTED;
    return BCJR_OK;
}

bool tuned(int32_t k, int32_t V) { return k == 2 && V == 1; }

int check_temp(float T) {
    if (!std::isfinite(T) || !(T >= kMinT)) return BCJR_ERR_TEMP;
    return BCJR_OK;
}

// Grid, slot count and per-slot workspace bytes of one entry point.  One slot per in-flight sequence.  ckpt > 0 (soft
// codeword and gradients): the checkpoint mode, every ckpt-th message row plus one segment's rows and the saved
// backward message(s); the gradients also keep each step's Q input offset.
Plan make_plan(int op, int64_t B, int64_t n, int L, int ckpt = 0) {
    const GeoRT g = geo_rt(L);
    const int64_t groups = (B + g.SPB - 1) / g.SPB;
    const int64_t cap = (int64_t)device_cus() * blocks_per_cu(L);
    Plan p{};
    p.grid = (int)(groups < cap ? groups : cap);
    p.slots = p.grid * g.SPB;
    const size_t msgs = TapeRows::rows(ckpt, (int)n) * (size_t)g.G * 4;   // one float per group per row
    const size_t nrm = (size_t)n * 4;                         // one normaliser per step
    switch (op) {
        case BCJR_OP_SOFT:   // + per-wave (S0, S1) of every step when a sequence spans several waves
            p.slot_bytes = align256(msgs) + align256(nrm) + (g.WPS > 1 ? align256((size_t)n * g.WPS * 8) : 0) +
                           (ckpt ? align256((size_t)g.G * 4) : 0);
            break;
        case BCJR_OP_GRAD:            // + per-wave (S0..S3) of every step when a sequence spans several waves
        case BCJR_OP_GRAD_CODEBOOK:   // + per state one float accumulator and two pending contributions
            p.slot_bytes = 2 * align256(msgs) + 2 * align256(nrm) + (g.WPS > 1 ? align256((size_t)n * g.WPS * 16) : 0) +
                           (op == BCJR_OP_GRAD_CODEBOOK ? 3 * align256(((size_t)1 << L) * 4) : 0) +
                           (ckpt ? align256(nrm) + align256((size_t)2 * g.G * 4) : 0);
            break;
        default: p.slot_bytes = align256(2 * (size_t)n * (size_t)g.TPS * 4); break;   // 2 back-pointer buffers
    }
    p.total = (size_t)p.slots * p.slot_bytes;
    return p;
}

// General trellis kernels: one sequence per workgroup of 2^L / SPT threads (SPT = 64 states per thread, all 2^L
// below L = 6), G = 2^(L-k) message floats per LDS buffer.
constexpr size_t kLdsBytes = 160 * 1024;
constexpr size_t kLdsStatic = 2048;   // the kernels' own reduction slots

struct GenPlan {
    bool ok;          // false: no kernel for these shapes (the messages exceed LDS)
    int grid, threads, dbl, ckpt;
    int nsq;          // Viterbi: sequences per workgroup (2 where the codebook streams and two fit in LDS)
    int qg;           // gradients: the Q^ message in the workspace (its two messages exceed LDS: k = 1, L = 16)
    size_t lds, slot_bytes, total;
    size_t acc_off;   // codebook gradient: offset of the slot's [2^L][V] accumulator
};

// The checkpoint interval of the recompute mode: about sqrt(n) rows stored and about sqrt(n) rebuilt per segment.
int checkpoint_interval(int64_t n) {
    int c = 1;
    while ((int64_t)c * c < n) ++c;
    return c;
}


// op: BCJR_OP_SOFT, BCJR_OP_GRAD, BCJR_OP_GRAD_CODEBOOK or BCJR_OP_VITERBI.  ckpt > 0 (not Viterbi): the
// checkpoint-and-recompute mode with that interval.
GenPlan make_gen_plan(int op, int64_t B, int64_t n, int32_t L, int32_t k, int32_t V, int ckpt = 0) {
    GenPlan p{};
    p.ckpt = ckpt;
    const int S = 1 << L;
    const int spt = S < 64 ? S : 64;
    const int tps = S / spt;
    const int wps = tps >= 64 ? tps / 64 : 1;
    const size_t G = (size_t)S >> k;
    const size_t msg = G * 4;
    if (op == BCJR_OP_GRAD || op == BCJR_OP_GRAD_CODEBOOK) {   // R and Q, one buffer each
        p.dbl = 0;
        // R~ in LDS, and Q^ too unless both exceed it: then Q^ goes to a buffer in the slot
        p.qg = 2 * msg + kLdsStatic > kLdsBytes && msg + kLdsStatic <= kLdsBytes ? 1 : 0;
        p.lds = p.qg ? msg : 2 * msg;
    } else {
        // Viterbi with V = 2 at L >= 12 reads its codebook through L1 every step: pair the sequences so each row
        // read serves two (their message buffers side by side)
        p.nsq = op == BCJR_OP_VITERBI && V == 2 && L >= 12 && 2 * msg + kLdsStatic <= kLdsBytes ? 2 : 1;
        p.dbl = ckpt == 0 && p.nsq * 2 * msg + kLdsStatic <= kLdsBytes;   // the recompute mode uses one buffer
        p.lds = p.nsq * (p.dbl ? 2 * msg : msg);
    }
    if (p.nsq < 1) p.nsq = 1;
    p.ok = p.lds + kLdsStatic <= kLdsBytes;
    p.threads = tps;
    // blocks per CU: 16 waves of at most 128 VGPRs, and the LDS
    const int waves = tps >= 64 ? tps / 64 : 1;
    int bpc = 16 / waves;
    const int bpc_lds = (int)(kLdsBytes / (p.lds + kLdsStatic));
    if (bpc_lds < bpc) bpc = bpc_lds;
    if (bpc < 1) bpc = 1;
    const int64_t cap = (int64_t)device_cus() * bpc;
    const int64_t rounds = (B + p.nsq - 1) / p.nsq;
    p.grid = (int)(rounds < cap ? rounds : cap);
    const size_t tapes = align256(TapeRows::rows(ckpt, (int)n) * G * 4);
    const size_t nrm = align256((size_t)n * 4);
    switch (op) {
        case BCJR_OP_SOFT:   // R~ rows, normalisers, per-wave (S0, S1[V]) of every step (+ the saved message)
            p.slot_bytes = tapes + nrm + (wps > 1 ? align256((size_t)n * wps * (1 + V) * 4) : 0) +
                           (ckpt ? align256(G * 4) : 0);
            break;
        case BCJR_OP_GRAD:   // R~ and Q^ tapes, normalisers and Q offsets, per-wave (S0, S1[V], S2, S3[V])
        case BCJR_OP_GRAD_CODEBOOK:   // + per state and component a float accumulator and two pending contributions
            p.acc_off = 2 * tapes + 2 * nrm + (wps > 1 ? align256((size_t)n * wps * (2 + 2 * V) * 4) : 0);
            p.slot_bytes = p.acc_off + (op == BCJR_OP_GRAD_CODEBOOK ? 3 * align256((size_t)S * V * 4) : 0) +
                           (ckpt ? nrm + align256(2 * G * 4) : 0) +   // + the Q input offsets, the saved messages
                           (p.qg ? align256(G * 4) : 0);              // + the Q^ message
            break;
        default:   // two back-pointer buffers (by round parity) of [n][threads] words per sequence of a round
            p.slot_bytes = align256(2 * (size_t)p.nsq * (size_t)n * (size_t)tps * 4);
            break;
    }
    p.total = (size_t)p.grid * p.slot_bytes;
    return p;
}

// Fewer persistent workgroups, each looping over more sequences, so that the plan's slots fit in `bytes` (the static
// scratch of bcjr_soft_codeword_noalloc).  False when the slots of one workgroup alone exceed it.
bool fit_grid(Plan& p, int spb, size_t bytes) {
    const size_t per_block = (size_t)spb * p.slot_bytes;
    if (per_block > bytes) return false;
    const size_t most = bytes / per_block;
    if ((size_t)p.grid > most) p.grid = (int)most;
    p.slots = p.grid * spb;
    p.total = (size_t)p.slots * p.slot_bytes;
    return true;
}

bool fit_grid(GenPlan& p, size_t bytes) {
    if (p.slot_bytes > bytes) return false;
    const size_t most = bytes / p.slot_bytes;
    if ((size_t)p.grid > most) p.grid = (int)most;
    p.total = (size_t)p.grid * p.slot_bytes;
    return true;
}

int check_workspace(const void* ws, size_t bytes, const Plan& p) {
    if (ws == nullptr || bytes < p.total) return BCJR_ERR_WORKSPACE;
    if (((uintptr_t)ws & 255u) != 0) return BCJR_ERR_WORKSPACE;
    return BCJR_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? BCJR_OK : BCJR_ERR_HIP; }

// Tail-biting workspace: the Viterbi slots (sized for the larger of its passes), then the per-(row, sigma) costs
// (exact) or the rotated pass's states (rotate), then the chosen sigma per row.
struct TailBitingPlan {
    Plan rows, first;        // the sigma-mode pass over the rows; the first pass (every sigma, or the rotated rows)
    size_t slots_bytes, aux_off, sigma_off, total;
};

TailBitingPlan make_tb_plan(int32_t mode, int64_t B, int64_t n, int32_t L) {
    TailBitingPlan t{};
    t.rows = make_plan(BCJR_OP_VITERBI, B, n, L);
    t.first = mode == BCJR_TB_EXACT ? make_plan(BCJR_OP_VITERBI, B << L, n, L) : t.rows;
    t.slots_bytes = align256(t.first.total > t.rows.total ? t.first.total : t.rows.total);
    t.aux_off = t.slots_bytes;
    const size_t aux = mode == BCJR_TB_EXACT ? (size_t)(B << L) * 4 : (size_t)B * (size_t)n * 4;
    t.sigma_off = t.aux_off + align256(aux);
    t.total = t.sigma_off + align256((size_t)B * 4);
    return t;
}

// Soft codeword / gradient under the tail-biting measure: the per-(row, sigma) passes' slots, then their outputs
// (w_soft and ln Z of every (row, sigma); the gradient also its per-sigma gradient).
struct MixturePlan {
    Plan soft, grad;
    size_t ws_off, lz_off, gr_off, total;
};

MixturePlan make_mixture_plan(bool with_grad, int64_t B, int64_t n, int32_t L) {
    MixturePlan m{};
    const int64_t V = B << L;
    m.soft = make_plan(BCJR_OP_SOFT, V, n, L);
    m.grad = with_grad ? make_plan(BCJR_OP_GRAD, V, n, L) : m.soft;
    m.ws_off = align256(m.grad.total > m.soft.total ? m.grad.total : m.soft.total);
    m.lz_off = m.ws_off + align256((size_t)V * (size_t)n * 4);
    m.gr_off = m.lz_off + align256((size_t)V * 4);
    m.total = m.gr_off + (with_grad ? align256((size_t)V * (size_t)n * 4) : 0);
    return m;
}

// The same two plans for the general trellis kernels (one sequence per workgroup; slots as in make_gen_plan).
struct GenTailBitingPlan {
    bool ok;
    GenPlan rows, first;
    size_t slots_bytes, aux_off, sigma_off, rotw_off, total;   // rotw: the rotated rows (rotate mode)
};

GenTailBitingPlan make_gen_tb_plan(int32_t mode, int64_t B, int64_t n, int32_t L, int32_t k, int32_t V) {
    GenTailBitingPlan t{};
    t.rows = make_gen_plan(BCJR_OP_VITERBI, B, n, L, k, V);
    t.first = mode == BCJR_TB_EXACT ? make_gen_plan(BCJR_OP_VITERBI, B << L, n, L, k, V) : t.rows;
    t.ok = t.rows.ok && t.first.ok;
    t.slots_bytes = align256(t.first.total > t.rows.total ? t.first.total : t.rows.total);
    t.aux_off = t.slots_bytes;
    const size_t aux = mode == BCJR_TB_EXACT ? (size_t)(B << L) * 4 : (size_t)B * (size_t)n * 4;
    t.sigma_off = t.aux_off + align256(aux);
    t.rotw_off = t.sigma_off + align256((size_t)B * 4);
    t.total = t.rotw_off + (mode == BCJR_TB_ROTATE ? align256((size_t)B * (size_t)n * V * 4) : 0);
    return t;
}

struct GenMixturePlan {
    bool ok;
    GenPlan soft, grad;
    size_t ws_off, lz_off, gr_off, total;
};

GenMixturePlan make_gen_mixture_plan(bool with_grad, int64_t B, int64_t n, int32_t L, int32_t k, int32_t V) {
    GenMixturePlan m{};
    const int64_t S = B << L;   // one virtual sequence per (row, sigma)
    m.soft = make_gen_plan(BCJR_OP_SOFT, S, n, L, k, V);
    m.grad = with_grad ? make_gen_plan(BCJR_OP_GRAD, S, n, L, k, V) : m.soft;
    m.ok = m.soft.ok && m.grad.ok;
    m.ws_off = align256(m.grad.total > m.soft.total ? m.grad.total : m.soft.total);
    m.lz_off = m.ws_off + align256((size_t)S * (size_t)n * V * 4);
    m.gr_off = m.lz_off + align256((size_t)S * 4);
    m.total = m.gr_off + (with_grad ? align256((size_t)S * (size_t)n * V * 4) : 0);
    return m;
}

int check_tb_mode(int32_t mode, int32_t L) {
    if (mode == BCJR_TB_ROTATE) return BCJR_OK;
    if (mode == BCJR_TB_EXACT && L <= kMaxTailBitingExactL) return BCJR_OK;
    return BCJR_ERR_UNSUPPORTED;
}

}  // namespace

extern "C" {

size_t bcjr_workspace_bytes_v(int32_t op, int64_t B, int64_t n, int32_t L, int32_t k, int32_t V) {
    if (op < BCJR_OP_SOFT || op > BCJR_OP_GRAD_TAIL_BITING) return 0;
    if (check_shape_v(B, n, L, k, V) != BCJR_OK) return 0;
    if (op == BCJR_OP_SOFT || op == BCJR_OP_GRAD || op == BCJR_OP_VITERBI || op == BCJR_OP_GRAD_CODEBOOK) {
        if (tuned(k, V)) return make_plan(op, B, n, L).total;
        const GenPlan p = make_gen_plan(op, B, n, L, k, V);
        return p.ok ? p.total : 0;
    }
    if (op == BCJR_OP_SOFT_TAIL_BITING || op == BCJR_OP_GRAD_TAIL_BITING) {
        if (L > kMaxTailBitingExactL) return 0;
        const bool with_grad = op == BCJR_OP_GRAD_TAIL_BITING;
        if (tuned(k, V)) return make_mixture_plan(with_grad, B, n, L).total;
        const GenMixturePlan m = make_gen_mixture_plan(with_grad, B, n, L, k, V);
        return m.ok ? m.total : 0;
    }
    const int32_t mode = op == BCJR_OP_VITERBI_TB_EXACT ? BCJR_TB_EXACT : BCJR_TB_ROTATE;
    if (check_tb_mode(mode, L) != BCJR_OK) return 0;
    if (tuned(k, V)) return make_tb_plan(mode, B, n, L).total;
    const GenTailBitingPlan t = make_gen_tb_plan(mode, B, n, L, k, V);
    return t.ok ? t.total : 0;
}

size_t bcjr_workspace_bytes_min(int32_t op, int64_t B, int64_t n, int32_t L, int32_t k, int32_t V) {
    const size_t full = bcjr_workspace_bytes_v(op, B, n, L, k, V);
    // only the soft codeword and the two gradients have a checkpoint mode
    if (full == 0 || (op != BCJR_OP_SOFT && op != BCJR_OP_GRAD && op != BCJR_OP_GRAD_CODEBOOK)) return full;
    if (tuned(k, V)) {   // the k = 2 kernels' own checkpoint mode
        const Plan p = make_plan(op, B, n, L, checkpoint_interval(n));
        return p.total < full ? p.total : full;
    }
    const GenPlan p = make_gen_plan(op, B, n, L, k, V, checkpoint_interval(n));
    return p.ok && p.total < full ? p.total : full;
}

size_t bcjr_workspace_bytes(int32_t op, int64_t B, int64_t n, int32_t L, int32_t k) {
    return bcjr_workspace_bytes_v(op, B, n, L, k, 1);
}

const char* bcjr_status_string(int32_t status) {
    switch (status) {
        case BCJR_OK: return "BCJR_OK: success";
        case BCJR_ERR_NULL: return "BCJR_ERR_NULL: a required pointer is NULL";
        case BCJR_ERR_SHAPE:
            return "BCJR_ERR_SHAPE: need 1 <= B < 2^31, 1 <= n <= 4096, k >= 1, 4 <= L <= 16 with L >= 2k, V >= 1";
        case BCJR_ERR_TEMP: return "BCJR_ERR_TEMP: temperature must be finite and >= 1e-12";
        case BCJR_ERR_UNSUPPORTED:
            return "BCJR_ERR_UNSUPPORTED: kernels exist for k <= 4 and V <= 2; exact tail-biting and the "
                   "tail-biting soft codeword and gradient need L <= 10";
        case BCJR_ERR_WORKSPACE:
            return "BCJR_ERR_WORKSPACE: workspace NULL, misaligned or smaller than bcjr_workspace_bytes(); or, for "
                   "bcjr_soft_codeword_noalloc, one sequence needs more than the library's static scratch holds";
        case BCJR_ERR_HIP: return "BCJR_ERR_HIP: the HIP runtime reported a launch error";
        default: return "BCJR: unknown status";
    }
}

}  // extern "C"

namespace {

int gen_workspace(void* workspace, size_t bytes, const GenPlan& p) {
    if (!p.ok) return BCJR_ERR_UNSUPPORTED;
    if (workspace == nullptr || bytes < p.total || ((uintptr_t)workspace & 255u) != 0) return BCJR_ERR_WORKSPACE;
    return BCJR_OK;
}

// fit: `workspace` is a fixed buffer of workspace_bytes (the static scratch), and the grid shrinks until the plan
// fits in it rather than the call failing when it is smaller than the plan.
int soft_impl(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L, int32_t k, int32_t V, float T,
              const int32_t* boundary_state, float* w_soft, float* log_z, void* workspace, size_t workspace_bytes,
              void* stream, bool fit = false) {
    if (!w || !codebook || !w_soft) return BCJR_ERR_NULL;
    int rc = check_shape_v(B, n, L, k, V);
    if (rc) return rc;
    if ((rc = check_temp(T))) return rc;
    const float scale = (float)std::sqrt(1.4426950408889634 / (double)T);
    // memory: the full tape when the workspace holds it, else checkpoints with per-segment recompute
    const size_t full = tuned(k, V) ? make_plan(BCJR_OP_SOFT, B, n, L).total : make_gen_plan(BCJR_OP_SOFT, B, n, L, k, V).total;
    const bool recompute = workspace != nullptr && workspace_bytes < full;
    if (!tuned(k, V)) {
        GenPlan p = make_gen_plan(BCJR_OP_SOFT, B, n, L, k, V, recompute ? checkpoint_interval(n) : 0);
        if (fit && p.ok && !fit_grid(p, workspace_bytes)) return BCJR_ERR_WORKSPACE;
        if ((rc = gen_workspace(workspace, workspace_bytes, p))) return rc;
        GenArgs a{};
        a.w = w;
        a.cb = codebook;
        a.B = B;
        a.n = (int)n;
        a.L = L;
        a.scale = scale;
        a.sigma = boundary_state;
        a.w_soft = w_soft;
        a.log_z = log_z;
        a.ws = static_cast<unsigned char*>(workspace);
        a.slot_bytes = p.slot_bytes;
        a.dbl = p.dbl;
        a.ckpt = p.ckpt;
        return hip_status(launch_general(0, k, V, a, p.grid, p.threads, p.lds, static_cast<hipStream_t>(stream)));
    }
    const int ckpt = recompute ? checkpoint_interval(n) : 0;
    Plan p = make_plan(BCJR_OP_SOFT, B, n, L, ckpt);
    if (fit && !fit_grid(p, geo_rt(L).SPB, workspace_bytes)) return BCJR_ERR_WORKSPACE;
    if ((rc = check_workspace(workspace, workspace_bytes, p))) return rc;
    SoftArgs a{};
    a.w = w;
    a.cb = codebook;
    a.B = B;
    a.n = (int)n;
    a.scale = scale;
    a.sigma = boundary_state;
    a.w_soft = w_soft;
    a.log_z = log_z;
    a.ws = static_cast<unsigned char*>(workspace);
    a.slot_bytes = p.slot_bytes;
    a.ckpt = ckpt;
    return hip_status(launch_soft(L, a, p.grid, static_cast<hipStream_t>(stream)));
}

int grad_impl(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L, int32_t k, int32_t V, float T,
              const int32_t* boundary_state, const float* grad_w_soft, float* grad_w, float* w_soft, void* workspace,
              size_t workspace_bytes, void* stream) {
    if (!w || !codebook || !grad_w_soft || !grad_w) return BCJR_ERR_NULL;
    int rc = check_shape_v(B, n, L, k, V);
    if (rc) return rc;
    if ((rc = check_temp(T))) return rc;
    const float scale = (float)std::sqrt(1.4426950408889634 / (double)T);
    const size_t full = tuned(k, V) ? make_plan(BCJR_OP_GRAD, B, n, L).total : make_gen_plan(BCJR_OP_GRAD, B, n, L, k, V).total;
    const bool recompute = workspace != nullptr && workspace_bytes < full;
    if (!tuned(k, V)) {
        const GenPlan p = make_gen_plan(BCJR_OP_GRAD, B, n, L, k, V, recompute ? checkpoint_interval(n) : 0);
        if ((rc = gen_workspace(workspace, workspace_bytes, p))) return rc;
        GenArgs a{};
        a.w = w;
        a.cb = codebook;
        a.g = grad_w_soft;
        a.B = B;
        a.n = (int)n;
        a.L = L;
        a.scale = scale;
        a.two_over_T = (float)(2.0 / (double)T);
        a.sigma = boundary_state;
        a.grad = grad_w;
        a.w_soft = w_soft;
        a.ws = static_cast<unsigned char*>(workspace);
        a.slot_bytes = p.slot_bytes;
        a.dbl = p.dbl;
        a.ckpt = p.ckpt;
        a.qg = p.qg;
        return hip_status(launch_general(1, k, V, a, p.grid, p.threads, p.lds, static_cast<hipStream_t>(stream)));
    }
    const int ckpt = recompute ? checkpoint_interval(n) : 0;
    const Plan p = make_plan(BCJR_OP_GRAD, B, n, L, ckpt);
    if ((rc = check_workspace(workspace, workspace_bytes, p))) return rc;
    GradArgs a{};
    a.w = w;
    a.cb = codebook;
    a.g = grad_w_soft;
    a.B = B;
    a.n = (int)n;
    a.scale = scale;
    a.two_over_T = (float)(2.0 / (double)T);
    a.sigma = boundary_state;
    a.grad = grad_w;
    a.w_soft = w_soft;
    a.ws = static_cast<unsigned char*>(workspace);
    a.slot_bytes = p.slot_bytes;
    a.ckpt = ckpt;
    return hip_status(launch_grad(L, a, p.grid, static_cast<hipStream_t>(stream)));
}

int grad_codebook_impl(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L, int32_t k, int32_t V,
                       float T, const int32_t* boundary_state, const float* grad_w_soft, float* grad_codebook,
                       float* grad_w, float* w_soft, void* workspace, size_t workspace_bytes, void* stream) {
    if (!w || !codebook || !grad_w_soft || !grad_codebook) return BCJR_ERR_NULL;
    int rc = check_shape_v(B, n, L, k, V);
    if (rc) return rc;
    if ((rc = check_temp(T))) return rc;
    const float scale = (float)std::sqrt(1.4426950408889634 / (double)T);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const size_t full = tuned(k, V) ? make_plan(BCJR_OP_GRAD_CODEBOOK, B, n, L).total
                                    : make_gen_plan(BCJR_OP_GRAD_CODEBOOK, B, n, L, k, V).total;
    const bool recompute = workspace != nullptr && workspace_bytes < full;
    if (!tuned(k, V)) {
        const GenPlan p = make_gen_plan(BCJR_OP_GRAD_CODEBOOK, B, n, L, k, V, recompute ? checkpoint_interval(n) : 0);
        if ((rc = gen_workspace(workspace, workspace_bytes, p))) return rc;
        GenArgs a{};
        a.w = w;
        a.cb = codebook;
        a.g = grad_w_soft;
        a.B = B;
        a.n = (int)n;
        a.L = L;
        a.scale = scale;
        a.two_over_T = (float)(2.0 / (double)T);
        a.sigma = boundary_state;
        a.grad = grad_w;
        a.w_soft = w_soft;
        a.ws = static_cast<unsigned char*>(workspace);
        a.slot_bytes = p.slot_bytes;
        a.dbl = p.dbl;
        a.ckpt = p.ckpt;
        a.qg = p.qg;
        hipError_t e = launch_general(3, k, V, a, p.grid, p.threads, p.lds, st);
        if (e != hipSuccess) return hip_status(e);
        return hip_status(launch_codebook_reduce(a.ws, p.slot_bytes, (uint32_t)p.acc_off, p.grid, (1 << L) * V,
                                                 grad_codebook, st));
    }
    const int ckpt = recompute ? checkpoint_interval(n) : 0;
    const Plan p = make_plan(BCJR_OP_GRAD_CODEBOOK, B, n, L, ckpt);
    if ((rc = check_workspace(workspace, workspace_bytes, p))) return rc;
    GradArgs a{};
    a.w = w;
    a.cb = codebook;
    a.g = grad_w_soft;
    a.B = B;
    a.n = (int)n;
    a.scale = scale;
    a.two_over_T = (float)(2.0 / (double)T);
    a.sigma = boundary_state;
    a.grad = grad_w;
    a.w_soft = w_soft;
    a.ws = static_cast<unsigned char*>(workspace);
    a.slot_bytes = p.slot_bytes;
    a.ckpt = ckpt;
    return hip_status(launch_grad_codebook(L, a, p.grid, st, grad_codebook));
}

int viterbi_impl(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L, int32_t k, int32_t V,
                 const int32_t* boundary_state, int32_t* states, float* w_hard, float* cost, void* workspace,
                 size_t workspace_bytes, void* stream) {
    if (!w || !codebook || !states) return BCJR_ERR_NULL;
    int rc = check_shape_v(B, n, L, k, V);
    if (rc) return rc;
    if (!tuned(k, V)) {
        const GenPlan p = make_gen_plan(BCJR_OP_VITERBI, B, n, L, k, V);
        if ((rc = gen_workspace(workspace, workspace_bytes, p))) return rc;
        GenArgs a{};
        a.w = w;
        a.cb = codebook;
        a.B = B;
        a.n = (int)n;
        a.L = L;
        a.sigma = boundary_state;
        a.states = states;
        a.w_hard = w_hard;
        a.cost = cost;
        a.ws = static_cast<unsigned char*>(workspace);
        a.slot_bytes = p.slot_bytes;
        a.dbl = p.dbl;
        a.nsq = p.nsq;
        return hip_status(launch_general(2, k, V, a, p.grid, p.threads, p.lds, static_cast<hipStream_t>(stream)));
    }
    const Plan p = make_plan(BCJR_OP_VITERBI, B, n, L);
    if ((rc = check_workspace(workspace, workspace_bytes, p))) return rc;
    ViterbiArgs a{};
    a.w = w;
    a.cb = codebook;
    a.B = B;
    a.n = (int)n;
    a.sigma = boundary_state;
    a.states = states;
    a.w_hard = w_hard;
    a.cost = cost;
    a.ws = static_cast<unsigned char*>(workspace);
    a.slot_bytes = p.slot_bytes;
    return hip_status(launch_viterbi(L, a, p.grid, static_cast<hipStream_t>(stream)));
}

// Tail-biting: the per-(row, sigma) or rotated passes of the k = 2, V = 1 kernels, or of the general ones, then the
// selection / combine kernels (which see a row as n V floats).
int soft_tb_impl(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L, int32_t k, int32_t V,
                 float T, float* w_soft, float* log_z, void* workspace, size_t workspace_bytes, void* stream) {
    if (!w || !codebook || !w_soft) return BCJR_ERR_NULL;
    int rc = check_shape_v(B, n, L, k, V);
    if (rc) return rc;
    if ((rc = check_temp(T))) return rc;
    if (L > kMaxTailBitingExactL) return BCJR_ERR_UNSUPPORTED;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const float scale = (float)std::sqrt(1.4426950408889634 / (double)T);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    hipError_t e;
    if (!tuned(k, V)) {
        const GenMixturePlan mp = make_gen_mixture_plan(false, B, n, L, k, V);
        if (!mp.ok) return BCJR_ERR_UNSUPPORTED;
        if (workspace == nullptr || workspace_bytes < mp.total || ((uintptr_t)workspace & 255u) != 0)
            return BCJR_ERR_WORKSPACE;
        float* ws_all = reinterpret_cast<float*>(ws + mp.ws_off);
        float* lz_all = reinterpret_cast<float*>(ws + mp.lz_off);
        GenArgs a{};
        a.w = w;
        a.cb = codebook;
        a.B = B << L;
        a.n = (int)n;
        a.L = L;
        a.scale = scale;
        a.w_soft = ws_all;
        a.log_z = lz_all;
        a.ws = ws;
        a.slot_bytes = mp.soft.slot_bytes;
        a.dbl = mp.soft.dbl;
        a.sigma_enum = 1;
        if ((e = launch_general(0, k, V, a, mp.soft.grid, mp.soft.threads, mp.soft.lds, st)) != hipSuccess)
            return hip_status(e);
        return hip_status(launch_tb_soft_combine(ws_all, lz_all, B, (int)(n * V), 1 << L, w_soft, log_z, st));
    }
    const MixturePlan mp = make_mixture_plan(false, B, n, L);
    if (workspace == nullptr || workspace_bytes < mp.total || ((uintptr_t)workspace & 255u) != 0)
        return BCJR_ERR_WORKSPACE;
    float* ws_all = reinterpret_cast<float*>(ws + mp.ws_off);
    float* lz_all = reinterpret_cast<float*>(ws + mp.lz_off);
    SoftArgs a{};
    a.w = w;
    a.cb = codebook;
    a.B = B << L;
    a.n = (int)n;
    a.scale = scale;
    a.w_soft = ws_all;
    a.log_z = lz_all;
    a.ws = ws;
    a.slot_bytes = mp.soft.slot_bytes;
    a.sigma_enum = 1;
    if ((e = launch_soft(L, a, mp.soft.grid, st)) != hipSuccess) return hip_status(e);
    return hip_status(launch_tb_soft_combine(ws_all, lz_all, B, (int)n, 1 << L, w_soft, log_z, st));
}

int grad_tb_impl(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L, int32_t k, int32_t V,
                 float T, const float* grad_w_soft, float* grad_w, float* w_soft, void* workspace,
                 size_t workspace_bytes, void* stream) {
    if (!w || !codebook || !grad_w_soft || !grad_w) return BCJR_ERR_NULL;
    int rc = check_shape_v(B, n, L, k, V);
    if (rc) return rc;
    if ((rc = check_temp(T))) return rc;
    if (L > kMaxTailBitingExactL) return BCJR_ERR_UNSUPPORTED;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const float scale = (float)std::sqrt(1.4426950408889634 / (double)T);
    const float two_over_T = (float)(2.0 / (double)T);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    hipError_t e;
    if (!tuned(k, V)) {
        const GenMixturePlan mp = make_gen_mixture_plan(true, B, n, L, k, V);
        if (!mp.ok) return BCJR_ERR_UNSUPPORTED;
        if (workspace == nullptr || workspace_bytes < mp.total || ((uintptr_t)workspace & 255u) != 0)
            return BCJR_ERR_WORKSPACE;
        float* ws_all = reinterpret_cast<float*>(ws + mp.ws_off);
        float* lz_all = reinterpret_cast<float*>(ws + mp.lz_off);
        float* gr_all = reinterpret_cast<float*>(ws + mp.gr_off);
        GenArgs a{};
        a.w = w;
        a.cb = codebook;
        a.B = B << L;
        a.n = (int)n;
        a.L = L;
        a.scale = scale;
        a.w_soft = ws_all;
        a.log_z = lz_all;
        a.ws = ws;
        a.slot_bytes = mp.soft.slot_bytes;
        a.dbl = mp.soft.dbl;
        a.sigma_enum = 1;
        if ((e = launch_general(0, k, V, a, mp.soft.grid, mp.soft.threads, mp.soft.lds, st)) != hipSuccess)
            return hip_status(e);
        GenArgs ga{};
        ga.w = w;
        ga.cb = codebook;
        ga.g = grad_w_soft;
        ga.B = B << L;
        ga.n = (int)n;
        ga.L = L;
        ga.scale = scale;
        ga.two_over_T = two_over_T;
        ga.grad = gr_all;
        ga.ws = ws;
        ga.slot_bytes = mp.grad.slot_bytes;
        ga.dbl = mp.grad.dbl;
        ga.qg = mp.grad.qg;
        ga.sigma_enum = 1;
        if ((e = launch_general(1, k, V, ga, mp.grad.grid, mp.grad.threads, mp.grad.lds, st)) != hipSuccess)
            return hip_status(e);
        return hip_status(launch_tb_grad_combine(ws_all, lz_all, gr_all, grad_w_soft, B, (int)(n * V), 1 << L,
                                                 two_over_T, grad_w, w_soft, st));
    }
    const MixturePlan mp = make_mixture_plan(true, B, n, L);
    if (workspace == nullptr || workspace_bytes < mp.total || ((uintptr_t)workspace & 255u) != 0)
        return BCJR_ERR_WORKSPACE;
    float* ws_all = reinterpret_cast<float*>(ws + mp.ws_off);
    float* lz_all = reinterpret_cast<float*>(ws + mp.lz_off);
    float* gr_all = reinterpret_cast<float*>(ws + mp.gr_off);
    SoftArgs a{};
    a.w = w;
    a.cb = codebook;
    a.B = B << L;
    a.n = (int)n;
    a.scale = scale;
    a.w_soft = ws_all;
    a.log_z = lz_all;
    a.ws = ws;
    a.slot_bytes = mp.soft.slot_bytes;
    a.sigma_enum = 1;
    if ((e = launch_soft(L, a, mp.soft.grid, st)) != hipSuccess) return hip_status(e);
    GradArgs ga{};
    ga.w = w;
    ga.cb = codebook;
    ga.g = grad_w_soft;
    ga.B = B << L;
    ga.n = (int)n;
    ga.scale = scale;
    ga.two_over_T = two_over_T;
    ga.grad = gr_all;
    ga.ws = ws;
    ga.slot_bytes = mp.grad.slot_bytes;
    ga.sigma_enum = 1;
    if ((e = launch_grad(L, ga, mp.grad.grid, st)) != hipSuccess) return hip_status(e);
    return hip_status(launch_tb_grad_combine(ws_all, lz_all, gr_all, grad_w_soft, B, (int)n, 1 << L, two_over_T,
                                             grad_w, w_soft, st));
}

int viterbi_tb_impl(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L, int32_t k, int32_t V,
                    int32_t mode, int32_t* states, float* w_hard, float* cost, int32_t* sigma, void* workspace,
                    size_t workspace_bytes, void* stream) {
    if (!w || !codebook || !states) return BCJR_ERR_NULL;
    int rc = check_shape_v(B, n, L, k, V);
    if (rc) return rc;
    if ((rc = check_tb_mode(mode, L))) return rc;
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const int r = (int)(n / 2);   // rotate: the rows rotated left by n / 2 trellis steps
    hipError_t e;
    if (!tuned(k, V)) {
        const GenTailBitingPlan tp = make_gen_tb_plan(mode, B, n, L, k, V);
        if (!tp.ok) return BCJR_ERR_UNSUPPORTED;
        if (workspace == nullptr || workspace_bytes < tp.total || ((uintptr_t)workspace & 255u) != 0)
            return BCJR_ERR_WORKSPACE;
        int32_t* sig_ws = reinterpret_cast<int32_t*>(ws + tp.sigma_off);
        GenArgs f{};
        f.w = w;
        f.cb = codebook;
        f.n = (int)n;
        f.L = L;
        f.ws = ws;
        f.slot_bytes = tp.first.slot_bytes;
        f.dbl = tp.first.dbl;
        f.nsq = tp.first.nsq;
        if (mode == BCJR_TB_EXACT) {   // the cost of every (row, sigma), no traceback
            float* costs = reinterpret_cast<float*>(ws + tp.aux_off);
            f.B = B << L;
            f.sigma_enum = 1;
            f.cost = costs;
            if ((e = launch_general(2, k, V, f, tp.first.grid, tp.first.threads, tp.first.lds, st)) != hipSuccess)
                return hip_status(e);
            if ((e = launch_tb_select(costs, B, 1 << L, sig_ws, sigma, st)) != hipSuccess) return hip_status(e);
        } else {   // the free decode of a rotated copy of the rows
            int32_t* rot_states = reinterpret_cast<int32_t*>(ws + tp.aux_off);
            float* rot_w = reinterpret_cast<float*>(ws + tp.rotw_off);
            if ((e = launch_tb_rotate_rows(w, B, (int)(n * V), r * V, rot_w, st)) != hipSuccess) return hip_status(e);
            f.w = rot_w;
            f.B = B;
            f.states = rot_states;
            if ((e = launch_general(2, k, V, f, tp.first.grid, tp.first.threads, tp.first.lds, st)) != hipSuccess)
                return hip_status(e);
            if ((e = launch_tb_rotate_sigma(rot_states, B, (int)n, (int)(n - 1 - r), sig_ws, sigma, st)) !=
                hipSuccess)
                return hip_status(e);
        }
        GenArgs a{};
        a.w = w;
        a.cb = codebook;
        a.B = B;
        a.n = (int)n;
        a.L = L;
        a.sigma = sig_ws;
        a.states = states;
        a.w_hard = w_hard;
        a.cost = cost;
        a.ws = ws;
        a.slot_bytes = tp.rows.slot_bytes;
        a.dbl = tp.rows.dbl;
        a.nsq = tp.rows.nsq;
        return hip_status(launch_general(2, k, V, a, tp.rows.grid, tp.rows.threads, tp.rows.lds, st));
    }
    const TailBitingPlan tp = make_tb_plan(mode, B, n, L);
    if (workspace == nullptr || workspace_bytes < tp.total || ((uintptr_t)workspace & 255u) != 0)
        return BCJR_ERR_WORKSPACE;
    int32_t* sig_ws = reinterpret_cast<int32_t*>(ws + tp.sigma_off);

    // first pass: the cost of every (row, sigma), or the free decode of the rows rotated left by n / 2
    ViterbiArgs f{};
    f.w = w;
    f.cb = codebook;
    f.n = (int)n;
    f.ws = ws;
    f.slot_bytes = tp.first.slot_bytes;
    if (mode == BCJR_TB_EXACT) {
        float* costs = reinterpret_cast<float*>(ws + tp.aux_off);
        f.B = B << L;
        f.sigma_enum = 1;
        f.cost = costs;
        if ((e = launch_viterbi(L, f, tp.first.grid, st)) != hipSuccess) return hip_status(e);
        if ((e = launch_tb_select(costs, B, 1 << L, sig_ws, sigma, st)) != hipSuccess) return hip_status(e);
    } else {
        int32_t* rot_states = reinterpret_cast<int32_t*>(ws + tp.aux_off);
        f.B = B;
        f.rot = r;
        f.states = rot_states;
        if ((e = launch_viterbi(L, f, tp.first.grid, st)) != hipSuccess) return hip_status(e);
        if ((e = launch_tb_rotate_sigma(rot_states, B, (int)n, (int)(n - 1 - r), sig_ws, sigma, st)) != hipSuccess)
            return hip_status(e);
    }
    // second pass: the sigma-constrained decode of the rows with the chosen start state
    ViterbiArgs a{};
    a.w = w;
    a.cb = codebook;
    a.B = B;
    a.n = (int)n;
    a.sigma = sig_ws;
    a.states = states;
    a.w_hard = w_hard;
    a.cost = cost;
    a.ws = ws;
    a.slot_bytes = tp.rows.slot_bytes;
    return hip_status(launch_viterbi(L, a, tp.rows.grid, st));
}

// ---------------------------------------------------------------------------------------------------------------
// The static scratch of bcjr_soft_codeword_noalloc: the workspace of callers that cannot allocate.  Each device that
// runs the library holds its own copy, at its own address, until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: kernels and copies get the address hipGetSymbolAddress returns for the
// current device, looked up once per device with that device current.

static __device__ __align__(256) unsigned char scratch[BCJR_NOALLOC_SCRATCH_BYTES];

struct ScratchAddress {
    std::once_flag once;
    void* ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchAddress g_scratch[kMaxDevices];

int scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return BCJR_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return BCJR_ERR_UNSUPPORTED;
    ScratchAddress& s = g_scratch[dev];
    std::call_once(s.once, [&s] { s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch)); });
    if (s.err != hipSuccess || s.ptr == nullptr) return BCJR_ERR_HIP;
    *out = s.ptr;
    return BCJR_OK;
}

}  // namespace

extern "C" {

int bcjr_soft_codeword_noalloc(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L, int32_t k,
                               float T, const int32_t* boundary_state, float* w_soft, float* log_z, void* stream) {
    // the host checks first, so that a bad call needs no device
    if (!w || !codebook || !w_soft) return BCJR_ERR_NULL;
    int rc = check_shape_v(B, n, L, k, 1);
    if (rc) return rc;
    if ((rc = check_temp(T))) return rc;
    void* ws = nullptr;
    if ((rc = scratch_address(&ws))) return rc;
    return soft_impl(w, codebook, B, n, L, k, 1, T, boundary_state, w_soft, log_z, ws, BCJR_NOALLOC_SCRATCH_BYTES,
                     stream, true);
}

int bcjr_soft_codeword(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L, int32_t k, float T,
                       const int32_t* boundary_state, float* w_soft, float* log_z, void* workspace,
                       size_t workspace_bytes, void* stream) {
    return soft_impl(w, codebook, B, n, L, k, 1, T, boundary_state, w_soft, log_z, workspace, workspace_bytes,
                     stream);
}

int bcjr_soft_codeword_v(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L, int32_t k,
                         int32_t V, float T, const int32_t* boundary_state, float* w_soft, float* log_z,
                         void* workspace, size_t workspace_bytes, void* stream) {
    return soft_impl(w, codebook, B, n, L, k, V, T, boundary_state, w_soft, log_z, workspace, workspace_bytes,
                     stream);
}

int bcjr_soft_codeword_grad(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L, int32_t k,
                            float T, const int32_t* boundary_state, const float* grad_w_soft, float* grad_w,
                            float* w_soft, void* workspace, size_t workspace_bytes, void* stream) {
    return grad_impl(w, codebook, B, n, L, k, 1, T, boundary_state, grad_w_soft, grad_w, w_soft, workspace,
                     workspace_bytes, stream);
}

int bcjr_soft_codeword_grad_v(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L, int32_t k,
                              int32_t V, float T, const int32_t* boundary_state, const float* grad_w_soft,
                              float* grad_w, float* w_soft, void* workspace, size_t workspace_bytes, void* stream) {
    return grad_impl(w, codebook, B, n, L, k, V, T, boundary_state, grad_w_soft, grad_w, w_soft, workspace,
                     workspace_bytes, stream);
}

int bcjr_soft_codeword_grad_codebook(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L,
                                     int32_t k, float T, const int32_t* boundary_state, const float* grad_w_soft,
                                     float* grad_codebook, float* grad_w, float* w_soft, void* workspace,
                                     size_t workspace_bytes, void* stream) {
    return grad_codebook_impl(w, codebook, B, n, L, k, 1, T, boundary_state, grad_w_soft, grad_codebook, grad_w,
                              w_soft, workspace, workspace_bytes, stream);
}

int bcjr_soft_codeword_grad_codebook_v(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L,
                                       int32_t k, int32_t V, float T, const int32_t* boundary_state,
                                       const float* grad_w_soft, float* grad_codebook, float* grad_w, float* w_soft,
                                       void* workspace, size_t workspace_bytes, void* stream) {
    return grad_codebook_impl(w, codebook, B, n, L, k, V, T, boundary_state, grad_w_soft, grad_codebook, grad_w,
                              w_soft, workspace, workspace_bytes, stream);
}

int viterbi_hard_code(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L, int32_t k,
                      const int32_t* boundary_state, int32_t* states, float* w_hard, float* cost, void* workspace,
                      size_t workspace_bytes, void* stream) {
    return viterbi_impl(w, codebook, B, n, L, k, 1, boundary_state, states, w_hard, cost, workspace,
                        workspace_bytes, stream);
}

int viterbi_hard_code_v(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L, int32_t k,
                        int32_t V, const int32_t* boundary_state, int32_t* states, float* w_hard, float* cost,
                        void* workspace, size_t workspace_bytes, void* stream) {
    return viterbi_impl(w, codebook, B, n, L, k, V, boundary_state, states, w_hard, cost, workspace,
                        workspace_bytes, stream);
}

int bcjr_soft_codeword_tail_biting(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L,
                                   int32_t k, float T, float* w_soft, float* log_z, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    return soft_tb_impl(w, codebook, B, n, L, k, 1, T, w_soft, log_z, workspace, workspace_bytes, stream);
}

int bcjr_soft_codeword_tail_biting_v(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L,
                                     int32_t k, int32_t V, float T, float* w_soft, float* log_z, void* workspace,
                                     size_t workspace_bytes, void* stream) {
    return soft_tb_impl(w, codebook, B, n, L, k, V, T, w_soft, log_z, workspace, workspace_bytes, stream);
}

int bcjr_soft_codeword_grad_tail_biting(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L,
                                        int32_t k, float T, const float* grad_w_soft, float* grad_w, float* w_soft,
                                        void* workspace, size_t workspace_bytes, void* stream) {
    return grad_tb_impl(w, codebook, B, n, L, k, 1, T, grad_w_soft, grad_w, w_soft, workspace, workspace_bytes,
                        stream);
}

int bcjr_soft_codeword_grad_tail_biting_v(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L,
                                          int32_t k, int32_t V, float T, const float* grad_w_soft, float* grad_w,
                                          float* w_soft, void* workspace, size_t workspace_bytes, void* stream) {
    return grad_tb_impl(w, codebook, B, n, L, k, V, T, grad_w_soft, grad_w, w_soft, workspace, workspace_bytes,
                        stream);
}

int viterbi_tail_biting(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L, int32_t k,
                        int32_t mode, int32_t* states, float* w_hard, float* cost, int32_t* sigma, void* workspace,
                        size_t workspace_bytes, void* stream) {
    return viterbi_tb_impl(w, codebook, B, n, L, k, 1, mode, states, w_hard, cost, sigma, workspace,
                           workspace_bytes, stream);
}

int viterbi_tail_biting_v(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L, int32_t k,
                          int32_t V, int32_t mode, int32_t* states, float* w_hard, float* cost, int32_t* sigma,
                          void* workspace, size_t workspace_bytes, void* stream) {
    return viterbi_tb_impl(w, codebook, B, n, L, k, V, mode, states, w_hard, cost, sigma, workspace,
                           workspace_bytes, stream);
}

}  // extern "C"
