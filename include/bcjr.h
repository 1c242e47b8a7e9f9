/*
 * bcjr.h -- C-ABI of libbcjr.so: the temperature-T BCJR forward-backward soft quantizer on a bitshift trellis,
 * its exact gradient, and the Viterbi hard code, as hand-written HIP kernels for gfx950 (MI355X).
 *
 * The method is "BCJR-QAT: A Differentiable Relaxation of Trellis-Coded Weight Quantization" (arXiv 2605.10655):
 * the hard Viterbi decision of trellis-coded quantization is replaced by the BCJR sum-product pass at temperature
 * T, whose output, the soft codeword, is the Boltzmann expectation of the emitted codebook value over all trellis
 * paths (abstract; gist.science Technical Summary, "Core Mechanism").  The soft codeword is exactly differentiable
 * in the weight pre-image, and T -> 0 gives back the hard code (same passages).
 *
 * Trellis and energy (readings of the pages, stated once here for every entry point):
 *   - state s_t: an L-bit integer, 0 <= s_t < 2^L; each step shifts in k new bits at the low end:
 *       s_{t+1} = ((s_t << k) & (2^L - 1)) | b,  b in [0, 2^k).   One weight per step (k bits per weight), or V
 *     weights per step with the _v entry points (k / V bits per weight).
 *   - a path s_1..s_n emits codebook[s_t] at step t; its energy is E = sum_t (w_t - codebook[s_t])^2 and its
 *     weight exp(-E / T).  Transitions carry no cost.  With V weights per step codebook[s] is a V-vector and
 *     (w_t - codebook[s_t])^2 is the squared Euclidean distance over its components.
 *   - boundary_state == NULL: free start and free end (s_1 and s_n unconstrained).
 *     boundary_state != NULL: sequence b starts from a non-emitting s_0 = sigma_b (so s_1 is a successor of
 *     sigma_b) and ends in s_n = sigma_b (tail-biting with a given state).  sigma_b is masked to its low L bits.
 *     If no path satisfies the constraint (possible only when n < L/k), that sequence's outputs are NaN
 *     (soft and gradient), log_z is -inf, and the Viterbi cost is +inf.
 *
 * Memory and execution, for every entry point:
 *   - every tensor pointer is a DEVICE pointer to contiguous row-major memory owned by the caller: w, w_soft,
 *     grad_w_soft, grad_w, w_hard are float32 [B, n]; codebook and grad_codebook are float32 [2^L];
 *     boundary_state, log_z and cost are [B]; states is int32 [B, n].  Outputs must not alias inputs or each other.
 *   - workspace is device scratch memory owned by the caller, at least bcjr_workspace_bytes(...) bytes, aligned
 *     to 256 bytes; its contents on entry do not matter and are clobbered.  The library allocates nothing,
 *     frees nothing, keeps no state between calls and never synchronizes: the work is enqueued on `stream`
 *     (a hipStream_t; NULL = the default stream) and outputs are valid once the caller synchronizes with it.
 *     Calls on different streams need different workspaces.
 *   - supported shapes: 1 <= n <= 4096, 1 <= B <= 2^31 - 1, 4 <= L <= 16 with L >= 2k, and
 *       every entry point: 1 <= k <= 4 and V = 1 or 2 (k = 2 with V = 1 runs kernels tuned for it, every other
 *       (k, V) one kernel family written for any k);
 *       exact tail-biting (the exact start-state choice, and the soft codeword and gradient under the
 *       tail-biting measure) needs L <= 10.
 *   - the kernels run persistent grids of one or more workgroups per compute unit of the current device, so the
 *     workspace sizes scale with its CU count (asked of the runtime once per device; 256, an MI355X's count, when
 *     no device is visible).  Query the workspace with the device current that will run the call.
 *   - every check except BCJR_ERR_HIP runs on the host before any kernel launch; on error nothing is enqueued and
 *     the outputs are untouched.  NaN/Inf inside w, codebook or grad_w_soft are not checked: they propagate
 *     into that sequence's outputs.
 */
#ifndef BCJR_H
#define BCJR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    BCJR_OK = 0,
    BCJR_ERR_NULL = -1,        /* a required pointer is NULL */
    BCJR_ERR_SHAPE = -2,       /* B < 1 or B >= 2^31, n < 1 or n > 4096, k < 1, L < 4, L < 2k or L > 16 */
    BCJR_ERR_TEMP = -3,        /* T not finite, or T < 1e-12 (soft and gradient only) */
    BCJR_ERR_UNSUPPORTED = -4, /* valid shape without a kernel: k > 4 or V > 2; exact tail-biting (choice of
                                  sigma, soft codeword or gradient under the tail-biting measure) with L > 10;
                                  unknown mode */
    BCJR_ERR_WORKSPACE = -5,   /* workspace NULL, not 256-byte aligned, or smaller than bcjr_workspace_bytes();
                                  bcjr_soft_codeword_noalloc: one sequence needs more than the static scratch */
    BCJR_ERR_HIP = -6          /* the HIP runtime reported an error at launch */
};

enum {
    BCJR_OP_SOFT = 0,
    BCJR_OP_GRAD = 1,
    BCJR_OP_VITERBI = 2,
    BCJR_OP_GRAD_CODEBOOK = 3,
    BCJR_OP_VITERBI_TB_EXACT = 4,  /* viterbi_tail_biting, mode BCJR_TB_EXACT */
    BCJR_OP_VITERBI_TB_ROTATE = 5, /* viterbi_tail_biting, mode BCJR_TB_ROTATE */
    BCJR_OP_SOFT_TAIL_BITING = 6,  /* bcjr_soft_codeword_tail_biting */
    BCJR_OP_GRAD_TAIL_BITING = 7   /* bcjr_soft_codeword_grad_tail_biting */
};

enum { BCJR_TB_EXACT = 0, BCJR_TB_ROTATE = 1 };

/*
 * Soft codeword (gist.science Technical Summary, "Core Mechanism"):
 *   w_soft[b, t] = sum_s codebook[s] * p_T(s_t = s | w_b),  p_T(path) proportional to exp(-E(path) / T),
 * computed exactly by the log-domain BCJR forward-backward recursion (abstract; "Key Technical Innovations").
 * log_z[b] = ln Z_b = ln sum_paths exp(-E / T) over the emitting states (optional output, may be NULL).
 * Returns BCJR_OK or a negative status.
 */
int bcjr_soft_codeword(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L, int32_t k, float T,
                       const int32_t* boundary_state, float* w_soft, float* log_z, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * Gradient of the soft codeword with respect to the weight pre-image w (the soft codeword is differentiable in w
 * without approximation, gist.science Technical Summary, "Core Mechanism"):
 *   grad_w[b, u] = sum_t grad_w_soft[b, t] * d w_soft[b, t] / d w[b, u]
 *               = (2 / T) * Cov_p( codebook[s_u], sum_t grad_w_soft[b, t] * codebook[s_t] ),
 * the covariance taken under the same Boltzmann path measure.  grad_w_soft is the upstream dL/dw_soft (required).
 * w_soft (optional, may be NULL) receives the soft codeword of the same pass.
 */
int bcjr_soft_codeword_grad(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L, int32_t k,
                            float T, const int32_t* boundary_state, const float* grad_w_soft, float* grad_w,
                            float* w_soft, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Gradient of the soft codeword with respect to the codebook values, the trellis parameters in which the soft
 * codeword is also exactly differentiable (gist.science Technical Summary, "Core Mechanism"), summed over the batch
 * because every sequence reads the same codebook:
 *   grad_codebook[v] = sum_b sum_t grad_w_soft[b, t] * d w_soft[b, t] / d codebook[v]
 *                    = sum_b sum_u p(s_u = v) * ( grad_w_soft[b, u]
 *                                                 + (2 / T) (w[b, u] - codebook[v]) (E[F_b | s_u = v] - E[F_b]) ),
 * with F_b = sum_t grad_w_soft[b, t] * codebook[s_t] and p the Boltzmann path measure of sequence b.  codebook[v]
 * enters w_soft both as the emitted value and through the path energies.  grad_codebook is float32 [2^L], written
 * in full (required).  grad_w (float32 [B, n]) and w_soft receive the same values as bcjr_soft_codeword_grad would
 * give, up to rounding; each may be NULL.  One sequence with no admissible path (see above) makes every entry of
 * grad_codebook NaN.  The result is deterministic: the per-slot partial sums are added in a fixed order.
 * The workspace holds, besides what bcjr_soft_codeword_grad needs, one float accumulator per state per slot.
 */
int bcjr_soft_codeword_grad_codebook(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L,
                                     int32_t k, float T, const int32_t* boundary_state, const float* grad_w_soft,
                                     float* grad_codebook, float* grad_w, float* w_soft, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * Viterbi hard code, the T -> 0 limit of the soft codeword (abstract): the path of minimum energy.  Arithmetic is
 * IEEE float32 in a fixed order, without fused multiply-add:
 *   M_1(s) = fl(d*d), d = fl(w_1 - codebook[s]);  M_t(s) = fl(fl(d*d) + min over predecessors p of M_{t-1}(p)),
 * ties between predecessors go to the one with the smallest index, ties between end states to the smallest state.
 * states[b, t] = s_t (int32, t = 1..n); w_hard[b, t] = codebook[s_t] (optional); cost[b] = M_n(s_n) (optional).
 * T plays no part.
 */
int viterbi_hard_code(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L, int32_t k,
                      const int32_t* boundary_state, int32_t* states, float* w_hard, float* cost, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * Soft codeword under the tail-biting measure: every path with s_0 = s_n weighs exp(-E / T), whatever that state
 * (the variant of the soft codeword whose start state equals its end state, that state summed over rather than
 * given).
 * It is the mixture over sigma of the sigma-mode measures with weights Z_sigma / sum Z, so
 *   w_soft[b, t] = sum_sigma pi_sigma w_soft_sigma[b, t],   log_z[b] = ln sum_sigma Z_sigma (optional output),
 * computed exactly from one sigma-mode pass per (row, sigma): L <= 10, else BCJR_ERR_UNSUPPORTED.  Workspace:
 * bcjr_workspace_bytes with BCJR_OP_SOFT_TAIL_BITING (it holds the 2^L per-sigma soft codewords of every row).
 */
int bcjr_soft_codeword_tail_biting(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L,
                                   int32_t k, float T, float* w_soft, float* log_z, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * Gradient with respect to the weights of the soft codeword under the tail-biting measure, for an upstream
 * grad_w_soft (required):  grad_w[b, u] = sum_t grad_w_soft[b, t] d w_soft[b, t] / d w[b, u].  With
 * d ln Z_sigma / d w_u = (2/T)(w_soft_sigma,u - w_u) this is the mixture of the sigma-mode gradients plus
 * (2/T) sum_sigma pi_sigma (w_soft_sigma,u - w_soft_u)(F_sigma - F_bar), F_sigma = sum_t grad_w_soft_t w_soft_sigma,t.
 * w_soft (optional) receives the tail-biting soft codeword.  L <= 10, else BCJR_ERR_UNSUPPORTED.  Workspace:
 * bcjr_workspace_bytes with BCJR_OP_GRAD_TAIL_BITING.
 */
int bcjr_soft_codeword_grad_tail_biting(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L,
                                        int32_t k, float T, const float* grad_w_soft, float* grad_w, float* w_soft,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Tail-biting Viterbi hard code with the start state chosen by the decoder: the minimum-energy path under the
 * constraint s_0 = s_n (the non-emitting start state equals the last emitting state), the hard code's variant whose
 * start state equals its end state.  The pages fix no rule for choosing the state; two are offered:
 *   BCJR_TB_EXACT   every sigma in [0, 2^L) is decoded as in viterbi_hard_code's sigma mode, and sigma is the
 *                   smallest state whose path cost is the minimum (L <= 10, else BCJR_ERR_UNSUPPORTED);
 *   BCJR_TB_ROTATE  rotate-and-decode: the sequence rotated left by n/2 (weight (t + n/2) mod n at step t) is
 *                   decoded with a free start and end, and sigma is that path's state at the original last weight,
 *                   where the cycle closes; any L.  A heuristic: its cost is never below the exact one.
 * Either way the result is the sigma-mode decode with that sigma, in the same float32 order and tie rules as
 * viterbi_hard_code: states [B, n] (required), w_hard and cost (optional), and sigma [B] int32 (optional) receives
 * the chosen start state.  An unknown mode gives BCJR_ERR_UNSUPPORTED.  Workspace: bcjr_workspace_bytes with
 * BCJR_OP_VITERBI_TB_EXACT or BCJR_OP_VITERBI_TB_ROTATE.
 */
int viterbi_tail_biting(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L, int32_t k,
                        int32_t mode, int32_t* states, float* w_hard, float* cost, int32_t* sigma, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * V weights per trellis step (the pages fix neither k nor V; a state then emits the V-vector codebook[s, 0..V-1]).
 * The same three operations as bcjr_soft_codeword, bcjr_soft_codeword_grad and viterbi_hard_code, with the same
 * arguments plus V, and these shapes: codebook float32 [2^L, V] (row-major: state-major, then component); w,
 * w_soft, grad_w_soft, grad_w and w_hard float32 [B, n V], where step t of row b owns w[b, t V .. t V + V - 1];
 * states int32 [B, n], one state per step; n counts trellis steps.  The energy of a path is
 * E = sum_t sum_v (w[b, t V + v] - codebook[s_t, v])^2, so per component
 *   w_soft[b, t V + v] = sum_s codebook[s, v] p_T(s_t = s | w_b),
 *   grad_w[b, u V + v] = (2 / T) Cov_p( codebook[s_u, v], sum_t sum_v' grad_w_soft[b, t V + v'] codebook[s_t, v'] ),
 * and the Viterbi metric adds the components' squares in index order, e = fl(d_0 d_0), e = fl(e + fl(d_v d_v)),
 * before adding the predecessor's metric, again without fused multiply-add.  V = 1 is the scalar trellis above, and
 * the entry points without _v are these with V = 1.  V must be 1 or 2 (BCJR_ERR_SHAPE below 1, BCJR_ERR_UNSUPPORTED
 * above 2).  Workspace: bcjr_workspace_bytes_v with the matching BCJR_OP_SOFT, BCJR_OP_GRAD, BCJR_OP_GRAD_CODEBOOK
 * or BCJR_OP_VITERBI.
 */
int bcjr_soft_codeword_v(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L, int32_t k,
                         int32_t V, float T, const int32_t* boundary_state, float* w_soft, float* log_z,
                         void* workspace, size_t workspace_bytes, void* stream);
int bcjr_soft_codeword_grad_v(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L, int32_t k,
                              int32_t V, float T, const int32_t* boundary_state, const float* grad_w_soft,
                              float* grad_w, float* w_soft, void* workspace, size_t workspace_bytes, void* stream);
int viterbi_hard_code_v(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L, int32_t k,
                        int32_t V, const int32_t* boundary_state, int32_t* states, float* w_hard, float* cost,
                        void* workspace, size_t workspace_bytes, void* stream);
/* The codebook gradient with V weights per step, per component:
 *   grad_codebook[s, v] = sum_b sum_u p(s_u = s) ( grad_w_soft[b, u V + v]
 *                                                  + (2 / T) (w[b, u V + v] - codebook[s, v]) (E[F_b | s_u = s] - E[F_b]) ),
 * F_b = sum_t sum_v grad_w_soft[b, t V + v] codebook[s_t, v]; grad_codebook is float32 [2^L, V].  Otherwise as
 * bcjr_soft_codeword_grad_codebook.  Workspace: bcjr_workspace_bytes_v with BCJR_OP_GRAD_CODEBOOK. */
int bcjr_soft_codeword_grad_codebook_v(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L,
                                       int32_t k, int32_t V, float T, const int32_t* boundary_state,
                                       const float* grad_w_soft, float* grad_codebook, float* grad_w, float* w_soft,
                                       void* workspace, size_t workspace_bytes, void* stream);
/* The three tail-biting entry points with V weights per step (shapes as above: w, w_soft, grad_w_soft, grad_w and
 * w_hard [B, n V], codebook [2^L, V], states [B, n]).  The mixture formulas hold per weight component, the sums over
 * t running over all n V weights of the row; BCJR_TB_ROTATE rotates by n/2 trellis steps (n/2 V weights).
 * Workspace: bcjr_workspace_bytes_v with the matching BCJR_OP_*_TAIL_BITING or BCJR_OP_VITERBI_TB_* value. */
int bcjr_soft_codeword_tail_biting_v(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L,
                                     int32_t k, int32_t V, float T, float* w_soft, float* log_z, void* workspace,
                                     size_t workspace_bytes, void* stream);
int bcjr_soft_codeword_grad_tail_biting_v(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L,
                                          int32_t k, int32_t V, float T, const float* grad_w_soft, float* grad_w,
                                          float* w_soft, void* workspace, size_t workspace_bytes, void* stream);
int viterbi_tail_biting_v(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L, int32_t k,
                          int32_t V, int32_t mode, int32_t* states, float* w_hard, float* cost, int32_t* sigma,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace the entry point `op` (one of the BCJR_OP_* values above) needs for
 * these shapes on the current device; 0 when the shapes are invalid or unsupported.  Enqueues nothing; the only
 * HIP call is the one-time query of the device's CU count.
 */
size_t bcjr_workspace_bytes(int32_t op, int64_t B, int64_t n, int32_t L, int32_t k);

/* The same for V weights per step, every op: bcjr_workspace_bytes(op, ...) is this with V = 1. */
size_t bcjr_workspace_bytes_v(int32_t op, int64_t B, int64_t n, int32_t L, int32_t k, int32_t V);

/*
 * The smallest workspace `op` runs with.  The soft codeword and the two gradients (BCJR_OP_SOFT, BCJR_OP_GRAD,
 * BCJR_OP_GRAD_CODEBOOK) have two memory modes, and the entry point picks one by the workspace_bytes it is given:
 *   - the full tape: every forward message row kept for the backward pass (bcjr_workspace_bytes[_v], the fastest);
 *   - checkpoints: every c-th row kept, c = ceil(sqrt(n)), and the backward pass recomputes the rows of each c-step
 *     segment from its checkpoint before it consumes them.  That costs one more forward pass of compute; the
 *     message rows per in-flight sequence drop from (n + 1) to about 2 sqrt(n), e.g. 4097 -> 128 rows at n = 4096
 *     (the gradients keep two such tapes; the codebook gradient's [2^L][V] accumulator per slot is not reduced).
 * A workspace at least bcjr_workspace_bytes_min but smaller than the full tape selects the second; the results are
 * the same up to rounding (the recomputed rows are bit-identical; the two modes may run different kernels).  Where
 * the rounding to 256-byte areas leaves checkpoints no smaller (n <= 3, or tiny rows), this equals the full tape.
 * For Viterbi and the tail-biting ops this is bcjr_workspace_bytes_v.  0 when the shapes are invalid or unsupported.
 */
size_t bcjr_workspace_bytes_min(int32_t op, int64_t B, int64_t n, int32_t L, int32_t k, int32_t V);

/* Bytes of the static device scratch that bcjr_soft_codeword_noalloc works in (per device). */
#define BCJR_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

/*
 * bcjr_soft_codeword without a workspace argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  It computes what bcjr_soft_codeword computes,
 * with the same arguments minus workspace and workspace_bytes, in a static device array of
 * BCJR_NOALLOC_SCRATCH_BYTES (256 MiB) that the library holds on each device it runs on until the process ends; it
 * calls no allocating routine.  The scratch's address is looked up on the first call on each device.
 *   - When the full message tape of every workgroup fits in the scratch it is used; otherwise the checkpoint mode of
 *     bcjr_workspace_bytes_min, with the persistent grid cut to the workgroups whose slots fit (each then decodes
 *     more sequences in turn).  At L = 16, k = 2, n = 256 that is the checkpoint mode on 122 workgroups.  The results
 *     are those bcjr_soft_codeword gives with a workspace of the same mode.
 *   - BCJR_ERR_WORKSPACE when one workgroup's slots alone exceed the scratch (no shape within the limits above does
 *     at L <= 16 with checkpoints; the error exists for the rule's sake).
 *   - Every call on one device shares that device's scratch, so calls that overlap in time on one device race and
 *     give wrong results: serialize them (one stream, or events).  The scratch keeps the last call's contents; the
 *     kernels need none of it on entry.
 */
int bcjr_soft_codeword_noalloc(const float* w, const float* codebook, int64_t B, int64_t n, int32_t L, int32_t k,
                               float T, const int32_t* boundary_state, float* w_soft, float* log_z, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* bcjr_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* BCJR_H */
