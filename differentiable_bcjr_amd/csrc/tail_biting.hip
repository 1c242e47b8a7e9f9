// tail_biting.hip -- soft codeword and weights' gradient under the tail-biting measure, on gfx950.
//
// The tail-biting measure weighs every path with s_0 = s_n, whatever that state is.  It is the mixture over sigma of
// the sigma-constrained measures (the soft pass's sigma mode) with weights pi_sigma = Z_sigma / sum Z, so
//   w_soft_t = sum_sigma pi_sigma w_soft_sigma,t,   ln Z = logsumexp_sigma ln Z_sigma,
// and, since d ln Z_sigma / d w_u = (2/T) (w_soft_sigma,u - w_u),
//   grad_u = sum_sigma pi_sigma grad_sigma,u + (2/T) sum_sigma pi_sigma (w_soft_sigma,u - w_soft_u)(F_sigma - F_bar),
// with F_sigma = sum_t g_t w_soft_sigma,t and F_bar = sum_sigma pi_sigma F_sigma (BCJR-QAT, arXiv 2605.10655: the
// Boltzmann path measure and its exact derivative, gist.science Technical Summary, "Core Mechanism").  The soft and
// gradient kernels produce the per-sigma quantities with one virtual sequence per (row, sigma); the kernels here
// combine them, one block per row, in double and in a fixed order.  A sigma with no admissible path has
// ln Z_sigma = -inf and weight 0; its (NaN) outputs are skipped.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bcjr {

namespace {

constexpr int kThreads = 256;

// Per row: the mixture weights pi[S] (S <= 1024) into LDS, and ln Z of the row.
__device__ __forceinline__ double mixture_weights(const float* lz, int S, double* pi, double* red) {
    const int tid = threadIdx.x;
    double m = -__builtin_huge_val();
    for (int s = tid; s < S; s += kThreads) m = fmax(m, (double)lz[s]);
    red[tid] = m;
    __syncthreads();
    for (int o = kThreads / 2; o > 0; o >>= 1) {
        if (tid < o) red[tid] = fmax(red[tid], red[tid + o]);
        __syncthreads();
    }
    m = red[0];
    __syncthreads();
    double z = 0.0;
    for (int s = tid; s < S; s += kThreads) {
        const double e = (double)lz[s] == -__builtin_huge_val() ? 0.0 : exp((double)lz[s] - m);
        pi[s] = e;
        z += e;
    }
    red[tid] = z;
    __syncthreads();
    for (int o = kThreads / 2; o > 0; o >>= 1) {   // fixed tree: the same sum on every run
        if (tid < o) red[tid] += red[tid + o];
        __syncthreads();
    }
    z = red[0];
    __syncthreads();
    for (int s = tid; s < S; s += kThreads) pi[s] /= z;
    __syncthreads();
    return m + log(z);
}

}  // namespace

// w_soft[row, t] = sum_sigma pi_sigma ws_all[row, sigma, t]; log_z[row] = logsumexp_sigma lz_all[row, sigma].
__global__ void __launch_bounds__(kThreads) tb_soft_combine_kernel(const float* ws_all, const float* lz_all, int n,
                                                                  int S, float* w_soft, float* log_z) {
    __shared__ double pi[1024];
    __shared__ double red[kThreads];
    const int64_t row = blockIdx.x;
    const double lnz = mixture_weights(lz_all + row * S, S, pi, red);
    if (threadIdx.x == 0 && log_z) log_z[row] = (float)lnz;
    const float* base = ws_all + row * (int64_t)S * n;
    for (int t = threadIdx.x; t < n; t += kThreads) {
        double acc = 0.0;
        for (int s = 0; s < S; ++s)
            if (pi[s] > 0.0) acc += pi[s] * (double)base[(int64_t)s * n + t];
        w_soft[row * n + t] = (float)acc;
    }
}

// The weights' gradient under the mixture (see the header), and optionally its soft codeword.
__global__ void __launch_bounds__(kThreads) tb_grad_combine_kernel(const float* ws_all, const float* lz_all,
                                                                  const float* gr_all, const float* g, int n, int S,
                                                                  float two_over_T, float* grad, float* w_soft) {
    __shared__ double pi[1024];
    __shared__ double F[1024];
    __shared__ double red[kThreads];
    const int64_t row = blockIdx.x;
    mixture_weights(lz_all + row * S, S, pi, red);
    const float* wsb = ws_all + row * (int64_t)S * n;
    const float* grb = gr_all + row * (int64_t)S * n;
    const float* gb = g + row * n;
    // F_sigma = sum_t g_t w_soft_sigma,t, one sigma per thread
    for (int s = threadIdx.x; s < S; s += kThreads) {
        double f = 0.0;
        if (pi[s] > 0.0)
            for (int t = 0; t < n; ++t) f += (double)gb[t] * (double)wsb[(int64_t)s * n + t];
        F[s] = f;
    }
    __syncthreads();
    double fbar = 0.0;   // every thread forms the same sum in the same order
    for (int s = 0; s < S; ++s) fbar += pi[s] * F[s];
    for (int u = threadIdx.x; u < n; u += kThreads) {
        double wsu = 0.0, gru = 0.0;
        for (int s = 0; s < S; ++s)
            if (pi[s] > 0.0) {
                wsu += pi[s] * (double)wsb[(int64_t)s * n + u];
                gru += pi[s] * (double)grb[(int64_t)s * n + u];
            }
        double mix = 0.0;
        for (int s = 0; s < S; ++s)
            if (pi[s] > 0.0) mix += pi[s] * ((double)wsb[(int64_t)s * n + u] - wsu) * (F[s] - fbar);
        grad[row * n + u] = (float)(gru + (double)two_over_T * mix);
        if (w_soft) w_soft[row * n + u] = (float)wsu;
    }
}

// Rows rotated left by `shift` floats: out[row, x] = w[row, (x + shift) mod nv].  The rotate-and-decode start-state
// choice on the general trellis decodes these copies (shift = n/2 trellis steps of V weights).
__global__ void __launch_bounds__(kThreads) tb_rotate_rows_kernel(const float* w, int64_t rows, int nv, int shift,
                                                                 float* out) {
    const int64_t total = rows * nv;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kThreads) {
        const int64_t row = i / nv;
        const int x = (int)(i - row * nv);
        const int src = x + shift < nv ? x + shift : x + shift - nv;
        out[i] = w[row * nv + src];
    }
}

hipError_t launch_tb_rotate_rows(const float* w, int64_t rows, int nv, int shift, float* out, hipStream_t st) {
    const int64_t blocks = (rows * nv + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(tb_rotate_rows_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(kThreads), 0, st,
                       w, rows, nv, shift, out);
    return hipGetLastError();
}

hipError_t launch_tb_soft_combine(const float* ws_all, const float* lz_all, int64_t rows, int n, int S,
                                  float* w_soft, float* log_z, hipStream_t st) {
    hipLaunchKernelGGL(tb_soft_combine_kernel, dim3((unsigned)rows), dim3(kThreads), 0, st, ws_all, lz_all, n, S,
                       w_soft, log_z);
    return hipGetLastError();
}

hipError_t launch_tb_grad_combine(const float* ws_all, const float* lz_all, const float* gr_all, const float* g,
                                  int64_t rows, int n, int S, float two_over_T, float* grad, float* w_soft,
                                  hipStream_t st) {
    hipLaunchKernelGGL(tb_grad_combine_kernel, dim3((unsigned)rows), dim3(kThreads), 0, st, ws_all, lz_all, gr_all,
                       g, n, S, two_over_T, grad, w_soft);
    return hipGetLastError();
}

}  // namespace bcjr
