// P1 zero-sum projection of the detached score gradient (gfx950).
//
// "Pretraining Transformers with Quantized Softmax in Attention" (paperlayer
// digest), App. B and section 5.1: the detached gradient of a row minus its
// mean over the row's causal keys, dS_tj = dS_det,tj - mu_t.  The row kernel
// runs the detach rule, stores dS_det, takes mu_t from its exact row sum and
// corrects dQ_t by -mu_t * sum_{j <= t} K_j / sqrt(d) (the causal prefix sums
// of K below).  The mean reaches dK the same way: dK_j carries
// -sum_{t >= j} mu_t Q_t / sqrt(d), the suffix sums of mu_t Q_t below, which
// the column kernel subtracts when it stores dK; so no pass over the dS tiles
// is needed.
#include "kia_common.hpp"
#include "kia_kernels.hpp"

namespace kia {

// Both sums run over the rows of one head, column by column, in fp64: the
// causal prefix sums of K (term_t = K_t) and the suffix sums of mu_t Q_t
// (term_t = mu_t Q_t).  A workgroup of 256 threads takes one 32-row chunk:
// G = 256 / d groups of d threads, group g owning rows g*R .. g*R+R-1 of the
// chunk (R = 32 / G) and thread (g, col) one column of them.  A first kernel
// forms each chunk's sum; the second adds the chunks before (prefix) or after
// (suffix) the workgroup's, then the groups before or after its own, and
// runs through its rows.
template <bool MU>
__device__ __forceinline__ double scan_term(const float* x, const float* mu, size_t row, int d, int col) {
    const double v = (double)x[row * d + col];
    return MU ? (double)mu[row] * v : v;
}

template <bool MU>
__global__ __launch_bounds__(256) void kia_chunk_sums_kernel(const float* x, const float* mu, float* chunk, int T,
                                                             int n_t, int d) {
    __shared__ double part[256];
    const int c = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
    const int col = tid % d, g = tid / d, G = 256 / d, R = kTile / G;
    const size_t r0 = (size_t)bh * T + (size_t)c * kTile;
    const int rows = min(kTile, T - c * kTile);
    double acc = 0.0;
    for (int i = g * R; i < min(g * R + R, rows); ++i) acc += scan_term<MU>(x, mu, r0 + i, d, col);
    part[tid] = acc;
    __syncthreads();
    if (g == 0) {
        double sum = 0.0;
        for (int gg = 0; gg < G; ++gg) sum += part[gg * d + col];
        chunk[((size_t)bh * n_t + c) * d + col] = (float)sum;
    }
}

template <bool MU, bool SUFFIX>
__global__ __launch_bounds__(256) void kia_scan_kernel(const float* x, const float* mu, const float* chunk, float* out,
                                                       int T, int n_t, int d) {
    __shared__ double other[256], own[256];
    const int c = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
    const int col = tid % d, g = tid / d, G = 256 / d, R = kTile / G;
    const size_t r0 = (size_t)bh * T + (size_t)c * kTile;
    const int rows = min(kTile, T - c * kTile);
    // the other chunks' sums, shared out over the groups
    double oth = 0.0;
    if (SUFFIX) {
        for (int cc = n_t - 1 - g; cc > c; cc -= G) oth += (double)chunk[((size_t)bh * n_t + cc) * d + col];
    } else {
        for (int cc = g; cc < c; cc += G) oth += (double)chunk[((size_t)bh * n_t + cc) * d + col];
    }
    const int lo = g * R, hi = min(g * R + R, rows);
    double mine = 0.0;
    for (int i = lo; i < hi; ++i) mine += scan_term<MU>(x, mu, r0 + i, d, col);
    other[tid] = oth;
    own[tid] = mine;
    __syncthreads();
    double run = 0.0;
    for (int gg = 0; gg < G; ++gg) run += other[gg * d + col];
    for (int gg = 0; gg < G; ++gg)
        if (SUFFIX ? gg > g : gg < g) run += own[gg * d + col];
    if (SUFFIX) {
        for (int i = hi - 1; i >= lo; --i) {
            run += scan_term<MU>(x, mu, r0 + i, d, col);
            out[(r0 + i) * d + col] = (float)run;
        }
    } else {
        for (int i = lo; i < hi; ++i) {
            run += scan_term<MU>(x, mu, r0 + i, d, col);
            out[(r0 + i) * d + col] = (float)run;
        }
    }
}

hipError_t launch_key_prefix(int d, const BwdArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)a.n_t, (unsigned)a.BH);
    hipLaunchKernelGGL((kia_chunk_sums_kernel<false>), grid, dim3(256), 0, s, a.k, nullptr, a.chunk_k, a.T, a.n_t, d);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((kia_scan_kernel<false, false>), grid, dim3(256), 0, s, a.k, nullptr, a.chunk_k, a.prefix_k, a.T,
                       a.n_t, d);
    return hipGetLastError();
}

hipError_t launch_query_suffix(int d, const BwdArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)a.n_t, (unsigned)a.BH);
    hipLaunchKernelGGL((kia_chunk_sums_kernel<true>), grid, dim3(256), 0, s, a.q, a.row_cm, a.chunk_k, a.T, a.n_t, d);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((kia_scan_kernel<true, true>), grid, dim3(256), 0, s, a.q, a.row_cm, a.chunk_k, a.suffix_q, a.T,
                       a.n_t, d);
    return hipGetLastError();
}

}  // namespace kia
