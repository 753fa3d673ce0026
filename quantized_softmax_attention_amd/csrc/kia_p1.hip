// P1 zero-sum projection of the detached score gradient (gfx950).
//
// "Pretraining Transformers with Quantized Softmax in Attention" (paperlayer
// digest), App. B and section 5.1: the detached gradient of a row minus its
// mean over the row's causal keys, dS_tj = dS_det,tj - mu_t.  The row kernel
// runs the detach rule, takes mu_t from its exact row sum and corrects
// dQ_t by -mu_t * sum_{j <= t} K_j / sqrt(d) (the causal prefix sums below);
// the centring kernel then subtracts mu_t from the stored dS tiles, so the
// column kernel's dK = dS^T Q / sqrt(d) needs no change.
#include "kia_common.hpp"
#include "kia_kernels.hpp"

namespace kia {

// Sums of K over each 32-row chunk: chunk_k[bh][c][col].  One thread per
// column (coalesced across the block), fp64 accumulation.
__global__ __launch_bounds__(128) void kia_key_chunk_sums_kernel(const float* k, float* chunk_k, int T, int n_t, int d) {
    const int c = blockIdx.x, bh = blockIdx.y, col = threadIdx.x;
    if (col >= d) return;
    const float* kp = k + ((size_t)bh * T + (size_t)c * kTile) * d + col;
    const int rows = min(kTile, T - c * kTile);
    double acc = 0.0;
    for (int i = 0; i < rows; ++i) acc += (double)kp[(size_t)i * d];
    chunk_k[((size_t)bh * n_t + c) * d + col] = (float)acc;
}

// Causal prefix sums of K: prefix_k[bh][t][col] = sum_{j <= t} K[bh][j][col],
// the earlier chunks' sums plus a running sum inside the chunk, in fp64.
__global__ __launch_bounds__(128) void kia_key_prefix_kernel(const float* k, const float* chunk_k, float* prefix_k,
                                                             int T, int n_t, int d) {
    const int c = blockIdx.x, bh = blockIdx.y, col = threadIdx.x;
    if (col >= d) return;
    double run = 0.0;
    for (int cc = 0; cc < c; ++cc) run += (double)chunk_k[((size_t)bh * n_t + cc) * d + col];
    const size_t base = ((size_t)bh * T + (size_t)c * kTile) * d + col;
    const int rows = min(kTile, T - c * kTile);
    for (int i = 0; i < rows; ++i) {
        run += (double)k[base + (size_t)i * d];
        prefix_k[base + (size_t)i * d] = (float)run;
    }
}

// dS_tj -= mu_t for every causal entry of the key-major dS tiles (mu_t in
// row_cm).  One workgroup per tile, one float4 (four queries, one key) per
// thread; entries past the row's causal range or the sequence end stay 0.
__global__ __launch_bounds__(256) void kia_center_rows_kernel(float* dscores, const float* mu, int T, int n_t,
                                                              int64_t tiles_per_head) {
    const int64_t g = blockIdx.x;
    const int bh = (int)(g / tiles_per_head);
    const int ti = (int)(g % tiles_per_head);
    int qt, kt;
    tile_coords(ti, qt, kt);
    float* tp = dscores + (size_t)g * kTileElems;
    const int o = threadIdx.x * 4;               // key-major offset of this float4
    const int inner = (o & 255) >> 2;
    const int kj = inner & 31;
    const int qi0 = (o >> 8) * 8 + (inner >> 5) * 4;
    const int k = kt * kTile + kj;
    f32x4 x = *(f32x4*)(tp + o);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int q = qt * kTile + qi0 + j;
        if (q < T && k <= q) x[j] -= mu[(size_t)bh * T + q];
    }
    *(f32x4*)(tp + o) = x;
}

hipError_t launch_key_prefix(int d, const BwdArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)a.n_t, (unsigned)a.BH);
    hipLaunchKernelGGL(kia_key_chunk_sums_kernel, grid, dim3(128), 0, s, a.k, a.chunk_k, a.T, a.n_t, d);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kia_key_prefix_kernel, grid, dim3(128), 0, s, a.k, a.chunk_k, a.prefix_k, a.T, a.n_t, d);
    return hipGetLastError();
}

hipError_t launch_center_rows(const BwdArgs& a, hipStream_t s) {
    const int64_t tiles_per_head = (int64_t)a.n_t * (a.n_t + 1) / 2;
    hipLaunchKernelGGL(kia_center_rows_kernel, dim3((unsigned)(a.BH * tiles_per_head)), dim3(256), 0, s, a.dscores,
                       a.row_cm, a.T, a.n_t, tiles_per_head);
    return hipGetLastError();
}

}  // namespace kia
