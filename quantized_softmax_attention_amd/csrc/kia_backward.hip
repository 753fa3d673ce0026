// K-interval attention backward (gfx950): three kernels in stream order.
//
//   rows    one wavefront per (b, h, 32-query tile), sweeping the causal key
//           tiles: reload the forward's scores, dP^T = V dO^T on the matrix
//           cores, normalisation Jacobian at the surrogate's evaluation
//           point, direct score gradient, running calibration sums; then
//           dQ^T += K^T dS^T.  P and dS are written transposed (key-major) for
//           the column kernel.  At the end of the row the calibration terms
//           are complete: they are added to dQ (gathering K at the argmax and
//           argmin keys) and stored per row.
//   cols    one wavefront per (b, h, 32-key tile), sweeping the query tiles
//           at or below the diagonal: dV^T += dO^T P and dK^T += Q^T dS.
//   scatter per (b, h, 64-key block): adds the calibration terms of every row
//           whose argmax / argmin key is in the block, C * Q_t / sqrt(d), to
//           dK in row order (deterministic, no atomics).
//
// Gradient rules: "Pretraining Transformers with Quantized Softmax in
// Attention" (paperlayer digest), section 3 "Calibration gradients" and
// "Surrogate placement", App. B "Gradient derivations"; max-only / min-only
// from App. F.  Per causal key j of row t, with u = (m - s)/h, LERP segment i,
// offset f, grid value g = exp(-i h), c = 1 - exp(-h):
//   dL/dw_j  = (dP_j - delta) / W_e           (normalisation Jacobian;
//              W_e, delta = dO . O_e at the hard point for LERP / Weight-STE,
//              at the LERP probabilities for Prob-STE)
//   dw/du    = -g c,   dw/dh|_u = -g (u - f (i+1) c)
//   direct   dS_j  = dL/dw_j * g c / h
//   MinMax   C_m = sum_j dL/dw_j (dw/du / h + Wd_j / K),  C_n = -sum_j dL/dw_j Wd_j / K
//            with Wd_j = dw/du * (-u/h) + dw/dh|_u = g ((c/h - 1) u + f (i+1) c)
//   FWM      C_m = sum_j dL/dw_j dw/du / h,  C_n = 0 (h does not depend on the row)
//   full adds C_m at the argmax and C_n at the argmin; detach adds neither;
//   max-only / min-only add one.  Degenerate rows: dS = P (dP - delta), no C.
#include "kia_common.hpp"
#include "kia_kernels.hpp"

namespace kia {

__device__ __forceinline__ void map_rows_task_b(int g, int BH, int n_t, int& bh, int& qt) {
    if ((BH & 7) == 0) {
        const int x = g & 7, s = g >> 3, per = BH >> 3;
        qt = n_t - 1 - s / per;
        bh = (s % per) * 8 + x;
    } else {
        qt = n_t - 1 - g / BH;
        bh = g % BH;
    }
}

// Key-stationary mapping: the first key tiles see the most query tiles.
__device__ __forceinline__ void map_cols_task(int g, int BH, int n_t, int& bh, int& kt) {
    if ((BH & 7) == 0) {
        const int x = g & 7, s = g >> 3, per = BH >> 3;
        kt = s / per;
        bh = (s % per) * 8 + x;
    } else {
        kt = g / BH;
        bh = g % BH;
    }
}

template <int D, int CAL, int REC, bool PROB>
__global__ __launch_bounds__(64) void kia_backward_rows_kernel(BwdArgs a) {
    constexpr int NB = D / 32;
    constexpr int LDS_STRIDE = kTile + 1;
    __shared__ float lds_p[kTile * LDS_STRIDE];
    __shared__ float lds_ds[kTile * LDS_STRIDE];

    const int lane = threadIdx.x;
    const int li = lane & 31, hl = lane >> 5;
    int bh, qt;
    map_rows_task_b(blockIdx.x, a.BH, a.n_t, bh, qt);
    const int T = a.T;
    const int q0 = qt * kTile;
    const int qrow = q0 + li;
    const bool qvalid = qrow < T;
    const size_t head = (size_t)bh * T * D;
    const float* Kp = a.k + head;
    const float* V = a.v + head;
    const int64_t tiles_per_head = (int64_t)a.n_t * (a.n_t + 1) / 2;
    const size_t tile0 = ((size_t)bh * tiles_per_head + tile_index(qt, 0)) * kTileElems;
    const float* stiles = a.tiles + tile0;
    float* ptiles = a.probs + tile0;
    float* dstiles = a.dscores + tile0;

    // B operand of dP^T = V dO^T (dO row of this lane's query), and delta.
    const float* oe = (REC == REC_NEAREST && PROB) ? a.o_lerp : a.o;
    float dof[D / 2];
    float dlt = 0.f;
#pragma unroll
    for (int p = 0; p < D / 8; ++p) {
        f32x4 x = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
        if (qvalid) {
            x = *(const f32x4*)(a.d_o + head + (size_t)qrow * D + 8 * p + 4 * hl);
            y = *(const f32x4*)(oe + head + (size_t)qrow * D + 8 * p + 4 * hl);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            dof[4 * p + j] = x[j];
            dlt = fmaf(x[j], y[j], dlt);
        }
    }
    dlt += __shfl_xor(dlt, 32);

    const size_t ri = (size_t)bh * T + (qvalid ? qrow : 0);
    const float m = qvalid ? a.row_m[ri] : 0.f;
    const float n = qvalid ? a.row_n[ri] : 0.f;
    const float W = qvalid ? a.row_w[ri] : 1.f;
    const float WL = qvalid ? a.row_wl[ri] : 1.f;
    const RowGrid rg = make_row_grid(m, n, a.K, a.tau, CAL);
    const float invW = 1.f / W;
    // a row with a single causal key has P = 1 whatever its score: zero gradient
    const float invWe = (qrow == 0) ? 0.f : ((REC == REC_NEAREST && PROB) ? 1.f / WL : invW);

    float SA = 0.f, SB = 0.f;  // row sums of the direct term and of dL/dw * Wd
    f32x16 dq[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) dq[b] = f32x16{};

    for (int kt = 0; kt <= qt; ++kt) {
        const int k0 = kt * kTile;
        const int krow = k0 + li;
        float sv[16];
        {
            const float* tp = stiles + (size_t)kt * kTileElems;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                f32x4 x = *(const f32x4*)(tp + p * 256 + lane * 4);
#pragma unroll
                for (int j = 0; j < 4; ++j) sv[4 * p + j] = x[j];
            }
        }
        // dP^T = V dO^T : A operand row = key
        float vf[D / 2];
#pragma unroll
        for (int p = 0; p < D / 8; ++p) {
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            if (krow < T) x = *(const f32x4*)(V + (size_t)krow * D + 8 * p + 4 * hl);
#pragma unroll
            for (int j = 0; j < 4; ++j) vf[4 * p + j] = x[j];
        }
        f32x16 dp = {};
#pragma unroll
        for (int kk = 0; kk < D / 2; ++kk) dp = mfma32x32x2(vf[kk], dof[kk], dp);

        float ds[16], pr[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = k0 + acc_row(r, hl);
            const bool valid = qvalid && key <= qrow;
            const Recon e = reconstruct<CAL, REC == REC_NEAREST>(rg, sv[r]);
            const bool keep = valid && e.inwin;
            const float wh = (REC == REC_LERP) ? e.wl : e.wn;
            pr[r] = keep ? wh * invW : 0.f;
            const float gt = (dp[r] - dlt) * invWe;
            const float A = gt * e.g * rg.coh;
            const float Wd = e.g * fmaf(rg.coh - 1.f, e.uc, e.f * (e.fi + 1.f) * rg.c);
            ds[r] = keep ? A : 0.f;
            SA += ds[r];
            SB += keep ? gt * Wd : 0.f;
        }

        // transpose P and dS to key-major through LDS
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kj = acc_row(r, hl);
            lds_p[kj * LDS_STRIDE + li] = pr[r];
            lds_ds[kj * LDS_STRIDE + li] = ds[r];
        }
        __syncthreads();
        {
            float* pp = ptiles + (size_t)kt * kTileElems;
            float* dd = dstiles + (size_t)kt * kTileElems;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                f32x4 x, y;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int qq = 2 * (4 * p + j) + hl;
                    x[j] = lds_p[li * LDS_STRIDE + qq];
                    y[j] = lds_ds[li * LDS_STRIDE + qq];
                }
                *(f32x4*)(pp + p * 256 + lane * 4) = x;
                *(f32x4*)(dd + p * 256 + lane * 4) = y;
            }
        }
        __syncthreads();

        // dQ^T += K^T dS^T
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) {
                const int key = k0 + acc_row(kk, hl);
                const float kv = key < T ? Kp[(size_t)key * D + 32 * b + li] : 0.f;
                dq[b] = mfma32x32x2(kv, ds[kk], dq[b]);
            }
        }
    }

    SA += __shfl_xor(SA, 32);
    SB += __shfl_xor(SB, 32);
    float Cm, Cn;
    if (CAL == CAL_MINMAX) {
        Cm = -SA + SB / rg.Kf;
        Cn = -SB / rg.Kf;
    } else {
        Cm = -SA;
        Cn = 0.f;
    }
    if (rg.degen) { Cm = 0.f; Cn = 0.f; }
    const bool use_max = (a.rule == GRAD_FULL || a.rule == GRAD_MAX_ONLY);
    const bool use_min = CAL == CAL_MINMAX && (a.rule == GRAD_FULL || a.rule == GRAD_MIN_ONLY);
    const float cm = use_max ? Cm : 0.f;
    const float cn = use_min ? Cn : 0.f;

    if (qvalid) {
        const int ka = a.row_a[ri];
        const int kb = a.row_b[ri];
        float* dqrow = a.dq + head + (size_t)qrow * D;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int c = 32 * b + 8 * p + 4 * hl;
                const f32x4 xa = *(const f32x4*)(Kp + (size_t)ka * D + c);
                const f32x4 xb = *(const f32x4*)(Kp + (size_t)kb * D + c);
                f32x4 y;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    y[j] = (dq[b][4 * p + j] + cm * xa[j] + cn * xb[j]) * a.scale;
                *(f32x4*)(dqrow + c) = y;
            }
        if (hl == 0) {
            a.row_cm[ri] = cm;
            a.row_cn[ri] = cn;
        }
    }
}

template <int D>
__global__ __launch_bounds__(64) void kia_backward_cols_kernel(BwdArgs a) {
    constexpr int NB = D / 32;
    const int lane = threadIdx.x;
    const int li = lane & 31, hl = lane >> 5;
    int bh, kt;
    map_cols_task(blockIdx.x, a.BH, a.n_t, bh, kt);
    const int T = a.T;
    const int krow = kt * kTile + li;
    const size_t head = (size_t)bh * T * D;
    const float* Q = a.q + head;
    const float* dO = a.d_o + head;
    const int64_t tiles_per_head = (int64_t)a.n_t * (a.n_t + 1) / 2;
    const size_t hbase = (size_t)bh * tiles_per_head;

    f32x16 dv[NB], dk[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) { dv[b] = f32x16{}; dk[b] = f32x16{}; }

    for (int qt = kt; qt < a.n_t; ++qt) {
        const size_t toff = (hbase + tile_index(qt, kt)) * kTileElems;
        float pv[16], dsv[16];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const f32x4 x = *(const f32x4*)(a.probs + toff + p * 256 + lane * 4);
            const f32x4 y = *(const f32x4*)(a.dscores + toff + p * 256 + lane * 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) { pv[4 * p + j] = x[j]; dsv[4 * p + j] = y[j]; }
        }
        const int q0 = qt * kTile;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) {
                const int q = q0 + 2 * kk + hl;
                const bool ok = q < T;
                const float dov = ok ? dO[(size_t)q * D + 32 * b + li] : 0.f;
                const float qv = ok ? Q[(size_t)q * D + 32 * b + li] : 0.f;
                dv[b] = mfma32x32x2(dov, pv[kk], dv[b]);
                dk[b] = mfma32x32x2(qv, dsv[kk], dk[b]);
            }
        }
    }
    if (krow < T) {
        float* dkrow = a.dk + head + (size_t)krow * D;
        float* dvrow = a.dv + head + (size_t)krow * D;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int c = 32 * b + 8 * p + 4 * hl;
                f32x4 x, y;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    x[j] = dk[b][4 * p + j] * a.scale;
                    y[j] = dv[b][4 * p + j];
                }
                *(f32x4*)(dkrow + c) = x;
                *(f32x4*)(dvrow + c) = y;
            }
    }
}

// Calibration terms onto dK: block of 64 keys, rows in ascending order.
template <int D>
__global__ __launch_bounds__(64) void kia_backward_scatter_kernel(BwdArgs a) {
    constexpr int KB = 64;
    __shared__ float acc[KB * D];
    const int lane = threadIdx.x;
    const int T = a.T;
    const int nkb = (T + KB - 1) / KB;
    const int bh = blockIdx.x / nkb;
    const int j0 = (blockIdx.x % nkb) * KB;
    const size_t head = (size_t)bh * T * D;
    const float* Q = a.q + head;
    for (int i = lane; i < KB * D; i += kWave) acc[i] = 0.f;
    __syncthreads();
    bool any = false;
    for (int t0 = j0; t0 < T; t0 += kWave) {
        const int t = t0 + lane;
        int ta = -1, tb = -1;
        float cm = 0.f, cn = 0.f;
        if (t < T) {
            const size_t ri = (size_t)bh * T + t;
            ta = a.row_a[ri];
            tb = a.row_b[ri];
            cm = a.row_cm[ri];
            cn = a.row_cn[ri];
        }
        const bool hit_a = cm != 0.f && ta >= j0 && ta < j0 + KB;
        const bool hit_b = cn != 0.f && tb >= j0 && tb < j0 + KB;
        unsigned long long bal = __ballot(hit_a || hit_b);
        while (bal) {
            const int src = __ffsll(bal) - 1;
            bal &= bal - 1;
            const int ts = t0 + src;
            const int as = __shfl(ta, src), bs = __shfl(tb, src);
            const float cms = __shfl(cm, src), cns = __shfl(cn, src);
            const bool ha = __shfl((int)hit_a, src) != 0;
            const bool hb = __shfl((int)hit_b, src) != 0;
            for (int c = lane; c < D; c += kWave) {
                const float qv = Q[(size_t)ts * D + c];
                if (ha) acc[(as - j0) * D + c] += cms * qv;
                if (hb) acc[(bs - j0) * D + c] += cns * qv;
            }
            any = true;
        }
    }
    if (!any) return;  // uniform across the wave (the ballot is)
    __syncthreads();
    for (int j = 0; j < KB; ++j) {
        const int key = j0 + j;
        if (key >= T) break;
        float* dkrow = a.dk + head + (size_t)key * D;
        for (int c = lane; c < D; c += kWave) dkrow[c] += acc[j * D + c] * a.scale;
    }
}

template <int D, int CAL, int REC, bool PROB>
static hipError_t launch_rows_t(const BwdArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((kia_backward_rows_kernel<D, CAL, REC, PROB>), dim3((unsigned)(a.BH * a.n_t)),
                       dim3(kWave), 0, s, a);
    return hipGetLastError();
}

template <int D, int CAL>
static hipError_t launch_rows_rec(const FwdConfig& c, const BwdArgs& a, hipStream_t s) {
    if (c.rec == REC_LERP) return launch_rows_t<D, CAL, REC_LERP, false>(a, s);
    return c.prob ? launch_rows_t<D, CAL, REC_NEAREST, true>(a, s)
                  : launch_rows_t<D, CAL, REC_NEAREST, false>(a, s);
}

template <int D>
static hipError_t launch_rows_d(const FwdConfig& c, const BwdArgs& a, hipStream_t s) {
    return c.cal == CAL_MINMAX ? launch_rows_rec<D, CAL_MINMAX>(c, a, s) : launch_rows_rec<D, CAL_FWM>(c, a, s);
}

hipError_t launch_backward_rows(const FwdConfig& c, const BwdArgs& a, hipStream_t s) {
    return c.d == 64 ? launch_rows_d<64>(c, a, s) : launch_rows_d<128>(c, a, s);
}

hipError_t launch_backward_cols(int d, const BwdArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)(a.BH * a.n_t));
    if (d == 64)
        hipLaunchKernelGGL((kia_backward_cols_kernel<64>), grid, dim3(kWave), 0, s, a);
    else
        hipLaunchKernelGGL((kia_backward_cols_kernel<128>), grid, dim3(kWave), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_backward_scatter(int d, const BwdArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)((a.T + 63) / 64 * a.BH));
    if (d == 64)
        hipLaunchKernelGGL((kia_backward_scatter_kernel<64>), grid, dim3(kWave), 0, s, a);
    else
        hipLaunchKernelGGL((kia_backward_scatter_kernel<128>), grid, dim3(kWave), 0, s, a);
    return hipGetLastError();
}

// ---- inspection: tile buffers to dense [BH, T, T] ---------------------------
__global__ __launch_bounds__(256) void kia_tiles_to_dense_kernel(int T, int n_t, const float* tiles,
                                                                 int key_major, float* dense) {
    const int bh = blockIdx.y;
    const int ti = blockIdx.x;
    // recover (qt, kt) from the triangular index qt*(qt+1)/2 + kt
    int qt = (int)((sqrtf(8.f * ti + 1.f) - 1.f) * 0.5f);
    while ((int64_t)qt * (qt + 1) / 2 > ti) --qt;
    while ((int64_t)(qt + 1) * (qt + 2) / 2 <= ti) ++qt;
    const int kt = ti - (int)tile_index(qt, 0);
    const int64_t tiles_per_head = (int64_t)n_t * (n_t + 1) / 2;
    const float* tp = tiles + ((size_t)bh * tiles_per_head + ti) * kTileElems;
    for (int e = threadIdx.x; e < kTileElems; e += blockDim.x) {
        const int qi = e >> 5, kj = e & 31;
        const int q = qt * kTile + qi, k = kt * kTile + kj;
        if (q >= T || k > q) continue;
        const int off = key_major ? kmajor_offset(qi, kj) : qmajor_offset(qi, kj);
        dense[((size_t)bh * T + q) * T + k] = tp[off];
    }
}

hipError_t launch_tiles_to_dense(int BH, int T, const float* tiles, int key_major, float* dense,
                                 hipStream_t s) {
    const int n_t = (T + kTile - 1) / kTile;
    const dim3 grid((unsigned)((int64_t)n_t * (n_t + 1) / 2), (unsigned)BH);
    hipLaunchKernelGGL(kia_tiles_to_dense_kernel, grid, dim3(256), 0, s, T, n_t, tiles, key_major, dense);
    return hipGetLastError();
}

}  // namespace kia
