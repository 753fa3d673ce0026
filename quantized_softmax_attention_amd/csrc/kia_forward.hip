// K-interval attention forward (gfx950).
//
// One wavefront per (b, h, 32-query tile).  Two sweeps over the causal key
// tiles, because both calibrations need the final row extremes before any
// weight is known (MinMax: h from the span; FWM: the window anchored at the
// max), and a moving anchor changes interval phases, so the weights cannot be
// rescaled on the fly as exact softmax can:
//   sweep 1: S^T = K Q^T on the fp32 matrix cores, scale 1/sqrt(d), causal
//            mask, running max/min with their key index; the scores are
//            stored once (query-major tiles) for sweep 2 and the backward;
//   sweep 2: reload the scores, reconstruct the weights on the grid, sum W,
//            accumulate O^T += V^T W^T on the matrix cores; O = acc / W.
// Operator: "Pretraining Transformers with Quantized Softmax in Attention"
// (paperlayer digest), section 3 "Calibration" / "Reconstruction" and App. A.
#include "kia_common.hpp"
#include "kia_kernels.hpp"

namespace kia {

// Work mapping for the query-stationary kernels: heaviest tiles (last query
// tiles, most causal keys) first; when B*H is a multiple of 8 a slice's tiles
// all land on one XCD (workgroups are dealt round-robin over the 8 XCDs) so
// its K and V stay in that XCD's L2.
__device__ __forceinline__ void map_rows_task(int g, int BH, int n_t, int& bh, int& qt) {
    if ((BH & 7) == 0) {
        const int x = g & 7, s = g >> 3, per = BH >> 3;
        qt = n_t - 1 - s / per;
        bh = (s % per) * 8 + x;
    } else {
        qt = n_t - 1 - g / BH;
        bh = g % BH;
    }
}

template <int D, int CAL, int REC, bool PROB, bool DUMP>
__global__ __launch_bounds__(64) void kia_forward_kernel(FwdArgs a) {
    static_assert(D % 32 == 0, "head dim must be a multiple of 32");
    constexpr int NB = D / 32;  // 32-wide blocks of the head dim
    const int lane = threadIdx.x;
    const int li = lane & 31, hl = lane >> 5;
    int bh, qt;
    map_rows_task(blockIdx.x, a.BH, a.n_t, bh, qt);
    const int T = a.T;
    const int q0 = qt * kTile;
    const int qrow = q0 + li;
    const bool qvalid = qrow < T;
    const size_t head = (size_t)bh * T * D;
    const float* Q = a.q + head;
    const float* Kp = a.k + head;
    const float* V = a.v + head;
    const int64_t tiles_per_head = (int64_t)a.n_t * (a.n_t + 1) / 2;
    float* tiles = a.tiles + ((size_t)bh * tiles_per_head + tile_index(qt, 0)) * kTileElems;

    // B operand of S^T = K Q^T: lane holds Q[qrow][c] for c = 8p + 4*hl + j.
    float qf[D / 2];
#pragma unroll
    for (int p = 0; p < D / 8; ++p) {
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (qvalid) x = *(const f32x4*)(Q + (size_t)qrow * D + 8 * p + 4 * hl);
#pragma unroll
        for (int j = 0; j < 4; ++j) qf[4 * p + j] = x[j];
    }

    // ---- sweep 1: scores, row extremes --------------------------------------
    float m = -INFINITY, n = INFINITY;
    int am = 0, an = 0;
    for (int kt = 0; kt <= qt; ++kt) {
        const int k0 = kt * kTile;
        const int krow = k0 + li;  // A operand row: key
        float kf[D / 2];
#pragma unroll
        for (int p = 0; p < D / 8; ++p) {
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            if (krow < T) x = *(const f32x4*)(Kp + (size_t)krow * D + 8 * p + 4 * hl);
#pragma unroll
            for (int j = 0; j < 4; ++j) kf[4 * p + j] = x[j];
        }
        f32x16 acc = {};
#pragma unroll
        for (int kk = 0; kk < D / 2; ++kk) acc = mfma32x32x2(kf[kk], qf[kk], acc);

        float sv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = k0 + acc_row(r, hl);
            const float s = acc[r] * a.scale;
            const bool valid = qvalid && key <= qrow;
            if (valid && s > m) { m = s; am = key; }
            if (CAL == CAL_MINMAX && valid && s < n) { n = s; an = key; }
            sv[r] = valid ? s : 0.f;
        }
        float* tp = tiles + (size_t)kt * kTileElems;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            f32x4 x = {sv[4 * p], sv[4 * p + 1], sv[4 * p + 2], sv[4 * p + 3]};
            *(f32x4*)(tp + p * 256 + lane * 4) = x;
        }
    }
    // the two lane halves of a query saw disjoint keys: merge, lowest index on ties
    {
        const float mo = __shfl_xor(m, 32);
        const int ao = __shfl_xor(am, 32);
        if (mo > m || (mo == m && ao < am)) { m = mo; am = ao; }
        if (CAL == CAL_MINMAX) {
            const float no = __shfl_xor(n, 32);
            const int bo = __shfl_xor(an, 32);
            if (no < n || (no == n && bo < an)) { n = no; an = bo; }
        }
    }
    if (!qvalid) { m = 0.f; n = 0.f; }
    const RowGrid rg = make_row_grid(m, n, a.K, a.tau, CAL);

    // ---- sweep 2: reconstruct, normalise, O = W V / sum(W) -----------------
    float W = 0.f, WL = 0.f;
    f32x16 oacc[NB];
    f32x16 olacc[PROB ? NB : 1];
#pragma unroll
    for (int b = 0; b < NB; ++b) oacc[b] = f32x16{};
#pragma unroll
    for (int b = 0; b < (PROB ? NB : 1); ++b) olacc[b] = f32x16{};

    for (int kt = 0; kt <= qt; ++kt) {
        const int k0 = kt * kTile;
        const float* tp = tiles + (size_t)kt * kTileElems;
        float sv[16];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            f32x4 x = *(const f32x4*)(tp + p * 256 + lane * 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) sv[4 * p + j] = x[j];
        }
        float w[16], wl[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = k0 + acc_row(r, hl);
            const bool valid = qvalid && key <= qrow;
            const Recon e = reconstruct<CAL, REC == REC_NEAREST>(rg, sv[r]);
            const bool keep = valid && e.inwin;
            const float wh = (REC == REC_LERP) ? e.wl : e.wn;
            w[r] = keep ? wh : 0.f;
            W += w[r];
            wl[r] = keep ? e.wl : 0.f;
            if (REC == REC_NEAREST) WL += wl[r];
            if (DUMP && valid) {
                int idx = (REC == REC_LERP) ? (int)e.fi : (int)floorf(e.uc + 0.5f);
                if (!e.inwin) idx = -1;
                a.idx_dump[((size_t)bh * T + qrow) * T + key] = idx;
            }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) {
                const int key = k0 + acc_row(kk, hl);
                const float vv = key < T ? V[(size_t)key * D + 32 * b + li] : 0.f;
                oacc[b] = mfma32x32x2(vv, w[kk], oacc[b]);
                if (PROB) olacc[b] = mfma32x32x2(vv, wl[kk], olacc[b]);
            }
        }
    }
    W += __shfl_xor(W, 32);
    if (REC == REC_NEAREST) WL += __shfl_xor(WL, 32);
    else WL = W;  // LERP: the forward weights are the LERP weights

    if (qvalid) {
        const float invW = 1.f / W;
        float* orow = a.o + head + (size_t)qrow * D;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                f32x4 x = {oacc[b][4 * p] * invW, oacc[b][4 * p + 1] * invW,
                           oacc[b][4 * p + 2] * invW, oacc[b][4 * p + 3] * invW};
                *(f32x4*)(orow + 32 * b + 8 * p + 4 * hl) = x;
            }
        if (PROB) {
            const float invWL = 1.f / WL;
            float* lrow = a.o_lerp + head + (size_t)qrow * D;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    f32x4 x = {olacc[b][4 * p] * invWL, olacc[b][4 * p + 1] * invWL,
                               olacc[b][4 * p + 2] * invWL, olacc[b][4 * p + 3] * invWL};
                    *(f32x4*)(lrow + 32 * b + 8 * p + 4 * hl) = x;
                }
        }
        if (hl == 0) {
            const size_t ri = (size_t)bh * T + qrow;
            a.row_m[ri] = m;
            a.row_n[ri] = (CAL == CAL_MINMAX) ? n : m;
            a.row_a[ri] = am;
            a.row_b[ri] = (CAL == CAL_MINMAX) ? an : am;
            a.row_w[ri] = W;
            a.row_wl[ri] = WL;
        }
    }
}

template <int D, int CAL, int REC, bool PROB, bool DUMP>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t s) {
    const unsigned grid = (unsigned)(a.BH * a.n_t);
    hipLaunchKernelGGL((kia_forward_kernel<D, CAL, REC, PROB, DUMP>), dim3(grid), dim3(kWave), 0, s, a);
    return hipGetLastError();
}

template <int D, int CAL>
static hipError_t launch_fwd_rec(const FwdConfig& c, const FwdArgs& a, hipStream_t s) {
    if (c.rec == REC_LERP)
        return c.dump ? launch_fwd_t<D, CAL, REC_LERP, false, true>(a, s)
                      : launch_fwd_t<D, CAL, REC_LERP, false, false>(a, s);
    if (c.prob)
        return c.dump ? launch_fwd_t<D, CAL, REC_NEAREST, true, true>(a, s)
                      : launch_fwd_t<D, CAL, REC_NEAREST, true, false>(a, s);
    return c.dump ? launch_fwd_t<D, CAL, REC_NEAREST, false, true>(a, s)
                  : launch_fwd_t<D, CAL, REC_NEAREST, false, false>(a, s);
}

template <int D>
static hipError_t launch_fwd_d(const FwdConfig& c, const FwdArgs& a, hipStream_t s) {
    return c.cal == CAL_MINMAX ? launch_fwd_rec<D, CAL_MINMAX>(c, a, s) : launch_fwd_rec<D, CAL_FWM>(c, a, s);
}

hipError_t launch_forward(const FwdConfig& c, const FwdArgs& a, hipStream_t s) {
    return c.d == 64 ? launch_fwd_d<64>(c, a, s) : launch_fwd_d<128>(c, a, s);
}

}  // namespace kia
