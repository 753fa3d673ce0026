// K-interval attention forward (gfx950).
//
// A workgroup (4 wavefronts) owns 128 queries of one (b, h) slice; each wave
// owns 32 of them.  Both calibrations need the final row extremes before any
// weight is known (MinMax: h from the span; FWM: the window anchored at the
// max), and a moving anchor shifts the interval phases, so weights cannot be
// rescaled on the fly as exact softmax can.  Hence two sweeps over the causal
// key tiles, with the tiles of K (sweep 1) and V (sweep 2) staged once per
// workgroup in LDS, double-buffered, the next tile's global loads in flight
// while the current one is used:
//   sweep 1: S^T = K Q^T on the fp32 matrix cores, scale 1/sqrt(d), causal
//            mask, running max/min with their key index; each wave stores its
//            score tiles once (query-major) for sweep 2 and the backward;
//   sweep 2: reload the wave's scores, reconstruct the weights on the grid,
//            sum W, accumulate O^T += V^T W^T on the matrix cores.
// Operator: "Pretraining Transformers with Quantized Softmax in Attention"
// (paperlayer digest), section 3 "Calibration" / "Reconstruction" and App. A.
#include "kia_common.hpp"
#include "kia_kernels.hpp"

namespace kia {

template <int D, int CAL, int REC, bool PROB, bool DUMP>
__global__ __launch_bounds__(kThreads, (D == 64 ? 2 : 1)) void kia_forward_kernel(FwdArgs a) {
    static_assert(D % 32 == 0, "head dim must be a multiple of 32");
    constexpr int NB = D / 32;  // 32-wide blocks of the head dim
    using ST = StreamTile<D>;
    constexpr int BUF = ST::kRM > ST::kTR ? ST::kRM : ST::kTR;
    __shared__ __attribute__((aligned(16))) float lds[2 * BUF];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int li = lane & 31, hl = lane >> 5;
    const int T = a.T, n_t = a.n_t;
    const int n_blk = (n_t + kBlockTiles - 1) / kBlockTiles;
    int bh, blk;
    map_block(blockIdx.x, a.BH, n_blk, true, bh, blk);
    const int qt = blk * kBlockTiles + wave;                   // this wave's query tile
    const bool active = qt < n_t;
    const int kt_end = min(blk * kBlockTiles + kBlockTiles - 1, n_t - 1);  // last key tile of the block
    const int qrow = qt * kTile + li;
    const bool qvalid = active && qrow < T;
    const size_t head = (size_t)bh * T * D;
    const float* Q = a.q + head;
    const float* Kp = a.k + head;
    const float* V = a.v + head;
    const int64_t tiles_per_head = (int64_t)n_t * (n_t + 1) / 2;
    float* tiles = a.tiles + ((size_t)bh * tiles_per_head + (active ? tile_index(qt, 0) : 0)) * kTileElems;

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
    ST st;
    st.load_rm(Kp, 0, T, tid);
    st.store_rm(lds, tid);
    __syncthreads();
    for (int kt = 0; kt <= kt_end; ++kt) {
        const float* cur = lds + (kt & 1) * BUF;
        if (kt < kt_end) st.load_rm(Kp, (kt + 1) * kTile, T, tid);
        if (active && kt <= qt) {
            const int k0 = kt * kTile;
            f32x16 acc = {};
#pragma unroll
            for (int p = 0; p < D / 8; ++p) {
                const f32x4 x = *(const f32x4*)(cur + rm_off<D>(li, 8 * p + 4 * hl));
#pragma unroll
                for (int j = 0; j < 4; ++j) acc = mfma32x32x2(x[j], qf[4 * p + j], acc);
            }
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
            for (int p = 0; p < 4; ++p)
                *(f32x4*)(tp + p * 256 + lane * 4) = f32x4{sv[4 * p], sv[4 * p + 1], sv[4 * p + 2], sv[4 * p + 3]};
        }
        if (kt < kt_end) st.store_rm(lds + ((kt + 1) & 1) * BUF, tid);
        __syncthreads();
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

    st.load_tr(V, 0, T, tid);
    st.store_tr(lds, tid);
    f32x4 snext[4];
    if (active) {
#pragma unroll
        for (int p = 0; p < 4; ++p) snext[p] = *(const f32x4*)(tiles + p * 256 + lane * 4);
    }
    __syncthreads();
    for (int kt = 0; kt <= kt_end; ++kt) {
        const float* cur = lds + (kt & 1) * BUF;
        if (kt < kt_end) st.load_tr(V, (kt + 1) * kTile, T, tid);
        if (active && kt <= qt) {
            const int k0 = kt * kTile;
            float sv[16];
#pragma unroll
            for (int p = 0; p < 4; ++p)
#pragma unroll
                for (int j = 0; j < 4; ++j) sv[4 * p + j] = snext[p][j];
            if (kt < qt) {
                const float* tp = tiles + (size_t)(kt + 1) * kTileElems;
#pragma unroll
                for (int p = 0; p < 4; ++p) snext[p] = *(const f32x4*)(tp + p * 256 + lane * 4);
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
                for (int p = 0; p < 4; ++p) {
                    const f32x4 x = *(const f32x4*)(cur + tr_off(32 * b + li, 8 * p + 4 * hl));
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        oacc[b] = mfma32x32x2(x[j], w[4 * p + j], oacc[b]);
                        if (PROB) olacc[b] = mfma32x32x2(x[j], wl[4 * p + j], olacc[b]);
                    }
                }
            }
        }
        if (kt < kt_end) st.store_tr(lds + ((kt + 1) & 1) * BUF, tid);
        __syncthreads();
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
            for (int p = 0; p < 4; ++p)
                *(f32x4*)(orow + 32 * b + 8 * p + 4 * hl) =
                    f32x4{oacc[b][4 * p] * invW, oacc[b][4 * p + 1] * invW, oacc[b][4 * p + 2] * invW,
                          oacc[b][4 * p + 3] * invW};
        if (PROB) {
            const float invWL = 1.f / WL;
            float* lrow = a.o_lerp + head + (size_t)qrow * D;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    *(f32x4*)(lrow + 32 * b + 8 * p + 4 * hl) =
                        f32x4{olacc[b][4 * p] * invWL, olacc[b][4 * p + 1] * invWL, olacc[b][4 * p + 2] * invWL,
                              olacc[b][4 * p + 3] * invWL};
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
    const int n_blk = (a.n_t + kBlockTiles - 1) / kBlockTiles;
    hipLaunchKernelGGL((kia_forward_kernel<D, CAL, REC, PROB, DUMP>), dim3((unsigned)(a.BH * n_blk)),
                       dim3(kThreads), 0, s, a);
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
