// Score-geometry probe: per causal row, statistics of the scores the forward
// stored and of how far the operator's probabilities sit from the softmax of
// the same scores ("Pretraining Transformers with Quantized Softmax in
// Attention", section 4 "Geometry probe"; section 5.4; App. D.6).  It is a
// row reduction over the score tiles with no matrix products, bound by
// memory traffic and by its per-score instruction issue.
//
// Fields, each an fp32 array over the B*H*T rows: span (max - min), native
// width h (the operator's interval width: MinMax span/K, 0 on degenerate
// rows; FWM and the untruncated step tau/K; the exact reference and its
// rounded-exponential baselines report the MinMax width), |Q_t|, |K_t|, entropy of P, entropy of the softmax (nats),
// total variation (1/2) sum |P - softmax|, and the softmax mass of the top
// rounding bucket (keys whose Nearest point on that grid is 0).
#include <type_traits>

#include "kia_common.hpp"
#include "kia_kernels.hpp"

namespace kia {

namespace {

constexpr int kGeoFields = 8;

// One workgroup of eight wavefronts per 32-row query tile; wave w takes the
// key tiles kt = w, w+8, ..., two at a time.  Lane l owns query l%32; of every
// 32-key tile it holds the 16 keys 8p + 4*(l/32) + j (p, j < 4), which the
// query-major storage lays out as four float4 loads of one contiguous kilobyte
// per wave.  The two lanes of a row combine with one exchange, the waves
// through LDS.  Blocks run the longest rows first, across all heads.
//
// Pass B needs the softmax normaliser Z of the whole row, so the tiles are
// read twice, and the second read is arranged to hit L2 where it can: eight
// waves per row block halve a block's lifetime (and so the tiles it holds in
// L2), pass B walks each wave's tiles in the reverse order of pass A, starting
// with the ones pass A read last, and its loads, each tile's last use, carry
// the non-temporal policy so they do not evict tiles other blocks still
// re-read.
constexpr int kGeoWaves = 8;

// u < this value exactly when floor(u + 1/2) == 0 in fp32, for u >= 0: the
// largest float below 1/2 plus 1/2 rounds (to even) up to 1
constexpr float kTopU = 0x1.fffffep-2f;

template <int CAL, int REC>
__global__ __launch_bounds__(kGeoWaves * kWave) void kia_geometry_kernel(GeoArgs a) {
    // the weights below repeat the forward's arithmetic operation for
    // operation, so P here is the forward's P bit for bit
#pragma clang fp contract(off)
    __shared__ float s_mn[kGeoWaves][kTile];
    __shared__ double s_sum[4][kGeoWaves][kTile];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int qi = lane & 31, hl = lane >> 5;
    const int bh = (int)(blockIdx.x % (unsigned)a.BH);
    const int qt = a.n_t - 1 - (int)(blockIdx.x / (unsigned)a.BH);
    const int qrow = qt * kTile + qi;
    const bool qvalid = qrow < a.T;
    const size_t row = (size_t)bh * a.T + (qvalid ? qrow : 0);
    const int64_t tiles_per_head = (int64_t)a.n_t * (a.n_t + 1) / 2;
    const float* tiles = a.tiles + ((size_t)bh * tiles_per_head + tile_index(qt, 0)) * kTileElems;
    auto load_tile = [&](int kt, f32x4* x) {
        const float* tp = tiles + (size_t)kt * kTileElems;
#pragma unroll
        for (int p = 0; p < 4; ++p) x[p] = *(const f32x4*)(tp + p * 256 + lane * 4);
    };
    // pass B's reads are each tile's last use
    auto load_tile_last = [&](int kt, f32x4* x) {
        const float* tp = tiles + (size_t)kt * kTileElems;
#pragma unroll
        for (int p = 0; p < 4; ++p) x[p] = __builtin_nontemporal_load((const f32x4*)(tp + p * 256 + lane * 4));
    };
    // reduction of per-wave row partials in a fixed order
    auto wave_sum = [&](int f) {
        double r = 0.0;
#pragma unroll
        for (int w = 0; w < kGeoWaves; ++w) r += s_sum[f][w][qi];
        return r;
    };

    // pass A: row min and the softmax normaliser Z (the max comes from the
    // forward's row statistics)
    const float m = qvalid ? a.row_m[row] : 0.f;
    float mn = INFINITY;
    double Z = 0.0;
    // below the diagonal every key of the tile is causal for every row (rows
    // past T compute values nobody reads); only the diagonal tile is masked
    auto pass_a = [&](int kt, const f32x4* x, auto diag_t) {
        constexpr bool DIAG = decltype(diag_t)::value;
        float Zt = 0.f;
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int key = kt * kTile + 8 * p + 4 * hl + j;
                if (!DIAG || key <= qrow) {
                    mn = fminf(mn, x[p][j]);
                    Zt += fast_exp2((x[p][j] - m) * kLog2e);
                }
            }
        Z += (double)Zt;
    };
    auto run_a = [&](int kt, const f32x4* x) {
        if (kt < qt) pass_a(kt, x, std::false_type{});
        else pass_a(kt, x, std::true_type{});
    };
    for (int kt = wv; kt <= qt; kt += 2 * kGeoWaves) {
        const int kt2 = kt + kGeoWaves;
        f32x4 x[4], y[4];
        load_tile(kt, x);
        if (kt2 <= qt) load_tile(kt2, y);
        run_a(kt, x);
        if (kt2 <= qt) run_a(kt2, y);
    }
    mn = fminf(mn, __shfl_xor(mn, 32));
    Z += __shfl_xor(Z, 32);
    if (hl == 0) {
        s_mn[wv][qi] = mn;
        s_sum[0][wv][qi] = Z;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kGeoWaves; ++w) mn = fminf(mn, s_mn[w][qi]);
    Z = wave_sum(0);
    __syncthreads();

    // the operator's grid; the exact reference lays a MinMax grid for the
    // reported width and the top bucket
    constexpr int GCAL = softmax_rec(REC) ? CAL_MINMAX : CAL;
    const RowGrid rg = make_row_grid(m, mn, a.K, a.tau, GCAL == CAL_MINMAX ? CAL_MINMAX : CAL_FWM);
    const float W = qvalid ? a.row_w[row] : 1.f;
    const float invW = 1.f / W;
    const float invZ = (float)(1.0 / Z);

    // pass B: total variation needs Z per key; the entropies and the top mass
    // are accumulated as sums divided by W or Z at the end:
    //   H(P) = ln W - (1/W) sum w ln w,  H(q) = ln Z - (1/Z) sum e (s - m),
    //   top = (1/Z) sum over the top bucket of e
    // (sum w = W up to rounding: the forward's W sums these same weights)
    double tv = 0.0, wlw = 0.0, es = 0.0, etop = 0.0;
    auto pass_b = [&](int kt, const f32x4* x, auto diag_t) {
        constexpr bool DIAG = decltype(diag_t)::value;
        float tvt = 0.f, wlwt = 0.f, est = 0.f, etopt = 0.f;
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int key = kt * kTile + 8 * p + 4 * hl + j;
                if (DIAG && key > qrow) continue;
                const float s = x[p][j];
                const float sm = s - m;
                const float xe = sm * kLog2e;
                const float e = fast_exp2(xe);
                const float u = (rg.m - s) * rg.invh;
                // w and w ln w; where w = exp2(x), ln w = x ln 2
                float w, wl;
                if (REC == REC_EXACT) {
                    w = e;
                    wl = e * (xe * kLn2);
                } else if (softmax_rec(REC)) {
                    w = round_exp<REC>(e);
                    wl = w > 0.f ? w * __logf(w) : 0.f;
                } else if (REC == REC_NEAREST) {
                    const float xr = -floorf(u + 0.5f) * rg.hl2;
                    const bool keep = (CAL == CAL_FWM) ? (u <= rg.Kf) : true;
                    w = keep ? fast_exp2(xr) : 0.f;
                    wl = w > 0.f ? w * (xr * kLn2) : 0.f;
                } else {
                    const bool keep = (CAL == CAL_FWM) ? (u <= rg.Kf) : true;
                    const float fi = floorf(u);
                    const float g = fast_exp2(-fi * rg.hl2);
                    w = keep ? g * fmaf(fi - u, rg.c, 1.f) : 0.f;
                    wl = w > 0.f ? w * __logf(w) : 0.f;
                }
                tvt += fabsf(w * invW - e * invZ);
                wlwt += wl;
                est = fmaf(e, sm, est);
                etopt += (u < kTopU) ? e : 0.f;
            }
        tv += (double)tvt;
        wlw += (double)wlwt;
        es += (double)est;
        etop += (double)etopt;
    };
    auto run_b = [&](int kt, const f32x4* x) {
        if (kt < qt) pass_b(kt, x, std::false_type{});
        else pass_b(kt, x, std::true_type{});
    };
    if (wv <= qt) {
        // the pairs of pass A, last pair first, the later tile of a pair first
        for (int kt = wv + ((qt - wv) / (2 * kGeoWaves)) * (2 * kGeoWaves); kt >= wv; kt -= 2 * kGeoWaves) {
            const int kt2 = kt + kGeoWaves;
            f32x4 x[4], y[4];
            if (kt2 <= qt) load_tile_last(kt2, y);
            load_tile_last(kt, x);
            if (kt2 <= qt) run_b(kt2, y);
            run_b(kt, x);
        }
    }
    tv += __shfl_xor(tv, 32);
    wlw += __shfl_xor(wlw, 32);
    es += __shfl_xor(es, 32);
    etop += __shfl_xor(etop, 32);
    if (hl == 0) {
        s_sum[0][wv][qi] = tv;
        s_sum[1][wv][qi] = wlw;
        s_sum[2][wv][qi] = es;
        s_sum[3][wv][qi] = etop;
    }
    __syncthreads();
    if (!qvalid) return;
    const size_t n_rows = (size_t)a.BH * a.T;
    float* g = a.geo + row;
    if (wv == 0 && hl == 0) {
        const double r_tv = wave_sum(0), r_wlw = wave_sum(1), r_es = wave_sum(2), r_top = wave_sum(3);
        const float span = m - mn;
        float h;
        if (GCAL == CAL_MINMAX) {
            h = rg.degen ? 0.f : span / (float)a.K;
        } else {
            h = a.tau / (float)a.K;
        }
        g[0] = span;
        g[1 * n_rows] = h;
        g[4 * n_rows] = (float)(log((double)W) - r_wlw / (double)W);
        g[5 * n_rows] = (float)(log(Z) - r_es / Z);
        g[6 * n_rows] = (float)(0.5 * r_tv);
        g[7 * n_rows] = (float)(r_top / Z);
    } else if (wv == 1) {
        // norms of the unscaled projections at this position: Q on the lower
        // half-wave, K on the upper
        const float* src = (hl == 0 ? a.q : a.k) + row * (size_t)a.d;
        double nrm = 0.0;
        for (int c = 0; c < a.d; c += 4) {
            const f32x4 x = *(const f32x4*)(src + c);
            float part = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) part = fmaf(x[j], x[j], part);
            nrm += (double)part;
        }
        g[(hl == 0 ? 2 : 3) * n_rows] = (float)sqrt(nrm);
    }
}

template <int CAL, int REC>
hipError_t launch_geo_t(const GeoArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((kia_geometry_kernel<CAL, REC>), dim3((unsigned)(a.BH * a.n_t)), dim3(kGeoWaves * kWave), 0,
                       s, a);
    return hipGetLastError();
}

template <int CAL>
hipError_t launch_geo_rec(int rec, const GeoArgs& a, hipStream_t s) {
    return rec == REC_NEAREST ? launch_geo_t<CAL, REC_NEAREST>(a, s) : launch_geo_t<CAL, REC_LERP>(a, s);
}

}  // namespace

hipError_t launch_geometry(int cal, int rec, const GeoArgs& a, hipStream_t s) {
    static_assert(kGeoFields == 8, "field count");
    if (rec == REC_EXACT) return launch_geo_t<CAL_MINMAX, REC_EXACT>(a, s);
    if (rec == REC_EXP_BF16) return launch_geo_t<CAL_MINMAX, REC_EXP_BF16>(a, s);
    if (rec == REC_EXP_FP8) return launch_geo_t<CAL_MINMAX, REC_EXP_FP8>(a, s);
    if (cal == CAL_MINMAX) return launch_geo_rec<CAL_MINMAX>(rec, a, s);
    if (cal == CAL_FWM) return launch_geo_rec<CAL_FWM>(rec, a, s);
    return launch_geo_rec<CAL_FWM_UNTRUNC>(rec, a, s);
}

}  // namespace kia
