// K-interval attention backward (gfx950): two kernels in stream order.
//
//   rows  a workgroup (4 wavefronts) owns 128 queries of one (b, h) slice and
//         sweeps the causal key tiles, V and K^T staged in LDS per tile
//         (double-buffered).  Per tile: reload the forward's scores,
//         dP^T = V dO^T on the matrix cores, normalisation Jacobian at the
//         surrogate's evaluation point, direct score gradient, running
//         calibration sums, dQ^T += K^T dS^T; P and dS are written key-major
//         for the column kernel.  At the end of the row the calibration terms
//         are complete: they are added to dQ (gathering K at the argmax and
//         argmin keys) and folded into the wave's own dS tiles at (t, argmax)
//         and (t, argmin), so the column kernel's dK contraction carries them.
//   cols  a workgroup owns 128 keys and sweeps the query tiles at or below
//         the diagonal, dO^T and Q^T staged in LDS: dV^T += dO^T P and
//         dK^T += Q^T dS.
// No atomics: every output element has one writer and a fixed summation order.
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
//   max-only / min-only add one.  Degenerate rows: dS = P (dP - delta), no C;
//   a row with a single causal key has P = 1 identically and dS = 0.
#include <type_traits>

#include "kia_common.hpp"
#include "kia_kernels.hpp"

namespace kia {

template <int D, int CAL, int REC, bool PROB, bool TAB>
__global__ __launch_bounds__(kThreads, (D == 64 ? 2 : 1)) void kia_backward_rows_kernel(BwdArgs a) {
    constexpr int NB = D / 32;
    using LT = LdsTile<D>;
    constexpr int BUF = 2 * LT::kFloats;    // V tile, then K tile
    constexpr int XS = 36;                  // row stride of the per-wave transpose scratch
    __shared__ __attribute__((aligned(16))) float lds[2 * BUF];
    __shared__ __attribute__((aligned(16))) float xpose[kWaves * kTile * XS];
    __shared__ float gtab[TAB ? kWaves * kTabWaveFloats : 1];  // each wave's grid table

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // wave index is uniform
    const int li = lane & 31, hl = lane >> 5;
    const int T = a.T, n_t = a.n_t;
    const int n_blk = (n_t + kBlockTiles - 1) / kBlockTiles;
    int bh, blk;
    map_block(blockIdx.x, a.BH, n_blk, true, bh, blk);
    set_length_priority(blk + 1, n_blk);
    const int qt = blk * kBlockTiles + wave;
    const bool active = qt < n_t;
    const int kt_end = min(blk * kBlockTiles + kBlockTiles - 1, n_t - 1);
    const int qrow = qt * kTile + li;
    const bool qvalid = active && qrow < T;
    const size_t head = (size_t)bh * T * D;
    const float* Kp = a.k + head;
    const float* V = a.v + head;
    const int64_t tiles_per_head = (int64_t)n_t * (n_t + 1) / 2;
    const size_t tile0 = ((size_t)bh * tiles_per_head + (active ? tile_index(qt, 0) : 0)) * kTileElems;
    const float* stiles = a.tiles + tile0;
    float* ptiles = a.probs + tile0;
    float* dstiles = a.dscores + tile0;
    float* xw = xpose + wave * kTile * XS;
    float* gt = gtab + (TAB ? wave * kTabWaveFloats : 0);

    // The first V and K tiles go out first, so their loads overlap those of
    // the row's operands and statistics below.
    LT::load(lds, V, 0, T, tid);
    LT::load(lds + LT::kFloats, Kp, 0, T, tid);

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
    // causal key indices by construction; clamped so no stats value can address outside the row
    const int ka = min(max(qvalid ? a.row_a[ri] : 0, 0), max(qrow, 0));
    const int kb = min(max(qvalid ? a.row_b[ri] : 0, 0), max(qrow, 0));
    const RowGrid rg = make_row_grid(m, n, a.K, a.tau, CAL);
    const float invW = 1.f / W;
    // a row with a single causal key has P = 1 whatever its score: zero gradient
    const float invWe = (qrow == 0) ? 0.f : ((REC == REC_NEAREST && PROB) ? 1.f / WL : invW);
    // log2 of the row's 1/W, -inf for rows past the sequence end (their P and dS become 0)
    const float lw = qvalid ? __log2f(invW) : -INFINITY;
    const float nd = -dlt * invWe;               // G = (dP * invWe + nd) * g
    const float gW = invWe * W, ndW = nd * W;    // the same with g / W folded into gw
    // c/h is folded into the grid factor, so the loop forms dS = G c/h in one
    // product; the row sums are accumulated in units of dS and 1/coh restores
    // G's units after the loop
    const float lc = __log2f(rg.coh);            // log2(c/h)
    const float lwc = lw + lc;                   // log2(c/(h W))
    const float icoh = 1.f / rg.coh, cicoh = rg.c * icoh;
    const float iwc = fast_exp2(lw - lc);        // 1/(W c/h): Nearest's hard P from its table entry
    if (TAB) {
        // the row's grid factors for indices 0..K: g_i c/(h W) under LERP,
        // g_i c/h under Nearest; the two lane halves fill alternate entries
#pragma unroll
        for (int j = 0; j < (kTabEntries + 1) / 2; ++j) {
            const int i = 2 * j + hl;
            if (i <= a.K) gt[tab_off(i, li)] = fast_exp2(fmaf(-(float)i, rg.hl2, REC == REC_LERP ? lwc : lc));
        }
        wait_lgkm0();
        __builtin_amdgcn_wave_barrier();
    }

    // Row sums of the direct term (SA) and of dL/dw * Wd (SB = (c/h - 1) SBu + c SBf).
    // SA is summed per tile in fp32 (in key order, no contraction) and across
    // tiles with a compensated (hi, lo) pair; under the full and max-only
    // rules it leaves out the argmax key's own term, since the argmax entry's
    // final value is formed in the epilogue from the other keys' direct terms.
    // SB / K enters the two routed terms with opposite signs and cancels
    // exactly, so an fp32 running sum suffices for it.
    const bool use_max = !rg.degen && (a.rule == GRAD_FULL || a.rule == GRAD_MAX_ONLY);
    float SA = 0.f, SBu = 0.f, SBf = 0.f;
    float SAhi = 0.f, SAlo = 0.f;  // compensated running sum of the per-tile SA
    // this query's dS entries at the argmax and argmin keys as the loop stores
    // them, picked up from the transpose scratch of their tiles
    float olda = 0.f, oldb = 0.f;
    f32x16 dq[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) dq[b] = f32x16{};

    wait_vmcnt<0>();
    __syncthreads();

    float scur[16];
    for (int kt = 0; kt <= kt_end; ++kt) {
        const float* vcur = lds + (kt & 1) * BUF;
        const float* kcur = vcur + LT::kFloats;
        const bool work = active && kt <= qt;
        if (kt < kt_end) {
            float* nxt = lds + ((kt + 1) & 1) * BUF;
            LT::load(nxt, V, (kt + 1) * kTile, T, tid);
            LT::load(nxt + LT::kFloats, Kp, (kt + 1) * kTile, T, tid);
        }
        // the staging loads stay ahead of every later memory operation of the
        // step (the wait at its end counts the P / dS stores behind them)
        __builtin_amdgcn_sched_barrier(0);
        // this tile's scores straight into registers, after the staging loads;
        // they are first needed after the dP products
        f32x4 sx[4];
        if (work) {
#pragma unroll
            for (int p = 0; p < 4; ++p)
                sx[p] = __builtin_nontemporal_load((const f32x4*)(stiles + (size_t)kt * kTileElems + p * 256 + lane * 4));
        }
        if (work) {
            const int k0 = kt * kTile;
            f32x4 xv[D / 8];
#pragma unroll
            for (int p = 0; p < D / 8; ++p) xv[p] = *(const f32x4*)(vcur + LT::off(li, 8 * p + 4 * hl));
            // dP^T = V dO^T : A operand row = key
            f32x16 dp = {};
#pragma unroll
            for (int s2 = 0; s2 < D / 2; ++s2) dp = mfma32x32x2(xv[s2 >> 2][s2 & 3], dof[s2], dp);
            // K^T operands of the dQ product (column reads), read while the elementwise work runs
            float xk[16 * NB];
#pragma unroll
            for (int s2 = 0; s2 < 16 * NB; ++s2) xk[s2] = kcur[LT::off(acc_row(s2 & 15, hl), 32 * (s2 >> 4) + li)];
            // nothing that reads the scores moves above this point (their loads
            // may still be in flight during the products)
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int p = 0; p < 4; ++p)
#pragma unroll
                for (int j = 0; j < 4; ++j) scur[4 * p + j] = sx[p][j];

            float ds[16], pr[16];
            // key a's position in this tile relative to the lane half's first row
            // (no register index matches when key a lies elsewhere)
            const int da = (use_max && (ka >> 5) == kt) ? (ka & 31) - 4 * hl : -1;
            auto grads = [&](auto diag_t) {
                // no contraction: SA must sum exactly the rounded dS values that are
                // stored, or the routed calibration terms stop cancelling them
#pragma clang fp contract(off)
                constexpr bool DIAG = decltype(diag_t)::value;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + acc_row(r, hl);
                    const bool valid = DIAG ? key <= qrow : true;
                    const float s = scur[r];
                    if (softmax_rec(REC)) {
                        // exact-softmax reference: P = exp(s - m) / W, direct term
                        // (dP - delta) P W / W_e.  The rounded baselines keep that
                        // direct term (straight-through) and store the rounded P.
                        const float pw = fast_exp2(fmaf(s - rg.m, kLog2e, lw));
                        if (REC == REC_EXACT)
                            pr[r] = valid ? pw : 0.f;
                        else
                            pr[r] = (valid && qvalid) ? round_exp<REC>(fast_exp2((s - rg.m) * kLog2e)) * invW : 0.f;
                        ds[r] = valid ? fmaf(dp[r], gW, ndW) * pw : 0.f;
                        SA += (acc_row(r, 0) == da) ? 0.f : ds[r];
                        continue;
                    }
                    const float u = (rg.m - s) * rg.invh;
                    const bool keep = valid && ((CAL == CAL_FWM) ? (u <= rg.Kf) : true);
                    // the untruncated step continues the grid past K (no clamp)
                    const float fi = (CAL == CAL_FWM_UNTRUNC) ? floorf(u) : fminf(floorf(u), rg.Kf - 1.f);
                    const float f = u - fi;
                    // G = dL/dw times the LERP segment's grid value g_i; the direct
                    // term and the h-derivative share it
                    // dS = G c/h with G = dL/dw times the LERP segment's grid value
                    // g_i; the direct term and the h-derivative share it
                    float Gc, pw;
                    if (REC == REC_LERP) {
                        // gwc = g_i c/(h W) from one table entry or exponential;
                        // P = g_i (1 - f c) / W = gwc (1 - f c) h/c
                        const float gwc = TAB ? gt[tab_off((int)fi, li)] : fast_exp2(fmaf(-fi, rg.hl2, lwc));
                        pw = gwc * fmaf(-f, cicoh, icoh);
                        Gc = fmaf(dp[r], gW, ndW) * gwc;
                    } else {
                        const float rn = floorf(u + 0.5f);
                        float gc;
                        if constexpr (TAB) {
                            gc = gt[tab_off((int)fi, li)];
                            // the hard weight's grid point (past K only outside the FWM window)
                            pw = gt[tab_off((int)((CAL == CAL_FWM) ? fminf(rn, rg.Kf) : rn), li)] * iwc;
                        } else {
                            // the table's values and products exactly, so both
                            // paths store the same P
                            gc = fast_exp2(fmaf(-fi, rg.hl2, lc));
                            pw = fast_exp2(fmaf(-rn, rg.hl2, lc)) * iwc;
                        }
                        Gc = fmaf(dp[r], invWe, nd) * gc;
                    }
                    pr[r] = keep ? pw : 0.f;
                    ds[r] = keep ? Gc : 0.f;
                    // the argmax key's own direct term stays out of SA (adding 0
                    // changes no sum): SA is then the other keys' sum exactly
                    SA += (acc_row(r, 0) == da) ? 0.f : ds[r];
                    if (CAL == CAL_MINMAX) {
                        // dL/dw * Wd with Wd / g = (c/h - 1) u + c f (i + 1); only h = span/K
                        // needs it (in units of dS: divided by c/h after the loop)
                        const float Gk = ds[r];
                        SBu = fmaf(Gk, u, SBu);
                        SBf = fmaf(Gk, fmaf(f, fi, f), SBf);
                    }
                }
            };
            if (kt == qt) grads(std::true_type{});
            else grads(std::false_type{});

            // P and dS to key-major tiles through the wave's LDS scratch; the
            // column kernel reads them once, so the stores are non-temporal
            float* pp = ptiles + (size_t)kt * kTileElems;
            float* dd = dstiles + (size_t)kt * kTileElems;
#pragma unroll
            for (int r = 0; r < 16; ++r) xw[acc_row(r, hl) * XS + li] = pr[r];
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int p = 0; p < 4; ++p)
                __builtin_nontemporal_store(*(const f32x4*)(xw + li * XS + 8 * p + 4 * hl), (f32x4*)(pp + p * 256 + lane * 4));
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int r = 0; r < 16; ++r) xw[acc_row(r, hl) * XS + li] = ds[r];
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int p = 0; p < 4; ++p)
                __builtin_nontemporal_store(*(const f32x4*)(xw + li * XS + 8 * p + 4 * hl), (f32x4*)(dd + p * 256 + lane * 4));
            {
                // scratch row = key, column = query
                const float va = xw[(ka & 31) * XS + li], vb = xw[(kb & 31) * XS + li];
                olda = (kt == (ka >> 5)) ? va : olda;
                oldb = (kt == (kb >> 5)) ? vb : oldb;
            }
            __builtin_amdgcn_wave_barrier();

            // dQ^T += K^T dS^T : A operand row = head-dim index
#pragma unroll
            for (int s2 = 0; s2 < 16 * NB; ++s2) {
                const int b = s2 >> 4, kk = s2 & 15;
                dq[b] = mfma32x32x2(xk[s2], ds[kk], dq[b]);
            }
            {   // error-free addition of the tile's sum (Knuth's TwoSum)
                const float sum = SAhi + SA;
                const float bv = sum - SAhi;
                SAlo += (SAhi - (sum - bv)) + (SA - bv);
                SAhi = sum;
                SA = 0.f;
            }
        }
        // the staging loads were issued before the scores (already consumed) and
        // the P / dS stores (8), which may stay in flight
        if (work) wait_vmcnt<8>();
        else wait_vmcnt<0>();
        lds_barrier();
    }

    SBu += __shfl_xor(SBu, 32);
    SBf += __shfl_xor(SBf, 32);
    const float SB = (rg.cohm1 * SBu + rg.c * SBf) * icoh;
    const bool p1 = a.rule == GRAD_P1;
    const bool use_min = !rg.degen && CAL == CAL_MINMAX && (a.rule == GRAD_FULL || a.rule == GRAD_MIN_ONLY);

    // K rows a(t), b(t) and the P1 prefix row; entry i holds columns 8 i + 4 hl .. + 3.
    // Their loads go out first: the wait below covers them and the loop's last
    // dS stores (the argmax / argmin entries are rewritten after it).
    f32x4 ra[4 * NB], rb[4 * NB], rp[4 * NB];
#pragma unroll
    for (int i = 0; i < 4 * NB; ++i) {
        ra[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        rb[i] = ra[i];
        rp[i] = ra[i];
    }
    if (qvalid) {
#pragma unroll
        for (int i = 0; i < 4 * NB; ++i) {
            const int c = 8 * i + 4 * hl;
            ra[i] = *(const f32x4*)(Kp + (size_t)ka * D + c);
            rb[i] = *(const f32x4*)(Kp + (size_t)kb * D + c);
        }
        if (p1) {
#pragma unroll
            for (int i = 0; i < 4 * NB; ++i)
                rp[i] = *(const f32x4*)(a.prefix_k + head + (size_t)qrow * D + 8 * i + 4 * hl);
        }
    }
    float* ea = dstiles + (size_t)(ka >> 5) * kTileElems + kmajor_offset(li, ka & 31);
    float* eb = dstiles + (size_t)(kb >> 5) * kTileElems + kmajor_offset(li, kb & 31);

    // The argmax entry receives C_m = -SA + SB/K (MinMax) or -SA (FWM), so its
    // final value is minus the other keys' direct terms (plus SB/K).  Where P
    // is saturated the argmax's own direct term is the fp32 noise of
    // dP - delta, far above the row's true gradient, and adding C_m to it would
    // cancel that noise only to its rounding.  So the loop leaves that term
    // out of SA and the final value is formed from the other keys alone.
    const double sa_lane = (double)SAhi + (double)SAlo;
    const double sa_excl = sa_lane + __shfl_xor(sa_lane, 32);
    double sbk = 0.0;
    if (CAL == CAL_MINMAX) sbk = (double)(SB / rg.Kf);
    const float cn = use_min ? (float)(-sbk) : 0.f;

    // P1: the row mean of the detached gradient (0 for a single-key row)
    const float mu = p1 ? (float)(sa_excl / (double)(qrow + 1)) : 0.f;
    // every store of this wave (the loop's dS tiles included) has completed
    // before the argmax / argmin entries are rewritten
    wait_vmcnt<0>();
    if (qvalid) {
        float cm = 0.f;
        if (use_max) {
            // both lane halves hold the loop's direct term (olda); the first writes the final value
            const float fin = (float)(sbk - sa_excl);
            cm = fin - olda;  // the routed C_m, as applied on top of the loop's direct term
            if (hl == 0) *ea = fin;
        }
        float* dqrow = a.dq + head + (size_t)qrow * D;
#pragma unroll
        for (int i = 0; i < 4 * NB; ++i) {
            const int b = i >> 2, p = i & 3;
            f32x4 y;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                y[j] = (dq[b][4 * p + j] + cm * ra[i][j] + cn * rb[i][j] - mu * rp[i][j]) * a.scale;
            *(f32x4*)(dqrow + 8 * i + 4 * hl) = y;
        }
        if (hl == 0) {
            a.row_cm[ri] = p1 ? mu : cm;
            a.row_cn[ri] = cn;
            // argmax != argmin whenever C_n is routed (non-degenerate rows)
            if (cn != 0.f) *eb = oldb + cn;
        }
    }
}

template <int D>
__global__ __launch_bounds__(kThreads, (D == 64 ? 2 : 1)) void kia_backward_cols_kernel(BwdArgs a) {
    constexpr int NB = D / 32;
    using LT = LdsTile<D>;
    constexpr int BUF = 2 * LT::kFloats;  // dO tile, then Q tile
    constexpr int NSTAGE = 2 * (D / 32);  // direct LDS loads per wave for one staged dO + Q pair
    __shared__ __attribute__((aligned(16))) float lds[2 * BUF];
    __shared__ __attribute__((aligned(16))) float pdbuf[kWaves * 2 * kTileElems];  // each wave's next P, dS tiles

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // wave index is uniform
    const int li = lane & 31, hl = lane >> 5;
    const int T = a.T, n_t = a.n_t;
    const int n_blk = (n_t + kBlockTiles - 1) / kBlockTiles;
    int bh, blk;
    map_block(blockIdx.x, a.BH, n_blk, false, bh, blk);
    set_length_priority(n_blk - blk, n_blk);
    const int kt = blk * kBlockTiles + wave;
    const bool active = kt < n_t;
    const int qt_begin = blk * kBlockTiles;
    const int krow = kt * kTile + li;
    const size_t head = (size_t)bh * T * D;
    const float* Q = a.q + head;
    const float* dO = a.d_o + head;
    const int64_t tiles_per_head = (int64_t)n_t * (n_t + 1) / 2;
    const size_t hbase = (size_t)bh * tiles_per_head;

    f32x16 dv[NB], dk[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) { dv[b] = f32x16{}; dk[b] = f32x16{}; }

    float* pw = pdbuf + wave * 2 * kTileElems;
    float* dw = pw + kTileElems;
    LT::load(lds, dO, qt_begin * kTile, T, tid);
    LT::load(lds + LT::kFloats, Q, qt_begin * kTile, T, tid);
    auto dma_pd = [&](int qt_t) {
        const size_t toff = (hbase + tile_index(qt_t, kt)) * kTileElems;
        dma_tile(pw, a.probs + toff, lane);
        dma_tile(dw, a.dscores + toff, lane);
    };
    if (active) dma_pd(kt);
    wait_vmcnt<0>();
    __syncthreads();

    float pc[16], dc[16];
    for (int qt = qt_begin; qt < n_t; ++qt) {
        const float* ocur = lds + (qt & 1) * BUF;
        const float* qcur = ocur + LT::kFloats;
        if (qt + 1 < n_t) {
            float* nxt = lds + ((qt + 1) & 1) * BUF;
            LT::load(nxt, dO, (qt + 1) * kTile, T, tid);
            LT::load(nxt + LT::kFloats, Q, (qt + 1) * kTile, T, tid);
        }
        const bool work = active && qt >= kt;
        const bool prefetch = work && qt + 1 < n_t;
        if (work) {
            // this tile's P and dS: direct-loaded during the previous tile, before
            // this tile's staging loads
            if (qt + 1 < n_t) wait_vmcnt<NSTAGE>();
            else wait_vmcnt<0>();
            read_tile(pw, lane, pc);
            read_tile(dw, lane, dc);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                // dO^T and Q^T operands: lane = head-dim column, one float per query
                float xo[16], xq[16];
#pragma unroll
                for (int kk = 0; kk < 16; ++kk) {
                    xo[kk] = ocur[LT::off(acc_row(kk, hl), 32 * b + li)];
                    xq[kk] = qcur[LT::off(acc_row(kk, hl), 32 * b + li)];
                }
#pragma unroll
                for (int kk = 0; kk < 16; ++kk) {
                    dv[b] = mfma32x32x2(xo[kk], pc[kk], dv[b]);
                    dk[b] = mfma32x32x2(xq[kk], dc[kk], dk[b]);
                    if (b == 0 && kk == 0 && prefetch) {
                        // the next P / dS tiles reuse the slot once its reads are
                        // done; waiting here, behind the first products, costs
                        // less than waiting before them
                        __builtin_amdgcn_sched_barrier(0);
                        wait_lgkm0();
                        dma_pd(qt + 1);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
        }
        // the staging loads were issued first; the P / dS prefetch (8) may stay in flight
        if (prefetch) wait_vmcnt<8>();
        else wait_vmcnt<0>();
        lds_barrier();
    }
    if (active && krow < T) {
        float* dkrow = a.dk + head + (size_t)krow * D;
        float* dvrow = a.dv + head + (size_t)krow * D;
        // P1: the row means enter dK as -sum_{t >= j} mu_t Q_t (the dS tiles
        // hold the detached gradient)
        const bool p1 = a.rule == GRAD_P1;
        const float* sqrow = p1 ? a.suffix_q + head + (size_t)krow * D : nullptr;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int c = 32 * b + 8 * p + 4 * hl;
                f32x4 sq = {0.f, 0.f, 0.f, 0.f};
                if (p1) sq = *(const f32x4*)(sqrow + c);
                *(f32x4*)(dkrow + c) = f32x4{(dk[b][4 * p] - sq[0]) * a.scale, (dk[b][4 * p + 1] - sq[1]) * a.scale,
                                             (dk[b][4 * p + 2] - sq[2]) * a.scale, (dk[b][4 * p + 3] - sq[3]) * a.scale};
                *(f32x4*)(dvrow + c) = f32x4{dv[b][4 * p], dv[b][4 * p + 1], dv[b][4 * p + 2], dv[b][4 * p + 3]};
            }
    }
}

template <int D, int CAL, int REC, bool PROB, bool TAB = false>
static hipError_t launch_rows_t(const BwdArgs& a, hipStream_t s) {
    const int n_blk = (a.n_t + kBlockTiles - 1) / kBlockTiles;
    hipLaunchKernelGGL((kia_backward_rows_kernel<D, CAL, REC, PROB, TAB>), dim3((unsigned)(a.BH * n_blk)),
                       dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

// Grid operators: the table instantiation when the row's grid fits the table.
template <int D, int CAL, int REC, bool PROB>
static hipError_t launch_rows_grid(const FwdConfig& c, const BwdArgs& a, hipStream_t s) {
    if constexpr (tab_capable(CAL, REC)) {
        if (c.tab) return launch_rows_t<D, CAL, REC, PROB, true>(a, s);
    }
    return launch_rows_t<D, CAL, REC, PROB>(a, s);
}

template <int D, int CAL>
static hipError_t launch_rows_rec(const FwdConfig& c, const BwdArgs& a, hipStream_t s) {
    if (softmax_rec(c.rec)) {
        if constexpr (CAL == CAL_FWM) {
            if (c.rec == REC_EXACT) return launch_rows_t<D, CAL, REC_EXACT, false>(a, s);
            if (c.rec == REC_EXP_BF16) return launch_rows_t<D, CAL, REC_EXP_BF16, false>(a, s);
            return launch_rows_t<D, CAL, REC_EXP_FP8, false>(a, s);
        }
        return hipErrorInvalidValue;
    }
    if (c.rec == REC_LERP) return launch_rows_grid<D, CAL, REC_LERP, false>(c, a, s);
    return c.prob ? launch_rows_grid<D, CAL, REC_NEAREST, true>(c, a, s)
                  : launch_rows_grid<D, CAL, REC_NEAREST, false>(c, a, s);
}

template <int D>
static hipError_t launch_rows_d(const FwdConfig& c, const BwdArgs& a, hipStream_t s) {
    if (c.cal == CAL_MINMAX) return launch_rows_rec<D, CAL_MINMAX>(c, a, s);
    if (c.cal == CAL_FWM) return launch_rows_rec<D, CAL_FWM>(c, a, s);
    return launch_rows_rec<D, CAL_FWM_UNTRUNC>(c, a, s);
}

hipError_t launch_backward_rows(const FwdConfig& c, const BwdArgs& a, hipStream_t s) {
    return c.d == 64 ? launch_rows_d<64>(c, a, s) : launch_rows_d<128>(c, a, s);
}

hipError_t launch_backward_cols(int d, const BwdArgs& a, hipStream_t s) {
    const int n_blk = (a.n_t + kBlockTiles - 1) / kBlockTiles;
    const dim3 grid((unsigned)(a.BH * n_blk));
    if (d == 64)
        hipLaunchKernelGGL((kia_backward_cols_kernel<64>), grid, dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((kia_backward_cols_kernel<128>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

// ---- inspection: tile buffers to dense [BH, T, T] ---------------------------
__global__ __launch_bounds__(256) void kia_tiles_to_dense_kernel(int T, int n_t, const float* tiles,
                                                                 int key_major, float* dense) {
    const int bh = blockIdx.y;
    const int ti = blockIdx.x;
    int qt, kt;
    tile_coords(ti, qt, kt);
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
