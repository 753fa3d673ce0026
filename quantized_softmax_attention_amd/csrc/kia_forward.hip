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
#include <type_traits>

#include "kia_common.hpp"
#include "kia_kernels.hpp"

namespace kia {

// Sweep 2 order.  SER: each tile is reconstructed right before its own
// products, with one set of weights, and the other workgroup on the CU fills
// the matrix cores meanwhile.  Otherwise (d = 64 without the Prob-STE extras,
// rows of at most kPipeMaxTiles tiles) tile kt+1 is reconstructed while the
// products of tile kt run, interleaved instruction by instruction.  The
// serial order needs fewer registers (two workgroups per CU also at d = 128,
// and with the Prob-STE extras at d = 64) and was measured faster on long
// rows; the interleaved one on the GPT-2-shaped rows of 1024 keys.
constexpr int kPipeMaxTiles = 32;

template <int D, int CAL, int REC, bool PROB, bool DUMP, bool SER>
__global__ __launch_bounds__(kThreads, (D == 128 && PROB) ? 1 : 2) void kia_forward_kernel(FwdArgs a) {
    static_assert(D % 32 == 0, "head dim must be a multiple of 32");
    static_assert(SER || (D == 64 && !PROB), "the interleaved order exists for d = 64 without Prob-STE only");
    constexpr int NB = D / 32;  // 32-wide blocks of the head dim
    constexpr bool PIPE = !SER;
    using LT = LdsTile<D>;
    constexpr int BUF = LT::kFloats;
    // K (sweep 1) / V (sweep 2) tiles, double-buffered.  The two buffers are
    // separate arrays and every access names its array statically (loops are
    // unrolled by two), so the compiler can tell a direct load into one buffer
    // from reads of the other and inserts no wait of its own between them.
    __shared__ __attribute__((aligned(16))) float lds0[BUF];
    __shared__ __attribute__((aligned(16))) float lds1[BUF];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // wave index is uniform
    const int li = lane & 31, hl = lane >> 5;
    const int T = a.T, n_t = a.n_t;
    const int n_blk = (n_t + kBlockTiles - 1) / kBlockTiles;
    int bh, blk;
    map_block(blockIdx.x, a.BH, n_blk, true, bh, blk);
    set_length_priority(blk + 1, n_blk);
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

    // B operand of S^T = K Q^T: lane holds Q[qrow][c] / sqrt(d) for c = 8p + 4*hl + j.
    float qf[D / 2];
#pragma unroll
    for (int p = 0; p < D / 8; ++p) {
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (qvalid) x = *(const f32x4*)(Q + (size_t)qrow * D + 8 * p + 4 * hl);
#pragma unroll
        for (int j = 0; j < 4; ++j) qf[4 * p + j] = x[j] * a.scale;
    }

    // ---- sweep 1: scores, row extremes --------------------------------------
    // K tiles arrive by direct global -> LDS loads one tile ahead.  Per wave
    // the matrix instructions of key tile kt interleave with the store and the
    // extreme tracking of tile kt-1.  Tracking is per tile: each lane keeps its
    // running max / min and the first tile where a strictly larger (smaller)
    // value appeared; the key index inside that tile is looked up once at the
    // end, so the lowest index among equal extremes is kept.  Only a wave's
    // last tile (the diagonal) needs the causal mask; lanes past the end of the
    // sequence compute values never stored as results.
    float m = -INFINITY, n = INFINITY;
    int amt = 0, ant = 0;  // tile of the first occurrence of this lane's extremes
    int am = 0, an = 0;    // row argmax / argmin (lowest key index)
    auto store_tile = [&](const f32x16& acc, int kt_t, bool diag) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            f32x4 x;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool ok = !diag || (kt_t * kTile + acc_row(4 * p + j, hl)) <= qrow;
                x[j] = ok ? acc[4 * p + j] : 0.f;
            }
            *(f32x4*)(tiles + (size_t)kt_t * kTileElems + p * 256 + lane * 4) = x;
        }
    };
    // Each lane keeps its 16 scores of the tile where its running max (min)
    // first appeared (NaN until a tile sets them), so the key index inside that
    // tile is found without reading the tile back (a read-back fetches a cache
    // line per lane for 16 bytes of it).  The interleaved sweep order keeps
    // them in registers (selects on every tile); the serial order, whose
    // registers go to d = 128 or the Prob-STE extras, in a per-wave LDS stash
    // written only when the extreme improves ([extreme][p][lane][4]: the b128
    // accesses of a wave are conflict-free).
    float bx[PIPE ? 16 : 1], by[(PIPE && CAL == CAL_MINMAX) ? 16 : 1];
    __shared__ __attribute__((aligned(16))) float stash[PIPE ? 1 : kWaves * 2 * kTileElems];
    float* const stw = stash + (PIPE ? 0 : wave * 2 * kTileElems);
    {
        const float q = __builtin_nanf("");
        if constexpr (PIPE) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                bx[r] = q;
                if (CAL == CAL_MINMAX) by[r] = q;
            }
        } else {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                *(f32x4*)(stw + p * 256 + lane * 4) = f32x4{q, q, q, q};
                if (CAL == CAL_MINMAX) *(f32x4*)(stw + kTileElems + p * 256 + lane * 4) = f32x4{q, q, q, q};
            }
        }
    }
    auto track_tile = [&](const f32x16& acc, int kt_t, bool diag) {
        float x[16], y[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const bool ok = !diag || (kt_t * kTile + acc_row(r, hl)) <= qrow;
            x[r] = ok ? acc[r] : -INFINITY;
            y[r] = ok ? acc[r] : INFINITY;
        }
        float mt = x[0], nt = y[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) {
            mt = fmaxf(mt, x[r]);
            if (CAL == CAL_MINMAX) nt = fminf(nt, y[r]);
        }
        const bool up = mt > m;
        amt = up ? kt_t : amt;
        m = up ? mt : m;
        if constexpr (PIPE) {
#pragma unroll
            for (int r = 0; r < 16; ++r) bx[r] = up ? x[r] : bx[r];
        } else if (up) {
#pragma unroll
            for (int p = 0; p < 4; ++p)
                *(f32x4*)(stw + p * 256 + lane * 4) = f32x4{x[4 * p], x[4 * p + 1], x[4 * p + 2], x[4 * p + 3]};
        }
        if (CAL == CAL_MINMAX) {
            const bool dn = nt < n;
            ant = dn ? kt_t : ant;
            n = dn ? nt : n;
            if constexpr (PIPE) {
#pragma unroll
                for (int r = 0; r < 16; ++r) by[r] = dn ? y[r] : by[r];
            } else if (dn) {
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    *(f32x4*)(stw + kTileElems + p * 256 + lane * 4) =
                        f32x4{y[4 * p], y[4 * p + 1], y[4 * p + 2], y[4 * p + 3]};
            }
        }
    };
    LT::load(lds0, Kp, 0, T, tid);
    wait_vmcnt<0>();
    __syncthreads();
    f32x16 accA = {}, accB = {};
    // key tile kt: MFMAs into acc, store + track the previous tile held in prv
    auto sweep1 = [&](int kt, const float* cur, float* nxt, f32x16& acc, const f32x16& prv)
        __attribute__((always_inline)) {
        if (kt < kt_end) LT::load(nxt, Kp, (kt + 1) * kTile, T, tid);
        // the staging loads stay ahead of every later memory operation of the
        // step: the wait at its end counts only the score stores behind them
        __builtin_amdgcn_sched_barrier(0);
        const bool stores = active && kt <= qt && kt > 0;
        if (active && kt <= qt) {
            f32x4 xk[D / 8];
#pragma unroll
            for (int p = 0; p < D / 8; ++p) xk[p] = *(const f32x4*)(cur + LT::off(li, 8 * p + 4 * hl));
            acc = f32x16{};
            if (kt > 0) {
                store_tile(prv, kt - 1, false);
                track_tile(prv, kt - 1, false);
            }
#pragma unroll
            for (int s = 0; s < D / 2; ++s) acc = mfma32x32x2(xk[s >> 2][s & 3], qf[s], acc);
            // two vector instructions per product where the tracking keeps its
            // tile copies in registers (about 60 per step), one otherwise
            if (kt > 0) pin_interleave<D / 2, PIPE ? 2 : 1, D / 8>();
        }
        // the K tile loads were issued first; the 4 score stores may stay in flight
        if (stores) wait_vmcnt<4>();
        else wait_vmcnt<0>();
        lds_barrier();
    };
    for (int kt = 0; kt <= kt_end; kt += 2) {
        sweep1(kt, lds0, lds1, accA, accB);
        if (kt + 1 <= kt_end) sweep1(kt + 1, lds1, lds0, accB, accA);
    }
    if (active) {
        // the diagonal tile qt sits in accA for even qt, accB for odd
        if (qt & 1) { store_tile(accB, qt, true); track_tile(accB, qt, true); }
        else { store_tile(accA, qt, true); track_tile(accA, qt, true); }
    }
    // Sweep 2's first V tile and this wave's first score tiles need no row
    // statistic: their loads go out here, ahead of the extremes' key search
    // below.
    float sv[16];
    f32x4 sx[4];
    LT::load(lds0, V, 0, T, tid);
    if (active) {
        if (PIPE) {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const f32x4 x = *(const f32x4*)(tiles + p * 256 + lane * 4);
#pragma unroll
                for (int j = 0; j < 4; ++j) sv[4 * p + j] = x[j];
            }
            if (qt > 0) {
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    sx[p] = __builtin_nontemporal_load((const f32x4*)(tiles + kTileElems + p * 256 + lane * 4));
            }
        } else {
#pragma unroll
            for (int p = 0; p < 4; ++p)
                sx[p] = __builtin_nontemporal_load((const f32x4*)(tiles + p * 256 + lane * 4));
        }
    }
    // Row extremes: the two lane halves of a query saw disjoint keys.  Each
    // half whose extreme equals the row's takes the first key attaining it
    // among its 16 kept scores of the tile where that extreme first appeared;
    // the smaller key of the two halves wins.  Masked diagonal entries hold
    // -inf / +inf there and are excluded by the causal test as well.
    {
        const float M = fmaxf(m, __shfl_xor(m, 32));
        const float N = (CAL == CAL_MINMAX) ? fminf(n, __shfl_xor(n, 32)) : 0.f;
        int ia = 0x7fffffff, ib = 0x7fffffff;
        if (active) {
            float xa[16], xb[16];
            if constexpr (PIPE) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    xa[r] = bx[r];
                    xb[r] = (CAL == CAL_MINMAX) ? by[r] : 0.f;
                }
            } else {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const f32x4 x = *(const f32x4*)(stw + p * 256 + lane * 4);
                    f32x4 y = {0.f, 0.f, 0.f, 0.f};
                    if (CAL == CAL_MINMAX) y = *(const f32x4*)(stw + kTileElems + p * 256 + lane * 4);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        xa[4 * p + j] = x[j];
                        xb[4 * p + j] = y[j];
                    }
                }
            }
#pragma unroll
            for (int r = 15; r >= 0; --r) {
                const int ka = amt * kTile + acc_row(r, hl);
                if (m == M && ka <= qrow && xa[r] == M) ia = ka;
                if (CAL == CAL_MINMAX) {
                    const int kb = ant * kTile + acc_row(r, hl);
                    if (n == N && kb <= qrow && xb[r] == N) ib = kb;
                }
            }
        }
        // a row with no finite extreme (NaN scores) finds no key: fall back to key 0
        m = M;
        am = min(ia, __shfl_xor(ia, 32));
        if (am == 0x7fffffff) am = 0;
        if (CAL == CAL_MINMAX) {
            n = N;
            an = min(ib, __shfl_xor(ib, 32));
            if (an == 0x7fffffff) an = 0;
        }
    }
    if (!qvalid) { m = 0.f; n = 0.f; }
    const RowGrid rg = make_row_grid(m, n, a.K, a.tau, CAL);

    // ---- sweep 2: reconstruct, normalise, O = W V / sum(W) -----------------
    // V tiles arrive like the K tiles; each wave's next score tile arrives by a
    // direct load into its LDS slot.  Per wave the matrix instructions of
    // tile kt (weights already computed) interleave with the reconstruction of
    // tile kt+1; the two unrolled halves swap weight registers.
    // Normalisers: each tile's 16 weights are summed in fp32, the tile sums in
    // fp64, so the rounding error stays at ~16 ulp of W for rows of any length.
    float Wt = 0.f, WLt = 0.f;
    double W64 = 0.0, WL64 = 0.0;
    auto flush_sums = [&]() {
        W64 += (double)Wt;
        Wt = 0.f;
        if (REC == REC_NEAREST) {
            WL64 += (double)WLt;
            WLt = 0.f;
        }
    };
    f32x16 oacc[NB];
    f32x16 olacc[PROB ? NB : 1];
#pragma unroll
    for (int b = 0; b < NB; ++b) oacc[b] = f32x16{};
#pragma unroll
    for (int b = 0; b < (PROB ? NB : 1); ++b) olacc[b] = f32x16{};

    float wA[16], wlA[PROB ? 16 : 1], wB[16], wlB[PROB ? 16 : 1];
    auto recon = [&](int kt_t, auto diag_t, int r, float* w, float* wl) {
        // no contraction: every instantiation (with or without the Prob-STE
        // extras) rounds the weights and their sums identically
#pragma clang fp contract(off)
        constexpr bool DIAG = decltype(diag_t)::value;
        const int key = kt_t * kTile + acc_row(r, hl);
        const bool valid = DIAG ? key <= qrow : true;
        const float s = sv[r];
        if (softmax_rec(REC)) {
            // exact-softmax reference w = exp(s - m), or its rounded baselines
            const float we = round_exp<REC>(fast_exp2((s - rg.m) * kLog2e));
            w[r] = valid ? we : 0.f;
            Wt += w[r];
            // the dump records the rounded value's fp32 bits (0 for the exact reference)
            if (DUMP && qvalid && valid)
                a.idx_dump[((size_t)bh * T + qrow) * T + key] = (REC == REC_EXACT) ? 0 : __float_as_int(we);
            return;
        }
        const float u = (rg.m - s) * rg.invh;
        const bool keep = valid && ((CAL == CAL_FWM) ? (u <= rg.Kf) : true);
        // unclamped segment: at u = K (the row min) the LERP value is g_K either
        // way, and the untruncated step continues the grid past K
        const float fi = floorf(u);
        const float g = fast_exp2(-fi * rg.hl2);
        const float wlv = g * fmaf(fi - u, rg.c, 1.f);
        float wv = wlv;
        if (REC == REC_NEAREST) wv = fast_exp2(-floorf(u + 0.5f) * rg.hl2);
        w[r] = keep ? wv : 0.f;
        Wt += w[r];
        if (REC == REC_NEAREST) WLt += keep ? wlv : 0.f;
        if (PROB) wl[r] = keep ? wlv : 0.f;
        if (DUMP && qvalid && valid) {
            int idx = (REC == REC_LERP) ? (CAL == CAL_FWM_UNTRUNC ? (int)fi : (int)fminf(fi, rg.Kf - 1.f))
                                        : (int)floorf(u + 0.5f);
            if (!keep) idx = -1;
            a.idx_dump[((size_t)bh * T + qrow) * T + key] = idx;
        }
    };

    // Score tiles go straight into registers, loaded one tile ahead of their
    // reconstruction (sx), which itself runs one tile ahead of the products
    // when PIPE.
    if (PIPE && active) {
        if (qt == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) recon(0, std::true_type{}, r, wA, wlA);
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) recon(0, std::false_type{}, r, wA, wlA);
        }
        flush_sums();
    }
    wait_vmcnt<0>();
    __syncthreads();
    // V^T operand: lane = head-dim column, one float per key (column reads)
    auto v_operand = [&](const float* cur, float* xv) __attribute__((always_inline)) {
#pragma unroll
        for (int s2 = 0; s2 < 16 * NB; ++s2) xv[s2] = cur[LT::off(acc_row(s2 & 15, hl), 32 * (s2 >> 4) + li)];
    };
    // tile kt: weights in (w, wl); reconstruct tile kt+1 into (wn, wln)
    auto sweep2 = [&](int kt, const float* cur, float* nxt, const float* w, const float* wl, float* wn, float* wln)
        __attribute__((always_inline)) {
        const bool more = active && kt + 1 <= qt;      // tile kt+1 exists for this wave
        const bool prefetch = active && kt + 2 <= qt;  // and tile kt+2
        if (more) {
            // scores of tile kt+1, loaded during the previous tile: the only
            // vector memory operations of this wave still outstanding here
            wait_vmcnt<0>();
#pragma unroll
            for (int p = 0; p < 4; ++p)
#pragma unroll
                for (int j = 0; j < 4; ++j) sv[4 * p + j] = sx[p][j];
        }
        if (kt < kt_end) LT::load(nxt, V, (kt + 1) * kTile, T, tid);
        // the staging loads stay ahead of the score loads: the wait at the end
        // of the step leaves only those 4 in flight
        __builtin_amdgcn_sched_barrier(0);
        if (prefetch) {
#pragma unroll
            for (int p = 0; p < 4; ++p)
                sx[p] = __builtin_nontemporal_load(
                    (const f32x4*)(tiles + (size_t)(kt + 2) * kTileElems + p * 256 + lane * 4));
        }
        // the score loads are issued here, ahead of this tile's work
        __builtin_amdgcn_sched_barrier(0);
        if (active && kt <= qt) {
            float xv[16 * NB];
            v_operand(cur, xv);
            auto mstep = [&](int s) {
                const int b = s >> 4, kk = s & 15;
                oacc[b] = mfma32x32x2(xv[s], w[kk], oacc[b]);
                if (PROB) olacc[b] = mfma32x32x2(xv[s], wl[kk], olacc[b]);
            };
            if (kt + 1 < qt) {
                interleave<16 * NB, 16>(mstep, [&](int r) { recon(kt + 1, std::false_type{}, r, wn, wln); });
                pin_interleave<16 * NB, (PROB ? 4 : 5) * 2 / NB, 16 * NB>();
            } else if (kt + 1 == qt) {
                interleave<16 * NB, 16>(mstep, [&](int r) { recon(kt + 1, std::true_type{}, r, wn, wln); });
                pin_interleave<16 * NB, (PROB ? 4 : 5) * 2 / NB, 16 * NB>();
            } else {
#pragma unroll
                for (int s = 0; s < 16 * NB; ++s) mstep(s);
            }
        }
        flush_sums();
        // the V tile loads were issued before the 4 score loads, which may stay in flight
        if (prefetch) wait_vmcnt<4>();
        else wait_vmcnt<0>();
        lds_barrier();
    };
    // tile kt reconstructed into (wA, wlA), then its products
    auto sweep2_serial = [&](int kt, const float* cur, float* nxt) __attribute__((always_inline)) {
        const bool here = active && kt <= qt;
        const bool prefetch = active && kt + 1 <= qt;
        if (here) {
            // scores of tile kt, loaded during the previous tile: the only
            // vector memory operations of this wave still outstanding here
            wait_vmcnt<0>();
#pragma unroll
            for (int p = 0; p < 4; ++p)
#pragma unroll
                for (int j = 0; j < 4; ++j) sv[4 * p + j] = sx[p][j];
        }
        if (kt < kt_end) LT::load(nxt, V, (kt + 1) * kTile, T, tid);
        // the staging loads stay ahead of the score loads: the wait at the end
        // of the step leaves only those 4 in flight
        __builtin_amdgcn_sched_barrier(0);
        if (prefetch) {
#pragma unroll
            for (int p = 0; p < 4; ++p)
                sx[p] = __builtin_nontemporal_load(
                    (const f32x4*)(tiles + (size_t)(kt + 1) * kTileElems + p * 256 + lane * 4));
        }
        __builtin_amdgcn_sched_barrier(0);
        if (here) {
            if (kt == qt) {
#pragma unroll
                for (int r = 0; r < 16; ++r) recon(kt, std::true_type{}, r, wA, wlA);
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) recon(kt, std::false_type{}, r, wA, wlA);
            }
            float xv[16 * NB];
            v_operand(cur, xv);
#pragma unroll
            for (int s = 0; s < 16 * NB; ++s) {
                const int b = s >> 4, kk = s & 15;
                oacc[b] = mfma32x32x2(xv[s], wA[kk], oacc[b]);
                if (PROB) olacc[b] = mfma32x32x2(xv[s], wlA[kk], olacc[b]);
            }
        }
        flush_sums();
        if (prefetch) wait_vmcnt<4>();
        else wait_vmcnt<0>();
        lds_barrier();
    };
    for (int kt = 0; kt <= kt_end; kt += 2) {
        if constexpr (PIPE) {
            sweep2(kt, lds0, lds1, wA, wlA, wB, wlB);
            if (kt + 1 <= kt_end) sweep2(kt + 1, lds1, lds0, wB, wlB, wA, wlA);
        } else {
            sweep2_serial(kt, lds0, lds1);
            if (kt + 1 <= kt_end) sweep2_serial(kt + 1, lds1, lds0);
        }
    }
    W64 += __shfl_xor(W64, 32);
    const float W = (float)W64;
    float WL = W;  // LERP: the forward weights are the LERP weights
    if (REC == REC_NEAREST) {
        WL64 += __shfl_xor(WL64, 32);
        WL = (float)WL64;
    }

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
    const dim3 grid((unsigned)(a.BH * n_blk));
    if constexpr (D == 64 && !PROB) {
        if (a.n_t <= kPipeMaxTiles) {
            hipLaunchKernelGGL((kia_forward_kernel<D, CAL, REC, PROB, DUMP, false>), grid, dim3(kThreads), 0, s, a);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((kia_forward_kernel<D, CAL, REC, PROB, DUMP, true>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int D, int CAL, int REC, bool PROB>
static hipError_t launch_fwd_grid(const FwdConfig& c, const FwdArgs& a, hipStream_t s) {
    return c.dump ? launch_fwd_t<D, CAL, REC, PROB, true>(a, s) : launch_fwd_t<D, CAL, REC, PROB, false>(a, s);
}

template <int D, int CAL>
static hipError_t launch_fwd_rec(const FwdConfig& c, const FwdArgs& a, hipStream_t s) {
    if (softmax_rec(c.rec)) {
        // softmax anchored at the max only: built on the FWM path
        if constexpr (CAL == CAL_FWM) {
            if (c.rec == REC_EXACT)
                return c.dump ? launch_fwd_t<D, CAL, REC_EXACT, false, true>(a, s)
                              : launch_fwd_t<D, CAL, REC_EXACT, false, false>(a, s);
            if (c.rec == REC_EXP_BF16)
                return c.dump ? launch_fwd_t<D, CAL, REC_EXP_BF16, false, true>(a, s)
                              : launch_fwd_t<D, CAL, REC_EXP_BF16, false, false>(a, s);
            return c.dump ? launch_fwd_t<D, CAL, REC_EXP_FP8, false, true>(a, s)
                          : launch_fwd_t<D, CAL, REC_EXP_FP8, false, false>(a, s);
        }
        return hipErrorInvalidValue;
    }
    if (c.rec == REC_LERP) return launch_fwd_grid<D, CAL, REC_LERP, false>(c, a, s);
    if (c.prob) return launch_fwd_grid<D, CAL, REC_NEAREST, true>(c, a, s);
    return launch_fwd_grid<D, CAL, REC_NEAREST, false>(c, a, s);
}

template <int D>
static hipError_t launch_fwd_d(const FwdConfig& c, const FwdArgs& a, hipStream_t s) {
    if (c.cal == CAL_MINMAX) return launch_fwd_rec<D, CAL_MINMAX>(c, a, s);
    if (c.cal == CAL_FWM) return launch_fwd_rec<D, CAL_FWM>(c, a, s);
    return launch_fwd_rec<D, CAL_FWM_UNTRUNC>(c, a, s);
}

hipError_t launch_forward(const FwdConfig& c, const FwdArgs& a, hipStream_t s) {
    return c.d == 64 ? launch_fwd_d<64>(c, a, s) : launch_fwd_d<128>(c, a, s);
}

}  // namespace kia
