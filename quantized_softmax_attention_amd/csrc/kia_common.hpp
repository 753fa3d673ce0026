// Device helpers shared by the K-interval attention kernels (gfx950).
//
// Tiling: a tile is 32 queries x 32 keys.  One wavefront (64 lanes) owns one
// tile row (32 queries) in the query-stationary kernels, or one tile column
// (32 keys) in the key-stationary kernel.  Contractions use the fp32 matrix
// instruction v_mfma_f32_32x32x2_f32: D(32x32) += A(32x2) * B(2x32), where
// lane l supplies A[l%32][l/32] and B[l/32][l%32], and the 16 accumulator
// registers of lane l hold D[row][l%32] for row = 8*(r/4) + 4*(l/32) + r%4.
//
// Score tiles are produced as S^T = K Q^T, so lane l%32 is the query and the
// 16 registers walk its keys; that accumulator is directly the B operand of
// O^T = V^T W^T when the contraction over keys takes key 8*(kk/4)+4*(l/32)+kk%4
// at step kk (the same walk), which is how every kernel here pairs them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kia {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 32;
constexpr int kTileElems = kTile * kTile;
constexpr int kWave = 64;

enum { CAL_MINMAX = 0, CAL_FWM = 1 };
enum { REC_LERP = 0, REC_NEAREST = 1 };
enum { GRAD_FULL = 0, GRAD_DETACH = 1, GRAD_MAX_ONLY = 2, GRAD_MIN_ONLY = 3 };

// Spans below this take the degenerate branch (App. A: branches for spans
// above or below 1e-12).
constexpr float kEpsSpan = 1e-12f;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mfma32x32x2(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Row (M) index held by accumulator register r of a lane in half hl, and the
// contraction index taken at step kk by lanes of half hl: the same walk.
__device__ __forceinline__ int acc_row(int r, int hl) { return 8 * (r >> 2) + 4 * hl + (r & 3); }

// Offset (in floats) of tile (qt, kt), kt <= qt, inside one (b, h) slice.
__host__ __device__ __forceinline__ int64_t tile_index(int qt, int kt) {
    return (int64_t)qt * (qt + 1) / 2 + kt;
}

// Query-major tile storage: lane l's registers 4p..4p+3 are the float4 at
// p*256 + 4*l, so a store or load of one p by a whole wave is one contiguous
// kilobyte.  Element (query qi, key kj) sits at lane qi + 32*((kj>>2)&1),
// register 4*(kj>>3) + (kj&3).
__host__ __device__ __forceinline__ int qmajor_offset(int qi, int kj) {
    return (kj >> 3) * 256 + (qi + 32 * ((kj >> 2) & 1)) * 4 + (kj & 3);
}

// Key-major tile storage used for P and dS in the backward: the same
// arrangement with the roles of query and key swapped, so lane l holds key
// l%32 and its registers walk the queries 8*(r/4) + 4*(l/32) + r%4.
__host__ __device__ __forceinline__ int kmajor_offset(int qi, int kj) { return qmajor_offset(kj, qi); }

// ---- workgroup tiling --------------------------------------------------------
// A workgroup of 4 wavefronts owns 128 stationary rows (32 per wave) and
// streams 32-row tiles of the other operand through LDS, double-buffered.
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kBlockTiles = kWaves;  // stationary 32-row tiles per workgroup

// LDS layouts of a streamed 32 x D tile (rows r of a row-major [T][D] tensor):
//  row-major  rm(r, c) = r*(D+4) + c: lane = row, float4 along c (no conflicts)
//  transposed tr(c, r) = c*32 + 4*((r/4) ^ (c%8)) + r%4: lane = column c,
//             float4 along 4 consecutive rows; the xor spreads both the
//             staging writes and the float4 reads over all banks.
template <int D>
__device__ __forceinline__ int rm_off(int r, int c) { return r * (D + 4) + c; }
__device__ __forceinline__ int tr_off(int c, int r) { return c * kTile + 4 * ((r >> 2) ^ (c & 7)) + (r & 3); }

template <int D>
struct StreamTile {
    static constexpr int kF4 = kTile * D / 4 / kThreads;  // float4 per thread
    static constexpr int kRM = kTile * (D + 4);          // floats of a row-major staged tile
    static constexpr int kTR = D * kTile;                // floats of a transposed staged tile
    f32x4 v[kF4];

    // row-major staging: consecutive threads read consecutive float4 of a row
    __device__ __forceinline__ void load_rm(const float* src, int r0, int T, int tid) {
#pragma unroll
        for (int i = 0; i < kF4; ++i) {
            const int e = tid + kThreads * i, r = e / (D / 4), c4 = e % (D / 4);
            v[i] = (r0 + r < T) ? *(const f32x4*)(src + (size_t)(r0 + r) * D + 4 * c4) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    __device__ __forceinline__ void store_rm(float* lds, int tid) const {
#pragma unroll
        for (int i = 0; i < kF4; ++i) {
            const int e = tid + kThreads * i, r = e / (D / 4), c4 = e % (D / 4);
            *(f32x4*)(lds + rm_off<D>(r, 4 * c4)) = v[i];
        }
    }
    // transposed staging: a wave's lanes take 32 consecutive rows of one float4 column
    __device__ __forceinline__ void load_tr(const float* src, int r0, int T, int tid) {
#pragma unroll
        for (int i = 0; i < kF4; ++i) {
            const int e = tid + kThreads * i, r = e & 31, c4 = e >> 5;
            v[i] = (r0 + r < T) ? *(const f32x4*)(src + (size_t)(r0 + r) * D + 4 * c4) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    __device__ __forceinline__ void store_tr(float* lds, int tid) const {
#pragma unroll
        for (int i = 0; i < kF4; ++i) {
            const int e = tid + kThreads * i, r = e & 31, c4 = e >> 5;
#pragma unroll
            for (int j = 0; j < 4; ++j) lds[tr_off(4 * c4 + j, r)] = v[i][j];
        }
    }
};

// Heaviest-first work order over (slice, 128-row block) pairs.  Blocks of one
// slice share K and V; workgroups are dealt round-robin to the 8 XCDs, so when
// B*H is a multiple of 8 all blocks of a slice are kept on one XCD (one L2).
// `descending` puts high block indices first (query-stationary kernels: the
// last query blocks see the most keys); otherwise low indices first.
__device__ __forceinline__ void map_block(int g, int BH, int nb, bool descending, int& bh, int& blk) {
    int s;
    if ((BH & 7) == 0) {
        const int x = g & 7, per = BH >> 3;
        s = g >> 3;
        bh = (s % per) * 8 + x;
        blk = s / per;
    } else {
        bh = g % BH;
        blk = g / BH;
    }
    if (descending) blk = nb - 1 - blk;
}

// Per-row grid constants derived from the calibration statistics.  Forward
// and backward both call this, so they see bitwise identical constants.
struct RowGrid {
    float m;      // row max (the anchor of the grid)
    float invh;   // 1/h (0 in the degenerate branch)
    float hl2;    // h * log2(e), so exp(-j h) = exp2(-j * hl2)
    float c;      // 1 - exp(-h): relative drop across one interval
    float coh;    // c / h (1 in the degenerate branch: the h -> 0 limit)
    float Kf;     // K as float
    bool degen;
};

__device__ __forceinline__ RowGrid make_row_grid(float m, float n, int K, float tau, int cal) {
    RowGrid g;
    g.m = m;
    g.Kf = (float)K;
    float h;
    if (cal == CAL_MINMAX) {
        float span = m - n;
        g.degen = span < kEpsSpan;
        h = span / (float)K;
    } else {
        g.degen = false;
        h = tau / (float)K;
    }
    if (g.degen) {
        g.invh = 0.f;
        g.hl2 = 0.f;
        g.c = 0.f;
        g.coh = 1.f;
    } else {
        g.invh = 1.f / h;
        g.hl2 = h * kLog2e;
        g.c = -expm1f(-h);
        g.coh = g.c * g.invh;
    }
    return g;
}

// Reconstruction of one score.  uc = min(u, K) with u = (m - s)/h; LERP
// segment i = min(floor(uc), K-1), f = uc - i, weight g_i (1 - f c) where
// g_i = exp(-i h) is grid value i; Nearest grid point r = floor(uc + 1/2),
// weight g_r.  `inwin` is the FWM window test u <= K (always true for
// MinMax).
struct Recon {
    float uc, fi, f, g, wl, wn;
    bool inwin;
};

template <int CAL, bool NEED_NEAREST>
__device__ __forceinline__ Recon reconstruct(const RowGrid& rg, float s) {
    Recon e;
    float u = (rg.m - s) * rg.invh;
    e.inwin = (CAL == CAL_MINMAX) ? true : (u <= rg.Kf);
    e.uc = fminf(u, rg.Kf);
    e.fi = fminf(fmaxf(floorf(e.uc), 0.f), rg.Kf - 1.f);
    e.f = e.uc - e.fi;
    e.g = exp2f(-e.fi * rg.hl2);
    e.wl = e.g * fmaf(-e.f, rg.c, 1.f);
    if (NEED_NEAREST) {
        float fr = floorf(e.uc + 0.5f);
        e.wn = exp2f(-fr * rg.hl2);
    } else {
        e.wn = 0.f;
    }
    return e;
}

}  // namespace kia
