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

enum { CAL_MINMAX = 0, CAL_FWM = 1, CAL_FWM_UNTRUNC = 2 };
enum { REC_LERP = 0, REC_NEAREST = 1, REC_EXACT = 2, REC_EXP_BF16 = 3, REC_EXP_FP8 = 4 };
// Softmax anchored at the row max, no grid: the exact reference and its
// rounded-exponential baselines.
constexpr bool softmax_rec(int rec) { return rec >= REC_EXACT; }

enum { GRAD_FULL = 0, GRAD_DETACH = 1, GRAD_MAX_ONLY = 2, GRAD_MIN_ONLY = 3, GRAD_P1 = 4 };

// Spans below this take the degenerate branch (App. A: branches for spans
// above or below 1e-12).
constexpr float kEpsSpan = 1e-12f;
constexpr float kLog2e = 1.4426950408889634f;  // log2(e): exp(x) = exp2(x * log2(e))
constexpr float kLn2 = 0.6931471805599453f;    // ln(2): ln(exp2(x)) = x * ln(2)

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

// A 32 x D tile of a row-major [T][D] tensor staged in LDS by the whole
// workgroup with direct global -> LDS loads (global_load_lds_dwordx4: each
// lane's 16 bytes land at slot lane of a 1 KB chunk, no registers involved).
// We choose which float4 of the tile each lane fetches, so the slots can be
// swizzled: float4 column c4 of row r sits at slot r*(D/4) + (c4 ^ swz(r)),
// swz a permutation of r's low 4 bits with bit 3 = bit 2 of r.  Then
//  - a row read (lane = row, one float4) by 16 lanes hits 16 distinct 4-bank
//    groups, and
//  - a column read (lane = column, one float) by 64 lanes whose two halves
//    take rows r and r+4 (r%8 < 4) hits 64 distinct banks.
// Rows at or past T are fetched from row T-1 (finite, and every consumer
// multiplies them by a zero weight, probability or score gradient).
// LDS destination of a direct global -> LDS load.  The address passes through
// an empty asm statement, so the compiler keeps no alias scope for the load's
// LDS target: it then orders the load conservatively against every LDS access
// but does not insert its own vmcnt waits before reads of other buffers.  The
// kernels order these loads with explicit wait_vmcnt + barrier pairs.
__device__ __forceinline__ __attribute__((address_space(3))) void* lds_dst(float* p) {
    uint32_t a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)p;
    asm volatile("" : "+v"(a));
    return (__attribute__((address_space(3))) void*)(uintptr_t)a;
}

template <int D>
struct LdsTile {
    static constexpr int kF4Row = D / 4;
    static constexpr int kFloats = kTile * D;
    static __device__ __forceinline__ int swz(int r) {
        return (r & 3) | (((r >> 3) & 1) << 2) | (((r >> 2) & 1) << 3);
    }
    static __device__ __forceinline__ int off(int r, int c) {
        return (r * kF4Row + ((c >> 2) ^ swz(r))) * 4 + (c & 3);
    }
    static __device__ __forceinline__ void load(float* lds_tile, const float* src, int r0, int T, int tid) {
        const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
        for (int k = 0; k < D / 32; ++k) {
            const int i = wave + kWaves * k;  // 1 KB chunk index
            const int slot = i * kWave + lane;
            const int r = slot / kF4Row;
            const int c4 = (slot % kF4Row) ^ swz(r);
            const float* g = src + (size_t)min(r0 + r, T - 1) * D + 4 * c4;
            __builtin_amdgcn_global_load_lds((const void*)g, lds_dst(lds_tile + i * 256),
                                             16, 0, 0);
        }
    }
};

// Direct global -> LDS copy of one wave's 4 KB fragment-native tile (the
// column kernel's probability and score-gradient tiles): lane l fetches its
// float4 of each 1 KB chunk, which lands at the same place in the wave's LDS
// slot, so the lane later reads back exactly the registers it would have
// loaded.  Each such tile is read once per kernel, so the loads are
// non-temporal (cache policy NT): they do not displace the Q and dO tiles
// that every workgroup of a slice re-reads from L2.
constexpr int kCpolNonTemporal = 2;
__device__ __forceinline__ void dma_tile(float* lds_wave, const float* src, int lane) {
#pragma unroll
    for (int p = 0; p < 4; ++p)
        __builtin_amdgcn_global_load_lds((const void*)(src + p * 256 + lane * 4), lds_dst(lds_wave + p * 256), 16,
                                         0, kCpolNonTemporal);
}
__device__ __forceinline__ void read_tile(const float* lds_wave, int lane, float* out) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const f32x4 x = *(const f32x4*)(lds_wave + p * 256 + lane * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) out[4 * p + j] = x[j];
    }
}

// Workgroup barrier that orders LDS only.  Each wave waits for its own LDS
// reads and writes (lgkmcnt) and then meets the others; global loads and
// stores stay in flight.  (__syncthreads also drains vmcnt, which would retire
// every prefetch and score store before the next tile could start.)  Direct
// global -> LDS loads are counted by vmcnt: a wave waits for its share with
// wait_vmcnt before calling this.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most N vector memory operations of this wave are outstanding
// (lgkm and exp counters left free).  On this architecture vector memory
// operations (loads, stores, global -> LDS loads) report completion to the
// wave in execution order; the one exception LLVM's AMDGPU memory model
// documents for GFX90A / GFX942 is a FLAT instruction that touches LDS, and
// these kernels issue only global_* instructions.  (The compiler's own wait
// insertion relies on the same ordering: it waits for a load by counting the
// vector memory operations issued after it, loads and stores alike.)  So
// this waits for everything issued before the last N.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Wait until this wave's LDS operations have completed (vector memory and
// export counters left free).
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0x0F | (0x7 << 4) | (0x3 << 14)); }

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

// Interleave NS matrix steps with NE vector steps (NE <= NS), spreading the
// vector steps evenly, so one wavefront keeps its matrix pipe busy while its
// vector ALU works on independent data (another tile's elementwise math).
template <int NS, int NE, typename FM, typename FV>
__device__ __forceinline__ void interleave(FM&& fm, FV&& fv) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        fm(s);
#pragma unroll
        for (int e = s * NE / NS; e < (s + 1) * NE / NS; ++e) fv(e);
    }
}

// Ask the scheduler to keep the interleave: NS groups of one matrix
// instruction followed by up to VPER vector ALU instructions.  Must sit in the
// same basic block as the code it orders.
template <int NS, int VPER, int NREAD = 0>
__device__ __forceinline__ void pin_interleave() {
    if (NREAD > 0) __builtin_amdgcn_sched_group_barrier(0x100, NREAD, 0);  // LDS reads first
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, VPER, 0);  // VALU
    }
}

// (qt, kt) of the triangular tile index ti = qt*(qt+1)/2 + kt.
__device__ __forceinline__ void tile_coords(int ti, int& qt, int& kt) {
    qt = (int)((sqrtf(8.f * ti + 1.f) - 1.f) * 0.5f);
    while ((int64_t)qt * (qt + 1) / 2 > ti) --qt;
    while ((int64_t)(qt + 1) * (qt + 2) / 2 <= ti) ++qt;
    kt = ti - (int)((int64_t)qt * (qt + 1) / 2);
}

// Wave priority by block length.  Blocks of a causal slice differ in length
// by up to n_blk x, and two workgroups share each CU; raising the issue
// priority of the longer block's waves (0..3 in proportion to its length)
// lets the launch's critical path run ahead while shorter blocks fill the
// remaining issue slots.  len is the block's tile count, max_len the longest.
__device__ __forceinline__ void set_length_priority(int len, int max_len) {
    const int prio = max_len > 0 ? min(3, (4 * len - 1) / max_len) : 0;
    switch (prio) {
        case 3: __builtin_amdgcn_s_setprio(3); break;
        case 2: __builtin_amdgcn_s_setprio(2); break;
        case 1: __builtin_amdgcn_s_setprio(1); break;
        default: break;
    }
}

// Per-row grid constants derived from the calibration statistics.  Forward
// and backward both call this, so they see bitwise identical constants.
struct RowGrid {
    float m;      // row max (the anchor of the grid)
    float invh;   // 1/h (0 in the degenerate branch)
    float hl2;    // h * log2(e), so exp(-j h) = exp2(-j * hl2)
    float c;      // 1 - exp(-h): relative drop across one interval
    float coh;    // c / h (1 in the degenerate branch: the h -> 0 limit)
    float cohm1;  // c / h - 1
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
    g.cohm1 = g.coh - 1.f;
    return g;
}

// Grid table: for rows whose grid has at most kTabMaxK intervals, the K+1
// values of the row's grid (scaled as the kernel needs them) are computed once
// per row block and kept in LDS, and each score's reconstruction reads its
// segment's or grid point's value instead of evaluating an exponential.  Each
// wave holds the table of its 32 rows, column-major: entry i of row li at
// i*32 + li, so the lanes of different rows read different banks whatever
// index they take (only the two lane halves of one row can collide).
constexpr int kTabMaxK = 32;
constexpr int kTabEntries = kTabMaxK + 1;
constexpr int kTabWaveFloats = kTabEntries * kTile;
__device__ __forceinline__ int tab_off(int i, int li) { return i * kTile + li; }

// Whether a (calibration, reconstruction) pair reads its grid values from the
// table: the finite grids (MinMax, FWM) under LERP and Nearest.  The
// untruncated step's grid is unbounded and the softmax family has none.
constexpr bool tab_capable(int cal, int rec) {
    return (cal == CAL_MINMAX || cal == CAL_FWM) && (rec == REC_LERP || rec == REC_NEAREST);
}

// exp2 on the hardware transcendental unit.  Results below the fp32 normal
// range (weights under 1.2e-38, i.e. more than 87 nats below the row max)
// may flush to zero; that changes a normalised probability by less than
// 1e-38 relative.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Rounded exponentials of the reduced-precision baselines (App. D.5): a
// non-negative fp32 value (at most 1 here) rounded to nearest, ties to even,
// in bf16 (7 fraction bits) or FP8 E4M3 (3 fraction bits, smallest normal
// 2^-6, subnormal step 2^-9), returned as the fp32 value it represents.
template <int REC>
__device__ __forceinline__ float round_exp(float e) {
    if constexpr (REC == REC_EXP_BF16) {
        uint32_t b = __float_as_uint(e);
        b += 0x7fffu + ((b >> 16) & 1u);
        return __uint_as_float(b & 0xffff0000u);
    } else if constexpr (REC == REC_EXP_FP8) {
        if (e < 0.015625f) return rintf(e * 512.f) * 0.001953125f;  // multiples of 2^-9
        uint32_t b = __float_as_uint(e);
        b += 0x7ffffu + ((b >> 20) & 1u);
        return __uint_as_float(b & 0xfff00000u);
    } else {
        return e;
    }
}

}  // namespace kia
