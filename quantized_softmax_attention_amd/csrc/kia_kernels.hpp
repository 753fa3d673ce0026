// Kernel argument blocks and launch entry points (internal to libkia).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kia {

struct FwdArgs {
    const float* q;
    const float* k;
    const float* v;
    float* o;
    float* tiles;        // score tiles, query-major
    float* row_m;
    float* row_n;
    int32_t* row_a;
    int32_t* row_b;
    float* row_w;
    float* row_wl;
    float* o_lerp;       // Prob-STE only
    int32_t* idx_dump;   // optional [BH, T, T]
    int BH, T, n_t, K;
    float tau, scale;
};

struct BwdArgs {
    const float* q;
    const float* k;
    const float* v;
    const float* o;
    const float* d_o;
    const float* tiles;
    const float* row_m;
    const float* row_n;
    const int32_t* row_a;
    const int32_t* row_b;
    const float* row_w;
    const float* row_wl;
    const float* o_lerp;
    float* dq;
    float* dk;
    float* dv;
    float* probs;        // key-major P tiles
    float* dscores;      // key-major dS tiles (calibration terms folded in)
    float* row_cm;       // P1: the subtracted row mean
    float* row_cn;
    float* prefix_k;     // P1 only: sum_{j <= t} K_j per row, [BH, T, d] (read by the row kernel)
    float* chunk_k;      // P1 only: per-32-row chunk sums of K, then of mu_t Q_t, [BH, n_t, d]
    float* suffix_q;     // P1 only: sum_{t' >= t} mu_t' Q_t' per row, [BH, T, d] (the
                         // prefix_k memory, rewritten after the row kernel; read by the column kernel)
    int BH, T, n_t, K;
    float tau, scale;
    int rule;
};

struct GeoArgs {
    const float* q;
    const float* k;
    const float* tiles;  // score tiles of a forward with the same flags
    const float* row_m;
    const float* row_w;
    float* geo;          // [8][BH * T]
    int BH, T, n_t, K, d;
    float tau;
};

struct FwdConfig {
    int d, cal, rec;
    bool prob, dump;
    bool tab;  // grid values from the per-row LDS table (K <= kTabMaxK, finite grid)
};

hipError_t launch_forward(const FwdConfig& c, const FwdArgs& a, hipStream_t s);
hipError_t launch_backward_rows(const FwdConfig& c, const BwdArgs& a, hipStream_t s);
hipError_t launch_backward_cols(int d, const BwdArgs& a, hipStream_t s);
hipError_t launch_key_prefix(int d, const BwdArgs& a, hipStream_t s);
hipError_t launch_query_suffix(int d, const BwdArgs& a, hipStream_t s);
hipError_t launch_geometry(int cal, int rec, const GeoArgs& a, hipStream_t s);
hipError_t launch_tiles_to_dense(int BH, int T, const float* tiles, int key_major, float* dense,
                                 hipStream_t s);

}  // namespace kia
