// C ABI of libkia: argument checks, buffer layouts and kernel dispatch.
// Every check runs before the first launch; the library never allocates,
// never synchronises and keeps no mutable global state.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/kia.h"
#include "kia_common.hpp"
#include "kia_kernels.hpp"

// Device scratch of the allocation-free backward (kia_backward_noalloc): it
// stands in for kia_backward's caller-supplied workspace.  Each device the
// library runs on holds its own copy until the process ends.  Host code
// addresses it only through the per-device pointer hipGetSymbolAddress
// returns; the array's name is a host-side stand-in, not a device address.
constexpr size_t kScratchBytes = (size_t)KIA_NOALLOC_SCRATCH_MIB << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxIntervals = 65536;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

kia_status check_params(const kia_params* p) {
    if (!p) return KIA_ERR_NULL;
    if (p->n_intervals < 1 || p->n_intervals > kMaxIntervals) return KIA_ERR_PARAM;
    if (p->calibration < KIA_CAL_MINMAX || p->calibration > KIA_CAL_FWM_UNTRUNC) return KIA_ERR_PARAM;
    if (p->reconstruction < KIA_REC_LERP || p->reconstruction > KIA_REC_EXP_FP8) return KIA_ERR_PARAM;
    if (p->surrogate != KIA_STE_WEIGHT && p->surrogate != KIA_STE_PROB) return KIA_ERR_PARAM;
    if (p->grad_rule < KIA_GRAD_FULL || p->grad_rule > KIA_GRAD_P1) return KIA_ERR_PARAM;
    if (p->calibration != KIA_CAL_MINMAX && p->reconstruction < KIA_REC_EXACT &&
        !(p->tau > 0.f && isfinite(p->tau)))
        return KIA_ERR_PARAM;
    return KIA_OK;
}

struct Shape {
    int64_t B, H, T, d, BH, n_t, tiles_per_head;
};

kia_status check_shape(int B, int H, int T, int d, Shape* s) {
    if (B < 1 || H < 1 || T < 1) return KIA_ERR_SHAPE;
    if (d != 64 && d != 128) return KIA_ERR_SHAPE;
    s->B = B; s->H = H; s->T = T; s->d = d;
    s->BH = (int64_t)B * H;
    s->n_t = ((int64_t)T + kia::kTile - 1) / kia::kTile;
    s->tiles_per_head = s->n_t * (s->n_t + 1) / 2;
    // grids are B*H*n_t workgroups; tensors and tile buffers are indexed in size_t
    if (s->BH > INT32_MAX || s->BH * s->n_t > INT32_MAX) return KIA_ERR_SHAPE;
    if ((double)s->BH * s->tiles_per_head * kia::kTileElems * 4.0 > 9.0e18) return KIA_ERR_SHAPE;
    return KIA_OK;
}

bool prob_extras(const kia_params* p) {
    return p->reconstruction == KIA_REC_NEAREST && p->surrogate == KIA_STE_PROB;
}

void stats_layout(const kia_params* p, const Shape& s, kia_stats_layout* L) {
    size_t off = 0;
    const size_t rows = (size_t)(s.BH * s.T);
    L->scores = off;       off = align_up(off + (size_t)s.BH * s.tiles_per_head * kia::kTileElems * 4);
    L->row_m = off;        off = align_up(off + rows * 4);
    L->row_n = off;        off = align_up(off + rows * 4);
    L->row_a = off;        off = align_up(off + rows * 4);
    L->row_b = off;        off = align_up(off + rows * 4);
    L->row_w = off;        off = align_up(off + rows * 4);
    L->row_wl = off;       off = align_up(off + rows * 4);
    if (prob_extras(p)) {
        L->o_lerp = off;   off = align_up(off + rows * (size_t)s.d * 4);
    } else {
        L->o_lerp = 0;
    }
    L->total_bytes = off;
    L->tiles_per_head = s.tiles_per_head;
}

void workspace_layout(const kia_params* p, const Shape& s, kia_workspace_layout* L) {
    size_t off = 0;
    const size_t rows = (size_t)(s.BH * s.T);
    const size_t tiles = (size_t)s.BH * s.tiles_per_head * kia::kTileElems * 4;
    L->probs = off;    off = align_up(off + tiles);
    L->dscores = off;  off = align_up(off + tiles);
    L->row_cm = off;   off = align_up(off + rows * 4);
    L->row_cn = off;   off = align_up(off + rows * 4);
    if (p->grad_rule == KIA_GRAD_P1) {
        L->prefix_k = off; off = align_up(off + rows * (size_t)s.d * 4);
        L->chunk_k = off;  off = align_up(off + (size_t)s.BH * s.n_t * (size_t)s.d * 4);
    } else {
        L->prefix_k = 0;
        L->chunk_k = 0;
    }
    L->total_bytes = off;
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

kia_status record(const kia_ext* ext, int i, hipStream_t st) {
    if (!ext || !ext->events || i >= ext->n_events || !ext->events[i]) return KIA_OK;
    return hipEventRecord((hipEvent_t)ext->events[i], st) == hipSuccess ? KIA_OK : KIA_ERR_HIP;
}

// The exact-softmax reference and its rounded baselines are anchored at the
// row max only; they run on the FWM instantiation, whose grid constants they
// never read.
bool exact(const kia_params* p) { return p->reconstruction >= KIA_REC_EXACT; }
float tau_of(const kia_params* p) { return exact(p) ? 1.f : p->tau; }

// KIA_GRID_TABLE=0 in the environment turns the row kernel's grid table off
// (one exponential per score instead): the results are bitwise the same, so
// the two can be compared by time and counters alone.
bool grid_table_enabled() {
    const char* e = getenv("KIA_GRID_TABLE");
    return !(e && e[0] == '0' && e[1] == '\0');
}

kia::FwdConfig config_of(const kia_params* p, int d, bool dump) {
    kia::FwdConfig c;
    c.d = d;
    c.cal = exact(p) ? KIA_CAL_FWM : p->calibration;
    c.rec = p->reconstruction;
    c.prob = prob_extras(p);
    c.dump = dump;
    c.tab = kia::tab_capable(c.cal, c.rec) && p->n_intervals <= kia::kTabMaxK && grid_table_enabled();
    return c;
}

}  // namespace

extern "C" {

size_t kia_stats_bytes(const kia_params* p, int B, int H, int T, int d) {
    Shape s;
    if (check_params(p) != KIA_OK || check_shape(B, H, T, d, &s) != KIA_OK) return 0;
    kia_stats_layout L;
    stats_layout(p, s, &L);
    return L.total_bytes;
}

size_t kia_workspace_bytes(const kia_params* p, int B, int H, int T, int d) {
    Shape s;
    if (check_params(p) != KIA_OK || check_shape(B, H, T, d, &s) != KIA_OK) return 0;
    kia_workspace_layout L;
    workspace_layout(p, s, &L);
    return L.total_bytes;
}

kia_status kia_stats_layout_query(const kia_params* p, int B, int H, int T, int d, kia_stats_layout* out) {
    if (!out) return KIA_ERR_NULL;
    kia_status st = check_params(p);
    if (st != KIA_OK) return st;
    Shape s;
    if ((st = check_shape(B, H, T, d, &s)) != KIA_OK) return st;
    stats_layout(p, s, out);
    return KIA_OK;
}

kia_status kia_workspace_layout_query(const kia_params* p, int B, int H, int T, int d,
                                      kia_workspace_layout* out) {
    if (!out) return KIA_ERR_NULL;
    kia_status st = check_params(p);
    if (st != KIA_OK) return st;
    Shape s;
    if ((st = check_shape(B, H, T, d, &s)) != KIA_OK) return st;
    workspace_layout(p, s, out);
    return KIA_OK;
}

kia_status kia_forward_ext(const kia_params* p, int B, int H, int T, int d, const float* q, const float* k,
                           const float* v, float* o, void* stats, size_t stats_bytes, void* stream,
                           const kia_ext* ext) {
    kia_status st = check_params(p);
    if (st != KIA_OK) return st;
    Shape s;
    if ((st = check_shape(B, H, T, d, &s)) != KIA_OK) return st;
    if (!q || !k || !v || !o || !stats) return KIA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(stats))
        return KIA_ERR_ALIGN;
    kia_stats_layout L;
    stats_layout(p, s, &L);
    if (stats_bytes < L.total_bytes) return KIA_ERR_BUFFER;
    if (ext && ext->n_events < 0) return KIA_ERR_PARAM;

    char* base = (char*)stats;
    kia::FwdArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o;
    a.tiles = (float*)(base + L.scores);
    a.row_m = (float*)(base + L.row_m);
    a.row_n = (float*)(base + L.row_n);
    a.row_a = (int32_t*)(base + L.row_a);
    a.row_b = (int32_t*)(base + L.row_b);
    a.row_w = (float*)(base + L.row_w);
    a.row_wl = (float*)(base + L.row_wl);
    a.o_lerp = prob_extras(p) ? (float*)(base + L.o_lerp) : nullptr;
    a.idx_dump = ext ? ext->idx_dump : nullptr;
    a.BH = (int)s.BH; a.T = T; a.n_t = (int)s.n_t; a.K = p->n_intervals;
    a.tau = tau_of(p);
    a.scale = 1.f / sqrtf((float)d);

    hipStream_t hs = (hipStream_t)stream;
    if ((st = record(ext, 0, hs)) != KIA_OK) return st;
    if (kia::launch_forward(config_of(p, d, a.idx_dump != nullptr), a, hs) != hipSuccess) return KIA_ERR_HIP;
    return record(ext, 1, hs);
}

kia_status kia_forward(const kia_params* p, int B, int H, int T, int d, const float* q, const float* k,
                       const float* v, float* o, void* stats, size_t stats_bytes, void* stream) {
    return kia_forward_ext(p, B, H, T, d, q, k, v, o, stats, stats_bytes, stream, nullptr);
}

}  // extern "C"

namespace {

struct BwdPtrs {
    const float *q, *k, *v, *o, *d_o;
    const void* stats;
    size_t stats_bytes;
    float *dq, *dk, *dv;
};

// Checks shared by the backward entry points (everything but the workspace).
kia_status check_backward(const kia_params* p, int B, int H, int T, int d, const BwdPtrs& b, Shape* s) {
    kia_status st = check_params(p);
    if (st != KIA_OK) return st;
    if ((st = check_shape(B, H, T, d, s)) != KIA_OK) return st;
    if (!b.q || !b.k || !b.v || !b.o || !b.d_o || !b.stats || !b.dq || !b.dk || !b.dv) return KIA_ERR_NULL;
    if (!aligned16(b.q) || !aligned16(b.k) || !aligned16(b.v) || !aligned16(b.o) || !aligned16(b.d_o) ||
        !aligned16(b.stats) || !aligned16(b.dq) || !aligned16(b.dk) || !aligned16(b.dv))
        return KIA_ERR_ALIGN;
    kia_stats_layout L;
    stats_layout(p, *s, &L);
    if (b.stats_bytes < L.total_bytes) return KIA_ERR_BUFFER;
    return KIA_OK;
}

// Shape of `n` of the slices of s (the same T and d).
Shape slices_of(const Shape& s, int64_t n) {
    Shape c = s;
    c.BH = n;
    c.B = 1;
    c.H = n;
    return c;
}

// Launch the backward over the slices [s0, s0 + n) of a checked shape s.  The
// inputs, outputs and the forward's statistics are addressed inside the
// whole-batch buffers; `ws` holds the workspace laid out for n slices.
// Slices never interact, so any split of the batch gives the same results.
kia_status run_backward(const kia_params* p, const Shape& s, int64_t s0, int64_t n, const BwdPtrs& b, char* ws,
                        const kia_ext* ext, hipStream_t hs) {
    const bool p1 = p->grad_rule == KIA_GRAD_P1;
    kia_stats_layout L;
    stats_layout(p, s, &L);
    const Shape c = slices_of(s, n);
    kia_workspace_layout WL;
    workspace_layout(p, c, &WL);

    const size_t rows0 = (size_t)(s0 * s.T);               // first row of the range
    const size_t elem0 = rows0 * (size_t)s.d;              // first element of a [B, H, T, d] tensor
    const size_t tile0 = (size_t)s0 * (size_t)s.tiles_per_head * kia::kTileElems;
    const char* sb = (const char*)b.stats;
    kia::BwdArgs a;
    a.q = b.q + elem0; a.k = b.k + elem0; a.v = b.v + elem0; a.o = b.o + elem0; a.d_o = b.d_o + elem0;
    a.tiles = (const float*)(sb + L.scores) + tile0;
    a.row_m = (const float*)(sb + L.row_m) + rows0;
    a.row_n = (const float*)(sb + L.row_n) + rows0;
    a.row_a = (const int32_t*)(sb + L.row_a) + rows0;
    a.row_b = (const int32_t*)(sb + L.row_b) + rows0;
    a.row_w = (const float*)(sb + L.row_w) + rows0;
    a.row_wl = (const float*)(sb + L.row_wl) + rows0;
    a.o_lerp = prob_extras(p) ? (const float*)(sb + L.o_lerp) + elem0 : nullptr;
    a.dq = b.dq + elem0; a.dk = b.dk + elem0; a.dv = b.dv + elem0;
    a.probs = (float*)(ws + WL.probs);
    a.dscores = (float*)(ws + WL.dscores);
    a.row_cm = (float*)(ws + WL.row_cm);
    a.row_cn = (float*)(ws + WL.row_cn);
    a.prefix_k = p1 ? (float*)(ws + WL.prefix_k) : nullptr;
    a.chunk_k = p1 ? (float*)(ws + WL.chunk_k) : nullptr;
    a.suffix_q = a.prefix_k;  // reused once the row kernel has read the prefix sums
    a.BH = (int)n; a.T = (int)s.T; a.n_t = (int)s.n_t; a.K = p->n_intervals;
    a.tau = tau_of(p);
    a.scale = 1.f / sqrtf((float)s.d);
    a.rule = p->grad_rule;

    kia_status st;
    const kia::FwdConfig cfg = config_of(p, (int)s.d, false);
    if ((st = record(ext, 0, hs)) != KIA_OK) return st;
    if (p1 && kia::launch_key_prefix((int)s.d, a, hs) != hipSuccess) return KIA_ERR_HIP;
    if (kia::launch_backward_rows(cfg, a, hs) != hipSuccess) return KIA_ERR_HIP;
    if (p1 && kia::launch_query_suffix((int)s.d, a, hs) != hipSuccess) return KIA_ERR_HIP;
    if ((st = record(ext, 1, hs)) != KIA_OK) return st;
    if ((st = record(ext, 2, hs)) != KIA_OK) return st;
    if (kia::launch_backward_cols((int)s.d, a, hs) != hipSuccess) return KIA_ERR_HIP;
    return record(ext, 3, hs);
}

// ---- the allocation-free backward -----------------------------------------
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch: looked up once per device (with the device
// current), then reused.
kia_status device_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KIA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return KIA_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return KIA_OK;
}

// Most slices whose workspace fits the scratch (0 when one slice does not).
int64_t slices_per_scratch(const kia_params* p, const Shape& s) {
    kia_workspace_layout WL;
    workspace_layout(p, slices_of(s, 1), &WL);
    if (WL.total_bytes > kScratchBytes) return 0;
    int64_t n = std::min<int64_t>(s.BH, (int64_t)(kScratchBytes / WL.total_bytes));
    for (; n > 1; --n) {
        workspace_layout(p, slices_of(s, n), &WL);
        if (WL.total_bytes <= kScratchBytes) break;
    }
    return n;
}

}  // namespace

extern "C" {

kia_status kia_backward_ext(const kia_params* p, int B, int H, int T, int d, const float* q, const float* k,
                            const float* v, const float* o, const float* d_o, const void* stats,
                            size_t stats_bytes, float* dq, float* dk, float* dv, void* ws, size_t ws_bytes,
                            void* stream, const kia_ext* ext) {
    const BwdPtrs b = {q, k, v, o, d_o, stats, stats_bytes, dq, dk, dv};
    Shape s;
    kia_status st = check_backward(p, B, H, T, d, b, &s);
    if (st != KIA_OK) return st;
    if (!ws) return KIA_ERR_NULL;
    if (!aligned16(ws)) return KIA_ERR_ALIGN;
    kia_workspace_layout WL;
    workspace_layout(p, s, &WL);
    if (ws_bytes < WL.total_bytes) return KIA_ERR_BUFFER;
    if (ext && ext->n_events < 0) return KIA_ERR_PARAM;
    return run_backward(p, s, 0, s.BH, b, (char*)ws, ext, (hipStream_t)stream);
}

kia_status kia_backward(const kia_params* p, int B, int H, int T, int d, const float* q, const float* k,
                        const float* v, const float* o, const float* d_o, const void* stats, size_t stats_bytes,
                        float* dq, float* dk, float* dv, void* ws, size_t ws_bytes, void* stream) {
    return kia_backward_ext(p, B, H, T, d, q, k, v, o, d_o, stats, stats_bytes, dq, dk, dv, ws, ws_bytes,
                            stream, nullptr);
}

kia_status kia_backward_noalloc(const kia_params* p, int B, int H, int T, int d, const float* q, const float* k,
                                const float* v, const float* o, const float* d_o, const void* stats,
                                size_t stats_bytes, float* dq, float* dk, float* dv, void* stream) {
    const BwdPtrs b = {q, k, v, o, d_o, stats, stats_bytes, dq, dk, dv};
    Shape s;
    kia_status st = check_backward(p, B, H, T, d, b, &s);
    if (st != KIA_OK) return st;
    const int64_t per = slices_per_scratch(p, s);
    if (per < 1) return KIA_ERR_SCRATCH;
    void* ws = nullptr;
    if ((st = device_scratch(&ws)) != KIA_OK) return st;
    // every workspace entry is written before it is read: nothing to clear
    for (int64_t s0 = 0; s0 < s.BH; s0 += per) {
        st = run_backward(p, s, s0, std::min<int64_t>(per, s.BH - s0), b, (char*)ws, nullptr, (hipStream_t)stream);
        if (st != KIA_OK) return st;
    }
    return KIA_OK;
}

size_t kia_geometry_bytes(int B, int H, int T) {
    if (B < 1 || H < 1 || T < 1) return 0;
    const double n = (double)B * H * T * KIA_GEO_FIELDS * 4.0;
    if (n > 9.0e18) return 0;
    return (size_t)B * H * T * KIA_GEO_FIELDS * 4;
}

kia_status kia_geometry(const kia_params* p, int B, int H, int T, int d, const float* q, const float* k,
                        const void* stats, size_t stats_bytes, float* geo, size_t geo_bytes, void* stream) {
    kia_status st = check_params(p);
    if (st != KIA_OK) return st;
    Shape s;
    if ((st = check_shape(B, H, T, d, &s)) != KIA_OK) return st;
    if (!q || !k || !stats || !geo) return KIA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(stats) || !aligned16(geo)) return KIA_ERR_ALIGN;
    kia_stats_layout L;
    stats_layout(p, s, &L);
    if (stats_bytes < L.total_bytes) return KIA_ERR_BUFFER;
    if (geo_bytes < kia_geometry_bytes(B, H, T)) return KIA_ERR_BUFFER;

    const char* sb = (const char*)stats;
    kia::GeoArgs a;
    a.q = q; a.k = k;
    a.tiles = (const float*)(sb + L.scores);
    a.row_m = (const float*)(sb + L.row_m);
    a.row_w = (const float*)(sb + L.row_w);
    a.geo = geo;
    a.BH = (int)s.BH; a.T = T; a.n_t = (int)s.n_t; a.K = p->n_intervals; a.d = d;
    a.tau = p->tau;
    return kia::launch_geometry(p->calibration, p->reconstruction, a, (hipStream_t)stream) == hipSuccess
               ? KIA_OK
               : KIA_ERR_HIP;
}

kia_status kia_tiles_to_dense(int B, int H, int T, const float* tiles, int key_major, float* dense,
                              void* stream) {
    if (!tiles || !dense) return KIA_ERR_NULL;
    if (B < 1 || H < 1 || T < 1) return KIA_ERR_SHAPE;
    if (key_major != 0 && key_major != 1) return KIA_ERR_PARAM;
    const int64_t BH = (int64_t)B * H;
    if (BH > 65535) return KIA_ERR_SHAPE;  // grid.y limit of the expansion kernel
    const int64_t n_t = ((int64_t)T + 31) / 32;
    if (n_t * (n_t + 1) / 2 > INT32_MAX) return KIA_ERR_SHAPE;
    return kia::launch_tiles_to_dense((int)BH, T, tiles, key_major, dense, (hipStream_t)stream) == hipSuccess
               ? KIA_OK
               : KIA_ERR_HIP;
}

const char* kia_status_str(kia_status s) {
    switch (s) {
        case KIA_OK: return "ok";
        case KIA_ERR_NULL: return "null pointer argument";
        case KIA_ERR_SHAPE: return "unsupported shape (B, H, T >= 1; d in {64, 128})";
        case KIA_ERR_PARAM: return "invalid operator parameter";
        case KIA_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
        case KIA_ERR_BUFFER: return "stats or workspace buffer too small";
        case KIA_ERR_HIP: return "HIP launch failed";
        case KIA_ERR_SCRATCH: return "one (batch, head) slice needs more workspace than kia_backward_noalloc's scratch holds";
    }
    return "unknown status";
}

int32_t kia_abi_version(void) { return 4; }

}  // extern "C"
