/*
 * kia.h - C ABI of the K-interval attention library (libkia.so, gfx950).
 *
 * K-interval attention is the attention operator of "Pretraining Transformers
 * with Quantized Softmax in Attention" (paperlayer digest of the paper).  Per
 * causal row of scores s_j = Q_t . K_j / sqrt(d) (key t included):
 *   - a row calibration sets a grid of K+1 values exp(-j h): MinMax takes
 *     h = (max - min) / K from the row span, FWM takes h = tau / K anchored at
 *     the row max and gives zero weight below max - tau (section 3
 *     "Calibration"; App. A "Operator definitions and edge cases");
 *   - each score is reconstructed from the grid, by linear interpolation
 *     between the two grid values around it (LERP) or by the grid value it
 *     rounds to (Nearest) (section 3 "Reconstruction", Figure 1; App. A);
 *   - weights are normalised, P_j = w_j / W, and O = P V (App. A);
 *   - the backward applies the normalisation Jacobian and carries the
 *     calibration derivatives through the row max and min (full), drops them
 *     (detach) or keeps one of them (max-only / min-only); for Nearest the
 *     LERP derivative is the surrogate, with the Jacobian evaluated at the hard
 *     weights (Weight-STE) or at the LERP probabilities (Prob-STE) (section 3
 *     "Calibration gradients", "Surrogate placement"; App. B "Gradient
 *     derivations"; App. F for max-only / min-only).
 * Spans below 1e-12 take the degenerate branch (App. A, Table S1): uniform
 * weights forward, the softmax-limit gradient dS = P (dP - delta) backward.
 *
 * Conventions for every entry point:
 *   - Tensors are fp32, contiguous [B, H, T, d], d in {64, 128}; tensor
 *     pointers are DEVICE pointers, 16-byte aligned, owned by the caller.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  The
 *     library launches only on that stream, never synchronises, never
 *     allocates, and keeps no mutable global state: calls are thread-safe.
 *   - Every argument check happens before the first launch; on error nothing
 *     is launched and a non-zero kia_status is returned.  Launch failures are
 *     reported as KIA_ERR_HIP.  Output contents are unspecified on error.
 *   - Results are deterministic: no atomics; repeated calls give identical
 *     bits, and a (b, h) slice does not depend on the rest of the batch.
 */
#ifndef KIA_H
#define KIA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kia_status {
    KIA_OK = 0,
    KIA_ERR_NULL = 1,      /* a required pointer is NULL */
    KIA_ERR_SHAPE = 2,     /* B, H, T < 1, d not in {64, 128}, or sizes overflow */
    KIA_ERR_PARAM = 3,     /* flag out of range, n_intervals < 1, tau <= 0 under FWM / FWM_UNTRUNC */
    KIA_ERR_ALIGN = 4,     /* a tensor pointer is not 16-byte aligned */
    KIA_ERR_BUFFER = 5,    /* stats or workspace smaller than the size query returns */
    KIA_ERR_HIP = 6,       /* a kernel launch failed */
    KIA_ERR_SCRATCH = 7    /* kia_backward_noalloc: one (b, h) slice's workspace exceeds its scratch */
} kia_status;

enum { KIA_CAL_MINMAX = 0, KIA_CAL_FWM = 1, KIA_CAL_FWM_UNTRUNC = 2 };
enum { KIA_REC_LERP = 0, KIA_REC_NEAREST = 1, KIA_REC_EXACT = 2, KIA_REC_EXP_BF16 = 3, KIA_REC_EXP_FP8 = 4 };
/* KIA_CAL_FWM_UNTRUNC is the untruncated fixed-step operator of the paper's
 * tail-policy comparison (App. D.4): FWM's step h = tau/K anchored at the row
 * max, with the grid continued below max - tau instead of a zero tail (the
 * LERP segment and the Nearest point are unbounded; only the max carries a
 * calibration term).  KIA_REC_EXACT is the exact-softmax reference on the
 * same path (App. D.5 compares against softmax): w = exp(s - max), with the
 * calibration, tau and surrogate flags ignored; its calibration term through
 * the max vanishes up to rounding, so every rule yields the softmax
 * gradient.  KIA_REC_EXP_BF16 and KIA_REC_EXP_FP8 are the reduced-precision
 * exponential baselines (App. D.5, Table S11): the exact reference with each
 * exp(s - max) rounded to nearest (ties to even) in bf16, or in FP8 E4M3
 * (3 fraction bits, subnormal step 2^-9; the pages name no FP8 format, E4M3
 * is the forward-pass one), before normalisation.  Their backward is
 * straight-through: the rounding counts as the identity, so the direct term
 * uses the unrounded exponential with the Jacobian at the rounded P, and the
 * max carries minus the row's direct sum under full and max-only. */
enum { KIA_STE_WEIGHT = 0, KIA_STE_PROB = 1 };  /* read only for Nearest */
enum { KIA_GRAD_FULL = 0, KIA_GRAD_DETACH = 1, KIA_GRAD_MAX_ONLY = 2, KIA_GRAD_MIN_ONLY = 3, KIA_GRAD_P1 = 4 };
/* KIA_GRAD_P1 is the zero-sum projection of the detached gradient (App. B;
 * section 5.1, "P1"): dS <- dS_detach - (mean of dS_detach over the row's
 * causal keys).  Its forward is the detach forward, bit for bit. */

/* Operator flags.  n_intervals is the method's K (grid of K+1 values); it is
 * named so it cannot be mistaken for the key tensor.  tau is the FWM window
 * in nats (ignored for MinMax).  The forward never reads grad_rule, and reads
 * surrogate only to decide whether to keep the Prob-STE extras, so forwards
 * that differ only in those flags are bitwise identical.  Under FWM the row
 * min plays no role: MIN_ONLY behaves as DETACH and MAX_ONLY as FULL. */
typedef struct kia_params {
    int32_t n_intervals;     /* 1 .. 65536 */
    float tau;               /* > 0 and finite under FWM and FWM_UNTRUNC */
    int32_t calibration;     /* KIA_CAL_* */
    int32_t reconstruction;  /* KIA_REC_* */
    int32_t surrogate;       /* KIA_STE_* */
    int32_t grad_rule;       /* KIA_GRAD_* */
} kia_params;

/* Byte offsets of the forward -> backward state inside `stats`.  The forward
 * materialises every causal score once (fp32, tiles of 32 queries x 32 keys,
 * per (b, h) slice the tiles (qt, kt), kt <= qt, in order qt*(qt+1)/2 + kt);
 * the backward reads them instead of recomputing Q K^T.  Row arrays are
 * [B*H*T]: max m, min n (fp32), argmax a, argmin b (int32, smallest key index
 * on ties), normaliser W and LERP normaliser WL (fp32).  o_lerp ([B,H,T,d]
 * fp32, the LERP-probability output used by the Prob-STE backward) is present
 * only for Nearest + Prob-STE (else o_lerp == 0). */
typedef struct kia_stats_layout {
    size_t total_bytes;
    size_t scores;
    size_t row_m, row_n, row_a, row_b, row_w, row_wl;
    size_t o_lerp;
    int64_t tiles_per_head;
} kia_stats_layout;

/* Byte offsets inside the backward workspace: the hard probabilities P and
 * the score gradient dS (calibration terms included) as tiles in key-major
 * order (per (b, h): tile (qt, kt) at the same index as the score tiles), and
 * the per-row calibration terms the gradient rule routed to the argmax key
 * (cm) and the argmin key (cn), fp32 [B*H*T].  Under KIA_GRAD_P1 the dS tiles
 * hold the detached gradient, cm holds the row mean the rule subtracts from
 * it (the projected gradient is dS - cm on each row's causal keys; dQ and dK
 * include the subtraction) and cn is 0; two more sections serve as scratch
 * for the P1 sums: [B,H,T,d] fp32 (prefix_k: the causal prefix sums of K,
 * then the suffix sums of cm_t Q_t) and per-32-row chunk sums (chunk_k);
 * both offsets are 0 under the other rules. */
typedef struct kia_workspace_layout {
    size_t total_bytes;
    size_t probs;
    size_t dscores;
    size_t row_cm, row_cn;
    size_t prefix_k, chunk_k;
} kia_workspace_layout;

/* Size queries.  Return 0 on invalid arguments (same checks as the calls). */
size_t kia_stats_bytes(const kia_params* p, int B, int H, int T, int d);
size_t kia_workspace_bytes(const kia_params* p, int B, int H, int T, int d);
kia_status kia_stats_layout_query(const kia_params* p, int B, int H, int T, int d,
                                  kia_stats_layout* out);
kia_status kia_workspace_layout_query(const kia_params* p, int B, int H, int T, int d,
                                      kia_workspace_layout* out);

/* Forward: O = P V with P the normalised K-interval weights (App. A).
 * q, k, v: inputs [B,H,T,d]; o: output [B,H,T,d]; stats: output, at least
 * kia_stats_bytes(...) bytes, read by kia_backward with the same p and shape. */
kia_status kia_forward(const kia_params* p, int B, int H, int T, int d,
                       const float* q, const float* k, const float* v, float* o,
                       void* stats, size_t stats_bytes, void* stream);

/* Backward: dQ, dK, dV of sum(dO * O) under p's gradient rule and surrogate
 * placement (section 3; App. B).  o and stats must come from kia_forward with
 * the same q, k, v, p and shape.  ws: scratch of kia_workspace_bytes(...)
 * bytes; on return it holds the tiles and row terms kia_workspace_layout
 * describes.  dq, dk, dv: outputs [B,H,T,d].
 * Where the row's grid has at most 32 intervals (MinMax or FWM under LERP or
 * Nearest), the backward reads each score's grid value from a per-row table
 * of the K+1 values instead of evaluating an exponential per score; the
 * environment variable KIA_GRID_TABLE=0 (read at each call) selects the
 * per-score exponential, with bitwise the same results. */
kia_status kia_backward(const kia_params* p, int B, int H, int T, int d,
                        const float* q, const float* k, const float* v,
                        const float* o, const float* d_o,
                        const void* stats, size_t stats_bytes,
                        float* dq, float* dk, float* dv,
                        void* ws, size_t ws_bytes, void* stream);

/* Backward without any allocation, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  The same computation and results as kia_backward, with
 * the workspace taken from a static device array the library holds on each
 * device it runs on: KIA_NOALLOC_SCRATCH_MIB MiB per device, kept until the
 * process ends.  Batches whose workspace exceeds it run in consecutive
 * groups of (b, h) slices on `stream`; a shape whose single slice needs more
 * than the scratch (e.g. T = 8192 at any d) returns KIA_ERR_SCRATCH before
 * any launch.  The call allocates nothing (no hipMalloc, no library
 * allocation); the first call on a device looks the array up once.  Every
 * call on one device shares that device's array: calls that overlap in time
 * on one device (other streams, other threads) race and give undefined
 * results.  Arguments and the other errors are those of kia_backward. */
#define KIA_NOALLOC_SCRATCH_MIB 256
kia_status kia_backward_noalloc(const kia_params* p, int B, int H, int T, int d,
                                const float* q, const float* k, const float* v,
                                const float* o, const float* d_o,
                                const void* stats, size_t stats_bytes,
                                float* dq, float* dk, float* dv, void* stream);

/* Optional extras for the two calls above.  events: NULL or an array of
 * hipEvent_t (as void*) recorded on `stream` around each kernel: forward
 * uses 2 (start/end of its one kernel), backward 4 (around its two kernels,
 * in launch order; under KIA_GRAD_P1 the first interval also covers the
 * launches of the key prefix sums and of the query suffix sums).  idx_dump (forward only): NULL
 * or int32 [B,H,T,T]; for every causal pair the kernel writes the grid index
 * it used (the LERP segment, or the Nearest grid point), -1 for keys outside
 * the FWM window; 0 under KIA_REC_EXACT (no grid); under the rounded
 * baselines the fp32 bit pattern of the rounded exponential, i.e. which of
 * the format's values the rounding chose; non-causal entries are left
 * untouched. */
typedef struct kia_ext {
    void* const* events;
    int32_t n_events;
    int32_t* idx_dump;
} kia_ext;

kia_status kia_forward_ext(const kia_params* p, int B, int H, int T, int d,
                           const float* q, const float* k, const float* v, float* o,
                           void* stats, size_t stats_bytes, void* stream, const kia_ext* ext);
kia_status kia_backward_ext(const kia_params* p, int B, int H, int T, int d,
                            const float* q, const float* k, const float* v,
                            const float* o, const float* d_o,
                            const void* stats, size_t stats_bytes,
                            float* dq, float* dk, float* dv,
                            void* ws, size_t ws_bytes, void* stream, const kia_ext* ext);

/* Score-geometry probe ("Pretraining Transformers with Quantized Softmax in
 * Attention", section 4 "Geometry probe"; section 5.4; App. D.6): per causal
 * row, statistics of the learned scores and of the operator's distortion of
 * the softmax, reduced from the score tiles a kia_forward call with the same
 * params and shape left in `stats` (q and k are that call's inputs; `stats`
 * is only read).  `geo` (device, fp32, 16-byte aligned, caller-owned, at least
 * kia_geometry_bytes(B, H, T) bytes) receives KIA_GEO_FIELDS arrays of B*H*T
 * values, field f of row (b, h, t) at geo[f * B*H*T + (b*H + h)*T + t]:
 *   SPAN      max - min of the row's scores
 *   WIDTH     the interval width h the operator lays on the row (MinMax
 *             span/K, 0 on rows below the degenerate span; FWM and
 *             FWM_UNTRUNC tau/K; under KIA_REC_EXACT and the rounded
 *             baselines the MinMax width span/K)
 *   Q_NORM    |Q_t|, K_NORM |K_t| (unscaled projections at position t)
 *   ENTROPY_P entropy (nats) of the operator's probabilities P
 *   ENTROPY_S entropy of the softmax of the same scores
 *   TV        total variation (1/2) sum_j |P_j - softmax_j|
 *   TOP_MASS  softmax mass of the top rounding bucket: keys whose Nearest
 *             point on that grid is 0, i.e. u = (max - s)/h < 1/2 (every key
 *             when the width is 0).
 * Reductions accumulate in fp32 within a 32-key tile and in fp64 across
 * tiles.  Errors as for kia_forward; KIA_ERR_BUFFER if `geo_bytes` is short.
 * Nothing is written for padding rows. */
enum {
    KIA_GEO_SPAN = 0, KIA_GEO_WIDTH = 1, KIA_GEO_Q_NORM = 2, KIA_GEO_K_NORM = 3,
    KIA_GEO_ENTROPY_P = 4, KIA_GEO_ENTROPY_S = 5, KIA_GEO_TV = 6, KIA_GEO_TOP_MASS = 7,
    KIA_GEO_FIELDS = 8
};
size_t kia_geometry_bytes(int B, int H, int T);
kia_status kia_geometry(const kia_params* p, int B, int H, int T, int d, const float* q, const float* k,
                        const void* stats, size_t stats_bytes, float* geo, size_t geo_bytes, void* stream);

/* Expand a tile buffer (scores from stats, or probs / dscores from the
 * workspace) into a dense fp32 [B,H,T,T] matrix for inspection.  key_major:
 * 0 for the score tiles, 1 for the workspace tiles.  Only causal entries are
 * written.  Device pointers; launches on `stream`. */
kia_status kia_tiles_to_dense(int B, int H, int T, const float* tiles, int key_major,
                              float* dense, void* stream);

const char* kia_status_str(kia_status s);
int32_t kia_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KIA_H */
