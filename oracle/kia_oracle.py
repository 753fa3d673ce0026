"""K-interval attention: plain fp64 CPU oracle.

TEST INFRASTRUCTURE ONLY.  Only the test suite, smoke() in __graft_entry__.py
and the benchmark's CPU-baseline leg may import or run this file.  It shares no code, constant table or helper with the HIP library, and
the library never calls it.

What it computes follows "Pretraining Transformers with Quantized Softmax in
Attention" (paperlayer digest of the paper):

* Operator family (section 3, "Operator family"; App. A "Operator definitions
  and edge cases"): per causal row of scores, a row calibration sets K+1 grid
  values exp(-j h); each score is reconstructed from the grid (LERP or
  Nearest), the reconstructed weights are normalised, P_j = w_j / W, and
  O = P V.  Future positions get no weight; the row is shifted by its maximum
  before exponentiation.
* Calibration (section 3 "Calibration"; App. A): MinMax takes h = (max-min)/K
  from the row span; FWM takes h = tau/K anchored at the row maximum and gives
  zero weight below max - tau.  Spans below eps = 1e-12 take a separate branch.
* Reconstruction (section 3 "Reconstruction", Figure 1; App. A): LERP
  interpolates linearly between the two grid values around a score; Nearest
  gives every score the grid value it rounds to, so one bin shares one weight.
* Gradients (section 3 "Calibration gradients", "Surrogate placement";
  App. B "Gradient derivations"): the normalisation Jacobian turns dL/dP into
  dL/dw; the full calibration gradient differentiates through the shifted
  scores, the grid values and h, i.e. through the row max and min, and its
  per-key partials sum to zero; detach drops the extremum terms; max-only and
  min-only keep one of them (App. F).  Nearest uses the LERP derivative as its
  surrogate; Weight-STE evaluates the normalisation Jacobian at the hard
  weights, Prob-STE at the LERP probabilities and normaliser.

Readings where the pages leave a step open:
  R1  Nearest rounds to the nearest grid point j*h (K+1 levels); a score
      exactly half-way rounds up in u, i.e. r = floor(u + 1/2).
  R2  LERP uses segment i = min(floor(u), K-1): at a knot the right-hand
      segment's derivative is used, the row minimum (u = K) uses segment K-1.
  R3  Ties for the row max / min: the smallest key index is the extremum.
  R4  Spans below eps: w = 1 for every causal key (uniform P); the backward is
      the h -> 0 limit dS = P (dP - delta) with no calibration terms.
  R5  Under FWM a key is in the window iff s >= max - tau (u <= K).
  R6  detach holds m (as the shift and inside h) and n constant; max-only
      holds n constant; min-only holds m constant.  Under FWM the min plays
      no role, so min-only equals detach and max-only equals full.
  R7  Scores are Q.K / sqrt(d); key t is causal for query t.
  R8  P1 (zero-sum projection of the detached gradient, App. B; section 5.1):
      dS <- dS_detach - mean over the row's causal keys.
  R11 The untruncated fixed-step operator (App. D.4, "tail policy"): FWM's
      step h = tau/K anchored at the max, with the grid continued below
      max - tau instead of a zero tail: LERP segment i = floor(u) and Nearest
      point r = floor(u + 1/2) without an upper bound, so every causal key
      keeps a nonzero weight.  Only the max carries a calibration term (h is
      fixed).
  R12 The exact-softmax reference on the same path (App. D.5 compares the
      operator against softmax): w = exp(s - m); the calibration and
      surrogate flags are ignored; its calibration term through m vanishes
      up to rounding, so every rule gives the softmax gradient P (dP - delta).
  R14 The reduced-precision exponential baselines (App. D.5, Table S11):
      exact softmax with each exp(s - m) rounded, before normalisation, to
      bf16 (BF16-exp) or to FP8 (FP8-exp), round to nearest, ties to even.
      The pages do not name the FP8 format; the forward-pass format E4M3
      (OCP: 3 fraction bits, exponent bias 7, subnormal step 2^-9) is taken.
      The backward is straight-through: the rounding counts as the identity,
      so dS_direct = gt * exp(s - m) with gt = (dP - delta)/W evaluated at the
      rounded P and W; the shift m carries -sum(dS_direct) to the argmax under
      full and max-only.  The calibration, tau and surrogate flags are
      ignored, as for the exact reference.
  R13 The geometry probe (section 4 "Geometry probe"; section 5.4; App. D.6)
      reports per causal row: the span max - min; the native width, i.e. the
      interval width h the operator lays on the row (MinMax span/K, 0 in the
      degenerate branch; FWM and the untruncated step tau/K; the exact
      reference has no grid of its own and reports the MinMax width of the
      given K, and so do the rounded-exponential baselines); the norms |Q_t| and |K_t| of the unscaled projections; the
      entropies (nats) of the operator's forward probabilities P and of the
      softmax of the same scores; their total variation (1/2) sum |P - softmax|;
      and the softmax mass of the top rounding bucket, the keys whose Nearest
      point on that grid is 0 (u = (m - s)/h < 1/2; every key when h = 0).
  R15 Scores are formed key by key as an fp64 sum over the head dimension in
      index order (not a library matrix product, whose blocking may differ
      between keys), so keys with equal vectors score exactly equal and the
      tie rule R3 applies to them.
  R16 Decisions (LERP segment, Nearest point, FWM window edge, the rounding
      direction of a rounded exponential) may be supplied per key instead of
      taken from u (the `decisions` argument): the pages define each decision
      on the real-valued u, and where two finite-precision evaluations of u
      fall on either side of a boundary both decisions read the pages
      correctly.  Tests use this only with decisions they have shown to be
      admissible for that key; with no override the oracle decides itself.

Parity: every function below is pinned by the CPU tests (closed forms,
brute force, finite differences, an autograd re-expression, the softmax
limit, the zero-sum identity; the whole-tensor forward / backward against the
per-head functions on slices that all differ, with planted index swaps; the
per-key decision override against closed forms); none is "parity unpinned".
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

MINMAX, FWM, FWM_UNTRUNC = 0, 1, 2
LERP, NEAREST, EXACT, EXP_BF16, EXP_FP8 = 0, 1, 2, 3, 4
EXP_FAMILY = (EXACT, EXP_BF16, EXP_FP8)   # softmax anchored at the max, no grid
WEIGHT_STE, PROB_STE = 0, 1
FULL, DETACH, MAX_ONLY, MIN_ONLY, P1 = 0, 1, 2, 3, 4

EPS_SPAN = 1e-12  # App. A: branches for spans above / below 1e-12


@dataclass(frozen=True)
class Params:
    K: int                     # number of intervals; the grid has K+1 values
    tau: float = 6.0           # FWM window in nats
    calibration: int = MINMAX
    reconstruction: int = LERP
    surrogate: int = WEIGHT_STE
    grad_rule: int = FULL

    def carries_max(self) -> bool:
        return self.grad_rule in (FULL, MAX_ONLY)

    def carries_min(self) -> bool:
        return (self.grad_rule in (FULL, MIN_ONLY) and self.calibration == MINMAX
                and self.reconstruction not in EXP_FAMILY)


# ---------------------------------------------------------------------------
# one causal row
# ---------------------------------------------------------------------------

def row_scores(q_t: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """s_j = Q_t . K_j / sqrt(d) over the causal keys (reading R7).

    Each key's dot product is summed by itself, in the same order for every
    key (not by a matrix-vector product, whose blocking can round equal rows
    differently), so equal keys get bitwise-equal scores and the lowest-index
    tie rule (R3) applies to them."""
    d = keys.shape[1]
    return (keys.astype(np.float64) * q_t.astype(np.float64)).sum(axis=1) / np.sqrt(d)


@dataclass
class Calibration:
    m: float          # row max
    a: int            # its key (smallest index on ties, R3)
    n: float          # row min
    b: int
    h: float          # grid width (0 in the degenerate branch)
    degenerate: bool  # MinMax span below eps (R4)


def calibrate(s: np.ndarray, p: Params) -> Calibration:
    """Row calibration: MinMax h = span/K, FWM h = tau/K (section 3; App. A).
    The untruncated fixed step (App. D.4) uses FWM's h = tau/K; the exact
    softmax reference uses only the max (its h is unused)."""
    a = int(np.argmax(s))   # numpy returns the first maximal index
    b = int(np.argmin(s))
    m, n = float(s[a]), float(s[b])
    if p.calibration == MINMAX and p.reconstruction not in EXP_FAMILY:
        span = m - n
        if span < EPS_SPAN:
            return Calibration(m, a, n, b, 0.0, True)
        return Calibration(m, a, n, b, span / p.K, False)
    return Calibration(m, a, n, b, p.tau / p.K, False)


def grid(h: float, K: int) -> np.ndarray:
    """The K+1 grid values exp(-j h), j = 0..K."""
    return np.exp(-h * np.arange(K + 1, dtype=np.float64))


@dataclass
class Recon:
    """Per-key reconstruction state of one row."""
    u: np.ndarray      # (m - s)/h, distance below the max in grid steps
    uc: np.ndarray     # u clamped to K (rounding guard, not differentiated; unclamped untruncated)
    mask: np.ndarray   # 1 in the window (always 1 for MinMax and the untruncated step)
    i: np.ndarray      # LERP segment
    f: np.ndarray      # position inside the segment
    r: np.ndarray      # Nearest grid point
    g: np.ndarray      # the grid values exp(-j h), j = 0..K
    gi: np.ndarray     # exp(-i h) at each key's segment start
    gi1: np.ndarray    # exp(-(i+1) h) at its end
    wL: np.ndarray     # LERP weights
    wN: np.ndarray     # Nearest weights


def reconstruct(s: np.ndarray, m: float, h: float, p: Params, clamp: bool = True,
                decisions: dict | None = None) -> Recon:
    """Grid reconstruction of a row (section 3 "Reconstruction"; App. A).

    ``clamp=False`` keeps u unclamped and lets the end segments extend
    linearly; it exists for derivative checks that move a score past the row
    extremes while the extremes are held fixed.

    ``decisions`` (test use) maps a key index to the integer decision taken
    for it instead of rounding this row's own u: the LERP segment i (LERP) or
    the Nearest point r (Nearest), or -1 for "outside the FWM window".  A
    decision that is taken in floating point (floor, the window test) can go
    either way for a key whose u lies within rounding of the boundary; this
    evaluates the same operator, in fp64 from the same u, on the other side.
    """
    K = p.K
    u = (m - s) / h
    if p.calibration == FWM:
        mask = (u <= K).astype(np.float64)                     # R5
    else:
        mask = np.ones_like(u)
    g = grid(h, K)
    if p.calibration == FWM_UNTRUNC:
        # the grid continues below max - tau (App. D.4): no clamp, no tail mask (R11)
        uc = u.copy()
        i = np.maximum(np.floor(uc), 0).astype(np.int64)
        r = np.maximum(np.floor(uc + 0.5), 0).astype(np.int64)
    else:
        uc = np.minimum(u, float(K)) if clamp else u.copy()
        i = np.clip(np.floor(uc), 0, K - 1).astype(np.int64)      # R2
        r = np.clip(np.floor(uc + 0.5), 0, K).astype(np.int64)    # R1
    for j, level in (decisions or {}).items():
        if level < 0:
            mask[j] = 0.0
            continue
        if p.calibration == FWM:
            mask[j] = 1.0
        if p.reconstruction == LERP:
            i[j] = level
        else:
            r[j] = level
    f = uc - i
    gi, gi1 = np.exp(-h * i), np.exp(-h * (i + 1))
    wL = mask * ((1.0 - f) * gi + f * gi1)                      # linear interpolation
    wN = mask * np.exp(-h * r)
    return Recon(u, uc, mask, i, f, r, g, gi, gi1, wL, wN)


def round_to_format(x: np.ndarray, frac_bits: int, emin: int) -> np.ndarray:
    """Round non-negative values to nearest, ties to even, in a binary
    floating-point format with `frac_bits` fraction bits and smallest normal
    exponent `emin` (gradual underflow below 2^emin; the values rounded here
    are at most 1, so the format's top end never matters).  bf16: 7, -126;
    FP8 E4M3: 3, -6 (R14)."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                        # x = f 2^e with f in [1/2, 1)
    quantum = np.ldexp(1.0, np.maximum(e - 1, emin) - frac_bits)
    return np.rint(x / quantum) * quantum      # np.rint rounds ties to even


FORMATS = {EXP_BF16: (7, -126), EXP_FP8: (3, -6)}


@dataclass
class RowForward:
    s: np.ndarray
    cal: Calibration
    rec: Recon | None
    w: np.ndarray       # forward weights (hard for Nearest)
    W: float
    P: np.ndarray
    wL: np.ndarray      # LERP weights (= w for LERP)
    WL: float


def format_neighbours(x: np.ndarray, frac_bits: int, emin: int):
    """The two adjacent values of the format that bracket each x >= 0 (lower,
    upper; equal when x is representable), with the same quantum as
    round_to_format."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    quantum = np.ldexp(1.0, np.maximum(e - 1, emin) - frac_bits)
    lo = np.floor(x / quantum) * quantum
    hi = np.ceil(x / quantum) * quantum
    return lo, hi


def row_forward(s: np.ndarray, p: Params, decisions: dict | None = None) -> RowForward:
    """Forward of one causal row.  ``decisions`` (test use) fixes the integer
    decisions at the listed keys: grid operators as in reconstruct; for the
    rounded exponentials 1 takes the format value above exp(s - m) and 0 the
    one below, instead of rounding to the nearer."""
    cal = calibrate(s, p)
    if p.reconstruction in EXP_FAMILY:                         # R12, R14: softmax
        w = np.exp(s - cal.m)
        if p.reconstruction in FORMATS:
            e = w
            w = round_to_format(e, *FORMATS[p.reconstruction])
            if decisions:
                lo, hi = format_neighbours(e, *FORMATS[p.reconstruction])
                for j, up in decisions.items():
                    w[j] = hi[j] if up else lo[j]
        W = float(w.sum())
        return RowForward(s, cal, None, w, W, w / W, w, W)
    if cal.degenerate:                                          # R4
        w = np.ones_like(s)
        W = float(w.sum())
        return RowForward(s, cal, None, w, W, w / W, w, W)
    rec = reconstruct(s, cal.m, cal.h, p, decisions=decisions)
    w = rec.wL if p.reconstruction == LERP else rec.wN          # Nearest computed directly
    W = float(w.sum())
    WL = float(rec.wL.sum())
    return RowForward(s, cal, rec, w, W, w / W, rec.wL, WL)


@dataclass
class RowBackward:
    dS: np.ndarray      # dL/ds over the causal keys, calibration terms included
    dS_direct: np.ndarray
    gt: np.ndarray      # dL/dw at the evaluation point
    Cm: float           # calibration sum routed to the argmax key
    Cn: float           # calibration sum routed to the argmin key
    delta: float
    We: float


def row_backward(fw: RowForward, dP: np.ndarray, p: Params) -> RowBackward:
    """Score gradient of one row given dP_j = dO_t . V_j (App. B)."""
    cal, rec = fw.cal, fw.rec
    if p.reconstruction in EXP_FAMILY:                         # R12, R14
        delta = float(np.dot(fw.P, dP))
        gt = (dP - delta) / fw.W
        e = np.exp(fw.s - cal.m)                                # straight through any rounding
        dS_direct = gt * e                                      # d exp(s - m) / ds
        Cm = -float(np.sum(gt * e))                             # through the shift m
        dS = dS_direct.copy()
        if p.grad_rule == P1:
            dS = dS - dS.mean()
        elif p.carries_max():
            dS[cal.a] += Cm
        return RowBackward(dS, dS_direct, gt, Cm, 0.0, delta, fw.W)
    if cal.degenerate:                                          # R4: softmax limit
        delta = float(np.dot(fw.P, dP))
        dS = fw.P * (dP - delta)
        gt = (dP - delta) / fw.W
        return RowBackward(dS, dS.copy(), gt, 0.0, 0.0, delta, fw.W)

    # Evaluation point of the normalisation Jacobian (section 3 "Surrogate placement")
    if p.reconstruction == NEAREST and p.surrogate == PROB_STE:
        Pe, We = rec.wL / fw.WL, fw.WL
    else:
        Pe, We = fw.P, fw.W
    delta = float(np.dot(Pe, dP))
    gt = (dP - delta) / We                                      # dL/dw_j

    # LERP derivatives (the surrogate for Nearest), zero outside the window
    gi, gi1, i, f, h, K = rec.gi, rec.gi1, rec.i, rec.f, cal.h, p.K
    dw_du = rec.mask * (gi1 - gi)
    dw_dh = rec.mask * ((1.0 - f) * (-i * gi) + f * (-(i + 1) * gi1))
    du_ds = -1.0 / h
    du_dm = 1.0 / h
    du_dh = -rec.uc / h
    dw_dh_total = dw_du * du_dh + dw_dh          # w's dependence on h at fixed s and m

    dS_direct = gt * dw_du * du_ds
    if p.calibration == MINMAX:
        dh_dm, dh_dn = 1.0 / K, -1.0 / K
        Cm = float(np.sum(gt * (dw_du * du_dm + dw_dh_total * dh_dm)))
        Cn = float(np.sum(gt * dw_dh_total * dh_dn))
    else:
        Cm = float(np.sum(gt * dw_du * du_dm))
        Cn = 0.0

    dS = dS_direct.copy()
    if p.grad_rule == P1:                                       # R8
        dS = dS - dS.mean()
    else:
        if p.carries_max():
            dS[cal.a] += Cm
        if p.carries_min():
            dS[cal.b] += Cn
    return RowBackward(dS, dS_direct, gt, Cm, Cn, delta, We)


# ---------------------------------------------------------------------------
# one (batch, head) slice
# ---------------------------------------------------------------------------

def head_forward(Q, Kt, V, p: Params, rows=None):
    """Forward over one head: Q, K, V are [T, d].  Returns a dict with O
    ([T, d], rows not asked for are NaN), the row statistics, and the
    per-row records of the rows asked for (``rows`` None means all)."""
    T, d = Q.shape
    rows = range(T) if rows is None else rows
    O = np.full((T, d), np.nan)
    st = {k: np.full(T, np.nan) for k in ("m", "n", "h", "W", "WL")}
    st["a"] = np.full(T, -1, dtype=np.int64)
    st["b"] = np.full(T, -1, dtype=np.int64)
    st["degenerate"] = np.zeros(T, dtype=bool)
    recs = {}
    V64 = V.astype(np.float64)
    for t in rows:
        s = row_scores(Q[t], Kt[: t + 1])
        fw = row_forward(s, p)
        O[t] = fw.P @ V64[: t + 1]
        c = fw.cal
        st["m"][t], st["n"][t], st["h"][t] = c.m, c.n, c.h
        st["a"][t], st["b"][t], st["degenerate"][t] = c.a, c.b, c.degenerate
        st["W"][t], st["WL"][t] = fw.W, fw.WL
        recs[t] = fw
    return {"O": O, "stats": st, "rows": recs}


def head_backward(Q, Kt, V, dO, p: Params, keep_rows: bool = False):
    """Forward + backward over one head.  Returns dQ, dK, dV ([T, d]) and
    per-row Cm, Cn, the row sum and L1 norm of dS; ``keep_rows`` also returns
    the per-row forward/backward records."""
    T, d = Q.shape
    scale = 1.0 / np.sqrt(d)
    Q64, K64, V64, dO64 = (x.astype(np.float64) for x in (Q, Kt, V, dO))
    dQ = np.zeros((T, d))
    dK = np.zeros((T, d))
    dV = np.zeros((T, d))
    Cm = np.zeros(T)
    Cn = np.zeros(T)
    dS_sum = np.zeros(T)
    dS_l1 = np.zeros(T)
    recs = {}
    for t in range(T):
        s = row_scores(Q64[t], K64[: t + 1])
        fw = row_forward(s, p)
        dP = V64[: t + 1] @ dO64[t]
        bw = row_backward(fw, dP, p)
        dQ[t] = (bw.dS @ K64[: t + 1]) * scale
        dK[: t + 1] += np.outer(bw.dS, Q64[t]) * scale
        dV[: t + 1] += np.outer(fw.P, dO64[t])               # forward (hard) P
        Cm[t], Cn[t] = bw.Cm, bw.Cn
        dS_sum[t] = bw.dS.sum()
        dS_l1[t] = np.abs(bw.dS).sum()
        if keep_rows:
            recs[t] = (fw, bw)
    out = {"dQ": dQ, "dK": dK, "dV": dV, "Cm": Cm, "Cn": Cn,
           "dS_sum": dS_sum, "dS_l1": dS_l1}
    if keep_rows:
        out["rows"] = recs
    return out


# ---------------------------------------------------------------------------
# whole [B, H, T, d] tensors
# ---------------------------------------------------------------------------

def forward(q, k, v, p: Params):
    """O and row statistics for [B, H, T, d] inputs."""
    B, H, T, d = q.shape
    O = np.zeros((B, H, T, d))
    stats = None
    for bi in range(B):
        for hi in range(H):
            r = head_forward(q[bi, hi], k[bi, hi], v[bi, hi], p)
            O[bi, hi] = r["O"]
            if stats is None:
                stats = {key: np.zeros((B, H, T), dtype=val.dtype) for key, val in r["stats"].items()}
            for key, val in r["stats"].items():
                stats[key][bi, hi] = val
    return O, stats


def backward(q, k, v, do, p: Params):
    """dQ, dK, dV for [B, H, T, d] inputs, plus per-row calibration sums."""
    B, H, T, d = q.shape
    out = {key: np.zeros((B, H, T, d)) for key in ("dQ", "dK", "dV")}
    for key in ("Cm", "Cn", "dS_sum", "dS_l1"):
        out[key] = np.zeros((B, H, T))
    for bi in range(B):
        for hi in range(H):
            r = head_backward(q[bi, hi], k[bi, hi], v[bi, hi], do[bi, hi], p)
            for key in out:
                out[key][bi, hi] = r[key]
    return out


# ---------------------------------------------------------------------------
# geometry probe (reading R13)
# ---------------------------------------------------------------------------

@dataclass
class RowGeometry:
    span: float          # max - min over the causal keys
    h: float             # native width: the operator's interval width
    entropy_p: float     # entropy of the operator's probabilities (nats)
    entropy_soft: float  # entropy of the softmax of the same scores
    tv: float            # total variation between the two
    top_mass: float      # softmax mass whose Nearest point on the grid is 0


GEOMETRY_FIELDS = ("span", "h", "q_norm", "k_norm", "entropy_p", "entropy_soft", "tv", "top_mass")


def _entropy(P: np.ndarray) -> float:
    nz = P[P > 0]
    return float(-(nz * np.log(nz)).sum())


def row_geometry(s: np.ndarray, p: Params) -> RowGeometry:
    """Score geometry of one causal row (section 4 "Geometry probe";
    section 5.4; App. D.6; reading R13)."""
    fw = row_forward(s, p)
    m, n = float(s.max()), float(s.min())
    span = m - n
    if p.calibration in (FWM, FWM_UNTRUNC) and p.reconstruction not in EXP_FAMILY:
        h = p.tau / p.K
    else:
        h = span / p.K if span >= EPS_SPAN else 0.0
    e = np.exp(s - m)
    soft = e / e.sum()
    if h > 0:
        top = (m - s) / h < 0.5
    else:
        top = np.ones(s.shape, dtype=bool)
    return RowGeometry(
        span=span,
        h=h,
        entropy_p=_entropy(fw.P),
        entropy_soft=_entropy(soft),
        tv=0.5 * float(np.abs(fw.P - soft).sum()),
        top_mass=float(soft[top].sum()),
    )


def head_geometry(Q, Kt, p: Params, rows=None):
    """Geometry probe over one head ([T, d] inputs): a dict of [T] arrays
    named by GEOMETRY_FIELDS (rows not asked for are NaN)."""
    T, d = Q.shape
    rows = range(T) if rows is None else rows
    out = {f: np.full(T, np.nan) for f in GEOMETRY_FIELDS}
    Q64, K64 = Q.astype(np.float64), Kt.astype(np.float64)
    for t in rows:
        g = row_geometry(row_scores(Q64[t], K64[: t + 1]), p)
        out["span"][t], out["h"][t] = g.span, g.h
        out["q_norm"][t] = np.sqrt((Q64[t] ** 2).sum())
        out["k_norm"][t] = np.sqrt((K64[t] ** 2).sum())
        out["entropy_p"][t], out["entropy_soft"][t] = g.entropy_p, g.entropy_soft
        out["tv"][t], out["top_mass"][t] = g.tv, g.top_mass
    return out


def geometry(q, k, p: Params):
    """Geometry probe over [B, H, T, d] inputs: a dict of [B, H, T] arrays."""
    B, H, T, d = q.shape
    out = {f: np.zeros((B, H, T)) for f in GEOMETRY_FIELDS}
    for bi in range(B):
        for hi in range(H):
            r = head_geometry(q[bi, hi], k[bi, hi], p)
            for f in GEOMETRY_FIELDS:
                out[f][bi, hi] = r[f]
    return out
