"""GPU-vs-oracle comparison machinery for the parity tests.

The HIP library is called through its C ABI (the ctypes binding); the oracle
runs on the CPU in fp64 on the same fp32 inputs.  Nothing computed by the GPU
is fed to the oracle as a value.

Decisions (LERP segment, Nearest grid point, FWM window edge, rounding
direction of the rounded exponentials, row argmax / argmin) are integers
decided by floating point.  The kernel decides them on its fp32 scores, the
oracle on fp64 scores, so a decision can legitimately differ when the
oracle's u = (m - s)/h sits closer to a boundary than the two sides' u can
differ.  That difference is bounded per pair by
  |u_gpu_inputs - u_ref| + 4 * 2^-24 * (u_ref + 1)
where u_gpu_inputs is (m - s)/h evaluated exactly on the GPU's own fp32
scores and row max / min (its scores are first checked against the a-priori
fp32 dot-product bound), and the second term covers the fp32 rounding of the
kernel's subtraction, reciprocal and product.  Pairs inside twice that band
are "ambiguous": both decisions are admissible.  With the kernel's index dump
the test checks that the kernel took one of the two and evaluates the oracle
row with that one (SliceCheck), so every output is compared; every decision
outside the band must match the oracle's exactly.
"""
from __future__ import annotations

import numpy as np

import oracle as O

TOL = 1e-4          # max error relative to the slice's max |reference| (fp32 path)
ZERO_SUM_TOL = 1e-5


def to_oracle_params(p):
    cal = {"minmax": O.MINMAX, "fwm": O.FWM, "fwm_untrunc": O.FWM_UNTRUNC}[p.calibration]
    rec = {"lerp": O.LERP, "nearest": O.NEAREST, "exact": O.EXACT, "exp_bf16": O.EXP_BF16,
           "exp_fp8": O.EXP_FP8}[p.reconstruction]
    ste = {"weight": O.WEIGHT_STE, "prob": O.PROB_STE}[p.surrogate]
    rule = {"full": O.FULL, "detach": O.DETACH, "max_only": O.MAX_ONLY, "min_only": O.MIN_ONLY,
            "p1": O.P1}[p.grad_rule]
    return O.Params(K=p.K, tau=p.tau, calibration=cal, reconstruction=rec, surrogate=ste, grad_rule=rule)


def run_gpu(q, k, v, do, params, want_dense=True, want_idx=True):
    """Run kia_forward / kia_backward on cuda:0.  Returns a dict of device
    tensors; SliceCheck copies out the (b, h) slices it needs."""
    import torch
    import quantized_softmax_attention_amd as kia

    dev = torch.device("cuda:0")
    tq, tk, tv, tdo = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (q, k, v, do))
    B, H, T, d = q.shape
    idx = None
    if want_idx:
        idx = torch.full((B, H, T, T), -7, dtype=torch.int32, device=dev)
    o, stats = kia.kia_forward(tq, tk, tv, params, idx_dump=idx)
    dq, dk, dv, ws = kia.kia_backward(tq, tk, tv, o, tdo, stats, params)
    L = kia.kia_stats_layout_query(params, B, H, T, d)
    WL = kia.kia_workspace_layout_query(params, B, H, T, d)
    n = B * H * T

    def rows(buf, off, dtype):
        return buf[off: off + n * 4].view(dtype).reshape(B, H, T)

    out = {
        "O": o, "dQ": dq, "dK": dk, "dV": dv,
        "m": rows(stats, L.row_m, torch.float32), "n": rows(stats, L.row_n, torch.float32),
        "a": rows(stats, L.row_a, torch.int32), "b": rows(stats, L.row_b, torch.int32),
        "W": rows(stats, L.row_w, torch.float32), "WL": rows(stats, L.row_wl, torch.float32),
        "cm": rows(ws, WL.row_cm, torch.float32), "cn": rows(ws, WL.row_cn, torch.float32),
        "_stats": stats, "_ws": ws,
    }
    if want_dense:
        out["S"] = kia.kia_tiles_to_dense(B, H, T, stats[L.scores:], False)
        out["P"] = kia.kia_tiles_to_dense(B, H, T, ws[WL.probs:], True)
        out["dS"] = kia.kia_tiles_to_dense(B, H, T, ws[WL.dscores:], True)
    if want_idx:
        out["idx"] = idx
    torch.cuda.synchronize()
    return out


def gpu_slice(gpu, b, h, rows=None):
    """numpy copies of every per-slice entry of a run_gpu result; the [T, T]
    entries only for the rows asked for (other rows left zero)."""
    out = {}
    for key, val in gpu.items():
        if key.startswith("_"):
            continue
        x = val[b, h]
        if rows is not None and x.dim() == 2 and x.shape[0] == x.shape[1]:
            import torch
            idx = torch.as_tensor(rows, device=x.device)
            dense = np.zeros(tuple(x.shape), dtype=np.int32 if x.dtype == torch.int32 else np.float32)
            dense[rows] = x.index_select(0, idx).cpu().numpy()
            out[key] = dense
        else:
            out[key] = x.cpu().numpy()
    return out


def score_bound(Qh, Kh):
    """A-priori bound on |fp32 score - exact score| per pair: a length-d fp32
    dot product, the scale applied to Q and the final rounding,
    (d + 3) * 2^-24 * sum_c |Q_c K_c| / sqrt(d)."""
    d = Qh.shape[1]
    absdot = np.abs(Qh.astype(np.float64)) @ np.abs(Kh.astype(np.float64)).T / np.sqrt(d)
    return (d + 3) * 2.0 ** -24 * absdot


def partial_head_backward(Qh, Kh, Vh, dOh, p_or, rows, tail):
    """The oracle's per-row forward + backward for the rows asked for, with dK
    and dV accumulated over the rows t >= tail only: exact for keys >= tail
    (every row that reaches such a key is >= tail), so long sequences can be
    checked on their last keys without the whole quadratic slice."""
    T, d = Qh.shape
    scale = 1.0 / np.sqrt(d)
    Q64, K64, V64, dO64 = (x.astype(np.float64) for x in (Qh, Kh, Vh, dOh))
    dQ = np.full((T, d), np.nan)
    dK = np.zeros((T, d))
    dV = np.zeros((T, d))
    recs = {}
    for t in sorted(set(rows) | set(range(tail, T))):
        s = O.row_scores(Q64[t], K64[: t + 1])
        fw = O.row_forward(s, p_or)
        bw = O.row_backward(fw, V64[: t + 1] @ dO64[t], p_or)
        dQ[t] = (bw.dS @ K64[: t + 1]) * scale
        if t >= tail:
            dK[tail: t + 1] += np.outer(bw.dS[tail:], Q64[t]) * scale
            dV[tail: t + 1] += np.outer(fw.P[tail:], dO64[t])
        recs[t] = (fw, bw)
    return {"dQ": dQ, "dK": dK, "dV": dV, "rows": recs}


class SliceCheck:
    """Oracle for one (b, h) slice plus the decision analysis against the GPU's run.

    rows=None checks the whole slice.  Otherwise only the listed rows and the
    rows t >= tail are recomputed; O and dQ are compared on those rows and dK,
    dV on the keys >= tail.

    Decisions near a boundary.  A key whose oracle u (or exponential) lies
    inside the two sides' rounding band of a boundary has two admissible
    decisions.  When the GPU run carries its index dump, the decision the
    kernel took there is checked to be one of the two, and the oracle row is
    evaluated in fp64 with that decision (O.row_forward's ``decisions``): the
    test accepts either admissible decision without excluding any output.
    Only what the dump does not record is excluded, narrowly: the LERP
    segment under Nearest (it moves only the surrogate derivative: the key's
    own dK, the row's dQ and the keys carrying the row's calibration terms),
    and near-ties of the row max / min (the same outputs).  Without a dump
    the analysis falls back to excluding every output an ambiguous decision
    could move; compare() reports how much each check covers."""

    def __init__(self, q, k, v, do, p_or, gpu, b, h, rows=None, tail=None):
        self.p = p_or
        Qh, Kh, Vh, dOh = q[b, h], k[b, h], v[b, h], do[b, h]
        self.T, self.d = Qh.shape
        self.Q64, self.K64, self.V64, self.dO64 = (x.astype(np.float64) for x in (Qh, Kh, Vh, dOh))
        if rows is None:
            self.ref = O.head_backward(Qh, Kh, Vh, dOh, p_or, keep_rows=True)
            self.tail = 0
        else:
            self.tail = self.T if tail is None else tail
            self.ref = partial_head_backward(Qh, Kh, Vh, dOh, p_or, rows, self.tail)
        self.rows = sorted(self.ref["rows"])
        self.O_ref = np.full((self.T, self.d), np.nan)
        for t in self.rows:
            self.O_ref[t] = self.ref["rows"][t][0].P @ self.V64[: t + 1]
        self.g = gpu_slice(gpu, b, h, self.rows)
        self.sb = {t: score_bound(Qh[t: t + 1], Kh[: t + 1])[0] for t in self.rows}
        self._analyse()

    def _replay(self, t, decisions):
        """Re-evaluate row t of the oracle with the given decisions and move
        the slice's references from the old row result to the new one."""
        fw, bw = self.ref["rows"][t]
        fw2 = O.row_forward(fw.s, self.p, decisions)
        bw2 = O.row_backward(fw2, self.V64[: t + 1] @ self.dO64[t], self.p)
        scale = 1.0 / np.sqrt(self.d)
        self.ref["dQ"][t] = (bw2.dS @ self.K64[: t + 1]) * scale
        if t >= self.tail:
            lo = self.tail
            self.ref["dK"][lo: t + 1] += np.outer(bw2.dS[lo:] - bw.dS[lo:], self.Q64[t]) * scale
            self.ref["dV"][lo: t + 1] += np.outer(fw2.P[lo:] - fw.P[lo:], self.dO64[t])
        self.O_ref[t] = fw2.P @ self.V64[: t + 1]
        self.ref["rows"][t] = (fw2, bw2)
        self.n_replayed += len(decisions)
        self.rows_replayed += 1

    def _take(self, t, keys, cands):
        """The kernel's decisions at ambiguous keys, each checked against its
        admissible candidates; returns {key: decision}."""
        gi = self.g["idx"][t]
        out = {}
        for j, c in zip(keys, cands):
            dec = int(gi[j])
            if dec not in c:
                self.idx_mismatch += 1
            out[int(j)] = dec
        return out

    def _analyse(self):
        p, T, g = self.p, self.T, self.g
        K = p.K
        has_idx = "idx" in g
        self.score_viol = 0
        self.amb_fwd = np.zeros(T, dtype=bool)     # fallback only: rows whose forward weights may differ
        self.amb_bwd = np.zeros(T, dtype=bool)     # rows with any boundary-near decision
        self.excl_rows_dq = set()                  # rows whose dQ a non-replayed decision moves
        self.excl_keys_dk = set()                  # keys whose dK a non-replayed decision moves
        self.fwd_unstable_rows = []                # fallback only: (t, relative jump)
        self.n_amb_pairs = 0
        self.n_replayed = 0
        self.rows_replayed = 0
        self.idx_mismatch = 0
        self.idx_checked = 0
        untrunc = p.calibration == O.FWM_UNTRUNC
        for t in self.rows:
            fw, bw = self.ref["rows"][t]
            s_ref = fw.s
            cal = fw.cal
            sg = g["S"][t, : t + 1].astype(np.float64) if "S" in g else None
            if sg is not None:
                viol = np.abs(sg - s_ref) > self.sb[t] * 1.0 + 1e-30
                self.score_viol += int(viol.sum())
            # argmax / argmin near ties: the kernel may name the other key
            ds_obs = np.abs(sg - s_ref).max() if sg is not None else 0.0
            tie_band = 2 * ds_obs + 4 * 2.0 ** -24 * (np.abs(s_ref).max() + 1)
            srt = np.sort(s_ref)
            uses_min = p.calibration == O.MINMAX and p.reconstruction not in O.EXP_FAMILY
            ab_amb = False
            if t >= 1:
                if srt[-1] - srt[-2] <= tie_band:
                    ab_amb = True
                if uses_min and srt[1] - srt[0] <= tie_band:
                    ab_amb = True
            if ab_amb:
                # either key is admissible; only a different choice moves outputs
                self.amb_bwd[t] = True
                if g["a"][t] != cal.a or (uses_min and g["b"][t] != cal.b):
                    self.excl_rows_dq.add(t)
                    self.excl_keys_dk.update({int(cal.a), int(cal.b), int(g["a"][t]), int(g["b"][t])})
            else:
                assert g["a"][t] == cal.a, ("argmax", t, g["a"][t], cal.a)
                if uses_min:
                    assert g["b"][t] == cal.b, ("argmin", t, g["b"][t], cal.b)
            if cal.degenerate or t == 0:
                continue
            if p.reconstruction in O.EXP_FAMILY:
                if p.reconstruction in O.FORMATS and sg is not None:
                    self._rounding_band(t, fw, sg, has_idx)
                continue
            # decision band in grid steps
            mg, ng = float(g["m"][t]), float(g["n"][t])
            hg = (mg - ng) / K if p.calibration == O.MINMAX else p.tau / K
            u_ref = fw.rec.u
            u_pred = (mg - sg) / hg if sg is not None else u_ref
            band = 2 * (np.abs(u_pred - u_ref) + 4 * 2.0 ** -24 * (np.abs(u_ref) + 1))
            uc = u_ref if untrunc else np.minimum(u_ref, K)
            knot = np.abs(uc - np.round(uc)) <= band                 # LERP segment boundaries
            if untrunc:
                knot &= uc > band                                      # the grid continues past K
            else:
                knot &= (uc > band) & (uc < K - band)                  # u = 0 / u = K are exact (max/min keys)
            edge = (np.abs(u_ref - K) <= band) if p.calibration == O.FWM else np.zeros_like(knot)
            nearest = p.reconstruction == O.NEAREST
            half = np.abs(uc - (np.floor(uc) + 0.5)) <= band if nearest else np.zeros_like(knot)
            amb = knot | edge | half
            self.n_amb_pairs += int(amb.sum())
            if amb.any():
                self.amb_bwd[t] = True
            replay = (half | edge) if nearest else (knot | edge)
            narrow = amb & ~replay                                   # Nearest: surrogate segment at a knot
            if has_idx and replay.any():
                keys = np.flatnonzero(replay)
                cands = []
                for j in keys:
                    c = set()
                    x = uc[j] + (0.5 if nearest else 0.0)
                    hi_lev = (K if nearest else K - 1) if not untrunc else np.inf
                    for y in (x - band[j], x + band[j]):
                        c.add(int(min(max(np.floor(y), 0), hi_lev)))
                    if edge[j]:
                        c.add(-1)
                    cands.append(c)
                self._replay(t, self._take(t, keys, cands))
            elif replay.any():
                self._fallback(t, fw, uc, replay, edge, narrow | replay, untrunc)
                continue
            if narrow.any():
                self.excl_rows_dq.add(t)
                self.excl_keys_dk.update(int(j) for j in np.flatnonzero(narrow))
                self.excl_keys_dk.update({int(cal.a), int(cal.b)})
            # every other decision is bit-exact
            if has_idx:
                fw2 = self.ref["rows"][t][0]
                gi = g["idx"][t, : t + 1]
                lev = fw2.rec.i if p.reconstruction == O.LERP else fw2.rec.r
                ri = np.where(fw2.rec.mask > 0, lev, -1)
                ok = ~amb
                self.idx_checked += int(ok.sum())
                self.idx_mismatch += int((gi[ok] != ri[ok]).sum())

        if p.grad_rule == O.P1:
            # P1 subtracts the row mean of the detached gradient over all t+1
            # causal keys: a decision that moves one key's dS in row t moves
            # the mean, and with it dS at every key j <= t
            for t in sorted(self.excl_rows_dq):
                self.excl_keys_dk.update(range(int(t) + 1))

    def _fallback(self, t, fw, uc, fwd_keys, edge, bwd_keys, untrunc):
        """No index dump: exclude every output an ambiguous decision can move."""
        K = self.p.K
        jumps = []
        for j in np.flatnonzero(fwd_keys):
            if self.p.reconstruction == O.LERP and not edge[j]:
                continue                                             # a LERP knot moves no weight
            if edge[j]:
                jumps.append(fw.rec.g[K])
            else:
                r = int(np.floor(uc[j] + 0.5))
                lo, hi = max(r - 1, 0), (r + 1 if untrunc else min(r + 1, K))
                gv = lambda x: float(np.exp(-fw.cal.h * x))
                jumps.append(max(abs(gv(r) - gv(lo)), abs(gv(hi) - gv(r))))
        if jumps and max(jumps) / fw.W > 1e-7:
            self.amb_fwd[t] = True
            self.fwd_unstable_rows.append((t, max(jumps) / fw.W))
        self.excl_rows_dq.add(t)
        self.excl_keys_dk.update(int(j) for j in np.flatnonzero(bwd_keys))
        self.excl_keys_dk.update({int(fw.cal.a), int(fw.cal.b)})

    def _rounding_band(self, t, fw, sg, has_idx):
        """Rounded-exponential baselines: a key whose exp(s - m) lies closer to
        a rounding midpoint of the format than the two sides' exponentials can
        differ may round either way.  The kernel's exponential carries the
        difference of its fp32 s - m from the oracle's, plus the rounding of
        the argument and of its exp2 (a few 2^-24 relative each).  The index
        dump holds the fp32 bits of each rounded value the kernel used: it
        must be the oracle's rounding away from midpoints, and one of the two
        neighbouring format values near one, which is then replayed."""
        frac_bits, emin = O.FORMATS[self.p.reconstruction]
        m_ref = fw.cal.m
        x_ref = fw.s - m_ref
        e_ref = np.exp(x_ref)
        d_obs = np.abs((sg - float(self.g["m"][t])) - x_ref)
        band = 2 * e_ref * (d_obs + 8 * 2.0 ** -24 * (np.abs(x_ref) + 1))
        _, ex = np.frexp(e_ref)
        q = np.ldexp(1.0, np.maximum(ex - 1, emin) - frac_bits)
        dist = np.abs(e_ref / q - np.floor(e_ref / q) - 0.5) * q
        amb = dist <= band
        tiny = e_ref < 2.0 ** -126                 # below fp32's normal range: the kernel's exp2 may flush
        if has_idx:
            wv = self.g["idx"][t, : t + 1].view(np.float32).astype(np.float64)
            ok = ~amb & ~tiny
            self.idx_checked += int(ok.sum())
            self.idx_mismatch += int((wv[ok] != fw.w[ok]).sum())
        if not amb.any():
            return
        self.n_amb_pairs += int(amb.sum())
        self.amb_bwd[t] = True
        if has_idx:
            keys = np.flatnonzero(amb)
            lo, hi = O.format_neighbours(e_ref[keys], frac_bits, emin)
            dec = {}
            for j, l, h in zip(keys, lo, hi):
                if wv[j] == h:
                    dec[int(j)] = 1
                elif wv[j] == l:
                    dec[int(j)] = 0
                else:
                    self.idx_mismatch += 1
            self._replay(t, dec)
            return
        rel = float(q[amb].max()) / fw.W          # one quantum against the row normaliser
        if rel > 1e-7:
            self.amb_fwd[t] = True
            self.fwd_unstable_rows.append((t, rel))
        self.excl_rows_dq.add(t)
        self.excl_keys_dk.update(int(j) for j in np.flatnonzero(amb))
        self.excl_keys_dk.add(int(fw.cal.a))

    # ------------------------------------------------------------------
    def compare(self, name, tol=TOL):
        """Max error of an output relative to the slice's max |reference|,
        over the entries no unreplayed decision can move.  Returns (error,
        entries compared, entries in the region checked)."""
        T = self.T
        ref = {"O": self.O_ref, "dQ": self.ref["dQ"], "dK": self.ref["dK"], "dV": self.ref["dV"]}[name]
        got = self.g[name].astype(np.float64)
        keep = np.zeros(T, dtype=bool)
        if name in ("O", "dQ"):
            keep[self.rows] = True
        else:
            keep[self.tail:] = True
        region = keep.copy()                 # entries this check covers, before exclusions
        if name == "O":
            keep &= ~self.amb_fwd
        elif name == "dQ":
            keep &= ~self.amb_fwd
            keep[sorted(self.excl_rows_dq)] = False
        else:
            if name == "dK":
                keep[sorted(self.excl_keys_dk)] = False
            for t, _ in self.fwd_unstable_rows:
                keep[: t + 1] = False
        n_region = int(region.sum())
        scale = np.abs(ref[region]).max() if region.any() else 0.0
        if scale == 0:
            return 0.0, int(keep.sum()), n_region
        err = np.abs(got[keep] - ref[keep]).max() / scale if keep.any() else 0.0
        return float(err), int(keep.sum()), n_region

    def zero_sum_violations(self, q, k, v, do, b, h):
        """Rows where |sum_j dS_tj| > 1e-5 * sum_j |dS_tj| on the GPU's own dS
        tiles (which carry the routed calibration terms at argmax / argmin).

        The calibration terms make the row sum vanish for any dL/dw, so fp32
        noise in dP and delta cancels there.  Degenerate-span rows have no
        calibration terms: their sum is sum_j P_j dP_j - delta, which cancels
        only to the rounding of two length-d fp32 dot products, so those rows
        also get a floor of 4 d 2^-24 sum_j P_j sum_c |dO_c V_jc|."""
        g = self.g
        Vh, dOh = v[b, h].astype(np.float64), do[b, h].astype(np.float64)
        bad = []
        for t in self.rows:
            row = g["dS"][t, : t + 1].astype(np.float64)
            if self.p.grad_rule == O.P1:
                # P1 stores the detached gradient; the row mean (cm) is taken
                # off through dQ and dK, so the projected row is dS - cm
                row = row - float(g["cm"][t])
            l1 = np.abs(row).sum()
            floor = 0.0
            fw = self.ref["rows"][t][0]
            if fw.cal.degenerate:
                floor = 4 * self.d * 2.0 ** -24 * float(fw.P @ (np.abs(Vh[: t + 1]) @ np.abs(dOh[t])))
            if abs(row.sum()) > ZERO_SUM_TOL * l1 + floor:
                bad.append((t, row.sum(), l1))
        return bad
