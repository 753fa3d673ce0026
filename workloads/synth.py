"""Seeded synthetic inputs for K-interval attention.

Both the test suite and the benchmark draw their inputs from here, so the CPU
oracle and the HIP library see identical fp32 bytes.  This module holds none
of the operator's arithmetic (no calibration, grid, reconstruction,
normalisation or gradient rule): only random draws and the shaping of query
rows that sets the score geometry the workloads call for.

Workload geometry follows "Pretraining Transformers with Quantized Softmax in
Attention" (paperlayer digest): an fp32 attention operator on GPT-2-style
shapes (section 4, Training setup; App. C.1), softmax-trained row spans of
25-32 nats and wider spans for MinMax-Weight rows (App. A; App. D.6).  The
pages ship no data, so every tensor here is drawn from numpy's PCG64
(``numpy.random.default_rng``), whose stream is stable across machines.

Draw order for every workload: Q, K, V, dO (``standard_normal`` in float64 at
[B, H, T, d]), then the structural draws of that workload in the order the
code below makes them; the fp32 cast happens last.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    """One synthetic input recipe.

    kind:
      "plain"      Q, K, V, dO ~ N(0, 1).
      "scaled"     Q multiplied by ``q_scale`` (sets the row score span).
      "spike_all"  Q multiplied by ``q_scale``; every row t >= 1 gets one
                   dominant key j*(t) ~ U{0..t} whose score sits ``gap`` nats
                   above the runner-up.
      "head_temp"  per-head score temperature c_h ~ U[lo, hi] multiplies Q.
      "spike_frac" a fraction ``frac`` of rows (t >= 1, drawn without
                   replacement) get one dominant key at ``gap`` nats above
                   the runner-up.
    """

    name: str
    B: int
    H: int
    T: int
    d: int
    kind: str = "plain"
    q_scale: float = 1.0
    gap: float = 0.0
    frac: float = 0.0
    lo: float = 0.5
    hi: float = 3.0
    seed: int = 0
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    def shape(self):
        return (self.B, self.H, self.T, self.d)

    def pairs(self) -> int:
        """Causal (query, key) pairs, self-key included."""
        return self.B * self.H * self.T * (self.T + 1) // 2

    def scaled(self, **kw) -> "Workload":
        """Same recipe at another size (for small parity cases)."""
        args = dict(self.__dict__)
        args.update(kw)
        return Workload(**args)


# The five workloads the build is measured and checked on.
WORKLOADS = {
    # single head, N(0,1): row spans of about 5 nats
    "c1": Workload("c1_single_head", 1, 1, 128, 64, "plain"),
    # GPT-2 124M attention layer; Q x2 gives full-row spans of about 12 nats
    "c2": Workload("c2_gpt2_124m", 8, 12, 1024, 64, "scaled", q_scale=2.0),
    # sharpened late-training geometry: Q x11 then one key per row at +20
    "c3": Workload("c3_gpt2_sharp", 8, 12, 1024, 64, "spike_all", q_scale=11.0, gap=20.0),
    # 1B-scale head shape with per-head temperature in [0.5, 3]
    "c4": Workload("c4_1b_heads", 4, 16, 2048, 128, "head_temp", lo=0.5, hi=3.0),
    # long rows; 1% of rows carry one outlier key at +40
    "c5": Workload("c5_long_rows", 1, 12, 8192, 64, "spike_frac", frac=0.01, gap=40.0),
}


def _spike_gamma(q_row: np.ndarray, keys: np.ndarray, jstar: int, gap: float, inv_sqrt_d: float) -> float:
    """Coefficient g such that adding g*K[j*] to the query row puts the score of
    key j* exactly ``gap`` above every other key of the row.

    Scores move linearly in g: s_j(g) = a_j + g*b_j.  The margin over key j is
    (a_j* - a_j) + g*(b_j* - b_j); the smallest g meeting every margin is the
    largest of (gap - (a_j* - a_j)) / (b_j* - b_j) over keys with a positive
    slope difference.
    """
    a = keys @ q_row * inv_sqrt_d
    b = keys @ keys[jstar] * inv_sqrt_d
    others = np.ones(keys.shape[0], dtype=bool)
    others[jstar] = False
    if not others.any():
        return 0.0
    da = a[jstar] - a[others]
    db = b[jstar] - b[others]
    if np.any(db <= 0):  # a key parallel to K[j*]: cannot be separated by this construction
        raise ValueError("spike construction: degenerate key geometry")
    return float(np.max((gap - da) / db))


def make_inputs(w: Workload):
    """Return (q, k, v, do) as float32 numpy arrays of shape [B, H, T, d]."""
    rng = np.random.default_rng(w.seed)
    shape = w.shape()
    q = rng.standard_normal(shape)
    k = rng.standard_normal(shape)
    v = rng.standard_normal(shape)
    do = rng.standard_normal(shape)
    inv_sqrt_d = 1.0 / np.sqrt(w.d)

    if w.kind == "plain":
        pass
    elif w.kind == "scaled":
        q *= w.q_scale
    elif w.kind == "head_temp":
        c = rng.uniform(w.lo, w.hi, size=w.H)
        q *= c[None, :, None, None]
    elif w.kind in ("spike_all", "spike_frac"):
        q *= w.q_scale
        if w.kind == "spike_all":
            rows = [(b, h, t) for b in range(w.B) for h in range(w.H) for t in range(1, w.T)]
        else:
            flat = np.array([(b * w.H + h) * w.T + t
                             for b in range(w.B) for h in range(w.H) for t in range(1, w.T)],
                            dtype=np.int64)
            n_pick = int(round(w.frac * flat.size))
            pick = np.sort(rng.choice(flat, size=n_pick, replace=False))
            rows = [(int(f // (w.H * w.T)), int((f // w.T) % w.H), int(f % w.T)) for f in pick]
        jstars = [int(rng.integers(0, t + 1)) for (_, _, t) in rows]
        for (b, h, t), js in zip(rows, jstars):
            keys = k[b, h, : t + 1]
            g = _spike_gamma(q[b, h, t], keys, js, w.gap, inv_sqrt_d)
            q[b, h, t] = q[b, h, t] + g * keys[js]
    else:
        raise ValueError(f"unknown workload kind {w.kind!r}")

    return (q.astype(np.float32), k.astype(np.float32),
            v.astype(np.float32), do.astype(np.float32))


def spike_rows(w: Workload):
    """The (b, h, t) rows that carry a constructed dominant key, with j*.

    Re-draws the same stream as ``make_inputs`` (draw order is fixed), so the
    answer matches the tensors it returns.
    """
    if w.kind not in ("spike_all", "spike_frac"):
        return []
    rng = np.random.default_rng(w.seed)
    shape = w.shape()
    for _ in range(4):
        rng.standard_normal(shape)
    if w.kind == "spike_all":
        rows = [(b, h, t) for b in range(w.B) for h in range(w.H) for t in range(1, w.T)]
    else:
        flat = np.array([(b * w.H + h) * w.T + t
                         for b in range(w.B) for h in range(w.H) for t in range(1, w.T)],
                        dtype=np.int64)
        n_pick = int(round(w.frac * flat.size))
        pick = np.sort(rng.choice(flat, size=n_pick, replace=False))
        rows = [(int(f // (w.H * w.T)), int((f // w.T) % w.H), int(f % w.T)) for f in pick]
    jstars = [int(rng.integers(0, t + 1)) for (_, _, t) in rows]
    return [(b, h, t, js) for (b, h, t), js in zip(rows, jstars)]
