"""Helpers of the GPU parity tests: run the HIP path through the C ABI, run the
oracle on the same seeded inputs, and compare to the tolerances of the
workload's dtype.

Tolerances:
  fp32: max |Y - Y_ref| <= 1e-4.
  bf16: ||Y - Y_ref|| / ||Y_ref|| <= 1e-2 over all compared elements,
        ||Y[r] - Y_ref[r]|| <= 1e-2 * max(||Y_ref[r]||, ROW_FLOOR * rms)
        for every output row r, where rms is the root mean square of the
        reference rows' norms (not applied when the whole reference is zero),
        and
        |Y[r, c] - Y_ref[r, c]| <= 2e-2 * max(1, max_c' |Y_ref[r, c']|)
        for every output row r.
The per-row bound catches an error confined to a few rows (one head's
columns wrong in one row, say), which the global relative L2 norm averages
away and which the elementwise bound misses wherever outputs are far below 1.
Its floor at a quarter of the typical row norm is for rows that cancel: a
weight-gradient row summed over a few tokens can be several times smaller
than the terms it sums, and a one-ulp difference in a bf16-rounded
intermediate (dV rounded from fp32 on the GPU, from fp64 in the oracle) then
moves it by more than 1% of its own norm (3.3% on a 4-token dWv row whose
norm is 0.15 of the typical row's). A row wrong at the typical magnitude is
still caught.
The elementwise bound scales with the row, not the element. Y[r, c] is a dot
product of the attention row A[r, :] with a column of Wo. Rounding A to bf16
(relative 2^-9 per element) therefore moves every element of the row by an
amount proportional to the row's magnitude, whatever that element's own
value is.
Y_ref is the float64 oracle with bf16 rounding at the Q/K/V/A/Y boundaries
for bf16 runs, and no rounding for fp32 runs.
"""
from __future__ import annotations

import sys
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np

import workloads as wl


ROW_FLOOR = 0.25


@dataclass
class Report:
    max_abs: float
    rel_l2: float
    worst_scaled: float      # max over rows of max_c |err[r, c]| / max(1, max_c |ref[r, c]|)
    worst_row_rel: float     # max over rows of ||err[r]|| / max(||ref[r]||, ROW_FLOOR * rms)
    ok: bool

    def __str__(self):
        return (f"max_abs={self.max_abs:.3e} rel_l2={self.rel_l2:.3e} "
                f"worst_scaled={self.worst_scaled:.3e} worst_row_rel={self.worst_row_rel:.3e} "
                f"{'OK' if self.ok else 'FAIL'}")


# Weight gradients sum over the batch's tokens; below this many tokens a row is
# a combination of so few bf16-rounded vectors that a one-ulp difference in
# one of them (dK rounded from fp32 on the GPU, from fp64 in the oracle) moves
# the row by several percent (up to 5% on 4-token dWk rows), and the per-row
# bound is not applied to them.
MIN_TOKENS_FOR_ROW_GATE = 64


def compare(got: np.ndarray, ref: np.ndarray, dtype: str, row_gate: bool = True) -> Report:
    """Compare outputs whose last axis is one output row (d_model wide).
    row_gate=False leaves out the per-row bound (bf16), for weight gradients
    summed over fewer than MIN_TOKENS_FOR_ROW_GATE tokens."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if not np.isfinite(got).all():
        return Report(float("inf"), float("inf"), float("inf"), float("inf"), False)
    if got.size == 0:
        return Report(0.0, 0.0, 0.0, 0.0, True)
    g2 = got.reshape(-1, got.shape[-1])
    r2 = ref.reshape(-1, ref.shape[-1])
    err = np.abs(g2 - r2)
    max_abs = float(err.max())
    nref = float(np.linalg.norm(r2))
    rel = float(np.linalg.norm(g2 - r2) / nref) if nref > 0 else float(np.linalg.norm(g2 - r2))
    row_scale = np.maximum(1.0, np.abs(r2).max(axis=1))
    scaled = float((err.max(axis=1) / row_scale).max())
    rn = np.linalg.norm(r2, axis=1)
    en = np.linalg.norm(g2 - r2, axis=1)
    den = np.maximum(rn, ROW_FLOOR * float(np.sqrt(np.mean(rn * rn))))
    # an all-zero reference (one-token gradients, say) has no row scale: the
    # absolute global and elementwise bounds decide alone
    row_rel = float((en / den).max()) if (den > 0).all() else 0.0
    if dtype == "fp32":
        ok = max_abs <= 1e-4
    else:
        ok = rel <= 1e-2 and scaled <= 2e-2 and (row_rel <= 1e-2 or not row_gate)
    return Report(max_abs, rel, scaled, row_rel, ok)


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def device_inputs(w: wl.Workload, device):
    """Seeded inputs rounded to the dtype: (host torch tensors, device tensors)."""
    host = wl.to_device_dtype(wl.draw(w), w.dtype)
    dev = {k: v.to(device) for k, v in host.items()}
    return host, dev


def oracle_inputs(host) -> Dict[str, np.ndarray]:
    return {k: wl.widen(v) for k, v in host.items()}


def sample_rows(w: wl.Workload, n_random: int = 96, seed: int = 0) -> np.ndarray:
    """Flat token rows for full-size parity: both ends of every sequence, rows
    around key/query tile boundaries, outlier rows, and random rows."""
    N, B = w.N, w.B
    rows = set()
    for b in (0, B - 1):
        base = b * N
        rows.update(base + t for t in range(min(N, 16)))
        rows.update(base + t for t in range(max(0, N - 16), N))
        for edge in (32, 64, 128, 256, N // 2, N - 257, N - 65):
            for t in (edge - 1, edge, edge + 1):
                if 0 <= t < N:
                    rows.add(base + t)
    out = wl.outlier_rows(w)
    if out.size:
        rng = np.random.default_rng(seed + 1)
        rows.update(rng.choice(out, size=min(48, out.size), replace=False).tolist())
    rng = np.random.default_rng(seed)
    rows.update(rng.integers(0, B * N, size=n_random).tolist())
    return np.array(sorted(rows), dtype=np.int64)
