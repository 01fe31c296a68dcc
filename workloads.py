"""Seeded synthetic inputs for the Sparse Query Attention forward pass.

This module only draws random numbers and names workloads. It holds none of the
method's arithmetic, and both the oracle side and the HIP side take their inputs
from it.

Every workload is one of the attention shapes below. The pages (arXiv 2510.01817,
abstract) measure SQA on long sequences of 32k to 200k tokens. The model cards
(ReactiveAI/GQA-Ref-Micro, results) name the sSQA and xSQA variants, and
ReactiveAI/xSMQAT-m names xSMQA. The pages give no dataset for the long-sequence
benchmark. X stands in for the embedded-token activations of such a sequence:
X ~ N(0, 1), and every weight is ~ N(0, 1/d_model).

Draw recipe (the same everywhere):
  * numpy ``default_rng(SeedSequence([seed, stream]))``. Stream 0 is X, 1..4 are
    Wq, Wk, Wv, Wo, and 5 picks the outlier token rows.
  * Draws are float32. The outlier rows (a fraction of the B*N token rows,
    distinct, uniform) are multiplied by a factor in float32.
  * ``to_device_dtype`` rounds once to the workload dtype with torch's
    round-to-nearest-even conversion. The oracle widens exactly those rounded
    values to float64, and the GPU receives the same rounded values.
  * A baseline run (MHA/GQA/MQA of the same shape) reuses X and draws its own
    weights, at its own widths, from the same streams.
  * A variable-length batch (sequences padded to N, as a training batch cut at
    a maximum sequence length holds them: model cards' training example) draws
    its lengths from stream 6, uniform integers in [varlen_min, N].
  * The backward pass takes an upstream gradient dY [B, N, d_model] from
    stream 7: N(0, 1/d_model) in float32, the scale of the gradient of a
    per-token mean loss through an output layer of the same width.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, Optional

import numpy as np

STREAM_X, STREAM_WQ, STREAM_WK, STREAM_WV, STREAM_WO, STREAM_OUTLIERS, STREAM_LENS, STREAM_DY = range(8)


@dataclass(frozen=True)
class Workload:
    """One SQA forward shape: tokens [B, N, d_model], H baseline heads,
    H_q query heads and H_kv key/value heads of width d_head = d_model / H."""

    name: str
    B: int
    N: int
    d_model: int
    H: int
    H_q: int
    H_kv: int
    causal: bool
    dtype: str  # "fp32" or "bf16"
    seed: int
    outlier_frac: float = 0.0
    outlier_scale: float = 20.0
    baseline_H_q: Optional[int] = None
    baseline_H_kv: Optional[int] = None
    varlen_min: Optional[int] = None   # variable-length batch: shortest sequence length

    @property
    def d_head(self) -> int:
        return self.d_model // self.H

    @property
    def tokens(self) -> int:
        return self.B * self.N

    def baseline(self) -> "Workload":
        """The equally shaped MHA/GQA/MQA run with H_q = H."""
        if self.baseline_H_q is None:
            raise ValueError(f"{self.name} has no baseline")
        return replace(self, name=self.name + "_baseline", H_q=self.baseline_H_q,
                       H_kv=self.baseline_H_kv, baseline_H_q=None, baseline_H_kv=None)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads.
TINY_SQA_FP32 = Workload("tiny_sqa_fp32_n256", B=1, N=256, d_model=256, H=8, H_q=4, H_kv=2,
                         causal=False, dtype="fp32", seed=1000)
SSQA_1K_CAUSAL = Workload("ssqa_bf16_causal_b16_n1024", B=16, N=1024, d_model=512, H=16, H_q=8,
                          H_kv=8, causal=True, dtype="bf16", seed=1001,
                          baseline_H_q=16, baseline_H_kv=4)
XSQA_32K = Workload("xsqa_bf16_n32768", B=1, N=32768, d_model=1024, H=16, H_q=4, H_kv=4,
                    causal=False, dtype="bf16", seed=1002, baseline_H_q=16, baseline_H_kv=16)
SQA_131K_CAUSAL = Workload("sqa_bf16_causal_n131072", B=1, N=131072, d_model=1024, H=16, H_q=8,
                           H_kv=4, causal=True, dtype="bf16", seed=1003,
                           baseline_H_q=16, baseline_H_kv=4)
XSMQA_200K = Workload("xsmqa_bf16_n200000_outliers", B=1, N=200000, d_model=1024, H=16, H_q=4,
                      H_kv=1, causal=False, dtype="bf16", seed=1004, outlier_frac=0.01,
                      baseline_H_q=16, baseline_H_kv=1)

# Standard SQA, causal, 8 sequences of 4096..32768 tokens padded to 32768.
SQA_VARLEN_32K = Workload("sqa_bf16_causal_varlen_b8_n32768", B=8, N=32768, d_model=1024, H=16,
                          H_q=8, H_kv=4, causal=True, dtype="bf16", seed=1005, varlen_min=4096)

WORKLOADS: Dict[str, Workload] = {w.name: w for w in
                                  (TINY_SQA_FP32, SSQA_1K_CAUSAL, XSQA_32K, SQA_131K_CAUSAL,
                                   XSMQA_200K, SQA_VARLEN_32K)}


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, stream]))


def draw_x(w: Workload) -> np.ndarray:
    """X [B, N, d_model] float32, N(0, 1), with the outlier rows scaled."""
    x = _rng(w.seed, STREAM_X).standard_normal((w.B * w.N, w.d_model), dtype=np.float32)
    n_out = int(np.floor(w.outlier_frac * w.B * w.N))
    if n_out > 0:
        rows = _rng(w.seed, STREAM_OUTLIERS).choice(w.B * w.N, size=n_out, replace=False)
        x[rows] *= np.float32(w.outlier_scale)
    return x.reshape(w.B, w.N, w.d_model)


def outlier_rows(w: Workload) -> np.ndarray:
    """Flat token-row indices (b * N + t) that ``draw_x`` scaled, sorted."""
    n_out = int(np.floor(w.outlier_frac * w.B * w.N))
    if n_out == 0:
        return np.zeros(0, dtype=np.int64)
    rows = _rng(w.seed, STREAM_OUTLIERS).choice(w.B * w.N, size=n_out, replace=False)
    return np.sort(rows.astype(np.int64))


def draw_weights(w: Workload) -> Dict[str, np.ndarray]:
    """Wq [d_model, H_q*d], Wk/Wv [d_model, H_kv*d], Wo [H_q*d, d_model], float32,
    each ~ N(0, 1/d_model), stored [in, out] so that y = x @ W."""
    d = w.d_head
    std = np.float32(1.0 / np.sqrt(w.d_model))
    shapes = {"Wq": (STREAM_WQ, (w.d_model, w.H_q * d)),
              "Wk": (STREAM_WK, (w.d_model, w.H_kv * d)),
              "Wv": (STREAM_WV, (w.d_model, w.H_kv * d)),
              "Wo": (STREAM_WO, (w.H_q * d, w.d_model))}
    return {k: _rng(w.seed, s).standard_normal(shp, dtype=np.float32) * std
            for k, (s, shp) in shapes.items()}


def draw_upstream_grad(w: Workload) -> np.ndarray:
    """dY [B, N, d_model] (float32) for the backward pass, from stream 7."""
    g = _rng(w.seed, STREAM_DY).standard_normal((w.B * w.N, w.d_model), dtype=np.float32)
    g *= np.float32(1.0 / np.sqrt(w.d_model))
    return g.reshape(w.B, w.N, w.d_model)


def draw_lens(w: Workload) -> np.ndarray:
    """Sequence lengths [B] int32 of a variable-length batch (all N otherwise)."""
    if w.varlen_min is None:
        return np.full(w.B, w.N, dtype=np.int32)
    return _rng(w.seed, STREAM_LENS).integers(w.varlen_min, w.N + 1, size=w.B).astype(np.int32)


def draw(w: Workload) -> Dict[str, np.ndarray]:
    out = {"X": draw_x(w)}
    out.update(draw_weights(w))
    return out


def to_device_dtype(arrays: Dict[str, np.ndarray], dtype: str):
    """Round the float32 draws once to the workload dtype as torch CPU tensors.
    bf16 uses torch's round-to-nearest-even conversion."""
    import torch
    tdt = {"fp32": torch.float32, "bf16": torch.bfloat16}[dtype]
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to(tdt) for k, v in arrays.items()}


def widen(t) -> np.ndarray:
    """Exact widening of a torch CPU tensor (fp32 or bf16) to a float64 array."""
    import torch
    return t.to(torch.float64).numpy()
