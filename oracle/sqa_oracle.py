"""Plain float64 CPU oracle for the Sparse Query Attention (SQA) forward pass.

TEST INFRASTRUCTURE. This module checks the HIP path; it is not part of it.
Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
it. It shares no code with the HIP library.

What it computes (sources):
  * "Sparse Query Attention (SQA): A Computationally Efficient Attention
    Mechanism with Query Heads Reduction" (arXiv 2510.01817), abstract: SQA
    keeps the MHA/GQA attention computation but uses fewer query heads,
    H_q < H. Score FLOPs therefore scale with H_q.
  * Model card ReactiveAI/GQA-Ref-Micro, description: SQA extends GQA, so
    key/value heads are still shared by groups of query heads (H_kv <= H_q).
    Its complexity expressions write the head width as d/heads.
  * Model card ReactiveAI/xSMQAT-m, description: the query projection and the
    output projection are narrowed to the H_q used heads.
  * The same model card's training example runs in bf16 autocast
    (use_amp=True, dtype=torch.bfloat16).

The pages never write the equations out. The reading taken here is:
    Q = X Wq, K = X Wk, V = X Wv  (y = x W, weights stored [in, out])
    query head i reads key/value head floor(i / (H_q / H_kv))
    S = Q_i K_kv^T / sqrt(d_head); causal: key c visible to query r iff c <= r
    P = row softmax(S); A[:, i*d:(i+1)*d] = P V_kv   (head-major columns)
    Y = A Wo
With ``bf16=True`` the results are rounded to the nearest bfloat16 (ties to
even) where an autocast bf16 run stores a tensor: Q, K, V, A and Y. Everything
between those points is float64.

Evaluation order: rows (queries) are computed in blocks. This only bounds
memory: each row's arithmetic is the definition above, unchanged. A
fully masked causal key contributes exp(-inf) = 0, so it is not visited.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Iterable, Optional, Sequence

import numpy as np

BF16_MAX = float.fromhex("0x1.fep127")  # largest finite bfloat16: (2 - 2**-7) * 2**127


def round_bf16(a) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), kept in float64.

    bfloat16 has one sign bit, 8 exponent bits (bias 127) and 7 fraction bits.
    A normal value (exponent -126..127) keeps 8 significant bits. Below 2**-126,
    values sit on the fixed grid of 2**-133 (the subnormals). Anything that
    rounds past the largest finite value becomes infinity. NaN stays NaN.
    """
    a = np.asarray(a, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        m, e = np.frexp(a)                  # a = m * 2**e, 0.5 <= |m| < 1
        bits = np.minimum(8, e + 133)       # significant bits that survive
        r = np.ldexp(np.rint(np.ldexp(m, bits)), e - bits)   # np.rint: ties to even
        r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, a), r)
    return r


def _maybe_round(a: np.ndarray, bf16: bool) -> np.ndarray:
    return round_bf16(a) if bf16 else a


def kv_head_for(i: int, H_q: int, H_kv: int) -> int:
    """Key/value head read by query head i: contiguous groups of g = H_q/H_kv."""
    return i // (H_q // H_kv)


def split_heads(Y: np.ndarray, n_heads: int, d_head: int) -> np.ndarray:
    """[B, N, n_heads*d_head] -> [B, n_heads, N, d_head]; head h owns columns
    [h*d_head, (h+1)*d_head)."""
    B, N, _ = Y.shape
    return Y.reshape(B, N, n_heads, d_head).transpose(0, 2, 1, 3)


def check_shapes(X, Wq, Wk, Wv, Wo, H_q, H_kv, d_head):
    B, N, D = X.shape
    if H_kv < 1 or H_q < H_kv or H_q % H_kv:
        raise ValueError("need 1 <= H_kv <= H_q and H_q % H_kv == 0")
    want = {"Wq": (D, H_q * d_head), "Wk": (D, H_kv * d_head), "Wv": (D, H_kv * d_head),
            "Wo": (H_q * d_head, D)}
    for name, w in zip(("Wq", "Wk", "Wv", "Wo"), (Wq, Wk, Wv, Wo)):
        if tuple(w.shape) != want[name]:
            raise ValueError(f"{name} has shape {w.shape}, expected {want[name]}")
    return B, N, D


def softmax_probs(q: np.ndarray, k: np.ndarray, q_pos: np.ndarray, causal: bool,
                  scale: float) -> np.ndarray:
    """Attention weights P [R, n_keys] of R queries (at sequence positions
    ``q_pos``) over the keys 0..n_keys-1 of one head."""
    s = (q @ k.T) * scale
    if causal:
        s = np.where(np.arange(k.shape[0])[None, :] <= q_pos[:, None], s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=1, keepdims=True)


def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos: np.ndarray,
                   causal: bool) -> np.ndarray:
    """Output rows of one head: softmax(q k^T / sqrt(d)) v, with q [R, d] at
    positions ``q_pos`` and k, v [N, d]. Causal rows only see keys c <= pos."""
    d = q.shape[1]
    n_keys = k.shape[0]
    if causal:
        n_keys = min(n_keys, int(q_pos.max()) + 1)   # later keys are all masked
    p = softmax_probs(q, k[:n_keys], q_pos, causal, 1.0 / math.sqrt(d))
    return p @ v[:n_keys]


def _pool_workers(workers: Optional[int]) -> int:
    if workers is not None:
        return max(1, workers)
    return max(1, len(os.sched_getaffinity(0)))


def _run_tasks(fn, tasks: Sequence, workers: int):
    """Run independent tasks on a thread pool with single-threaded BLAS inside
    each worker (numpy releases the GIL in its kernels)."""
    if workers == 1 or len(tasks) <= 1:
        for t in tasks:
            fn(t)
        return
    try:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(limits=1)
    except ImportError:  # pragma: no cover - threadpoolctl is installed here
        ctx = None
    try:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fn, tasks))
    finally:
        if ctx is not None:
            ctx.unregister()


def sqa_forward(X, Wq, Wk, Wv, Wo, H_q: int, H_kv: int, d_head: int, causal: bool,
                bf16: bool, row_block: int = 256, workers: Optional[int] = None
                ) -> Dict[str, np.ndarray]:
    """Full SQA forward. Returns the float64 arrays
    Q [B,N,H_q*d], K, V [B,N,H_kv*d], A [B,N,H_q*d] and Y [B,N,d_model]."""
    X, Wq, Wk, Wv, Wo = (np.asarray(t, dtype=np.float64) for t in (X, Wq, Wk, Wv, Wo))
    B, N, D = check_shapes(X, Wq, Wk, Wv, Wo, H_q, H_kv, d_head)
    Q = _maybe_round(X @ Wq, bf16)
    K = _maybe_round(X @ Wk, bf16)
    V = _maybe_round(X @ Wv, bf16)
    Qh, Kh, Vh = split_heads(Q, H_q, d_head), split_heads(K, H_kv, d_head), split_heads(V, H_kv, d_head)
    A = np.empty((B, N, H_q * d_head), dtype=np.float64)

    tasks = [(b, i, r0) for b in range(B) for i in range(H_q) for r0 in range(0, N, row_block)]

    def one(task):
        b, i, r0 = task
        r1 = min(N, r0 + row_block)
        kv = kv_head_for(i, H_q, H_kv)
        pos = np.arange(r0, r1)
        A[b, r0:r1, i * d_head:(i + 1) * d_head] = attention_rows(
            Qh[b, i, r0:r1], Kh[b, kv], Vh[b, kv], pos, causal)

    _run_tasks(one, tasks, _pool_workers(workers))
    A = _maybe_round(A, bf16)
    Y = _maybe_round(A @ Wo, bf16)
    return {"Q": Q, "K": K, "V": V, "A": A, "Y": Y}


def sqa_forward_rows(X, Wq, Wk, Wv, Wo, H_q: int, H_kv: int, d_head: int, causal: bool,
                     bf16: bool, rows: Iterable[int], workers: Optional[int] = None,
                     row_block: int = 128, kv_cache: Optional[Dict[int, tuple]] = None) -> Dict[str, np.ndarray]:
    """The same forward, evaluated only at the flat token rows ``rows``
    (row = b*N + t). Every key and value is still projected.

    Returns A_rows [R, H_q*d] and Y_rows [R, d_model] in the order of ``rows``.
    ``kv_cache`` may hold {b: (K_b, V_b)} computed by an earlier call on the
    same inputs. This saves re-projecting keys and values; the arithmetic is
    unchanged.
    """
    X, Wq, Wk, Wv, Wo = (np.asarray(t, dtype=np.float64) for t in (X, Wq, Wk, Wv, Wo))
    B, N, D = check_shapes(X, Wq, Wk, Wv, Wo, H_q, H_kv, d_head)
    rows = np.asarray(list(rows), dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= B * N):
        raise ValueError("row index out of range")
    A_rows = np.empty((rows.size, H_q * d_head), dtype=np.float64)
    cache = kv_cache if kv_cache is not None else {}
    for b in np.unique(rows // N):
        b = int(b)
        sel = np.nonzero(rows // N == b)[0]
        pos = rows[sel] % N
        if b not in cache:
            cache[b] = (_maybe_round(X[b] @ Wk, bf16), _maybe_round(X[b] @ Wv, bf16))
        Kb, Vb = cache[b]
        Qb = _maybe_round(X[b, pos] @ Wq, bf16)
        out = np.empty((sel.size, H_q * d_head), dtype=np.float64)
        tasks = [(i, r0) for i in range(H_q) for r0 in range(0, sel.size, row_block)]

        def one(task):
            i, r0 = task
            r1 = min(sel.size, r0 + row_block)
            kv = kv_head_for(i, H_q, H_kv)
            cols = slice(kv * d_head, (kv + 1) * d_head)
            out[r0:r1, i * d_head:(i + 1) * d_head] = attention_rows(
                Qb[r0:r1, i * d_head:(i + 1) * d_head], Kb[:, cols], Vb[:, cols],
                pos[r0:r1], causal)

        _run_tasks(one, tasks, _pool_workers(workers))
        A_rows[sel] = out
    A_rows = _maybe_round(A_rows, bf16)
    Y_rows = _maybe_round(A_rows @ Wo, bf16)
    return {"A_rows": A_rows, "Y_rows": Y_rows}


def check_lens(lens, B: int, N: int) -> np.ndarray:
    lens = np.asarray(lens, dtype=np.int64).reshape(-1)
    if lens.size != B or (lens.size and (lens.min() < 0 or lens.max() > N)):
        raise ValueError("lens must hold B lengths in [0, N]")
    return lens


def sqa_forward_varlen(X, Wq, Wk, Wv, Wo, lens, H_q: int, H_kv: int, d_head: int, causal: bool,
                       bf16: bool, workers: Optional[int] = None) -> np.ndarray:
    """SQA forward over a batch of sequences padded to a common length N.

    The model cards' training examples build their datasets with a maximum
    sequence length (ReactiveAI/xSMQAT-m and ReactiveAI/GQA-Ref-Micro, training
    example), so a batch holds sequences of up to N tokens. Sequence b is the
    first lens[b] rows of X[b]; it is one SQA forward over those tokens alone
    (its keys end at lens[b], whatever the padding rows hold). The pages define
    no output at padding positions; those rows of Y are zero.
    Returns Y [B, N, d_model] as float64.
    """
    X = np.asarray(X, dtype=np.float64)
    B, N, D = check_shapes(X, Wq, Wk, Wv, Wo, H_q, H_kv, d_head)
    lens = check_lens(lens, B, N)
    Y = np.zeros((B, N, D), dtype=np.float64)
    for b in range(B):
        L = int(lens[b])
        if L:
            Y[b, :L] = sqa_forward(X[b:b + 1, :L], Wq, Wk, Wv, Wo, H_q, H_kv, d_head, causal, bf16,
                                   workers=workers)["Y"][0]
    return Y


def sqa_forward_varlen_rows(X, Wq, Wk, Wv, Wo, lens, H_q: int, H_kv: int, d_head: int,
                            causal: bool, bf16: bool, rows: Iterable[int],
                            workers: Optional[int] = None) -> np.ndarray:
    """sqa_forward_varlen evaluated only at the flat rows ``rows`` (row = b*N + t).
    Returns Y_rows [R, d_model] in the order of ``rows``."""
    X = np.asarray(X, dtype=np.float64)
    B, N, D = check_shapes(X, Wq, Wk, Wv, Wo, H_q, H_kv, d_head)
    lens = check_lens(lens, B, N)
    rows = np.asarray(list(rows), dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= B * N):
        raise ValueError("row index out of range")
    Y_rows = np.zeros((rows.size, D), dtype=np.float64)
    for b in np.unique(rows // N):
        b = int(b)
        L = int(lens[b])
        sel = np.nonzero((rows // N == b) & (rows % N < L))[0]
        if sel.size:
            Y_rows[sel] = sqa_forward_rows(X[b:b + 1, :L], Wq, Wk, Wv, Wo, H_q, H_kv, d_head, causal,
                                           bf16, rows=rows[sel] % N, workers=workers)["Y_rows"]
    return Y_rows
