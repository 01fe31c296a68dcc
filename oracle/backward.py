"""Plain float64 CPU oracle for the gradients of the SQA forward pass.

TEST INFRASTRUCTURE. This module checks the HIP path; it is not part of it.
Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
it. It shares no code with the HIP library.

What it computes. The model cards (ReactiveAI/GQA-Ref-Micro and
ReactiveAI/xSMQAT-m, training examples) train the SQA layer in bf16 autocast;
the paper's abstract puts SQA's gains in training and full-sequence
processing. The pages print no backward pass, so this is the gradient of the
forward defined in ``sqa_oracle`` (same reading), by the chain rule:

    L = sum(Y * dY) for a given upstream gradient dY [B, N, d_model]
    dA = dY Wo^T                 dWo = A^T dY          (A as stored by the forward)
    per query head i, key/value head j = floor(i / (H_q/H_kv)):
        dO = dA[:, head i]       P = softmax(Q_i K_j^T / sqrt(d) [+ causal mask])
        O = P V_j (exact)        D = rowsum(dO * O)
        dP = dO V_j^T            dS = P * (dP - D)          (softmax backward)
        dQ_i = dS K_j / sqrt(d)
        dK_j += dS^T Q_i / sqrt(d),  dV_j += P^T dO        (sum over the g heads of j)
    dX = dQ Wq^T + dK Wk^T + dV Wv^T
    dWq = X^T dQ, dWk = X^T dK, dWv = X^T dV          (summed over the batch)

With ``bf16=True`` the forward rounds as in ``sqa_oracle`` (Q, K, V, A, Y),
and a rounding step counts as the identity in the derivative, as autograd
treats a dtype cast. The gradients are rounded once to bfloat16 where an
autocast bf16 run stores a tensor: dA, dQ, dK, dV (the attention backward's
outputs), dX, and each weight gradient. Everything between those points is
float64; in particular D uses the exact O = P V, not the rounded A.

Evaluation order: each head's query rows are taken in blocks, which only
bounds memory; every sum is the definition above.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

from .sqa_oracle import (_maybe_round, _pool_workers, _run_tasks, check_shapes, kv_head_for,
                         split_heads, sqa_forward)


def softmax_backward(P: np.ndarray, dP: np.ndarray, D: np.ndarray) -> np.ndarray:
    """dS = P * (dP - D): gradient of the scores through a row softmax whose
    output P received gradient dP, with D = rowsum(dP * P) given per row."""
    return P * (dP - D[:, None])


def attention_head_backward(q, k, v, do, causal: bool, row_block: int = 512):
    """Gradients of one query head through softmax(q k^T / sqrt(d)) v.

    q [N, d], k, v [N, d], do [N, d]. Returns (dq, dk, dv) of that head alone
    (dk, dv before the sum over the heads that share k, v)."""
    N, d = q.shape
    scale = 1.0 / math.sqrt(d)
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, N, row_block):
        r1 = min(N, r0 + row_block)
        n_keys = r1 if causal else N          # later keys are masked for every row here
        s = (q[r0:r1] @ k[:n_keys].T) * scale
        if causal:
            s = np.where(np.arange(n_keys)[None, :] <= np.arange(r0, r1)[:, None], s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        e = np.exp(s)
        p = e / e.sum(axis=1, keepdims=True)
        o = p @ v[:n_keys]
        D = np.sum(do[r0:r1] * o, axis=1)
        dp = do[r0:r1] @ v[:n_keys].T
        ds = softmax_backward(p, dp, D)
        dq[r0:r1] = (ds @ k[:n_keys]) * scale
        dk[:n_keys] += (ds.T @ q[r0:r1]) * scale
        dv[:n_keys] += p.T @ do[r0:r1]
    return dq, dk, dv


def sqa_backward(X, Wq, Wk, Wv, Wo, dY, H_q: int, H_kv: int, d_head: int, causal: bool,
                 bf16: bool, workers: Optional[int] = None, row_block: int = 512
                 ) -> Dict[str, np.ndarray]:
    """Gradients of L = sum(Y * dY) with respect to X, Wq, Wk, Wv and Wo.

    Returns float64 arrays dX [B,N,d_model], dWq, dWk, dWv, dWo (shapes of the
    weights) and the intermediates dA [B,N,H_q*d], dQ, dK, dV (the layouts of
    Q, K, V: [B,N,heads*d])."""
    X, Wq, Wk, Wv, Wo, dY = (np.asarray(t, dtype=np.float64) for t in (X, Wq, Wk, Wv, Wo, dY))
    B, N, D = check_shapes(X, Wq, Wk, Wv, Wo, H_q, H_kv, d_head)
    if dY.shape != (B, N, D):
        raise ValueError(f"dY has shape {dY.shape}, expected {(B, N, D)}")
    fwd = sqa_forward(X, Wq, Wk, Wv, Wo, H_q, H_kv, d_head, causal, bf16, workers=workers)
    Qh = split_heads(fwd["Q"], H_q, d_head)
    Kh = split_heads(fwd["K"], H_kv, d_head)
    Vh = split_heads(fwd["V"], H_kv, d_head)
    dA = _maybe_round(dY @ Wo.T, bf16)
    dAh = split_heads(dA, H_q, d_head)
    dQh = np.empty((B, H_q, N, d_head))
    dK_head = np.empty((B, H_q, N, d_head))   # each query head's share of dK and dV
    dV_head = np.empty((B, H_q, N, d_head))

    def one(task):   # query head i of batch b
        b, i = task
        j = kv_head_for(i, H_q, H_kv)
        dQh[b, i], dK_head[b, i], dV_head[b, i] = attention_head_backward(
            Qh[b, i], Kh[b, j], Vh[b, j], dAh[b, i], causal, row_block)

    _run_tasks(one, [(b, i) for b in range(B) for i in range(H_q)], _pool_workers(workers))
    dKh = np.zeros((B, H_kv, N, d_head))
    dVh = np.zeros((B, H_kv, N, d_head))
    for i in range(H_q):   # dK_j, dV_j: sums over the query heads i of group j, in head order
        j = kv_head_for(i, H_q, H_kv)
        dKh[:, j] += dK_head[:, i]
        dVh[:, j] += dV_head[:, i]

    def merge(h):   # [B, heads, N, d] -> [B, N, heads*d], head-major columns
        return h.transpose(0, 2, 1, 3).reshape(B, N, -1)

    dQ = _maybe_round(merge(dQh), bf16)
    dK = _maybe_round(merge(dKh), bf16)
    dV = _maybe_round(merge(dVh), bf16)
    dX = _maybe_round(dQ @ Wq.T + dK @ Wk.T + dV @ Wv.T, bf16)
    Xf = X.reshape(B * N, D)
    dWq = _maybe_round(Xf.T @ dQ.reshape(B * N, -1), bf16)
    dWk = _maybe_round(Xf.T @ dK.reshape(B * N, -1), bf16)
    dWv = _maybe_round(Xf.T @ dV.reshape(B * N, -1), bf16)
    dWo = _maybe_round(fwd["A"].reshape(B * N, -1).T @ dY.reshape(B * N, D), bf16)
    return {"dX": dX, "dWq": dWq, "dWk": dWk, "dWv": dWv, "dWo": dWo,
            "dA": dA, "dQ": dQ, "dK": dK, "dV": dV}


def sqa_backward_rows(X, Wq, Wk, Wv, Wo, dY, H_q: int, H_kv: int, d_head: int, causal: bool,
                      bf16: bool, rows, workers: Optional[int] = None, row_block: int = 128
                      ) -> Dict[str, np.ndarray]:
    """dX of ``sqa_backward`` evaluated only at the flat token rows ``rows``
    (row = b*N + t), with the same definitions and rounding points.

    Row t of dX takes row t of dQ, dK and dV. dQ[t] needs query row t's
    softmax; dK[t] and dV[t] need every query row that attends key t: rows
    t..N-1 when causal, all rows otherwise. Per sequence this evaluates the
    query rows from the first sampled position on (all of them without the
    mask) against all keys, so it is cheap for rows near the end of a causal
    sequence. Returns dX_rows [R, d_model] and dQ_rows, dK_rows, dV_rows
    [R, heads*d] in the order of ``rows``.
    """
    X, Wq, Wk, Wv, Wo, dY = (np.asarray(t, dtype=np.float64) for t in (X, Wq, Wk, Wv, Wo, dY))
    B, N, D = check_shapes(X, Wq, Wk, Wv, Wo, H_q, H_kv, d_head)
    if dY.shape != (B, N, D):
        raise ValueError(f"dY has shape {dY.shape}, expected {(B, N, D)}")
    rows = np.asarray(list(rows), dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= B * N):
        raise ValueError("row index out of range")
    d = d_head
    scale = 1.0 / math.sqrt(d)
    dQr = np.zeros((rows.size, H_q * d))
    dKr = np.zeros((rows.size, H_kv * d))
    dVr = np.zeros((rows.size, H_kv * d))
    for b in np.unique(rows // N):
        b = int(b)
        sel = np.nonzero(rows // N == b)[0]
        pos = rows[sel] % N
        lo = int(pos.min()) if causal else 0      # earlier query rows attend no sampled key
        Kb = _maybe_round(X[b] @ Wk, bf16)
        Vb = _maybe_round(X[b] @ Wv, bf16)
        Qr = _maybe_round(X[b, lo:] @ Wq, bf16)
        dAr = _maybe_round(dY[b, lo:] @ Wo.T, bf16)
        qpos = np.arange(lo, N)

        def one(j):   # every query head of key/value head j
            kc = slice(j * d, (j + 1) * d)
            k, v = Kb[:, kc], Vb[:, kc]
            for i in range(H_q):
                if kv_head_for(i, H_q, H_kv) != j:
                    continue
                hc = slice(i * d, (i + 1) * d)
                for r0 in range(0, qpos.size, row_block):
                    r1 = min(qpos.size, r0 + row_block)
                    q, do = Qr[r0:r1, hc], dAr[r0:r1, hc]
                    s = (q @ k.T) * scale
                    if causal:
                        s = np.where(np.arange(N)[None, :] <= qpos[r0:r1, None], s, -np.inf)
                    s = s - s.max(axis=1, keepdims=True)
                    e = np.exp(s)
                    p = e / e.sum(axis=1, keepdims=True)
                    o = p @ v
                    Dr = np.sum(do * o, axis=1)
                    ds = softmax_backward(p, do @ v.T, Dr)
                    here = np.nonzero((pos >= qpos[r0]) & (pos < qpos[r1 - 1] + 1))[0]
                    if here.size:
                        dQr[sel[here], hc] = (ds[pos[here] - qpos[r0]] @ k) * scale
                    dKr[sel, kc] += (ds[:, pos].T @ q) * scale
                    dVr[sel, kc] += p[:, pos].T @ do

        _run_tasks(one, list(range(H_kv)), _pool_workers(workers))
    dQr, dKr, dVr = (_maybe_round(t, bf16) for t in (dQr, dKr, dVr))
    dXr = _maybe_round(dQr @ Wq.T + dKr @ Wk.T + dVr @ Wv.T, bf16)
    return {"dX_rows": dXr, "dQ_rows": dQr, "dK_rows": dKr, "dV_rows": dVr}


def sqa_backward_dy_rows(X, Wq, Wk, Wv, Wo, dY, H_q: int, H_kv: int, d_head: int, causal: bool,
                         bf16: bool, rows, workers: Optional[int] = None, row_block: int = 128
                         ) -> Dict[str, np.ndarray]:
    """``sqa_backward`` for an upstream gradient dY that is zero outside the
    flat token rows ``rows`` (row = b*N + t); it raises if dY is not.

    Every result is the one ``sqa_backward`` defines, at every position. Only
    work that is exactly zero is left out: a query row r with dY[r] = 0 has
    dA[r] = 0, so dO = 0, D = 0, dP = 0 and dS = 0 in that row, and it adds
    nothing to dQ, dK or dV. So only the given query rows run the forward and
    the softmax backward, each against all of its keys (keys 0..r when
    causal); dK and dV are summed from those rows for every key, and dX and
    the weight gradients are formed over all tokens as in ``sqa_backward``.
    Returns dX [B,N,d_model], dWq, dWk, dWv, dWo and dQ, dK, dV [B,N,heads*d].
    """
    X, Wq, Wk, Wv, Wo, dY = (np.asarray(t, dtype=np.float64) for t in (X, Wq, Wk, Wv, Wo, dY))
    B, N, D = check_shapes(X, Wq, Wk, Wv, Wo, H_q, H_kv, d_head)
    if dY.shape != (B, N, D):
        raise ValueError(f"dY has shape {dY.shape}, expected {(B, N, D)}")
    rows = np.unique(np.asarray(list(rows), dtype=np.int64))
    if rows.size and (rows.min() < 0 or rows.max() >= B * N):
        raise ValueError("row index out of range")
    outside = np.ones(B * N, dtype=bool)
    outside[rows] = False
    if np.any(dY.reshape(B * N, D)[outside] != 0):
        raise ValueError("dY is nonzero outside the given rows")
    d = d_head
    scale = 1.0 / math.sqrt(d)
    dQh = np.zeros((B, H_q, N, d))
    dKh = np.zeros((B, H_kv, N, d))
    dVh = np.zeros((B, H_kv, N, d))
    A = np.zeros((B, N, H_q * d))
    for b in np.unique(rows // N):
        b = int(b)
        pos = rows[rows // N == b] % N
        n_keys = int(pos.max()) + 1 if causal else N   # later keys are masked for every row
        Kb = split_heads(_maybe_round(X[b:b + 1, :n_keys] @ Wk, bf16), H_kv, d)[0]
        Vb = split_heads(_maybe_round(X[b:b + 1, :n_keys] @ Wv, bf16), H_kv, d)[0]
        Qr = _maybe_round(X[b, pos] @ Wq, bf16)
        dAr = _maybe_round(dY[b, pos] @ Wo.T, bf16)

        def one(j):   # every query head of key/value head j
            k, v = Kb[j], Vb[j]
            for i in range(H_q):
                if kv_head_for(i, H_q, H_kv) != j:
                    continue
                hc = slice(i * d, (i + 1) * d)
                for r0 in range(0, pos.size, row_block):
                    r1 = min(pos.size, r0 + row_block)
                    nk = int(pos[r1 - 1]) + 1 if causal else N
                    q, do = Qr[r0:r1, hc], dAr[r0:r1, hc]
                    s = (q @ k[:nk].T) * scale
                    if causal:
                        s = np.where(np.arange(nk)[None, :] <= pos[r0:r1, None], s, -np.inf)
                    s = s - s.max(axis=1, keepdims=True)
                    e = np.exp(s)
                    p = e / e.sum(axis=1, keepdims=True)
                    o = p @ v[:nk]
                    A[b, pos[r0:r1], hc] = o
                    Dr = np.sum(do * o, axis=1)
                    ds = softmax_backward(p, do @ v[:nk].T, Dr)
                    dQh[b, i, pos[r0:r1]] = (ds @ k[:nk]) * scale
                    dKh[b, j, :nk] += (ds.T @ q) * scale
                    dVh[b, j, :nk] += p.T @ do

        _run_tasks(one, list(range(H_kv)), _pool_workers(workers))

    def merge(h):   # [B, heads, N, d] -> [B, N, heads*d], head-major columns
        return h.transpose(0, 2, 1, 3).reshape(B, N, -1)

    dQ = _maybe_round(merge(dQh), bf16)
    dK = _maybe_round(merge(dKh), bf16)
    dV = _maybe_round(merge(dVh), bf16)
    dX = _maybe_round(dQ @ Wq.T + dK @ Wk.T + dV @ Wv.T, bf16)
    Xf = X.reshape(B * N, D)
    dWq = _maybe_round(Xf.T @ dQ.reshape(B * N, -1), bf16)
    dWk = _maybe_round(Xf.T @ dK.reshape(B * N, -1), bf16)
    dWv = _maybe_round(Xf.T @ dV.reshape(B * N, -1), bf16)
    # A's rows outside `rows` meet zero rows of dY
    dWo = _maybe_round(_maybe_round(A, bf16).reshape(B * N, -1).T @ dY.reshape(B * N, D), bf16)
    return {"dX": dX, "dWq": dWq, "dWk": dWk, "dWv": dWv, "dWo": dWo, "dQ": dQ, "dK": dK, "dV": dV}
