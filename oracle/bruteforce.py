"""Element-by-element SQA forward in plain Python, for tiny inputs only.

TEST INFRASTRUCTURE. It pins the vectorised oracle (``sqa_oracle``) against
the same definition written as explicit scalar loops. It has its own scalar
bfloat16 rounding and shares no code with ``sqa_oracle``.

Definition followed (the method as described in "Sparse Query Attention
(SQA): A Computationally Efficient Attention Mechanism with Query Heads
Reduction", abstract, and the ReactiveAI/GQA-Ref-Micro and ReactiveAI/xSMQAT-m
model card descriptions): H_q query heads; query head i uses key/value head
floor(i / (H_q/H_kv)); scaled dot-product scores; softmax over the visible keys;
weighted sum of values; heads concatenated in head order; output projection.
"""
from __future__ import annotations

import math


def _bf16_scalar(x: float) -> float:
    """Nearest bfloat16 to a float (ties to even). Finite values of normal
    bfloat16 magnitude only, which is all the tiny tests use."""
    if x == 0.0 or math.isnan(x) or math.isinf(x):
        return x
    m, e = math.frexp(x)               # x = m * 2**e, 0.5 <= |m| < 1
    if e - 1 < -126 or e - 1 > 127:
        raise ValueError("outside the normal bfloat16 range")
    n = round(m * 256.0)               # Python round(): ties to even
    return math.ldexp(n, e - 8)


def sqa_forward_bruteforce(X, Wq, Wk, Wv, Wo, H_q, H_kv, d_head, causal, bf16):
    """X is indexed X[b][t][c]; weights W[in][out]. Returns Y as nested lists
    [B][N][d_model] of floats, and A as [B][N][H_q*d_head]."""
    rnd = _bf16_scalar if bf16 else (lambda v: v)
    B, N, D = len(X), len(X[0]), len(X[0][0])
    g = H_q // H_kv
    scale = 1.0 / math.sqrt(d_head)

    def proj(W, width):
        return [[[rnd(sum(float(X[b][t][c]) * float(W[c][o]) for c in range(D)))
                  for o in range(width)] for t in range(N)] for b in range(B)]

    q = proj(Wq, H_q * d_head)
    k = proj(Wk, H_kv * d_head)
    v = proj(Wv, H_kv * d_head)

    A = [[[0.0] * (H_q * d_head) for _ in range(N)] for _ in range(B)]
    for b in range(B):
        for i in range(H_q):
            h = i // g
            for r in range(N):
                visible = [c for c in range(N) if (not causal) or c <= r]
                scores = []
                for c in visible:
                    dot = 0.0
                    for j in range(d_head):
                        dot += q[b][r][i * d_head + j] * k[b][c][h * d_head + j]
                    scores.append(dot * scale)
                top = max(scores)
                w = [math.exp(s - top) for s in scores]
                z = sum(w)
                for j in range(d_head):
                    acc = 0.0
                    for wc, c in zip(w, visible):
                        acc += wc * v[b][c][h * d_head + j]
                    A[b][r][i * d_head + j] = rnd(acc / z)

    Y = [[[rnd(sum(A[b][t][c] * float(Wo[c][o]) for c in range(H_q * d_head)))
           for o in range(D)] for t in range(N)] for b in range(B)]
    return Y, A
