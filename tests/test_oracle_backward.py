"""Pins of the backward oracle (oracle/backward.py) to things other than itself (CPU only).

* Finite differences: central differences of L = sum(Y * dY), with Y from the
  scalar brute-force forward (oracle/bruteforce.py), along random directions
  of every input, against the oracle's gradients (float64, no rounding).
* torch autograd: a forward written here with torch float64 ops (GQA through
  repeat_interleave) differentiated by autograd, with bf16 rounding placed as
  a cast whose backward rounds the incoming gradient. This pins the float64
  gradients and where the bf16 mode rounds.
* Planted mistakes in the oracle (a dropped softmax term, a wrong head map, a
  missing score scale, no rounding) must fail those pins.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as sb
from oracle.bruteforce import sqa_forward_bruteforce


def _problem(seed, B, N, H, d, H_q, H_kv):
    rng = np.random.default_rng(seed)
    D = H * d
    X = rng.standard_normal((B, N, D))
    Wq = rng.standard_normal((D, H_q * d)) / math.sqrt(D)
    Wk = rng.standard_normal((D, H_kv * d)) / math.sqrt(D)
    Wv = rng.standard_normal((D, H_kv * d)) / math.sqrt(D)
    Wo = rng.standard_normal((H_q * d, D)) / math.sqrt(D)
    dY = rng.standard_normal((B, N, D))
    return [X, Wq, Wk, Wv, Wo], dY


NAMES = ["X", "Wq", "Wk", "Wv", "Wo"]
GRADS = ["dX", "dWq", "dWk", "dWv", "dWo"]


def _loss(params, dY, H_q, H_kv, d, causal):
    Y, _ = sqa_forward_bruteforce(*params, H_q, H_kv, d, causal, False)
    return float(np.sum(np.asarray(Y) * dY))


def _fd_errors(grads, params, dY, H_q, H_kv, d, causal, seed=5, h=1e-5):
    """Relative error of <grad, E> against the central difference along E, per input."""
    rng = np.random.default_rng(seed)
    errs = {}
    for name, gname, idx in zip(NAMES, GRADS, range(5)):
        E = rng.standard_normal(params[idx].shape)
        plus = [p.copy() for p in params]
        minus = [p.copy() for p in params]
        plus[idx] = plus[idx] + h * E
        minus[idx] = minus[idx] - h * E
        fd = (_loss(plus, dY, H_q, H_kv, d, causal) - _loss(minus, dY, H_q, H_kv, d, causal)) / (2 * h)
        an = float(np.sum(grads[gname] * E))
        errs[name] = abs(fd - an) / max(1.0, abs(an))
    return errs


FD_CASES = [(4, 2, 2, 1, False), (4, 2, 2, 1, True), (4, 2, 4, 2, True), (4, 2, 4, 4, False),
            (4, 2, 4, 1, True)]


@pytest.mark.parametrize("H,d,H_q,H_kv,causal", FD_CASES)
def test_gradients_match_finite_differences(H, d, H_q, H_kv, causal):
    params, dY = _problem(11 + H_q + 3 * H_kv, 2, 5, H, d, H_q, H_kv)
    g = oracle.sqa_backward(*params, dY, H_q, H_kv, d, causal, bf16=False, workers=1)
    errs = _fd_errors(g, params, dY, H_q, H_kv, d, causal)
    assert max(errs.values()) < 1e-7, errs


class _RoundBf16(torch.autograd.Function):
    """A bf16 cast in an autocast graph: rounds the value on the way in and
    the gradient on the way back."""

    @staticmethod
    def forward(ctx, x):
        return x.to(torch.bfloat16).to(torch.float64)

    @staticmethod
    def backward(ctx, g):
        return g.to(torch.bfloat16).to(torch.float64)


def _torch_grads(params, dY, H_q, H_kv, d, causal, bf16):
    t = [torch.tensor(p, dtype=torch.float64, requires_grad=True) for p in params]
    x, wq, wk, wv, wo = t
    R = _RoundBf16.apply if bf16 else (lambda v: v)
    B, N, D = x.shape
    q = R(x @ wq).view(B, N, H_q, d).transpose(1, 2)
    k = R(x @ wk).view(B, N, H_kv, d).transpose(1, 2).repeat_interleave(H_q // H_kv, dim=1)
    v = R(x @ wv).view(B, N, H_kv, d).transpose(1, 2).repeat_interleave(H_q // H_kv, dim=1)
    s = (q @ k.transpose(-1, -2)) / math.sqrt(d)
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
    o = torch.softmax(s, dim=-1) @ v
    a = R(o.transpose(1, 2).reshape(B, N, H_q * d))
    y = R(a @ wo)
    (y * torch.from_numpy(dY)).sum().backward()
    out = {}
    for name, gname, p in zip(NAMES, GRADS, t):
        gr = p.grad
        out[gname] = (gr.to(torch.bfloat16).to(torch.float64) if bf16 else gr).numpy()
    return out


def _rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


AUTOGRAD_CASES = [(4, 8, 4, 2, True), (4, 8, 4, 2, False), (8, 8, 4, 1, True), (4, 8, 4, 4, True),
                  (8, 4, 8, 2, False)]


@pytest.mark.parametrize("H,d,H_q,H_kv,causal", AUTOGRAD_CASES)
@pytest.mark.parametrize("bf16", [False, True])
def test_gradients_match_torch_autograd(H, d, H_q, H_kv, causal, bf16):
    params, dY = _problem(40 + H + H_q, 2, 37, H, d, H_q, H_kv)
    if bf16:
        params = [oracle.round_bf16(p) for p in params]
        dY = oracle.round_bf16(dY)
    g = oracle.sqa_backward(*params, dY, H_q, H_kv, d, causal, bf16=bf16, row_block=16)
    ref = _torch_grads(params, dY, H_q, H_kv, d, causal, bf16)
    for k in GRADS:
        err = _rel_l2(g[k], ref[k])
        assert err < (1e-5 if bf16 else 1e-12), (k, err)
        if bf16:
            assert np.array_equal(oracle.round_bf16(g[k]), g[k]), k   # on the bf16 grid


def test_intermediates_have_the_forward_layouts():
    params, dY = _problem(3, 2, 9, 4, 4, 4, 2)
    g = oracle.sqa_backward(*params, dY, 4, 2, 4, True, bf16=False)
    assert g["dA"].shape == (2, 9, 16) and g["dQ"].shape == (2, 9, 16)
    assert g["dK"].shape == (2, 9, 8) and g["dV"].shape == (2, 9, 8)
    # dWq = X^T dQ and dX's query part: the intermediates are the ones the outputs use
    X = params[0].reshape(18, 16)
    assert np.allclose(g["dWq"], X.T @ g["dQ"].reshape(18, 16), rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------------------------
# sampled rows: sqa_backward_rows is sqa_backward (pinned above) restricted to some rows of dX

@pytest.mark.parametrize("causal,bf16,H_q,H_kv", [(True, False, 4, 2), (True, True, 4, 2),
                                                  (False, False, 2, 1), (False, True, 4, 4),
                                                  (True, True, 4, 1)])
def test_backward_rows_are_the_full_backward_at_those_rows(causal, bf16, H_q, H_kv):
    d, N, B = 4, 41, 2
    params, dY = _problem(91, B, N, 4, d, H_q, H_kv)
    if bf16:
        params = [oracle.round_bf16(p) for p in params]
        dY = oracle.round_bf16(dY)
    full = oracle.sqa_backward(*params, dY, H_q, H_kv, d, causal, bf16=bf16)
    rows = [0, 1, 17, 40, N + 0, N + 23, N + 39, N + 40, 17]   # both sequences, ends, a repeat
    got = oracle.sqa_backward_rows(*params, dY, H_q, H_kv, d, causal, bf16, rows, row_block=8)
    flat = {k: full[k].reshape(B * N, -1) for k in ("dX", "dQ", "dK", "dV")}
    for k in ("dX", "dQ", "dK", "dV"):
        np.testing.assert_allclose(got[k + "_rows"], flat[k][rows], rtol=1e-12, atol=1e-14,
                                   err_msg=k)


def test_backward_rows_late_causal_rows_skip_the_early_queries():
    """Causal rows near the end evaluate only the query rows from the first
    sampled position on; the result is still the full backward's."""
    d, N, H_q, H_kv = 4, 64, 2, 1
    params, dY = _problem(92, 1, N, 2, d, H_q, H_kv)
    full = oracle.sqa_backward(*params, dY, H_q, H_kv, d, True, bf16=False)
    rows = [N - 1, N - 5, N - 9]
    got = oracle.sqa_backward_rows(*params, dY, H_q, H_kv, d, True, False, rows)
    np.testing.assert_allclose(got["dX_rows"], full["dX"][0, rows], rtol=1e-12, atol=1e-14)


def test_backward_rows_reject_bad_rows():
    params, dY = _problem(93, 1, 5, 2, 4, 2, 1)
    with pytest.raises(ValueError):
        oracle.sqa_backward_rows(*params, dY, 2, 1, 4, True, False, [5])


# ----------------------------------------------------------------------------------------------
# an upstream gradient on a few rows: sqa_backward_dy_rows against autograd and the full backward

def _dy_on_rows(dY, rows):
    B, N, D = dY.shape
    out = np.zeros_like(dY).reshape(B * N, D)
    out[rows] = dY.reshape(B * N, D)[rows]
    return out.reshape(B, N, D)


DY_ROWS_CASES = [(True, False, 4, 2), (True, True, 4, 2), (False, False, 4, 1),
                 (False, True, 2, 2), (True, True, 8, 1)]


@pytest.mark.parametrize("causal,bf16,H_q,H_kv", DY_ROWS_CASES)
def test_dy_rows_backward_matches_torch_autograd(causal, bf16, H_q, H_kv):
    """Every gradient, at every position, against autograd through a forward
    written with torch ops, for dY zero outside a few rows of each sequence."""
    d, N, B = 4, 37, 2
    params, dY = _problem(95 + H_q, B, N, 8, d, H_q, H_kv)
    rows = [3, 4, 20, 36, N + 0, N + 30]
    dY = _dy_on_rows(dY, rows)
    if bf16:
        params = [oracle.round_bf16(p) for p in params]
        dY = oracle.round_bf16(dY)
    g = oracle.sqa_backward_dy_rows(*params, dY, H_q, H_kv, d, causal, bf16, rows, row_block=2)
    ref = _torch_grads(params, dY, H_q, H_kv, d, causal, bf16)
    for k in GRADS:
        err = _rel_l2(g[k], ref[k])
        assert err < (1e-5 if bf16 else 1e-12), (k, err)
    if causal:   # keys past the last row carrying dY get nothing
        assert not g["dX"][1, 31:].any() and g["dX"][1, 30].any()


def test_dy_rows_backward_is_the_full_backward():
    d, N, B, H_q, H_kv = 4, 50, 1, 4, 2
    params, dY = _problem(96, B, N, 4, d, H_q, H_kv)
    rows = list(range(10, 19)) + [44]
    dY = _dy_on_rows(dY, rows)
    full = oracle.sqa_backward(*params, dY, H_q, H_kv, d, True, bf16=False)
    got = oracle.sqa_backward_dy_rows(*params, dY, H_q, H_kv, d, True, False, rows, row_block=4)
    for k in GRADS + ["dQ", "dK", "dV"]:
        np.testing.assert_allclose(got[k], full[k], rtol=1e-12, atol=1e-14, err_msg=k)


def test_dy_rows_backward_rejects_dy_outside_the_rows():
    params, dY = _problem(97, 1, 6, 2, 4, 2, 1)
    with pytest.raises(ValueError):
        oracle.sqa_backward_dy_rows(*params, dY, 2, 1, 4, True, False, [0, 1, 2])
    with pytest.raises(ValueError):
        oracle.sqa_backward_dy_rows(*params, _dy_on_rows(dY, [1]), 2, 1, 4, True, False, [6])


# ----------------------------------------------------------------------------------------------
# planted mistakes: each must make a pin fail

def _fd_fails(monkeypatch_apply, case=(4, 2, 4, 2, True)):
    H, d, H_q, H_kv, causal = case
    params, dY = _problem(7, 2, 5, H, d, H_q, H_kv)
    g = oracle.sqa_backward(*params, dY, H_q, H_kv, d, causal, bf16=False, workers=1)
    return max(_fd_errors(g, params, dY, H_q, H_kv, d, causal).values()) > 1e-4


def test_planted_dropped_softmax_term_is_caught(monkeypatch):
    monkeypatch.setattr(sb, "softmax_backward", lambda P, dP, D: P * dP)
    assert _fd_fails(None)


def test_planted_wrong_head_map_is_caught(monkeypatch):
    monkeypatch.setattr(sb, "kv_head_for", lambda i, H_q, H_kv: i % H_kv)
    assert _fd_fails(None)


def test_planted_missing_key_scale_is_caught(monkeypatch):
    real = sb.attention_head_backward

    def wrong(q, k, v, do, causal, row_block=512):
        dq, dk, dv = real(q, k, v, do, causal, row_block)
        return dq, dk * math.sqrt(q.shape[1]), dv
    monkeypatch.setattr(sb, "attention_head_backward", wrong)
    assert _fd_fails(None)


def test_planted_missing_rounding_is_caught(monkeypatch):
    H, d, H_q, H_kv, causal = 4, 8, 4, 2, True
    params, dY = _problem(44, 2, 37, H, d, H_q, H_kv)
    params = [oracle.round_bf16(p) for p in params]
    dY = oracle.round_bf16(dY)
    ref = _torch_grads(params, dY, H_q, H_kv, d, causal, True)
    real = sb._maybe_round
    monkeypatch.setattr(sb, "_maybe_round", lambda a, bf16: a)   # dA, dQ, dK, dV kept exact
    g = oracle.sqa_backward(*params, dY, H_q, H_kv, d, causal, bf16=True)
    g = {k: real(v, True) for k, v in g.items()}
    assert max(_rel_l2(g[k], ref[k]) for k in GRADS) > 1e-5
