"""Pins of the CPU oracle to things other than itself (CPU only).

Each test ties the oracle to the mathematics or to an independent routine:
hand-derived closed forms (tests/golden), a brute-force scalar loop, textbook
MHA written with torch, torch's SDPA with grouped heads, and invariants of
softmax attention. The last tests plant mistakes in the oracle and check that
the pins catch them.
"""
import glob
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import sqa_oracle
from oracle.bruteforce import sqa_forward_bruteforce, _bf16_scalar

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------------------------
# helpers

def _rand_problem(seed, B, N, H, d_head, H_q, H_kv, scale_x=1.0):
    rng = np.random.default_rng(seed)
    D = H * d_head
    X = rng.standard_normal((B, N, D)) * scale_x
    Wq = rng.standard_normal((D, H_q * d_head)) / math.sqrt(D)
    Wk = rng.standard_normal((D, H_kv * d_head)) / math.sqrt(D)
    Wv = rng.standard_normal((D, H_kv * d_head)) / math.sqrt(D)
    Wo = rng.standard_normal((H_q * d_head, D)) / math.sqrt(D)
    return X, Wq, Wk, Wv, Wo


def _parse(v):
    v = v.strip()
    if "ln(" in v:
        coef, _, rest = v.partition("ln(")
        c = float(Fraction(coef.rstrip("*"))) if coef else 1.0
        return c * math.log(float(Fraction(rest.rstrip(")"))))
    return float(Fraction(v))


def _arr(nested):
    return np.vectorize(_parse, otypes=[np.float64])(np.array(nested, dtype=object))


def _textbook_mha(X, Wq, Wk, Wv, Wo, H, causal):
    """Standard multi-head attention written with torch float64 ops."""
    x = torch.from_numpy(X)
    B, N, D = x.shape
    d = Wq.shape[1] // H
    q = (x @ torch.from_numpy(Wq)).view(B, N, H, d).transpose(1, 2)
    k = (x @ torch.from_numpy(Wk)).view(B, N, H, d).transpose(1, 2)
    v = (x @ torch.from_numpy(Wv)).view(B, N, H, d).transpose(1, 2)
    s = q @ k.transpose(-1, -2) / math.sqrt(d)
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    a = torch.softmax(s, dim=-1) @ v
    a = a.transpose(1, 2).reshape(B, N, H * d)
    return (a @ torch.from_numpy(Wo)).numpy(), a.numpy()


# ----------------------------------------------------------------------------------------------
# bfloat16 rounding helper

def test_bf16_matches_torch_rne_on_fp32_values():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    # ties: low 16 bits exactly 0x8000, upper half both even and odd
    ties = (rng.integers(0, 2**16, size=20000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    # fp32 subnormals and values around the bf16 overflow threshold
    sub = rng.integers(1, 2**23, size=5000, dtype=np.uint64).astype(np.uint32)
    big = np.arange(0x7F7F0000, 0x7F800000, 7, dtype=np.uint64).astype(np.uint32)
    special = np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000], dtype=np.uint32)
    allbits = np.concatenate([bits, ties, sub, big, special, big | 0x80000000])
    f32 = allbits.view(np.float32)
    with np.errstate(invalid="ignore"):    # signalling NaN patterns
        f64 = f32.astype(np.float64)
    want = torch.from_numpy(f32.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(f64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # signed zeros survive
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


@pytest.mark.parametrize("x,expect", [
    (1 + 2**-8, 1.0),                       # tie between 1 and 1+2^-7 -> even (1)
    (1 + 3 * 2**-8, 1 + 2**-6),             # tie between 1+2^-7 and 1+2^-6 -> even (1+2^-6)
    (1 + 2**-8 + 2**-40, 1 + 2**-7),        # just above the tie rounds up
    (-(1 + 2**-8), -1.0),
    (255.5, 256.0),                         # carry into the next binade (8 significant bits)
    (2**-134, 0.0),                         # half of the smallest subnormal -> even (0)
    (3 * 2**-134, 2**-132),                 # 1.5 quanta -> 2 quanta
    (float.fromhex("0x1.fep127") + 2**119, math.inf),   # max finite + half ulp -> inf
    (float.fromhex("0x1.fep127") + 2**118, float.fromhex("0x1.fep127")),
])
def test_bf16_hand_cases(x, expect):
    assert oracle.round_bf16(np.array([x]))[0] == expect
    if 2**-126 <= abs(x) < 2**127:
        assert _bf16_scalar(x) == expect


# ----------------------------------------------------------------------------------------------
# hand-derived closed forms

@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(GOLDEN, "closed_form_*.json"))))
@pytest.mark.parametrize("causal", [False, True])
def test_golden_closed_forms(path, causal):
    g = json.load(open(path))
    X, Wq, Wk, Wv, Wo = (_arr(g[k]) for k in ("X", "Wq", "Wk", "Wv", "Wo"))
    d_head = g["d_model"] // g["H"]
    want = _arr(g["Y_causal" if causal else "Y_noncausal"])
    out = oracle.sqa_forward(X, Wq, Wk, Wv, Wo, g["H_q"], g["H_kv"], d_head, causal, g["bf16"])
    np.testing.assert_allclose(out["Y"], want, rtol=1e-13, atol=1e-13)
    y_bf, _ = sqa_forward_bruteforce(X, Wq, Wk, Wv, Wo, g["H_q"], g["H_kv"], d_head, causal, g["bf16"])
    np.testing.assert_allclose(np.array(y_bf), want, rtol=1e-13, atol=1e-13)
    rows = list(range(g["B"] * g["N"]))
    r = oracle.sqa_forward_rows(X, Wq, Wk, Wv, Wo, g["H_q"], g["H_kv"], d_head, causal, g["bf16"], rows)
    np.testing.assert_allclose(r["Y_rows"], want.reshape(-1, g["d_model"]), rtol=1e-13, atol=1e-13)


# ----------------------------------------------------------------------------------------------
# brute force on tiny inputs

HEADS = [(4, 4, 4), (4, 4, 2), (4, 4, 1), (4, 2, 1), (4, 2, 2), (4, 1, 1), (8, 8, 2)]


@pytest.mark.parametrize("H,H_q,H_kv", HEADS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bf16", [False, True])
def test_oracle_matches_bruteforce(H, H_q, H_kv, causal, bf16):
    X, Wq, Wk, Wv, Wo = _rand_problem(11 + H_q * 3 + H_kv, B=2, N=5, H=H, d_head=2, H_q=H_q, H_kv=H_kv)
    if bf16:
        X, Wq, Wk, Wv, Wo = (oracle.round_bf16(t) for t in (X, Wq, Wk, Wv, Wo))
    out = oracle.sqa_forward(X, Wq, Wk, Wv, Wo, H_q, H_kv, 2, causal, bf16, row_block=2, workers=3)
    y_bf, a_bf = sqa_forward_bruteforce(X, Wq, Wk, Wv, Wo, H_q, H_kv, 2, causal, bf16)
    np.testing.assert_allclose(out["A"], np.array(a_bf), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out["Y"], np.array(y_bf), rtol=1e-12, atol=1e-14)
    rows = [0, 3, 4, 5, 9]
    r = oracle.sqa_forward_rows(X, Wq, Wk, Wv, Wo, H_q, H_kv, 2, causal, bf16, rows, workers=2)
    np.testing.assert_allclose(r["Y_rows"], np.array(y_bf).reshape(-1, H * 2)[rows], rtol=1e-12,
                               atol=1e-14)


# ----------------------------------------------------------------------------------------------
# reductions to standard attention

@pytest.mark.parametrize("causal", [False, True])
def test_reduces_to_textbook_mha(causal):
    H = 4
    X, Wq, Wk, Wv, Wo = _rand_problem(3, B=2, N=37, H=H, d_head=8, H_q=H, H_kv=H)
    out = oracle.sqa_forward(X, Wq, Wk, Wv, Wo, H, H, 8, causal, False, row_block=16)
    y, a = _textbook_mha(X, Wq, Wk, Wv, Wo, H, causal)
    np.testing.assert_allclose(out["A"], a, rtol=0, atol=1e-12)
    np.testing.assert_allclose(out["Y"], y, rtol=0, atol=1e-12)


@pytest.mark.parametrize("H_q,H_kv", [(4, 2), (4, 1), (8, 2), (6, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_explicit_kv_repeat_is_identical(H_q, H_kv, causal):
    d = 4
    X, Wq, Wk, Wv, Wo = _rand_problem(5, B=2, N=19, H=8, d_head=d, H_q=H_q, H_kv=H_kv)
    g = H_q // H_kv
    rep = lambda W: np.repeat(W.reshape(W.shape[0], H_kv, d), g, axis=1).reshape(W.shape[0], H_q * d)
    grouped = oracle.sqa_forward(X, Wq, Wk, Wv, Wo, H_q, H_kv, d, causal, False)
    repeated = oracle.sqa_forward(X, Wq, rep(Wk), rep(Wv), Wo, H_q, H_q, d, causal, False)
    # identical up to the BLAS summation order of the wider projection matmul
    np.testing.assert_allclose(repeated["A"], grouped["A"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(repeated["Y"], grouped["Y"], rtol=0, atol=1e-13)


@pytest.mark.parametrize("H_q,H_kv", [(4, 4), (4, 2), (4, 1), (8, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_enable_gqa(H_q, H_kv, causal):
    d = 8
    X, Wq, Wk, Wv, Wo = _rand_problem(9, B=2, N=33, H=8, d_head=d, H_q=H_q, H_kv=H_kv)
    out = oracle.sqa_forward(X, Wq, Wk, Wv, Wo, H_q, H_kv, d, causal, False)
    x = torch.from_numpy(X)
    q = (x @ torch.from_numpy(Wq)).view(2, 33, H_q, d).transpose(1, 2)
    k = (x @ torch.from_numpy(Wk)).view(2, 33, H_kv, d).transpose(1, 2)
    v = (x @ torch.from_numpy(Wv)).view(2, 33, H_kv, d).transpose(1, 2)
    a = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, enable_gqa=True)
    a = a.transpose(1, 2).reshape(2, 33, H_q * d).numpy()
    np.testing.assert_allclose(out["A"], a, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------------------------
# softmax invariants and closed forms

@pytest.mark.parametrize("causal", [False, True])
def test_softmax_rows_sum_to_one(causal):
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal((50, 16)) * 4, rng.standard_normal((70, 16)) * 4
    pos = np.arange(20, 70)
    p = sqa_oracle.softmax_probs(q, k, pos, causal, 0.25)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert (p >= 0).all()
    if causal:
        assert (p[np.arange(70)[None, :] > pos[:, None]] == 0).all()


@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_give_constant_output(causal):
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal((40, 8)) * 3, rng.standard_normal((40, 8)) * 3
    c = rng.standard_normal(8)
    v = np.tile(c, (40, 1))
    a = oracle.attention_rows(q, k, v, np.arange(40), causal)
    np.testing.assert_allclose(a, np.tile(c, (40, 1)), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_weights_give_mean_of_values(causal):
    """Wq = 0 makes every score 0, so the weights are uniform over the visible
    keys: the column mean of V (non-causal) or its prefix mean (causal)."""
    H, d = 4, 4
    X, Wq, Wk, Wv, Wo = _rand_problem(4, B=2, N=23, H=H, d_head=d, H_q=4, H_kv=2)
    out = oracle.sqa_forward(X, np.zeros_like(Wq), Wk, Wv, Wo, 4, 2, d, causal, False)
    V = X @ Wv                                                   # [B, N, 2*d]
    if causal:
        mean = np.cumsum(V, axis=1) / np.arange(1, 24)[None, :, None]
    else:
        mean = np.broadcast_to(V.mean(axis=1, keepdims=True), V.shape)
    want = np.concatenate([mean[..., :d], mean[..., :d], mean[..., d:], mean[..., d:]], axis=-1)
    np.testing.assert_allclose(out["A"], want, rtol=1e-12, atol=1e-13)


def test_causal_first_row_is_first_value():
    X, Wq, Wk, Wv, Wo = _rand_problem(6, B=3, N=9, H=4, d_head=4, H_q=2, H_kv=1)
    out = oracle.sqa_forward(X, Wq, Wk, Wv, Wo, 2, 1, 4, True, False)
    V0 = (X @ Wv)[:, 0, :]
    np.testing.assert_array_equal(out["A"][:, 0, :4], V0)
    np.testing.assert_array_equal(out["A"][:, 0, 4:], V0)


@pytest.mark.parametrize("causal", [False, True])
def test_shifting_all_keys_leaves_output_unchanged(causal):
    """Adding one vector u to every key adds q.u/sqrt(d) to a whole score row;
    softmax ignores a per-row constant."""
    rng = np.random.default_rng(8)
    q, k, v = (rng.standard_normal((30, 8)) for _ in range(3))
    u = rng.standard_normal(8) * 5
    pos = np.arange(30)
    np.testing.assert_allclose(oracle.attention_rows(q, k + u, v, pos, causal),
                               oracle.attention_rows(q, k, v, pos, causal), rtol=1e-11, atol=1e-12)


def test_noncausal_token_permutation_equivariance():
    X, Wq, Wk, Wv, Wo = _rand_problem(10, B=1, N=31, H=4, d_head=4, H_q=2, H_kv=1)
    perm = np.random.default_rng(0).permutation(31)
    y = oracle.sqa_forward(X, Wq, Wk, Wv, Wo, 2, 1, 4, False, False)["Y"]
    yp = oracle.sqa_forward(X[:, perm], Wq, Wk, Wv, Wo, 2, 1, 4, False, False)["Y"]
    np.testing.assert_allclose(yp, y[:, perm], rtol=1e-12, atol=1e-13)


def test_output_projection_is_linear_and_identity_passes_through():
    X, Wq, Wk, Wv, Wo = _rand_problem(12, B=2, N=11, H=4, d_head=4, H_q=4, H_kv=2)
    Wo2 = np.random.default_rng(3).standard_normal(Wo.shape)
    f = lambda W: oracle.sqa_forward(X, Wq, Wk, Wv, W, 4, 2, 4, True, False)
    np.testing.assert_allclose(f(Wo + Wo2)["Y"], f(Wo)["Y"] + f(Wo2)["Y"], rtol=1e-12, atol=1e-12)
    out = f(np.eye(16))
    np.testing.assert_allclose(out["Y"], out["A"], rtol=0, atol=0)


# ----------------------------------------------------------------------------------------------
# planted mistakes: the pins above must catch each of them

def _golden_fails(monkeypatch_apply):
    fails = 0
    for path in sorted(glob.glob(os.path.join(GOLDEN, "closed_form_*.json"))):
        g = json.load(open(path))
        X, Wq, Wk, Wv, Wo = (_arr(g[k]) for k in ("X", "Wq", "Wk", "Wv", "Wo"))
        for causal in (False, True):
            want = _arr(g["Y_causal" if causal else "Y_noncausal"])
            y = oracle.sqa_forward(X, Wq, Wk, Wv, Wo, g["H_q"], g["H_kv"], g["d_model"] // g["H"],
                                   causal, False)["Y"]
            fails += not np.allclose(y, want, rtol=1e-12, atol=1e-12)
    return fails


def test_planted_wrong_head_map_is_caught(monkeypatch):
    monkeypatch.setattr(sqa_oracle, "kv_head_for", lambda i, H_q, H_kv: i % H_kv)
    assert _golden_fails(None) > 0


def test_planted_wrong_scale_is_caught(monkeypatch):
    orig = sqa_oracle.softmax_probs
    monkeypatch.setattr(sqa_oracle, "softmax_probs",
                        lambda q, k, pos, causal, scale: orig(q, k, pos, causal, 1.0))
    assert _golden_fails(None) > 0


@pytest.mark.filterwarnings("ignore::RuntimeWarning")   # the fully masked row 0 gives NaN
def test_planted_strict_causal_mask_is_caught(monkeypatch):
    def strict(q, k, pos, causal, scale):
        s = (q @ k.T) * scale
        if causal:
            s = np.where(np.arange(k.shape[0])[None, :] < pos[:, None], s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        e = np.exp(s)
        return e / e.sum(axis=1, keepdims=True)
    monkeypatch.setattr(sqa_oracle, "softmax_probs", strict)
    assert _golden_fails(None) > 0


def test_planted_transposed_head_split_is_caught(monkeypatch):
    def bad_split(Y, n_heads, d_head):
        B, N, _ = Y.shape
        return Y.reshape(B, N, d_head, n_heads).transpose(0, 3, 1, 2)
    monkeypatch.setattr(sqa_oracle, "split_heads", bad_split)
    X, Wq, Wk, Wv, Wo = _rand_problem(13, B=1, N=5, H=4, d_head=2, H_q=4, H_kv=2)
    y_bf, _ = sqa_forward_bruteforce(X, Wq, Wk, Wv, Wo, 4, 2, 2, False, False)
    y = oracle.sqa_forward(X, Wq, Wk, Wv, Wo, 4, 2, 2, False, False)["Y"]
    assert not np.allclose(y, np.array(y_bf), rtol=1e-9, atol=1e-9)


# ----------------------------------------------------------------------------------------------
# variable-length batches (sequences padded to a common N)

def test_varlen_with_full_lengths_is_the_plain_forward():
    X, Wq, Wk, Wv, Wo = _rand_problem(61, B=3, N=40, H=4, d_head=8, H_q=2, H_kv=1)
    for causal in (False, True):
        y = oracle.sqa_forward_varlen(X, Wq, Wk, Wv, Wo, [40, 40, 40], 2, 1, 8, causal, True)
        ref = oracle.sqa_forward(X, Wq, Wk, Wv, Wo, 2, 1, 8, causal, True)["Y"]
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_matches_bruteforce_per_sequence(causal):
    """Each sequence against the independent scalar-loop forward run on that
    sequence's own tokens; padding rows are zero."""
    X, Wq, Wk, Wv, Wo = _rand_problem(62, B=4, N=7, H=4, d_head=2, H_q=2, H_kv=1)
    lens = [7, 3, 0, 1]
    y = oracle.sqa_forward_varlen(X, Wq, Wk, Wv, Wo, lens, 2, 1, 2, causal, False)
    for b, L in enumerate(lens):
        if L:
            yb, _ = sqa_forward_bruteforce(X[b:b + 1, :L], Wq, Wk, Wv, Wo, 2, 1, 2, causal, False)
            np.testing.assert_allclose(y[b, :L], np.array(yb)[0], rtol=1e-12, atol=1e-14)
        assert not y[b, L:].any()


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_ignores_padding_and_other_sequences(causal):
    X, Wq, Wk, Wv, Wo = _rand_problem(63, B=3, N=33, H=4, d_head=8, H_q=4, H_kv=2)
    lens = [20, 33, 5]
    y0 = oracle.sqa_forward_varlen(X, Wq, Wk, Wv, Wo, lens, 4, 2, 8, causal, True)
    X2 = X.copy()
    X2[0, 20:] = np.nan                 # padding of sequence 0
    X2[2, 5:] = 1e30                    # padding of sequence 2
    y1 = oracle.sqa_forward_varlen(X2, Wq, Wk, Wv, Wo, lens, 4, 2, 8, causal, True)
    np.testing.assert_array_equal(y0, y1)
    X3 = X.copy()
    X3[1] *= -3.0                       # a different sequence 1 leaves 0 and 2 alone
    y2 = oracle.sqa_forward_varlen(X3, Wq, Wk, Wv, Wo, lens, 4, 2, 8, causal, True)
    np.testing.assert_array_equal(y0[[0, 2]], y2[[0, 2]])
    assert not np.array_equal(y0[1], y2[1])


def test_varlen_causal_prefix_equals_full_run():
    """Causal row t sees keys <= t only, so cutting a sequence at L leaves its
    first L rows as in the uncut run."""
    X, Wq, Wk, Wv, Wo = _rand_problem(64, B=2, N=50, H=4, d_head=8, H_q=2, H_kv=2)
    full = oracle.sqa_forward(X, Wq, Wk, Wv, Wo, 2, 2, 8, True, True)["Y"]
    y = oracle.sqa_forward_varlen(X, Wq, Wk, Wv, Wo, [50, 17], 2, 2, 8, True, True)
    np.testing.assert_allclose(y[0], full[0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(y[1, :17], full[1, :17], rtol=1e-12, atol=1e-14)
    # without the causal mask the cut changes the kept rows (keys past 17 matter)
    nc = oracle.sqa_forward(X, Wq, Wk, Wv, Wo, 2, 2, 8, False, True)["Y"]
    ync = oracle.sqa_forward_varlen(X, Wq, Wk, Wv, Wo, [50, 17], 2, 2, 8, False, True)
    assert not np.allclose(ync[1, :17], nc[1, :17])


def test_varlen_rows_match_full_varlen():
    X, Wq, Wk, Wv, Wo = _rand_problem(65, B=3, N=30, H=4, d_head=8, H_q=2, H_kv=1)
    lens = [30, 0, 11]
    for causal in (False, True):
        y = oracle.sqa_forward_varlen(X, Wq, Wk, Wv, Wo, lens, 2, 1, 8, causal, True)
        rows = [0, 29, 30, 45, 60, 70, 71, 89]
        yr = oracle.sqa_forward_varlen_rows(X, Wq, Wk, Wv, Wo, lens, 2, 1, 8, causal, True, rows)
        np.testing.assert_allclose(yr, y.reshape(-1, 32)[rows], rtol=1e-12, atol=1e-14)


def test_varlen_rejects_bad_lengths():
    X, Wq, Wk, Wv, Wo = _rand_problem(66, B=2, N=8, H=4, d_head=2, H_q=2, H_kv=1)
    for lens in ([9, 1], [-1, 1], [1]):
        with pytest.raises(ValueError):
            oracle.sqa_forward_varlen(X, Wq, Wk, Wv, Wo, lens, 2, 1, 2, False, False)


def _bad_varlen_full_keys(X, Wq, Wk, Wv, Wo, lens, H_q, H_kv, d_head, causal, bf16, workers=None):
    """Planted: queries stop at lens[b] but every padded key is still attended."""
    Y = oracle.sqa_forward(X, Wq, Wk, Wv, Wo, H_q, H_kv, d_head, causal, bf16)["Y"]
    for b, L in enumerate(lens):
        Y[b, L:] = 0.0
    return Y


def _bad_varlen_unzeroed_padding(X, Wq, Wk, Wv, Wo, lens, H_q, H_kv, d_head, causal, bf16, workers=None):
    """Planted: right valid rows, but padding rows keep computed values."""
    X = np.asarray(X, dtype=np.float64)
    Y = oracle.sqa_forward(X, Wq, Wk, Wv, Wo, H_q, H_kv, d_head, causal, bf16)["Y"]
    for b, L in enumerate(lens):
        if L:
            Y[b, :L] = oracle.sqa_forward(X[b:b + 1, :L], Wq, Wk, Wv, Wo, H_q, H_kv, d_head, causal,
                                          bf16)["Y"][0]
    return Y


@pytest.mark.parametrize("bad", [_bad_varlen_full_keys, _bad_varlen_unzeroed_padding])
def test_planted_varlen_mistakes_are_caught(monkeypatch, bad):
    monkeypatch.setattr(oracle, "sqa_forward_varlen", bad)
    with pytest.raises(AssertionError):
        test_varlen_matches_bruteforce_per_sequence(False)
