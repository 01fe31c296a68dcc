"""The attention step alone (sqa_attention through the C ABI) on crafted
Q/K/V, against the oracle's attention core.

The inputs target the online softmax: scores that grow along the keys (the
running max rises in every key block), scores that fall (the first block
holds the max), logits large enough to overflow any stale reference, all-equal
scores, and one dominant key. Q, K and V are given as bf16 values, so the
oracle sees exactly what the kernel sees; only A is rounded to bf16 at the end.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_query_attention_amd as sqa
import workloads as wl
from parity import compare, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sqa._lib.load()
    return torch.device("cuda:0")


def run_case(dev, q, k, v, causal, dtype="bf16"):
    """q [B,H_q,N,d], k/v [B,H_kv,N,d] float64 arrays of dtype-representable values."""
    B, H_q, N, d = q.shape
    H_kv = k.shape[1]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    Np = sqa.padded_length(N)
    qp = torch.zeros((B, H_q, Np, d), dtype=tdt)
    kp = torch.zeros((B, H_kv, Np, d), dtype=tdt)
    vtp = torch.zeros((B, H_kv, d, Np), dtype=tdt)
    qp[:, :, :N] = torch.from_numpy(q).to(tdt)
    kp[:, :, :N] = torch.from_numpy(k).to(tdt)
    vtp[..., :N] = torch.from_numpy(v).to(tdt).transpose(-1, -2)
    a = sqa.attention(qp.to(dev), kp.to(dev), vtp.to(dev), N=N, causal=causal)
    torch.cuda.synchronize()
    got = wl.widen(a.cpu()).reshape(B, N, H_q * d)
    g = H_q // H_kv
    ref = np.empty((B, N, H_q * d))
    for b in range(B):
        for i in range(H_q):
            ref[b, :, i * d:(i + 1) * d] = oracle.attention_rows(q[b, i], k[b, i // g], v[b, i // g],
                                                                 np.arange(N), causal)
    if dtype == "bf16":
        ref = oracle.round_bf16(ref)
    return got, ref


def bf16(a):
    return oracle.round_bf16(np.asarray(a, dtype=np.float64))


@pytest.mark.parametrize("causal", [False, True])
def test_scores_growing_along_keys_rescale_every_block(dev, causal):
    """k_j = (1 + j/16) * u: every query's scores grow with j, so each 32-key
    block raises the running max and forces the exact rescale."""
    rng = np.random.default_rng(1)
    B, H_q, H_kv, N, d = 1, 4, 2, 700, 64
    u = rng.standard_normal((H_kv, 1, d))
    k = bf16(u * (1 + np.arange(N)[None, :, None] / 16.0) + 0.05 * rng.standard_normal((H_kv, N, d)))[None]
    q = bf16(np.repeat(u, 2, axis=0) * np.ones((1, N, 1)) * 0.3 + 0.1 * rng.standard_normal((H_q, N, d)))[None]
    v = bf16(rng.standard_normal((1, H_kv, N, d)))
    got, ref = run_case(dev, q, k, v, causal)
    rep = compare(got, ref, "bf16")
    log(f"  growing scores causal={causal}: {rep}")
    assert rep.ok


@pytest.mark.parametrize("causal", [False, True])
def test_scores_falling_along_keys(dev, causal):
    rng = np.random.default_rng(2)
    B, H_q, H_kv, N, d = 1, 2, 2, 513, 64
    u = rng.standard_normal((H_kv, 1, d))
    k = bf16(u * (8 - np.arange(N)[None, :, None] / 64.0))[None]
    q = bf16(u * np.ones((1, N, 1)) * 0.5)[None]
    v = bf16(rng.standard_normal((1, H_kv, N, d)))
    got, ref = run_case(dev, q, k, v, causal)
    rep = compare(got, ref, "bf16")
    log(f"  falling scores causal={causal}: {rep}")
    assert rep.ok


@pytest.mark.parametrize("scale", [30.0, 300.0])
def test_huge_logits_overflow_a_stale_reference(dev, scale):
    """Logits in the thousands: exp2 against a stale reference overflows to
    inf, which must route the block through the exact rescale."""
    rng = np.random.default_rng(3)
    B, H_q, H_kv, N, d = 2, 4, 1, 300, 64
    q = bf16(rng.standard_normal((B, H_q, N, d)) * scale / 8)
    k = bf16(rng.standard_normal((B, H_kv, N, d)) * np.linspace(0.2, 3.0, N)[None, None, :, None])
    v = bf16(rng.standard_normal((B, H_kv, N, d)))
    for causal in (False, True):
        got, ref = run_case(dev, q, k, v, causal)
        rep = compare(got, ref, "bf16")
        log(f"  huge logits scale={scale} causal={causal}: {rep}")
        assert rep.ok


def test_equal_scores_give_the_mean_of_values(dev):
    rng = np.random.default_rng(4)
    B, H_q, H_kv, N, d = 1, 2, 1, 1000, 32
    q = np.zeros((B, H_q, N, d))
    k = bf16(rng.standard_normal((B, H_kv, N, d)))
    v = bf16(rng.standard_normal((B, H_kv, N, d)))
    for causal in (False, True):
        got, ref = run_case(dev, q, k, v, causal)
        rep = compare(got, ref, "bf16")
        log(f"  equal scores causal={causal}: {rep}")
        assert rep.ok


def test_one_dominant_key(dev):
    """Every query matches key 417 by a margin of ~100 nats: the output is
    that key's value row (to bf16 rounding)."""
    rng = np.random.default_rng(5)
    B, H_q, H_kv, N, d = 1, 4, 4, 1000, 64
    k = bf16(rng.standard_normal((B, H_kv, N, d)) * 0.1)
    k[:, :, 417] = bf16(np.ones(d) * 2.0)
    q = bf16(np.ones((B, H_q, N, d)) * 6.0)
    v = bf16(rng.standard_normal((B, H_kv, N, d)))
    got, ref = run_case(dev, q, k, v, False)
    rep = compare(got, ref, "bf16")
    log(f"  dominant key: {rep}")
    assert rep.ok
    np.testing.assert_allclose(got[0, :, 0:64], np.tile(v[0, 0, 417], (N, 1)), atol=1e-2)


@pytest.mark.parametrize("N", [1, 31, 32, 33, 64, 65, 200])
def test_fp32_attention_stage_ragged_lengths(dev, N):
    rng = np.random.default_rng(6 + N)
    B, H_q, H_kv, d = 2, 4, 2, 32
    q = rng.standard_normal((B, H_q, N, d)).astype(np.float32).astype(np.float64)
    k = rng.standard_normal((B, H_kv, N, d)).astype(np.float32).astype(np.float64)
    v = rng.standard_normal((B, H_kv, N, d)).astype(np.float32).astype(np.float64)
    for causal in (False, True):
        got, ref = run_case(dev, q, k, v, causal, dtype="fp32")
        rep = compare(got, ref, "fp32")
        assert rep.ok, f"N={N} causal={causal}: {rep}"
