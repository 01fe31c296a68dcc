"""Backward pass (sqa_backward) on the GPU against the float64 oracle.

Every output (dx, dWq, dWk, dWv, dWo) is compared element by element with
oracle.sqa_backward on the same seeded inputs (workloads.py: X, weights and the
upstream gradient dY), with the tolerances of the workload's dtype
(tests/parity.py). Weight gradients are compared row by row of the weight
matrix. Shapes span several key and query tiles with ragged tails, every
group size the kernels treat differently, both head widths and both dtypes.
The headline head shape (H=16, H_q=8, H_kv=4, d_head=64, causal) is compared
whole at 32768 tokens. At the full 131072-token size the whole oracle cannot
run in a test, so two checks share it:
  * dX at sampled rows of the last 1024 positions: each such row takes dQ
    from one query row against every key, and dK and dV from every later
    query row, so the oracle computes them one by one
    (oracle.sqa_backward_rows);
  * an upstream gradient that is zero outside two windows of query rows (the
    middle and the end of the sequence): every key then still collects dK
    and dV over the whole causal range of query tiles, the weight gradients
    still sum over every token, and the oracle only runs the rows that carry
    a gradient (oracle.sqa_backward_dy_rows). All five gradients are compared
    at every position.
Determinism and exact scaling in dY are checked on every output.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_query_attention_amd as sqa
import workloads as wl
from parity import MIN_TOKENS_FOR_ROW_GATE, compare, log

pytestmark = pytest.mark.gpu

GRADS = ("dX", "dWq", "dWk", "dWv", "dWo")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sqa._lib.load()   # the HIP library, never a stand-in
    return torch.device("cuda:0")


def _inputs(w, dev):
    arrays = wl.draw(w)
    arrays["dY"] = wl.draw_upstream_grad(w)
    host = wl.to_device_dtype(arrays, w.dtype)
    return host, {k: v.to(dev) for k, v in host.items()}


def _run(w, d):
    return sqa.backward(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], d["dY"], H=w.H, H_q=w.H_q,
                        H_kv=w.H_kv, causal=w.causal)


def _oracle(w, host):
    o = {k: wl.widen(v) for k, v in host.items()}
    return oracle.sqa_backward(o["X"], o["Wq"], o["Wk"], o["Wv"], o["Wo"], o["dY"], w.H_q, w.H_kv,
                               w.d_head, w.causal, bf16=(w.dtype == "bf16"))


CASES = [
    # name, B, N, H, d_head, H_q, H_kv, causal, dtype
    ("g2_causal", 2, 300, 8, 64, 4, 2, True, "bf16"),
    ("g2_full", 2, 300, 8, 64, 4, 2, False, "bf16"),
    ("g1", 1, 200, 8, 64, 4, 4, True, "bf16"),
    ("g4_d1024", 1, 257, 16, 64, 8, 2, True, "bf16"),
    ("g4_d32", 2, 333, 8, 32, 4, 1, True, "bf16"),
    ("g16", 1, 129, 16, 64, 16, 1, False, "bf16"),
    ("g64", 1, 150, 64, 32, 64, 1, True, "bf16"),
    ("mha_d32_full", 1, 100, 8, 32, 8, 8, False, "bf16"),
    ("fp32_full", 2, 150, 8, 32, 4, 2, False, "fp32"),
    ("fp32_causal_d64", 1, 90, 4, 64, 4, 2, True, "fp32"),
    ("one_token", 2, 1, 8, 64, 4, 2, True, "bf16"),
    ("sqa_n2048", 1, 2048, 16, 64, 8, 4, True, "bf16"),
    ("sqa_n4097", 1, 4097, 16, 64, 8, 4, True, "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(dev, case):
    name, B, N, H, dh, H_q, H_kv, causal, dtype = case
    w = wl.Workload(name, B=B, N=N, d_model=H * dh, H=H, H_q=H_q, H_kv=H_kv, causal=causal,
                    dtype=dtype, seed=300 + N + H_q)
    log(f"case backward {name}: B={B} N={N} H={H} d={dh} H_q={H_q} H_kv={H_kv} "
        f"causal={causal} {dtype}")
    host, d = _inputs(w, dev)
    got = _run(w, d)
    torch.cuda.synchronize()
    ref = _oracle(w, host)
    bad = []
    for k, g in zip(GRADS, got):
        rep = compare(wl.widen(g.cpu()), ref[k], dtype,
                      k == "dX" or w.tokens >= MIN_TOKENS_FOR_ROW_GATE)
        log(f"  {k}: {rep}")
        if not rep.ok:
            bad.append(k)
    assert not bad, bad


def test_backward_is_deterministic_and_linear_in_dy(dev):
    """Same inputs give bitwise the same gradients (no atomics), and 2*dY gives
    exactly twice every gradient (scaling by 2 commutes with each rounding)."""
    w = wl.Workload("det", B=2, N=700, d_model=1024, H=16, H_q=8, H_kv=4, causal=True,
                    dtype="bf16", seed=401)
    _, d = _inputs(w, dev)
    a = _run(w, d)
    b = _run(w, d)
    d2 = dict(d, dY=d["dY"] * 2)
    c = _run(w, d2)
    torch.cuda.synchronize()
    for k, x, y, z in zip(GRADS, a, b, c):
        assert torch.equal(x, y), k
        assert torch.equal(z, x * 2), k


def test_backward_at_full_size_matches_sampled_rows_is_deterministic_and_scales(dev):
    """The 131072-token causal SQA shape of the forward benchmark, in the launch
    configuration the benchmark times."""
    w = wl.SQA_131K_CAUSAL
    log(f"case backward full size {w.name}")
    host, d = _inputs(w, dev)
    a = _run(w, d)
    b = _run(w, d)
    d["dY"] = d["dY"] * 2
    c = _run(w, d)
    torch.cuda.synchronize()
    for k, x, y, z in zip(GRADS, a, b, c):
        assert bool(torch.isfinite(x).all()), k
        assert float(x.abs().max()) > 0, k
        assert torch.equal(x, y), k
        assert torch.equal(z, x * 2), k
    N = w.N
    rows = [N - 1, N - 2, N - 31, N - 64, N - 200, N - 511, N - 700, N - 1024]
    o = {k: wl.widen(v) for k, v in host.items()}
    ref = oracle.sqa_backward_rows(o["X"], o["Wq"], o["Wk"], o["Wv"], o["Wo"], o["dY"], w.H_q,
                                   w.H_kv, w.d_head, True, True, rows)
    got = wl.widen(a[0].reshape(w.B * N, -1)[rows].cpu())
    rep = compare(got, ref["dX_rows"], w.dtype)
    log(f"  dX at rows {rows}: {rep}")
    assert rep.ok, rep


def test_backward_headline_heads_at_32768_tokens_all_gradients(dev):
    """The benchmark's head shape (H=16, H_q=8, H_kv=4, d_head=64, causal) at
    32768 tokens: every element of all five gradients against the oracle.
    Early keys collect dK and dV over 32k query rows here, and the split-K
    weight gradients sum over 32768 tokens."""
    w = wl.SQA_131K_CAUSAL.with_(name="sqa_bf16_causal_n32768", N=32768)
    log(f"case backward all gradients {w.name}")
    host, d = _inputs(w, dev)
    got = [g.cpu() for g in _run(w, d)]
    torch.cuda.synchronize()
    del d
    ref = _oracle(w, host)
    bad = []
    for k, g in zip(GRADS, got):
        rep = compare(wl.widen(g), ref[k], w.dtype)
        log(f"  {k}: {rep}")
        if not rep.ok:
            bad.append(k)
    assert not bad, bad


def _dy_windows(N):
    """Query rows that carry an upstream gradient: 1024 rows around the middle
    of the sequence and its last 512 rows."""
    return np.r_[np.arange(N // 2 - 512, N // 2 + 512), np.arange(N - 512, N)]


def test_backward_at_full_size_with_dy_on_two_windows_all_gradients(dev):
    """131072 tokens, causal, in the benchmark's launch, with dY zero outside
    two windows of rows: all five gradients at every position against the
    oracle. Every key's dK and dV sum over the whole causal range of query
    tiles (most of them carry zeros), and dWk and dWv sum over all 131072
    tokens."""
    w = wl.SQA_131K_CAUSAL
    rows = _dy_windows(w.N)
    log(f"case backward full size, dY on {rows.size} rows, {w.name}")
    arrays = wl.draw(w)
    dy = np.zeros_like(wl.draw_upstream_grad(w))
    dy[0, rows] = wl.draw_upstream_grad(w)[0, rows]
    arrays["dY"] = dy
    host = wl.to_device_dtype(arrays, w.dtype)
    d = {k: v.to(dev) for k, v in host.items()}
    got = [g.cpu() for g in _run(w, d)]
    torch.cuda.synchronize()
    del d
    o = {k: wl.widen(v) for k, v in host.items()}
    ref = oracle.sqa_backward_dy_rows(o["X"], o["Wq"], o["Wk"], o["Wv"], o["Wo"], o["dY"], w.H_q,
                                      w.H_kv, w.d_head, True, True, rows)
    bad = []
    for k, g in zip(GRADS, got):
        rep = compare(wl.widen(g), ref[k], w.dtype)
        log(f"  {k}: {rep}")
        if not rep.ok:
            bad.append(k)
    # rows before the first window still get gradients (through dK and dV)
    assert (np.abs(ref["dX"][0, :1024]).max(axis=1) > 0).all()
    assert not bad, bad


def test_backward_non_causal_key_split_tail_all_gradients(dev):
    """20000 tokens, non-causal, 8 KV heads: the forward's partial last round of
    work items runs split over the keys and merged (output and log-sum-exp),
    both in forward_train and in the backward that recomputes them. The two
    give bitwise the same gradients, and with dY on two windows of rows all
    five gradients match the oracle at every position."""
    w = wl.Workload("key_split_bwd", B=1, N=20000, d_model=1024, H=16, H_q=8, H_kv=8,
                    causal=False, dtype="bf16", seed=3302)
    rows = np.r_[np.arange(9000, 9512), np.arange(w.N - 300, w.N)]
    log(f"case backward key split {w.name}, dY on {rows.size} rows")
    arrays = wl.draw(w)
    dy = np.zeros_like(wl.draw_upstream_grad(w))
    dy[0, rows] = wl.draw_upstream_grad(w)[0, rows]
    arrays["dY"] = dy
    host = wl.to_device_dtype(arrays, w.dtype)
    d = {k: v.to(dev) for k, v in host.items()}
    kw = dict(H=w.H, H_q=w.H_q, H_kv=w.H_kv, causal=False)
    y = sqa.forward(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], **kw)
    y2, saved = sqa.forward_train(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], **kw)
    g_saved = sqa.backward(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], d["dY"], saved=saved, **kw)
    g_re = _run(w, d)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    for k, x, z in zip(GRADS, g_saved, g_re):
        assert torch.equal(x, z), k
    got = [g.cpu() for g in g_re]
    del d, saved, g_saved
    o = {k: wl.widen(v) for k, v in host.items()}
    ref = oracle.sqa_backward_dy_rows(o["X"], o["Wq"], o["Wk"], o["Wv"], o["Wo"], o["dY"], w.H_q,
                                      w.H_kv, w.d_head, False, True, rows)
    bad = []
    for k, g in zip(GRADS, got):
        rep = compare(wl.widen(g), ref[k], w.dtype)
        log(f"  {k}: {rep}")
        if not rep.ok:
            bad.append(k)
    assert not bad, bad


@pytest.mark.parametrize("causal,dtype,dh", [(True, "bf16", 64), (False, "bf16", 32), (True, "fp32", 32)])
def test_saved_activations_give_the_same_results(dev, causal, dtype, dh):
    """forward_train is bitwise forward, and backward from its saved activations
    is bitwise backward with recomputed ones (the same kernels produce them)."""
    w = wl.Workload("train", B=2, N=333, d_model=8 * dh, H=8, H_q=4, H_kv=2, causal=causal,
                    dtype=dtype, seed=410)
    _, d = _inputs(w, dev)
    y = sqa.forward(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], H=w.H, H_q=w.H_q, H_kv=w.H_kv,
                    causal=causal)
    y2, saved = sqa.forward_train(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], H=w.H, H_q=w.H_q,
                                  H_kv=w.H_kv, causal=causal)
    g = _run(w, d)
    g2 = sqa.backward(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], d["dY"], H=w.H, H_q=w.H_q,
                      H_kv=w.H_kv, causal=causal, saved=saved)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    for k, a, b in zip(GRADS, g, g2):
        assert torch.equal(a, b), k


def test_backward_past_65535_row_tiles(dev):
    """N = 65536*64 + 64 tokens (one head, d_head 32, causal): the transposes
    of the backward take more than 65535 tiles of 64 rows, which a 2-D grid
    with rows along y could not launch. dX near the end against the oracle."""
    N = 65536 * 64 + 64
    w = wl.Workload("past_y_limit", B=1, N=N, d_model=32, H=1, H_q=1, H_kv=1, causal=True,
                    dtype="bf16", seed=4322)
    log(f"case backward N={N}")
    host, d = _inputs(w, dev)
    got = _run(w, d)
    torch.cuda.synchronize()
    for k, x in zip(GRADS, got):
        assert bool(torch.isfinite(x).all()), k
    rows = [N - 1, N - 2, N - 33, N - 64]
    gx = wl.widen(got[0].reshape(N, -1)[rows].cpu())
    del d, got
    o = {k: wl.widen(v) for k, v in host.items()}
    ref = oracle.sqa_backward_rows(o["X"], o["Wq"], o["Wk"], o["Wv"], o["Wo"], o["dY"], 1, 1, 32,
                                   True, True, rows, row_block=8)
    rep = compare(gx, ref["dX_rows"], w.dtype)
    log(f"  dX at rows {rows}: {rep}; max |dX| {float(np.abs(ref['dX_rows']).max()):.3e}")
    assert float(np.abs(ref["dX_rows"]).max()) > 0
    assert rep.ok, rep



def test_backward_of_more_than_65535_sequence_heads(dev):
    """B * H_q = 65600 (sequence, query head) pairs of 3 tokens each: the
    per-head transposes take them along the grid's x dimension. Every gradient
    against the oracle."""
    w = wl.Workload("wide_batch", B=8200, N=3, d_model=256, H=8, H_q=8, H_kv=2, causal=True,
                    dtype="bf16", seed=4323)
    log(f"case backward B={w.B} N={w.N}")
    host, d = _inputs(w, dev)
    got = _run(w, d)
    torch.cuda.synchronize()
    ref = _oracle(w, host)
    for k, g in zip(GRADS, got):
        rep = compare(wl.widen(g.cpu()), ref[k], w.dtype)
        log(f"  {k}: {rep}")
        assert rep.ok, (k, rep)
