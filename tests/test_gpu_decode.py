"""Prefill and key/value-cache decode (sqa_prefill, sqa_decode_step) on the GPU.

A decode step for token t of a sequence must give row t of the causal SQA
forward over the sequence's first t+1 tokens; the oracle computes exactly that
row (oracle.sqa_forward_rows, causal). The caches must hold the step-1 keys and
values of the cached tokens.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_query_attention_amd as sqa
import workloads as wl
from parity import compare, device_inputs, log, oracle_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sqa._lib.load()   # the HIP library, never a stand-in
    return torch.device("cuda:0")


def _caches(w, N_max, dev, fill=float("nan")):
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    shp = (w.B, w.H_kv, N_max, w.d_head)
    return (torch.full(shp, fill, dtype=tdt, device=dev), torch.full(shp, fill, dtype=tdt, device=dev))


def _oracle_rows(host, w, rows):
    o = oracle_inputs(host)
    return oracle.sqa_forward_rows(o["X"], o["Wq"], o["Wk"], o["Wv"], o["Wo"], w.H_q, w.H_kv,
                                   w.d_head, True, bf16=(w.dtype == "bf16"), rows=rows)["Y_rows"]


def test_prefill_is_the_causal_forward_and_fills_the_caches(dev):
    w = wl.Workload("prefill", B=2, N=300, d_model=1024, H=16, H_q=8, H_kv=4, causal=True,
                    dtype="bf16", seed=81)
    _, d = device_inputs(w, dev)
    kc, vc = _caches(w, 512, dev)
    y = sqa.prefill(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], kc, vc, H=w.H, H_q=w.H_q, H_kv=w.H_kv)
    y_ref = sqa.forward(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], H=w.H, H_q=w.H_q, H_kv=w.H_kv,
                        causal=True)
    q, k, vt = sqa.qkv_projection(d["X"], d["Wq"], d["Wk"], d["Wv"], H=w.H, H_q=w.H_q, H_kv=w.H_kv)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    assert torch.equal(kc[:, :, :w.N], k[:, :, :w.N])
    assert torch.equal(vc[:, :, :w.N], vt[..., :w.N].transpose(-1, -2))
    assert bool(torch.isnan(kc[:, :, w.N:]).all()) and bool(torch.isnan(vc[:, :, w.N:]).all())



def test_prefill_of_more_than_65535_sequence_heads(dev):
    """B * H_kv = 65600 (sequence, key/value head) pairs: the cache fill strides
    them over a grid of at most 65535 rows."""
    w = wl.Workload("prefill_wide", B=16400, N=3, d_model=128, H=4, H_q=4, H_kv=4, causal=True,
                    dtype="bf16", seed=83)
    _, d = device_inputs(w, dev)
    kc, vc = _caches(w, 4, dev)
    y = sqa.prefill(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], kc, vc, H=w.H, H_q=w.H_q, H_kv=w.H_kv)
    y_ref = sqa.forward(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], H=w.H, H_q=w.H_q, H_kv=w.H_kv,
                        causal=True)
    q, k, vt = sqa.qkv_projection(d["X"], d["Wq"], d["Wk"], d["Wv"], H=w.H, H_q=w.H_q, H_kv=w.H_kv)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    assert torch.equal(kc[:, :, :w.N], k[:, :, :w.N])
    assert torch.equal(vc[:, :, :w.N], vt[..., :w.N].transpose(-1, -2))
    assert bool(torch.isnan(kc[:, :, w.N:]).all()) and bool(torch.isnan(vc[:, :, w.N:]).all())

DECODE_SHAPES = [
    # (H, d_head, H_q, H_kv, dtype): g = 2, 1, 4, 16 (two head groups), fp32, d = 32, and
    # d_model = 160 (projection widths that are not multiples of the 256-column blocks), and
    # g = 64 (eight head groups of one key/value head)
    (16, 64, 8, 4, "bf16"), (16, 64, 4, 4, "bf16"), (16, 64, 4, 1, "bf16"),
    (16, 64, 16, 1, "bf16"), (8, 32, 4, 2, "fp32"), (8, 32, 6, 2, "bf16"), (5, 32, 5, 1, "bf16"),
    (64, 32, 64, 1, "bf16"),
]


@pytest.mark.parametrize("H,dh,H_q,H_kv,dtype", DECODE_SHAPES, ids=lambda v: str(v))
def test_generation_loop_matches_causal_forward(dev, H, dh, H_q, H_kv, dtype):
    """Prefill 150 tokens, then decode tokens 150..157 one step at a time."""
    T, t0, N_max = 158, 150, 256
    w = wl.Workload("gen", B=3, N=T, d_model=H * dh, H=H, H_q=H_q, H_kv=H_kv, causal=True,
                    dtype=dtype, seed=82 + H_q * 7 + H_kv)
    log(f"case decode loop H={H} d={dh} H_q={H_q} H_kv={H_kv} {dtype}")
    host, d = device_inputs(w, dev)
    kc, vc = _caches(w, N_max, dev)
    sqa.prefill(d["X"][:, :t0].contiguous(), d["Wq"], d["Wk"], d["Wv"], d["Wo"], kc, vc, H=w.H,
                H_q=w.H_q, H_kv=w.H_kv)
    ys = []
    for t in range(t0, T):
        pos = torch.full((w.B,), t, dtype=torch.int32, device=dev)
        ys.append(sqa.decode_step(d["X"][:, t].contiguous(), d["Wq"], d["Wk"], d["Wv"], d["Wo"], kc, vc,
                                  pos, H=w.H, H_q=w.H_q, H_kv=w.H_kv))
    torch.cuda.synchronize()
    got = np.stack([wl.widen(y.cpu()) for y in ys], axis=1)          # [B, steps, d_model]
    rows = np.array([b * T + t for b in range(w.B) for t in range(t0, T)])
    ref = _oracle_rows(host, w, rows).reshape(w.B, T - t0, w.d_model)
    rep = compare(got, ref, dtype)
    log(f"  {rep}")
    assert rep.ok, rep


def test_decode_at_mixed_positions_and_clamped_positions(dev):
    """Each sequence at its own position; out-of-range positions are clamped."""
    w = wl.Workload("mixed", B=5, N=400, d_model=1024, H=16, H_q=8, H_kv=2, causal=True,
                    dtype="bf16", seed=90)
    host, d = device_inputs(w, dev)
    kc, vc = _caches(w, w.N, dev)
    sqa.prefill(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], kc, vc, H=w.H, H_q=w.H_q, H_kv=w.H_kv)
    pos_in = np.array([0, 1, 399, 137, -4], dtype=np.int32)     # -4 behaves as 0
    p = np.clip(pos_in, 0, w.N - 1)
    x_new = torch.stack([d["X"][b, int(p[b])] for b in range(w.B)])
    y = sqa.decode_step(x_new, d["Wq"], d["Wk"], d["Wv"], d["Wo"], kc, vc,
                        torch.from_numpy(pos_in).to(dev), H=w.H, H_q=w.H_q, H_kv=w.H_kv)
    torch.cuda.synchronize()
    ref = _oracle_rows(host, w, [b * w.N + int(p[b]) for b in range(w.B)])
    rep = compare(wl.widen(y.cpu()), ref, "bf16")
    log(f"  mixed positions: {rep}")
    assert rep.ok, rep


def test_decode_over_a_long_cache(dev):
    """32k-token caches: many key chunks per sequence, merged across workgroups."""
    w = wl.Workload("long_decode", B=4, N=32768, d_model=1024, H=16, H_q=8, H_kv=4, causal=True,
                    dtype="bf16", seed=91)
    host, d = device_inputs(w, dev)
    kc, vc = _caches(w, w.N, dev)
    sqa.prefill(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], kc, vc, H=w.H, H_q=w.H_q, H_kv=w.H_kv)
    p = np.array([32767, 20000, 64, 4097], dtype=np.int32)
    x_new = torch.stack([d["X"][b, int(p[b])] for b in range(w.B)])
    y = sqa.decode_step(x_new, d["Wq"], d["Wk"], d["Wv"], d["Wo"], kc, vc,
                        torch.from_numpy(p).to(dev), H=w.H, H_q=w.H_q, H_kv=w.H_kv)
    torch.cuda.synchronize()
    ref = _oracle_rows(host, w, [b * w.N + int(p[b]) for b in range(w.B)])
    rep = compare(wl.widen(y.cpu()), ref, "bf16")
    log(f"  long cache: {rep}")
    assert rep.ok, rep


def test_decode_batch_of_many_sequences(dev):
    """B = 19 sequences: the projections take the tokens in several chunks."""
    w = wl.Workload("many", B=19, N=130, d_model=512, H=8, H_q=4, H_kv=2, causal=True,
                    dtype="bf16", seed=92)
    host, d = device_inputs(w, dev)
    kc, vc = _caches(w, w.N, dev)
    sqa.prefill(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], kc, vc, H=w.H, H_q=w.H_q, H_kv=w.H_kv)
    p = (np.arange(w.B, dtype=np.int32) * 7) % w.N
    x_new = torch.stack([d["X"][b, int(p[b])] for b in range(w.B)])
    y = sqa.decode_step(x_new, d["Wq"], d["Wk"], d["Wv"], d["Wo"], kc, vc,
                        torch.from_numpy(p).to(dev), H=w.H, H_q=w.H_q, H_kv=w.H_kv)
    torch.cuda.synchronize()
    ref = _oracle_rows(host, w, [b * w.N + int(p[b]) for b in range(w.B)])
    rep = compare(wl.widen(y.cpu()), ref, "bf16")
    log(f"  19 sequences: {rep}")
    assert rep.ok, rep


@pytest.mark.parametrize("H_q", [8, 16], ids=["sqa", "gqa_baseline"])
def test_decode_in_the_benchmark_launch(dev, H_q):
    """The decode step the benchmark times: 8 sequences whose caches hold
    32767 tokens from sqa_prefill, each stepping its token 32767 (same shapes
    and seed), for SQA (H_q = 8) and its GQA baseline (H_q = 16)."""
    w = wl.Workload("sqa_bf16_decode_b8_cache32768", B=8, N=32768, d_model=1024, H=16, H_q=H_q,
                    H_kv=4, causal=True, dtype="bf16", seed=1006)
    log(f"case decode benchmark launch H_q={H_q}")
    host, d = device_inputs(w, dev)
    kc, vc = _caches(w, w.N, dev)
    sqa.prefill(d["X"][:, :w.N - 1].contiguous(), d["Wq"], d["Wk"], d["Wv"], d["Wo"], kc, vc,
                H=w.H, H_q=w.H_q, H_kv=w.H_kv)
    pos = torch.full((w.B,), w.N - 1, dtype=torch.int32, device=dev)
    y = sqa.decode_step(d["X"][:, w.N - 1].contiguous(), d["Wq"], d["Wk"], d["Wv"], d["Wo"], kc,
                        vc, pos, H=w.H, H_q=w.H_q, H_kv=w.H_kv)
    torch.cuda.synchronize()
    ref = _oracle_rows(host, w, [b * w.N + w.N - 1 for b in range(w.B)])
    rep = compare(wl.widen(y.cpu()), ref, "bf16")
    log(f"  benchmark decode launch H_q={H_q}: {rep}")
    assert rep.ok, rep


def test_decode_workspace_kept_per_stream(dev):
    """The decode step keeps its workspace per stream between calls. A step on
    a second stream, and a larger step after a smaller one on the same stream
    (the workspace grows), each equal bitwise the same step on the default
    stream."""
    def setup(B, N, seed):
        w = wl.Workload("dec_ws", B=B, N=N, d_model=512, H=8, H_q=4, H_kv=2, causal=True,
                        dtype="bf16", seed=seed)
        _, d = device_inputs(w, dev)
        kc, vc = _caches(w, N, dev, fill=0.0)
        sqa.prefill(d["X"][:, :N - 1].contiguous(), d["Wq"], d["Wk"], d["Wv"], d["Wo"], kc, vc,
                    H=w.H, H_q=w.H_q, H_kv=w.H_kv)
        pos = torch.full((B,), N - 1, dtype=torch.int32, device=dev)
        return w, d, kc, vc, pos

    def step(w, d, kc, vc, pos):
        return sqa.decode_step(d["X"][:, w.N - 1].contiguous(), d["Wq"], d["Wk"], d["Wv"], d["Wo"],
                               kc, vc, pos, H=w.H, H_q=w.H_q, H_kv=w.H_kv)

    small = setup(2, 700, 91)
    large = setup(6, 5000, 92)
    ref_small, ref_large = step(*small), step(*large)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        got_small = step(*small)   # the side stream's first call
        got_large = step(*large)   # needs more than that: the workspace grows
        got_small2 = step(*small)  # fits what is there
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    for got, ref in ((got_small, ref_small), (got_large, ref_large), (got_small2, ref_small)):
        assert torch.equal(got, ref)
