"""sqa_forward_noalloc (the forward that allocates nothing) through the C ABI,
against sqa_forward on the same inputs: bitwise equal outputs on two calls in
a row, the second on a smaller input, so the second call runs on what the
first left in the fixed device array. Also the host-side rejection of a
workspace beyond the array (SQA_ERR_UNSUPPORTED, nothing written)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import sparse_query_attention_amd as sqa
import workloads as wl
from parity import compare, log
from sparse_query_attention_amd import _lib

pytestmark = pytest.mark.gpu

LIMIT = 128 << 20   # SQA_NOALLOC_SCRATCH_BYTES


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()   # the HIP library, never a stand-in
    return torch.device("cuda:0")


def _inputs(w, dev):
    host = wl.to_device_dtype(wl.draw(w), w.dtype)
    return host, {k: v.to(dev) for k, v in host.items()}


def _both(w, d):
    kw = dict(H=w.H, H_q=w.H_q, H_kv=w.H_kv, causal=w.causal)
    y_ref = sqa.forward(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], **kw)
    y = torch.full_like(d["X"], float("nan"))
    sqa.forward_noalloc(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], out=y, **kw)
    torch.cuda.synchronize()
    return y, y_ref


def test_noalloc_matches_forward_on_two_calls_the_second_smaller(dev):
    # 1) the headline head shape at 32768 tokens (a workspace of about 104 MB)
    big = wl.SQA_131K_CAUSAL.with_(name="noalloc_big", N=32768, seed=2201)
    # 2) a smaller, ragged, non-causal call: it reuses the array's first bytes
    small = wl.Workload("noalloc_small", B=3, N=777, d_model=512, H=16, H_q=4, H_kv=2,
                        causal=False, dtype="bf16", seed=2202)
    for w in (big, small):
        log(f"case noalloc {w.name}: B={w.B} N={w.N} H_q={w.H_q} H_kv={w.H_kv} causal={w.causal}")
        host, d = _inputs(w, dev)
        y, y_ref = _both(w, d)
        assert torch.equal(y, y_ref), w.name
        if w is small:   # and the oracle, to the bf16 tolerances
            o = {k: wl.widen(v) for k, v in host.items()}
            ref = oracle.sqa_forward(o["X"], o["Wq"], o["Wk"], o["Wv"], o["Wo"], w.H_q, w.H_kv,
                                     w.d_head, w.causal, bf16=True)["Y"]
            rep = compare(wl.widen(y.cpu()), ref, w.dtype)
            log(f"  Y: {rep}")
            assert rep.ok, rep


def test_noalloc_key_split_tail(dev):
    """A non-causal grid of 320 work items on 256 CUs, whose partial last round
    runs split over the keys: the split states sit in the fixed array too
    (about 120 MB of workspace in all), and the result is bitwise sqa_forward's."""
    w = wl.Workload("noalloc_split", B=1, N=20000, d_model=1024, H=16, H_q=8, H_kv=8,
                    causal=False, dtype="bf16", seed=2204)
    log(f"case noalloc {w.name}: B={w.B} N={w.N} H_q={w.H_q} H_kv={w.H_kv} causal={w.causal}")
    _, d = _inputs(w, dev)
    for _ in range(2):
        y, y_ref = _both(w, d)
        assert torch.equal(y, y_ref)


def test_noalloc_fp32_and_repeat(dev):
    w = wl.TINY_SQA_FP32
    _, d = _inputs(w, dev)
    for _ in range(2):
        y, y_ref = _both(w, d)
        assert torch.equal(y, y_ref)


def test_noalloc_rejects_a_workspace_beyond_the_array(dev):
    """The headline head shape at 65536 tokens needs about 200 MB of workspace:
    SQA_ERR_UNSUPPORTED before anything is enqueued, and out untouched."""
    w = wl.SQA_131K_CAUSAL.with_(name="noalloc_too_big", N=65536, seed=2203)
    _, d = _inputs(w, dev)
    out = torch.zeros_like(d["X"])
    with pytest.raises(NotImplementedError, match="SQA_NOALLOC_SCRATCH_BYTES"):
        sqa.forward_noalloc(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], H=w.H, H_q=w.H_q,
                            H_kv=w.H_kv, causal=True, out=out)
    torch.cuda.synchronize()
    assert not out.any()
