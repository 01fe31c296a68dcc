"""Variable-length batches (sqa_forward_varlen) against the oracle: sequences
padded to N, each an independent forward over its own tokens, zero rows in the
padding. The padding rows of x hold NaN, so anything read from them would show."""
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


def _run(w, lens, dev, nan_padding=True):
    host, d = device_inputs(w, dev)
    x = d["X"].clone()
    if nan_padding:
        for b, L in enumerate(np.clip(lens, 0, w.N)):
            x[b, int(L):] = float("nan")
    lt = torch.tensor(np.asarray(lens, dtype=np.int32), device=dev)
    y = sqa.forward_varlen(x, d["Wq"], d["Wk"], d["Wv"], d["Wo"], lt, H=w.H, H_q=w.H_q,
                           H_kv=w.H_kv, causal=w.causal)
    torch.cuda.synchronize()
    return host, wl.widen(y.cpu())


def _check_all_rows(w, lens, dev):
    log(f"case {w.name}: lens={list(lens)} causal={w.causal} dtype={w.dtype}")
    host, got = _run(w, lens, dev)
    o = oracle_inputs(host)
    Lc = np.clip(lens, 0, w.N)
    ref = oracle.sqa_forward_varlen(o["X"], o["Wq"], o["Wk"], o["Wv"], o["Wo"], Lc, w.H_q, w.H_kv,
                                    w.d_head, w.causal, bf16=(w.dtype == "bf16"))
    for b, L in enumerate(Lc):
        assert not np.any(got[b, int(L):]), f"padding rows of sequence {b} are not zero"
    rep = compare(got, ref, w.dtype)
    log(f"  {rep}")
    assert rep.ok, rep


SMALL = [
    wl.Workload("varlen_small_d32", B=5, N=300, d_model=256, H=8, H_q=4, H_kv=2, causal=False,
                dtype="bf16", seed=71),
    wl.Workload("varlen_small_d64", B=3, N=1500, d_model=1024, H=16, H_q=8, H_kv=4, causal=False,
                dtype="bf16", seed=72),
    wl.Workload("varlen_small_fp32", B=4, N=200, d_model=256, H=8, H_q=4, H_kv=4, causal=False,
                dtype="fp32", seed=73),
]
LENS = {"varlen_small_d32": [300, 1, 0, 157, 256], "varlen_small_d64": [1500, 700, 33],
        "varlen_small_fp32": [200, 65, 64, 0]}


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_ragged_batches_match_oracle(dev, w, causal):
    _check_all_rows(w.with_(causal=causal), LENS[w.name], dev)


def test_out_of_range_lengths_are_clamped(dev):
    w = SMALL[0].with_(causal=True)
    _check_all_rows(w, [-7, 10 * w.N, 3, 0, 2 ** 31 - 1], dev)


def test_full_lengths_equal_plain_forward(dev):
    w = wl.Workload("varlen_full", B=2, N=777, d_model=1024, H=16, H_q=8, H_kv=2, causal=True,
                    dtype="bf16", seed=74)
    _, d = device_inputs(w, dev)
    lt = torch.full((w.B,), w.N, dtype=torch.int32, device=dev)
    y1 = sqa.forward_varlen(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], lt, H=w.H, H_q=w.H_q,
                            H_kv=w.H_kv, causal=True)
    y2 = sqa.forward(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], H=w.H, H_q=w.H_q, H_kv=w.H_kv,
                     causal=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def _varlen_rows(w, lens, n_random=24, seed=0):
    rng = np.random.default_rng(seed)
    rows = []
    for b, L in enumerate(lens):
        L = int(L)
        ts = {0, 1, 31, 32, 63, 64, 255, 256, L // 2, L - 257, L - 65, L - 2, L - 1}
        ts.update(rng.integers(0, max(L, 1), size=n_random // len(lens) + 1).tolist())
        ts = {t for t in ts if 0 <= t < L}
        ts.update(t for t in (L, L + 1, w.N - 1) if L <= t < w.N)   # padding rows
        rows.extend(b * w.N + t for t in sorted(ts))
    return np.asarray(rows, dtype=np.int64)


def test_full_size_length_mix_on_sampled_rows(dev):
    w = wl.SQA_VARLEN_32K
    lens = wl.draw_lens(w)
    log(f"case {w.name}: lens={lens.tolist()}")
    host, d = device_inputs(w, dev)
    x = d["X"].clone()
    for b, L in enumerate(lens):
        x[b, int(L):] = float("nan")
    y = sqa.forward_varlen(x, d["Wq"], d["Wk"], d["Wv"], d["Wo"],
                           torch.from_numpy(lens).to(dev), H=w.H, H_q=w.H_q, H_kv=w.H_kv,
                           causal=w.causal)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all())
    rows = _varlen_rows(w, lens)
    yg = wl.widen(y.reshape(-1, w.d_model)[torch.from_numpy(rows).to(dev)].cpu())
    del d, x, y
    o = oracle_inputs(host)
    ref = oracle.sqa_forward_varlen_rows(o["X"], o["Wq"], o["Wk"], o["Wv"], o["Wo"], lens, w.H_q,
                                         w.H_kv, w.d_head, w.causal, bf16=True, rows=rows)
    rep = compare(yg, ref, w.dtype)
    log(f"  {rows.size} rows: {rep}")
    assert rep.ok, rep
