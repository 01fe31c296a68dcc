"""Randomized shape sweep of every entry point against the oracle (GPU).

Each case draws (from a fixed seed) a batch size, a sequence length that is
usually not a multiple of any tile, a head width, head counts with
H_kv | H_q <= H, a mask and a dtype. It then checks:
- sqa_forward;
- sqa_forward_varlen with random lengths, including 0;
- sqa_prefill followed by decode steps, and the causal forward rows;
- sqa_backward, from saved activations or recomputing them.
Each is compared with the oracle under the dtype's tolerance (tests/parity.py).
The sweep complements the hand-picked shapes of the other GPU tests:
tile-boundary lengths, odd head counts, one-token sequences and d_model not a
multiple of 64 all come up.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_query_attention_amd as sqa
import workloads as wl
from parity import MIN_TOKENS_FOR_ROW_GATE, compare, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sqa._lib.load()   # the HIP library, never a stand-in
    return torch.device("cuda:0")


def _shape(seed):
    r = np.random.default_rng([2024, seed])
    d = int(r.choice([32, 64]))
    H = int(r.integers(1, 9))
    divisors = [h for h in range(1, H + 1)]
    H_q = int(r.choice(divisors))
    H_kv = int(r.choice([k for k in range(1, H_q + 1) if H_q % k == 0]))
    B = int(r.integers(1, 4))
    N = int(r.choice([1, 2, 31, 33, 63, 65, 127, 129, 255, 257, 300, 511, 513, 700]))
    causal = bool(r.integers(0, 2))
    dtype = "fp32" if r.random() < 0.25 else "bf16"
    return wl.Workload(f"sweep{seed}", B=B, N=N, d_model=H * d, H=H, H_q=H_q, H_kv=H_kv,
                       causal=causal, dtype=dtype, seed=5000 + seed)


def _inputs(w, dev, grad=False):
    arrays = wl.draw(w)
    if grad:
        arrays["dY"] = wl.draw_upstream_grad(w)
    host = wl.to_device_dtype(arrays, w.dtype)
    return {k: wl.widen(v) for k, v in host.items()}, {k: v.to(dev) for k, v in host.items()}


def _check(got, ref, dtype, what, row_gate=True):
    rep = compare(wl.widen(got.cpu()), ref, dtype, row_gate)
    log(f"  {what}: {rep}")
    assert rep.ok, (what, rep)


SEEDS = list(range(48))


@pytest.mark.parametrize("seed", SEEDS)
def test_sweep_forward_and_varlen(dev, seed):
    w = _shape(seed)
    log(f"case sweep {seed}: B={w.B} N={w.N} H={w.H} d={w.d_head} H_q={w.H_q} H_kv={w.H_kv} "
        f"causal={w.causal} {w.dtype}")
    o, d = _inputs(w, dev)
    bf = w.dtype == "bf16"
    y = sqa.forward(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], H=w.H, H_q=w.H_q, H_kv=w.H_kv,
                    causal=w.causal)
    ref = oracle.sqa_forward(o["X"], o["Wq"], o["Wk"], o["Wv"], o["Wo"], w.H_q, w.H_kv, w.d_head,
                             w.causal, bf)["Y"]
    torch.cuda.synchronize()
    _check(y, ref, w.dtype, "forward")
    r = np.random.default_rng([77, seed])
    lens = r.integers(0, w.N + 1, size=w.B).astype(np.int32)
    lens[r.integers(0, w.B)] = w.N if r.random() < 0.5 else 0
    yv = sqa.forward_varlen(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"],
                            torch.from_numpy(lens).to(dev), H=w.H, H_q=w.H_q, H_kv=w.H_kv,
                            causal=w.causal)
    refv = oracle.sqa_forward_varlen(o["X"], o["Wq"], o["Wk"], o["Wv"], o["Wo"], lens, w.H_q,
                                     w.H_kv, w.d_head, w.causal, bf)
    torch.cuda.synchronize()
    _check(yv, refv, w.dtype, f"varlen lens={lens.tolist()}")


@pytest.mark.parametrize("seed", SEEDS[:24])
def test_sweep_prefill_and_decode(dev, seed):
    w = _shape(seed)
    w = w.with_(causal=True, N=max(w.N, 3))
    log(f"case sweep decode {seed}: B={w.B} N={w.N} H={w.H} d={w.d_head} H_q={w.H_q} "
        f"H_kv={w.H_kv} {w.dtype}")
    o, d = _inputs(w, dev)
    tdt = d["X"].dtype
    n_pre = max(1, w.N - 3)
    N_max = w.N + 5
    kc = torch.full((w.B, w.H_kv, N_max, w.d_head), float("nan"), dtype=tdt, device=dev)
    vc = torch.full_like(kc, float("nan"))
    sqa.prefill(d["X"][:, :n_pre].contiguous(), d["Wq"], d["Wk"], d["Wv"], d["Wo"], kc, vc,
                H=w.H, H_q=w.H_q, H_kv=w.H_kv)
    ys = []
    for t in range(n_pre, w.N):
        pos = torch.full((w.B,), t, dtype=torch.int32, device=dev)
        ys.append(sqa.decode_step(d["X"][:, t].contiguous(), d["Wq"], d["Wk"], d["Wv"], d["Wo"],
                                  kc, vc, pos, H=w.H, H_q=w.H_q, H_kv=w.H_kv))
    torch.cuda.synchronize()
    got = np.stack([wl.widen(y.cpu()) for y in ys], axis=1)
    rows = np.array([b * w.N + t for b in range(w.B) for t in range(n_pre, w.N)])
    ref = oracle.sqa_forward_rows(o["X"], o["Wq"], o["Wk"], o["Wv"], o["Wo"], w.H_q, w.H_kv,
                                  w.d_head, True, bf16=(w.dtype == "bf16"), rows=rows)["Y_rows"]
    rep = compare(got, ref.reshape(w.B, w.N - n_pre, w.d_model), w.dtype)
    log(f"  decode: {rep}")
    assert rep.ok, rep


@pytest.mark.parametrize("seed", SEEDS[:32])
def test_sweep_backward(dev, seed):
    w = _shape(seed)
    log(f"case sweep backward {seed}: B={w.B} N={w.N} H={w.H} d={w.d_head} H_q={w.H_q} "
        f"H_kv={w.H_kv} causal={w.causal} {w.dtype}")
    o, d = _inputs(w, dev, grad=True)
    saved = None
    if seed % 2:
        _, saved = sqa.forward_train(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], H=w.H, H_q=w.H_q,
                                     H_kv=w.H_kv, causal=w.causal)
    got = sqa.backward(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], d["dY"], H=w.H, H_q=w.H_q,
                       H_kv=w.H_kv, causal=w.causal, saved=saved)
    torch.cuda.synchronize()
    ref = oracle.sqa_backward(o["X"], o["Wq"], o["Wk"], o["Wv"], o["Wo"], o["dY"], w.H_q, w.H_kv,
                              w.d_head, w.causal, bf16=(w.dtype == "bf16"))
    for k, g in zip(("dX", "dWq", "dWk", "dWv", "dWo"), got):
        _check(g, ref[k], w.dtype, k, k == "dX" or w.tokens >= MIN_TOKENS_FOR_ROW_GATE)
