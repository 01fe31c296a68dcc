"""Parity of the HIP path (through the C ABI) with the float64 CPU oracle.

Small shapes are compared element by element over the whole output. They
span several key/query tiles plus a ragged tail, every query-group size, both
head widths, both dtypes and both masks. The five full workloads run at their
real sizes in the launch configuration the benchmark times. Their outputs are
compared on sampled rows that the oracle computes one by one.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
import sparse_query_attention_amd as sqa
import workloads as wl
from parity import compare, device_inputs, log, oracle_inputs, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sqa._lib.load()   # the HIP library, never a stand-in
    return torch.device("cuda:0")


def run_forward(w, d):
    return sqa.forward(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], H=w.H, H_q=w.H_q, H_kv=w.H_kv,
                       causal=w.causal)


def full_check(w, dev, stages=False):
    log(f"case {w.name}: B={w.B} N={w.N} d_model={w.d_model} H={w.H} H_q={w.H_q} H_kv={w.H_kv} "
        f"causal={w.causal} dtype={w.dtype}")
    host, d = device_inputs(w, dev)
    y = run_forward(w, d)
    torch.cuda.synchronize()
    o = oracle_inputs(host)
    ref = oracle.sqa_forward(o["X"], o["Wq"], o["Wk"], o["Wv"], o["Wo"], w.H_q, w.H_kv, w.d_head,
                             w.causal, bf16=(w.dtype == "bf16"))
    rep = compare(wl.widen(y.cpu()), ref["Y"], w.dtype)
    log(f"  Y: {rep}")
    assert rep.ok, f"{w.name}: {rep}"
    if stages:
        check_stages(w, d, ref, o)
    return y


def check_stages(w, d, ref, o):
    """Each C-ABI step against the oracle's intermediate of the same name."""
    q, k, vt = sqa.qkv_projection(d["X"], d["Wq"], d["Wk"], d["Wv"], H=w.H, H_q=w.H_q, H_kv=w.H_kv)
    a = sqa.attention(q, k, vt, N=w.N, causal=w.causal)
    y = sqa.output_projection(a, d["Wo"])
    torch.cuda.synchronize()
    B, N, dh = w.B, w.N, w.d_head
    Np = sqa.padded_length(N)
    qh = wl.widen(q.cpu())
    kh = wl.widen(k.cpu())
    vh = wl.widen(vt.cpu())
    # padded rows are zeros (the attention step relies on finite padding)
    assert not qh[:, :, N:].any() and not kh[:, :, N:].any() and not vh[..., N:].any()
    Q = ref["Q"].reshape(B, N, w.H_q, dh).transpose(0, 2, 1, 3)
    K = ref["K"].reshape(B, N, w.H_kv, dh).transpose(0, 2, 1, 3)
    V = ref["V"].reshape(B, N, w.H_kv, dh).transpose(0, 2, 3, 1)
    # Projections: the GPU sums K = d_model products in fp32 and rounds once.
    # It may miss the exactly rounded value by one bf16 ulp plus the fp32
    # summation error bound K * 2^-24 * sum_k |x_k w_k|; the latter dominates
    # for results near zero that come from cancelling terms.
    def heads(M, n, t):
        return M.reshape(B, N, n, dh).transpose(*t)
    absx = np.abs(o["X"])
    bounds = {nm: w.d_model * 2.0 ** -24 * (absx @ np.abs(o[wn]))
              for nm, wn in (("Q", "Wq"), ("K", "Wk"), ("V^T", "Wv"))}
    for name, got, want, n, t in (("Q", qh[:, :, :N], Q, w.H_q, (0, 2, 1, 3)),
                                  ("K", kh[:, :, :N], K, w.H_kv, (0, 2, 1, 3)),
                                  ("V^T", vh[..., :N], V, w.H_kv, (0, 2, 3, 1))):
        bound = heads(bounds[name], n, t)
        diff = np.abs(got - want)
        if w.dtype == "bf16":
            ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(want), 1e-30))) - 7)
            bad = diff > ulp * 1.0001 + bound
            exact = float((diff == 0).mean())
            log(f"  {name}: exact={exact:.5f} beyond_bound={int(bad.sum())}")
            assert not bad.any() and exact > 0.99, name
        else:
            bad = diff > 2.0 ** -24 * np.abs(want) + bound
            log(f"  {name}: max_abs={float(diff.max()):.3e} beyond_bound={int(bad.sum())}")
            assert not bad.any(), name
    rep_a = compare(wl.widen(a.cpu()).reshape(B, N, -1), ref["A"], w.dtype)
    log(f"  A: {rep_a}")
    assert rep_a.ok
    rep_y = compare(wl.widen(y.cpu()).reshape(B, N, -1), ref["Y"], w.dtype)
    log(f"  Y (staged): {rep_y}")
    assert rep_y.ok


# ----------------------------------------------------------------------------------------------
# small shapes: whole outputs

HEADS = [  # (H, d_head, H_q, H_kv): g = 1, 2, 16, 2, 8, 3
    (16, 64, 4, 4), (16, 64, 8, 4), (16, 64, 16, 1), (8, 32, 4, 2), (16, 32, 16, 2), (8, 32, 6, 2),
]
LENGTHS = [(1, False), (2, True), (17, False), (63, True), (64, False), (65, True), (127, False),
           (255, True), (257, False), (1000, True), (4097, True), (2500, False)]


def _small_cases():
    cases = []
    for dtype in ("bf16", "fp32"):
        for i, (N, causal) in enumerate(LENGTHS):
            H, dh, H_q, H_kv = HEADS[(i + (dtype == "fp32")) % len(HEADS)]
            B = 3 if i % 3 == 0 else 1
            cases.append(wl.Workload(f"small_{dtype}_N{N}_{'c' if causal else 'nc'}_g{H_q // H_kv}",
                                     B=B, N=N, d_model=H * dh, H=H, H_q=H_q, H_kv=H_kv,
                                     causal=causal, dtype=dtype, seed=500 + i))
    return cases


@pytest.mark.parametrize("w", _small_cases(), ids=lambda w: w.name)
def test_small_shapes_match_oracle(dev, w):
    full_check(w, dev)


@pytest.mark.parametrize("H,dh,H_q,H_kv", HEADS, ids=lambda v: str(v))
@pytest.mark.parametrize("dtype,causal", [("bf16", True), ("fp32", False)])
def test_every_stage_matches_oracle(dev, H, dh, H_q, H_kv, dtype, causal):
    w = wl.Workload(f"stages_{dtype}_{H_q}_{H_kv}_{dh}", B=2, N=333, d_model=H * dh, H=H, H_q=H_q,
                    H_kv=H_kv, causal=causal, dtype=dtype, seed=77)
    full_check(w, dev, stages=True)


def test_tiny_fp32_workload(dev):
    full_check(wl.TINY_SQA_FP32, dev, stages=True)


def test_ssqa_1k_causal_workload_and_gqa_baseline(dev):
    full_check(wl.SSQA_1K_CAUSAL, dev, stages=True)
    full_check(wl.SSQA_1K_CAUSAL.baseline(), dev)


# ----------------------------------------------------------------------------------------------
# full sizes: sampled rows

LONG = [wl.XSQA_32K, wl.SQA_131K_CAUSAL, wl.XSMQA_200K]
# fixed H_q = 4 at 32k tokens with fewer key/value heads (the bench's H_kv sweep)
HKV_SWEEP = [wl.XSQA_32K.with_(name=f"xsqa_bf16_n32768_hkv{h}", H_kv=h, baseline_H_q=None,
                               baseline_H_kv=None) for h in (2, 1)]


@pytest.mark.parametrize("w", LONG + [x.baseline() for x in LONG] + HKV_SWEEP, ids=lambda w: w.name)
def test_long_workloads_on_sampled_rows(dev, w):
    log(f"case {w.name}: B={w.B} N={w.N} H_q={w.H_q} H_kv={w.H_kv} causal={w.causal}")
    host, d = device_inputs(w, dev)
    y = run_forward(w, d)
    torch.cuda.synchronize()
    rows = sample_rows(w, n_random=64 if w.H_q > 8 else 96)
    yg = wl.widen(y.reshape(-1, w.d_model)[torch.from_numpy(rows).to(dev)].cpu())
    del d, y
    o = oracle_inputs(host)
    ref = oracle.sqa_forward_rows(o["X"], o["Wq"], o["Wk"], o["Wv"], o["Wo"], w.H_q, w.H_kv,
                                  w.d_head, w.causal, bf16=True, rows=rows)["Y_rows"]
    rep = compare(yg, ref, w.dtype)
    log(f"  {rows.size} rows: {rep}")
    assert rep.ok, f"{w.name}: {rep}"


@pytest.mark.parametrize("w", LONG, ids=lambda w: w.name)
def test_long_workloads_write_every_element(dev, w):
    """Every output element of every step is written, at the full sizes and
    launch shapes that the bench times (work-unit order, tails, padding): the
    buffers start as NaN and must come back finite."""
    log(f"case {w.name}: every element written")
    _, d = device_inputs(w, dev)
    Np = sqa.padded_length(w.N)
    nan = float("nan")
    q = torch.full((w.B, w.H_q, Np, w.d_head), nan, dtype=torch.bfloat16, device=dev)
    k = torch.full((w.B, w.H_kv, Np, w.d_head), nan, dtype=torch.bfloat16, device=dev)
    vt = torch.full((w.B, w.H_kv, w.d_head, Np), nan, dtype=torch.bfloat16, device=dev)
    sqa.qkv_projection(d["X"], d["Wq"], d["Wk"], d["Wv"], H=w.H, H_q=w.H_q, H_kv=w.H_kv, q=q, k=k, vt=vt)
    a = torch.full((w.B * w.N, w.H_q * w.d_head), nan, dtype=torch.bfloat16, device=dev)
    sqa.attention(q, k, vt, N=w.N, causal=w.causal, a=a)
    y = torch.full((w.B * w.N, w.d_model), nan, dtype=torch.bfloat16, device=dev)
    sqa.output_projection(a, d["Wo"], out=y)
    torch.cuda.synchronize()
    for name, t in (("q", q), ("k", k), ("vt", vt), ("a", a), ("y", y)):
        assert bool(torch.isfinite(t).all()), f"{w.name}: {name} has unwritten elements"
    assert not bool(q[:, :, w.N:].any()) and not bool(vt[..., w.N:].any()), "padding rows not zero"


# A non-causal grid of 8 KV heads x 40 query tiles = 320 work items on 256 CUs: the 64 items
# of the partial last round are split into 4 key ranges of 5056 keys (the last one ragged,
# 4832 keys) and merged. Heads 6 and 7 hold the split items.
KEY_SPLIT = wl.Workload("key_split_bf16_n20000", B=1, N=20000, d_model=1024, H=16, H_q=8, H_kv=8,
                        causal=False, dtype="bf16", seed=3301)


def test_key_split_tail_on_sampled_rows(dev):
    w = KEY_SPLIT
    log(f"case {w.name}: B={w.B} N={w.N} H_q={w.H_q} H_kv={w.H_kv} causal={w.causal}")
    host, d = device_inputs(w, dev)
    y = run_forward(w, d)
    q, k, vt = sqa.qkv_projection(d["X"], d["Wq"], d["Wk"], d["Wv"], H=w.H, H_q=w.H_q, H_kv=w.H_kv)
    a = sqa.attention(q, k, vt, N=w.N, causal=w.causal)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[sample_rows(w, n_random=96), np.arange(w.N - 70, w.N)])
    idx = torch.from_numpy(rows).to(dev)
    ag = wl.widen(a.reshape(-1, w.H_q * w.d_head)[idx].cpu())
    yg = wl.widen(y.reshape(-1, w.d_model)[idx].cpu())
    o = oracle_inputs(host)
    ref = oracle.sqa_forward_rows(o["X"], o["Wq"], o["Wk"], o["Wv"], o["Wo"], w.H_q, w.H_kv,
                                  w.d_head, w.causal, bf16=True, rows=rows)
    for name, got, r in (("A", ag, ref["A_rows"]), ("Y", yg, ref["Y_rows"])):
        rep = compare(got, r, w.dtype)
        log(f"  {name} on {rows.size} rows: {rep}")
        assert rep.ok, f"{w.name} {name}: {rep}"
    # the split heads (6 and 7) on their own
    split_cols = slice(6 * w.d_head, 8 * w.d_head)
    rep = compare(ag[:, split_cols], ref["A_rows"][:, split_cols], w.dtype)
    log(f"  A of heads 6-7: {rep}")
    assert rep.ok, rep


def test_key_split_tail_two_sequences_head_pairs_d32(dev):
    """2 sequences x 4 KV heads x 40 query tiles of 256 rows (2 query heads per
    KV head, d_head 32) = 320 items: the 64 split items all lie in the second
    sequence (heads 4-7 of it), 4 parts of 2560 keys, the last 2320. Every row
    of that sequence against the oracle, and sampled rows of the first."""
    w = wl.Workload("key_split_bf16_b2_n10000_d32", B=2, N=10000, d_model=512, H=16, H_q=8,
                    H_kv=4, causal=False, dtype="bf16", seed=3303)
    log(f"case {w.name}: B={w.B} N={w.N} H_q={w.H_q} H_kv={w.H_kv} d_head={w.d_head}")
    host, d = device_inputs(w, dev)
    q, k, vt = sqa.qkv_projection(d["X"], d["Wq"], d["Wk"], d["Wv"], H=w.H, H_q=w.H_q, H_kv=w.H_kv)
    a = sqa.attention(q, k, vt, N=w.N, causal=w.causal)
    y = run_forward(w, d)
    torch.cuda.synchronize()
    rows = np.r_[np.arange(0, w.N, 97), np.arange(w.N, 2 * w.N)]
    idx = torch.from_numpy(rows).to(dev)
    ag = wl.widen(a.reshape(-1, w.H_q * w.d_head)[idx].cpu())
    yg = wl.widen(y.reshape(-1, w.d_model)[idx].cpu())
    o = oracle_inputs(host)
    ref = oracle.sqa_forward_rows(o["X"], o["Wq"], o["Wk"], o["Wv"], o["Wo"], w.H_q, w.H_kv,
                                  w.d_head, w.causal, bf16=True, rows=rows)
    for name, got, r in (("A", ag, ref["A_rows"]), ("Y", yg, ref["Y_rows"])):
        rep = compare(got, r, w.dtype)
        log(f"  {name} on {rows.size} rows: {rep}")
        assert rep.ok, f"{w.name} {name}: {rep}"


# ----------------------------------------------------------------------------------------------
# determinism and edge cases

def test_bitwise_deterministic_across_calls_and_streams(dev):
    w = wl.Workload("determinism", B=2, N=777, d_model=1024, H=16, H_q=8, H_kv=2, causal=True,
                    dtype="bf16", seed=5)
    _, d = device_inputs(w, dev)
    y1 = run_forward(w, d)
    y2 = run_forward(w, d)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y3 = run_forward(w, d)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(y1, y3)


def test_single_token_returns_projected_value(dev):
    """N = 1: softmax over one key is 1, so A = V and Y = V Wo per head."""
    w = wl.Workload("one_token", B=4, N=1, d_model=512, H=8, H_q=4, H_kv=2, causal=False,
                    dtype="fp32", seed=9)
    host, d = device_inputs(w, dev)
    y = run_forward(w, d)
    o = oracle_inputs(host)
    V = o["X"] @ o["Wv"]
    A = np.concatenate([V[..., 0:64], V[..., 0:64], V[..., 64:128], V[..., 64:128]], axis=-1)
    rep = compare(wl.widen(y.cpu()), A @ o["Wo"], "fp32")
    log(f"  {rep}")
    assert rep.ok


def test_empty_batch_is_a_no_op(dev):
    x = torch.empty((0, 5, 256), dtype=torch.bfloat16, device=dev)
    W = {k: torch.zeros(s, dtype=torch.bfloat16, device=dev)
         for k, s in (("q", (256, 128)), ("k", (256, 64)), ("v", (256, 64)), ("o", (128, 256)))}
    y = sqa.forward(x, W["q"], W["k"], W["v"], W["o"], H=8, H_q=4, H_kv=2)
    assert y.shape == (0, 5, 256)


def test_maximum_sequence_length_on_sampled_rows(dev):
    """N = SQA_MAX_N = 2^24 tokens (one head, d_head 32, causal): every token,
    tile and workgroup index of the path at its largest, against the oracle on
    rows spread over the whole sequence."""
    N = 1 << 24
    w = wl.Workload("max_n_causal", B=1, N=N, d_model=32, H=1, H_q=1, H_kv=1, causal=True,
                    dtype="bf16", seed=1234)
    log(f"case maximum length: N={N}")
    host, d = device_inputs(w, dev)
    y = run_forward(w, d)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all())
    rows = np.array([0, 1, 31, 32, 511, 512, 65535, 65536, (1 << 23) - 1, 1 << 23, 12345678,
                     N - 513, N - 512, N - 2, N - 1], dtype=np.int64)
    yg = wl.widen(y.reshape(-1, w.d_model)[torch.from_numpy(rows).to(dev)].cpu())
    del d, y
    o = oracle_inputs(host)
    ref = oracle.sqa_forward_rows(o["X"], o["Wq"], o["Wk"], o["Wv"], o["Wo"], w.H_q, w.H_kv,
                                  w.d_head, w.causal, bf16=True, rows=rows, row_block=1)["Y_rows"]
    rep = compare(yg, ref, w.dtype)
    log(f"  {rows.size} rows: {rep}")
    assert rep.ok, rep



@pytest.mark.parametrize("causal", [True, False])
def test_sixty_four_query_heads_per_key_value_head(dev, causal):
    """g = 64 (H_q = 64, H_kv = 1): eight 8-head workgroups per key/value
    stream in the attention, every stage against the oracle."""
    w = wl.Workload(f"g64_{'c' if causal else 'nc'}", B=1, N=150, d_model=64 * 32, H=64, H_q=64,
                    H_kv=1, causal=causal, dtype="bf16", seed=777)
    full_check(w, dev, stages=True)
