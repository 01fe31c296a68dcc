"""The seeded input module: deterministic, right shapes, right outlier count."""
import numpy as np
import pytest

import workloads as wl


def test_all_five_workloads_have_the_stated_shapes():
    w = [wl.TINY_SQA_FP32, wl.SSQA_1K_CAUSAL, wl.XSQA_32K, wl.SQA_131K_CAUSAL, wl.XSMQA_200K]
    assert all(wl.WORKLOADS[x.name] is x for x in w)
    assert [x.N for x in w] == [256, 1024, 32768, 131072, 200000]
    assert [x.d_head for x in w] == [32, 32, 64, 64, 64]
    assert [(x.H_q, x.H_kv) for x in w] == [(4, 2), (8, 8), (4, 4), (8, 4), (4, 1)]
    assert [(x.baseline().H_q, x.baseline().H_kv) for x in w[1:]] == \
        [(16, 4), (16, 16), (16, 4), (16, 1)]
    with pytest.raises(ValueError):
        wl.TINY_SQA_FP32.baseline()


def test_draws_are_deterministic_and_shaped():
    w = wl.XSMQA_200K.with_(N=3000)
    a, b = wl.draw(w), wl.draw(w)
    for k in a:
        assert np.array_equal(a[k], b[k])
    assert a["X"].shape == (1, 3000, 1024)
    assert a["Wq"].shape == (1024, 256) and a["Wk"].shape == (1024, 64)
    assert a["Wo"].shape == (256, 1024)
    # the baseline reuses X and draws wider weights from the same streams
    base = wl.draw(w.baseline())
    assert np.array_equal(base["X"], a["X"]) and base["Wq"].shape == (1024, 1024)


def test_outliers_are_one_percent_of_rows_scaled_by_twenty():
    w = wl.XSMQA_200K.with_(N=5000)
    rows = wl.outlier_rows(w)
    assert rows.size == 50 and np.unique(rows).size == 50
    x = wl.draw_x(w).reshape(-1, 1024)
    plain = wl.draw_x(w.with_(outlier_frac=0.0)).reshape(-1, 1024)
    np.testing.assert_array_equal(x[rows], plain[rows] * np.float32(20))
    mask = np.ones(5000, bool)
    mask[rows] = False
    np.testing.assert_array_equal(x[mask], plain[mask])


def test_weight_scale_is_one_over_sqrt_d_model():
    w = wl.SQA_131K_CAUSAL.with_(N=8)
    W = wl.draw_weights(w)["Wq"].astype(np.float64)
    assert abs(W.std() - 1 / 32) < 1e-3


def test_device_dtype_rounding_is_exact_to_widen():
    import torch
    t = wl.to_device_dtype(wl.draw(wl.SSQA_1K_CAUSAL.with_(B=1, N=4)), "bf16")
    assert t["X"].dtype == torch.bfloat16
    x = wl.widen(t["X"])
    assert x.dtype == np.float64
    assert np.array_equal(wl.widen(torch.from_numpy(x).to(torch.bfloat16)), x)


def test_varlen_lengths_are_seeded_and_in_range():
    w = wl.SQA_VARLEN_32K
    a, b = wl.draw_lens(w), wl.draw_lens(w)
    assert a.dtype == np.int32 and a.shape == (w.B,)
    np.testing.assert_array_equal(a, b)
    assert a.min() >= w.varlen_min and a.max() <= w.N
    assert len(set(a.tolist())) > 1          # a real length mix
    np.testing.assert_array_equal(wl.draw_lens(wl.XSQA_32K), [wl.XSQA_32K.N])
