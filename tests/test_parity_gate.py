"""The comparison helper of the GPU parity tests (tests/parity.py), on the CPU:
bf16-level noise passes, and errors confined to a few rows or columns fail
even where the global relative L2 norm and the elementwise bound let them
through."""
import numpy as np

from parity import compare


def _ref(seed=0, rows=1000, cols=512, scale=0.016):
    rng = np.random.default_rng(seed)
    return rng, rng.standard_normal((rows, cols)) * scale


def test_bf16_rounding_noise_passes():
    rng, ref = _ref()
    got = ref * (1 + rng.standard_normal(ref.shape) * 2 ** -9)
    rep = compare(got, ref, "bf16")
    assert rep.ok, rep


def test_one_head_wrong_in_one_row_fails():
    """One head's 64 columns zeroed in one row of 3000: the global relative L2
    norm stays under 1e-2 and every element under 2e-2 (outputs of size
    0.004), but the row gate fails it."""
    rng, ref = _ref(1, rows=3000, scale=0.004)
    got = ref * (1 + rng.standard_normal(ref.shape) * 2 ** -9)
    got[417, 128:192] = 0
    rep = compare(got, ref, "bf16")
    assert rep.rel_l2 < 1e-2 and rep.worst_scaled < 2e-2
    assert not rep.ok and rep.worst_row_rel > 0.1


def test_a_cancelling_row_is_judged_against_the_typical_row():
    """A row 20x smaller than the others (a sum that cancels) with an error of
    2% of its own norm, i.e. 0.1% of a typical row: passes."""
    rng, ref = _ref(2, rows=64, cols=64, scale=1.0)
    ref[5] *= 0.05
    got = ref.copy()
    got[5] += rng.standard_normal(64) * 0.02 * np.linalg.norm(ref[5]) / 8
    rep = compare(got, ref, "bf16")
    assert rep.ok, rep


def test_zero_rows_must_stay_zero():
    _, ref = _ref(3, rows=10, cols=8, scale=1.0)
    ref[4] = 0
    got = ref.copy()
    got[4] = 0.3
    assert not compare(got, ref, "bf16").ok


def test_fp32_gate_is_max_abs():
    _, ref = _ref(4, rows=4, cols=4, scale=1.0)
    assert compare(ref + 5e-5, ref, "fp32").ok
    assert not compare(ref + 2e-4, ref, "fp32").ok
