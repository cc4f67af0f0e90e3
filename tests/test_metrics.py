"""The tolerance readings of tests/parity.py, checked on hand-made arrays (CPU).

Each metric is exercised with an error planted at a known place and size, so
that a wrong reduction axis, a missing absolute value or a wrong floor in a
metric shows up here rather than as a silently lenient GPU parity test.
"""
import numpy as np
import pytest

from parity import check, head_normwise, m_error


def _ref(B=2, NH=3, T=5, d=4, seed=0):
    return np.random.default_rng(seed).standard_normal((B, NH, T, d))


def test_head_normwise_is_zero_on_equal_arrays():
    r = _ref()
    assert head_normwise(r, r) == 0.0


def test_head_normwise_scales_by_the_head_maximum_of_the_reference():
    r = _ref()
    g = r.copy()
    g[1, 2, 3, 0] += 0.5  # one entry of head (1, 2)
    expect = 0.5 / np.abs(r[1, 2]).max()
    assert head_normwise(g, r) == pytest.approx(expect, rel=1e-12)
    # the worst head decides, not the mean over heads
    g[0, 0, 0, 0] += 1e-3
    assert head_normwise(g, r) == pytest.approx(max(expect, 1e-3 / np.abs(r[0, 0]).max()),
                                                rel=1e-12)


def test_head_normwise_on_per_row_arrays_and_sign():
    n = np.abs(_ref()[..., 0]) + 1.0  # [B, NH, T]
    g = n.copy()
    g[0, 1, 2] -= 0.25  # an error of either sign counts
    assert head_normwise(g, n) == pytest.approx(0.25 / n[0, 1].max(), rel=1e-12)


def test_m_error_is_relative_above_one_and_absolute_below():
    m = np.array([[[-3.0, 0.2, 10.0]]])
    g = m.copy()
    g[0, 0, 1] += 1e-6  # |m| < 1: absolute
    assert m_error(g, m) == pytest.approx(1e-6, rel=1e-9)
    g = m.copy()
    g[0, 0, 2] += 1e-4  # |m| = 10: relative
    assert m_error(g, m) == pytest.approx(1e-5, rel=1e-9)
    g = m.copy()
    g[0, 0, 0] -= 3e-5  # negative m: |m| = 3
    assert m_error(g, m) == pytest.approx(1e-5, rel=1e-9)


def _case(seed=1):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((1, 2, 6, 4))
    m = rng.standard_normal((1, 2, 6))
    n = np.abs(rng.standard_normal((1, 2, 6))) + 0.5
    return h, m, n


def test_check_passes_within_and_fails_outside_each_bar():
    h, m, n = _case()
    out = check(h, m, n, h, m, n, 2e-2)
    assert out["h"] == out["m"] == out["n"] == 0.0
    hb = h.copy()
    hb[0, 1, 2, 3] += 3e-2 * np.abs(h[0, 1]).max()
    with pytest.raises(AssertionError):
        check(hb, m, n, h, m, n, 2e-2)
    check(hb, m, n, h, m, n, 4e-2)
    mb = m.copy()
    mb[0, 0, 0] += 2e-5 * max(abs(m[0, 0, 0]), 1.0)
    with pytest.raises(AssertionError):
        check(h, mb, n, h, m, n, 2e-2)
    nb = n.copy()
    nb[0, 1, 5] *= 1 + 2e-5 * n[0, 1].max() / n[0, 1, 5]
    with pytest.raises(AssertionError):
        check(h, m, nb, h, m, n, 2e-2)


def test_check_excludes_only_cancellation_rows_and_still_checks_their_numerator():
    h, m, _ = _case(2)
    n = np.ones_like(m)
    n[0, 0, 4] = 1e-3  # a row whose normalizer is tiny: h~ there amplifies errors
    kappa = np.ones_like(n)
    kappa[0, 0, 4] = 1e5
    hb = h.copy()
    hb[0, 0, 4] += 0.1 * np.abs(h[0, 0]).max()  # 10 % of the head's max in h~ ...
    # ... but 1e-4 of the head's max in the numerator n h~: passes when excluded
    out = check(hb, m, n, h, m, n, 2e-2, kappa=kappa, kappa_max=1e3)
    assert out["excluded_rows"] == 1 and out["h"] == 0.0
    assert 0.0 < out["numerator"] <= 2e-2
    # checked when kappa is below the cut
    with pytest.raises(AssertionError):
        check(hb, m, n, h, m, n, 2e-2, kappa=np.ones_like(n), kappa_max=1e3)
    # an error that is large in the numerator fails even on an excluded row
    hc = h.copy()
    hc[0, 0, 4] += 1e3 * np.abs(h[0, 0]).max()
    with pytest.raises(AssertionError):
        check(hc, m, n, h, m, n, 2e-2, kappa=kappa, kappa_max=1e3)
