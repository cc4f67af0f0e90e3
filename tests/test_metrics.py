"""The tolerance readings of tests/parity.py, checked on hand-made arrays (CPU).

Each metric is exercised with an error planted at a known place and size, so
that a wrong reduction axis, a missing absolute value or a wrong floor in a
metric shows up here rather than as a silently lenient GPU parity test.  The
last tests plant errors that the earlier per-head normwise reading (max error
over a head divided by the head's largest value) accepted, and check that the
per-element and per-row readings reject them.
"""
import numpy as np
import pytest

from parity import K_N, check, conditions, head_normwise, m_error, n_bar, n_relative, row_relative


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
    g[0, 0, 0, 0] += 1e-3  # the worst head decides, not the mean over heads
    assert head_normwise(g, r) == pytest.approx(max(expect, 1e-3 / np.abs(r[0, 0]).max()),
                                                rel=1e-12)


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


def test_n_relative_and_its_bar():
    n = np.array([[[2.0, 1e-3, 5.0]]])
    g = n.copy()
    g[0, 0, 1] *= 1 - 3e-6  # an error of either sign counts, relative to that row
    assert n_relative(g, n)[0, 0, 1] == pytest.approx(3e-6, rel=1e-9)
    assert n_relative(g, n)[0, 0, 0] == 0.0
    # the bar is 1e-5 up to kappa = K_N, then grows linearly
    assert np.allclose(n_bar([0.1, 1.0, K_N, 4 * K_N]), [1e-5, 1e-5, 1e-5, 4e-5])


def test_row_relative_scales_by_each_rows_own_maximum():
    r = _ref()
    g = r.copy()
    g[1, 0, 2, 3] += 0.25
    e = row_relative(g, r)
    assert e.shape == r.shape[:-1]
    assert e[1, 0, 2] == pytest.approx(0.25 / np.abs(r[1, 0, 2]).max(), rel=1e-12)
    assert (np.delete(e.reshape(-1), np.ravel_multi_index((1, 0, 2), e.shape)) == 0).all()
    # an all-zero reference row counts the absolute error
    z = np.zeros((1, 1, 2, 3))
    gz = z.copy()
    gz[0, 0, 1, 2] = 1e-3
    assert row_relative(gz, z)[0, 0, 1] == pytest.approx(1e-3)


def _case(seed=1, T=6, d=4):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((1, 2, T, d))
    m = rng.standard_normal((1, 2, T))
    n = np.abs(rng.standard_normal((1, 2, T))) + 0.5
    kappa = np.ones((1, 2, T))
    return h, m, n, kappa


def test_check_passes_within_and_fails_outside_each_bar():
    h, m, n, kap = _case()
    out = check(h, m, n, h, m, n, kap, np.ones_like(kap), 2e-2, 1e3, 2e4)
    assert out["h_rows"] == out["m"] == out["n_strict"] == out["numerator_rows"] == 0.0
    hb = h.copy()
    hb[0, 1, 2, 3] += 3e-2 * np.abs(h[0, 1, 2]).max()
    with pytest.raises(AssertionError):
        check(hb, m, n, h, m, n, kap, np.ones_like(kap), 2e-2, 1e3, 2e4)
    check(hb, m, n, h, m, n, kap, np.ones_like(kap), 4e-2, 1e3, 2e4)
    mb = m.copy()
    mb[0, 0, 0] += 2e-5 * max(abs(m[0, 0, 0]), 1.0)
    with pytest.raises(AssertionError):
        check(h, mb, n, h, m, n, kap, np.ones_like(kap), 2e-2, 1e3, 2e4)
    nb = n.copy()
    nb[0, 1, 5] *= 1 + 2e-5
    with pytest.raises(AssertionError):
        check(h, m, nb, h, m, n, kap, np.ones_like(kap), 2e-2, 1e3, 2e4)
    # the same n error passes on a row whose condition number allows it
    k2 = kap.copy()
    k2[0, 1, 5] = 3 * K_N
    out = check(h, m, nb, h, m, n, k2, np.ones_like(k2), 2e-2, 1e3, 2e4)
    assert out["n_strict"] == pytest.approx(2e-5, rel=1e-6)
    assert out["n_over_bar"] == pytest.approx(2e-5 / 3e-5, rel=1e-6)


def test_check_excludes_only_cancellation_rows_and_still_checks_their_numerator():
    """On a row with cancellation (kappa 1e5), an n off by 5 % is within its
    bar, and h~ = numerator / n is then off by the same 5 %: the h~ reading
    skips the row (kappa > kappa_h) while its numerator n h~ is exact."""
    h, m, n, kap = _case(2)
    kap[0, 0, 4] = 1e5
    nb = n.copy()
    nb[0, 0, 4] *= 1.05
    hb = h.copy()
    hb[0, 0, 4] = h[0, 0, 4] * n[0, 0, 4] / nb[0, 0, 4]
    out = check(hb, m, nb, h, m, n, kap, np.ones_like(kap), 2e-2, 1e3, 2e4)
    assert out["rows_not_in_h_check"] == 1 and out["h_rows"] == 0.0
    assert out["h_rows_all"] == pytest.approx(0.05 / 1.05, rel=1e-6)
    assert out["numerator_rows"] <= 1e-12
    # an h~ error that is also in the numerator is rejected on that row
    hc = hb.copy()
    hc[0, 0, 4, 0] += 0.1 * np.abs(hb[0, 0, 4]).max()
    with pytest.raises(AssertionError):
        check(hc, m, nb, h, m, n, kap, np.ones_like(kap), 2e-2, 1e3, 2e4)
    # the same row below kappa_h: the h~ reading itself rejects the 5 %
    k1 = kap.copy()
    k1[0, 0, 4] = 2e2  # n's bar at kappa 200 is 2e-4: use an exact n
    hd = h.copy()
    hd[0, 0, 4] *= 1.05
    with pytest.raises(AssertionError):
        check(hd, m, n, h, m, n, k1, np.ones_like(k1), 2e-2, 1e3, 2e4)


def test_per_row_readings_reject_what_the_head_normwise_reading_accepted():
    """One head of 64 rows.  Row 0 sits at the normalizer floor with a huge n
    (exp(-m) for m = -20) and large h~; row 9 has n of order one.  A 1 % error
    in row 9's n, or a 30 % error in its h~, disappears in the head-normwise
    reading but fails the per-row ones."""
    rng = np.random.default_rng(3)
    T, d = 64, 8
    h = rng.standard_normal((1, 1, T, d))
    h[0, 0, 0] *= 1e4
    m = rng.uniform(-1, 1, (1, 1, T))
    m[0, 0, 0] = -20.0
    n = np.abs(rng.standard_normal((1, 1, T))) + 0.5
    n[0, 0, 0] = np.exp(20.0)
    kap = np.full((1, 1, T), 2.0)
    nb = n.copy()
    nb[0, 0, 9] *= 1.01
    assert head_normwise(nb, n) <= 1e-5  # the old n reading: accepted
    with pytest.raises(AssertionError):
        check(h, m, nb, h, m, n, kap, np.ones_like(kap), 2e-2, 1e3, 2e4)
    hb = h.copy()
    hb[0, 0, 9] *= 1.3
    assert head_normwise(hb, h) <= 2e-2  # the old h~ reading: accepted
    with pytest.raises(AssertionError):
        check(hb, m, n, h, m, n, kap, np.ones_like(kap), 2e-2, 1e3, 2e4)


def test_conditions_from_the_oracle_diagnostics():
    n = np.array([[[2.0, 0.5]]])
    h = np.array([[[[1.0, -3.0], [0.25, 0.5]]]])
    kap, kapn = conditions(n, h, rho=np.array([[[20.0, 0.5]]]), rho_num=np.array([[[60.0, 2.5]]]))
    assert np.allclose(kap, [[[10.0, 1.0]]])
    # numerators n h~: row 0 max |(2, -6)| = 6, row 1 max |(0.125, 0.25)| = 0.25
    assert np.allclose(kapn, [[[10.0, 10.0]]])


def test_numerator_bar_scales_with_its_condition_number():
    """A float32 row whose numerator cancels (kappa_num 1.7e4, the floor row
    of the recurrent stress case) may miss 1e-4 by its condition number; the
    same error on a well-conditioned row fails."""
    h, m, n, kap = _case(4)
    kn = np.ones_like(kap)
    kn[0, 1, 3] = 1.7e4
    hb = h.copy()
    hb[0, 1, 3] *= 1 + 3.5e-4  # numerator and h~ both off by 3.5e-4
    out = check(hb, m, n, h, m, n, kap, kn, 1e-4, 100.0, 100.0)
    assert out["rows_not_in_h_check"] == 1
    assert out["numerator_over_bar"] == pytest.approx(3.5e-4 / (1e-4 * 170), rel=1e-6)
    with pytest.raises(AssertionError):
        check(hb, m, n, h, m, n, kap, np.ones_like(kap), 1e-4, 100.0, 100.0)
