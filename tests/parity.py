"""Tolerance readings used by the GPU parity tests (test infrastructure).

Required bars: max relative error 1e-4 (float32 inputs) and 2e-2 (bf16 in,
float32 accumulate) for h~; 1e-5 relative for m and n.  "Relative" is read as
follows, because m crosses zero and single rows of n and h~ can be
cancellation-amplified (b_i is a signed sum, Eq. 83):

* m: elementwise |dm| / max(|m_ref|, 1) <= 1e-5.
* n: per head, max |dn| / max n_ref <= 1e-5 (normwise).
* h~: per head, max |dh| / max |h_ref| <= tol (normwise), tol 1e-4 / 2e-2.
  Rows whose cancellation factor kappa_i = sum_j |C~'_ij| / n_i exceeds
  ``kappa_max`` may be excluded from the h~ check; the numerator n_i h~_i =
  sum_j C~'_ij v_j is then checked on every row at the same tolerance.
"""
import numpy as np


def head_normwise(got, ref, axis_head=(0, 1)):
    """max over heads of max|got-ref| / max|ref| within the head."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    red = tuple(range(2, got.ndim))
    num = err.max(axis=red) if red else err
    den = np.abs(ref).max(axis=red) if red else np.abs(ref)
    return float((num / np.maximum(den, 1e-300)).max())


def m_error(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float((np.abs(got - ref) / np.maximum(np.abs(ref), 1.0)).max())


def check(h, m, n, h_ref, m_ref, n_ref, tol_h, tol_mn=1e-5, kappa=None, kappa_max=None):
    """Assert the readings above; returns a dict of the measured errors."""
    out = {"m": m_error(m, m_ref), "n": head_normwise(n, n_ref)}
    if kappa is not None and kappa_max is not None:
        keep = kappa <= kappa_max
        hh = np.where(keep[..., None], h, 0.0)
        hr = np.where(keep[..., None], h_ref, 0.0)
        out["h"] = head_normwise(hh, hr)
        num = np.asarray(h, np.float64) * np.asarray(n, np.float64)[..., None]
        num_ref = np.asarray(h_ref, np.float64) * np.asarray(n_ref, np.float64)[..., None]
        out["numerator"] = head_normwise(num, num_ref)
        out["excluded_rows"] = int((~keep).sum())
        assert out["numerator"] <= tol_h, out
    else:
        out["h"] = head_normwise(h, h_ref)
    assert out["m"] <= tol_mn, out
    assert out["n"] <= tol_mn, out
    assert out["h"] <= tol_h, out
    return out
