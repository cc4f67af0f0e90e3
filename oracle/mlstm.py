"""Plain, slow, obviously-correct CPU evaluation of the mLSTM forward pass.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the GPU
library imports or calls this module.

Source: "xLSTM: Extended Long Short-Term Memory", Appendix A.3.

* Eq. 71 forget gate matrix F, Eq. 72 input gate pre-activation matrix I~,
  Eq. 73 D = F (.) exp(I~), Eq. 76 unstabilized H~ = C V.
* Eqs. 74-75 and 77: stabilization by the row maximum of log D.
* Eqs. 79-86 (the stabilized forward pass restated at the start of "Parallel
  mLSTM Backward Pass"): D~ = logF + I~, m = row max, D' = exp(D~ - m 1^T),
  C~' = (Q K^T / sqrt(d)) (.) D', b = C~' 1, n = max(|b|, exp(-m)),
  C = C~' (.) (n^-1 1^T), H~ = C V.
* Eq. 101: log F_ij = -inf (i < j), 0 (i = j), sum_{k=j+1..i} log sigma(f~_k).
* Eq. 78: output gate H = sigma(O~) (.) H~.
* The recurrent form (C_t = f_t C_{t-1} + i_t v_t k_t^T, n_t = f_t n_{t-1} +
  i_t k_t, h~_t = C_t q_t / max(|n_t^T q_t|, 1)) is read off the recurrent
  backward pass, Eqs. 59-70, whose forward equations are cited but not shown
  on the page; the appendix extracts the 1/sqrt(d) of the keys explicitly in
  the parallel form, so the recurrent keys carry it (k_t / sqrt(d)), and the
  states start at zero.

Shapes: q, k, v are [B, NH, T, d]; igate (i~), fgate (f~) are [B, NH, T].
Heads are independent (the page on the xLSTM cell notes there is no memory
mixing between heads), so every function loops over (b, h) and works on one
head at a time, exactly as the appendix presents it.
"""

import math

import numpy as np


def log_sigmoid(x):
    """f-bar = log sigma(x) of Eq. 101, as min(x, 0) - log1p(exp(-|x|)).

    The rewrite is algebraically exact: log sigma(x) = -log(1 + e^-x) for
    x >= 0 and x - log(1 + e^x) for x < 0; it never forms e^{+|x|}.
    """
    x = np.asarray(x, dtype=np.float64)
    return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))


def _sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    # 1 / (1 + e^-x), evaluated without overflow for either sign.
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


FORGET_ACTIVATIONS = ("sigmoid", "exp")


def forget_gate(fgate, forget="sigmoid"):
    """The forget gate f_t from its pre-activation: sigma(f~) (Eq. 71's
    activation, the one the parallel form fixes) or exp(f~) (the other
    activation the pages allow for the forget gate)."""
    if forget == "sigmoid":
        return _sigmoid(fgate)
    if forget == "exp":
        return np.exp(np.asarray(fgate, dtype=np.float64))
    raise ValueError(f"unknown forget activation {forget!r}")


def log_forget(fgate, forget="sigmoid"):
    """f-bar = log f_t (Eq. 101): log sigma(f~), or f~ itself for exp."""
    if forget == "sigmoid":
        return log_sigmoid(fgate)
    if forget == "exp":
        return np.asarray(fgate, dtype=np.float64)
    raise ValueError(f"unknown forget activation {forget!r}")


def dlog_forget(fgate, forget="sigmoid"):
    """d f-bar / d f~: sigma(-f~) (Eq. 104) for sigmoid, 1 for exp."""
    if forget == "sigmoid":
        return _sigmoid(-np.asarray(fgate, dtype=np.float64))
    if forget == "exp":
        return np.ones_like(np.asarray(fgate, dtype=np.float64))
    raise ValueError(f"unknown forget activation {forget!r}")


def gate_matrices(fgate, igate, forget="sigmoid"):
    """F (Eq. 71) and I~ (Eq. 72) for ONE head, by their definitions.

    F_ij = 0 for i < j, 1 for i = j, prod_{k=j+1..i} sigma(f~_k) for i > j:
    every entry below the diagonal is the explicit product, formed as a
    running product down each column.  I~_ij = 0 for i < j, i~_j for i >= j.
    Returns (F, Itilde) as float64 [T, T].
    """
    f = np.asarray(fgate, dtype=np.float64).reshape(-1)
    ig = np.asarray(igate, dtype=np.float64).reshape(-1)
    T = f.shape[0]
    sig = forget_gate(f, forget)
    F = np.zeros((T, T), dtype=np.float64)
    for j in range(T):
        F[j, j] = 1.0
        prod = 1.0
        for i in range(j + 1, T):
            prod *= sig[i]
            F[i, j] = prod
    It = np.zeros((T, T), dtype=np.float64)
    for i in range(T):
        It[i, : i + 1] = ig[: i + 1]
    return F, It


def log_gate_matrix(fgate, igate, rows=None, dtype=np.float64, forget="sigmoid"):
    """D~ = log F + I~ (Eqs. 74, 79, with log F from Eq. 101) for ONE head.

    log F_ij is the sum of f-bar_k over k = j+1..i, written as the difference
    of the inclusive prefix sums cs_i - cs_j of f-bar; -inf above the diagonal.
    ``rows`` selects row indices (default: all).  Returns [len(rows), T].
    """
    fbar = log_forget(fgate, forget).astype(dtype)
    ig = np.asarray(igate, dtype=np.float64).reshape(-1).astype(dtype)
    T = fbar.shape[0]
    cs = np.cumsum(fbar, dtype=dtype)
    rows = np.arange(T) if rows is None else np.asarray(rows)
    Dt = cs[rows][:, None] - cs[None, :] + ig[None, :]
    upper = np.arange(T)[None, :] > rows[:, None]
    Dt[upper] = -np.inf
    # Eq. 101 fixes log F_ii = 0 exactly (cs_i - cs_i is already exactly 0).
    return Dt


def _rows_one_head(q, k, v, ig, fg, rows, dtype, forget="sigmoid"):
    """Eqs. 79-86 for the listed rows of one head.  Rows are independent."""
    T, d = q.shape
    rows = np.asarray(rows)
    ncol = int(rows.max()) + 1  # columns j > every listed row are exactly 0 (Eq. 71)
    Dt = log_gate_matrix(fg[:ncol], ig[:ncol], rows=rows, dtype=dtype, forget=forget)  # Eq. 79
    m = Dt.max(axis=1)  # Eq. 80, row-wise maximum
    Dp = np.exp(Dt - m[:, None])  # Eq. 81, exp(-inf) = 0 above the diagonal
    S = (q[rows].astype(dtype) @ k[:ncol].astype(dtype).T) / dtype(math.sqrt(d))
    Ct = S * Dp  # Eq. 82
    b = Ct.sum(axis=1)  # Eq. 83, row sum over j = 1..T
    n = np.maximum(np.abs(b), np.exp(-m))  # Eq. 84
    C = Ct / n[:, None]  # Eq. 85
    h = C @ v[:ncol].astype(dtype)  # Eq. 86
    # diagnostics, not part of the method: b_i is a sum over j and c of the
    # products D'_ij q_ic k_jc / sqrt(d); rho_i sums their magnitudes.  Each
    # numerator n_i h~_ic = sum_j C~'_ij v_jc is a sum over j and c' of
    # D'_ij q_ic' k_jc' v_jc / sqrt(d); rho_num_i is the largest over c of the
    # sums of their magnitudes.
    Sabs = (np.abs(q[rows]).astype(dtype) @ np.abs(k[:ncol]).astype(dtype).T) / dtype(math.sqrt(d))
    rho = (Sabs * Dp).sum(axis=1)
    rho_num = ((Sabs * Dp) @ np.abs(v[:ncol]).astype(dtype)).max(axis=1)
    return h, m, n, b, rho, rho_num


def forward_stabilized(q, k, v, igate, fgate, block_rows=256, dtype=np.float64,
                       return_diag=False, forget="sigmoid"):
    """Stabilized parallel forward pass, Eqs. 79-86, densely, per head.

    Rows are processed in blocks of ``block_rows`` only to bound memory; each
    row's arithmetic is independent of every other row's.
    Returns (h [B,NH,T,d], m [B,NH,T], n [B,NH,T]); with ``return_diag`` also
    (b, rho) where b is the signed row sum (Eq. 83) and
    rho_i = sum_j D'_ij sum_c |q_ic k_jc| / sqrt(d), the sum of the magnitudes
    of all the products whose signed sum is b_i, so that rho / n is the
    condition number of n_i: a relative error eps in every product moves n_i
    by at most eps * rho_i / n_i relative to n_i.  Last, rho_num
    [B,NH,T]: max over c of sum_j D'_ij (sum_c' |q_ic' k_jc'|) |v_jc| / sqrt(d),
    the same for the numerators n_i h~_ic (its ratio to max_c |n_i h~_ic| is
    the condition number of the row's numerator).
    """
    q = np.asarray(q)
    B, NH, T, d = q.shape
    h = np.empty((B, NH, T, d), dtype=dtype)
    m = np.empty((B, NH, T), dtype=dtype)
    n = np.empty((B, NH, T), dtype=dtype)
    bsum = np.empty((B, NH, T), dtype=dtype)
    rho = np.empty((B, NH, T), dtype=dtype)
    rho_num = np.empty((B, NH, T), dtype=dtype)
    for bi in range(B):
        for hi in range(NH):
            qh, kh, vh = (np.asarray(a[bi, hi], dtype=np.float64) for a in (q, k, v))
            ig = np.asarray(igate[bi, hi], dtype=np.float64)
            fg = np.asarray(fgate[bi, hi], dtype=np.float64)
            for r0 in range(0, T, block_rows):
                rows = np.arange(r0, min(T, r0 + block_rows))
                hh, mm, nn, bb, rr, rn = _rows_one_head(qh, kh, vh, ig, fg, rows, dtype, forget)
                h[bi, hi, rows] = hh
                m[bi, hi, rows] = mm
                n[bi, hi, rows] = nn
                bsum[bi, hi, rows] = bb
                rho[bi, hi, rows] = rr
                rho_num[bi, hi, rows] = rn
    if return_diag:
        return h, m, n, bsum, rho, rho_num
    return h, m, n


def forward_rows(q, k, v, igate, fgate, bi, hi, rows, dtype=np.float64, forget="sigmoid"):
    """Eqs. 79-86 for selected rows ``rows`` of head (bi, hi) only.

    Costs O(len(rows) * max(rows) * d): used to check single outputs of very
    long sequences one by one.  Returns (h [R, d], m [R], n [R], b [R], rho [R],
    rho_num [R]) (the diagnostics of ``forward_stabilized``).
    """
    qh, kh, vh = (np.asarray(a[bi, hi], dtype=np.float64) for a in (q, k, v))
    ig = np.asarray(igate[bi, hi], dtype=np.float64)
    fg = np.asarray(fgate[bi, hi], dtype=np.float64)
    return _rows_one_head(qh, kh, vh, ig, fg, np.asarray(rows), dtype, forget)


def forward_recurrent(q, k, v, igate, fgate, forget="sigmoid"):
    """The recurrent mLSTM, step by step, unstabilized, in float64.

    C_0 = 0 (d x d), n_0 = 0 (d); for t = 1..T: f_t = sigma(f~_t),
    i_t = exp(i~_t), k'_t = k_t / sqrt(d); C_t = f_t C_{t-1} + i_t v_t k'_t^T;
    n_t = f_t n_{t-1} + i_t k'_t; h~_t = C_t q_t / max(|n_t^T q_t|, 1).
    Returns (h [B,NH,T,d], nq [B,NH,T]) with nq_t = n_t^T q_t, the recurrent
    normalizer argument.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, NH, T, d = q.shape
    h = np.empty((B, NH, T, d))
    nq = np.empty((B, NH, T))
    scale = 1.0 / math.sqrt(d)
    for bi in range(B):
        for hi in range(NH):
            C = np.zeros((d, d))
            nvec = np.zeros(d)
            for t in range(T):
                f_t = float(forget_gate(fgate[bi, hi, t], forget))
                i_t = math.exp(float(igate[bi, hi, t]))
                kt = k[bi, hi, t] * scale
                vt = v[bi, hi, t]
                C = f_t * C + i_t * np.outer(vt, kt)
                nvec = f_t * nvec + i_t * kt
                qt = q[bi, hi, t]
                den = float(nvec @ qt)
                nq[bi, hi, t] = den
                h[bi, hi, t] = (C @ qt) / max(abs(den), 1.0)
    return h, nq


def recurrent_step_stabilized(q_t, k_t, v_t, ig_t, fg_t, C, nvec, m, forget="sigmoid"):
    """One step of the recurrent mLSTM for ONE head with stabilized states,
    float64.

    The pages stabilize the recurrent mLSTM as the sLSTM (its Eq. 15 is not on
    the pages); the reading used here is the plainest one consistent with the
    parallel form: the stabilizer is the running maximum of the log gates,
        m_t = max(fbar_t + m_{t-1}, i~_t),   m_0 = -inf,
    which is the row maximum m of Eq. 80 (split j = t from j < t), and the
    states are the unstabilized ones of the recurrent form scaled by
    exp(-m_t):
        f'_t = exp(fbar_t + m_{t-1} - m_t),   i'_t = exp(i~_t - m_t),
        C_t = f'_t C_{t-1} + i'_t v_t k'_t^T,  n_t = f'_t n_{t-1} + i'_t k'_t,
    with k'_t = k_t / sqrt(d).  Dividing C_t q_t by max(|n_t . q_t|, 1) in the
    unstabilized scale is then dividing by max(|n_t . q_t|, exp(-m_t)) here,
    the normalizer of Eq. 84.

    Inputs: vectors q_t, k_t, v_t (d), scalars ig_t (i~), fg_t (f~), state
    C (d x d, rows indexed by the value dimension), nvec (d), m (scalar;
    -inf for a fresh state).  Returns (h_t, C_t, n_t, m_t, den_t).
    """
    q_t = np.asarray(q_t, dtype=np.float64)
    k_t = np.asarray(k_t, dtype=np.float64)
    v_t = np.asarray(v_t, dtype=np.float64)
    d = q_t.shape[0]
    fbar = float(log_forget(fg_t, forget))
    ig = float(ig_t)
    m_new = max(fbar + m, ig)
    f_p = math.exp(fbar + m - m_new) if m != -math.inf else 0.0
    i_p = math.exp(ig - m_new)
    kp = k_t / math.sqrt(d)
    C_new = f_p * np.asarray(C, dtype=np.float64) + i_p * np.outer(v_t, kp)
    n_new = f_p * np.asarray(nvec, dtype=np.float64) + i_p * kp
    den = max(abs(float(n_new @ q_t)), math.exp(-m_new))
    h = (C_new @ q_t) / den
    return h, C_new, n_new, m_new, den


def forward_recurrent_stabilized(q, k, v, igate, fgate, forget="sigmoid"):
    """``recurrent_step_stabilized`` from a fresh state (C = 0, n = 0,
    m = -inf) over every position of every head.

    Returns (h [B,NH,T,d], m [B,NH,T], den [B,NH,T], C_T [B,NH,d,d],
    n_T [B,NH,d]).
    """
    q = np.asarray(q, dtype=np.float64)
    B, NH, T, d = q.shape
    h = np.empty((B, NH, T, d))
    mm = np.empty((B, NH, T))
    den = np.empty((B, NH, T))
    CT = np.empty((B, NH, d, d))
    nT = np.empty((B, NH, d))
    for bi in range(B):
        for hi in range(NH):
            C = np.zeros((d, d))
            nvec = np.zeros(d)
            m = -math.inf
            for t in range(T):
                h[bi, hi, t], C, nvec, m, den[bi, hi, t] = recurrent_step_stabilized(
                    q[bi, hi, t], k[bi, hi, t], v[bi, hi, t], igate[bi, hi, t], fgate[bi, hi, t],
                    C, nvec, m, forget)
                mm[bi, hi, t] = m
            CT[bi, hi], nT[bi, hi] = C, nvec
    return h, mm, den, CT, nT


def forward_unstabilized(q, k, v, igate, fgate, forget="sigmoid"):
    """Unstabilized parallel form, Eqs. 71-73 and 76, by brute force.

    D = F (.) exp(I~) with F built from explicit products (``gate_matrices``);
    C~ = (Q K^T / sqrt(d)) (.) D; H~ = C~ V / max(|C~ 1|, 1).  Overflows for
    large input gates, which is what the stabilization exists to avoid.
    Returns h [B,NH,T,d].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, NH, T, d = q.shape
    h = np.empty((B, NH, T, d))
    for bi in range(B):
        for hi in range(NH):
            F, It = gate_matrices(fgate[bi, hi], igate[bi, hi], forget)
            D = F * np.exp(It)  # Eq. 73
            Ct = (q[bi, hi] @ k[bi, hi].T) / math.sqrt(d) * D
            den = np.maximum(np.abs(Ct.sum(axis=1)), 1.0)
            h[bi, hi] = (Ct / den[:, None]) @ v[bi, hi]
    return h


def backward_stabilized(q, k, v, igate, fgate, dh, forget="sigmoid"):
    """Gradients of the stabilized parallel forward pass (Eqs. 87-105) for
    every head, float64, dense T x T per head.

    Given dh = dL/dH~ ([B,NH,T,d]), returns (dq, dk, dv [B,NH,T,d],
    digate, dfgate [B,NH,T]).  The forward quantities (D', C~', b, n, m) are
    recomputed from the inputs exactly as in ``forward_stabilized``.  m is held
    constant: its contributions cancel (H~ does not depend on the stabilizer).

    Reading of Eq. 90: the page writes sign(n), but n = max(|b|, exp(-m)) is
    positive; the derivative of |b| is sign(b), which is what is used here.
    Eq. 102 is evaluated literally as the double sum over j < k <= i.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dh = np.asarray(dh, dtype=np.float64)
    B, NH, T, d = q.shape
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    di = np.empty((B, NH, T))
    df = np.empty((B, NH, T))
    rs = 1.0 / math.sqrt(d)
    for bi in range(B):
        for hi in range(NH):
            Dt = log_gate_matrix(fgate[bi, hi], igate[bi, hi], forget=forget)  # Eq. 79
            m = Dt.max(axis=1)                                             # Eq. 80
            Dp = np.exp(Dt - m[:, None])                                   # Eq. 81
            S = (q[bi, hi] @ k[bi, hi].T) * rs
            Ct = S * Dp                                                    # Eq. 82
            b = Ct.sum(axis=1)                                             # Eq. 83
            n = np.maximum(np.abs(b), np.exp(-m))                          # Eq. 84
            Cn = Ct / n[:, None]                                           # Eq. 85
            dC = dh[bi, hi] @ v[bi, hi].T                                  # Eq. 87 (dC, T x T)
            dn = -((Ct * dC).sum(axis=1)) / n ** 2                         # Eqs. 88-89
            db = np.sign(b) * dn * (np.abs(b) > np.exp(-m))                # Eq. 90 (sign(b))
            dCt = dC / n[:, None] + db[:, None]                            # Eqs. 91-93
            dDp = S * dCt                                                  # Eq. 94
            dDt = Dp * dDp                                                 # Eq. 95
            P = Dp * dCt
            dq[bi, hi] = (P @ k[bi, hi]) * rs                              # Eq. 98
            dk[bi, hi] = (P.T @ q[bi, hi]) * rs                            # Eq. 99
            dv[bi, hi] = Cn.T @ dh[bi, hi]                                 # Eq. 100
            # Eqs. 96-97: dFbar = dI = dD~ (zero above the diagonal, where
            # D' = 0); Eq. 105: column sums; Eq. 102: double sum
            di[bi, hi] = dDt.sum(axis=0)
            dfbar = np.zeros(T)
            for kk in range(T):
                dfbar[kk] = dDt[kk:, :kk].sum()
            fg = np.asarray(fgate[bi, hi], dtype=np.float64)
            df[bi, hi] = dlog_forget(fg, forget) * dfbar                   # Eqs. 103-104
    return dq, dk, dv, di, df


def output_gate(h, ogate):
    """Eq. 78: H = sigma(O~) (.) H~, elementwise."""
    return _sigmoid(ogate) * np.asarray(h, dtype=np.float64)
