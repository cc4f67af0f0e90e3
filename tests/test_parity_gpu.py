"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every input is drawn by ``workloads.make`` and handed, identically, to the
GPU library and to ``oracle``.  Tolerances are the readings in
``tests/parity.py``.  Shapes span several 128-row and 32-key tiles with ragged
tails; the named workloads run at full size, where the oracle recomputes a
sample of rows one by one.
"""
import numpy as np
import pytest

import oracle
from linear_recurrent_sequence_amd import workloads as W
from parity import K_H, K_N, K_NUM, b_over_bar, check, conditions, head_normwise, m_error, row_relative

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from linear_recurrent_sequence_amd import mlstm

TOL_H = {"fp32": 1e-4, "bf16": 2e-2}


def _dev(x):
    spec = x["spec"]
    dt = torch.bfloat16 if spec["dtype"] == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x[n]).to("cuda").to(dt).contiguous() for n in ("q", "k", "v"))
    ig = torch.from_numpy(x["igate"]).to("cuda").contiguous()
    fg = torch.from_numpy(x["fgate"]).to("cuda").contiguous()
    return q, k, v, ig, fg


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


def run_gpu(x, kernel="auto"):
    """mlstm_parallel_fwd (kernel "auto"), or the two stages with the given
    tile kernel ("auto_staged": the two stages with the kernel auto picks)"""
    q, k, v, ig, fg = _dev(x)
    if kernel == "auto":
        h, m, n = mlstm.parallel_fwd(q, k, v, ig, fg)
    else:
        h, m, n = mlstm.parallel_fwd_staged(q, k, v, ig, fg,
                                            kernel="auto" if kernel == "auto_staged" else kernel)
    torch.cuda.synchronize()
    return _host(h), _host(m), _host(n)


def oracle_full(x, forget="sigmoid"):
    """(h, m, n, b, rho, rho_num) of the oracle on every row; rho and rho_num
    give each row's condition numbers (tests/parity.py)."""
    return oracle.forward_stabilized(x["q"], x["k"], x["v"], x["igate"], x["fgate"],
                                     return_diag=True, forget=forget)


def check_full(h, m, n, x, dtype, tol_h=None, forget="sigmoid", h_ref=None):
    """The readings of tests/parity.py on every row against the oracle
    (h_ref replaces the oracle's h~, e.g. by its output-gated value)."""
    hr, mr, nr, _, rho, rho_num = oracle_full(x, forget)
    kap, kapn = conditions(nr, hr, rho, rho_num)
    out = check(h, m, n, hr if h_ref is None else h_ref, mr, nr, kap, kapn,
                TOL_H[dtype] if tol_h is None else tol_h, K_H[dtype], K_NUM[dtype])
    print(out)
    return out


def m_every_position(x, forget="sigmoid"):
    """m_i = max_j D~_ij (Eq. 80) at every position, from the oracle's D~
    taken in blocks of rows."""
    B, NH, T = x["igate"].shape
    M = np.empty((B, NH, T))
    for b in range(B):
        for hh in range(NH):
            for r0 in range(0, T, 1024):
                rows = np.arange(r0, min(T, r0 + 1024))
                M[b, hh, rows] = oracle.log_gate_matrix(x["fgate"][b, hh], x["igate"][b, hh],
                                                        rows=rows, forget=forget).max(axis=1)
    return M


def spec(B, NH, T, d, dtype="bf16", ig=("normal", 0.0, 1.0), fg=("normal", 3.0, 1.0), **kw):
    s = dict(B=B, NH=NH, T=T, d=d, dtype=dtype, igate=ig, fgate=fg)
    s.update(kw)
    return s


# ---------------------------------------------------------------------------
# full comparison at sizes the oracle finishes in seconds
# ---------------------------------------------------------------------------

RAGGED = [
    spec(1, 1, 1, 16), spec(1, 1, 2, 16), spec(1, 2, 63, 48), spec(1, 1, 65, 80),
    spec(2, 3, 300, 64, ig=("normal", 0, 2), fg=("normal", 3, 1.5)),
    spec(1, 2, 257, 128), spec(2, 1, 129, 96), spec(1, 1, 200, 256),
    spec(1, 1, 160, 384), spec(1, 1, 140, 512), spec(1, 3, 384, 32),
    spec(1, 1, 333, 160, ig=("uniform", -20, 20), fg=("normal", 0, 4), fgate_floor=(0.01, -30.0)),
    spec(8, 1, 130, 64),  # head count divisible by 8 (XCD-grouped schedule)
]


def _id(s):
    return f"{s['B']}x{s['NH']}x{s['T']}x{s['d']}-{s['dtype']}"


@pytest.mark.parametrize("s", RAGGED, ids=_id)
def test_bf16_ragged_full(s):
    x = W.make(s, seed=1)
    h, m, n = run_gpu(x)
    check_full(h, m, n, x, "bf16")


@pytest.mark.parametrize("s", [spec(1, 2, 100, 32, "fp32"), spec(2, 1, 77, 512, "fp32"),
                               spec(1, 1, 1, 16, "fp32"), spec(1, 1, 300, 64, "fp32")], ids=_id)
def test_fp32_ragged_full(s):
    x = W.make(s, seed=2)
    h, m, n = run_gpu(x)
    check_full(h, m, n, x, "fp32")


F32_MFMA_CASES = [
    spec(1, 1, 4, 32, "fp32"), spec(1, 2, 129, 96, "fp32"), spec(2, 1, 260, 192, "fp32"),
    spec(1, 1, 200, 256, "fp32"), spec(1, 1, 161, 320, "fp32"), spec(1, 2, 140, 384, "fp32"),
    spec(1, 1, 150, 512, "fp32"),
    spec(1, 2, 500, 64, "fp32", ig=("uniform", -20, 20), fg=("normal", 0, 4),
         fgate_floor=(0.01, -30.0)),
    spec(1, 1, 333, 128, "fp32", ig=("uniform", -40, 40), fg=("normal", -2, 3)),
    spec(8, 1, 100, 32, "fp32"),  # head count divisible by 8 (XCD-grouped schedule)
]


@pytest.mark.parametrize("s", F32_MFMA_CASES, ids=_id)
def test_fp32_matrix_core_kernel_full(s):
    """Float32 inputs with d a multiple of 32 up to 256 (and 320, 384, 512,
    where two or four workgroups per row block split the columns) run on the
    float32 matrix instruction: against the oracle on every row (ragged
    tails, several row tiles, tiles skipped under strong decay), and against
    the float32 vector kernel (the same exponents, other summation orders)."""
    x = W.make(s, seed=3)
    h, m, n = run_gpu(x)
    check_full(h, m, n, x, "fp32")
    hv, mv, nv = run_gpu(x, kernel="vector")
    assert np.array_equal(m, mv)
    # both within their bars of the oracle, so within twice the bar of each
    # other, on the rows where those bars are the flat ones
    hr, _, nr, _, rho, rho_num = oracle_full(x)
    kap, kapn = conditions(nr, hr, rho, rho_num)
    well = kap <= K_N
    assert (np.abs(n - nv) / nv)[well].max() <= 2e-5
    keep = (kap <= K_H["fp32"]) & (kapn <= K_NUM["fp32"])
    assert row_relative(h, hv)[keep].max() <= 2 * TOL_H["fp32"]


def test_fp32_matrix_core_kernel_epilogues():
    """Output gate, stored h~ and b through the float32 matrix-core kernel
    (Eqs. 78, 83), at a head dim that splits the columns."""
    s = spec(1, 2, 150, 384, "fp32")
    x = W.make(s, seed=4)
    q, k, v, ig, fg = _dev(x)
    og = torch.from_numpy(np.random.default_rng(5).standard_normal(
        x["q"].shape).astype(np.float32)).to("cuda")
    hg, ht, m, n = mlstm.parallel_fwd_gated(q, k, v, ig, fg, og, htilde=True)
    h0, m0, n0 = mlstm.parallel_fwd(q, k, v, ig, fg)
    h2, m2, n2, b2 = mlstm.parallel_fwd_train(q, k, v, ig, fg)
    torch.cuda.synchronize()
    assert torch.equal(ht, h0) and torch.equal(n, n0) and torch.equal(h2, h0)
    hr, mr, nr, br, rho, rho_num = oracle_full(x)
    kap, kapn = conditions(nr, hr, rho, rho_num)
    gate = 1.0 / (1.0 + np.exp(-_host(og)))
    check(_host(hg), _host(m), _host(n), hr * gate, mr, nr, kap, kapn, TOL_H["fp32"],
          K_H["fp32"], K_NUM["fp32"])
    assert b_over_bar(_host(b2), br, nr, kap) <= 1.0


def test_fp32_matrix_core_kernel_exp_forget():
    s = spec(1, 2, 257, 128, "fp32", fg=("normal", -0.05, 0.03))
    x = W.make(s, seed=6)
    q, k, v, ig, fg = _dev(x)
    h, m, n, b = mlstm.parallel_fwd_train(q, k, v, ig, fg, forget="exp")
    torch.cuda.synchronize()
    check_full(_host(h), _host(m), _host(n), x, "fp32", forget="exp")


def test_tiny_fp32_workload():
    x = W.make("tiny_fp32", seed=0)
    h, m, n = run_gpu(x)
    check_full(h, m, n, x, "fp32")
    # the recurrent form agrees too (the oracle is pinned to it), row by row
    hrec, _ = oracle.forward_recurrent(x["q"], x["k"], x["v"], x["igate"], x["fgate"])
    hr, _, nr, _, rho, rho_num = oracle_full(x)
    kap, kapn = conditions(nr, hr, rho, rho_num)
    keep = (kap <= K_H["fp32"]) & (kapn <= K_NUM["fp32"])
    assert row_relative(h, hrec)[keep].max() <= TOL_H["fp32"]


@pytest.mark.parametrize("name", ["tiny_fp32", "small_bf16"])
def test_plain_entry_point_on_the_null_stream(name):
    """mlstm_parallel_fwd itself (no stream argument: the null stream) through
    the C ABI: against the oracle, and bitwise equal to the stream variant."""
    x = W.make(name, seed=0)
    q, k, v, ig, fg = _dev(x)
    B, NH, T, d = q.shape
    h = torch.empty_like(q)
    m = torch.empty((B, NH, T), dtype=torch.float32, device=q.device)
    n = torch.empty_like(m)
    lib = mlstm.load_library()
    torch.cuda.synchronize()  # the inputs are in place before the null-stream call
    st = lib.mlstm_parallel_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), ig.data_ptr(),
                                fg.data_ptr(), h.data_ptr(), m.data_ptr(), n.data_ptr(),
                                B, NH, T, d, mlstm._dtype_code(q))
    assert st == 0, mlstm.strerror(st)
    torch.cuda.synchronize()
    h2, m2, n2 = mlstm.parallel_fwd(q, k, v, ig, fg)
    torch.cuda.synchronize()
    assert torch.equal(h, h2) and torch.equal(m, m2) and torch.equal(n, n2)
    check_full(_host(h), _host(m), _host(n), x, x["spec"]["dtype"])


def test_small_bf16_workload():
    x = W.make("small_bf16", seed=0)
    h, m, n = run_gpu(x)
    check_full(h, m, n, x, "bf16")


@pytest.mark.parametrize("s", [spec(1, 2, 257, 128), spec(1, 1, 150, 384),
                               spec(1, 1, 200, 64, ig=("uniform", -20, 20), fg=("normal", 0, 4))],
                         ids=_id)
def test_vector_kernel_bf16_inputs(s):
    """The float32 vector kernel on bf16 inputs never rounds C~' to bf16: its
    only bf16 rounding is that of the stored h~ (half an ulp, 2^-8 relative),
    so it meets a 4e-3 bar on h~ and the float32 bars on m and n.  An
    independent GPU evaluation of the same pass."""
    x = W.make(s, seed=3)
    h, m, n = run_gpu(x, kernel="vector")
    check_full(h, m, n, x, "bf16", tol_h=4e-3)


def test_gate_scan_m_matches_oracle():
    x = W.make(spec(2, 3, 1000, 64, ig=("uniform", -20, 20), fg=("normal", 0, 4),
                    fgate_floor=(0.01, -30.0)), seed=4)
    q, k, v, ig, fg = _dev(x)
    ws = mlstm.alloc_workspace(2, 3, 1000, "cuda")
    m = _host(mlstm.gate_scan(ig, fg, 64, ws))
    assert m_error(m, m_every_position(x)) <= 1e-5


# ---------------------------------------------------------------------------
# full-size workloads: sampled rows recomputed by the oracle one by one
# ---------------------------------------------------------------------------

def _sample_rows(T, rng, count=40):
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 129, 255, 256, T // 2, T - 129, T - 128, T - 33,
             T - 32, T - 2, T - 1]
    rows = set(r for r in fixed if 0 <= r < T)
    rows.update(int(r) for r in rng.integers(0, T, size=count))
    return np.array(sorted(rows))


def _sampled_reference(x, rows):
    B, NH = x["spec"]["B"], x["spec"]["NH"]
    d = x["spec"]["d"]
    H = np.empty((B, NH, len(rows), d))
    M = np.empty((B, NH, len(rows)))
    N = np.empty((B, NH, len(rows)))
    R = np.empty((B, NH, len(rows)))
    RN = np.empty((B, NH, len(rows)))
    for b in range(B):
        for hh in range(NH):
            h, m, n, bb, rho, rho_num = oracle.forward_rows(x["q"], x["k"], x["v"], x["igate"],
                                                            x["fgate"], b, hh, rows)
            H[b, hh], M[b, hh], N[b, hh], R[b, hh], RN[b, hh] = h, m, n, rho, rho_num
    return H, M, N, R, RN


def _check_sampled(h, m, n, x, rows, seed_label, h_ref=None):
    """h~ and n on the sampled rows, m at every position."""
    hr, mr, nr, rho, rho_num = _sampled_reference(x, rows)
    assert m_error(m, m_every_position(x)) <= 1e-5
    kap, kapn = conditions(nr, hr, rho, rho_num)
    out = check(h[:, :, rows], m[:, :, rows], n[:, :, rows], hr if h_ref is None else h_ref, mr,
                nr, kap, kapn, TOL_H["bf16"], K_H["bf16"], K_NUM["bf16"])
    print(seed_label, out)
    assert np.isfinite(h).all() and np.isfinite(n).all() and np.isfinite(m).all()
    return out


@pytest.mark.parametrize("name", ["xlstm125m_layer", "xlstm1p3b_layer"])
def test_language_model_workloads_sampled(name):
    x = W.make(name, seed=0)
    h, m, n = run_gpu(x)
    rows = _sample_rows(x["spec"]["T"], np.random.default_rng(5))
    _check_sampled(h, m, n, x, rows, name)


def test_long_context_workload_sampled():
    x = W.make("long_context_16k", seed=0)
    h, m, n = run_gpu(x)
    rows = _sample_rows(x["spec"]["T"], np.random.default_rng(6), count=30)
    _check_sampled(h, m, n, x, rows, "long_context_16k")


# ---------------------------------------------------------------------------
# properties that hold at any size
# ---------------------------------------------------------------------------

def test_deterministic_bitwise():
    x = W.make(spec(2, 2, 700, 128), seed=7)
    q, k, v, ig, fg = _dev(x)
    a = mlstm.parallel_fwd(q, k, v, ig, fg)
    b = mlstm.parallel_fwd(q, k, v, ig, fg)
    torch.cuda.synchronize()
    for ta, tb in zip(a, b):
        assert torch.equal(ta, tb)


@pytest.mark.parametrize("kernel", ["auto", "vector"])
def test_causality_bitwise(kernel):
    """Changing any input after position t0 leaves every output at <= t0 unchanged."""
    x = W.make(spec(1, 2, 400, 64), seed=8)
    t0 = 201
    y = {k_: (v_.copy() if isinstance(v_, np.ndarray) else v_) for k_, v_ in x.items()}
    rng = np.random.default_rng(9)
    for key in ("q", "k", "v"):
        y[key][:, :, t0 + 1:] = W.round_bf16(rng.standard_normal(y[key][:, :, t0 + 1:].shape)
                                             .astype(np.float32))
    for key in ("igate", "fgate"):
        y[key][:, :, t0 + 1:] = rng.normal(0, 3, y[key][:, :, t0 + 1:].shape).astype(np.float32)
    a = run_gpu(x, kernel)
    b = run_gpu(y, kernel)
    for ta, tb in zip(a, b):
        assert np.array_equal(ta[:, :, :t0 + 1], tb[:, :, :t0 + 1])


def test_head_permutation_bitwise():
    x = W.make(spec(2, 4, 260, 64), seed=10)
    perm = np.random.default_rng(11).permutation(8)
    y = dict(x)
    for key in ("q", "k", "v", "igate", "fgate"):
        a = x[key].reshape((8,) + x[key].shape[2:])[perm]
        y[key] = np.ascontiguousarray(a.reshape(x[key].shape))
    a = run_gpu(x)
    b = run_gpu(y)
    for ta, tb in zip(a, b):
        fa = ta.reshape((8,) + ta.shape[2:])
        fb = tb.reshape((8,) + tb.shape[2:])
        assert np.array_equal(fa[perm], fb)


def test_errors_raise_on_gpu():
    x = W.make(spec(1, 1, 64, 16), seed=0)
    q, k, v, ig, fg = _dev(x)
    with pytest.raises(ValueError):
        mlstm.parallel_fwd(q, k, v, ig[..., :10].contiguous(), fg)
    with pytest.raises(mlstm.MlstmError) as e:
        bad = torch.zeros((1, 1, 64, 24), dtype=torch.bfloat16, device="cuda")
        mlstm.parallel_fwd(bad, bad, bad, ig, fg)
    assert e.value.status == -4
    with pytest.raises(mlstm.MlstmError) as e:
        z = torch.zeros((1, 1, 0, 16), dtype=torch.bfloat16, device="cuda")
        g = torch.zeros((1, 1, 0), dtype=torch.float32, device="cuda")
        mlstm.parallel_fwd(z, z, z, g, g)
    assert e.value.status == -2


# ---------------------------------------------------------------------------
# output gate fused into the epilogue (Eq. 78)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("s", [spec(1, 2, 257, 128), spec(2, 1, 160, 384), spec(1, 1, 140, 512),
                               spec(1, 2, 100, 48), spec(1, 2, 130, 64, "fp32")], ids=_id)
def test_output_gate_fused(s):
    """h = sigmoid(O~) * h~ against the oracle's Eq. 78 on its h~; the h~ the
    gated call stores is bitwise the ungated call's h."""
    x = W.make(s, seed=12)
    og = W.make_ogate(x["spec"], seed=12)
    q, k, v, ig, fg = _dev(x)
    dt = q.dtype
    o_dev = torch.from_numpy(og).to("cuda").to(dt).contiguous()
    h, ht, m, n = mlstm.parallel_fwd_gated(q, k, v, ig, fg, o_dev, htilde=True)
    h0, m0, n0 = mlstm.parallel_fwd(q, k, v, ig, fg)
    h2, m2, n2 = mlstm.parallel_fwd_gated(q, k, v, ig, fg, o_dev)
    torch.cuda.synchronize()
    assert torch.equal(ht, h0) and torch.equal(m, m0) and torch.equal(n, n0)
    assert torch.equal(h, h2) and torch.equal(m2, m0) and torch.equal(n2, n0)
    hr = oracle_full(x)[0]
    check_full(_host(h), _host(m), _host(n), x, s["dtype"], h_ref=oracle.output_gate(hr, og))


def test_output_gate_language_model_sampled():
    x = W.make("xlstm125m_layer", seed=0)
    og = W.make_ogate(x["spec"], seed=0)
    q, k, v, ig, fg = _dev(x)
    o_dev = torch.from_numpy(og).to("cuda").to(torch.bfloat16).contiguous()
    h, m, n = mlstm.parallel_fwd_gated(q, k, v, ig, fg, o_dev)
    torch.cuda.synchronize()
    h, m, n = _host(h), _host(m), _host(n)
    rows = _sample_rows(x["spec"]["T"], np.random.default_rng(13), count=20)
    hr = _sampled_reference(x, rows)[0]
    _check_sampled(h, m, n, x, rows, "gated", h_ref=oracle.output_gate(hr, og[:, :, rows]))


# ---------------------------------------------------------------------------
# decay-aware tile skipping: identical results to visiting every causal tile
# ---------------------------------------------------------------------------

def _staged(x, kernel):
    q, k, v, ig, fg = _dev(x)
    h, m, n = mlstm.parallel_fwd_staged(q, k, v, ig, fg, kernel=kernel)
    torch.cuda.synchronize()
    return h, m, n


@pytest.mark.parametrize("s", [
    spec(1, 4, 3000, 64, ig=("uniform", -20, 20), fg=("normal", 0, 4), fgate_floor=(0.01, -30.0)),
    spec(2, 2, 1500, 128, ig=("uniform", -40, 40), fg=("normal", -2, 3)),
    spec(1, 2, 2100, 256, ig=("normal", 0, 1), fg=("normal", -4, 1)),
    spec(1, 1, 700, 384),  # slow decay: nothing to skip
], ids=_id)
def test_tile_skipping_matches_all_tiles_and_oracle(s):
    x = W.make(s, seed=14)
    a = _staged(x, "mfma")
    b = _staged(x, "mfma_all_tiles")
    for ta, tb in zip(a, b):
        assert torch.equal(ta, tb)  # equal values (an exact zero may differ in sign)
    check_full(_host(a[0]), _host(a[1]), _host(a[2]), x, "bf16")


@pytest.mark.parametrize("s", [
    spec(1, 2, 1500, 512, ig=("uniform", -40, 40), fg=("normal", -2, 3)),
    spec(1, 1, 1000, 448, ig=("uniform", -20, 20), fg=("normal", 0, 4), fgate_floor=(0.01, -30.0)),
    spec(2, 1, 333, 400, ig=("normal", 0, 2), fg=("normal", 0, 2)),
], ids=_id)
def test_single_wave_kernel_skipping_matches_all_tiles_and_oracle(s):
    """Above d = 384 the one-wave-per-SIMD kernel runs.  Its first product
    carries the next tile's copies, so it runs on every tile of the loop, also
    where a wave skips the tile: skipping must still give the values of
    visiting every tile, and both must pass the oracle's readings (ragged
    tails, padded head dimensions, decay strong enough to skip tiles)."""
    x = W.make(s, seed=15)
    a = _staged(x, "mfma")
    b = _staged(x, "mfma_all_tiles")
    for ta, tb in zip(a, b):
        assert torch.equal(ta, tb)
    check_full(_host(a[0]), _host(a[1]), _host(a[2]), x, "bf16")


@pytest.mark.parametrize("s", [
    spec(1, 2, 700, 64, ig=("uniform", -20, 20), fg=("normal", 0, 4), fgate_floor=(0.01, -30.0)),
    spec(2, 1, 333, 208),
    spec(1, 1, 97, 16),
    spec(1, 1, 260, 32, ig=("normal", 0, 2), fg=("normal", 3, 1.5)),
], ids=_id)
def test_single_wave_kernel_at_small_head_dims(s):
    """The one-wave-per-SIMD kernel selected explicitly at small head
    dimensions (1 to 13 chunks of 16 bytes per row, so that a row copy leaves
    most lanes idle) against the oracle."""
    x = W.make(s, seed=16)
    h, m, n = _staged(x, "mfma_single")
    check_full(_host(h), _host(m), _host(n), x, "bf16")


FUSED_CASES = [
    spec(1, 1, 4, 16), spec(1, 2, 64, 48), spec(1, 1, 68, 80), spec(2, 1, 132, 96),
    spec(2, 3, 300, 64, ig=("normal", 0, 2), fg=("normal", 3, 1.5)), spec(1, 2, 260, 128),
    spec(1, 1, 2044, 192), spec(1, 2, 2048, 256), spec(1, 1, 1000, 320), spec(2, 2, 2048, 384),
    spec(1, 1, 1, 16), spec(1, 2, 63, 48),  # lengths not divisible by 4: the two stages
    spec(1, 2, 2048, 64, ig=("uniform", -20, 20), fg=("normal", 0, 4), fgate_floor=(0.01, -30.0)),
    spec(1, 2, 1500, 128, ig=("uniform", -40, 40), fg=("normal", -2, 3)),
    # 384 < d <= 512: the one-wave kernel with its own scan
    spec(1, 1, 4, 400), spec(2, 1, 132, 416), spec(1, 2, 1000, 448), spec(2, 2, 2048, 512),
    spec(1, 1, 260, 512, ig=("normal", 0, 2), fg=("normal", 3, 1.5)),
    spec(1, 2, 2048, 480, ig=("uniform", -20, 20), fg=("normal", 0, 4), fgate_floor=(0.01, -30.0)),
    spec(1, 1, 63, 512),  # a length not divisible by 4: the two stages
]


def _pipelined(s):
    """Whether the one-launch forward pass runs the software-pipelined kernel
    (bf16, d a multiple of 64 up to 192, T <= 2048 divisible by 4)."""
    return (s["dtype"] == "bf16" and s["d"] % 64 == 0 and s["d"] <= 192 and s["T"] <= 2048
            and s["T"] % 4 == 0)


@pytest.mark.parametrize("forget", ["sigmoid", "exp"])
@pytest.mark.parametrize("s", FUSED_CASES, ids=_id)
def test_fused_scan_equals_the_two_stage_pass_bitwise(s, forget):
    """Up to 2048 positions (bf16, head dim up to 512, length divisible by 4)
    the one-shot entry points run a single tile kernel that scans the gates in
    its prologue.  The scan there has the gate-scan kernel's block structure
    (run by 256 threads, two scan threads each, in the one-wave kernels), so
    h, m and n must be the bits of the two-stage pass: gate scan, then the
    tile kernel with the same arithmetic on the workspace (the two-wave pair
    kernel for 192 < d <= 384; for d <= 192 the one-launch pass runs the
    pipelined kernel, whose sums are those of the one-wave kernel)."""
    x = W.make(s, seed=71)
    if forget == "exp":  # log f = f~, small and negative
        x["fgate"] = (-0.02 * np.abs(x["fgate"])).astype(np.float32)
    q, k, v, ig, fg = _dev(x)
    if forget == "sigmoid":
        a = mlstm.parallel_fwd(q, k, v, ig, fg)
    else:
        a = mlstm.parallel_fwd_train(q, k, v, ig, fg, forget="exp")[:3]
    b = mlstm.parallel_fwd_staged(q, k, v, ig, fg, kernel="mfma_single" if _pipelined(s) else "mfma",
                                  forget=forget)
    torch.cuda.synchronize()
    for name, ta, tb in zip("hmn", a, b):
        assert torch.equal(ta, tb), name
    if s["T"] <= 300:
        check_full(_host(a[0]), _host(a[1]), _host(a[2]), x, "bf16", forget=forget)


PIPELINED_CASES = [
    spec(1, 1, 4, 64), spec(1, 2, 100, 64), spec(2, 1, 512, 128), spec(1, 1, 252, 192),
    spec(3, 1, 388, 64, ig=("normal", 0, 2), fg=("normal", 3, 1.5)),
    spec(1, 2, 600, 128, ig=("uniform", -20, 20), fg=("normal", 0, 4), fgate_floor=(0.01, -30.0)),
    spec(1, 1, 520, 192, ig=("uniform", -40, 40), fg=("normal", -2, 3)),
    spec(8, 1, 136, 64),  # head count divisible by 8 (XCD-grouped schedule)
]


@pytest.mark.parametrize("s", PIPELINED_CASES, ids=_id)
def test_pipelined_kernel_full(s):
    """The software-pipelined kernel (one wave per SIMD, K and V staged
    through registers, d <= 192) against the oracle on every row: ragged
    tails, several row tiles, tiles skipped under strong decay."""
    assert _pipelined(s)
    x = W.make(s, seed=5)
    h, m, n = run_gpu(x)
    check_full(h, m, n, x, "bf16")


def test_pipelined_kernel_epilogues():
    """Output gate, stored h~ and the row sums b through the pipelined kernel:
    the gated h is sigma(o~) h~ of the ungated pass's float32 h~, b matches
    the oracle's (Eqs. 78, 83)."""
    s = spec(2, 1, 300, 128)
    x = W.make(s, seed=6)
    q, k, v, ig, fg = _dev(x)
    og = torch.from_numpy(W.round_bf16(np.random.default_rng(3).standard_normal(
        x["q"].shape).astype(np.float32))).to("cuda").to(torch.bfloat16)
    hg, ht, m, n = mlstm.parallel_fwd_gated(q, k, v, ig, fg, og, htilde=True)
    h0, m0, n0 = mlstm.parallel_fwd(q, k, v, ig, fg)
    ht2, m2, n2, b2 = mlstm.parallel_fwd_train(q, k, v, ig, fg)
    torch.cuda.synchronize()
    assert torch.equal(ht, h0) and torch.equal(m, m0) and torch.equal(n, n0)
    assert torch.equal(ht2, h0) and torch.equal(n2, n0)
    hr, mr, nr, br, rho, rho_num = oracle_full(x)
    kap, kapn = conditions(nr, hr, rho, rho_num)
    gate = 1.0 / (1.0 + np.exp(-_host(og)))
    check(_host(hg), _host(m), _host(n), hr * gate, mr, nr, kap, kapn, TOL_H["bf16"], K_H["bf16"],
          K_NUM["bf16"])
    assert b_over_bar(_host(b2), br, nr, kap) <= 1.0


def test_tile_skipping_long_context_full_size():
    x = W.make("long_context_16k", seed=0)
    a = _staged(x, "auto")
    b = _staged(x, "mfma_all_tiles")
    for ta, tb in zip(a, b):
        assert torch.equal(ta, tb)


# ---------------------------------------------------------------------------
# recurrent step (generation): T steps from a fresh state against the oracle
# ---------------------------------------------------------------------------

def _run_steps(x, in_place=True):
    q, k, v, ig, fg = _dev(x)
    B, NH, T, d = q.shape
    state = mlstm.recurrent_state(B, NH, d, "cuda")
    hs, ms, dens = [], [], []
    for t in range(T):
        C, n, m = state
        out = (C if in_place else torch.empty_like(C), torch.empty_like(n), torch.empty_like(m))
        h, state, den = mlstm.recurrent_step(q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                                             v[:, :, t].contiguous(), ig[:, :, t].contiguous(),
                                             fg[:, :, t].contiguous(), state, out_state=out,
                                             den=True)
        hs.append(h)
        ms.append(state[2].clone())
        dens.append(den)
    torch.cuda.synchronize()
    H = torch.stack(hs, dim=2)
    M = torch.stack(ms, dim=2)
    N = torch.stack(dens, dim=2)
    return _host(H), _host(M), _host(N), tuple(_host(s) for s in state)


@pytest.mark.parametrize("s", [
    spec(1, 2, 40, 64, "fp32"), spec(2, 1, 33, 128, "fp32"),
    spec(1, 2, 40, 64), spec(1, 1, 30, 384), spec(1, 1, 20, 512), spec(1, 3, 25, 16),
    spec(1, 2, 60, 64, "fp32", ig=("uniform", -20, 20), fg=("normal", 0, 4),
         fgate_floor=(0.05, -30.0)),
], ids=_id)
def test_recurrent_steps_match_oracle(s):
    x = W.make(s, seed=15)
    h, m, den, (C, n, mT) = _run_steps(x)
    hr, mr, denr, CT, nT = oracle.forward_recurrent_stabilized(
        x["q"], x["k"], x["v"], x["igate"], x["fgate"])
    dt = s["dtype"]
    # the denominator is row t's n (Eq. 84): the parallel form gives its condition number
    hp, mp, npar, _, rho, rho_num = oracle_full(x)
    kap, kapn = conditions(npar, hp, rho, rho_num)
    print(check(h, m, den, hr, mr, denr, kap, kapn, TOL_H[dt], K_H[dt], K_NUM[dt]))
    # final states (float32 recurrences; states are not rounded to bf16)
    assert head_normwise(C.reshape(C.shape[0], C.shape[1], -1),
                         CT.reshape(CT.shape[0], CT.shape[1], -1)) <= 1e-4
    assert head_normwise(n, nT) <= 1e-4
    # the recurrent step and the parallel pass agree on h~, m and n
    print(check(h, m, den, hp, mp, npar, kap, kapn, TOL_H[dt], K_H[dt], K_NUM[dt]))


def test_recurrent_step_in_place_equals_out_of_place_bitwise():
    x = W.make(spec(2, 2, 12, 128), seed=16)
    a = _run_steps(x, in_place=True)
    b = _run_steps(x, in_place=False)
    for ta, tb in zip(a[:3], b[:3]):
        assert np.array_equal(ta, tb)
    for ta, tb in zip(a[3], b[3]):
        assert np.array_equal(ta, tb)


def test_recurrent_step_full_size_decode_shape():
    """One step of the 125M-shaped layer (B=8, NH=4, d=384) from a random
    state; sampled heads against the oracle step."""
    rng = np.random.default_rng(17)
    B, NH, d = 8, 4, 384
    q, k, v = (W.round_bf16(rng.standard_normal((B, NH, d)).astype(np.float32)) for _ in range(3))
    ig = rng.standard_normal((B, NH)).astype(np.float32)
    fg = (3.0 + rng.standard_normal((B, NH))).astype(np.float32)
    C0 = (0.1 * rng.standard_normal((B, NH, d, d))).astype(np.float32)
    n0 = (0.1 * rng.standard_normal((B, NH, d))).astype(np.float32)
    m0 = rng.standard_normal((B, NH)).astype(np.float32)
    dev = lambda a, dt=torch.float32: torch.from_numpy(a).to("cuda").to(dt).contiguous()
    state = (dev(C0), dev(n0), dev(m0))
    h, (C1, n1, m1), den = mlstm.recurrent_step(dev(q, torch.bfloat16), dev(k, torch.bfloat16),
                                                dev(v, torch.bfloat16), dev(ig), dev(fg), state,
                                                den=True)
    torch.cuda.synchronize()
    h, C1, n1, m1, den = (_host(t) for t in (h, C1, n1, m1, den))
    for bi, hi in [(0, 0), (3, 2), (7, 3)]:
        hr, Cr, nr, mr, dr = oracle.recurrent_step_stabilized(
            q[bi, hi], k[bi, hi], v[bi, hi], ig[bi, hi], fg[bi, hi], C0[bi, hi], n0[bi, hi],
            float(m0[bi, hi]))
        assert abs(m1[bi, hi] - mr) <= 1e-5 * max(abs(mr), 1.0)
        assert abs(den[bi, hi] - dr) <= 1e-5 * dr
        assert np.abs(h[bi, hi] - hr).max() <= 2e-2 * np.abs(hr).max()
        assert np.abs(C1[bi, hi] - Cr).max() <= 1e-5 * np.abs(Cr).max()
        assert np.abs(n1[bi, hi] - nr).max() <= 1e-5 * np.abs(nr).max()


def test_recurrent_step_alias_rejected_on_gpu():
    q = torch.zeros((1, 1, 64), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((1, 1), dtype=torch.float32, device="cuda")
    state = mlstm.recurrent_state(1, 1, 64, "cuda")
    with pytest.raises(mlstm.MlstmError) as e:
        mlstm.recurrent_step(q, q, q, g, g, state, out_state=state)
    assert e.value.status == -9


# ---------------------------------------------------------------------------
# training forward (b) and backward pass (Eqs. 87-105)
# ---------------------------------------------------------------------------

def test_training_forward_returns_b():
    x = W.make(spec(2, 2, 300, 64, ig=("normal", 0, 2)), seed=18)
    q, k, v, ig, fg = _dev(x)
    h, m, n, b = mlstm.parallel_fwd_train(q, k, v, ig, fg)
    h0, m0, n0 = mlstm.parallel_fwd(q, k, v, ig, fg)
    torch.cuda.synchronize()
    assert torch.equal(h, h0) and torch.equal(m, m0) and torch.equal(n, n0)
    _, _, nr, br, rho, _ = oracle_full(x)
    bb = _host(b)
    assert b_over_bar(bb, br, nr, rho / nr) <= 1.0
    # n = max(|b|, exp(-m)) (Eq. 84): exactly |b| above the floor
    nn, floor = _host(n), np.exp(-_host(m))
    above = np.abs(bb) > floor * (1 + 1e-6)
    assert above.any() and (~above).any()
    assert np.array_equal(nn[above], np.abs(bb[above]))
    assert np.allclose(nn[~above], np.maximum(np.abs(bb[~above]), floor[~above]), rtol=1e-6)


BWD_CASES = [
    spec(1, 2, 50, 16, "fp32"), spec(1, 1, 77, 64, "fp32", ig=("normal", 0, 2), fg=("normal", 1, 2)),
    spec(2, 1, 130, 128, "fp32"),
    spec(1, 2, 100, 64), spec(1, 1, 140, 384), spec(1, 1, 66, 512),
    spec(1, 1, 200, 32, "fp32", ig=("uniform", -20, 20), fg=("normal", 0, 4),
         fgate_floor=(0.02, -30.0)),
]


@pytest.mark.parametrize("s", BWD_CASES, ids=_id)
def test_backward_matches_oracle(s):
    x = W.make(s, seed=19)
    q, k, v, ig, fg = _dev(x)
    rng = np.random.default_rng(20)
    dh_np = rng.standard_normal(x["q"].shape).astype(np.float32)
    if s["dtype"] == "bf16":
        dh_np = W.round_bf16(dh_np)
    dh = torch.from_numpy(dh_np).to("cuda").to(q.dtype).contiguous()
    h, m, n, b = mlstm.parallel_fwd_train(q, k, v, ig, fg)
    grads = mlstm.parallel_bwd(q, k, v, ig, fg, h, m, n, b, dh)
    torch.cuda.synchronize()
    got = [_host(t) for t in grads]
    ref = oracle.backward_stabilized(x["q"], x["k"], x["v"], x["igate"], x["fgate"], dh_np)
    hr = oracle_full(x)[0]
    _check_backward(got, ref, head_normwise(_host(h), hr), s["dtype"])


def test_backward_deterministic_bitwise():
    x = W.make(spec(1, 2, 150, 128), seed=21)
    q, k, v, ig, fg = _dev(x)
    dh = torch.randn(q.shape, generator=torch.Generator().manual_seed(0)).to("cuda").to(q.dtype)
    h, m, n, b = mlstm.parallel_fwd_train(q, k, v, ig, fg)
    a = mlstm.parallel_bwd(q, k, v, ig, fg, h, m, n, b, dh)
    c = mlstm.parallel_bwd(q, k, v, ig, fg, h, m, n, b, dh)
    torch.cuda.synchronize()
    for ta, tc in zip(a, c):
        assert torch.equal(ta, tc)


# ---------------------------------------------------------------------------
# exponential forget gate (f = exp(f~)): forward, recurrent step and backward
# ---------------------------------------------------------------------------

EXP_CASES = [
    spec(1, 2, 130, 64, "fp32", fg=("normal", -0.05, 0.03)),
    spec(1, 2, 257, 128, fg=("normal", -0.05, 0.03)),
    spec(1, 1, 160, 384, fg=("normal", -0.02, 0.02)),
    spec(2, 1, 200, 64, ig=("uniform", -10, 10), fg=("uniform", -3.0, 0.5)),  # some f > 1
]


@pytest.mark.parametrize("s", EXP_CASES, ids=_id)
def test_exp_forget_forward_matches_oracle(s):
    x = W.make(s, seed=22)
    q, k, v, ig, fg = _dev(x)
    # the two-stage pass with the tile kernel whose sums the one-launch pass
    # reproduces (the one-wave kernel where the pipelined kernel runs)
    kern = "mfma_single" if _pipelined(s) else "auto"
    h, m, n = mlstm.parallel_fwd_staged(q, k, v, ig, fg, kernel=kern, forget="exp")
    ht, mt, nt, b = mlstm.parallel_fwd_train(q, k, v, ig, fg, forget="exp")
    hs, ms, ns = mlstm.parallel_fwd_staged(q, k, v, ig, fg)  # sigmoid: must differ
    torch.cuda.synchronize()
    assert torch.equal(h, ht) and torch.equal(m, mt) and torch.equal(n, nt)
    assert not torch.equal(m, ms)
    check_full(_host(h), _host(m), _host(n), x, s["dtype"], forget="exp")
    _, _, nr, br, rho, _ = oracle_full(x, forget="exp")
    assert b_over_bar(_host(b), br, nr, rho / nr) <= 1.0


@pytest.mark.parametrize("s", [spec(1, 2, 40, 64, "fp32", fg=("normal", -0.05, 0.03)),
                               spec(1, 1, 30, 384, fg=("uniform", -2.0, 0.3))], ids=_id)
def test_exp_forget_recurrent_steps_match_oracle(s):
    x = W.make(s, seed=23)
    q, k, v, ig, fg = _dev(x)
    B, NH, T, d = q.shape
    state = mlstm.recurrent_state(B, NH, d, "cuda")
    hs, ms, dens = [], [], []
    for t in range(T):
        h, state, den = mlstm.recurrent_step(
            q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(),
            ig[:, :, t].contiguous(), fg[:, :, t].contiguous(), state, den=True, forget="exp")
        hs.append(h)
        ms.append(state[2].clone())
        dens.append(den)
    torch.cuda.synchronize()
    h, m, den = (_host(torch.stack(a, dim=2)) for a in (hs, ms, dens))
    hr, mr, denr, CT, nT = oracle.forward_recurrent_stabilized(
        x["q"], x["k"], x["v"], x["igate"], x["fgate"], forget="exp")
    hp, _, npar, _, rho, rho_num = oracle_full(x, forget="exp")
    kap, kapn = conditions(npar, hp, rho, rho_num)
    dt = s["dtype"]
    print(check(h, m, den, hr, mr, denr, kap, kapn, TOL_H[dt], K_H[dt], K_NUM[dt]))
    C = _host(state[0])
    assert head_normwise(C.reshape(B, NH, -1), CT.reshape(B, NH, -1)) <= 1e-4
    assert head_normwise(_host(state[1]), nT) <= 1e-4


@pytest.mark.parametrize("s", [spec(1, 2, 77, 64, "fp32", fg=("normal", -0.05, 0.03)),
                               spec(1, 1, 100, 128, fg=("uniform", -2.0, 0.3))], ids=_id)
def test_exp_forget_backward_matches_oracle(s):
    x = W.make(s, seed=24)
    q, k, v, ig, fg = _dev(x)
    rng = np.random.default_rng(25)
    dh_np = rng.standard_normal(x["q"].shape).astype(np.float32)
    if s["dtype"] == "bf16":
        dh_np = W.round_bf16(dh_np)
    dh = torch.from_numpy(dh_np).to("cuda").to(q.dtype).contiguous()
    h, m, n, b = mlstm.parallel_fwd_train(q, k, v, ig, fg, forget="exp")
    grads = mlstm.parallel_bwd(q, k, v, ig, fg, h, m, n, b, dh, forget="exp")
    torch.cuda.synchronize()
    ref = oracle.backward_stabilized(x["q"], x["k"], x["v"], x["igate"], x["fgate"], dh_np,
                                     forget="exp")
    hr = oracle.forward_stabilized(x["q"], x["k"], x["v"], x["igate"], x["fgate"],
                                   forget="exp")[0]
    _check_backward([_host(g) for g in grads], ref, head_normwise(_host(h), hr), s["dtype"])


# ---------------------------------------------------------------------------
# wide heads (d up to 1024): the four-member MFMA kernel, the float32 vector
# kernel's shared K/V buffer and the wider recurrent step
# ---------------------------------------------------------------------------

WIDE_CASES = [
    spec(1, 1, 1, 1024), spec(1, 1, 33, 1024), spec(1, 2, 161, 1024),
    spec(2, 1, 100, 544), spec(1, 1, 130, 640), spec(1, 1, 97, 768), spec(1, 1, 70, 896),
    spec(1, 1, 300, 1024, ig=("uniform", -20, 20), fg=("normal", 0, 4),
         fgate_floor=(0.01, -30.0)),
    spec(8, 1, 65, 1024),  # head count divisible by 8 (XCD-grouped schedule)
]


@pytest.mark.parametrize("s", WIDE_CASES, ids=_id)
def test_wide_heads_full(s):
    x = W.make(s, seed=21)
    h, m, n = run_gpu(x)
    check_full(h, m, n, x, "bf16")


@pytest.mark.parametrize("s", [spec(1, 1, 40, 16), spec(1, 2, 150, 64), spec(1, 1, 200, 384),
                               spec(2, 1, 129, 512), spec(1, 1, 90, 1008)], ids=_id)
def test_wide_kernel_forced_any_head_dim(s):
    """The wide kernel pads d up to a multiple of 128 (at least 512); zero
    columns add nothing, so it is correct for every head dimension."""
    x = W.make(s, seed=22)
    h, m, n = run_gpu(x, kernel="mfma_wide")
    check_full(h, m, n, x, "bf16")


@pytest.mark.parametrize("s", [spec(1, 1, 70, 1024, "fp32"), spec(1, 2, 45, 640, "fp32")],
                         ids=_id)
def test_wide_heads_fp32(s):
    x = W.make(s, seed=23)
    h, m, n = run_gpu(x)
    check_full(h, m, n, x, "fp32")


def test_wide_heads_vector_kernel_bf16_inputs():
    x = W.make(spec(1, 1, 120, 1024), seed=24)
    h, m, n = run_gpu(x, kernel="vector")
    check_full(h, m, n, x, "bf16", tol_h=4e-3)


def test_wide_heads_skipping_matches_all_tiles():
    x = W.make(spec(1, 2, 700, 1024, ig=("uniform", -40, 40), fg=("normal", -2, 3)), seed=25)
    a = _staged(x, "mfma")
    b = _staged(x, "mfma_all_tiles")
    for ta, tb in zip(a, b):
        assert torch.equal(ta, tb)
    check_full(_host(a[0]), _host(a[1]), _host(a[2]), x, "bf16")


def test_wide_heads_deterministic_and_causal_bitwise():
    x = W.make(spec(1, 2, 300, 1024), seed=26)
    a = run_gpu(x)
    b = run_gpu(x)
    for ta, tb in zip(a, b):
        assert np.array_equal(ta, tb)
    t0 = 150
    y = {k_: (v_.copy() if isinstance(v_, np.ndarray) else v_) for k_, v_ in x.items()}
    rng = np.random.default_rng(27)
    for key in ("q", "k", "v"):
        y[key][:, :, t0 + 1:] = W.round_bf16(rng.standard_normal(y[key][:, :, t0 + 1:].shape)
                                             .astype(np.float32))
    c = run_gpu(y)
    for ta, tc in zip(a, c):
        assert np.array_equal(ta[:, :, :t0 + 1], tc[:, :, :t0 + 1])


def test_wide_heads_output_gate_and_b():
    x = W.make(spec(1, 2, 140, 1024, ig=("normal", 0, 2)), seed=28)
    og_np = W.make_ogate(x["spec"], seed=28)
    q, k, v, ig, fg = _dev(x)
    og = torch.from_numpy(og_np).to("cuda").to(torch.bfloat16).contiguous()
    h, ht, m, n = mlstm.parallel_fwd_gated(q, k, v, ig, fg, og, htilde=True)
    h0, m0, n0 = mlstm.parallel_fwd(q, k, v, ig, fg)
    _, _, _, b = mlstm.parallel_fwd_train(q, k, v, ig, fg)
    torch.cuda.synchronize()
    assert torch.equal(ht, h0) and torch.equal(m, m0) and torch.equal(n, n0)
    hr, mr, nr, br, rho, _ = oracle_full(x)
    check_full(_host(h), _host(m), _host(n), x, "bf16", h_ref=oracle.output_gate(hr, og_np))
    assert b_over_bar(_host(b), br, nr, rho / nr) <= 1.0


def test_wide_heads_recurrent_steps_match_oracle():
    x = W.make(spec(1, 2, 12, 1024), seed=29)
    h, m, den, (C, n, mT) = _run_steps(x)
    hr, mr, denr, CT, nT = oracle.forward_recurrent_stabilized(
        x["q"], x["k"], x["v"], x["igate"], x["fgate"])
    hp, _, npar, _, rho, rho_num = oracle_full(x)
    kap, kapn = conditions(npar, hp, rho, rho_num)
    print(check(h, m, den, hr, mr, denr, kap, kapn, TOL_H["bf16"], K_H["bf16"], K_NUM["bf16"]))
    assert head_normwise(C.reshape(C.shape[0], C.shape[1], -1),
                         CT.reshape(CT.shape[0], CT.shape[1], -1)) <= 1e-4
    assert head_normwise(n, nT) <= 1e-4


WIDE_BWD_CASES = [
    spec(1, 1, 40, 528, "fp32"),
    spec(1, 2, 70, 640, "fp32", ig=("normal", 0, 2), fg=("normal", 1, 2)),
    spec(1, 1, 33, 1024, "fp32"),
    # the stress gate law in float32 (as for the narrow vector passes): with
    # bf16 inputs its conditioning amplifies the bf16 rounding of the stored
    # h~ that dL/dn reads (Eqs. 88-89) to about the 2e-2 bar itself
    spec(2, 1, 40, 544, "fp32", ig=("uniform", -20, 20), fg=("normal", 0, 4),
         fgate_floor=(0.02, -30.0)),
    spec(1, 1, 90, 768), spec(1, 2, 50, 1024),
    spec(2, 1, 60, 576, ig=("normal", 0, 2), fg=("normal", 1, 2)),
]


@pytest.mark.parametrize("s", WIDE_BWD_CASES, ids=_id)
def test_wide_heads_backward_matches_oracle(s):
    """Above d = 512 the backward runs the float32 vector passes in
    head-dimension chunks of 256, for float32 and bf16 inputs alike."""
    x = W.make(s, seed=30)
    rng = np.random.default_rng(31)
    dh_np = rng.standard_normal(x["q"].shape).astype(np.float32)
    if s["dtype"] == "bf16":
        dh_np = W.round_bf16(dh_np)
    got, ref, fwd = _backward_case(x, dh_np)
    _check_backward(got, ref, fwd, s["dtype"])


def test_wide_heads_workload_sampled():
    """The 1.3B-shaped layer with true heads of 1024 (B=4, NH=4, T=2048)."""
    x = W.make("xlstm1p3b_layer_d1024", seed=0)
    h, m, n = run_gpu(x)
    rows = _sample_rows(x["spec"]["T"], np.random.default_rng(31), count=24)
    _check_sampled(h, m, n, x, rows, "xlstm1p3b_layer_d1024")


# ---------------------------------------------------------------------------
# backward on the matrix cores (bf16, d <= 384): dQ / r, dK / c, dV passes
# ---------------------------------------------------------------------------

BWD_MFMA_CASES = [
    spec(1, 1, 1, 16), spec(1, 1, 33, 96), spec(1, 2, 300, 64), spec(2, 1, 257, 128),
    spec(1, 3, 200, 48), spec(1, 1, 130, 384), spec(1, 1, 161, 320),
    spec(8, 1, 140, 64),  # head count divisible by 8 (XCD-grouped schedule)
    spec(1, 2, 333, 160, ig=("uniform", -20, 20), fg=("normal", 0, 4), fgate_floor=(0.01, -30.0)),
    spec(1, 1, 200, 64, ig=("normal", 0, 2), fg=("normal", 1, 2)),
    spec(1, 1, 150, 448), spec(2, 1, 129, 512),  # output columns split over two workgroups
]


def _backward_case(x, dh_np, heads=None):
    q, k, v, ig, fg = _dev(x)
    dh = torch.from_numpy(dh_np).to("cuda").to(q.dtype).contiguous()
    h, m, n, b = mlstm.parallel_fwd_train(q, k, v, ig, fg)
    grads = mlstm.parallel_bwd(q, k, v, ig, fg, h, m, n, b, dh)
    torch.cuda.synchronize()
    got = [_host(t) for t in grads]
    if heads is None:
        ref = oracle.backward_stabilized(x["q"], x["k"], x["v"], x["igate"], x["fgate"], dh_np)
        hr = oracle_full(x)[0]
        return got, ref, head_normwise(_host(h), hr)
    out_got, out_ref, fwd = [], [], 0.0
    for bi, hi in heads:
        sl = (slice(bi, bi + 1), slice(hi, hi + 1))
        ref = oracle.backward_stabilized(x["q"][sl], x["k"][sl], x["v"][sl], x["igate"][sl],
                                         x["fgate"][sl], dh_np[sl])
        out_got.append([g[sl] for g in got])
        out_ref.append(ref)
        hr = oracle.forward_stabilized(x["q"][sl], x["k"][sl], x["v"][sl], x["igate"][sl],
                                       x["fgate"][sl])[0]
        fwd = max(fwd, head_normwise(_host(h)[sl], hr))
    cat = lambda parts, i: np.concatenate([p[i] for p in parts], axis=1)
    return ([cat(out_got, i) for i in range(5)], [cat(out_ref, i) for i in range(5)], fwd)


def _check_backward(got, ref, fwd_err, dtype="bf16"):
    """Gradients per head, normwise, against the oracle's Eqs. 87-105.  bf16:
    2e-2 for all five (the products' operands are rounded to bf16 like the
    forward's C~').  float32: 1e-4, or three times the forward's own h~ error
    on the same inputs if that is larger: dL/dn_i = -(dh_i . h~_i) / n_i uses
    the forward's h~, so the backward cannot be more accurate than it."""
    tol = 2e-2 if dtype == "bf16" else max(1e-4, 3.0 * fwd_err)
    errs = {name: head_normwise(g, r) for name, g, r in
            zip(("dq", "dk", "dv", "digate", "dfgate"), got, ref)}
    print(errs, "forward h error", fwd_err)
    for name, e in errs.items():
        assert e <= tol, (name, errs)
    return errs


@pytest.mark.parametrize("s", BWD_MFMA_CASES, ids=_id)
def test_backward_mfma_matches_oracle(s):
    x = W.make(s, seed=32)
    dh_np = W.round_bf16(np.random.default_rng(33).standard_normal(x["q"].shape)
                         .astype(np.float32))
    got, ref, fwd = _backward_case(x, dh_np)
    _check_backward(got, ref, fwd)


def test_backward_mfma_full_size_sampled_heads():
    """The 125M-shaped layer (B=8, NH=4, T=2048, d=384): two heads against the oracle."""
    x = W.make("xlstm125m_layer", seed=0)
    dh_np = W.round_bf16(np.random.default_rng(34).standard_normal(x["q"].shape)
                         .astype(np.float32))
    got, ref, fwd = _backward_case(x, dh_np, heads=[(0, 0), (7, 3)])
    _check_backward(got, ref, fwd)


def test_backward_mfma_full_size_sub_heads_of_512():
    """The 1.3B-shaped layer as sub-heads of 512 (B=4, NH=8, T=2048): two heads."""
    x = W.make("xlstm1p3b_layer", seed=0)
    dh_np = W.round_bf16(np.random.default_rng(35).standard_normal(x["q"].shape)
                         .astype(np.float32))
    got, ref, fwd = _backward_case(x, dh_np, heads=[(0, 1), (3, 7)])
    _check_backward(got, ref, fwd)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_first_forget_gate_gradient_is_exactly_zero(dtype):
    """f_0 enters no product F_ij (Eq. 101): its gradient is exactly 0, as in
    the oracle's double sum over j < 0 (the suffix-sum form would leave the
    rounding of sum r - sum c there)."""
    for T in (1, 2, 77):
        x = W.make(spec(2, 2, T, 32, dtype), seed=42)
        q, k, v, ig, fg = _dev(x)
        h, m, n, b = mlstm.parallel_fwd_train(q, k, v, ig, fg)
        dh = torch.ones_like(q)
        dfg = mlstm.parallel_bwd(q, k, v, ig, fg, h, m, n, b, dh)[4]
        torch.cuda.synchronize()
        assert bool((dfg[..., 0] == 0).all()), (T, dfg[..., 0])
        assert torch.isfinite(dfg).all()


@pytest.mark.parametrize("shape", [(2, 2, 600, 384), (1, 2, 300, 512), (1, 1, 129, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_backward_stored_operands_against_the_recomputing_passes(shape, monkeypatch):
    """By default the keys pass stores the operands of the values and rows
    passes (bf16(C~'/n) and bf16(P)), which then only accumulate;
    MLSTM_BWD_STORE_MAX=0 makes them recompute S and G instead.  dV comes
    from the same arithmetic either way and must be bitwise equal.  The rest
    differ by rounding: dQ takes P from the keys pass's orientation of S and
    G, the row sums r come from their closed form dh . h~ + db b, and the
    per-row kernel sums dh . h~ (hence db, used by dK) in another order than
    the recomputing rows pass; both paths must pass the oracle's readings."""
    B, NH, T, d = shape
    x = W.make(spec(B, NH, T, d), seed=40)
    dh_np = W.round_bf16(np.random.default_rng(41).standard_normal(x["q"].shape)
                         .astype(np.float32))
    heads = [(0, 0), (B - 1, NH - 1)] if B * NH > 1 else None
    monkeypatch.delenv("MLSTM_BWD_STORE_MAX", raising=False)
    stored, ref, fwd = _backward_case(x, dh_np, heads=heads)
    _check_backward(stored, ref, fwd)
    monkeypatch.setenv("MLSTM_BWD_STORE_MAX", "0")
    recomputed, ref2, fwd2 = _backward_case(x, dh_np, heads=heads)
    _check_backward(recomputed, ref2, fwd2)
    assert np.array_equal(stored[2], recomputed[2]), "dv"


# ---------------------------------------------------------------------------
# float32 head dims outside the float32 matrix-core kernel, T <= 2048: the
# vector kernel scans its head's gates itself (one launch, no workspace)
# ---------------------------------------------------------------------------

VECTOR_FUSED_CASES = [
    spec(1, 1, 64, 16, "fp32"), spec(1, 1, 1, 16, "fp32"), spec(2, 3, 77, 48, "fp32"),
    spec(1, 2, 2048, 16, "fp32"), spec(1, 1, 301, 80, "fp32", ig=("normal", 0, 2)),
    spec(1, 1, 130, 544, "fp32"), spec(1, 1, 65, 1024, "fp32"),
    spec(1, 2, 500, 112, "fp32", ig=("uniform", -20, 20), fg=("normal", 0, 4),
         fgate_floor=(0.01, -30.0)),
]


@pytest.mark.parametrize("s", VECTOR_FUSED_CASES, ids=_id)
def test_vector_kernel_fused_scan_matches_two_launches(s):
    """Bitwise the same h, m, n as the gate-scan launch followed by the vector
    kernel (the same scan arithmetic in the same order), and the oracle's
    readings."""
    x = W.make(s, seed=46)
    h, m, n = run_gpu(x)
    h2, m2, n2 = run_gpu(x, kernel="vector")
    assert np.array_equal(m, m2) and np.array_equal(n, n2) and np.array_equal(h, h2)
    check_full(h, m, n, x, "fp32")


@pytest.mark.parametrize("forget", ["sigmoid", "exp"])
def test_vector_kernel_fused_scan_exp_forget_and_b(forget):
    s = spec(1, 2, 99, 48, "fp32", fg=("normal", -0.05, 0.03) if forget == "exp" else
             ("normal", 3.0, 1.0))
    x = W.make(s, seed=47)
    q, k, v, ig, fg = _dev(x)
    h, m, n, b = mlstm.parallel_fwd_train(q, k, v, ig, fg, forget=forget)
    h2, m2, n2 = mlstm.parallel_fwd_staged(q, k, v, ig, fg, kernel="vector", forget=forget)
    torch.cuda.synchronize()
    assert torch.equal(h, h2) and torch.equal(m, m2) and torch.equal(n, n2)
    hr, mr, nr, br, rho, _ = oracle_full(x, forget)
    assert b_over_bar(_host(b), br, nr, rho / nr) <= 1.0


F32_FUSED_CASES = [
    spec(1, 1, 1, 32, "fp32"), spec(2, 3, 77, 64, "fp32"), spec(1, 2, 2048, 128, "fp32"),
    spec(1, 1, 301, 256, "fp32", ig=("normal", 0, 2)), spec(1, 2, 500, 384, "fp32"),
    spec(1, 1, 130, 512, "fp32"), spec(8, 1, 200, 96, "fp32"),
    spec(1, 2, 700, 160, "fp32", ig=("uniform", -20, 20), fg=("normal", 0, 4),
         fgate_floor=(0.01, -30.0)),
]


@pytest.mark.parametrize("s", F32_FUSED_CASES, ids=_id)
def test_fp32_matrix_core_fused_scan_matches_two_launches(s):
    """The float32 matrix-core kernel scanning its own gates (one launch):
    bitwise the gate-scan launch followed by the same kernel, and the
    oracle's readings."""
    x = W.make(s, seed=49)
    h, m, n = run_gpu(x)
    h2, m2, n2 = run_gpu(x, kernel="auto_staged")
    assert np.array_equal(m, m2) and np.array_equal(n, n2) and np.array_equal(h, h2)
    check_full(h, m, n, x, "fp32")


@pytest.mark.parametrize("forget", ["sigmoid", "exp"])
def test_fp32_matrix_core_fused_scan_epilogues(forget):
    s = spec(1, 2, 199, 384, "fp32", fg=("normal", -0.05, 0.03) if forget == "exp" else
             ("normal", 3.0, 1.0))
    x = W.make(s, seed=50)
    q, k, v, ig, fg = _dev(x)
    h, m, n, b = mlstm.parallel_fwd_train(q, k, v, ig, fg, forget=forget)
    h2, m2, n2 = mlstm.parallel_fwd_staged(q, k, v, ig, fg, forget=forget)
    og = torch.from_numpy(W.make_ogate(s, seed=51)).to("cuda")
    hg, ht, mg, ng = mlstm.parallel_fwd_gated(q, k, v, ig, fg, og, htilde=True) \
        if forget == "sigmoid" else (None, None, None, None)
    torch.cuda.synchronize()
    assert torch.equal(h, h2) and torch.equal(m, m2) and torch.equal(n, n2)
    hr, mr, nr, br, rho, _ = oracle_full(x, forget)
    assert b_over_bar(_host(b), br, nr, rho / nr) <= 1.0
    if hg is not None:
        assert torch.equal(ht, h)
        ref = _host(ht) / (1.0 + np.exp(-W.make_ogate(s, seed=51)))
        assert np.allclose(_host(hg), ref, rtol=1e-5, atol=1e-6)


def test_vector_kernel_just_past_the_fused_scan():
    """T = 2049 takes the two launches again (the fused scan covers 2048)."""
    x = W.make(spec(1, 1, 2049, 16, "fp32"), seed=48)
    h, m, n = run_gpu(x)
    check_full(h, m, n, x, "fp32")


# ---------------------------------------------------------------------------
# backward on the float32 matrix instruction (float32 inputs, d a multiple of
# 32 up to 384); d = 352 and 384 put the partial products in the spare tile
# buffer (three barriers per tile)
# ---------------------------------------------------------------------------

BWD_F32_CASES = [
    spec(1, 1, 1, 32, "fp32"), spec(1, 2, 77, 64, "fp32"), spec(1, 1, 100, 96, "fp32"),
    spec(2, 1, 161, 128, "fp32", ig=("normal", 0, 2), fg=("normal", 1, 2)),
    spec(8, 1, 70, 64, "fp32"),  # head count divisible by 8 (XCD-grouped schedule)
    spec(1, 1, 130, 256, "fp32"), spec(1, 1, 99, 320, "fp32"), spec(1, 1, 140, 352, "fp32"),
    spec(1, 2, 200, 384, "fp32"), spec(1, 1, 33, 224, "fp32"),
    spec(1, 2, 150, 160, "fp32", ig=("uniform", -20, 20), fg=("normal", 0, 4),
         fgate_floor=(0.01, -30.0)),
    spec(1, 1, 3000, 64, "fp32"),  # 94 tiles of 32 rows, ragged tail
]


def _grads_gpu(x, dh_np):
    q, k, v, ig, fg = _dev(x)
    dh = torch.from_numpy(dh_np).to("cuda").to(q.dtype).contiguous()
    h, m, n, b = mlstm.parallel_fwd_train(q, k, v, ig, fg)
    grads = mlstm.parallel_bwd(q, k, v, ig, fg, h, m, n, b, dh)
    torch.cuda.synchronize()
    return [_host(t) for t in grads]


@pytest.mark.parametrize("s", BWD_F32_CASES, ids=_id)
def test_backward_f32_matrix_core_matches_oracle(s, monkeypatch):
    """Against the oracle's Eqs. 87-105, and against the float32 vector passes
    on the same inputs (same per-entry formulas and exponents, the products
    summed in another order): both to the float32 bar."""
    x = W.make(s, seed=43)
    dh_np = np.random.default_rng(44).standard_normal(x["q"].shape).astype(np.float32)
    monkeypatch.delenv("MLSTM_BWD_F32", raising=False)
    got, ref, fwd = _backward_case(x, dh_np)
    _check_backward(got, ref, fwd, "fp32")
    monkeypatch.setenv("MLSTM_BWD_F32", "vector")
    vec = _grads_gpu(x, dh_np)
    _check_backward(got, vec, fwd, "fp32")
    again = _grads_gpu(x, dh_np)
    monkeypatch.delenv("MLSTM_BWD_F32")
    assert all(np.array_equal(a, b) for a, b in zip(vec, again))
    assert all(np.array_equal(a, b) for a, b in zip(got, _grads_gpu(x, dh_np))), "deterministic"


def test_backward_f32_matrix_core_full_size_sampled_heads():
    """The 125M-shaped layer (B=8, NH=4, T=2048, d=384) in float32: two heads
    against the oracle."""
    base = W.WORKLOADS["xlstm125m_layer"]
    x = W.make(dict(base, dtype="fp32"), seed=0)
    dh_np = np.random.default_rng(45).standard_normal(x["q"].shape).astype(np.float32)
    got, ref, fwd = _backward_case(x, dh_np, heads=[(0, 0), (7, 3)])
    _check_backward(got, ref, fwd, "fp32")


# ---------------------------------------------------------------------------
# large shapes: a 65536-position head (512 row tiles, 2048 key tiles) and a
# thousand small heads (grid and index arithmetic at size)
# ---------------------------------------------------------------------------

def test_long_sequence_sampled():
    x = W.make(spec(1, 1, 65536, 64), seed=36)
    h, m, n = run_gpu(x)
    rows = _sample_rows(x["spec"]["T"], np.random.default_rng(37), count=24)
    # m on the sampled rows only here: its row maxima at every position would
    # take the oracle 65536^2 entries
    hr, mr, nr, rho, rho_num = _sampled_reference(x, rows)
    kap, kapn = conditions(nr, hr, rho, rho_num)
    print(check(h[:, :, rows], m[:, :, rows], n[:, :, rows], hr, mr, nr, kap, kapn,
                TOL_H["bf16"], K_H["bf16"], K_NUM["bf16"]))
    assert np.isfinite(h).all() and np.isfinite(n).all()


def test_many_small_heads():
    x = W.make(spec(16, 64, 48, 16), seed=38)
    h, m, n = run_gpu(x)
    check_full(h, m, n, x, "bf16")


def test_aliased_outputs_rejected_on_gpu():
    x = W.make(spec(1, 1, 64, 16), seed=39)
    q, k, v, ig, fg = _dev(x)
    m = torch.empty((1, 1, 64), dtype=torch.float32, device="cuda")
    n = torch.empty_like(m)
    with pytest.raises(mlstm.MlstmError) as e:
        mlstm.parallel_fwd(q, k, v, ig, fg, out=(q, m, n))
    assert e.value.status == -9
    with pytest.raises(mlstm.MlstmError) as e:
        mlstm.parallel_fwd(q, k, v, ig, fg, out=(torch.empty_like(q), m, m))
    assert e.value.status == -9
    # inputs may alias each other: q as its own key
    h, m2, n2 = mlstm.parallel_fwd(q, q, v, ig, fg)
    torch.cuda.synchronize()
    y = dict(x, k=x["q"])
    check_full(_host(h), _host(m2), _host(n2), y, "bf16")


# ---------------------------------------------------------------------------
# HIP graphs and concurrent streams
# ---------------------------------------------------------------------------

def _inputs_into(bufs, x):
    for name, t in zip(("q", "k", "v", "igate", "fgate"), bufs):
        t.copy_(torch.from_numpy(x[name]).to(t.dtype))


def test_graph_capture_replays_match_eager():
    """mlstm_parallel_fwd (stream-ordered workspace) and the staged entry
    points (caller workspace) captured into HIP graphs: every replay, with new
    inputs copied in and eager work in between, equals the eager call bitwise
    (the staged pass runs the one-wave kernel, whose sums the pipelined
    kernel of the one-launch pass reproduces at this head dimension)."""
    s = spec(2, 2, 300, 64)
    assert _pipelined(s)
    xs = [W.make(s, seed=40 + i) for i in range(3)]
    q, k, v, ig, fg = _dev(xs[0])
    bufs = (q, k, v, ig, fg)
    h = torch.empty_like(q)
    m = torch.empty((2, 2, 300), dtype=torch.float32, device="cuda")
    n = torch.empty_like(m)
    ws = mlstm.alloc_workspace(2, 2, 300, q.device)
    h2, n2, m2 = torch.empty_like(h), torch.empty_like(n), torch.empty_like(m)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up on the capture stream
        mlstm.parallel_fwd(q, k, v, ig, fg, out=(h, m, n))
        mlstm.gate_scan(ig, fg, 64, ws, m=m2)
        mlstm.causal_tiles(q, k, v, m2, ws, kernel="mfma_single", out=(h2, n2))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g1, g2 = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1):
        mlstm.parallel_fwd(q, k, v, ig, fg, out=(h, m, n))
    with torch.cuda.graph(g2):
        mlstm.gate_scan(ig, fg, 64, ws, m=m2)
        mlstm.causal_tiles(q, k, v, m2, ws, kernel="mfma_single", out=(h2, n2))
    for x in xs + xs[:1]:
        _inputs_into(bufs, x)
        g1.replay()
        g2.replay()
        torch.cuda.synchronize()
        eh, em, en = mlstm.parallel_fwd(q, k, v, ig, fg)  # eager, between replays
        torch.cuda.synchronize()
        for a, b in ((h, eh), (m, em), (n, en), (h2, eh), (m2, em), (n2, en)):
            assert torch.equal(a, b)


def test_concurrent_streams_match_serial():
    xa = W.make(spec(1, 4, 700, 128), seed=44)
    xb = W.make(spec(2, 2, 513, 64), seed=45)
    da, db = _dev(xa), _dev(xb)
    ra = mlstm.parallel_fwd(*da)
    rb = mlstm.parallel_fwd(*db)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(sa):
            oa = mlstm.parallel_fwd(*da)
        with torch.cuda.stream(sb):
            ob = mlstm.parallel_fwd(*db)
        outs.append((oa, ob))
    torch.cuda.synchronize()
    for oa, ob in outs:
        for t, r in zip(oa + ob, ra + rb):
            assert torch.equal(t, r)


# ---------------------------------------------------------------------------
# the gate scan over long sequences: two passes from four 2048-position
# chunks on (chunk elements, then each chunk's carry folded from them)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", [6144, 6145, 8192, 8193, 20000])
def test_long_scan_m_matches_oracle(T):
    """m on rows around every chunk boundary and a random sample, against the
    oracle's row maximum of D~ (Eq. 80) taken row by row."""
    x = W.make(spec(1, 3, T, 16, ig=("uniform", -20, 20), fg=("normal", 0, 4),
                    fgate_floor=(0.01, -30.0)), seed=46)
    q, k, v, ig, fg = _dev(x)
    ws = mlstm.alloc_workspace(1, 3, T, "cuda")
    m = _host(mlstm.gate_scan(ig, fg, 16, ws))
    torch.cuda.synchronize()
    edges = [c * 2048 + o for c in range(1, T // 2048 + 1) for o in (-2, -1, 0, 1)]
    rows = np.array(sorted(set(r for r in edges if 0 <= r < T) |
                           set(_sample_rows(T, np.random.default_rng(49), count=20))))
    mr = np.stack([oracle.forward_rows(x["q"], x["k"], x["v"], x["igate"], x["fgate"], 0, hh,
                                       rows)[1] for hh in range(3)])[None]
    assert m_error(m[:, :, rows], mr) <= 1e-5


@pytest.mark.parametrize("forget", ["sigmoid", "exp"])
def test_long_scan_forward_sampled(forget):
    fg = ("normal", 3, 1) if forget == "sigmoid" else ("uniform", -0.3, 0.0)
    x = W.make(spec(1, 2, 12000, 64, fg=fg), seed=47)
    q, k, v, ig, fgt = _dev(x)
    h, m, n, b = mlstm.parallel_fwd_train(q, k, v, ig, fgt, forget=forget)
    torch.cuda.synchronize()
    rows = _sample_rows(12000, np.random.default_rng(48), count=24)
    H = np.empty((1, 2, len(rows), 64)); M = np.empty((1, 2, len(rows))); N = np.empty_like(M)
    R = np.empty_like(M)
    RN = np.empty_like(M)
    for hh in range(2):
        hr, mr, nr, _, rho, rho_num = oracle.forward_rows(x["q"], x["k"], x["v"], x["igate"],
                                                          x["fgate"], 0, hh, rows, forget=forget)
        H[0, hh], M[0, hh], N[0, hh], R[0, hh], RN[0, hh] = hr, mr, nr, rho, rho_num
    assert m_error(_host(m), m_every_position(x, forget)) <= 1e-5
    kap, kapn = conditions(N, H, R, RN)
    print(check(_host(h)[:, :, rows], _host(m)[:, :, rows], _host(n)[:, :, rows], H, M, N, kap,
                kapn, TOL_H["bf16"], K_H["bf16"], K_NUM["bf16"]))


# ---------------------------------------------------------------------------
# a seeded sweep of random shapes and gate laws through the default path
# ---------------------------------------------------------------------------

def _random_specs(count=24, seed=50):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        d = int(rng.choice([16, 32, 48, 64, 80, 128, 192, 256, 320, 384, 448, 512, 640, 1024]))
        T = int(rng.integers(1, 700 if d <= 512 else 260))
        dtype = "fp32" if rng.random() < 0.2 and d <= 512 else "bf16"
        B, NH = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        law = int(rng.integers(0, 3))
        if law == 0:
            ig, fg, floor = ("normal", 0.0, float(rng.uniform(0.5, 2))), ("normal", 3.0, 1.0), None
        elif law == 1:
            ig, fg, floor = ("uniform", -20.0, 20.0), ("normal", 0.0, 4.0), (0.01, -30.0)
        else:
            ig, fg, floor = ("normal", 0.0, 1.0), ("normal", float(rng.uniform(-3, 5)), 2.0), None
        s = spec(B, NH, T, d, dtype, ig=ig, fg=fg)
        if floor:
            s["fgate_floor"] = floor
        out.append(s)
    return out


@pytest.mark.parametrize("s", _random_specs(), ids=_id)
def test_random_shapes_match_oracle(s):
    x = W.make(s, seed=51)
    h, m, n = run_gpu(x)
    check_full(h, m, n, x, s["dtype"])
