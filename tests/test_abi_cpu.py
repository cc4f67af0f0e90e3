"""The C-ABI library loads and exports every symbol include/mlstm.h declares,
and its host-side argument checks reject bad calls before any device work.

No call here reaches the HIP runtime: every call fails validation, which runs
first and touches no device state.
"""
import ctypes
import os
import re

import pytest

from linear_recurrent_sequence_amd import mlstm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mlstm.h")

needs_lib = pytest.mark.skipif(not os.path.exists(mlstm.LIB_PATH),
                               reason="libmlstm.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mlstm_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("mlstm_parallel_fwd", "mlstm_parallel_fwd_stream", "mlstm_gate_scan",
                 "mlstm_causal_tiles", "mlstm_workspace_bytes", "mlstm_strerror"):
        assert want in names


@needs_lib
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(mlstm.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


@needs_lib
def test_strerror_and_workspace_size():
    for st in (0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10, -11):
        msg = mlstm.strerror(st)
        assert msg and msg != "unknown status"
    assert mlstm.strerror(-99) == "unknown status"
    lib = mlstm.load_library()
    # two float64 terms and one float32 term per position, two float64 tile
    # bounds per 32 positions and two float64 scan-chunk terms per 2048
    # positions, T padded to 128, each region 256-byte aligned
    assert lib.mlstm_workspace_bytes(1, 1, 64) == 2 * 1024 + 512 + 2 * 256 + 256
    assert lib.mlstm_workspace_bytes(8, 4, 2048) == (2 * 32 * 2048 * 8 + 32 * 2048 * 4
                                                     + 2 * 32 * 64 * 8 + 512)
    # 8 heads of 16384: 8 scan chunks each
    assert lib.mlstm_workspace_bytes(1, 8, 16384) == (2 * 8 * 16384 * 8 + 8 * 16384 * 4
                                                      + 2 * 8 * 512 * 8 + 8 * 8 * 16)
    assert lib.mlstm_workspace_bytes(0, 4, 2048) == 0
    assert lib.mlstm_workspace_bytes(1, 1, 0) == 0


FAKE = 1 << 20  # a 16-byte-aligned non-null address; never dereferenced


@needs_lib
@pytest.mark.parametrize("case,status", [
    (dict(q=0), -1), (dict(igate=0), -1), (dict(n_out=0), -1),
    (dict(B=0), -2), (dict(T=0), -2), (dict(NH=-3), -2), (dict(d=0), -2),
    (dict(dtype=2), -3), (dict(dtype=-1), -3),
    (dict(d=8), -4), (dict(d=24), -4), (dict(d=1040), -4), (dict(d=2048), -4),
    (dict(q=FAKE + 8), -5), (dict(m_out=FAKE + 4), -5),
])
def test_parallel_fwd_rejects_before_device_work(case, status):
    lib = mlstm.load_library()
    args = dict(q=FAKE, k=FAKE, v=FAKE, igate=FAKE, fgate=FAKE, h_out=FAKE, m_out=FAKE,
                n_out=FAKE, B=1, NH=1, T=64, d=16, dtype=1)
    args.update(case)
    order = ["q", "k", "v", "igate", "fgate", "h_out", "m_out", "n_out", "B", "NH", "T", "d", "dtype"]
    st = lib.mlstm_parallel_fwd(*[args[k] or None if k in order[:8] else args[k] for k in order])
    assert st == status


@needs_lib
def test_staged_entry_points_reject_before_device_work():
    lib = mlstm.load_library()
    # workspace too small
    assert lib.mlstm_gate_scan(FAKE, FAKE, FAKE, FAKE, 10, 1, 1, 64, 16, 0, None) == -7
    # misaligned workspace (needs 256 bytes)
    assert lib.mlstm_gate_scan(FAKE, FAKE, FAKE, FAKE + 16, 1 << 20, 1, 1, 64, 16, 0, None) == -5
    # unknown forget-gate activation
    assert lib.mlstm_gate_scan(FAKE, FAKE, FAKE, FAKE, 1 << 20, 1, 1, 64, 16, 2, None) == -10
    assert lib.mlstm_gate_scan(FAKE, FAKE, FAKE, FAKE, 1 << 20, 1, 1, 64, 16, -1, None) == -10
    # MFMA kernel for float32 inputs
    assert lib.mlstm_causal_tiles(FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, FAKE, FAKE,
                                  1, 1, 64, 16, 0, 1, None) == -8
    assert lib.mlstm_causal_tiles(FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, FAKE, FAKE,
                                  1, 1, 64, 16, 0, 3, None) == -8
    # unknown kernel selector
    assert lib.mlstm_causal_tiles(FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, FAKE, FAKE,
                                  1, 1, 64, 16, 1, 7, None) == -8
    assert lib.mlstm_causal_tiles(FAKE, FAKE, FAKE, None, FAKE, 1 << 20, FAKE, FAKE,
                                  1, 1, 64, 16, 1, 0, None) == -1
    assert lib.mlstm_causal_tiles(FAKE, FAKE, FAKE, FAKE, FAKE, 10, FAKE, FAKE,
                                  1, 1, 64, 16, 1, 0, None) == -7


@needs_lib
@pytest.mark.parametrize("case,status", [
    (dict(ogate=0), -1), (dict(q=0), -1), (dict(ogate=FAKE + 8), -5),
    (dict(htilde_out=FAKE + 2), -5), (dict(d=24), -4), (dict(dtype=3), -3), (dict(T=0), -2),
])
def test_gated_forward_rejects_before_device_work(case, status):
    lib = mlstm.load_library()
    args = dict(q=FAKE, k=FAKE, v=FAKE, igate=FAKE, fgate=FAKE, ogate=FAKE, h_out=FAKE,
                htilde_out=0, m_out=FAKE, n_out=FAKE, B=1, NH=1, T=64, d=16, dtype=1)
    args.update(case)
    ptrs = ["q", "k", "v", "igate", "fgate", "ogate", "h_out", "htilde_out", "m_out", "n_out"]
    st = lib.mlstm_parallel_fwd_gated(*[args[k] or None for k in ptrs],
                                      args["B"], args["NH"], args["T"], args["d"], args["dtype"],
                                      None)
    assert st == status


@needs_lib
@pytest.mark.parametrize("case,status", [
    (dict(q=0), -1), (dict(C_in=0), -1), (dict(h_out=0), -1),
    (dict(d=24), -4), (dict(d=1040), -4), (dict(B=0), -2), (dict(dtype=5), -3),
    (dict(C_in=FAKE + 8), -5), (dict(igate=FAKE + 2), -5),
    (dict(n_out=FAKE), -9),                       # n_out is n_in
    (dict(m_out=FAKE + (1 << 16)), -9),           # m_out is m_in
    (dict(C_out=FAKE + (1 << 12)), -9),           # C_out overlaps C_in, shifted
    (dict(forget=2), -10),
])
def test_recurrent_step_rejects_before_device_work(case, status):
    lib = mlstm.load_library()
    args = dict(q=FAKE, k=FAKE, v=FAKE, igate=FAKE, fgate=FAKE,
                C_in=FAKE, n_in=FAKE, m_in=FAKE + (1 << 16),
                C_out=FAKE, n_out=FAKE + (1 << 24), m_out=FAKE + (1 << 25),
                h_out=FAKE, den_out=0, B=1, NH=1, d=64, dtype=1, forget=0)
    args.update(case)
    ptrs = ["q", "k", "v", "igate", "fgate", "C_in", "n_in", "m_in", "C_out", "n_out", "m_out",
            "h_out", "den_out"]
    st = lib.mlstm_recurrent_step(*[args[k] or None for k in ptrs], args["B"], args["NH"],
                                  args["d"], args["dtype"], args["forget"], None)
    assert st == status


@needs_lib
def test_training_entry_points_reject_unknown_forget_activation():
    lib = mlstm.load_library()
    assert lib.mlstm_parallel_fwd_train(*[FAKE] * 9, 1, 1, 64, 16, 1, 2, None) == -10
    assert lib.mlstm_parallel_bwd(*[FAKE] * 15, 1, 1, 64, 16, 1, 7, None) == -10
    # the activation is checked after the other arguments' own checks
    assert lib.mlstm_parallel_fwd_train(*[FAKE] * 8, None, 1, 1, 64, 16, 1, 0, None) == -1
    with pytest.raises(ValueError):
        mlstm._forget_code("tanh")


@needs_lib
def test_backward_rejects_head_dims_above_its_limit():
    lib = mlstm.load_library()
    # the backward takes every forward head dimension; d = 1040 or one not a
    # multiple of 16 is beyond every entry point
    assert lib.mlstm_parallel_bwd(*[FAKE] * 15, 1, 1, 64, 1040, 1, 0, None) == -4
    assert lib.mlstm_parallel_bwd(*[FAKE] * 15, 1, 1, 64, 1040, 0, 0, None) == -4
    assert lib.mlstm_parallel_bwd(*[FAKE] * 15, 1, 1, 64, 520, 0, 0, None) == -4
    # the one-wave MFMA kernel stops at 512; the selector is checked first
    assert lib.mlstm_causal_tiles(FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, FAKE, FAKE,
                                  1, 1, 64, 1024, 0, 5, None) == -8


def _addrs(names):
    """Distinct 16-byte-aligned fake addresses 16 MiB apart (never dereferenced)."""
    return {n: FAKE + (i + 1) * (1 << 24) for i, n in enumerate(names)}


@needs_lib
@pytest.mark.parametrize("alias", [("h_out", "q"), ("h_out", "v", 1024), ("m_out", "n_out"),
                                   ("n_out", "igate"), ("m_out", "fgate", 128)])
def test_forward_rejects_outputs_that_alias(alias):
    lib = mlstm.load_library()
    names = ["q", "k", "v", "igate", "fgate", "h_out", "m_out", "n_out"]
    a = _addrs(names)
    a[alias[0]] = a[alias[1]] + (alias[2] if len(alias) > 2 else 0)
    # B=1, NH=1, T=64, d=16, bf16: 2 KiB tensors, 256-byte gate rows
    assert lib.mlstm_parallel_fwd(*[a[n] for n in names], 1, 1, 64, 16, 1) == -9


@needs_lib
def test_other_entry_points_reject_outputs_that_alias():
    lib = mlstm.load_library()
    # gated forward: h~ onto h, and h onto the output gate
    names = ["q", "k", "v", "igate", "fgate", "ogate", "h_out", "htilde_out", "m_out", "n_out"]
    a = _addrs(names)
    b = dict(a, htilde_out=a["h_out"])
    assert lib.mlstm_parallel_fwd_gated(*[b[n] for n in names], 1, 1, 64, 16, 1, None) == -9
    b = dict(a, h_out=a["ogate"])
    assert lib.mlstm_parallel_fwd_gated(*[b[n] for n in names], 1, 1, 64, 16, 1, None) == -9
    # training forward: b onto n
    names = ["q", "k", "v", "igate", "fgate", "h_out", "m_out", "n_out", "b_out"]
    a = _addrs(names)
    b = dict(a, b_out=a["n_out"])
    assert lib.mlstm_parallel_fwd_train(*[b[n] for n in names], 1, 1, 64, 16, 1, 0, None) == -9
    # backward: dq onto q, df~ onto f~
    names = ["q", "k", "v", "igate", "fgate", "h", "m", "n", "b", "dh", "dq", "dk", "dv",
             "digate", "dfgate"]
    a = _addrs(names)
    for out, inp in (("dq", "q"), ("dfgate", "fgate"), ("dk", "dv")):
        b = dict(a, **{out: a[inp]})
        assert lib.mlstm_parallel_bwd(*[b[n] for n in names], 1, 1, 64, 16, 1, 0, None) == -9
    # staged: m onto i~, m inside the workspace, h onto q
    ws = FAKE + (1 << 30)
    wsb = lib.mlstm_workspace_bytes(1, 1, 64)
    a = _addrs(["igate", "fgate", "m"])
    assert lib.mlstm_gate_scan(a["igate"], a["fgate"], a["igate"], ws, wsb, 1, 1, 64, 16, 0,
                               None) == -9
    assert lib.mlstm_gate_scan(a["igate"], a["fgate"], ws + 256, ws, wsb, 1, 1, 64, 16, 0,
                               None) == -9
    a = _addrs(["q", "k", "v", "m", "h", "n"])
    assert lib.mlstm_causal_tiles(a["q"], a["k"], a["v"], a["m"], ws, wsb, a["q"], a["n"],
                                  1, 1, 64, 16, 1, 0, None) == -9


@needs_lib
def test_noalloc_entry_point_rejects_before_device_work():
    lib = mlstm.load_library()
    lib.mlstm_parallel_fwd_noalloc.argtypes = [ctypes.c_void_p] * 8 + [ctypes.c_int64] * 4 + [
        ctypes.c_int, ctypes.c_void_p]
    names = ["q", "k", "v", "igate", "fgate", "h_out", "m_out", "n_out"]
    a = {n: FAKE + (i + 1) * (1 << 40) for i, n in enumerate(names)}
    call = lambda B, NH, T, d, **kw: lib.mlstm_parallel_fwd_noalloc(
        *[kw.get(n, a[n]) for n in names], B, NH, T, d, 1, None)
    limit = 16 << 20
    # the fixed workspace: 32 heads of 2048 fit; 128 heads of 8192 do not
    assert lib.mlstm_workspace_bytes(8, 4, 2048) <= limit
    assert lib.mlstm_workspace_bytes(16, 8, 8192) > limit
    assert call(16, 8, 8192, 64) == -11
    assert call(1, 1, 1 << 20, 64) == -11
    # the ordinary checks come first
    assert call(16, 8, 8192, 24) == -4
    assert call(1, 1, 64, 16, q=None) == -1
    assert call(1, 1, 64, 16, h_out=a["q"]) == -9
