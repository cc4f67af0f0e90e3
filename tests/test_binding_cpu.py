"""The Python binding validates every tensor it hands to the C ABI (CPU only).

A host tensor, a wrong element type, a wrong shape or a non-contiguous view
must raise in Python, before any pointer reaches the library: the kernels
would otherwise read or write out of range.  No call here reaches the HIP
runtime.
"""
import pytest
import torch

from linear_recurrent_sequence_amd import mlstm


class Stop(Exception):
    """Raised by the patched validator at the argument under test."""


def _t(*shape, dtype=torch.float32):
    return torch.zeros(shape, dtype=dtype)


def test_require_rejects_each_malformed_tensor():
    dev = torch.device("cuda", 0)
    good_shape, dt = (2, 3), torch.float32
    with pytest.raises(TypeError):
        mlstm._require("x", [0.0], good_shape, dt, dev)
    with pytest.raises(ValueError, match="shape"):
        mlstm._require("x", _t(3, 2), good_shape, dt, dev)
    with pytest.raises(ValueError, match="float32"):
        mlstm._require("x", _t(2, 3, dtype=torch.float64), good_shape, dt, dev)
    with pytest.raises(ValueError, match="contiguous"):
        mlstm._require("x", _t(3, 2).t(), good_shape, dt, dev)
    with pytest.raises(ValueError, match="GPU tensor"):
        mlstm._require("x", _t(2, 3), good_shape, dt, dev)
    with pytest.raises(ValueError, match="1-D"):
        mlstm._require_workspace(_t(4, 4, dtype=torch.uint8), dev)


def test_public_calls_reject_host_and_malformed_inputs():
    q = _t(1, 2, 64, 16, dtype=torch.bfloat16)
    g = _t(1, 2, 64)
    with pytest.raises(ValueError, match="GPU tensor"):
        mlstm.parallel_fwd(q, q, q, g, g)
    with pytest.raises(ValueError, match="shape"):
        mlstm.parallel_fwd(q, q, q, g[..., :10], g)
    with pytest.raises(TypeError):
        mlstm.parallel_fwd(q.to(torch.float16), q, q, g, g)
    with pytest.raises(ValueError, match="4"):
        mlstm.parallel_fwd(q[0], q, q, g, g)
    with pytest.raises(ValueError, match="bfloat16"):
        mlstm.parallel_fwd(q, q.float(), q, g, g)
    with pytest.raises(ValueError, match="contiguous"):
        mlstm.parallel_fwd(q, q.transpose(2, 3).contiguous().transpose(2, 3), q, g, g)
    with pytest.raises(ValueError):
        mlstm.gate_scan(g, g[..., :5], 16, _t(100, dtype=torch.uint8))
    with pytest.raises(ValueError):
        mlstm.recurrent_step(_t(1, 2, 16), _t(1, 2, 16), _t(1, 2, 16), _t(1, 2), _t(1, 2),
                             (_t(1, 2, 16, 16), _t(1, 2, 16), _t(1, 2)))


def _stop_at(monkeypatch, target):
    """Let every validation pass except the ones of argument ``target``."""
    def fake(name, t, *rest):
        if name == target:
            raise Stop(name)
    monkeypatch.setattr(mlstm, "_require", fake)
    monkeypatch.setattr(mlstm, "_require_device", fake)


def _forward_args():
    q = _t(1, 2, 64, 16, dtype=torch.bfloat16)
    return q, q.clone(), q.clone(), _t(1, 2, 64), _t(1, 2, 64)


# every tensor argument of every entry point, by the name the binding gives it
CALLS = {
    "parallel_fwd": (lambda a: mlstm.parallel_fwd(*a, out=(a[0].clone(), a[3].clone(),
                                                          a[3].clone())),
                     ["q", "k", "v", "igate", "fgate", "h", "m", "n"]),
    "parallel_fwd_gated": (lambda a: mlstm.parallel_fwd_gated(*a, a[0].clone()),
                           ["q", "k", "v", "igate", "fgate", "ogate"]),
    "gate_scan": (lambda a: mlstm.gate_scan(a[3], a[4], 16, _t(4096, dtype=torch.uint8),
                                            m=a[3].clone()),
                  ["igate", "fgate", "workspace", "m"]),
    "causal_tiles": (lambda a: mlstm.causal_tiles(a[0], a[1], a[2], a[3],
                                                  _t(4096, dtype=torch.uint8),
                                                  out=(a[0].clone(), a[3].clone())),
                     ["q", "k", "v", "igate", "workspace", "h", "n"]),
    "parallel_fwd_train": (lambda a: mlstm.parallel_fwd_train(*a),
                           ["q", "k", "v", "igate", "fgate"]),
    "parallel_bwd": (lambda a: mlstm.parallel_bwd(*a, a[0], a[3], a[3], a[3], a[0]),
                     ["q", "k", "v", "igate", "fgate", "h", "dh", "m", "n", "b"]),
    "recurrent_step": (lambda a: mlstm.recurrent_step(
        _t(1, 2, 16), _t(1, 2, 16), _t(1, 2, 16), _t(1, 2), _t(1, 2),
        (_t(1, 2, 16, 16), _t(1, 2, 16), _t(1, 2)),
        out_state=(_t(1, 2, 16, 16), _t(1, 2, 16), _t(1, 2))),
        ["q", "k", "v", "igate", "fgate", "C", "n", "m", "C_out", "n_out", "m_out"]),
}


@pytest.mark.parametrize("call,arg", [(c, a) for c, (_, args) in CALLS.items() for a in args])
def test_every_tensor_argument_is_validated_before_the_call(monkeypatch, call, arg):
    fn = CALLS[call][0]
    args = _forward_args()
    _stop_at(monkeypatch, arg)
    with pytest.raises(Stop):
        fn(args)
