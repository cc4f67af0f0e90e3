"""Thin ctypes binding over libmlstm.so (the C ABI in include/mlstm.h).

Argument marshalling only: every step of the forward pass runs in the HIP
kernels of the library.  PyTorch supplies device memory and the current
stream.  There is no fallback: if the library is missing or the tensors are
not on a GPU, the call raises.

    h, m, n = parallel_fwd(q, k, v, igate, fgate)

q, k, v: [B, NH, T, d] contiguous, float32 or bfloat16, on the current GPU.
igate, fgate: [B, NH, T] contiguous float32 (input / forget gate pre-activations).
Returns h~ (same dtype as q), m and n (float32), as defined by Eqs. 80, 84 and
86 of the xLSTM appendix ("Parallel mLSTM Backward Pass" restates the
stabilized forward pass).
"""

import contextlib
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmlstm.so")

MLSTM_FP32, MLSTM_BF16 = 0, 1
KERNELS = {"auto": 0, "mfma": 1, "vector": 2, "mfma_all_tiles": 3, "mfma_single": 4,
           "mfma_wide": 5}
FORGET_ACTIVATIONS = {"sigmoid": 0, "exp": 1}

_lib = None


class MlstmError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


def load_library():
    """Load libmlstm.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m linear_recurrent_sequence_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.mlstm_parallel_fwd.argtypes = [vp] * 8 + [i64] * 4 + [i32]
    lib.mlstm_parallel_fwd.restype = i32
    lib.mlstm_parallel_fwd_stream.argtypes = [vp] * 8 + [i64] * 4 + [i32, vp]
    lib.mlstm_parallel_fwd_stream.restype = i32
    lib.mlstm_parallel_fwd_noalloc.argtypes = [vp] * 8 + [i64] * 4 + [i32, vp]
    lib.mlstm_parallel_fwd_noalloc.restype = i32
    lib.mlstm_parallel_fwd_gated.argtypes = [vp] * 10 + [i64] * 4 + [i32, vp]
    lib.mlstm_parallel_fwd_gated.restype = i32
    lib.mlstm_recurrent_step.argtypes = [vp] * 13 + [i64] * 3 + [i32, i32, vp]
    lib.mlstm_recurrent_step.restype = i32
    lib.mlstm_parallel_fwd_train.argtypes = [vp] * 9 + [i64] * 4 + [i32, i32, vp]
    lib.mlstm_parallel_fwd_train.restype = i32
    lib.mlstm_parallel_bwd.argtypes = [vp] * 15 + [i64] * 4 + [i32, i32, vp]
    lib.mlstm_parallel_bwd.restype = i32
    lib.mlstm_workspace_bytes.argtypes = [i64] * 3
    lib.mlstm_workspace_bytes.restype = f
    lib.mlstm_gate_scan.argtypes = [vp] * 4 + [f] + [i64] * 4 + [i32, vp]
    lib.mlstm_gate_scan.restype = i32
    lib.mlstm_causal_tiles.argtypes = [vp] * 5 + [f] + [vp] * 2 + [i64] * 4 + [i32, i32, vp]
    lib.mlstm_causal_tiles.restype = i32
    lib.mlstm_strerror.argtypes = [i32]
    lib.mlstm_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def strerror(status):
    return load_library().mlstm_strerror(int(status)).decode()


def _dtype_code(t):
    if t.dtype == torch.float32:
        return MLSTM_FP32
    if t.dtype == torch.bfloat16:
        return MLSTM_BF16
    raise TypeError(f"q/k/v must be float32 or bfloat16, got {t.dtype}")


def _forget_code(forget):
    """The C-ABI code of a forget-gate activation name ("sigmoid" or "exp")."""
    if forget not in FORGET_ACTIVATIONS:
        raise ValueError(f"forget must be one of {tuple(FORGET_ACTIVATIONS)}, got {forget!r}")
    return FORGET_ACTIVATIONS[forget]


def _require(name, t, shape, dtype, device=None):
    """Raise unless ``t`` is a contiguous tensor of exactly ``shape`` and
    ``dtype`` (and, if ``device`` is given, on that GPU).  Every tensor handed
    to the C ABI goes through here first: a host pointer, a wrong element type
    or a short buffer would otherwise reach the kernels."""
    # the common case in one expression (each tensor attribute read costs the
    # host time of a small kernel launch); the messages below on failure
    if (isinstance(t, torch.Tensor) and t.dtype == dtype and t.shape == shape
            and t.is_contiguous() and (device is None or t.device == device)):
        if device is None or device.type == "cuda":
            return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None:
        _require_device(name, t, device)


def _require_device(name, t, device):
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (there is no CPU path), got {t.device}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other tensors on {device}")


def _require_workspace(ws, device):
    """A workspace: a contiguous 1-D uint8 GPU tensor on ``device`` (its size
    is checked by the library against mlstm_workspace_bytes)."""
    if not isinstance(ws, torch.Tensor) or ws.dim() != 1:
        raise ValueError("workspace must be a 1-D tensor (see alloc_workspace)")
    _require("workspace", ws, ws.shape, torch.uint8, device)


def _check_inputs(q, k, v, igate, fgate):
    if not isinstance(q, torch.Tensor):
        raise TypeError(f"q must be a torch.Tensor, got {type(q).__name__}")
    if q.dim() != 4:
        raise ValueError(f"q must be [B, NH, T, d], got shape {tuple(q.shape)}")
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"q/k/v must be float32 or bfloat16, got {q.dtype}")
    B, NH, T, d = q.shape
    named = (("q", q), ("k", k), ("v", v), ("igate", igate), ("fgate", fgate))
    for name, t in named[:3]:
        _require(name, t, q.shape, q.dtype)
    for name, t in named[3:]:
        _require(name, t, (B, NH, T), torch.float32)
    dev = q.device
    if dev.type == "cuda" and k.device == dev and v.device == dev and igate.device == dev \
            and fgate.device == dev:
        return B, NH, T, d
    for name, t in named:  # devices last: a malformed tensor is named first
        _require_device(name, t, dev)
    return B, NH, T, d


def _stream_ptr(device):
    """The current HIP stream of ``device`` (torch's raw-stream query where
    this build has it: it skips building a Stream object)."""
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return ctypes.c_void_p(raw(device.index if device.index is not None
                                   else torch.cuda.current_device()))
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _on(device):
    """torch.cuda.device(device), or nothing when it is already current."""
    if device.index is None or device.index == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(device)


def parallel_fwd(q, k, v, igate, fgate, out=None):
    """Stabilized parallel mLSTM forward for B x NH heads -> (h, m, n).

    ``out`` may be a tuple (h, m, n) of preallocated outputs.
    """
    lib = load_library()
    B, NH, T, d = _check_inputs(q, k, v, igate, fgate)
    if out is None:
        h = torch.empty_like(q)
        m = torch.empty((B, NH, T), dtype=torch.float32, device=q.device)
        n = torch.empty((B, NH, T), dtype=torch.float32, device=q.device)
    else:
        h, m, n = out
        _require("h", h, q.shape, q.dtype, q.device)
        _require("m", m, (B, NH, T), torch.float32, q.device)
        _require("n", n, (B, NH, T), torch.float32, q.device)
    with _on(q.device):
        st = lib.mlstm_parallel_fwd_stream(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), igate.data_ptr(), fgate.data_ptr(),
            h.data_ptr(), m.data_ptr(), n.data_ptr(), B, NH, T, d, _dtype_code(q),
            _stream_ptr(q.device))
    if st != 0:
        raise MlstmError(st, "mlstm_parallel_fwd")
    return h, m, n


def parallel_fwd_noalloc(q, k, v, igate, fgate, out):
    """parallel_fwd through mlstm_parallel_fwd_noalloc: the library allocates
    nothing (its workspace is a fixed per-GPU array, shared by every call on
    that GPU, so calls must not overlap).  ``out`` = (h, m, n) is required:
    this path allocates no outputs either."""
    lib = load_library()
    B, NH, T, d = _check_inputs(q, k, v, igate, fgate)
    h, m, n = out
    _require("h", h, q.shape, q.dtype, q.device)
    _require("m", m, (B, NH, T), torch.float32, q.device)
    _require("n", n, (B, NH, T), torch.float32, q.device)
    with _on(q.device):
        st = lib.mlstm_parallel_fwd_noalloc(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), igate.data_ptr(), fgate.data_ptr(),
            h.data_ptr(), m.data_ptr(), n.data_ptr(), B, NH, T, d, _dtype_code(q),
            _stream_ptr(q.device))
    if st != 0:
        raise MlstmError(st, "mlstm_parallel_fwd_noalloc")
    return h, m, n


def parallel_fwd_gated(q, k, v, igate, fgate, ogate, htilde=False):
    """Forward pass with the output gate of Eq. 78 fused into the epilogue.

    ogate: O~, same shape, dtype and device as q.  Returns (h, m, n), or
    (h, h_tilde, m, n) with ``htilde=True``, where h = sigmoid(O~) * h_tilde.
    """
    lib = load_library()
    B, NH, T, d = _check_inputs(q, k, v, igate, fgate)
    _require("ogate", ogate, q.shape, q.dtype, q.device)
    h = torch.empty_like(q)
    ht = torch.empty_like(q) if htilde else None
    m = torch.empty((B, NH, T), dtype=torch.float32, device=q.device)
    n = torch.empty((B, NH, T), dtype=torch.float32, device=q.device)
    with _on(q.device):
        st = lib.mlstm_parallel_fwd_gated(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), igate.data_ptr(), fgate.data_ptr(),
            ogate.data_ptr(), h.data_ptr(), ht.data_ptr() if htilde else None, m.data_ptr(),
            n.data_ptr(), B, NH, T, d, _dtype_code(q), _stream_ptr(q.device))
    if st != 0:
        raise MlstmError(st, "mlstm_parallel_fwd_gated")
    return (h, ht, m, n) if htilde else (h, m, n)


def workspace_bytes(B, NH, T):
    return int(load_library().mlstm_workspace_bytes(B, NH, T))


def alloc_workspace(B, NH, T, device):
    """A device workspace for gate_scan / causal_tiles (256-byte aligned)."""
    nbytes = workspace_bytes(B, NH, T)
    if nbytes == 0:
        raise ValueError("invalid sizes")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def gate_scan(igate, fgate, d, workspace, m=None, forget="sigmoid"):
    """Stage 1: m (Eq. 80) and the exponent terms, written into ``workspace``."""
    lib = load_library()
    if not isinstance(igate, torch.Tensor) or igate.dim() != 3:
        raise ValueError("igate must be a [B, NH, T] tensor")
    B, NH, T = igate.shape
    _require("igate", igate, (B, NH, T), torch.float32, igate.device)
    _require("fgate", fgate, (B, NH, T), torch.float32, igate.device)
    _require_workspace(workspace, igate.device)
    if m is None:
        m = torch.empty((B, NH, T), dtype=torch.float32, device=igate.device)
    else:
        _require("m", m, (B, NH, T), torch.float32, igate.device)
    with _on(igate.device):
        st = lib.mlstm_gate_scan(igate.data_ptr(), fgate.data_ptr(), m.data_ptr(),
                                 workspace.data_ptr(), workspace.numel(), B, NH, T, d,
                                 _forget_code(forget), _stream_ptr(igate.device))
    if st != 0:
        raise MlstmError(st, "mlstm_gate_scan")
    return m


def causal_tiles(q, k, v, m, workspace, kernel="auto", out=None):
    """Stage 2: h~ and n from q, k, v and the stage-1 results -> (h, n)."""
    lib = load_library()
    B, NH, T, d = _check_inputs(q, k, v, m, m)
    _require_workspace(workspace, q.device)
    if kernel not in KERNELS:
        raise ValueError(f"kernel must be one of {tuple(KERNELS)}, got {kernel!r}")
    if out is None:
        h = torch.empty_like(q)
        n = torch.empty((B, NH, T), dtype=torch.float32, device=q.device)
    else:
        h, n = out
        _require("h", h, q.shape, q.dtype, q.device)
        _require("n", n, (B, NH, T), torch.float32, q.device)
    with _on(q.device):
        st = lib.mlstm_causal_tiles(q.data_ptr(), k.data_ptr(), v.data_ptr(), m.data_ptr(),
                                    workspace.data_ptr(), workspace.numel(), h.data_ptr(),
                                    n.data_ptr(), B, NH, T, d, _dtype_code(q), KERNELS[kernel],
                                    _stream_ptr(q.device))
    if st != 0:
        raise MlstmError(st, "mlstm_causal_tiles")
    return h, n


def parallel_fwd_staged(q, k, v, igate, fgate, kernel="auto", forget="sigmoid"):
    """Both stages with an explicit workspace and a chosen tile kernel."""
    B, NH, T, d = _check_inputs(q, k, v, igate, fgate)
    ws = alloc_workspace(B, NH, T, q.device)
    m = gate_scan(igate, fgate, d, ws, forget=forget)
    h, n = causal_tiles(q, k, v, m, ws, kernel=kernel)
    return h, m, n


def recurrent_state(B, NH, d, device):
    """A fresh recurrent state (C = 0, n = 0, m = -inf), float32."""
    C = torch.zeros((B, NH, d, d), dtype=torch.float32, device=device)
    n = torch.zeros((B, NH, d), dtype=torch.float32, device=device)
    m = torch.full((B, NH), float("-inf"), dtype=torch.float32, device=device)
    return C, n, m


def recurrent_step(q, k, v, igate, fgate, state, out_state=None, den=False, forget="sigmoid"):
    """One stabilized recurrent step -> (h, new_state[, den]).

    q, k, v: [B, NH, d] (float32 or bfloat16); igate, fgate: [B, NH] float32;
    state = (C [B,NH,d,d], n [B,NH,d], m [B,NH]) float32.  ``out_state``
    receives the new state (its C may be the input C: updated in place); by
    default C is updated in place and new n, m are allocated.
    """
    lib = load_library()
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q must be a [B, NH, d] tensor")
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"q/k/v must be float32 or bfloat16, got {q.dtype}")
    B, NH, d = q.shape
    C, n, m = state
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require(name, t, q.shape, q.dtype, q.device)
    for name, t, shp in (("igate", igate, (B, NH)), ("fgate", fgate, (B, NH)),
                         ("C", C, (B, NH, d, d)), ("n", n, (B, NH, d)), ("m", m, (B, NH))):
        _require(name, t, shp, torch.float32, q.device)
    if out_state is None:
        out_state = (C, torch.empty_like(n), torch.empty_like(m))
    Co, no, mo = out_state
    for name, t, shp in (("C_out", Co, (B, NH, d, d)), ("n_out", no, (B, NH, d)),
                         ("m_out", mo, (B, NH))):
        _require(name, t, shp, torch.float32, q.device)
    h = torch.empty_like(q)
    dn = torch.empty((B, NH), dtype=torch.float32, device=q.device) if den else None
    with _on(q.device):
        st = lib.mlstm_recurrent_step(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), igate.data_ptr(), fgate.data_ptr(),
            C.data_ptr(), n.data_ptr(), m.data_ptr(), Co.data_ptr(), no.data_ptr(), mo.data_ptr(),
            h.data_ptr(), dn.data_ptr() if den else None, B, NH, d, _dtype_code(q),
            _forget_code(forget), _stream_ptr(q.device))
    if st != 0:
        raise MlstmError(st, "mlstm_recurrent_step")
    return (h, out_state, dn) if den else (h, out_state)


def parallel_fwd_train(q, k, v, igate, fgate, forget="sigmoid"):
    """Forward pass that also returns the row sums b -> (h, m, n, b)."""
    lib = load_library()
    B, NH, T, d = _check_inputs(q, k, v, igate, fgate)
    h = torch.empty_like(q)
    m, n, b = (torch.empty((B, NH, T), dtype=torch.float32, device=q.device) for _ in range(3))
    with _on(q.device):
        st = lib.mlstm_parallel_fwd_train(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), igate.data_ptr(), fgate.data_ptr(),
            h.data_ptr(), m.data_ptr(), n.data_ptr(), b.data_ptr(), B, NH, T, d, _dtype_code(q),
            _forget_code(forget), _stream_ptr(q.device))
    if st != 0:
        raise MlstmError(st, "mlstm_parallel_fwd_train")
    return h, m, n, b


def parallel_bwd(q, k, v, igate, fgate, h, m, n, b, dh, forget="sigmoid"):
    """Gradients (dq, dk, dv, digate, dfgate) of the forward pass given dh = dL/dh~."""
    lib = load_library()
    B, NH, T, d = _check_inputs(q, k, v, igate, fgate)
    for name, t in (("h", h), ("dh", dh)):
        _require(name, t, q.shape, q.dtype, q.device)
    for name, t in (("m", m), ("n", n), ("b", b)):
        _require(name, t, (B, NH, T), torch.float32, q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dig, dfg = torch.empty_like(igate), torch.empty_like(fgate)
    with _on(q.device):
        st = lib.mlstm_parallel_bwd(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), igate.data_ptr(), fgate.data_ptr(),
            h.data_ptr(), m.data_ptr(), n.data_ptr(), b.data_ptr(), dh.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dig.data_ptr(), dfg.data_ptr(),
            B, NH, T, d, _dtype_code(q), _forget_code(forget), _stream_ptr(q.device))
    if st != 0:
        raise MlstmError(st, "mlstm_parallel_bwd")
    return dq, dk, dv, dig, dfg

