"""The allocation-free forward entry point (GPU): mlstm_parallel_fwd_noalloc
through the C ABI against mlstm_parallel_fwd_stream, which runs the same
kernels on a stream-ordered workspace.  Two calls in a row, the second on a
smaller problem, so the second runs on a workspace the first has written."""
import numpy as np
import pytest

from linear_recurrent_sequence_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from linear_recurrent_sequence_amd import mlstm


def _spec(B, NH, T, d, ig=("normal", 0.0, 1.0), fg=("normal", 3.0, 1.0), **kw):
    s = dict(B=B, NH=NH, T=T, d=d, dtype="bf16", igate=ig, fgate=fg)
    s.update(kw)
    return s


CASES = [
    # four or more 2048-position chunks: the two-pass scan and its chunk terms
    _spec(1, 4, 8200, 64, ig=("uniform", -20, 20), fg=("normal", 0, 4), fgate_floor=(0.01, -30.0)),
    _spec(2, 2, 3000, 128),  # smaller: only part of the workspace is rewritten
    # up to 2048 positions the pass is one kernel that needs no workspace
    _spec(8, 4, 2048, 384),  # the ~125M-parameter layer
    _spec(1, 1, 65, 64),
]


def _run_both(x):
    dev = torch.device("cuda", 0)
    q, k, v = (torch.from_numpy(x[n]).to(dev).to(torch.bfloat16).contiguous() for n in "qkv")
    ig = torch.from_numpy(x["igate"]).to(dev).contiguous()
    fg = torch.from_numpy(x["fgate"]).to(dev).contiguous()
    B, NH, T, _ = q.shape
    out = (torch.empty_like(q), torch.empty((B, NH, T), dtype=torch.float32, device=dev),
           torch.empty((B, NH, T), dtype=torch.float32, device=dev))
    mlstm.parallel_fwd_noalloc(q, k, v, ig, fg, out)
    ref = mlstm.parallel_fwd(q, k, v, ig, fg)
    torch.cuda.synchronize()
    return out, ref


def test_noalloc_matches_the_stream_entry_point_on_consecutive_calls():
    for i, s in enumerate(CASES):
        print("noalloc case", i, {k: s[k] for k in ("B", "NH", "T", "d")}, flush=True)
        x = W.make(s, seed=60 + i)
        out, ref = _run_both(x)
        for name, a, b in zip(("h", "m", "n"), out, ref):
            assert torch.equal(a, b), (i, name)
        assert torch.isfinite(out[0].float()).all()


@pytest.mark.parametrize("d", [16, 512])
def test_noalloc_single_launch_needs_no_workspace_at_any_size(d):
    """512 heads of 2048 need 21.5 MB of workspace in the two-launch form,
    beyond the fixed array, but run as one launch with none (the pair kernel
    at d = 16, the one-wave kernel at d = 512)."""
    x = W.make(_spec(32, 16, 2048, d), seed=70)
    out, ref = _run_both(x)
    for name, a, b in zip(("h", "m", "n"), out, ref):
        assert torch.equal(a, b), name


def test_noalloc_rejects_oversize_problems():
    dev = torch.device("cuda", 0)
    B, NH, T, d = 16, 8, 8192, 16  # 128 heads of 8192: beyond the fixed workspace
    q = torch.zeros((B, NH, T, d), dtype=torch.bfloat16, device=dev)
    g = torch.zeros((B, NH, T), dtype=torch.float32, device=dev)
    out = (torch.empty_like(q), torch.empty_like(g), torch.empty_like(g))
    with pytest.raises(mlstm.MlstmError) as e:
        mlstm.parallel_fwd_noalloc(q, q, q, g, g, out)
    assert e.value.status == -11
