"""Seeded synthetic inputs for the parallel mLSTM forward pass.

This module only draws random numbers and rounds them to the storage type; it
holds none of the method's arithmetic.  Both the GPU path (tests, benchmark)
and the CPU oracle receive exactly the arrays it returns.

Recipe (one ``numpy.random.Generator(PCG64(seed))`` per call):
  1. q, k, v: each ``standard_normal((B, NH, T, d), dtype=float32)``, drawn in
     that order; for bf16 workloads rounded to bfloat16 (round to nearest even)
     on the host, so both sides see the identical bf16 values.
  2. igate (i~): float64 draws cast to float32, shape (B, NH, T).
  3. fgate (f~): float64 draws cast to float32, shape (B, NH, T).
  4. Optionally, exactly round(frac * B * NH * T) fgate entries chosen without
     replacement (after all other draws) are overwritten with a fixed value.
A normal draw N(mu, s) uses s as the standard deviation.

The named workloads are the shapes of the xLSTM language-model layers and the
stress cases this library is measured and checked on; the data is synthetic
(Gaussian activations stand in for projected text embeddings).
"""

import numpy as np

# name -> (B, NH, T, d, dtype, igate law, fgate law, fgate floor)
WORKLOADS = {
    # one tiny head in fp32; also small enough for the recurrent form
    "tiny_fp32": dict(B=1, NH=1, T=64, d=16, dtype="fp32",
                      igate=("normal", 0.0, 1.0), fgate=("normal", 3.0, 1.0)),
    # small, launch-bound
    "small_bf16": dict(B=4, NH=4, T=512, d=64, dtype="bf16",
                       igate=("normal", 0.0, 2.0), fgate=("normal", 3.0, 1.5)),
    # ~125M-parameter xLSTM mLSTM layer: embed 768, x2 up-projection -> 1536,
    # 4 heads of 384, context 2048, batch 8
    "xlstm125m_layer": dict(B=8, NH=4, T=2048, d=384, dtype="bf16",
                            igate=("normal", 0.0, 1.0), fgate=("normal", 3.0, 1.0)),
    # ~1.3B-parameter layer: embed 2048, inner 4096, 4 heads of 1024 run as
    # 8 independent sub-heads of 512, context 2048, batch 4
    "xlstm1p3b_layer": dict(B=4, NH=8, T=2048, d=512, dtype="bf16",
                            igate=("normal", 0.0, 1.0), fgate=("normal", 3.0, 1.0)),
    # the same layer with true heads of 1024 (4 heads, one normalizer each)
    "xlstm1p3b_layer_d1024": dict(B=4, NH=4, T=2048, d=1024, dtype="bf16",
                                  igate=("normal", 0.0, 1.0), fgate=("normal", 3.0, 1.0)),
    # long-context stabilization stress: input gates across the exp overflow
    # range, fast and occasionally near-total forgetting
    "long_context_16k": dict(B=1, NH=8, T=16384, d=256, dtype="bf16",
                             igate=("uniform", -20.0, 20.0), fgate=("normal", 0.0, 4.0),
                             fgate_floor=(0.01, -30.0)),
}


def round_bf16(x):
    """Round float32 values to the nearest bfloat16 (ties to even); float32 out."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    return u.view(np.float32).reshape(x.shape)


def _draw(rng, law, shape):
    kind, a, b = law
    if kind == "normal":
        return (a + b * rng.standard_normal(shape)).astype(np.float32)
    if kind == "uniform":
        return rng.uniform(a, b, shape).astype(np.float32)
    if kind == "const":
        return np.full(shape, a, dtype=np.float32)
    raise ValueError(f"unknown law {kind!r}")


def make(spec, seed=0):
    """Draw one batch of inputs.

    ``spec`` is a workload name or a dict with keys B, NH, T, d, dtype
    ("fp32" | "bf16"), igate, fgate (laws ``(kind, a, b)`` with kind
    "normal" | "uniform" | "const") and optional fgate_floor ``(frac, value)``.
    Returns a dict with float32 arrays q, k, v [B,NH,T,d] (bf16-representable
    for bf16), igate, fgate [B,NH,T], and the resolved spec under "spec".
    """
    if isinstance(spec, str):
        name = spec
        spec = dict(WORKLOADS[spec])
        spec["name"] = name
    else:
        spec = dict(spec)
        spec.setdefault("name", "custom")
    B, NH, T, d = spec["B"], spec["NH"], spec["T"], spec["d"]
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((B, NH, T, d), dtype=np.float32)
    k = rng.standard_normal((B, NH, T, d), dtype=np.float32)
    v = rng.standard_normal((B, NH, T, d), dtype=np.float32)
    if spec["dtype"] == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    elif spec["dtype"] != "fp32":
        raise ValueError(f"unknown dtype {spec['dtype']!r}")
    igate = _draw(rng, spec["igate"], (B, NH, T))
    fgate = _draw(rng, spec["fgate"], (B, NH, T))
    floor = spec.get("fgate_floor")
    if floor is not None:
        frac, value = floor
        count = int(round(frac * B * NH * T))
        idx = rng.choice(B * NH * T, size=count, replace=False)
        fgate.reshape(-1)[idx] = np.float32(value)
    return dict(q=q, k=k, v=v, igate=igate, fgate=fgate, spec=spec)


def make_ogate(spec, seed=0, loc=0.0, scale=2.0):
    """Output gate pre-activations O~ [B,NH,T,d] for a drawn batch's spec.

    Drawn from a generator of its own, seeded (seed, 78), so that adding an
    output gate never changes the other inputs of the same seed.  N(loc, scale),
    float32, rounded to bf16 for bf16 workloads.
    """
    B, NH, T, d = spec["B"], spec["NH"], spec["T"], spec["d"]
    rng = np.random.Generator(np.random.PCG64([seed, 78]))
    o = (loc + scale * rng.standard_normal((B, NH, T, d))).astype(np.float32)
    return round_bf16(o) if spec["dtype"] == "bf16" else o


def counted_flops(B, NH, T, d):
    """Causal work counted as 2 * T^2 * d per head (both contractions, causal half)."""
    return 2.0 * T * T * d * B * NH
