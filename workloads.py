"""Seeded synthetic inputs for causal RoPE attention.

This module only draws random numbers and rounds them to the working dtype; it
holds none of the attention arithmetic. Both the GPU tests/benchmark and the
float64 oracle take their inputs from here, so they see the exact same values.

Recipe (identical for every workload): numpy's PCG64 generator seeded with the
given seed (0 by default) draws float64 arrays of shape [B, H, T, D] in C order,
in the order q, k, v, dO. They are then rounded to the workload dtype with
round-to-nearest-even (torch's cast). "N(0, s^2)" is a normal with standard
deviation s; "U(-1, 1)" is uniform on [-1, 1).

The workload shapes are the attention layer of the GPT-2-small-scale model the
pages describe (12 heads, model width 768, so head dimension 64), plus a
head-dimension-128 variant with the same model width.
"""

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    D: int
    dtype: str                 # "bf16", "f16" or "f32"
    qk: tuple = ("normal", 1.0)
    v: tuple = ("normal", 1.0)
    do: tuple = ("normal", 0.1)
    base: float = 10000.0

    @property
    def shape(self):
        return (self.B, self.H, self.T, self.D)


WORKLOADS = {
    w.name: w
    for w in (
        # tiny fp32 case the oracle finishes instantly; every tensor N(0, 1)
        Workload("tiny_f32_b1h2t64d64", 1, 2, 64, 64, "f32",
                 do=("normal", 1.0)),
        # one attention layer of the 12-head, 768-wide model at T = 1024
        Workload("gpt2s_bf16_b8h12t1024d64", 8, 12, 1024, 64, "bf16"),
        # the same layer with fp16 tensors
        Workload("gpt2s_f16_b8h12t1024d64", 8, 12, 1024, 64, "f16"),
        # byte-level long context, most key tiles above the diagonal skipped
        Workload("longctx_bf16_b2h12t4096d64", 2, 12, 4096, 64, "bf16"),
        # peaky logits (q, k with std 3) and bounded values
        Workload("peaky_bf16_b16h12t2048d64", 16, 12, 2048, 64, "bf16",
                 qk=("normal", 3.0), v=("uniform", 1.0)),
        # wide heads (6 x 128 = 768) at T = 8192
        Workload("wide_bf16_b1h6t8192d128", 1, 6, 8192, 128, "bf16"),
        # generation over a key/value cache: 8 sequences of the 12-head layer with
        # 1024 cached positions; the step's query is q at the last position
        Workload("decode_bf16_b8h12t1024d64", 8, 12, 1024, 64, "bf16"),
    )
}

# the per-layer kernels next to attention, over the headline batch's B*T = 8192
# token rows: RMSNorm over the model width 768, SwiGLU over a feed-forward width
# of 2048 (two thirds of 4 x 768, the usual SwiGLU sizing)
LAYER_WORKLOADS = {
    "rmsnorm_bf16_n8192c768": ("rmsnorm", 8192, 768, "bf16"),
    "swiglu_bf16_n8192f2048": ("swiglu", 8192, 2048, "bf16"),
}


def layer_inputs(kind, N, width, dtype, seed=0):
    """Seeded inputs of a per-layer kernel as CPU torch tensors in `dtype`.

    rmsnorm (width C): x, r ~ N(0, 1) [N, C]; g ~ 1 + N(0, 0.1^2) [C];
    dy, dres ~ N(0, 0.1^2) [N, C]. swiglu (width F): u ~ N(0, 1) [N, 2F];
    dout ~ N(0, 0.1^2) [N, F]. Drawn in that order with PCG64(seed).
    """
    import torch
    rng = np.random.default_rng(seed)
    td = torch_dtype(dtype)
    t = lambda a: torch.from_numpy(a).to(td)
    if kind == "rmsnorm":
        x = rng.standard_normal((N, width))
        r = rng.standard_normal((N, width))
        g = 1.0 + 0.1 * rng.standard_normal(width)
        dy = 0.1 * rng.standard_normal((N, width))
        dres = 0.1 * rng.standard_normal((N, width))
        return dict(x=t(x), r=t(r), g=t(g), dy=t(dy), dres=t(dres))
    if kind == "swiglu":
        u = rng.standard_normal((N, 2 * width))
        dout = 0.1 * rng.standard_normal((N, width))
        return dict(u=t(u), dout=t(dout))
    raise ValueError(f"unknown layer kind {kind!r}")


# the workload the throughput figure is quoted on
HEADLINE = "gpt2s_bf16_b8h12t1024d64"
TINY = "tiny_f32_b1h2t64d64"


def _draw(rng, kind, shape):
    dist, scale = kind
    if dist == "normal":
        return scale * rng.standard_normal(shape)
    if dist == "uniform":
        return rng.uniform(-scale, scale, shape)
    raise ValueError(f"unknown distribution {dist!r}")


def draw(shape, qk=("normal", 1.0), v=("normal", 1.0), do=("normal", 0.1), seed=0):
    """float64 q, k, v, dO of the given [B, H, T, D] shape, drawn in that order."""
    rng = np.random.default_rng(seed)
    q = _draw(rng, qk, shape)
    k = _draw(rng, qk, shape)
    vv = _draw(rng, v, shape)
    d = _draw(rng, do, shape)
    return q, k, vv, d


def torch_dtype(dtype):
    import torch
    return {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]


def make(workload, seed=0, shape=None):
    """Inputs for a workload as CPU torch tensors in the workload dtype.

    Returns dict(q, k, v, do). `shape` overrides the workload's [B, H, T, D]
    (same distributions) for parity cases at other sizes.
    """
    import torch
    w = WORKLOADS[workload] if isinstance(workload, str) else workload
    shp = tuple(shape) if shape is not None else w.shape
    arrs = draw(shp, w.qk, w.v, w.do, seed)
    td = torch_dtype(w.dtype)
    return {n: torch.from_numpy(a).to(td) for n, a in zip(("q", "k", "v", "do"), arrs)}


def as_float64(t):
    """Exact float64 copy of a (bf16, fp16 or fp32) CPU tensor, as a numpy array."""
    import torch
    return t.detach().to("cpu", torch.float64).numpy()
