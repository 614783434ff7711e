"""Seeded synthetic inputs for the gated-delta-rule prefill forward.

This module holds no arithmetic of the method itself: it only draws random
numbers and shapes them into the value distributions of the workloads (unit-norm
query/key rows, already-activated log-gates, sigmoid betas).  Both the oracle
side and the GPU side of the tests and the benchmark take their inputs from
here; it imports neither.

Draw order per workload (one ``numpy.random.default_rng(seed)``): sequence
lengths (packed workload only) -> q -> k -> v -> gate -> beta -> h0.

* q, k ~ N(0, 1), then divided by their L2 norm over the head dimension per
  (token, head), then cast to the input dtype (round-to-nearest-even for bf16);
* v ~ N(0, 1);
* log-gate g = -softplus(N(mu, 1)) computed in fp64 (fp32 tensor for the
  scalar gate; the input dtype for the per-channel gate);
* beta = sigmoid(N(0, 1));
* h0 ~ N(0, 0.1^2) in fp32 when the workload has an initial state.
"""
from dataclasses import dataclass, field, replace

import numpy as np
import torch

_DT = {"fp32": torch.float32, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    H: int
    D: int
    dtype: str                    # "fp32" | "bf16": q, k, v, beta, o (and gk for the channel gate)
    B: int = 1
    T: int = 0                    # per-sequence length for the batched form
    n_seqs: int = 0               # > 0: packed variable-length form (B == 1)
    len_range: tuple = (0, 0)     # inclusive integer range of packed lengths
    lens: tuple = ()              # explicit packed lengths (overrides len_range)
    gate: str = "scalar"          # "scalar" (GDN) | "channel" (KDA)
    mu: float = -2.0              # log-gate g = -softplus(N(mu, 1)); None => g == 0
    h0: bool = False
    seed: int = 0
    H_qk: int = 0                 # 0 => H (no grouped value heads)
    chunk_size: int = 64

    @property
    def hqk(self):
        return self.H_qk or self.H


# The five workloads the path is measured and checked on.
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", B=1, H=2, T=256, D=64, dtype="fp32", mu=-2.0),
    "qwen3next_bf16": Workload("qwen3next_bf16", B=4, H=16, T=4096, D=128, dtype="bf16", mu=-2.0),
    "longctx_bf16": Workload("longctx_bf16", B=1, H=4, T=65536, D=128, dtype="bf16", mu=-2.0, h0=True),
    "varlen_bf16": Workload("varlen_bf16", n_seqs=16, len_range=(256, 8192), H=16, D=128, dtype="bf16",
                            mu=-2.0, h0=True),
    "kda_bf16": Workload("kda_bf16", B=2, H=32, T=16384, D=128, dtype="bf16", gate="channel", mu=-3.0),
}


def workload(name, **overrides):
    return replace(WORKLOADS[name], **overrides) if overrides else WORKLOADS[name]


def _softplus(x):
    return np.logaddexp(0.0, x)


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def make_inputs(w: Workload):
    """Return a dict of CPU torch tensors (input dtypes) plus metadata for workload ``w``."""
    rng = np.random.default_rng(w.seed)
    if w.n_seqs:
        if w.lens:
            lens = np.asarray(w.lens, dtype=np.int64)
        else:
            lens = rng.integers(w.len_range[0], w.len_range[1] + 1, size=w.n_seqs)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        B, T, N = 1, int(cu[-1]), w.n_seqs
    else:
        cu = None
        B, T, N = w.B, w.T, w.B
    Hq, Hv, D = w.hqk, w.H, w.D
    dt = _DT[w.dtype]

    def cast(a, to):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(to)

    q = cast(_unit_rows(rng.standard_normal((B, T, Hq, D))), dt)
    k = cast(_unit_rows(rng.standard_normal((B, T, Hq, D))), dt)
    v = cast(rng.standard_normal((B, T, Hv, D)), dt)
    gshape = (B, T, Hv) if w.gate == "scalar" else (B, T, Hv, D)
    if w.mu is None:
        g = np.zeros(gshape)
    else:
        g = -_softplus(rng.standard_normal(gshape) + w.mu)
    g = cast(g, torch.float32 if w.gate == "scalar" else dt)
    beta = cast(1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, Hv)))), dt)
    h0 = cast(0.1 * rng.standard_normal((N, Hv, D, D)), torch.float32) if w.h0 else None
    return dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0,
                cu_seqlens=None if cu is None else torch.from_numpy(cu),
                scale=float(D) ** -0.5, gate=w.gate, chunk_size=w.chunk_size, n_seqs=N,
                tokens=B * T, workload=w)


def make_prologue_inputs(w: Workload, lower_bound=0.0, seed_offset=1000):
    """Raw inputs for the in-kernel prologue, shaped like workload ``w``: q and k rows of random
    lengths (Gaussian rows times exp(N(0, 0.5))), raw gate inputs ~ N(-1, 1), beta logits ~ N(0, 1),
    A_log = log U(0.1, 1) per value head and dt_bias ~ N(0, 0.3) ([H] or [H, D]).  v, h0 and the
    packed lengths are those of make_inputs(w).  Returns (inputs, prologue options)."""
    x = make_inputs(w)
    rng = np.random.default_rng(w.seed + seed_offset)
    dt = x["q"].dtype
    qs, gs = tuple(x["q"].shape), tuple(x["g"].shape)
    Hv, D = x["v"].shape[2], x["q"].shape[3]

    def cast(a, to):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(to)

    def rows():
        return rng.standard_normal(qs) * np.exp(0.5 * rng.standard_normal(qs[:-1] + (1,)))

    x = dict(x, q=cast(rows(), dt), k=cast(rows(), dt),
             g=cast(rng.standard_normal(gs) - 1.0, torch.float32 if w.gate == "scalar" else dt),
             beta=cast(rng.standard_normal(tuple(x["beta"].shape)), dt))
    pro = dict(qk_l2norm=True, beta_sigmoid=True,
               A_log=cast(np.log(rng.uniform(0.1, 1.0, Hv)), torch.float32),
               dt_bias=cast(0.3 * rng.standard_normal((Hv,) if w.gate == "scalar" else (Hv, D)), torch.float32),
               gate_lower_bound=float(lower_bound))
    return x, pro


def to_f64(x):
    """Exact upcast of a (CPU) torch tensor to a numpy fp64 array (None passes through)."""
    return None if x is None else x.detach().to("cpu", torch.float64).numpy()
