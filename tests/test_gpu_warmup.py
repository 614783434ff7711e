"""GPU parity of warmup context parallelism (cp_mode "warmup"; FlashQLA announcement, section
"further optimisation through gate decay") through the C ABI.

With the default bound (2^-24) the warmup's error is far below the parity tolerance, so the GPU
result is checked against the exact fp64 recurrence at the usual bound (1e-4 * RMS fp32 inputs,
2e-2 * RMS bf16).  With a loose bound the approximation is visible, and the GPU result is checked
against the fp64 warmup oracle (oracle/warmup.py) on gates whose warmup lengths are far from a
rounding decision."""
import numpy as np
import pytest
import torch

from chunkwise_linear_attention_chunk_amd import synth
from oracle.warmup import warmup_cp
from parity_util import TOL, check, gpu_run, rel_max_err

pytestmark = pytest.mark.gpu
f64 = synth.to_f64


def _w(name, **kw):
    return synth.make_inputs(synth.workload(name, **kw))


def test_warmup_bf16_decaying_gates_match_exact():
    x = _w("qwen3next_bf16", B=1, H=4, T=20 * 64 + 17, h0=True, seed=500)
    check(x, TOL["bf16"], label="warmup bf16", cp_mode="warmup", cp_segment_chunks=4)


def test_warmup_without_decay_is_exact():
    # g == 0: no warmup is ever short enough, every segment restarts from h0 at its sequence start
    x = _w("tiny_fp32", B=2, H=2, T=9 * 64 + 5, mu=None, h0=True, seed=501)
    check(x, TOL["fp32"], label="warmup g=0", cp_mode="warmup", cp_segment_chunks=2)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_warmup_loose_bound_matches_warmup_oracle(gate):
    # constant log-gate -0.05 per token: a chunk decays by e^-3.2, the bound e^-8 takes W = 3 chunks
    # (W = 2 leaves e^-6.4); per channel one channel carries the slow rate, the rest decay faster
    x = _w("tiny_fp32", B=1, H=2, T=14 * 64 + 9, h0=True, gate=gate, seed=502)
    g = torch.full_like(x["g"], -0.05)
    if gate == "channel":
        g[..., 1:] = -0.3
    x["g"] = g
    tol = float(np.exp(-8.0))
    o_g, f_g = gpu_run(x, cp_mode="warmup", cp_segment_chunks=4, cp_warmup_tol=tol)
    o_r, f_r, W, _ = warmup_cp(*(f64(x[n]) for n in ("q", "k", "v", "g", "beta")), x["scale"], h0=f64(x["h0"]),
                               gate=gate, seg_chunks=4, tol=tol)
    assert {w for (n, j, h), w in W.items() if j > 0} == {3}
    eo, ef = rel_max_err(f64(o_g), o_r), rel_max_err(f64(f_g), f_r)
    print(f"[parity] warmup loose bound {gate}: {eo:.3e} {ef:.3e}", flush=True)
    assert eo <= TOL["fp32"] and ef <= TOL["fp32"]


def test_warmup_packed_ragged():
    x = _w("varlen_bf16", n_seqs=5, lens=(0, 1, 300, 1000, 9 * 64), H=3, h0=True, seed=503)
    check(x, TOL["bf16"], label="warmup packed", cp_mode="warmup", cp_segment_chunks=2)


def test_warmup_per_channel_gate():
    x = _w("kda_bf16", B=1, H=2, T=12 * 64, h0=True, seed=504)
    check(x, TOL["bf16"], label="warmup KDA", cp_mode="warmup", cp_segment_chunks=4)


def test_warmup_two_workgroups_per_cu_build():
    x = _w("qwen3next_bf16", B=8, H=16, T=8 * 64, seed=505)
    check(x, TOL["bf16"], batches=[0, 7], heads=[0, 5, 15], label="warmup, 1024 workgroups", cp_mode="warmup",
          cp_segment_chunks=4)


def test_warmup_longctx_full_size_sampled():
    # the long-context workload (one sequence, 4 heads, 1024 chunks) in warmup mode: two heads
    x = _w("longctx_bf16")
    check(x, TOL["bf16"], heads=[0, 3], label="longctx warmup (sampled heads)", cp_mode="warmup")
