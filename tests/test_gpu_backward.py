"""GPU parity of the backward (gdn_bwd, scalar gate) against the fp64 autograd oracle
(oracle/backward.py), through the C ABI.

Bound per gradient tensor: max|delta| <= tol * RMS(oracle gradient), tol 1e-4 for fp32 inputs
and 2e-2 for bf16 inputs (the forward's bounds).  The chunk states are recomputed by the forward's
main pass, the reverse state-gradient scan of bf16 inputs runs on the matrix cores with bf16 operand
pairs (as the forward), the rest in fp32."""
import numpy as np
import pytest
import torch

from chunkwise_linear_attention_chunk_amd import bwd, synth
from oracle.backward import gdn_backward
from parity_util import rel_max_err

pytestmark = pytest.mark.gpu
f64 = synth.to_f64
TOL = {"fp32": 1e-4, "bf16": 2e-2}


def _check(x, tol, label, seed=0, dht=True, tol_dg=None):
    rng = np.random.default_rng(1000 + seed)
    dt = x["q"].dtype
    do = torch.from_numpy(rng.standard_normal(tuple(x["v"].shape)).astype(np.float32)).to(dt)
    N, H, D, Dv = x["n_seqs"], x["v"].shape[2], x["q"].shape[3], x["v"].shape[3]
    dh = torch.from_numpy(rng.standard_normal((N, H, D, Dv)).astype(np.float32)) if dht else None
    dev = torch.device("cuda:0")
    t = lambda a: None if a is None else a.to(dev)
    gr = bwd(t(x["q"]), t(x["k"]), t(x["v"]), t(x["g"]), t(x["beta"]), t(do), scale=x["scale"],
             initial_state=t(x["h0"]), dht=t(dh), cu_seqlens=x["cu_seqlens"])
    torch.cuda.synchronize()
    cu = None if x["cu_seqlens"] is None else x["cu_seqlens"].numpy()
    r = gdn_backward(*(f64(x[n]) for n in ("q", "k", "v", "g", "beta")), x["scale"], f64(do), f64(x["h0"]),
                     f64(dh), cu_seqlens=cu)
    for n in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        got = f64(gr[n].cpu())
        assert np.isfinite(got).all(), f"{label} {n}: non-finite"
        e = rel_max_err(got, r[n])
        t = tol_dg if (n == "dg" and tol_dg is not None) else tol
        print(f"[parity] backward {label} {n}: max|d|/rms = {e:.3e} (tol {t})", flush=True)
        assert e <= t, f"{label} {n}: {e:.3e} > {t}"


@pytest.mark.parametrize("T", [1, 64, 150])
def test_backward_fp32(T):
    x = synth.make_inputs(synth.workload("tiny_fp32", B=2, H=2, T=T, h0=True, seed=600 + T))
    _check(x, TOL["fp32"], f"fp32 T={T}", seed=T)


def test_backward_fp32_head_dim_128_grouped_heads():
    x = synth.make_inputs(synth.workload("tiny_fp32", B=1, H=4, H_qk=2, D=128, T=130, h0=True, seed=610))
    _check(x, TOL["fp32"], "fp32 D=128 H_v=4 H_qk=2", seed=1)


def test_backward_fp32_no_initial_state_no_dht():
    x = synth.make_inputs(synth.workload("tiny_fp32", B=1, H=2, T=100, seed=611))
    _check(x, TOL["fp32"], "fp32 h0=0 dht=0", seed=2, dht=False)


def test_backward_bf16():
    x = synth.make_inputs(synth.workload("qwen3next_bf16", B=1, H=2, T=300, h0=True, seed=612))
    _check(x, TOL["bf16"], "bf16", seed=3)


@pytest.mark.parametrize("mu", [-7.0, None], ids=["weak", "none"])
def test_backward_bf16_many_chunks_slow_decay(mu):
    # the reverse scan carries dS over 21 chunks with weak decay, or none
    x = synth.make_inputs(synth.workload("qwen3next_bf16", B=1, H=2, T=64 * 20 + 17, mu=mu, h0=True, seed=614))
    _check(x, TOL["bf16"], f"bf16 T=1297 mu={mu}", seed=5)


def test_backward_bf16_head_dim_64_grouped_heads():
    x = synth.make_inputs(synth.workload("qwen3next_bf16", B=2, H=4, H_qk=2, D=64, T=200, h0=True, seed=615))
    _check(x, TOL["bf16"], "bf16 D=64 H_v=4 H_qk=2", seed=6)


def test_backward_packed():
    x = synth.make_inputs(synth.workload("varlen_bf16", n_seqs=4, lens=(1, 0, 130, 64), H=2, h0=True, seed=613))
    _check(x, TOL["bf16"], "bf16 packed", seed=4)


@pytest.mark.parametrize("T", [1, 64, 150])
def test_backward_per_channel_fp32(T):
    x = synth.make_inputs(synth.workload("tiny_fp32", B=2, H=2, T=T, gate="channel", h0=True, seed=620 + T))
    _check(x, TOL["fp32"], f"KDA fp32 T={T}", seed=10 + T)


def test_backward_per_channel_fp32_head_dim_128_grouped_heads():
    x = synth.make_inputs(synth.workload("tiny_fp32", B=1, H=4, H_qk=2, D=128, T=100, gate="channel", h0=True,
                                         seed=630))
    _check(x, TOL["fp32"], "KDA fp32 D=128 H_v=4 H_qk=2", seed=11)


def test_backward_per_channel_bf16():
    x = synth.make_inputs(synth.workload("kda_bf16", B=1, H=2, T=200, h0=True, seed=631))
    _check(x, TOL["bf16"], "KDA bf16", seed=12)


def test_backward_per_channel_bf16_head_dim_64_grouped_heads():
    x = synth.make_inputs(synth.workload("kda_bf16", B=2, H=4, H_qk=2, D=64, T=200, h0=True, seed=633))
    _check(x, TOL["bf16"], "KDA bf16 D=64 H_v=4 H_qk=2", seed=14)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("dk,dv", [(128, 64), (64, 128)])
def test_backward_bf16_key_and_value_dims_differ(gate, dk, dv):
    from test_gpu_parity import _dims
    name = "qwen3next_bf16" if gate == "scalar" else "kda_bf16"
    x = _dims(synth.make_inputs(synth.workload(name, B=1, H=2, T=64 * 3 + 29, h0=True, seed=634 + dk)), dk, dv)
    _check(x, TOL["bf16"], f"{gate} bf16 D_k={dk} D_v={dv}", seed=15)


def test_backward_per_channel_packed():
    x = synth.make_inputs(synth.workload("kda_bf16", B=1, n_seqs=4, lens=(1, 0, 130, 64), H=2, h0=True, seed=632))
    _check(x, TOL["bf16"], "KDA bf16 packed", seed=13, dht=False)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("mu", [1.0, -6.0])
def test_backward_fp32_gate_strengths(gate, mu):
    # strong decay (about -1.3 per token: a chunk spans ~e^-80) and weak decay (~2.5e-3 per token);
    # the per-channel P splits its decay factors within 16-token blocks, which strong gates stress
    x = synth.make_inputs(synth.workload("tiny_fp32", B=1, H=2, T=150, gate=gate, mu=mu, h0=True,
                                         seed=640 + int(mu) + (10 if gate == "channel" else 0)))
    _check(x, TOL["fp32"], f"{gate} fp32 mu={mu}", seed=20 + int(mu))


# --------------------------------------------------------------------------- full sizes, sampled
# The backward of the Qwen3-Next-shaped and KDA-shaped workloads at their full sizes, in the
# launch configuration bench.py times, against the oracle on sampled (sequence, head) slices
# (heads are independent).  For the KDA shape the oracle takes one head's last `suffix` tokens: the
# gradients of those tokens depend only on them, on dht and on the state entering them, which the
# C token recurrence gives from the prefix (dh0 would need the whole reverse pass and is not
# compared there).
from oracle.recurrent import gdn_recurrent


def _check_sampled(x, tol, label, b, heads, suffix=None, gate="scalar", seed=0):
    rng = np.random.default_rng(2000 + seed)
    dt = x["q"].dtype
    do = torch.from_numpy(rng.standard_normal(tuple(x["v"].shape)).astype(np.float32)).to(dt)
    B, T, H = x["q"].shape[0], x["q"].shape[1], x["v"].shape[2]
    D, Dv = x["q"].shape[3], x["v"].shape[3]
    dh = torch.from_numpy(rng.standard_normal((B, H, D, Dv)).astype(np.float32))
    dev = torch.device("cuda:0")
    t = lambda a: None if a is None else a.to(dev)
    gr = bwd(t(x["q"]), t(x["k"]), t(x["v"]), t(x["g"]), t(x["beta"]), t(do), scale=x["scale"],
             initial_state=t(x["h0"]), dht=t(dh))
    torch.cuda.synchronize()
    gr = {n: v.cpu() for n, v in gr.items()}
    assert x["q"].shape[2] == H, "sampled slices assume H_qk == H_v"
    for h in heads:
        sl = lambda a: f64(a[b:b + 1, :, h:h + 1])
        q, k, v, g, be, dos = tuple(sl(x[n]) for n in ("q", "k", "v", "g", "beta")) + (sl(do),)
        h0 = None if x["h0"] is None else f64(x["h0"][b:b + 1, h:h + 1])
        t0 = 0 if suffix is None else T - suffix
        if t0 > 0:   # the state entering the suffix, from the C token recurrence over the prefix
            _, h0 = gdn_recurrent(q[:, :t0], k[:, :t0], v[:, :t0], g[:, :t0], be[:, :t0], x["scale"], h0=h0, gate=gate)
        cut = lambda a: a[:, t0:]
        r = gdn_backward(*(cut(a) for a in (q, k, v, g, be)), x["scale"], cut(dos), h0,
                         f64(dh[b:b + 1, h:h + 1]))
        names = ("dq", "dk", "dv", "dg", "dbeta") + (("dh0",) if t0 == 0 else ())
        for n in names:
            got = f64(gr[n][b:b + 1, h:h + 1]) if n == "dh0" else f64(gr[n][b:b + 1, t0:, h:h + 1])
            assert np.isfinite(got).all(), f"{label} head {h} {n}: non-finite"
            e = rel_max_err(got, r[n])
            print(f"[parity] backward {label} b={b} head {h} {n}: max|d|/rms = {e:.3e} (tol {tol})", flush=True)
            assert e <= tol, f"{label} head {h} {n}: {e:.3e} > {tol}"


def test_backward_qwen3next_shape_full_size_sampled():
    x = synth.make_inputs(synth.workload("qwen3next_bf16", seed=630))     # B=4, H=16, T=4096, d=128
    _check_sampled(x, TOL["bf16"], "qwen3next_bf16 full size", b=2, heads=[3, 11], seed=1)


def test_backward_kda_shape_full_size_sampled():
    x = synth.make_inputs(synth.workload("kda_bf16", seed=631))           # B=2, H=32, T=16384, d=128
    _check_sampled(x, TOL["bf16"], "kda_bf16 full size, last 512 tokens", b=1, heads=[21], suffix=512,
                   gate="channel", seed=2)
