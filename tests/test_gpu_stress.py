"""GPU parity under gates the workloads do not exercise, against the fp64 oracle.

The workloads' gates decay fast (about e^-11.7 per chunk for the scalar gate), so the state carried
between chunks, and the transition M of context parallelism, barely reach the output there.  These
cases take the long-context shape (B = 1, H = 4, d = 128, nonzero h0) with weak decay
(g = -softplus(N(-7, 1)), about -1e-3 per token) and with no decay at all (g == 0), through the
serial pass and through context parallelism with segments of 8 (automatic), 16 and 64 chunks, in
both forms of the pre-process, so that S* and M accumulate over many slowly decaying chunks and the
fix-up runs several steps (FlashQLA announcement, the CP pre-process and fix-up).  The full
long-context workload runs with weak decay on two sampled heads.

Per-channel gates that decay steeply inside a 16-token block (around -8 per token, and around -3
where only some blocks are steep) exercise the per-pair path of the per-chunk kernel, forward and
backward.
"""
import pytest
import torch

from chunkwise_linear_attention_chunk_amd import synth
from parity_util import TOL, check

pytestmark = pytest.mark.gpu


def _w(name, **kw):
    return synth.make_inputs(synth.workload(name, **kw))


@pytest.mark.parametrize("mu", [-7.0, None], ids=["weak", "none"])
@pytest.mark.parametrize("cp,seg,form", [("off", 0, "auto"), ("auto", 0, "auto"), ("on", 16, "chain"),
                                         ("on", 64, "chain"), ("on", 16, "xyz"), ("on", 64, "xyz")])
def test_longctx_shape_slow_decay(mu, cp, seg, form):
    x = _w("longctx_bf16", T=8192, mu=mu, seed=800)
    check(x, TOL["bf16"], label=f"B=1 H=4 T=8192 mu={mu} cp={cp} L={seg} {form}", cp_mode=cp, cp_segment_chunks=seg,
          cp_form=form)


@pytest.mark.parametrize("seg,form", [(0, "auto"), (16, "xyz")])
def test_longctx_workload_weak_decay_cp_sampled(seg, form):
    # (L = 16: the segment count that makes the automatic choice take the X/Y/Z pre-process)
    x = _w("longctx_bf16", mu=-7.0, seed=801)
    check(x, TOL["bf16"], heads=[0, 3], label=f"longctx_bf16 mu=-7 CP L={seg} {form} (sampled)", cp_mode="on",
          cp_segment_chunks=seg, cp_form=form)


@pytest.mark.parametrize("mu", [8.0, 3.0], ids=["steep", "mixed"])
def test_kda_steep_channel_gates(mu):
    x = _w("kda_bf16", B=2, H=3, T=64 * 5 + 23, mu=mu, h0=True, seed=810)
    check(x, TOL["bf16"], label=f"KDA bf16 mu={mu}")
    x = _w("tiny_fp32", B=1, H=2, D=128, T=64 * 3 + 9, gate="channel", mu=mu, h0=True, seed=811)
    check(x, TOL["fp32"], label=f"KDA fp32 mu={mu}")


def _dg_bound_fp32(g, C=64):
    """Bound on the fp32 backward's relative gate-gradient error from its chunk-local cumsum of the
    log-gates: every partial sum rounds with an error of at most half an ulp of the largest |G| of its
    chunk, so G_i - G_j is off by at most 2 C 2^-24 max|G|, and so is every factor e^(G_i - G_j)
    relatively.  With steep gates the gate gradient is itself of the size of those factors' terms,
    so that bound, not the fp32 tolerance, is what its relative error can be held to."""
    gc = torch.cumsum(g.double().reshape(g.shape[0], -1, C, *g.shape[2:]), dim=2)
    return max(1e-4, 2 * C * 2.0 ** -24 * float(gc.abs().max()))


@pytest.mark.parametrize("mu", [8.0, 3.0], ids=["steep", "mixed"])
def test_kda_steep_channel_gates_backward(mu):
    from test_gpu_backward import TOL as BTOL, _check
    x = _w("tiny_fp32", B=1, H=2, T=128, gate="channel", mu=mu, h0=True, seed=812)
    _check(x, BTOL["fp32"], f"KDA fp32 mu={mu}", seed=7, tol_dg=_dg_bound_fp32(x["g"]))
    x = _w("kda_bf16", B=1, H=2, T=200, mu=mu, h0=True, seed=813)
    _check(x, BTOL["bf16"], f"KDA bf16 mu={mu}", seed=8)
