"""GPU parity of the token-by-token path (gdn_fwd_recurrent, the decode form) against the fp64
oracle, through the C ABI.

The kernel keeps the state and every product in fp32 and reads the inputs exactly (bf16 upcasts
without rounding), so its error is fp32 accumulation over D_k terms per token: the bound is
1e-4 * RMS for every dtype, on o before storage rounding and on the final state (a bf16 output
adds half a bf16 ulp per element, as for the chunked path)."""
import numpy as np
import pytest
import torch

from chunkwise_linear_attention_chunk_amd import fwd_recurrent, synth
from parity_util import check, oracle_run, rel_max_err

pytestmark = pytest.mark.gpu
TOL = 1e-4


def _w(name, **kw):
    return synth.make_inputs(synth.workload(name, **kw))


@pytest.mark.parametrize("T", [1, 2, 37, 64, 130])
def test_fp32_lengths(T):
    x = _w("tiny_fp32", B=3, T=T, h0=True, seed=400 + T)
    check(x, TOL, label=f"recurrent fp32 T={T}", recurrent=True)


def test_fp32_no_initial_state_head_dim_128():
    x = _w("tiny_fp32", B=2, H=3, D=128, T=50, seed=410)
    check(x, TOL, label="recurrent fp32 D=128", recurrent=True)


@pytest.mark.parametrize("mu", [None, 2.0])
def test_fp32_gate_strengths(mu):
    x = _w("tiny_fp32", B=1, H=2, T=90, h0=True, mu=mu, seed=411)
    check(x, TOL, label=f"recurrent fp32 mu={mu}", recurrent=True)


def test_bf16_decode_batch():
    # one token per sequence: the decode step on a Qwen3-Next-shaped head set
    x = _w("qwen3next_bf16", B=64, H=16, T=1, h0=True, seed=412)
    check(x, TOL, label="recurrent bf16 decode B=64", recurrent=True)


@pytest.mark.parametrize("D", [64, 128])
def test_bf16_multi_token(D):
    x = _w("qwen3next_bf16", B=2, H=3, D=D, T=64, h0=True, seed=413)
    check(x, TOL, label=f"recurrent bf16 T=64 D={D}", recurrent=True)


def test_grouped_heads():
    x = _w("qwen3next_bf16", B=2, H=4, H_qk=2, T=20, h0=True, seed=414)
    check(x, TOL, label="recurrent H_v=4 H_qk=2", recurrent=True)


def test_packed_ragged_with_empty_sequences():
    x = _w("varlen_bf16", n_seqs=5, lens=(1, 0, 5, 64, 3), H=3, h0=True, seed=415)
    check(x, TOL, label="recurrent packed", recurrent=True)


@pytest.mark.parametrize("dt", ["kda_bf16", "tiny_fp32"])
def test_per_channel_gate(dt):
    kw = dict(B=2, H=2, T=33, h0=True, seed=416)
    x = _w(dt, gate="channel", **kw) if dt == "tiny_fp32" else _w(dt, **kw)
    check(x, TOL, label=f"recurrent per-channel {dt}", recurrent=True)


@pytest.mark.parametrize("name,lb", [("qwen3next_bf16", 0.0), ("qwen3next_bf16", -5.0), ("kda_bf16", 0.0),
                                     ("kda_bf16", -5.0)])
def test_prologue(name, lb):
    x, pro = synth.make_prologue_inputs(synth.workload(name, B=2, H=2, T=20, h0=True, seed=417), lb)
    check(x, TOL, prologue=pro, label=f"recurrent prologue {name} lb={lb}", recurrent=True)


def test_in_place_decode_steps_match_one_call():
    # T successive one-token calls updating the state in place == one call over T tokens == oracle
    x = _w("qwen3next_bf16", B=4, H=3, T=6, h0=True, seed=418)
    dev = torch.device("cuda:0")
    t = {n: x[n].to(dev) for n in ("q", "k", "v", "g", "beta")}
    state = x["h0"].to(dev).clone()
    outs = []
    for i in range(x["q"].shape[1]):
        o, fs = fwd_recurrent(*(t[n][:, i:i + 1].contiguous() for n in ("q", "k", "v", "g", "beta")),
                              scale=x["scale"], initial_state=state, state_in_place=True, out_dtype=torch.float32)
        assert fs.data_ptr() == state.data_ptr()
        outs.append(o)
    o_steps = torch.cat(outs, dim=1)
    o_one, f_one = fwd_recurrent(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=x["scale"],
                                 initial_state=x["h0"].to(dev), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o_steps, o_one), "stepwise and one-call outputs differ"
    assert torch.equal(state, f_one), "stepwise and one-call final states differ"
    o_r, f_r, pick = oracle_run(x)
    o_s, f_s = pick(o_one.cpu(), f_one.cpu())
    assert rel_max_err(o_s, o_r) <= TOL and rel_max_err(f_s, f_r) <= TOL


def test_recurrent_matches_chunked_path():
    # the two entry points compute the same operation (the chunked one to its bf16 bound)
    from parity_util import gpu_run
    x = _w("qwen3next_bf16", B=2, H=2, T=150, h0=True, seed=419)
    o_c, f_c = gpu_run(x, out_dtype=torch.float32)
    o_t, f_t = gpu_run(x, out_dtype=torch.float32, recurrent=True)
    assert rel_max_err(o_c.double().numpy(), o_t.double().numpy()) <= 2e-2
    assert rel_max_err(f_c.double().numpy(), f_t.double().numpy()) <= 2e-2
