"""GPU parity at the edges of the planning tables: more segments than the plan kernel ranks
(identity order past 1024), more sequences than it fills in shared memory (direct fill past 4096),
for the chunked forward, the decode path and the backward; and a long single sequence through
the decode path.  Sampled sequences are compared with the fp64 oracle one by one."""
import numpy as np
import pytest
import torch

from chunkwise_linear_attention_chunk_amd import bwd, synth
from oracle.backward import gdn_backward
from parity_util import TOL, check, rel_max_err

pytestmark = pytest.mark.gpu
f64 = synth.to_f64


def _packed(n, hi, seed, H=2, D=64, dtype="varlen_bf16", h0=True):
    lens = tuple(int(v) for v in np.random.default_rng(seed).integers(0, hi + 1, n))
    return synth.make_inputs(synth.workload(dtype, n_seqs=n, lens=lens, H=H, D=D, h0=h0, seed=seed))


def _sample(x, k=6):
    cu = x["cu_seqlens"].numpy()
    lens = np.diff(cu)
    n = len(lens)
    picks = {0, n - 1, int(np.argmax(lens)), n // 2}
    picks |= {int(i) for i in np.flatnonzero(lens == 0)[:1]}
    return sorted(picks)[:k]


def test_more_segments_than_the_ranked_order():
    # 1500 one-chunk sequences (lengths 0..100): 1500 segments, past the 1024 the plan ranks
    x = _packed(1500, 100, seed=800)
    check(x, TOL["bf16"], seqs=_sample(x), label="1500 sequences")


def test_more_sequences_than_the_shared_fill():
    # 5000 sequences of 0..3 tokens: the chunk table is filled sequence by sequence
    x = _packed(5000, 3, seed=801, H=1)
    check(x, TOL["bf16"], seqs=_sample(x), label="5000 sequences")
    check(x, 1e-4, seqs=_sample(x), label="5000 sequences, decode", recurrent=True)


def test_decode_long_sequence():
    x = synth.make_inputs(synth.workload("qwen3next_bf16", B=1, H=2, D=64, T=2000, h0=True, seed=802))
    check(x, 1e-4, label="decode over 2000 tokens", recurrent=True)


def test_backward_many_packed_sequences():
    x = _packed(1100, 6, seed=803, H=1, dtype="tiny_fp32")
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(804)
    do = torch.from_numpy(rng.standard_normal(tuple(x["v"].shape)).astype(np.float32))
    gr = bwd(*(x[n].to(dev) for n in ("q", "k", "v", "g", "beta")), do.to(dev), scale=x["scale"],
             initial_state=x["h0"].to(dev), cu_seqlens=x["cu_seqlens"])
    torch.cuda.synchronize()
    ref = gdn_backward(*(f64(x[n]) for n in ("q", "k", "v", "g", "beta")), x["scale"], f64(do), f64(x["h0"]),
                       cu_seqlens=x["cu_seqlens"].numpy())
    for n in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        e = rel_max_err(f64(gr[n].cpu()), ref[n])
        print(f"[parity] backward 1100 sequences {n}: {e:.3e}", flush=True)
        assert e <= TOL["fp32"], f"{n}: {e:.3e}"
