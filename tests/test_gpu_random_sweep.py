"""GPU parity of gdn_fwd on a fixed-seed random sweep of configurations against the fp64 oracle:
gate kind, dtype, value and query/key head counts (grouped heads), key and value head dims, gate
strength, initial state, batched or packed (with empty, one-token and chunk-edge lengths), CP mode
(auto, off, exact with either pre-process form, warmup) and segment length, and the 16-column
recurrence build.  Each case is small enough for the oracle to run whole."""
import os
import random

import pytest
import torch

from chunkwise_linear_attention_chunk_amd import synth
from parity_util import TOL, check

pytestmark = pytest.mark.gpu


def _dims(x, dk, dv):
    y = dict(x)
    for n in ("q", "k"):
        a = x[n][..., :dk].double()
        y[n] = (a / a.norm(dim=-1, keepdim=True)).to(x[n].dtype)
    y["v"] = x["v"][..., :dv].contiguous()
    if x["gate"] == "channel":
        y["g"] = x["g"][..., :dk].contiguous()
    if x["h0"] is not None:
        y["h0"] = x["h0"][:, :, :dk, :dv].contiguous()
    y["scale"] = float(dk) ** -0.5
    return y


def _cases(seed=20261202, n=48):
    r = random.Random(seed)
    out = []
    for i in range(n):
        c = dict(i=i, gate=r.choice(["scalar", "scalar", "channel"]), dtype=r.choice(["bf16", "bf16", "fp32"]))
        c["Hv"] = r.choice([1, 2, 3, 4, 6])
        c["Hq"] = r.choice([d for d in (1, 2, 3, 4, 6) if c["Hv"] % d == 0])
        c["dk"], c["dv"] = r.choice([64, 128]), r.choice([64, 128])
        c["mu"] = r.choice([None, -6.0, -3.0, -2.0, -1.0, 0.0])
        c["h0"] = r.random() < 0.6
        if r.random() < 0.35:
            ns = r.randint(1, 6)
            c["lens"] = tuple(r.choice([0, 1, r.randint(1, 200), r.randint(60, 70), r.randint(100, 900)]) for _ in range(ns))
        else:
            c["B"], c["T"] = r.randint(1, 3), r.choice([1, 63, 64, 65, r.randint(2, 1500)])
        cp = r.choice(["auto", "off", "on", "warmup"])
        c["kw"] = {"cp_mode": cp}
        if cp in ("on", "warmup"):
            c["kw"]["cp_segment_chunks"] = r.randint(1, 8)
        if cp == "on" and c["gate"] == "scalar" and c["dtype"] == "bf16" and c["dk"] == c["dv"] and r.random() < 0.5:
            c["kw"]["cp_form"] = "xyz"
        c["bv16"] = c["gate"] == "scalar" and c["dtype"] == "bf16" and r.random() < 0.25
        out.append(c)
    return out


def _id(c):
    shape = ("lens" + "_".join(str(n) for n in c["lens"])) if "lens" in c else f"B{c['B']}T{c['T']}"
    return (f"{c['i']}-{c['gate']}-{c['dtype']}-Hv{c['Hv']}Hq{c['Hq']}-dk{c['dk']}dv{c['dv']}-mu{c['mu']}-"
            f"h0{int(c['h0'])}-{shape}-{c['kw'].get('cp_mode')}{c['kw'].get('cp_segment_chunks', '')}"
            f"{c['kw'].get('cp_form', '')}{'-bv16' if c['bv16'] else ''}")


@pytest.mark.parametrize("c", _cases(), ids=_id)
def test_random_configuration(c, monkeypatch):
    monkeypatch.setenv("GDN_BV", "16" if c["bv16"] else "0")
    common = dict(H=c["Hv"], H_qk=c["Hq"], D=128, dtype=c["dtype"], gate=c["gate"], mu=c["mu"], h0=c["h0"],
                  seed=9000 + c["i"])
    if "lens" in c:
        w = synth.workload("varlen_bf16", n_seqs=len(c["lens"]), lens=c["lens"], **common)
    else:
        w = synth.workload("qwen3next_bf16", B=c["B"], T=c["T"], **common)
    x = _dims(synth.make_inputs(w), c["dk"], c["dv"])
    check(x, TOL[c["dtype"]], label=_id(c), **c["kw"])


def _decode_cases(seed=20261204, n=16):
    r = random.Random(seed)
    out = []
    for i in range(n):
        c = dict(i=i, gate=r.choice(["scalar", "channel"]), dtype=r.choice(["bf16", "fp32"]))
        c["Hv"] = r.choice([1, 2, 4, 6])
        c["Hq"] = r.choice([d for d in (1, 2, 3, 6) if c["Hv"] % d == 0])
        c["dk"], c["dv"] = r.choice([64, 128]), r.choice([64, 128])
        c["mu"] = r.choice([None, -3.0, -2.0, 0.0])
        c["h0"] = r.random() < 0.7
        if r.random() < 0.4:
            c["lens"] = tuple(r.choice([0, 1, 2, r.randint(1, 40)]) for _ in range(r.randint(1, 8)))
        else:
            c["B"], c["T"] = r.randint(1, 8), r.choice([1, 1, 2, r.randint(1, 40)])
        out.append(c)
    return out


def _decode_id(c):
    shape = ("lens" + "_".join(str(n) for n in c["lens"])) if "lens" in c else f"B{c['B']}T{c['T']}"
    return (f"{c['i']}-{c['gate']}-{c['dtype']}-Hv{c['Hv']}Hq{c['Hq']}-dk{c['dk']}dv{c['dv']}-mu{c['mu']}-"
            f"h0{int(c['h0'])}-{shape}")


@pytest.mark.parametrize("c", _decode_cases(), ids=_decode_id)
def test_random_decode_configuration(c):
    # gdn_fwd_recurrent (token by token) on a random configuration
    common = dict(H=c["Hv"], H_qk=c["Hq"], D=128, dtype=c["dtype"], gate=c["gate"], mu=c["mu"], h0=c["h0"],
                  seed=9800 + c["i"])
    if "lens" in c:
        w = synth.workload("varlen_bf16", n_seqs=len(c["lens"]), lens=c["lens"], **common)
    else:
        w = synth.workload("qwen3next_bf16", B=c["B"], T=c["T"], **common)
    x = _dims(synth.make_inputs(w), c["dk"], c["dv"])
    check(x, TOL[c["dtype"]], label=_decode_id(c), recurrent=True)
