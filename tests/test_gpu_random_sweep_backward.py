"""GPU parity of gdn_bwd on a fixed-seed random sweep of configurations against the fp64 autograd
oracle: gate kind, dtype, value and query/key head counts (grouped heads), key and value head dims,
gate strength, initial state and dht, batched or packed (with empty and chunk-edge lengths).  Each
case is small enough for the autograd oracle to run whole."""
import random

import pytest

from chunkwise_linear_attention_chunk_amd import synth
from test_gpu_backward import TOL, _check
from test_gpu_random_sweep import _dims

pytestmark = pytest.mark.gpu


def _cases(seed=20261203, n=16):
    r = random.Random(seed)
    out = []
    for i in range(n):
        c = dict(i=i, gate=r.choice(["scalar", "channel"]), dtype=r.choice(["bf16", "bf16", "fp32"]))
        c["Hv"] = r.choice([1, 2, 4])
        c["Hq"] = r.choice([d for d in (1, 2, 4) if c["Hv"] % d == 0])
        c["dk"], c["dv"] = r.choice([64, 128]), r.choice([64, 128])
        c["mu"] = r.choice([None, -6.0, -3.0, -2.0, 0.0])
        c["h0"], c["dht"] = r.random() < 0.6, r.random() < 0.7
        if r.random() < 0.35:
            c["lens"] = tuple(r.choice([0, 1, r.randint(60, 70), r.randint(2, 260)]) for _ in range(r.randint(1, 4)))
        else:
            c["B"], c["T"] = r.randint(1, 2), r.choice([1, 64, 65, r.randint(2, 300)])
        out.append(c)
    return out


def _id(c):
    shape = ("lens" + "_".join(str(n) for n in c["lens"])) if "lens" in c else f"B{c['B']}T{c['T']}"
    return (f"{c['i']}-{c['gate']}-{c['dtype']}-Hv{c['Hv']}Hq{c['Hq']}-dk{c['dk']}dv{c['dv']}-mu{c['mu']}-"
            f"h0{int(c['h0'])}-dht{int(c['dht'])}-{shape}")


@pytest.mark.parametrize("c", _cases(), ids=_id)
def test_random_backward_configuration(c):
    common = dict(H=c["Hv"], H_qk=c["Hq"], D=128, dtype=c["dtype"], gate=c["gate"], mu=c["mu"], h0=c["h0"],
                  seed=9500 + c["i"])
    if "lens" in c:
        w = synth.workload("varlen_bf16", n_seqs=len(c["lens"]), lens=c["lens"], **common)
    else:
        w = synth.workload("qwen3next_bf16", B=c["B"], T=c["T"], **common)
    x = _dims(synth.make_inputs(w), c["dk"], c["dv"])
    _check(x, TOL[c["dtype"]], _id(c), seed=c["i"], dht=c["dht"])
