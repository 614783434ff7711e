"""Shared helpers for the GPU parity tests: run the HIP path and the fp64 oracle on the same
seeded inputs and compare with the tolerance rule max|delta| <= tol * RMS(oracle).

Reading of the rule for a bf16 output: rounding the exact result to bf16 alone moves the largest
outputs (about 10 RMS on the full-size workloads) by up to half a bf16 ulp, more than 2e-2 RMS.
So the bound applies to the computation: every bf16-workload case is checked twice,
  * with an fp32 output (the result before its storage rounding) against tol * RMS, and
  * with the bf16 output against tol * RMS plus half a bf16 ulp of that element.
The final state is fp32 and is always checked against tol * RMS."""
import numpy as np
import torch

from chunkwise_linear_attention_chunk_amd import fwd, fwd_recurrent, synth
from oracle.recurrent import gdn_recurrent
from oracle.prologue import apply_prologue

TOL = {"fp32": 1e-4, "bf16": 2e-2}
f64 = synth.to_f64


def half_ulp_bf16(a):
    """Half a bf16 ulp at |a| (0 at a == 0): 2^(floor(log2|a|) - 8)."""
    m, e = np.frexp(np.abs(a))
    return np.where(a == 0, 0.0, np.ldexp(1.0, e - 9))


def gpu_run(x, prologue=None, recurrent=False, **kw):
    """The HIP path on x: gdn_fwd (chunked), or gdn_fwd_recurrent (token by token) if recurrent."""
    dev = torch.device("cuda:0")
    t = lambda a: None if a is None else a.to(dev)
    pro = {} if prologue is None else {n: (t(a) if isinstance(a, torch.Tensor) else a) for n, a in prologue.items()}
    run = fwd_recurrent if recurrent else fwd
    o, fs = run(t(x["q"]), t(x["k"]), t(x["v"]), t(x["g"]), t(x["beta"]), scale=x["scale"],
                initial_state=t(x["h0"]), cu_seqlens=x["cu_seqlens"], **pro, **kw)
    torch.cuda.synchronize()
    return o.cpu(), fs.cpu()


def oracle_run(x, batches=None, heads=None, seqs=None, prologue=None):
    """fp64 oracle on all of x, or on the selected batch rows / heads / packed sequences.

    Returns (o, final) shaped like the selection, plus a function mapping full GPU outputs to
    the same selection."""
    q, k, v, g, b = (f64(x[n]) for n in ("q", "k", "v", "g", "beta"))
    h0 = f64(x["h0"])
    gate = x["gate"]
    if prologue is not None:
        pro = {n: (f64(a) if isinstance(a, torch.Tensor) else a) for n, a in prologue.items()}
        q, k, g, b = apply_prologue(q, k, g, b, gate, **pro)
    H = v.shape[2]
    hs = list(range(H)) if heads is None else list(heads)
    G = H // q.shape[2]
    hq = sorted(set(h // G for h in hs))
    assert G == 1 or heads is None, "head sampling assumes H_qk == H_v"
    cu = None if x["cu_seqlens"] is None else x["cu_seqlens"].numpy().astype(np.int64)
    if cu is None:
        bs = list(range(q.shape[0])) if batches is None else list(batches)
        sel = lambda a, hh: a[bs][:, :, hh]
        qq, kk = sel(q, hq if G == 1 else slice(None)), sel(k, hq if G == 1 else slice(None))
        vv, gg, bb = sel(v, hs), g[bs][:, :, hs], b[bs][:, :, hs]
        hh0 = None if h0 is None else h0[bs][:, hs]
        o, fin = gdn_recurrent(qq, kk, vv, gg, bb, x["scale"], h0=hh0, gate=gate)

        def pick(o_gpu, f_gpu):
            return f64(o_gpu)[bs][:, :, hs], f64(f_gpu)[bs][:, hs]
        return o, fin, pick
    ns = list(range(len(cu) - 1)) if seqs is None else list(seqs)
    rows = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in ns]) if ns else np.zeros(0, np.int64)
    lens = [cu[n + 1] - cu[n] for n in ns]
    cu_s = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    sel = lambda a, hh: a[:, rows][:, :, hh]
    o, fin = gdn_recurrent(sel(q, hq if G == 1 else slice(None)), sel(k, hq if G == 1 else slice(None)),
                           sel(v, hs), g[:, rows][:, :, hs], b[:, rows][:, :, hs], x["scale"],
                           h0=None if h0 is None else h0[ns][:, hs], cu_seqlens=cu_s, gate=gate)

    def pick(o_gpu, f_gpu):
        return f64(o_gpu)[:, rows][:, :, hs], f64(f_gpu)[ns][:, hs]
    return o, fin, pick


def _over_rms(err, ref):
    """err / RMS(ref); an all-zero reference (an empty sequence without h0) allows no error at all."""
    if ref.size == 0:
        return 0.0
    rms = np.sqrt(np.mean(ref ** 2))
    if rms == 0.0:
        return 0.0 if err <= 0.0 else float("inf")
    return float(err / rms)


def rel_max_err(got, ref):
    return _over_rms(float(np.abs(got - ref).max()) if ref.size else 0.0, ref)


def rel_max_err_rounded(got, ref):
    """max_i (|got_i - ref_i| - half_ulp_bf16(max(|got_i|, |ref_i|))) / RMS(ref), floored at 0."""
    if ref.size == 0:
        return 0.0
    excess = np.abs(got - ref) - half_ulp_bf16(np.maximum(np.abs(got), np.abs(ref)))
    return max(_over_rms(float(excess.max()), ref), 0.0)


def check(x, tol, batches=None, heads=None, seqs=None, label="", prologue=None, **kw):
    o_r, f_r, pick = oracle_run(x, batches, heads, seqs, prologue)
    bf16 = x["q"].dtype == torch.bfloat16
    runs = [("fp32-out", torch.float32), ("bf16-out", None)] if bf16 else [("", None)]
    worst = (0.0, 0.0)
    for tag, odt in runs:
        o_g, f_g = gpu_run(x, prologue, out_dtype=odt, **kw)
        assert torch.isfinite(o_g.float()).all() and torch.isfinite(f_g).all(), f"{label}: non-finite output"
        o_s, f_s = pick(o_g, f_g)
        eo = rel_max_err_rounded(o_s, o_r) if tag == "bf16-out" else rel_max_err(o_s, o_r)
        ef = rel_max_err(f_s, f_r)
        print(f"[parity] {label} {tag}: max|do|/rms(o) = {eo:.3e}  max|dS|/rms(S) = {ef:.3e}  (tol {tol})",
              flush=True)
        assert eo <= tol, f"{label} {tag}: output error {eo:.3e} > {tol}"
        assert ef <= tol, f"{label} {tag}: final-state error {ef:.3e} > {tol}"
        worst = (max(worst[0], eo), max(worst[1], ef))
    return worst
