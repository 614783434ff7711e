"""GPU checks of the allocation-free entry point gdn_fwd_noalloc (include/gdn.h), through the C ABI.

It runs the same kernels as gdn_fwd on the library's static per-GPU scratch array instead of a
caller workspace, so its results must equal gdn_fwd's bit for bit on the same inputs (both are
deterministic).  Two calls in a row, the second with a smaller input, check that nothing depends
on what the previous call left in the scratch array.
"""
import pytest
import torch

from chunkwise_linear_attention_chunk_amd import gdn, synth

pytestmark = pytest.mark.gpu


def _prepare(x, dev, cp_mode="auto", cp_segment_chunks=0):
    t = {n: x[n].to(dev) for n in ("q", "k", "v", "g", "beta")}
    h0 = None if x["h0"] is None else x["h0"].to(dev)
    cu_host = None if x["cu_seqlens"] is None else x["cu_seqlens"].to(torch.int32)
    cu_dev = None if cu_host is None else cu_host.to(dev)
    N = x["n_seqs"]
    shape_s = (N, t["v"].shape[2], t["k"].shape[3], t["v"].shape[3])
    outs = []
    for _ in range(2):   # one output set per entry point, filled with NaN so that unwritten values show
        o = torch.full(t["v"].shape, float("nan"), dtype=t["q"].dtype, device=dev)
        fs = torch.full(shape_s, float("nan"), dtype=torch.float32, device=dev)
        a = gdn.make_args(t["q"], t["k"], t["v"], t["g"], t["beta"], x["scale"], h0, cu_dev, cu_host, 64, o, fs,
                          cp_mode, cp_segment_chunks)
        outs.append((a, o, fs))
    return t, outs


def _compare(x, dev, label, **kw):
    t, ((a_ref, o_ref, f_ref), (a_na, o_na, f_na)) = _prepare(x, dev, **kw)
    stream = torch.cuda.current_stream(dev).cuda_stream
    nbytes = gdn.workspace_bytes(a_ref)
    assert 0 < nbytes <= gdn.NOALLOC_SCRATCH_BYTES, f"{label}: workspace {nbytes}"
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    gdn.fwd_raw(a_ref, ws.data_ptr(), ws.numel(), stream)
    gdn.fwd_noalloc_raw(a_na, stream)
    torch.cuda.synchronize()
    print(f"[noalloc] {label}: workspace {nbytes} bytes, o {tuple(o_na.shape)}", flush=True)
    assert torch.isfinite(o_na.float()).all() and torch.isfinite(f_na).all(), f"{label}: unwritten output"
    assert torch.equal(o_na, o_ref), f"{label}: o differs from gdn_fwd"
    assert torch.equal(f_na, f_ref), f"{label}: final state differs from gdn_fwd"


def test_noalloc_matches_gdn_fwd_then_smaller_input():
    dev = torch.device("cuda:0")
    big = synth.make_inputs(synth.workload("qwen3next_bf16", B=2, H=4, T=64 * 15 + 40, h0=True, seed=901))
    small = synth.make_inputs(synth.workload("qwen3next_bf16", B=1, H=2, T=64 * 3 + 5, h0=True, seed=902))
    _compare(big, dev, "bf16 B=2 H=4 T=1000")
    _compare(small, dev, "bf16 B=1 H=2 T=197 (second call, smaller)")


def test_noalloc_packed_cp_and_channel_gates():
    dev = torch.device("cuda:0")
    _compare(synth.make_inputs(synth.workload("varlen_bf16", n_seqs=5, lens=(0, 65, 300, 1, 700), H=3, h0=True,
                                              seed=903)), dev, "packed, CP L=2", cp_mode="on", cp_segment_chunks=2)
    _compare(synth.make_inputs(synth.workload("kda_bf16", B=1, H=2, T=64 * 4 + 9, h0=True, seed=904)), dev,
             "per-channel gates")
    _compare(synth.make_inputs(synth.workload("tiny_fp32", B=2, T=100, h0=True, seed=905)), dev, "fp32 T=100")
