"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Tolerance: max|delta| <= 1e-4 * RMS for fp32 inputs and <= 2e-2 * RMS for bf16 inputs, on the
output o and on the final state.  Small cases are compared in full; the full-size workloads
are compared on sampled (sequence, head) pairs that the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

from chunkwise_linear_attention_chunk_amd import synth
from parity_util import TOL, check, gpu_run

pytestmark = pytest.mark.gpu


def _w(name, **kw):
    return synth.make_inputs(synth.workload(name, **kw))


# --------------------------------------------------------------------------- fp32
def test_tiny_fp32_workload():
    x = _w("tiny_fp32")
    check(x, TOL["fp32"], label="tiny_fp32")


@pytest.mark.parametrize("T", [1, 63, 64, 65, 200, 1000])
def test_fp32_ragged_lengths_with_initial_state(T):
    x = _w("tiny_fp32", T=T, B=2, h0=True, seed=T)
    check(x, TOL["fp32"], label=f"fp32 T={T}")


@pytest.mark.parametrize("mu", [None, -7.0, 2.0])
def test_fp32_gate_strengths(mu):
    # g == 0, weak decay (~1e-3 per token) and strong decay: the inter-chunk state matters
    x = _w("tiny_fp32", T=640, H=3, h0=True, mu=mu, seed=5)
    check(x, TOL["fp32"], label=f"fp32 mu={mu}")


def test_fp32_head_dim_128_and_grouped_heads():
    x = _w("tiny_fp32", T=333, H=4, H_qk=2, D=128, h0=True, seed=9)
    check(x, TOL["fp32"], label="fp32 D=128 H_v=4 H_qk=2")


def test_fp32_packed_ragged():
    x = _w("tiny_fp32", n_seqs=7, lens=(1, 63, 64, 65, 129, 7, 300), H=2, h0=True, seed=3)
    check(x, TOL["fp32"], label="fp32 packed")


# --------------------------------------------------------------------------- bf16
@pytest.mark.parametrize("T,mu", [(300, -2.0), (1000, -7.0), (777, None)])
def test_bf16_small(T, mu):
    x = _w("qwen3next_bf16", B=2, H=3, T=T, mu=mu, h0=True, seed=T)
    check(x, TOL["bf16"], label=f"bf16 T={T} mu={mu}")


def test_bf16_head_dim_64_grouped():
    x = _w("qwen3next_bf16", B=1, H=4, H_qk=1, D=64, T=500, h0=True, seed=11)
    check(x, TOL["bf16"], label="bf16 D=64 H_v=4 H_qk=1")


def test_bf16_packed_ragged():
    x = _w("varlen_bf16", n_seqs=8, lens=(0, 1, 63, 64, 65, 1000, 129, 7), H=3, seed=4)
    check(x, TOL["bf16"], label="bf16 packed ragged")


def test_bf16_two_workgroups_per_cu_build():
    # 8 sequences x 16 heads x 4 column groups = 512 recurrence workgroups: enough for two per CU,
    # which selects the one-buffer build of the recurrence; compared in full, ragged last chunk
    x = _w("qwen3next_bf16", B=8, H=16, T=64 * 3 + 17, h0=True, seed=77)
    check(x, TOL["bf16"], label="bf16 512 workgroups")


def test_packed_two_workgroups_per_cu_build():
    # packed ragged sequences with the one-buffer build (9 x 16 x 4 = 576 workgroups)
    x = _w("varlen_bf16", n_seqs=9, lens=(0, 1, 63, 64, 65, 300, 129, 7, 200), H=16, seed=78)
    check(x, TOL["bf16"], label="bf16 packed, 576 workgroups")


def test_qwen3next_workload_sampled():
    x = _w("qwen3next_bf16")
    check(x, TOL["bf16"], batches=[0, 3], heads=[0, 7, 15], label="qwen3next_bf16 (sampled)")


def test_longctx_workload_sampled():
    x = _w("longctx_bf16")
    check(x, TOL["bf16"], heads=[0, 3], label="longctx_bf16 serial (sampled)", cp_mode="off")


def test_varlen_workload_sampled():
    x = _w("varlen_bf16")
    lens = np.diff(x["cu_seqlens"].numpy())
    seqs = [int(np.argmax(lens)), int(np.argmin(lens)), 5]
    check(x, TOL["bf16"], heads=[0, 9], seqs=seqs, label="varlen_bf16 (sampled)")


# --------------------------------------------------------------------------- context parallelism
# Sequences split into segments of L chunks: per-segment S* and M, serial fix-up of the segment
# start states, then the main pass per segment (FlashQLA page, the CP pre-process).  bf16 with a
# scalar gate runs either form of the pre-process (the recurrence's chain, or X/Y/Z).
FORMS = ["chain", "xyz"]


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("L", [1, 2, 3, 7])
def test_cp_bf16_segment_lengths(L, form):
    x = _w("qwen3next_bf16", B=2, H=2, T=64 * 20 + 17, h0=True, seed=40 + L)
    check(x, TOL["bf16"], label=f"bf16 CP L={L} {form}", cp_mode="on", cp_segment_chunks=L, cp_form=form)


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("L", [1, 3])
def test_cp_without_initial_state(L, form):
    # the first segment's M is never formed without h0: the fix-up must not use it
    x = _w("qwen3next_bf16", B=1, H=2, T=64 * 9, mu=-7.0, seed=50 + L)
    check(x, TOL["bf16"], label=f"bf16 CP no h0 L={L} {form}", cp_mode="on", cp_segment_chunks=L, cp_form=form)


@pytest.mark.parametrize("L", [1, 4])
def test_cp_fp32(L):
    x = _w("tiny_fp32", B=2, T=64 * 11 + 5, h0=True, mu=-7.0, seed=60 + L)
    check(x, TOL["fp32"], label=f"fp32 CP L={L}", cp_mode="on", cp_segment_chunks=L)
    x = _w("tiny_fp32", T=64 * 6 + 40, H=4, H_qk=2, D=128, h0=True, seed=70 + L)
    check(x, TOL["fp32"], label=f"fp32 D=128 CP L={L}", cp_mode="on", cp_segment_chunks=L)


@pytest.mark.parametrize("form", FORMS)
def test_cp_packed_ragged(form):
    x = _w("varlen_bf16", n_seqs=8, lens=(0, 1, 63, 64, 65, 1000, 129, 700), H=3, h0=True, seed=80)
    check(x, TOL["bf16"], label=f"bf16 packed CP L=2 {form}", cp_mode="on", cp_segment_chunks=2, cp_form=form)


@pytest.mark.parametrize("form", FORMS)
def test_cp_bf16_head_dim_64(form):
    x = _w("qwen3next_bf16", B=1, H=4, H_qk=1, D=64, T=900, h0=True, seed=90)
    check(x, TOL["bf16"], label=f"bf16 D=64 CP L=3 {form}", cp_mode="on", cp_segment_chunks=3, cp_form=form)


def test_cp_forms_agree():
    # the two forms of the pre-process compute the same maps; they differ only by rounding order
    x = _w("qwen3next_bf16", B=1, H=2, T=64 * 40, h0=True, mu=-7.0, seed=92)
    o1, f1 = gpu_run(x, cp_mode="on", cp_segment_chunks=5, cp_form="chain", out_dtype=torch.float32)
    o2, f2 = gpu_run(x, cp_mode="on", cp_segment_chunks=5, cp_form="xyz", out_dtype=torch.float32)
    rms_o, rms_f = o1.double().pow(2).mean().sqrt(), f1.double().pow(2).mean().sqrt()
    assert (o1 - o2).abs().max() <= 1e-2 * rms_o
    assert (f1 - f2).abs().max() <= 1e-2 * rms_f


def test_cp_matches_serial_pass():
    # the two schedules compute the same quantities; they differ only by rounding order
    x = _w("qwen3next_bf16", B=1, H=2, T=64 * 40, h0=True, mu=-7.0, seed=91)
    o1, f1 = gpu_run(x, cp_mode="off", out_dtype=torch.float32)
    o2, f2 = gpu_run(x, cp_mode="on", cp_segment_chunks=5, out_dtype=torch.float32)
    rms_o, rms_f = o1.double().pow(2).mean().sqrt(), f1.double().pow(2).mean().sqrt()
    assert (o1 - o2).abs().max() <= 1e-2 * rms_o
    assert (f1 - f2).abs().max() <= 1e-2 * rms_f


def test_longctx_workload_cp_auto_sampled():
    # B*H = 4: the automatic choice splits the sequence into segments
    x = _w("longctx_bf16")
    check(x, TOL["bf16"], heads=[1, 2], label="longctx_bf16 CP auto (sampled)", cp_mode="auto")


# --------------------------------------------------------------------------- per-channel gates (KDA)
@pytest.mark.parametrize("T", [64, 200, 700])
def test_kda_fp32(T):
    x = _w("tiny_fp32", T=T, B=2, gate="channel", mu=-3.0, h0=True, seed=100 + T)
    check(x, TOL["fp32"], label=f"KDA fp32 T={T}")


def test_kda_fp32_head_dim_128_grouped():
    x = _w("tiny_fp32", T=333, H=4, H_qk=2, D=128, gate="channel", mu=-3.0, h0=True, seed=110)
    check(x, TOL["fp32"], label="KDA fp32 D=128 H_v=4 H_qk=2")


@pytest.mark.parametrize("T,mu", [(300, -3.0), (1000, -6.0), (777, -1.0)])
def test_kda_bf16_small(T, mu):
    x = _w("kda_bf16", B=2, H=3, T=T, mu=mu, h0=True, seed=120 + T)
    check(x, TOL["bf16"], label=f"KDA bf16 T={T} mu={mu}")


def test_kda_bf16_head_dim_64_grouped():
    x = _w("kda_bf16", B=1, H=4, H_qk=1, D=64, T=500, h0=True, seed=130)
    check(x, TOL["bf16"], label="KDA bf16 D=64 H_v=4 H_qk=1")


def test_kda_packed_ragged():
    x = _w("kda_bf16", B=1, n_seqs=6, lens=(1, 63, 65, 0, 300, 129), H=2, h0=True, seed=140)
    check(x, TOL["bf16"], label="KDA bf16 packed")


@pytest.mark.parametrize("L", [1, 3])
def test_kda_cp(L):
    x = _w("kda_bf16", B=1, H=2, T=64 * 10 + 9, h0=True, seed=150 + L)
    check(x, TOL["bf16"], label=f"KDA bf16 CP L={L}", cp_mode="on", cp_segment_chunks=L)


def test_kda_workload_sampled():
    x = _w("kda_bf16")
    check(x, TOL["bf16"], batches=[1], heads=[0, 31], label="kda_bf16 (sampled)")


# --------------------------------------------------------------------------- D_k != D_v
def _dims(x, dk, dv):
    """Inputs of a D = 128 workload cut to key dim dk and value dim dv (q, k re-normalised over dk,
    the per-channel gate cut with them); both sides of the comparison take the same tensors."""
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


@pytest.mark.parametrize("dk,dv", [(128, 64), (64, 128)])
@pytest.mark.parametrize("cp", ["off", "chain", "xyz"])
def test_bf16_key_and_value_dims_differ(dk, dv, cp):
    x = _dims(_w("qwen3next_bf16", B=2, H=2, T=64 * 7 + 21, h0=True, mu=-7.0, seed=200 + dk), dk, dv)
    mode = dict(cp_mode="off") if cp == "off" else dict(cp_mode="on", cp_form=cp)
    check(x, TOL["bf16"], label=f"bf16 D_k={dk} D_v={dv} CP {cp}", cp_segment_chunks=2, **mode)


def test_fp32_key_and_value_dims_differ():
    x = _dims(_w("tiny_fp32", T=300, H=2, D=128, h0=True, seed=210), 128, 64)
    check(x, TOL["fp32"], label="fp32 D_k=128 D_v=64")


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64)])
def test_kda_key_and_value_dims_differ(dk, dv):
    # (128, 64): two column slices per head, fewer L2-prefetch slots than prefetch units
    x = _dims(_w("kda_bf16", B=1, H=2, T=400, h0=True, seed=220 + dv), dk, dv)
    check(x, TOL["bf16"], label=f"KDA bf16 D_k={dk} D_v={dv}")


@pytest.mark.parametrize("gate,dtype", [("scalar", "bf16"), ("channel", "fp32")])
def test_empty_sequences_without_initial_state(gate, dtype):
    # packed input whose sequences are all empty, no h0: every final state is zero (written, not left over)
    x = _w("varlen_bf16", n_seqs=2, lens=(0, 0), H=2, dtype=dtype, gate=gate, seed=231)
    check(x, TOL[dtype], label=f"empty sequences {gate} {dtype}")
    dev = torch.device("cuda:0")
    t = {n: x[n].to(dev) for n in ("q", "k", "v", "g", "beta")}
    torch.cuda.synchronize()
    fs = torch.full((2, 2, 128, 128), 7.0, device=dev)
    o = torch.empty(t["v"].shape, dtype=t["v"].dtype, device=dev)
    from chunkwise_linear_attention_chunk_amd import gdn
    cu = x["cu_seqlens"].to(torch.int32)
    a = gdn.make_args(t["q"], t["k"], t["v"], t["g"], t["beta"], x["scale"], None, cu.to(dev), cu, 64, o, fs)
    ws = torch.empty(max(gdn.workspace_bytes(a), 1), dtype=torch.uint8, device=dev)
    gdn.fwd_raw(a, ws.data_ptr(), ws.numel(), torch.cuda.current_stream(dev).cuda_stream)
    torch.cuda.synchronize()
    assert bool((fs == 0).all()), "the final states of empty sequences must be written as zeros"


def test_empty_sequence_returns_initial_state():
    x = _w("qwen3next_bf16", B=2, H=2, T=0, h0=True, seed=230)
    o, fs = gpu_run(x)
    assert o.numel() == 0
    assert torch.equal(fs, x["h0"])


# --------------------------------------------------------------------------- 16-column workgroups
# GDN_BV=16 selects the recurrence build with one chain and one output wave per workgroup (16 value
# columns), whose single output wave owns all four token tiles and stores them one chunk late.
@pytest.mark.parametrize("dk", [64, 128])
def test_sixteen_column_workgroups_bf16(dk, monkeypatch):
    monkeypatch.setenv("GDN_BV", "16")
    x = _w("qwen3next_bf16", B=2, H=2, D=dk, T=64 * 9 + 21, h0=True, seed=740 + dk)
    check(x, TOL["bf16"], label=f"BV=16 bf16 D={dk}", cp_mode="off")
    # with warmup CP: the early chunks of a segment produce no output
    x = _w("qwen3next_bf16", B=1, H=1, D=dk, T=64 * 40 + 5, seed=750 + dk)
    check(x, TOL["bf16"], label=f"BV=16 bf16 D={dk} warmup CP", cp_mode="warmup", cp_segment_chunks=8)


# --------------------------------------------------------------------------- pieces
# Batched input without CP is cut into chunk ranges: the per-chunk kernel of range j + 1 runs on a
# side stream while the recurrence runs range j from the end state of range j - 1.
@pytest.mark.parametrize("pieces", [1, 2, 3, 8])
def test_pieces_bf16(pieces, monkeypatch):
    monkeypatch.setenv("GDN_PIECES", str(pieces))
    x = _w("qwen3next_bf16", B=2, H=3, T=64 * 17 + 13, h0=True, seed=700 + pieces)
    check(x, TOL["bf16"], label=f"pieces={pieces}", cp_mode="off")   # (few chains would pick CP)


def test_pieces_fp32_and_kda(monkeypatch):
    monkeypatch.setenv("GDN_PIECES", "3")
    check(_w("tiny_fp32", B=2, T=64 * 7 + 5, h0=True, seed=710), TOL["fp32"], label="pieces=3 fp32", cp_mode="off")
    check(_w("kda_bf16", B=1, H=2, T=64 * 9, h0=True, seed=711), TOL["bf16"], label="pieces=3 KDA", cp_mode="off")


def test_pieces_plan_and_repeat_calls(monkeypatch):
    # the schedule with four pieces, and back-to-back calls that reuse the side stream
    from chunkwise_linear_attention_chunk_amd import gdn
    monkeypatch.setenv("GDN_PIECES", "4")
    x = _w("qwen3next_bf16", B=4, H=16, T=64 * 12, seed=712)
    o1, f1 = gpu_run(x)
    o2, f2 = gpu_run(x)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    dev = torch.device("cuda:0")
    t = {n: x[n].to(dev) for n in ("q", "k", "v", "g", "beta")}
    o = torch.empty(t["v"].shape, dtype=t["v"].dtype, device=dev)
    a = gdn.make_args(t["q"], t["k"], t["v"], t["g"], t["beta"], x["scale"], o=o)
    assert gdn.plan(a)["pieces"] == 4


# --------------------------------------------------------------------------- in-kernel prologue
# Raw inputs (q, k rows of random length, raw gate inputs, beta logits) with the prologue switched on:
# the oracle applies oracle/prologue.py in fp64, the library inside its kernels.
def _wp(name, lower_bound=0.0, **kw):
    return synth.make_prologue_inputs(synth.workload(name, **kw), lower_bound)


@pytest.mark.parametrize("T", [64, 300])
def test_prologue_fp32(T):
    x, pro = _wp("tiny_fp32", B=2, T=T, h0=True, seed=300 + T)
    check(x, TOL["fp32"], prologue=pro, label=f"prologue fp32 T={T}")


def test_prologue_fp32_head_dim_128():
    x, pro = _wp("tiny_fp32", B=1, H=2, D=128, T=200, h0=True, seed=305)
    check(x, TOL["fp32"], prologue=pro, label="prologue fp32 D=128")


def test_prologue_bf16():
    x, pro = _wp("qwen3next_bf16", B=2, H=3, T=700, h0=True, seed=310)
    check(x, TOL["bf16"], prologue=pro, label="prologue bf16")


def test_prologue_lower_bound_grouped_heads():
    x, pro = _wp("qwen3next_bf16", lower_bound=-5.0, B=1, H=4, H_qk=2, T=333, h0=True, seed=311)
    check(x, TOL["bf16"], prologue=pro, label="prologue lower bound, H_v=4 H_qk=2")


def test_prologue_bf16_head_dim_64():
    x, pro = _wp("qwen3next_bf16", B=1, H=2, D=64, T=260, h0=True, seed=312)
    check(x, TOL["bf16"], prologue=pro, label="prologue bf16 D=64")


def test_prologue_packed_and_cp():
    x, pro = _wp("varlen_bf16", n_seqs=5, lens=(1, 65, 300, 0, 700), H=3, h0=True, seed=313)
    check(x, TOL["bf16"], prologue=pro, label="prologue packed")
    check(x, TOL["bf16"], prologue=pro, label="prologue packed, CP", cp_mode="on", cp_segment_chunks=2)


def test_prologue_two_workgroups_per_cu_build():
    x, pro = _wp("qwen3next_bf16", B=8, H=16, T=150, seed=314)
    check(x, TOL["bf16"], prologue=pro, label="prologue, 512 workgroups")


def test_prologue_kda():
    x, pro = _wp("kda_bf16", B=1, H=2, T=400, h0=True, seed=315)
    check(x, TOL["bf16"], prologue=pro, label="prologue KDA bf16")
    x, pro = _wp("kda_bf16", lower_bound=-5.0, B=1, n_seqs=3, lens=(65, 0, 200), H=2, seed=316)
    check(x, TOL["bf16"], prologue=pro, label="prologue KDA bf16 lower bound, packed")


@pytest.mark.parametrize("name", ["qwen3next_bf16", "kda_bf16"])
@pytest.mark.parametrize("part", ["gates", "l2norm"])
def test_prologue_parts(name, part):
    """One part of the prologue on, the other inputs already in final form."""
    w = synth.workload(name, B=1, H=2, T=333, h0=True, seed=320)
    x0 = synth.make_inputs(w)
    x, pro = synth.make_prologue_inputs(w)
    if part == "gates":      # gate activation and sigma(beta); q, k as generated (unit rows)
        x = dict(x, q=x0["q"], k=x0["k"])
        pro = dict(pro, qk_l2norm=False)
    else:                    # q/k L2 norm only; final gates and beta
        x = dict(x, g=x0["g"], beta=x0["beta"])
        pro = dict(qk_l2norm=True)
    check(x, TOL["bf16"], prologue=pro, label=f"prologue {part} only, {name}")


def test_prologue_kda_fp32():
    x, pro = _wp("tiny_fp32", B=2, T=200, gate="channel", h0=True, seed=317)
    check(x, TOL["fp32"], prologue=pro, label="prologue KDA fp32")


# --------------------------------------------------------------------------- properties
def test_deterministic():
    x = _w("qwen3next_bf16", B=1, H=4, T=700, h0=True, seed=21)
    o1, f1 = gpu_run(x)
    o2, f2 = gpu_run(x)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_continuation():
    # running T1 and then T2 from the final state equals running T1 + T2 (up to tolerance)
    x = _w("tiny_fp32", T=512, h0=True, mu=-7.0, seed=31)
    o_full, f_full = gpu_run(x)
    cut = 200
    part = lambda d, a, b: {**d, **{n: d[n][:, a:b].contiguous() for n in ("q", "k", "v", "g", "beta")}}
    o1, f1 = gpu_run(part(x, 0, cut))
    o2, f2 = gpu_run({**part(x, cut, 512), "h0": f1})
    rms = o_full.double().pow(2).mean().sqrt()
    assert (torch.cat([o1, o2], 1) - o_full).abs().max() <= 1e-4 * rms
    assert (f2 - f_full).abs().max() <= 1e-4 * f_full.double().pow(2).mean().sqrt()


# --------------------------------------------------------------------------- timed entry point
@pytest.mark.parametrize("pieces", [1, 2])
def test_timed_call_with_null_events_matches_untimed(pieces, monkeypatch):
    # gdn_fwd_timed with only some events given (NULL entries are not recorded): same results as
    # gdn_fwd, and the recorded events give the recurrence's time
    import ctypes
    from chunkwise_linear_attention_chunk_amd import gdn
    monkeypatch.setenv("GDN_PIECES", str(pieces))
    x = _w("qwen3next_bf16", B=2, H=2, T=64 * 6 + 9, h0=True, seed=760 + pieces)
    dev = torch.device("cuda:0")
    t = {n: x[n].to(dev) for n in ("q", "k", "v", "g", "beta", "h0")}
    outs = []
    for timed in (False, True):
        o = torch.empty(t["v"].shape, dtype=t["v"].dtype, device=dev)
        fs = torch.empty(t["h0"].shape, dtype=torch.float32, device=dev)
        a = gdn.make_args(t["q"], t["k"], t["v"], t["g"], t["beta"], x["scale"], t["h0"], None, None, 64, o, fs,
                          cp_mode="off")
        ws = torch.empty(max(gdn.workspace_bytes(a), 1), dtype=torch.uint8, device=dev)
        s = torch.cuda.current_stream(dev).cuda_stream
        if timed:
            # torch's timing events (hipEvent_t handles underneath), created by a first record
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            for e in evs:
                e.record()
            torch.cuda.synchronize()
            arr = (ctypes.c_void_p * (len(gdn.STAGES) + 1))()   # every entry NULL but these two
            arr[gdn.STAGES.index("intra") + 1] = evs[0].cuda_event
            arr[gdn.STAGES.index("chunk") + 1] = evs[1].cuda_event
            mask = gdn.fwd_timed_raw(a, ws.data_ptr(), ws.numel(), s, arr)
            torch.cuda.synchronize()
            assert (mask >> gdn.STAGES.index("intra")) & 1 and (mask >> gdn.STAGES.index("chunk")) & 1
            assert evs[0].elapsed_time(evs[1]) > 0.0
        else:
            gdn.fwd_raw(a, ws.data_ptr(), ws.numel(), s)
            torch.cuda.synchronize()
        outs.append((o.cpu(), fs.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
