#!/usr/bin/env python3
"""Benchmark of the gated-delta-rule chunked-prefill forward on one MI355X.

One step = one gdn_fwd call (plan, kernel (a), [CP stages], kernels (b)+(d)) over the whole batch
of the workload, with every input already resident in HBM.  Three input copies are rotated so
the 256 MB last-level cache cannot hold a step's working set from the previous step.

Prints one JSON line: tokens/s, per-stage times from HIP events recorded on the launch stream
inside the timed region, the roofline of the dominant kernel (algorithmic bytes per launch /
its mean duration), and the fp64 oracle timed on the host cores as a reported CPU baseline.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN chunked-prefill fwd tokens/s at 1 GPU + % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X published HBM3E bandwidth
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
_CSRC = "chunkwise_linear_attention_chunk_amd/csrc/"
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence
_HEADERS = [_CSRC + "gdn_device.h", _CSRC + "gdn_internal.h"]
# each kernel's source file and the headers it includes (the counters of profiles/traffic_*.json
# are current only while all of them are unchanged)
KERNEL_SOURCES = {"recurrent": [_CSRC + "gdn_recurrent.hip"] + _HEADERS,
                  "chunk": [_CSRC + "gdn_chunk.hip"] + _HEADERS,
                  "cp_pre": [_CSRC + "gdn_chunk.hip"] + _HEADERS,
                  "intra": [_CSRC + "gdn_intra.hip"] + _HEADERS}


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3next_bf16")
    ap.add_argument("--copies", type=int, default=3)
    ap.add_argument("--cp", default="auto", choices=["auto", "off", "on", "warmup"],
                    help="in-GPU context parallelism (auto: on when too few (sequence, head) chains fill the chip)")
    ap.add_argument("--cp-segment-chunks", type=int, default=0, help="CP segment length in chunks (0: automatic)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other configurations (reported by default with the Qwen3-Next-shaped headline)")
    ap.add_argument("--extra-steps", type=int, default=10)
    ap.add_argument("--extra-warmup", type=int, default=3)
    ap.add_argument("--settle-ms", type=float, default=60.0,
                    help="untimed run of each measured step before its warmup (0: none); see settle()")
    ap.add_argument("--cpu-threads", type=int, default=0, help="oracle threads (0: all host cores)")
    ap.add_argument("--path", default="prefill", choices=["prefill", "decode", "backward"],
                    help="prefill: gdn_fwd on --workload; decode: gdn_fwd_recurrent, one token per sequence "
                         "of a --decode-batch batch with the Qwen3-Next head shape, state updated in place; "
                         "backward: gdn_bwd on --workload (scalar gate)")
    ap.add_argument("--decode-batch", type=int, default=256)
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a 1 GiB device copy (calibrates the HBM byte counters)")
    return ap.parse_args()


def hip_runtime():
    """The HIP runtime torch already loaded (one runtime per process)."""
    maps = open("/proc/self/maps").read().splitlines()
    paths = sorted({l.split()[-1] for l in maps if "libamdhip64" in l and l.split()[-1].startswith("/")})
    if not paths:
        raise RuntimeError("libamdhip64 is not loaded")
    hip = ctypes.CDLL(paths[0])
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return hip


def algorithmic_bytes(x, esz):
    """Compulsory HBM bytes of one forward: inputs read once, outputs written once."""
    q, v = x["q"], x["v"]
    tokens = q.shape[0] * q.shape[1]
    H_qk, D_k, H_v, D_v = q.shape[2], q.shape[3], v.shape[2], v.shape[3]
    b = tokens * (2 * H_qk * D_k * esz + 2 * H_v * D_v * esz + H_v * esz)   # q, k, v, o, beta
    b += x["g"].numel() * x["g"].element_size()                            # gate
    state = x["n_seqs"] * H_v * D_k * D_v * 4
    b += state + (state if x["h0"] is not None else 0)                     # final state, h0
    return b


def stage_algorithmic_bytes(stage, x, esz, plan):
    """Compulsory bytes of one launch of a stage's kernel: the op's inputs it must read (and outputs
    it must write), each counted once.
      intra  (per-chunk kernel): k, the gate and beta (and q with per-channel gates, whose P it forms);
      chunk  (recurrence + output): q, k, v, gate, beta, h0 in; o and the final state out;
      cp_pre (segment maps): k, v, gate and beta of the tokens in segments that are not a
             sequence's last (the last segment's maps are never formed)."""
    q, k, v, g = x["q"], x["k"], x["v"], x["g"]
    H_qk, D_k, H_v, D_v = q.shape[2], q.shape[3], v.shape[2], v.shape[3]
    gate_per_token = g.numel() // (q.shape[0] * q.shape[1]) * g.element_size()
    if stage == "intra":
        tokens = q.shape[0] * q.shape[1]
        qk = 2 if g.dim() == 4 else 1
        return tokens * (qk * H_qk * D_k * esz + gate_per_token + H_v * esz)
    if stage == "cp_pre":
        sl = plan["segment_chunks"]
        if x["cu_seqlens"] is None:
            lens = [q.shape[1]] * q.shape[0]
        else:
            cu = x["cu_seqlens"].tolist()
            lens = [cu[i + 1] - cu[i] for i in range(len(cu) - 1)]
        tokens = 0
        for L in lens:
            ns = max(1, -(-(-(-L // 64)) // sl))
            tokens += min(L, (ns - 1) * sl * 64)
        return tokens * (H_qk * D_k * esz + H_v * D_v * esz + gate_per_token + H_v * esz)
    return algorithmic_bytes(x, esz)


def algorithmic_flops(x):
    """6 d^2 + 5 C d + C^2 / 3 per token-head (d = head dim, C = 64), triangular halves counted."""
    tokens = x["q"].shape[0] * x["q"].shape[1]
    d, C = x["q"].shape[3], 64
    return tokens * x["v"].shape[2] * (6 * d * d + 5 * C * d + C * C / 3)


def settle(step, torch, ms):
    """Run step(i) untimed, in batches of eight, until `ms` of wall time have passed; returns the count.

    After the host has kept the GPU idle (input generation, the CPU baseline), the first tens of steps
    run at a lower clock: on one MI355X the Qwen3-Next-shaped forward took 0.200 ms per step right
    after 2 s of idle and 0.165 ms after 200 steps (0.170 after 300 ms of bf16 matrix products).
    Settling with the measured step itself brings the GPU to the clock that workload sustains; the
    W warm-up steps and the K timed steps then follow exactly as requested."""
    n = 0
    t0 = time.perf_counter()
    while ms > 0 and (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            step(n)
            n += 1
        torch.cuda.synchronize()
    return n


def source_hash(kernel):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, if taken on the current source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256_16") != source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(x, threads):
    from chunkwise_linear_attention_chunk_amd import synth
    from oracle.recurrent import gdn_recurrent
    f64 = synth.to_f64
    args = [f64(x[n]) for n in ("q", "k", "v", "g", "beta")]
    cu = None if x["cu_seqlens"] is None else x["cu_seqlens"].numpy()
    nt = threads or os.cpu_count() or 1
    t0 = time.perf_counter()
    gdn_recurrent(*args, x["scale"], h0=f64(x["h0"]), cu_seqlens=cu, gate=x["gate"], n_threads=nt)
    dt = time.perf_counter() - t0
    return {"value": x["tokens"] / dt, "unit": "tokens/s", "cores": nt, "kind": "oracle",
            "sample": f"the whole workload once ({x['tokens']} tokens x {x['v'].shape[2]} heads), "
                      f"fp64 token recurrence, {dt:.2f} s wall"}


def bench_decode(a, torch, gdn, synth, dev):
    """Decode steps: one token for each of B sequences (Qwen3-Next heads: H = 16, d = 128, bf16),
    state read and written in place.  Three state/input copies rotate so the last-level cache
    cannot hold the previous step's state.  The kernel's compulsory bytes: the state read and
    written (2 x 4 d^2 per sequence-head) plus q, k, v, o, g, beta of the tokens."""
    w = synth.workload("qwen3next_bf16", B=a.decode_batch, T=1, h0=True, seed=7)
    x = synth.make_inputs(w)
    esz = x["q"].element_size()
    copies = []
    for _ in range(max(1, a.copies)):
        t = {n: x[n].to(dev) for n in ("q", "k", "v", "g", "beta")}
        t["state"] = x["h0"].to(dev).clone()
        t["o"] = torch.empty(x["v"].shape, dtype=x["q"].dtype, device=dev)
        copies.append(t)
    argv = [gdn.make_args(c["q"], c["k"], c["v"], c["g"], c["beta"], x["scale"], c["state"], None, None, 1,
                          c["o"], c["state"]) for c in copies]
    stream = torch.cuda.current_stream(dev).cuda_stream
    n_settle = settle(lambda i: gdn.fwd_recurrent_raw(argv[i % len(argv)], stream), torch, a.settle_ms)
    for i in range(a.warmup):
        gdn.fwd_recurrent_raw(argv[i % len(argv)], stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        ev[i][0].record()
        gdn.fwd_recurrent_raw(argv[i % len(argv)], stream)   # on torch's current stream, as the events
        ev[i][1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    k_ms = sum(e0.elapsed_time(e1) for e0, e1 in ev) / a.steps
    alg = algorithmic_bytes(x, esz)
    achieved = alg / (k_ms * 1e-3) / 1e9
    rec = {
        "metric": "GDN decode (token-by-token) tokens/s at 1 GPU + % of HBM roofline", "value": x["tokens"] * a.steps / elapsed,
        "unit": "tokens/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": elapsed / a.steps * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"decode_qwen3next_bf16_b{a.decode_batch}", "B": a.decode_batch, "T": 1,
                   "H_qk": w.hqk, "H_v": w.H, "d_k": w.D, "d_v": w.D, "gate": w.gate, "state_in_place": True,
                   "input_copies": len(copies)},
        "roofline": {"bound": "hbm", "kernel": "recurrent", "alg_bytes": alg, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic("recurrent", f"decode_qwen3next_bf16_b{a.decode_batch}")},
        "stage_ms": {"recurrent": k_ms},
        "clock_settle": {"ms": a.settle_ms, "untimed_steps": n_settle},
    }
    if not a.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(x, a.cpu_threads)
    print(json.dumps(rec), flush=True)


def bench_backward(a, torch, gdn, synth, dev):
    """Backward steps (gdn_bwd) on --workload with a random output gradient and a random final-state
    gradient.  Compulsory bytes: the forward's inputs and dO (and dht) read once, the fp32 gradients
    written once."""
    w = synth.workload(a.workload)
    x = synth.make_inputs(w)
    esz = x["q"].element_size()
    gen = torch.Generator().manual_seed(11)
    N, H, D, Dv = x["n_seqs"], x["v"].shape[2], x["q"].shape[3], x["v"].shape[3]
    t = {n: x[n].to(dev) for n in ("q", "k", "v", "g", "beta")}
    h0 = None if x["h0"] is None else x["h0"].to(dev)
    do = torch.randn(tuple(x["v"].shape), generator=gen).to(x["q"].dtype).to(dev)
    dht = torch.randn((N, H, D, Dv), generator=gen).to(dev)
    f32 = dict(dtype=torch.float32, device=dev)
    grads = {"dq": torch.empty(t["q"].shape, **f32), "dk": torch.empty(t["k"].shape, **f32),
             "dv": torch.empty(t["v"].shape, **f32), "dg": torch.empty(t["g"].shape, **f32),
             "dbeta": torch.empty(t["beta"].shape, **f32), "dh0": torch.empty((N, H, D, Dv), **f32)}
    cu_host = None if x["cu_seqlens"] is None else x["cu_seqlens"].to(torch.int32)
    cu_dev = None if cu_host is None else cu_host.to(dev)
    args = gdn.make_bwd_args(t["q"], t["k"], t["v"], t["g"], t["beta"], do, grads, x["scale"], h0, dht, cu_dev, cu_host)
    L = gdn.lib()
    nbytes = int(L.gdn_bwd_workspace_bytes(ctypes.byref(args)))
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    run = lambda: gdn._check(L.gdn_bwd(ctypes.byref(args), ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(nbytes),
                                       ctypes.c_void_p(stream)))
    n_settle = settle(lambda i: run(), torch, a.settle_ms)
    for _ in range(a.warmup):
        run()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        ev[i][0].record()
        run()
        ev[i][1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = sum(e0.elapsed_time(e1) for e0, e1 in ev) / a.steps
    tokens = x["tokens"]
    H_qk = x["q"].shape[2]
    alg = algorithmic_bytes(x, esz) + N * H * D * Dv * 4     # q, k, v, dO, beta, g, h0, dht read, dh0 written
    alg += sum(grads[n].numel() for n in ("dq", "dk", "dv", "dg", "dbeta")) * 4   # gradients written (fp32)
    achieved = alg / (ms * 1e-3) / 1e9
    rec = {
        "metric": "GDN chunked backward tokens/s at 1 GPU + % of HBM roofline", "value": tokens * a.steps / elapsed,
        "unit": "tokens/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": elapsed / a.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": {2: "bf16", 4: "f32"}[esz],
        "data": "synthetic",
        "config": {"workload": w.name, "T_total": tokens, "seqs": N, "H_qk": H_qk, "H_v": H, "d_k": D, "d_v": Dv,
                   "chunk": 64, "gate": w.gate, "h0": w.h0},
        "roofline": {"bound": "hbm", "kernel": "whole backward", "alg_bytes": alg, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": None},
        "stage_ms": {"backward": ms},
        "clock_settle": {"ms": a.settle_ms, "untimed_steps": n_settle},
    }
    if not a.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_backward(x, do, dht)
    print(json.dumps(rec), flush=True)


def cpu_baseline_backward(x, do, dht, T=256, heads=2):
    """The fp64 autograd backward oracle on a bounded sample: the first T tokens of sequence 0 and
    its first `heads` value heads (with their query/key heads), scaled to tokens/s at the full head
    count."""
    import torch
    from chunkwise_linear_attention_chunk_amd import synth
    from oracle.backward import gdn_backward
    f64 = synth.to_f64
    H, Hq = x["v"].shape[2], x["q"].shape[2]
    hq = max(1, heads * Hq // H)
    sl = lambda a, hh: f64(a[:1, :T, :hh]) if a is not None else None
    args = [sl(x["q"], hq), sl(x["k"], hq), sl(x["v"], heads), sl(x["g"], heads), sl(x["beta"], heads)]
    h0 = None if x["h0"] is None else f64(x["h0"][:1, :heads])
    threads = torch.get_num_threads()
    t0 = time.perf_counter()
    gdn_backward(*args, x["scale"], f64(do.cpu()[:1, :T, :heads]), h0, f64(dht.cpu()[:1, :heads]))
    dt = time.perf_counter() - t0
    return {"value": T * heads / H / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"sequence 0, first {T} tokens, {heads} of {H} value heads (fp64 autograd through the token "
                      f"recurrence), scaled to all heads; {dt:.2f} s wall"}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {a.gpus}); "
              "heads and sequences would shard across GPUs with no communication.", file=sys.stderr)
        sys.exit(2)
    import torch
    from chunkwise_linear_attention_chunk_amd import gdn, synth

    dev = torch.device("cuda:0")
    torch.cuda.init()
    if a.copy_probe:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": src.numel() * 4, "copy_probe_bytes_written": dst.numel() * 4}))
        return

    if a.path == "decode":
        return bench_decode(a, torch, gdn, synth, dev)
    if a.path == "backward":
        return bench_backward(a, torch, gdn, synth, dev)
    rec, x = measure_prefill(a.workload, a.steps, a.warmup, a.copies, a.cp, a.cp_segment_chunks, torch, gdn, synth,
                             dev, a.settle_ms)
    if not a.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(x, a.cpu_threads)
    del x
    if not a.no_extras and a.workload == "qwen3next_bf16" and a.cp == "auto":
        rec["extra_configs"] = extra_configs(a, torch, gdn, synth, dev)
    print(json.dumps(rec), flush=True)


# The other configurations of the path, measured in the same run (one line each in extra_configs):
# (label, workload, cp mode).  The long-context workload is reported with exact context parallelism
# (the automatic choice) and, labelled, with its warmup form (an approximation with a stated bound).
EXTRAS = (("tiny_fp32", "tiny_fp32", "auto"), ("longctx_bf16", "longctx_bf16", "auto"),
          ("longctx_bf16_warmup_cp", "longctx_bf16", "warmup"), ("varlen_bf16", "varlen_bf16", "auto"),
          ("kda_bf16", "kda_bf16", "auto"))


def extra_configs(a, torch, gdn, synth, dev):
    out = {}
    for label, name, cp in EXTRAS:
        print(f"[bench] extra config {label}", file=sys.stderr, flush=True)
        r, x = measure_prefill(name, a.extra_steps, a.extra_warmup, a.copies, cp, 0, torch, gdn, synth, dev,
                               a.settle_ms)
        del x
        torch.cuda.empty_cache()
        out[label] = {"workload": name, "cp": cp, "cp_ran": r["config"]["cp_ran"],
                      "cp_segment_chunks": r["config"]["cp_segment_chunks"], "ms_per_step": r["ms_per_step"],
                      "tokens_per_s": r["value"], "dtype": r["dtype"],
                      "whole_op_roofline_frac": r["whole_op"]["roofline_frac"],
                      "dominant_kernel": r["roofline"]["kernel"], "dominant_kernel_frac": r["roofline"]["frac"],
                      "stage_ms": r["stage_ms"], "serial_chain": r["serial_chain"]}
    return out


def serial_chain(x, plan, chunk_ms):
    """The recurrence's serial chain: chunks per chain (a CP segment, else the longest sequence), the
    chunk step (recurrence time / chunks per chain: the time per chunk when every chain runs at once,
    an upper bound when the workgroups run in several rounds, as with many packed sequences), and the
    floor a chain over the longest sequence would take at that step without CP."""
    if x["cu_seqlens"] is not None:
        cu = x["cu_seqlens"].tolist()
        longest = max((b - a for a, b in zip(cu[:-1], cu[1:])), default=0)
    else:
        longest = x["q"].shape[1]
    seq_chunks = -(-longest // 64)
    chain = min(plan["segment_chunks"], seq_chunks) if plan["cp"] else seq_chunks
    step_us = chunk_ms * 1e3 / chain if chain else None
    return {"chunks_per_chain": chain, "chunk_step_us": step_us, "longest_sequence_chunks": seq_chunks,
            "no_cp_floor_ms": step_us * seq_chunks * 1e-3 if step_us else None}


def measure_prefill(name, steps, warmup, n_copies, cp, cp_segment_chunks, torch, gdn, synth, dev, settle_ms=0.0):
    """Time `steps` gdn_fwd_timed calls on workload `name` (after settling the clock and `warmup`
    untimed calls), rotating n_copies input copies.  Returns (record without cpu_baseline, host inputs)."""
    w = synth.workload(name)
    x = synth.make_inputs(w)
    esz = x["q"].element_size()
    names = ("q", "k", "v", "g", "beta")
    copies = []
    for _ in range(max(1, n_copies)):
        t = {n: x[n].to(dev) for n in names}
        t["h0"] = None if x["h0"] is None else x["h0"].to(dev)
        copies.append(t)
    cu_host = None if x["cu_seqlens"] is None else x["cu_seqlens"].to(torch.int32)
    cu_dev = None if cu_host is None else cu_host.to(dev)
    o = torch.empty(x["v"].shape, dtype=x["q"].dtype, device=dev)
    fs = torch.empty((x["n_seqs"],) + tuple(x["v"].shape[2:3]) + (x["q"].shape[3], x["v"].shape[3]),
                     dtype=torch.float32, device=dev)
    argv = [gdn.make_args(c["q"], c["k"], c["v"], c["g"], c["beta"], x["scale"], c["h0"], cu_dev, cu_host,
                          64, o, fs, cp, cp_segment_chunks) for c in copies]
    nbytes = gdn.workspace_bytes(argv[0])
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    hip = hip_runtime()
    n_ev = len(gdn.STAGES) + 1
    # The stage-end events only, without the system-scope fence (they serve timing alone): a start
    # event in each call's first dispatch cost about 5 us per step, so each step's first stage is
    # timed from the previous step's last event (the gap between the calls included) and the first
    # step's first stage is not timed.
    hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    events = []
    for _ in range(steps):
        arr = (ctypes.c_void_p * n_ev)()
        arr[0] = None
        for j in range(1, n_ev):
            ev = ctypes.c_void_p()
            if hip.hipEventCreateWithFlags(ctypes.byref(ev), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            arr[j] = ev.value
        events.append(arr)

    n_settle = settle(lambda i: gdn.fwd_raw(argv[i % len(argv)], ws.data_ptr(), ws.numel(), stream), torch, settle_ms)
    for i in range(warmup):
        gdn.fwd_raw(argv[i % len(argv)], ws.data_ptr(), ws.numel(), stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ran = []
    for i in range(steps):
        ran.append(gdn.fwd_timed_raw(argv[i % len(argv)], ws.data_ptr(), ws.numel(), stream, events[i]))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    stage_ms = {s: 0.0 for s in gdn.STAGES}
    counts = {s: 0 for s in gdn.STAGES}
    prev = None  # the last recorded boundary (the previous step's last event at a step's start)
    for arr, mask in zip(events, ran):
        for j, s in enumerate(gdn.STAGES):
            if not (mask >> j) & 1:
                continue
            if prev is not None:
                ms = ctypes.c_float()
                if hip.hipEventElapsedTime(ctypes.byref(ms), prev, arr[j + 1]) != 0:
                    raise RuntimeError("hipEventElapsedTime failed")
                stage_ms[s] += ms.value
                counts[s] += 1
            prev = arr[j + 1]
    for s in gdn.STAGES:
        stage_ms[s] = stage_ms[s] / counts[s] if counts[s] else 0.0
    for arr in events:
        for j in range(1, n_ev):
            hip.hipEventDestroy(arr[j])
    plan = gdn.plan(argv[0])
    dominant = max(("intra", "cp_pre", "chunk"), key=lambda s: stage_ms[s])
    alg_bytes = algorithmic_bytes(x, esz)
    alg_bytes_dom = stage_algorithmic_bytes(dominant, x, esz, plan)
    t_dom = stage_ms[dominant] * 1e-3
    achieved = alg_bytes_dom / t_dom / 1e9
    ms_step = elapsed / steps * 1e3
    value = x["tokens"] * steps / elapsed
    t_bound = max(alg_bytes / (HBM_PEAK_GBS * 1e9), algorithmic_flops(x) / (BF16_PEAK_TFLOPS * 1e12))
    rec = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": {2: "bf16", 4: "f32"}[esz], "data": "synthetic",
        "config": {"workload": w.name, "B": w.B if not w.n_seqs else 1, "T_total": x["tokens"],
                   "seqs": x["n_seqs"], "H_qk": w.hqk, "H_v": w.H, "d_k": w.D, "d_v": w.D,
                   "chunk": 64, "gate": w.gate, "h0": w.h0, "input_copies": len(copies),
                   "cp": cp, "cp_ran": bool((ran[-1] >> gdn.STAGES.index("cp_pre")) & 1),
                   "cp_segment_chunks": plan["segment_chunks"] if plan["cp"] else None,
                   "value_cols_per_group": plan["value_cols_per_group"], "pieces": plan["pieces"]},
        "roofline": {"bound": "hbm", "kernel": dominant, "alg_bytes": alg_bytes_dom, "achieved": achieved,
                     "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(dominant, w.name)},
        "stage_ms": stage_ms,
        "whole_op": {"alg_bytes": alg_bytes, "alg_flops": algorithmic_flops(x), "t_bound_ms": t_bound * 1e3,
                     "roofline_frac": t_bound / (ms_step * 1e-3)},
        "clock_settle": {"ms": settle_ms, "untimed_steps": n_settle},
        "serial_chain": serial_chain(x, plan, stage_ms["chunk"]),
    }
    del copies, argv, ws, o, fs
    return rec, x


if __name__ == "__main__":
    main()
