"""C-ABI checks that need no GPU: exported symbols, struct layout, argument validation, planning.

Validation runs before any launch, so every error path here returns without touching HIP.
"""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from chunkwise_linear_attention_chunk_amd import gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    names = _declared_functions()
    assert {"gdn_fwd", "gdn_fwd_timed", "gdn_fwd_workspace_bytes", "gdn_fwd_plan", "gdn_fwd_recurrent",
            "gdn_status_string", "gdn_last_error"} <= set(names)
    lib = ctypes.CDLL(gdn.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} is declared in gdn.h but not exported"
    assert set(gdn.EXPORTED) == set(names)


def test_struct_layout_matches_header():
    fields = [f[0] for f in gdn.FwdArgs._fields_]
    src = "#include <stdio.h>\n#include <stddef.h>\n#include \"gdn.h\"\nint main(void){\n"
    src += 'printf("%zu\\n", sizeof(gdn_fwd_args));\n'
    src += "".join(f'printf("%zu\\n", offsetof(gdn_fwd_args, {f}));\n' for f in fields)
    src += "return 0;}\n"
    with tempfile.TemporaryDirectory() as d:
        c, exe = os.path.join(d, "probe.c"), os.path.join(d, "probe")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), c, "-o", exe], check=True)
        out = [int(x) for x in subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()]
    assert out[0] == ctypes.sizeof(gdn.FwdArgs)
    for f, off in zip(fields, out[1:]):
        assert getattr(gdn.FwdArgs, f).offset == off, f"field {f}: ctypes {getattr(gdn.FwdArgs, f).offset} vs C {off}"


def test_backward_struct_layout_matches_header():
    fields = [f[0] for f in gdn.BwdArgs._fields_]
    src = "#include <stdio.h>\n#include <stddef.h>\n#include \"gdn.h\"\nint main(void){\n"
    src += 'printf("%zu\\n", sizeof(gdn_bwd_args));\n'
    src += "".join(f'printf("%zu\\n", offsetof(gdn_bwd_args, {f}));\n' for f in fields)
    src += "return 0;}\n"
    with tempfile.TemporaryDirectory() as d:
        c, exe = os.path.join(d, "probe.c"), os.path.join(d, "probe")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), c, "-o", exe], check=True)
        out = [int(x) for x in subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()]
    assert out[0] == ctypes.sizeof(gdn.BwdArgs)
    for f, off in zip(fields, out[1:]):
        assert getattr(gdn.BwdArgs, f).offset == off, f"field {f}"


def test_backward_validation():
    a = gdn.BwdArgs()
    a.B, a.T, a.H_qk, a.H_v, a.D_k, a.D_v, a.N = 1, 100, 2, 2, 64, 64, 1
    a.chunk_size, a.dtype, a.gate_kind, a.scale = 64, gdn.DTYPE_F32, gdn.GATE_SCALAR, 0.125
    fake = ctypes.c_void_p(0x1000)
    a.q = a.k = a.v = a.g = a.beta = a.dout = fake
    L = gdn.lib()
    assert L.gdn_bwd(ctypes.byref(a), None, 0, None) == gdn.GDN_ERR_INVALID_ARG     # no gradient outputs
    assert "dq, dk, dv" in L.gdn_last_error().decode()
    a.dq = a.dk = a.dv = a.dg = a.dbeta = fake
    n = L.gdn_bwd_workspace_bytes(ctypes.byref(a))
    assert n >= 2 * 2 * 2 * 64 * 64 * 4                                              # states and dS per chunk
    assert L.gdn_bwd(ctypes.byref(a), None, 0, None) == gdn.GDN_ERR_WORKSPACE
    a.gate_kind = gdn.GATE_CHANNEL                                                   # both gate kinds
    assert L.gdn_bwd_workspace_bytes(ctypes.byref(a)) > n                            # + V' and dL per chunk
    assert L.gdn_bwd(ctypes.byref(a), None, 0, None) == gdn.GDN_ERR_WORKSPACE
    a.gate_kind, a.chunk_size = gdn.GATE_SCALAR, 32
    assert L.gdn_bwd(ctypes.byref(a), None, 0, None) == gdn.GDN_ERR_UNSUPPORTED


def test_status_strings():
    lib = gdn.lib()
    for code, name in enumerate(["GDN_OK", "GDN_ERR_INVALID_ARG", "GDN_ERR_UNSUPPORTED", "GDN_ERR_WORKSPACE",
                                 "GDN_ERR_HIP"]):
        assert lib.gdn_status_string(code).decode() == name


def _args(**kw):
    a = gdn.FwdArgs()
    a.B, a.T, a.H_qk, a.H_v, a.D_k, a.D_v = 2, 300, 4, 8, 128, 128
    a.chunk_size, a.dtype, a.gate_kind, a.scale, a.N = 64, gdn.DTYPE_BF16, gdn.GATE_SCALAR, 0.088, 2
    a.o_dtype = gdn.DTYPE_BF16
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every case fails validation or sizing first
    a.q = a.k = a.v = a.g = a.beta = a.o = fake
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _status(a, workspace=None, nbytes=0):
    return gdn.lib().gdn_fwd(ctypes.byref(a), workspace, nbytes, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(chunk_size=48), gdn.GDN_ERR_INVALID_ARG, "power of two"),
    (dict(chunk_size=32), gdn.GDN_ERR_UNSUPPORTED, "chunk_size"),
    (dict(D_k=512, D_v=512), gdn.GDN_ERR_UNSUPPORTED, "D_k=512"),
    (dict(D_k=96), gdn.GDN_ERR_UNSUPPORTED, "D_k=96"),
    (dict(H_v=6), gdn.GDN_ERR_INVALID_ARG, "multiple"),
    (dict(dtype=7), gdn.GDN_ERR_INVALID_ARG, "dtype"),
    (dict(o_dtype=gdn.DTYPE_BF16, dtype=gdn.DTYPE_F32), gdn.GDN_ERR_INVALID_ARG, "o_dtype"),
    (dict(N=3), gdn.GDN_ERR_INVALID_ARG, "N=3"),
    (dict(q=None), gdn.GDN_ERR_INVALID_ARG, "required"),
    (dict(B=-1), gdn.GDN_ERR_INVALID_ARG, "B=-1"),
    (dict(cp_mode=9), gdn.GDN_ERR_INVALID_ARG, "cp_mode"),
    (dict(cp_mode=3, cp_warmup_tol=1.0), gdn.GDN_ERR_INVALID_ARG, "cp_warmup_tol"),
    (dict(cp_warmup_tol=-0.5), gdn.GDN_ERR_INVALID_ARG, "cp_warmup_tol"),
    (dict(cp_warmup_tol=float("nan")), gdn.GDN_ERR_INVALID_ARG, "cp_warmup_tol"),
    (dict(scale=float("nan")), gdn.GDN_ERR_INVALID_ARG, "scale"),
    (dict(qk_l2norm=2), gdn.GDN_ERR_INVALID_ARG, "qk_l2norm"),
    (dict(beta_sigmoid=-1), gdn.GDN_ERR_INVALID_ARG, "beta_sigmoid"),
    (dict(dt_bias=ctypes.c_void_p(0x3000)), gdn.GDN_ERR_INVALID_ARG, "need A_log"),
    (dict(gate_lower_bound=-5.0), gdn.GDN_ERR_INVALID_ARG, "need A_log"),
    (dict(A_log=ctypes.c_void_p(0x3000), gate_lower_bound=2.0), gdn.GDN_ERR_INVALID_ARG, "gate_lower_bound"),
    (dict(A_log=ctypes.c_void_p(0x3000), gate_lower_bound=float("-inf")), gdn.GDN_ERR_INVALID_ARG, "gate_lower_bound"),
])
def test_invalid_arguments_are_rejected_before_launch(kw, status, msg):
    a = _args(**kw)
    assert _status(a) == status
    assert msg in gdn.lib().gdn_last_error().decode()
    assert gdn.workspace_bytes(a) == 0


@pytest.mark.parametrize("kw,status,msg", [
    (dict(chunk_size=64), gdn.GDN_ERR_UNSUPPORTED, "takes 1"),
    (dict(D_k=96), gdn.GDN_ERR_UNSUPPORTED, "D_k=96"),
    (dict(H_v=6), gdn.GDN_ERR_INVALID_ARG, "multiple"),
    (dict(N=3), gdn.GDN_ERR_INVALID_ARG, "N=3"),
    (dict(v=None), gdn.GDN_ERR_INVALID_ARG, "required"),
    (dict(o_dtype=gdn.DTYPE_BF16, dtype=gdn.DTYPE_F32), gdn.GDN_ERR_INVALID_ARG, "o_dtype"),
    (dict(dt_bias=ctypes.c_void_p(0x3000)), gdn.GDN_ERR_INVALID_ARG, "need A_log"),
])
def test_recurrent_entry_validates_before_launch(kw, status, msg):
    a = _args(**{"chunk_size": 1, **kw})
    assert gdn.lib().gdn_fwd_recurrent(ctypes.byref(a), None) == status
    assert msg in gdn.lib().gdn_last_error().decode()


def test_chunked_entry_rejects_chunk_size_one():
    a = _args(chunk_size=1)
    assert _status(a) == gdn.GDN_ERR_UNSUPPORTED
    assert "takes 64" in gdn.lib().gdn_last_error().decode()


def _packed(cu, **kw):
    arr = (ctypes.c_int32 * len(cu))(*cu)
    kw = {"T": cu[-1], **kw}
    a = _args(B=1, N=len(cu) - 1, cu_seqlens_host=ctypes.cast(arr, ctypes.c_void_p),
              cu_seqlens_dev=ctypes.c_void_p(0x2000), **kw)
    return a, arr


@pytest.mark.parametrize("cu,msg", [([1, 5, 9], "cu_seqlens[0]"), ([0, 9, 5], "decreases"), ([0, 4, 9], None)])
def test_packed_sequence_validation(cu, msg):
    a, keep = _packed(cu, T=8) if msg is None else _packed(cu)
    assert _status(a) == gdn.GDN_ERR_INVALID_ARG
    assert (msg or "!= T") in gdn.lib().gdn_last_error().decode()


def test_packed_needs_single_batch_row_and_host_copy():
    a, keep = _packed([0, 10, 20])
    a.B = 2
    assert _status(a) == gdn.GDN_ERR_INVALID_ARG
    a, keep = _packed([0, 10, 20])
    a.cu_seqlens_host = None
    assert _status(a) == gdn.GDN_ERR_INVALID_ARG


def test_workspace_size_and_checks():
    a = _args()
    n = gdn.workspace_bytes(a)
    # per chunk-head (scalar gate): A [64][64] bf16 and a 2 KiB gate block (the recurrence forms P
    # itself); ceil(300/64) = 5 chunks per sequence x 2 sequences x 8 heads, plus small tables
    per = 64 * 64 * 2 + 512 * 4
    assert n >= 10 * 8 * per
    assert n < 10 * 8 * per + 4096
    assert _status(a, None, 0) == gdn.GDN_ERR_WORKSPACE
    assert _status(a, ctypes.c_void_p(0x10000), n - 1) == gdn.GDN_ERR_WORKSPACE
    assert _status(a, ctypes.c_void_p(0x10001), n) == gdn.GDN_ERR_WORKSPACE  # misaligned
    assert "aligned" in gdn.lib().gdn_last_error().decode()
    # packed lengths change the chunk count: ceil(1/64) + ceil(64/64) + ceil(65/64) = 4 chunks
    p, keep = _packed([0, 1, 65, 130])
    assert gdn.workspace_bytes(p) >= 4 * 8 * per
    assert gdn.workspace_bytes(p) < 4 * 8 * per + 4096


def test_workspace_with_context_parallelism():
    # CP on with 2-chunk segments: 5 chunks per sequence -> 3 segments each, 6 in all; per segment
    # and head the workspace holds S* [128][128], M [128][128] and the start state [128][128] in fp32
    base = gdn.workspace_bytes(_args(cp_mode=gdn.CP_MODES["off"]))
    on = gdn.workspace_bytes(_args(cp_mode=gdn.CP_MODES["on"], cp_segment_chunks=2))
    maps = 6 * 8 * 3 * 128 * 128 * 4
    assert maps <= on - base < maps + 4096
    # warmup CP: no maps, one int (the warmup length) per segment and head
    warm = gdn.workspace_bytes(_args(cp_mode=gdn.CP_MODES["warmup"], cp_segment_chunks=2))
    assert 6 * 8 * 4 <= warm - base < 6 * 8 * 4 + 4096
    info = gdn.plan(_args(cp_mode=gdn.CP_MODES["warmup"], cp_segment_chunks=2))
    assert info["cp"] == 1 and info["segment_chunks"] == 2 and info["total_segments"] == 6
    # automatic choice: B*H_v = 4 with 1024 chunks splits the sequence; B*H_v = 64 does not
    per = 64 * 64 * 2 + 512 * 4
    long = gdn.workspace_bytes(_args(B=1, N=1, T=65536, H_qk=4, H_v=4))
    assert long > 1024 * 4 * per + 4 * 3 * 128 * 128 * 4
    wide = gdn.workspace_bytes(_args(B=4, N=4, T=4096, H_qk=16, H_v=16))
    assert wide < 4 * 64 * 16 * per + 4096
    info = gdn.plan(_args(B=4, N=4, T=4096, H_qk=16, H_v=16))
    assert info["cp"] == 0 and info["pieces"] == 1


def test_workspace_with_pieces(monkeypatch):
    # GDN_PIECES=4 without CP: four ranges of 16 chunks, the start states of ranges 1..3 in fp32
    monkeypatch.setenv("GDN_PIECES", "4")
    per = 64 * 64 * 2 + 512 * 4
    wide = gdn.workspace_bytes(_args(B=4, N=4, T=4096, H_qk=16, H_v=16))
    pieces = 4 * 4 * 16 * 128 * 128 * 4
    assert pieces + 4 * 64 * 16 * per <= wide < pieces + 4 * 64 * 16 * per + 4096
    assert gdn.plan(_args(B=4, N=4, T=4096, H_qk=16, H_v=16))["pieces"] == 4


def test_plan_query():
    # the long-context shape (B * H_v = 4) splits its 1024 chunks into segments
    a = _args(B=1, N=1, T=65536, H_qk=4, H_v=4)
    info = gdn.plan(a)
    assert info["cp"] == 1 and info["value_cols_per_group"] == 32
    assert info["total_segments"] == -(-1024 // info["segment_chunks"])
    assert info["workspace_bytes"] == gdn.workspace_bytes(a)
    off = gdn.plan(_args(B=1, N=1, T=65536, H_qk=4, H_v=4, cp_mode=gdn.CP_MODES["off"]))
    assert off["cp"] == 0 and off["pieces"] == 1 and off["total_segments"] == 1 and off["segment_chunks"] == 1024
    with pytest.raises(gdn.GdnError):
        gdn.plan(_args(chunk_size=48))


def test_plan_reports_the_pre_process_form():
    # the long-context shape: the automatic segment length (64 chunks) leaves 16 x 4 (segment,
    # head) pairs, fewer than the compute units, so the chain form; 16-chunk segments give 64 x 4,
    # and the X/Y/Z form (the plan assumes 256 compute units when no device answers)
    long = dict(B=1, N=1, T=65536, H_qk=4, H_v=4)
    assert gdn.plan(_args(**long))["cp_form"] == gdn.CP_FORMS["chain"]
    assert gdn.plan(_args(**long, cp_segment_chunks=16))["cp_form"] == gdn.CP_FORMS["xyz"]
    assert gdn.plan(_args(**long, cp_segment_chunks=16, cp_form=gdn.CP_FORMS["chain"]))["cp_form"] == gdn.CP_FORMS["chain"]
    assert gdn.plan(_args(**long, cp_form=gdn.CP_FORMS["xyz"]))["cp_form"] == gdn.CP_FORMS["xyz"]
    # no exact pre-process: no form
    assert gdn.plan(_args(**long, cp_mode=gdn.CP_MODES["off"]))["cp_form"] == 0
    assert gdn.plan(_args(**long, cp_mode=gdn.CP_MODES["warmup"]))["cp_form"] == 0
    # the X/Y/Z form is bf16 with a scalar gate only; out-of-range forms are invalid
    for kw in (dict(dtype=gdn.DTYPE_F32, o_dtype=gdn.DTYPE_F32), dict(gate_kind=gdn.GATE_CHANNEL)):
        assert _status(_args(**long, cp_form=gdn.CP_FORMS["xyz"], **kw)) == gdn.GDN_ERR_UNSUPPORTED
        assert "XYZ" in gdn.lib().gdn_last_error().decode()
    assert _status(_args(cp_form=3)) == gdn.GDN_ERR_INVALID_ARG
    assert "cp_form" in gdn.lib().gdn_last_error().decode()


def test_backward_gradient_shapes_are_checked_on_the_host():
    # the kernels write dg shaped like g ([B, T, H_v, D_k] per channel): a buffer shaped like beta
    # must be rejected before anything is launched
    import torch
    from chunkwise_linear_attention_chunk_amd import synth
    x = synth.make_inputs(synth.workload("kda_bf16", B=1, H=2, T=64))
    t = {n: x[n] for n in ("q", "k", "v", "g", "beta")}
    f32 = dict(dtype=torch.float32)
    grads = {"dq": torch.empty(t["q"].shape, **f32), "dk": torch.empty(t["k"].shape, **f32),
             "dv": torch.empty(t["v"].shape, **f32), "dg": torch.empty(t["g"].shape, **f32),
             "dbeta": torch.empty(t["beta"].shape, **f32)}
    gdn.make_bwd_args(t["q"], t["k"], t["v"], t["g"], t["beta"], t["v"], grads, x["scale"])
    with pytest.raises(gdn.GdnError, match="dg must be"):
        gdn.make_bwd_args(t["q"], t["k"], t["v"], t["g"], t["beta"], t["v"], dict(grads, dg=torch.empty(t["beta"].shape, **f32)),
                          x["scale"])


def test_noalloc_entry_validates_and_bounds_its_scratch():
    # gdn_fwd_noalloc validates like gdn_fwd and rejects work whose workspace exceeds the static
    # scratch array, before touching the GPU (no launch, no scratch lookup)
    L = gdn.lib()
    a = _args(chunk_size=48)
    assert L.gdn_fwd_noalloc(ctypes.byref(a), None) == gdn.GDN_ERR_INVALID_ARG
    assert "power of two" in L.gdn_last_error().decode()
    big = _args(B=16, N=16, T=8192, H_qk=16, H_v=16, cp_mode=gdn.CP_MODES["off"])
    need = gdn.workspace_bytes(big)
    assert need > gdn.NOALLOC_SCRATCH_BYTES
    assert L.gdn_fwd_noalloc(ctypes.byref(big), None) == gdn.GDN_ERR_WORKSPACE
    msg = L.gdn_last_error().decode()
    assert str(need) in msg and str(gdn.NOALLOC_SCRATCH_BYTES) in msg
    # the Qwen3-Next-shaped workload fits
    assert gdn.workspace_bytes(_args(B=4, N=4, T=4096, H_qk=16, H_v=16)) <= gdn.NOALLOC_SCRATCH_BYTES


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define GDN_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == gdn.NOALLOC_SCRATCH_BYTES


def _cpu_inputs(gate="scalar"):
    import torch
    from chunkwise_linear_attention_chunk_amd import synth
    name = "qwen3next_bf16" if gate == "scalar" else "kda_bf16"
    x = synth.make_inputs(synth.workload(name, B=2, H=4, T=70, h0=True, seed=1))
    return torch, x


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_binding_rejects_mismatched_inputs_before_any_call(gate):
    # the C ABI sees only pointers, so the binding checks every tensor's shape and dtype on the host
    torch, x = _cpu_inputs(gate)
    q, k, v, g, beta, h0 = (x[n] for n in ("q", "k", "v", "g", "beta", "h0"))
    gdn.make_args(q, k, v, g, beta, x["scale"], h0)                  # consistent inputs pass
    bad = {
        "k": dict(k=k[:, :, :, :64].contiguous()),
        "v": dict(v=v[:, :50].contiguous()),
        "g": dict(g=g.to(torch.bfloat16) if gate == "scalar" else g.float()),
        "beta": dict(beta=beta.float()),
        "initial_state": dict(h0=h0.to(torch.bfloat16)),
    }
    for name, over in bad.items():
        args = {**dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0), **over}
        with pytest.raises(gdn.GdnError, match=name):
            gdn.make_args(args["q"], args["k"], args["v"], args["g"], args["beta"], x["scale"], args["h0"])
    with pytest.raises(gdn.GdnError, match="initial_state"):
        gdn.make_args(q, k, v, g, beta, x["scale"], h0[:1].contiguous())
    with pytest.raises(gdn.GdnError, match="A_log"):
        gdn.make_args(q, k, v, g, beta, x["scale"], h0, A_log=torch.zeros(3))
    dtb = torch.zeros(4, 128) if gate == "scalar" else torch.zeros(4)
    with pytest.raises(gdn.GdnError, match="dt_bias"):
        gdn.make_args(q, k, v, g, beta, x["scale"], h0, A_log=torch.zeros(4), dt_bias=dtb)
    with pytest.raises(gdn.GdnError, match="final_state"):
        gdn.make_args(q, k, v, g, beta, x["scale"], h0, final_state=torch.zeros(2, 4, 128, 64))
    with pytest.raises(gdn.GdnError, match="o must be"):
        gdn.make_args(q, k, v, g, beta, x["scale"], h0, o=torch.zeros(v.shape, dtype=torch.float16))


def test_binding_checks_backward_inputs():
    torch, x = _cpu_inputs()
    q, k, v, g, beta = (x[n] for n in ("q", "k", "v", "g", "beta"))
    f32 = dict(dtype=torch.float32)
    grads = {"dq": torch.empty(q.shape, **f32), "dk": torch.empty(k.shape, **f32), "dv": torch.empty(v.shape, **f32),
             "dg": torch.empty(g.shape, **f32), "dbeta": torch.empty(beta.shape, **f32)}
    with pytest.raises(gdn.GdnError, match="dout"):
        gdn.make_bwd_args(q, k, v, g, beta, v.float(), grads, x["scale"])
    with pytest.raises(gdn.GdnError, match="dht"):
        gdn.make_bwd_args(q, k, v, g, beta, v, grads, x["scale"], dht=torch.zeros(2, 4, 64, 128))
