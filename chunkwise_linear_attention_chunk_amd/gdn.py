"""Thin ctypes binding of libgdn (include/gdn.h): argument marshalling only.

Every step of the forward runs in the HIP kernels behind ``gdn_fwd``; PyTorch is
used here for device memory (outputs and the workspace) and for the current
stream.  There is no fallback: if ``libgdn.so`` has not been built, or a tensor
is not on a GPU, the call raises.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_OK, GDN_ERR_INVALID_ARG, GDN_ERR_UNSUPPORTED, GDN_ERR_WORKSPACE, GDN_ERR_HIP = range(5)
DTYPE_F32, DTYPE_BF16 = 0, 1
GATE_SCALAR, GATE_CHANNEL = 0, 1
CP_MODES = {"auto": 0, "off": 1, "on": 2, "warmup": 3}
CP_FORMS = {"auto": 0, "chain": 1, "xyz": 2}
EXPORTED = ("gdn_fwd", "gdn_fwd_timed", "gdn_fwd_workspace_bytes", "gdn_fwd_plan", "gdn_fwd_noalloc",
            "gdn_fwd_recurrent", "gdn_bwd", "gdn_bwd_workspace_bytes", "gdn_status_string", "gdn_last_error")
NOALLOC_SCRATCH_BYTES = 64 << 20   # GDN_NOALLOC_SCRATCH_BYTES of include/gdn.h
STAGES = ("plan", "intra", "cp_pre", "cp_fix", "chunk")  # order of gdn_fwd_timed's stages


class GdnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(message)
        self.status = status


class FwdArgs(ctypes.Structure):
    """Mirror of gdn_fwd_args."""
    _fields_ = [
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H_qk", ctypes.c_int32), ("H_v", ctypes.c_int32),
        ("D_k", ctypes.c_int32), ("D_v", ctypes.c_int32), ("chunk_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("gate_kind", ctypes.c_int32), ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("g", ctypes.c_void_p),
        ("beta", ctypes.c_void_p), ("h0", ctypes.c_void_p), ("cu_seqlens_dev", ctypes.c_void_p),
        ("cu_seqlens_host", ctypes.c_void_p), ("N", ctypes.c_int32), ("o", ctypes.c_void_p),
        ("final_state", ctypes.c_void_p), ("cp_mode", ctypes.c_int32), ("cp_segment_chunks", ctypes.c_int32),
        ("o_dtype", ctypes.c_int32),
        ("qk_l2norm", ctypes.c_int32), ("beta_sigmoid", ctypes.c_int32), ("A_log", ctypes.c_void_p),
        ("dt_bias", ctypes.c_void_p), ("gate_lower_bound", ctypes.c_float), ("cp_warmup_tol", ctypes.c_float),
        ("cp_form", ctypes.c_int32),
    ]


class BwdArgs(ctypes.Structure):
    """Mirror of gdn_bwd_args."""
    _fields_ = [
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H_qk", ctypes.c_int32), ("H_v", ctypes.c_int32),
        ("D_k", ctypes.c_int32), ("D_v", ctypes.c_int32), ("chunk_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("gate_kind", ctypes.c_int32), ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("g", ctypes.c_void_p),
        ("beta", ctypes.c_void_p), ("h0", ctypes.c_void_p), ("cu_seqlens_dev", ctypes.c_void_p),
        ("cu_seqlens_host", ctypes.c_void_p), ("N", ctypes.c_int32), ("dout", ctypes.c_void_p),
        ("dht", ctypes.c_void_p), ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("dg", ctypes.c_void_p), ("dbeta", ctypes.c_void_p), ("dh0", ctypes.c_void_p),
    ]


class PlanInfo(ctypes.Structure):
    """Mirror of gdn_plan_info."""
    _fields_ = [("cp", ctypes.c_int32), ("segment_chunks", ctypes.c_int32), ("total_segments", ctypes.c_int64),
                ("value_cols_per_group", ctypes.c_int32), ("pieces", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_size_t), ("cp_form", ctypes.c_int32)]


_lib = None


def lib():
    """Load libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise GdnError(GDN_ERR_HIP, f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.gdn_fwd_workspace_bytes.argtypes = [ctypes.POINTER(FwdArgs)]
        L.gdn_fwd_workspace_bytes.restype = ctypes.c_size_t
        L.gdn_fwd.argtypes = [ctypes.POINTER(FwdArgs), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.gdn_fwd.restype = ctypes.c_int
        L.gdn_fwd_timed.argtypes = [ctypes.POINTER(FwdArgs), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint32)]
        L.gdn_fwd_timed.restype = ctypes.c_int
        L.gdn_fwd_plan.argtypes = [ctypes.POINTER(FwdArgs), ctypes.POINTER(PlanInfo)]
        L.gdn_fwd_plan.restype = ctypes.c_int
        L.gdn_bwd_workspace_bytes.argtypes = [ctypes.POINTER(BwdArgs)]
        L.gdn_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.gdn_bwd.argtypes = [ctypes.POINTER(BwdArgs), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.gdn_bwd.restype = ctypes.c_int
        L.gdn_fwd_noalloc.argtypes = [ctypes.POINTER(FwdArgs), ctypes.c_void_p]
        L.gdn_fwd_noalloc.restype = ctypes.c_int
        L.gdn_fwd_recurrent.argtypes = [ctypes.POINTER(FwdArgs), ctypes.c_void_p]
        L.gdn_fwd_recurrent.restype = ctypes.c_int
        L.gdn_status_string.argtypes = [ctypes.c_int]
        L.gdn_status_string.restype = ctypes.c_char_p
        L.gdn_last_error.argtypes = []
        L.gdn_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(status):
    if status != GDN_OK:
        L = lib()
        raise GdnError(status, f"{L.gdn_status_string(status).decode()}: {L.gdn_last_error().decode()}")


def _expect(name, t, shape, dtype):
    """Raise GdnError unless tensor t (if given) is contiguous with this shape and dtype: the C ABI
    takes plain pointers and cannot see sizes or element types."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise GdnError(GDN_ERR_INVALID_ARG, f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} "
                                            f"(got {t.dtype} {tuple(t.shape)})")


def check_inputs(q, k, v, g, beta, initial_state=None, cu_seqlens=None, A_log=None, dt_bias=None, o=None,
                 final_state=None, dout=None, dht=None):
    """Host-side shape and dtype checks of every tensor the kernels read or write (include/gdn.h
    layouts).  Returns (B, T, H_qk, D_k, H_v, D_v, N, gate kind)."""
    if q.dim() != 4:
        raise GdnError(GDN_ERR_INVALID_ARG, "q must be [B, T, H_qk, D_k]")
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise GdnError(GDN_ERR_UNSUPPORTED, f"dtype {q.dtype} (supported: float32, bfloat16)")
    B, T, H_qk, D_k = q.shape
    if v.dim() != 4 or tuple(v.shape[:2]) != (B, T):
        raise GdnError(GDN_ERR_INVALID_ARG, f"v must be [B={B}, T={T}, H_v, D_v] (got {tuple(v.shape)})")
    H_v, D_v = v.shape[2], v.shape[3]
    if g.dim() not in (3, 4):
        raise GdnError(GDN_ERR_INVALID_ARG, "g must be [B, T, H_v] (scalar gate) or [B, T, H_v, D_k] (per channel)")
    gate = GATE_SCALAR if g.dim() == 3 else GATE_CHANNEL
    if cu_seqlens is not None and (cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2
                                   or cu_seqlens.dtype not in (torch.int32, torch.int64)):
        raise GdnError(GDN_ERR_INVALID_ARG, "cu_seqlens must be a 1-D integer tensor of N + 1 offsets")
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    _expect("k", k, q.shape, q.dtype)
    _expect("v", v, v.shape, q.dtype)
    if gate == GATE_SCALAR:
        _expect("g", g, (B, T, H_v), torch.float32)
    else:
        _expect("g", g, (B, T, H_v, D_k), q.dtype)
    _expect("beta", beta, (B, T, H_v), q.dtype)
    state = (N, H_v, D_k, D_v)
    _expect("initial_state", initial_state, state, torch.float32)
    _expect("final_state", final_state, state, torch.float32)
    _expect("A_log", A_log, (H_v,), torch.float32)
    _expect("dt_bias", dt_bias, (H_v,) if gate == GATE_SCALAR else (H_v, D_k), torch.float32)
    if o is not None:
        _expect("o", o, v.shape, o.dtype if o.dtype in (q.dtype, torch.float32) else q.dtype)
    _expect("dout", dout, v.shape, q.dtype)
    _expect("dht", dht, state, torch.float32)
    return B, T, H_qk, D_k, H_v, D_v, N, gate


def make_args(q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None, cu_seqlens_cpu=None,
              chunk_size=64, o=None, final_state=None, cp_mode="auto", cp_segment_chunks=0,
              qk_l2norm=False, beta_sigmoid=False, A_log=None, dt_bias=None, gate_lower_bound=0.0,
              cp_warmup_tol=0.0, cp_form="auto"):
    """Fill a gdn_fwd_args from tensors (shapes and dtypes are checked, nothing is computed)."""
    B, T, H_qk, D_k, H_v, D_v, N, gate = check_inputs(q, k, v, g, beta, initial_state, cu_seqlens, A_log, dt_bias,
                                                      o, final_state)
    dt = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}[q.dtype]
    a = FwdArgs()
    a.B, a.T, a.H_qk, a.H_v, a.D_k, a.D_v = B, T, H_qk, H_v, D_k, D_v
    a.chunk_size, a.dtype, a.gate_kind = chunk_size, dt, gate
    a.scale = float(D_k ** -0.5 if scale is None else scale)
    a.q, a.k, a.v, a.g, a.beta = (_ptr(t) for t in (q, k, v, g, beta))
    a.h0 = _ptr(initial_state)
    a.cu_seqlens_dev = _ptr(cu_seqlens)
    a.cu_seqlens_host = _ptr(cu_seqlens_cpu)
    a.N = N
    a.o = _ptr(o)
    a.final_state = _ptr(final_state)
    a.cp_mode = CP_MODES[cp_mode] if isinstance(cp_mode, str) else int(cp_mode)
    a.cp_segment_chunks = int(cp_segment_chunks)
    a.o_dtype = dt if o is None else {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}[o.dtype]
    a.qk_l2norm, a.beta_sigmoid = int(bool(qk_l2norm)), int(bool(beta_sigmoid))
    a.A_log, a.dt_bias = _ptr(A_log), _ptr(dt_bias)
    a.gate_lower_bound = float(gate_lower_bound)
    a.cp_warmup_tol = float(cp_warmup_tol)
    a.cp_form = CP_FORMS[cp_form] if isinstance(cp_form, str) else int(cp_form)
    return a


def _require_gpu(name, t):
    if t is not None and (not t.is_cuda or not t.is_contiguous()):
        raise GdnError(GDN_ERR_INVALID_ARG, f"{name} must be a contiguous GPU tensor")


def workspace_bytes(args):
    return int(lib().gdn_fwd_workspace_bytes(ctypes.byref(args)))


def plan(args):
    """The schedule gdn_fwd would use: dict(cp, segment_chunks, total_segments, value_cols_per_group,
    pieces, workspace_bytes).  Host-only; raises on invalid arguments."""
    info = PlanInfo()
    _check(lib().gdn_fwd_plan(ctypes.byref(args), ctypes.byref(info)))
    return {f: getattr(info, f) for f, _ in PlanInfo._fields_}


def fwd_raw(args, workspace, workspace_bytes_, stream):
    """Call gdn_fwd with a prepared FwdArgs, a workspace pointer (int) and a stream handle (int)."""
    _check(lib().gdn_fwd(ctypes.byref(args), ctypes.c_void_p(workspace), ctypes.c_size_t(workspace_bytes_),
                         ctypes.c_void_p(stream)))


def fwd_noalloc_raw(args, stream):
    """Call gdn_fwd_noalloc (no workspace argument: the library's static device scratch) with a
    prepared FwdArgs and a stream handle (int)."""
    _check(lib().gdn_fwd_noalloc(ctypes.byref(args), ctypes.c_void_p(stream)))


def fwd_timed_raw(args, workspace, workspace_bytes_, stream, events):
    """gdn_fwd_timed with events = a ctypes array of len(STAGES) + 1 hipEvent_t handles.

    Returns the bit mask of the stages that ran (their events were recorded)."""
    ran = ctypes.c_uint32(0)
    _check(lib().gdn_fwd_timed(ctypes.byref(args), ctypes.c_void_p(workspace), ctypes.c_size_t(workspace_bytes_),
                               ctypes.c_void_p(stream), ctypes.cast(events, ctypes.c_void_p), ctypes.byref(ran)))
    return ran.value


def fwd(q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None, chunk_size=64,
        output_final_state=True, cp_mode="auto", cp_segment_chunks=0, workspace=None, out_dtype=None,
        qk_l2norm=False, beta_sigmoid=False, A_log=None, dt_bias=None, gate_lower_bound=0.0,
        cp_warmup_tol=0.0, cp_form="auto"):
    """Chunked-prefill forward of the gated delta rule on the GPU.

    q, k: [B, T, H_qk, D_k]; v: [B, T, H_v, D_v]; g: [B, T, H_v] fp32 log-gates (or
    [B, T, H_v, D_k] per-channel); beta: [B, T, H_v]; initial_state: [N, H_v, D_k, D_v] fp32;
    cu_seqlens: [N + 1] int32 token offsets of packed sequences (B == 1).
    out_dtype: dtype of o (default q's dtype; torch.float32 returns the unrounded fp32 result).
    In-kernel prologue (gdn_fwd_args in include/gdn.h): qk_l2norm normalises q and k rows, beta_sigmoid
    takes beta as logits, A_log ([H_v] fp32) with dt_bias ([H_v] or [H_v, D_k] fp32) and
    gate_lower_bound takes g as raw gate inputs.
    cp_mode "warmup" with cp_warmup_tol: the approximate warmup form of context parallelism (gdn.h);
    cp_form "chain" or "xyz" picks the form of the exact pre-process (gdn.h, gdn_cp_form).
    Returns (o [B, T, H_v, D_v], final_state [N, H_v, D_k, D_v] fp32 or None).
    """
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("initial_state", initial_state),
                    ("A_log", A_log), ("dt_bias", dt_bias)):
        _require_gpu(name, t)
    cu_dev = cu_host = None
    if cu_seqlens is not None:
        cu_host = cu_seqlens.detach().to("cpu", torch.int32).contiguous()
        cu_dev = cu_seqlens if cu_seqlens.is_cuda else cu_host.to(q.device)
        cu_dev = cu_dev.to(torch.int32).contiguous()
    N = q.shape[0] if cu_seqlens is None else cu_host.numel() - 1
    o = torch.empty(v.shape, dtype=q.dtype if out_dtype is None else out_dtype, device=q.device)
    fs = (torch.empty((N, v.shape[2], k.shape[3], v.shape[3]), dtype=torch.float32, device=q.device)
          if output_final_state else None)
    a = make_args(q, k, v, g, beta, scale, initial_state, cu_dev, cu_host, chunk_size, o, fs, cp_mode,
                  cp_segment_chunks, qk_l2norm, beta_sigmoid, A_log, dt_bias, gate_lower_bound, cp_warmup_tol,
                  cp_form)
    nbytes = workspace_bytes(a)
    if nbytes == 0 and q.numel() > 0:
        _check(lib().gdn_fwd(ctypes.byref(a), None, 0, None))  # reports the validation error
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    fwd_raw(a, workspace.data_ptr(), workspace.numel(), stream)
    return o, fs


def fwd_recurrent(q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None, output_final_state=True,
                  state_in_place=False, out_dtype=None, qk_l2norm=False, beta_sigmoid=False, A_log=None,
                  dt_bias=None, gate_lower_bound=0.0):
    """Token-by-token (decode) forward on the GPU: gdn_fwd_recurrent, same arguments as ``fwd``.

    state_in_place: write the final state into ``initial_state`` (which must be given) instead of
    a new tensor.  Returns (o, final_state or None)."""
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("initial_state", initial_state),
                    ("A_log", A_log), ("dt_bias", dt_bias)):
        _require_gpu(name, t)
    if state_in_place and initial_state is None:
        raise GdnError(GDN_ERR_INVALID_ARG, "state_in_place needs initial_state")
    cu_dev = cu_host = None
    if cu_seqlens is not None:
        cu_host = cu_seqlens.detach().to("cpu", torch.int32).contiguous()
        cu_dev = cu_seqlens if cu_seqlens.is_cuda else cu_host.to(q.device)
        cu_dev = cu_dev.to(torch.int32).contiguous()
    N = q.shape[0] if cu_seqlens is None else cu_host.numel() - 1
    o = torch.empty(v.shape, dtype=q.dtype if out_dtype is None else out_dtype, device=q.device)
    if state_in_place:
        fs = initial_state
    elif output_final_state:
        fs = torch.empty((N, v.shape[2], k.shape[3], v.shape[3]), dtype=torch.float32, device=q.device)
    else:
        fs = None
    a = make_args(q, k, v, g, beta, scale, initial_state, cu_dev, cu_host, 1, o, fs, "auto", 0,
                  qk_l2norm, beta_sigmoid, A_log, dt_bias, gate_lower_bound)
    fwd_recurrent_raw(a, torch.cuda.current_stream(q.device).cuda_stream)
    return o, fs


def fwd_recurrent_raw(args, stream):
    """Call gdn_fwd_recurrent with a prepared FwdArgs (chunk_size 1) and a stream handle (int)."""
    _check(lib().gdn_fwd_recurrent(ctypes.byref(args), ctypes.c_void_p(stream)))


def make_bwd_args(q, k, v, g, beta, dout, grads, scale=None, initial_state=None, dht=None, cu_seqlens=None,
                  cu_seqlens_cpu=None):
    """Fill a gdn_bwd_args; grads: dict of fp32 output tensors dq, dk, dv, dg, dbeta and optional dh0
    (checked here against the shapes the kernels write: the C ABI cannot see buffer sizes)."""
    N = q.shape[0] if cu_seqlens is None else cu_seqlens.numel() - 1
    want = {"dq": q.shape, "dk": k.shape, "dv": v.shape, "dg": g.shape, "dbeta": beta.shape,
            "dh0": (N, v.shape[2], k.shape[3], v.shape[3])}
    for n, shape in want.items():
        t = grads.get(n)
        if t is None and n == "dh0":
            continue
        if t is None or tuple(t.shape) != tuple(shape) or t.dtype != torch.float32 or not t.is_contiguous():
            raise GdnError(GDN_ERR_INVALID_ARG, f"{n} must be a contiguous fp32 tensor of shape {tuple(shape)}")
    check_inputs(q, k, v, g, beta, initial_state, cu_seqlens, dout=dout, dht=dht)
    f = make_args(q, k, v, g, beta, scale, initial_state, cu_seqlens, cu_seqlens_cpu)
    a = BwdArgs()
    for n in ("B", "T", "H_qk", "H_v", "D_k", "D_v", "chunk_size", "dtype", "gate_kind", "scale", "q", "k", "v", "g",
              "beta", "h0", "cu_seqlens_dev", "cu_seqlens_host", "N"):
        setattr(a, n, getattr(f, n))
    a.dout, a.dht = _ptr(dout), _ptr(dht)
    for n in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        setattr(a, n, _ptr(grads.get(n)))
    return a


def bwd(q, k, v, g, beta, dout, scale=None, initial_state=None, dht=None, cu_seqlens=None, want_dh0=True):
    """Backward of ``fwd`` (both gate kinds): gdn_bwd.  Returns a dict of fp32 gradients dq, dk, dv, dg,
    dbeta and dh0 (None unless want_dh0), shaped like the inputs."""
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("dout", dout),
                    ("initial_state", initial_state), ("dht", dht)):
        _require_gpu(name, t)
    cu_dev = cu_host = None
    if cu_seqlens is not None:
        cu_host = cu_seqlens.detach().to("cpu", torch.int32).contiguous()
        cu_dev = cu_seqlens if cu_seqlens.is_cuda else cu_host.to(q.device)
        cu_dev = cu_dev.to(torch.int32).contiguous()
    N = q.shape[0] if cu_seqlens is None else cu_host.numel() - 1
    f32 = dict(dtype=torch.float32, device=q.device)
    grads = {"dq": torch.empty(q.shape, **f32), "dk": torch.empty(k.shape, **f32), "dv": torch.empty(v.shape, **f32),
             "dg": torch.empty(g.shape, **f32), "dbeta": torch.empty(beta.shape, **f32),
             "dh0": torch.empty((N, v.shape[2], k.shape[3], v.shape[3]), **f32) if want_dh0 else None}
    a = make_bwd_args(q, k, v, g, beta, dout, grads, scale, initial_state, dht, cu_dev, cu_host)
    nbytes = int(lib().gdn_bwd_workspace_bytes(ctypes.byref(a)))
    if nbytes == 0 and q.numel() > 0:
        _check(lib().gdn_bwd(ctypes.byref(a), None, 0, None))  # reports the validation error
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(lib().gdn_bwd(ctypes.byref(a), ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel()),
                         ctypes.c_void_p(stream)))
    return grads
