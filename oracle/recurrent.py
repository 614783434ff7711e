"""Token-by-token fp64 recurrence (TEST INFRASTRUCTURE ONLY): ctypes wrapper of gdn_recurrent.c.

Definition followed (see the header of gdn_recurrent.c for the sources):
    S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,   o_t = scale * S_t^T q_t
with a scalar alpha_t = exp(g_t) (Gated DeltaNet) or a per-key-channel
alpha_t = Diag(exp(gk_t)) applied before the read and the erase (KDA).

Pinned by tests/test_oracle_recurrent.py (closed forms, hand-derived values)
and tests/test_oracle_chunkwise.py (agreement with the independent chunkwise
evaluation of the pages' formulas).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle_gdn.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        lib.oracle_gdn_recurrent.argtypes = [
            ctypes.c_int, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            P, P, P, P, P, ctypes.c_double, P, P, P, ctypes.c_int]
        lib.oracle_gdn_recurrent.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def flatten_batch(q, k, v, g, beta, cu_seqlens):
    """[B,T,H,D] inputs -> token-major [B*T,H,D] plus sequence offsets [N+1]."""
    q = np.asarray(q)
    if q.ndim == 4:
        B, T = q.shape[:2]
        if cu_seqlens is not None:
            assert B == 1, "packed sequences need B == 1"
            cu = np.asarray(cu_seqlens, dtype=np.int64)
        else:
            cu = np.arange(B + 1, dtype=np.int64) * T
        fl = lambda a: None if a is None else np.asarray(a).reshape((B * T,) + np.asarray(a).shape[2:])
        return fl(q), fl(k), fl(v), fl(g), fl(beta), cu, (B, T)
    cu = np.asarray(cu_seqlens if cu_seqlens is not None else [0, q.shape[0]], dtype=np.int64)
    return q, k, v, g, beta, cu, None


def gdn_recurrent(q, k, v, g, beta, scale, h0=None, cu_seqlens=None, gate="scalar", n_threads=None):
    """Run the fp64 token recurrence.

    q, k: [B,T,H_qk,D_k] (or token-major [T,H_qk,D_k]); v: [...,H_v,D_v];
    g: [...,H_v] (gate="scalar") or [...,H_v,D_k] (gate="channel"); beta: [...,H_v];
    h0: [N,H_v,D_k,D_v] or None.  Returns (o shaped like v, final [N,H_v,D_k,D_v]).
    """
    qf, kf, vf, gf, bf, cu, bt = flatten_batch(q, k, v, g, beta, cu_seqlens)
    qf, kf, vf, gf, bf = map(_f64, (qf, kf, vf, gf, bf))
    Ttot, H_qk, Dk = qf.shape
    H_v, Dv = vf.shape[1], vf.shape[2]
    N = len(cu) - 1
    gate_kind = {"scalar": 0, "channel": 1}[gate]
    if gate_kind == 0:
        assert gf.shape == (Ttot, H_v)
    else:
        assert gf.shape == (Ttot, H_v, Dk)
    assert bf.shape == (Ttot, H_v) and cu[-1] == Ttot
    h0f = None if h0 is None else _f64(h0)
    if h0f is not None:
        assert h0f.shape == (N, H_v, Dk, Dv)
    o = np.zeros((Ttot, H_v, Dv))
    fin = np.zeros((N, H_v, Dk, Dv))
    cu64 = np.ascontiguousarray(cu, dtype=np.int64)
    nt = n_threads or os.cpu_count() or 1
    rc = _load().oracle_gdn_recurrent(N, _ptr(cu64), H_qk, H_v, Dk, Dv, gate_kind, _ptr(qf), _ptr(kf),
                                      _ptr(vf), _ptr(gf), _ptr(bf), float(scale), _ptr(h0f), _ptr(o),
                                      _ptr(fin), int(nt))
    if rc != 0:
        raise RuntimeError(f"oracle_gdn_recurrent failed with code {rc}")
    if bt is not None:
        o = o.reshape(bt + (H_v, Dv))
    return o, fin
