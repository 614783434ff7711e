"""fp64 gradients of the gated delta rule (TEST INFRASTRUCTURE ONLY).

The forward is the token recurrence written in plain PyTorch fp64 CPU ops,
    S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,   o_t = scale S_t^T q_t,
alpha_t = exp(g_t) (scalar gate; per-channel gate: Diag(exp(gk_t)) on the rows of S, applied
before the read and the erase as on the KDA walk-through page, section 3), S_0 = h0 (FlashQLA
announcement, gate-decay section; Flash Linear Attention page, section 8), and the gradients of
the loss <o, do> + <S_T, dS_T> with respect to q, k, v, g, beta and h0 come from torch.autograd (a
library primitive standing in for the backward's algebra; the GDN-in-FLA notes, backward Steps
1-7, derive the same gradients in chunked form).  Pinned by tests/test_oracle_backward.py: the
forward equals the C oracle, the gradients match central finite differences of the C oracle on
tiny inputs (both gate kinds), closed forms at beta = 0, and equal channel gates reduce to the
scalar gate.
"""
import numpy as np
import torch


def _recurrence(q, k, v, g, beta, scale, h0, cu):
    """Token-major fp64 tensors q, k [T, H_qk, D_k], v [T, H_v, D_v], g [T, H_v] or [T, H_v, D_k],
    beta [T, H_v]; h0 [N, H_v, D_k, D_v] or None.  Returns (o [T, H_v, D_v], final [N, H_v, D_k, D_v])."""
    T, H_qk, D_k = q.shape
    H_v, D_v = v.shape[1], v.shape[2]
    G = H_v // H_qk
    N = len(cu) - 1
    hq = torch.arange(H_v) // G
    outs, fins = [], []
    for n in range(N):
        S = h0[n] if h0 is not None else torch.zeros(H_v, D_k, D_v, dtype=torch.float64)
        for t in range(int(cu[n]), int(cu[n + 1])):
            kt, qt, vt = k[t, hq], q[t, hq], v[t]                      # [H_v, D_k], [H_v, D_k], [H_v, D_v]
            a = torch.exp(g[t])
            S = (a[:, None, None] if a.dim() == 1 else a[:, :, None]) * S   # decay (rows per channel)
            u = torch.einsum("hk,hkv->hv", kt, S)                      # S^T k
            w = beta[t][:, None] * (vt - u)
            S = S + kt[:, :, None] * w[:, None, :]                     # erase and write
            outs.append(scale * torch.einsum("hk,hkv->hv", qt, S))
        fins.append(S)
    o = torch.stack(outs) if outs else torch.zeros(0, H_v, D_v, dtype=torch.float64)
    return o, torch.stack(fins)


def gdn_backward(q, k, v, g, beta, scale, do, h0=None, dht=None, cu_seqlens=None):
    """Gradients of <o, do> + <final, dht> (dht None: 0).  Inputs as numpy arrays shaped like the
    library's ([B, T, H, D] or packed with B = 1 and cu_seqlens; g [B, T, H_v] for the scalar gate or
    [B, T, H_v, D_k] per channel).  Returns a dict of numpy fp64 arrays dq, dk, dv, dg, dbeta shaped
    like the inputs, dh0 [N, H_v, D_k, D_v], plus o and final."""
    q = np.asarray(q, dtype=np.float64)
    B, T = q.shape[:2]
    cu = (np.arange(B + 1) * T) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    flat = lambda a: torch.tensor(np.asarray(a, dtype=np.float64).reshape((B * T,) + np.asarray(a).shape[2:]),
                                  requires_grad=True)
    tq, tk, tv, tg, tb = (flat(a) for a in (q, k, v, g, beta))
    N = len(cu) - 1
    H_v, D_k, D_v = tv.shape[1], tq.shape[2], tv.shape[2]
    th0 = torch.tensor(np.asarray(h0, dtype=np.float64) if h0 is not None else np.zeros((N, H_v, D_k, D_v)),
                       requires_grad=True)
    o, fin = _recurrence(tq, tk, tv, tg, tb, scale, th0, cu)
    loss = (o * torch.tensor(np.asarray(do, dtype=np.float64).reshape(o.shape))).sum()
    if dht is not None:
        loss = loss + (fin * torch.tensor(np.asarray(dht, dtype=np.float64))).sum()
    grads = torch.autograd.grad(loss, [tq, tk, tv, tg, tb, th0], allow_unused=True)
    shape = lambda gr, like: (torch.zeros_like(like) if gr is None else gr).detach().numpy().reshape(
        (B, T) + tuple(like.shape[1:]))
    out = {n: shape(gr, t) for n, gr, t in zip(("dq", "dk", "dv", "dg", "dbeta"), grads[:5], (tq, tk, tv, tg, tb))}
    out["dh0"] = grads[5].detach().numpy()
    out["o"] = o.detach().numpy().reshape((B, T, H_v, D_v))
    out["final"] = fin.detach().numpy()
    return out
