"""fp64 in-kernel prologue of the forward (TEST INFRASTRUCTURE ONLY): what the library applies to
raw inputs when gdn_fwd_args asks for it, written out as plain definitions.

Sources: KDA source walk-through (FLA), section 2, the chunked gate cumsum kernel: with A_log
and an optional dt_bias the log-gate of a raw input x is
    -exp(A_log[h]) * softplus(x + dt_bias)                     (no lower bound)
    lower_bound * sigmoid(exp(A_log[h]) * (x + dt_bias))       (with a lower bound)
(dt_bias per head for a scalar gate, per head and key channel for a per-channel gate); and the
same page's section on the FlashKDA backend: the L2 norm of q and k and sigma(beta) taken inside
the kernel.  The pages do not state the L2 norm's epsilon; the reading here is
x / sqrt(sum x^2 + 1e-6) over the D_k values of one token and head.

Pinned by tests/test_oracle_prologue.py (closed forms of each piece, invariance of the
normalised forward under row scaling of q and k).
"""
import numpy as np

L2_EPS = 1e-6


def softplus(x):
    return np.logaddexp(0.0, x)


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def l2norm_rows(x):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + L2_EPS)


def gate_activation(x, A_log, dt_bias=None, lower_bound=0.0, gate="scalar"):
    """Log-gates from raw inputs x ([..., H] scalar gate, [..., H, D] per-channel gate)."""
    x = np.asarray(x, dtype=np.float64)
    A_log = np.asarray(A_log, dtype=np.float64)
    a = np.exp(A_log) if gate == "scalar" else np.exp(A_log)[:, None]
    y = x if dt_bias is None else x + np.asarray(dt_bias, dtype=np.float64)
    if lower_bound < 0.0:
        return lower_bound * sigmoid(a * y)
    return -a * softplus(y)


def apply_prologue(q, k, g, beta, gate="scalar", qk_l2norm=False, beta_sigmoid=False, A_log=None,
                   dt_bias=None, gate_lower_bound=0.0):
    """(q, k, g, beta) as the recurrence consumes them, from raw inputs (fp64 arrays)."""
    if qk_l2norm:
        q, k = l2norm_rows(q), l2norm_rows(k)
    if beta_sigmoid:
        beta = sigmoid(beta)
    if A_log is not None:
        g = gate_activation(g, A_log, dt_bias, gate_lower_bound, gate)
    return q, k, g, beta
