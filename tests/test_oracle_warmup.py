"""Pins of the warmup-CP oracle (oracle/warmup.py) to the exact recurrence and to the error bound
that justifies it (FlashQLA announcement, section "further optimisation through gate decay")."""
import numpy as np
import pytest

from oracle.recurrent import gdn_recurrent
from oracle.warmup import chunk_log_decay_bounds, warmup_cp, warmup_length

C = 64


def _inputs(T, H=2, D=16, gate="scalar", g_fn=None, seed=0, n_seqs=None):
    rng = np.random.default_rng(seed)
    shape = (1, T, H, D)
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    q, k = unit(rng.standard_normal(shape)), unit(rng.standard_normal(shape))
    v = rng.standard_normal(shape)
    b = rng.uniform(0.05, 0.95, (1, T, H))
    gshape = (1, T, H) if gate == "scalar" else (1, T, H, D)
    g = g_fn(rng, gshape) if g_fn else -np.logaddexp(0.0, rng.standard_normal(gshape) - 2.0)
    h0 = 0.1 * rng.standard_normal((1 if n_seqs is None else n_seqs, H, D, D))
    return q, k, v, g, b, h0


def test_warmup_length_closed_forms():
    lb = np.full(10, -3.2)                      # every chunk decays by e^-3.2
    assert warmup_length(lb, 8, np.exp(-8.0)) == 3      # e^-6.4 > e^-8 >= e^-9.6
    assert warmup_length(lb, 2, np.exp(-8.0)) == 2      # not enough chunks before: the whole prefix
    assert warmup_length(lb, 5, np.exp(-3.2)) == 1      # <= tol reached on equality
    assert warmup_length(np.zeros(10), 7, 1e-6) == 7    # no decay: the whole prefix
    assert warmup_length(lb, 6, 0.0) == 6               # tol 0: never, the whole prefix


def test_chunk_decay_bounds():
    g = -np.arange(130, dtype=np.float64) / 100.0
    np.testing.assert_allclose(chunk_log_decay_bounds(g, C, "scalar"),
                               [g[:64].sum(), g[64:128].sum(), g[128:].sum()], rtol=1e-14)
    gk = np.stack([g, 2 * g, g / 2], axis=-1)          # channel 2 decays slowest on every token
    np.testing.assert_allclose(chunk_log_decay_bounds(gk, C, "channel"),
                               [(g / 2)[:64].sum(), (g / 2)[64:128].sum(), (g / 2)[128:].sum()], rtol=1e-14)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_whole_prefix_warmup_is_the_exact_recurrence(gate):
    # tol 0 (and g == 0) leave no shorter warmup: every segment restarts at its sequence start
    # from h0 and must reproduce the serial recurrence
    q, k, v, g, b, h0 = _inputs(7 * C + 11, gate=gate, seed=1)
    o_r, f_r = gdn_recurrent(q, k, v, g, b, 0.25, h0=h0, gate=gate)
    o_w, f_w, W, _ = warmup_cp(q, k, v, g, b, 0.25, h0=h0, gate=gate, seg_chunks=3, tol=0.0)
    assert W[(0, 2, 1)] == 6
    np.testing.assert_allclose(o_w, o_r, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(f_w, f_r, rtol=1e-12, atol=1e-14)
    z = np.zeros_like(g)
    o_z, f_z, W, _ = warmup_cp(q, k, v, z, b, 0.25, h0=h0, gate=gate, seg_chunks=2, tol=1e-3)
    o_r, f_r = gdn_recurrent(q, k, v, z, b, 0.25, h0=h0, gate=gate)
    assert all(W[(0, j, h)] == 2 * j for j in range(4) for h in range(2))
    np.testing.assert_allclose(o_z, o_r, rtol=1e-12, atol=1e-14)


def test_constant_gate_warmup_lengths():
    q, k, v, g, b, h0 = _inputs(9 * C, g_fn=lambda rng, s: np.full(s, -0.05), seed=2)
    _, _, W, _ = warmup_cp(q, k, v, g, b, 0.25, h0=h0, seg_chunks=2, tol=np.exp(-8.0))
    # chunk decay e^-3.2: three chunks reach e^-8, fewer chunks exist only before segment 1
    assert {W[(0, j, 0)] for j in range(1, 5)} == {2, 3} and W[(0, 1, 0)] == 2 and W[(0, 4, 1)] == 3


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_state_error_within_the_decay_bound(gate):
    # warmup starts from 0 instead of the exact state S_w: every later state is off by at most
    # prod(chunk decay bounds over the warmup) * ||S_w||_2 (spectral norms)
    T, L, tol = 24 * C, 8, 1e-3

    def gates(rng, s):
        g = -np.logaddexp(0.0, rng.standard_normal(s) - 3.0)
        if gate == "channel":
            g[..., 0] = -0.012      # one slow channel: the bound (slowest channel per token) is tight
        return g
    q, k, v, g, b, h0 = _inputs(T, gate=gate, seed=3, g_fn=gates)
    b = 0.05 * b                    # weak erases: the decay, not the erase, forgets the state
    o_w, f_w, W, ends = warmup_cp(q, k, v, g, b, 0.25, h0=h0, gate=gate, seg_chunks=L, tol=tol)
    worst = 0.0   # largest err / bound seen
    for (n, j, h), Wj in W.items():
        if j == 0:
            continue
        c0 = j * L
        if Wj == c0:
            continue                             # whole prefix: exact, checked elsewhere
        lb = chunk_log_decay_bounds(g[0, :, h], C, gate)
        bound = np.exp(lb[c0 - Wj:c0].sum())
        assert bound <= tol and (Wj == 1 or np.exp(lb[c0 - Wj + 1:c0].sum()) > tol)
        _, s_w = gdn_recurrent(q[:, :(c0 - Wj) * C], k[:, :(c0 - Wj) * C], v[:, :(c0 - Wj) * C],
                               g[:, :(c0 - Wj) * C], b[:, :(c0 - Wj) * C], 0.25, h0=h0, gate=gate)
        e = min((c0 + L) * C, T)
        _, s_e = gdn_recurrent(q[:, :e], k[:, :e], v[:, :e], g[:, :e], b[:, :e], 0.25, h0=h0, gate=gate)
        err = np.linalg.norm(ends[(n, j, h)] - s_e[0, h], 2)
        lim = bound * np.linalg.norm(s_w[0, h], 2)
        assert err <= lim * (1 + 1e-9) + 1e-13, (j, h, err, lim)
        worst = max(worst, err / lim)
    assert sum(1 for (n, j, h), Wj in W.items() if 0 < Wj < j * L) >= 2
    o_r, f_r = gdn_recurrent(q, k, v, g, b, 0.25, h0=h0, gate=gate)
    assert np.abs(o_w - o_r).max() > 1e-9, "the warmup must actually approximate in this test"
    # the first segment runs exactly, and no warmup token overwrites an earlier segment's output
    np.testing.assert_allclose(o_w[:, :L * C], o_r[:, :L * C], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(f_w, f_r, atol=tol * np.abs(f_r).max())


def test_packed_sequences_and_grouped_heads():
    rng = np.random.default_rng(4)
    lens = [0, 1, 3 * C + 5, 5 * C]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H, Hq, D = int(cu[-1]), 4, 2, 16
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    q, k = unit(rng.standard_normal((1, T, Hq, D))), unit(rng.standard_normal((1, T, Hq, D)))
    v, b = rng.standard_normal((1, T, H, D)), rng.uniform(0.1, 0.9, (1, T, H))
    g = -np.logaddexp(0.0, rng.standard_normal((1, T, H)) - 1.0)
    h0 = 0.1 * rng.standard_normal((4, H, D, D))
    o_w, f_w, W, _ = warmup_cp(q, k, v, g, b, 0.3, h0=h0, cu_seqlens=cu, seg_chunks=2, tol=2.0 ** -40)
    o_r, f_r = gdn_recurrent(q, k, v, g, b, 0.3, h0=h0, cu_seqlens=cu)
    np.testing.assert_allclose(o_w, o_r, atol=1e-9)
    np.testing.assert_allclose(f_w, f_r, atol=1e-9)
    np.testing.assert_array_equal(f_w[0], h0[0])                      # empty sequence keeps h0
