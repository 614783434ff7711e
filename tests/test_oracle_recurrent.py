"""Pins of the fp64 token-recurrence oracle to closed forms and hand-derived values.

Each case is chosen so that a plausible slip in the oracle (erase sign, beta on
the wrong factor, decay after the read, output before the update, a transposed
state, the wrong qk head for a value head, a per-channel decay applied after the
erase) changes the result.
"""
import json
import os

import numpy as np
import pytest

from oracle.recurrent import gdn_recurrent

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng0 = np.random.default_rng


def _rand_inputs(rng, T, H, Dk, Dv, gate="scalar", mu=-2.0, batch=1):
    q = rng.standard_normal((batch, T, H, Dk))
    k = rng.standard_normal((batch, T, H, Dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((batch, T, H, Dv))
    gs = (batch, T, H) if gate == "scalar" else (batch, T, H, Dk)
    g = -np.logaddexp(0, rng.standard_normal(gs) + mu)
    beta = 1 / (1 + np.exp(-rng.standard_normal((batch, T, H))))
    return q, k, v, g, beta


def test_scalar_fixed_point_closed_form():
    # D_k = D_v = 1, k = q = 1, constant alpha, beta, v:  s_t = alpha (1 - beta) s_{t-1} + beta v,
    # so s_t = s* + (s0 - s*) rho^t with rho = alpha (1 - beta), s* = beta v / (1 - rho).
    T, alpha, beta, v0, s0, scale = 37, 0.9, 0.3, 1.7, -0.4, 0.5
    ones = np.ones((1, T, 1, 1))
    o, fin = gdn_recurrent(ones, ones, np.full((1, T, 1, 1), v0), np.full((1, T, 1), np.log(alpha)),
                           np.full((1, T, 1), beta), scale, h0=np.full((1, 1, 1, 1), s0))
    rho = alpha * (1 - beta)
    star = beta * v0 / (1 - rho)
    t = np.arange(1, T + 1)
    expect = star + (s0 - star) * rho ** t
    np.testing.assert_allclose(o[0, :, 0, 0], scale * expect, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(fin[0, 0, 0, 0], expect[-1], rtol=1e-13)


def test_beta_zero_is_decayed_initial_state_readout():
    # beta = 0: nothing is written; S_t = exp(sum_{s<=t} g_s) h0 and o_t = scale * S_t^T q_t.
    rng = rng0(1)
    q, k, v, g, beta = _rand_inputs(rng, 50, 2, 8, 5)
    h0 = rng.standard_normal((1, 2, 8, 5))
    o, fin = gdn_recurrent(q, k, v, g, np.zeros_like(beta), 0.3, h0=h0)
    cum = np.exp(np.cumsum(g[0], axis=0))  # [T, H]
    expect = 0.3 * cum[:, :, None] * np.einsum("thk,hkv->thv", q[0], h0[0])
    np.testing.assert_allclose(o[0], expect, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(fin[0], cum[-1][:, None, None] * h0[0], rtol=1e-12)


def test_alpha_one_beta_zero():
    rng = rng0(2)
    q, k, v, g, beta = _rand_inputs(rng, 20, 3, 6, 7)
    h0 = rng.standard_normal((1, 3, 6, 7))
    o, fin = gdn_recurrent(q, k, v, np.zeros_like(g), np.zeros_like(beta), 1.25, h0=h0)
    np.testing.assert_allclose(o[0], 1.25 * np.einsum("thk,hkv->thv", q[0], h0[0]), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(fin[0], h0[0], rtol=0, atol=0)


def test_same_key_overwrite():
    # beta = 1 and k_t = e_j for all t: the row of S along e_j is replaced by v_t at every step,
    # the other rows only decay:  S_t = (prod_{s<=t} alpha_s)(I - e e^T) h0 + e v_t^T.
    rng = rng0(3)
    T, Dk, Dv, j = 30, 6, 4, 2
    q, _, v, g, _ = _rand_inputs(rng, T, 1, Dk, Dv)
    k = np.zeros((1, T, 1, Dk)); k[..., j] = 1.0
    h0 = rng.standard_normal((1, 1, Dk, Dv))
    o, fin = gdn_recurrent(q, k, v, g, np.ones((1, T, 1)), 1.0, h0=h0)
    P = np.eye(Dk); P[j, j] = 0.0
    cum = np.exp(np.cumsum(g[0, :, 0]))
    for t in [0, 1, 17, T - 1]:
        S_t = cum[t] * (P @ h0[0, 0]) + np.outer(np.eye(Dk)[j], v[0, t, 0])
        np.testing.assert_allclose(o[0, t, 0], S_t.T @ q[0, t, 0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(fin[0, 0], cum[-1] * (P @ h0[0, 0]) + np.outer(np.eye(Dk)[j], v[0, -1, 0]),
                               rtol=1e-12, atol=1e-14)


def test_unit_key_reads_back_its_value():
    # alpha = 1, beta = 1, unit-norm k_t: after the update S_t^T k_t = v_t exactly (delta rule).
    rng = rng0(4)
    q, k, v, g, _ = _rand_inputs(rng, 12, 1, 9, 3)
    h0 = rng.standard_normal((1, 1, 9, 3))
    for t in range(1, 13):
        _, fin = gdn_recurrent(q[:, :t], k[:, :t], v[:, :t], np.zeros_like(g[:, :t]), np.ones((1, t, 1)),
                               1.0, h0=h0)
        np.testing.assert_allclose(fin[0, 0].T @ k[0, t - 1, 0], v[0, t - 1, 0], rtol=1e-12, atol=1e-12)


def test_kda_decay_order_golden():
    d = json.load(open(os.path.join(GOLDEN, "kda_decay_order.json")))
    x = d["inputs"]
    q = np.array(x["q"]).reshape(1, 1, 1, 2)
    k = np.array(x["k"]).reshape(1, 1, 1, 2)
    v = np.array(x["v"]).reshape(1, 1, 1, 1)
    gk = np.array(x["gk"]).reshape(1, 1, 1, 2)
    h0 = np.array(x["h0"]).reshape(1, 1, 2, 1)
    o, fin = gdn_recurrent(q, k, v, gk, np.full((1, 1, 1), x["beta"]), x["scale"], h0=h0, gate="channel")
    np.testing.assert_allclose(fin[0, 0], np.array(d["expected"]["final"]), rtol=1e-14)
    np.testing.assert_allclose(o[0, 0, 0], np.array(d["expected"]["o"]), rtol=1e-14)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_matrix_form_on_tiny_inputs(gate):
    # S_t = (I - beta k k^T) A_t S_{t-1} + beta k v^T with A_t = alpha_t I or Diag(alpha_t), as dense
    # matrix products -- a different writing of the definition than the C loop.
    rng = rng0(5)
    T, Dk, Dv = 9, 4, 3
    q, k, v, g, beta = _rand_inputs(rng, T, 1, Dk, Dv, gate=gate)
    h0 = rng.standard_normal((1, 1, Dk, Dv))
    o, fin = gdn_recurrent(q, k, v, g, beta, 0.7, h0=h0, gate=gate)
    S = h0[0, 0].copy()
    for t in range(T):
        kt, b = k[0, t, 0], beta[0, t, 0]
        At = np.exp(g[0, t, 0]) * np.eye(Dk) if gate == "scalar" else np.diag(np.exp(g[0, t, 0]))
        S = (np.eye(Dk) - b * np.outer(kt, kt)) @ At @ S + b * np.outer(kt, v[0, t, 0])
        np.testing.assert_allclose(o[0, t, 0], 0.7 * S.T @ q[0, t, 0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(fin[0, 0], S, rtol=1e-12, atol=1e-14)


def test_packed_equals_separate_and_continuation():
    rng = rng0(6)
    lens = [5, 64, 1, 130, 77]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, beta = _rand_inputs(rng, cu[-1], 2, 8, 8)
    h0 = rng.standard_normal((len(lens), 2, 8, 8))
    o, fin = gdn_recurrent(q, k, v, g, beta, 0.4, h0=h0, cu_seqlens=cu)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        on, fn = gdn_recurrent(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b], 0.4, h0=h0[n:n + 1])
        np.testing.assert_array_equal(o[0, a:b], on[0])
        np.testing.assert_array_equal(fin[n], fn[0])
    # continuation: the final state of a prefix is the initial state of the rest
    a, m, b = cu[3], cu[3] + 50, cu[4]
    _, f1 = gdn_recurrent(q[:, a:m], k[:, a:m], v[:, a:m], g[:, a:m], beta[:, a:m], 0.4, h0=h0[3:4])
    o2, f2 = gdn_recurrent(q[:, m:b], k[:, m:b], v[:, m:b], g[:, m:b], beta[:, m:b], 0.4, h0=f1)
    np.testing.assert_allclose(o2[0], o[0, m:b], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(f2[0], fin[3], rtol=1e-12, atol=1e-14)


def test_grouped_value_heads_use_their_qk_head():
    # H_v = 2 H_qk: value head h reads query/key head h // 2; same as repeating q, k per value head.
    rng = rng0(7)
    q, k, v, g, beta = _rand_inputs(rng, 40, 4, 8, 8)
    q2, k2 = q[:, :, :2], k[:, :, :2]
    o, fin = gdn_recurrent(q2, k2, v, g, beta, 0.5)
    rep = lambda x: np.repeat(x, 2, axis=2)
    o_r, fin_r = gdn_recurrent(rep(q2), rep(k2), v, g, beta, 0.5)
    np.testing.assert_array_equal(o, o_r)
    np.testing.assert_array_equal(fin, fin_r)
