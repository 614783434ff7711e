"""Pins of the backward oracle (oracle/backward.py): its forward against the C token oracle, its
gradients against central finite differences and against closed forms at beta = 0."""
import numpy as np
import pytest

from oracle.backward import gdn_backward
from oracle.recurrent import gdn_recurrent


def _inputs(B=1, T=7, H=2, Hq=None, D=3, seed=0):
    rng = np.random.default_rng(seed)
    Hq = Hq or H
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    q, k = unit(rng.standard_normal((B, T, Hq, D))), unit(rng.standard_normal((B, T, Hq, D)))
    v = rng.standard_normal((B, T, H, D))
    g = -np.logaddexp(0.0, rng.standard_normal((B, T, H)) - 1.0)
    b = rng.uniform(0.1, 0.9, (B, T, H))
    h0 = 0.3 * rng.standard_normal((B, H, D, D))
    do = rng.standard_normal((B, T, H, D))
    dht = rng.standard_normal((B, H, D, D))
    return q, k, v, g, b, h0, do, dht


def test_forward_matches_c_oracle():
    q, k, v, g, b, h0, do, dht = _inputs(B=2, T=9, H=4, Hq=2, D=5, seed=1)
    r = gdn_backward(q, k, v, g, b, 0.4, do, h0, dht)
    o, f = gdn_recurrent(q, k, v, g, b, 0.4, h0=h0)
    np.testing.assert_allclose(r["o"], o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r["final"], f, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "h0"])
def test_gradients_match_finite_differences(name):
    q, k, v, g, b, h0, do, dht = _inputs(B=1, T=6, H=2, Hq=1, D=3, seed=2)
    args = dict(q=q, k=k, v=v, g=g, beta=b, h0=h0)
    r = gdn_backward(q, k, v, g, b, 0.7, do, h0, dht)

    def loss(a):
        o, f = gdn_recurrent(a["q"], a["k"], a["v"], a["g"], a["beta"], 0.7, h0=a["h0"])
        return float((o * do).sum() + (f * dht).sum())
    x = args[name]
    fd = np.zeros_like(x)
    eps = 1e-6
    for idx in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += eps
        xm[idx] -= eps
        fd[idx] = (loss({**args, name: xp}) - loss({**args, name: xm})) / (2 * eps)
    key = {"beta": "dbeta", "h0": "dh0"}.get(name, "d" + name)
    np.testing.assert_allclose(r[key], fd, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("name", ["k", "g", "beta", "h0"])
def test_per_channel_gradients_match_finite_differences(name):
    q, k, v, g, b, h0, do, dht = _inputs(B=1, T=6, H=2, Hq=1, D=3, seed=7)
    gk = -np.logaddexp(0.0, np.random.default_rng(8).standard_normal((1, 6, 2, 3)) - 1.0)
    args = dict(q=q, k=k, v=v, g=gk, beta=b, h0=h0)
    r = gdn_backward(q, k, v, gk, b, 0.7, do, h0, dht)
    assert r["dg"].shape == gk.shape

    def loss(a):
        o, f = gdn_recurrent(a["q"], a["k"], a["v"], a["g"], a["beta"], 0.7, h0=a["h0"], gate="channel")
        return float((o * do).sum() + (f * dht).sum())
    x = args[name]
    fd = np.zeros_like(x)
    eps = 1e-6
    for idx in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += eps
        xm[idx] -= eps
        fd[idx] = (loss({**args, name: xp}) - loss({**args, name: xm})) / (2 * eps)
    key = {"beta": "dbeta", "h0": "dh0"}.get(name, "d" + name)
    np.testing.assert_allclose(r[key], fd, rtol=1e-6, atol=1e-8)


def test_per_channel_gate_with_equal_channels_is_the_scalar_gate():
    q, k, v, g, b, h0, do, dht = _inputs(B=1, T=9, H=2, D=4, seed=9)
    gk = np.repeat(g[..., None], 4, axis=-1)
    r1 = gdn_backward(q, k, v, g, b, 0.5, do, h0, dht)
    r2 = gdn_backward(q, k, v, gk, b, 0.5, do, h0, dht)
    for n in ("dq", "dk", "dv", "dbeta", "dh0"):
        np.testing.assert_allclose(r2[n], r1[n], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r2["dg"].sum(-1), r1["dg"], rtol=1e-10, atol=1e-12)   # chain rule over copies


def test_closed_forms_at_beta_zero():
    # beta = 0: S_t = (prod alpha) h0, o_t = scale S_t^T q_t, so dv = 0, dq_t = scale S_t do_t and
    # dh0 = sum_t scale A_t q_t do_t^T + A_T dht with A_t the decay product through t
    q, k, v, g, b, h0, do, dht = _inputs(B=1, T=5, H=1, D=4, seed=3)
    b = np.zeros_like(b)
    r = gdn_backward(q, k, v, g, b, 0.5, do, h0, dht)
    a = np.exp(np.cumsum(g[0, :, 0]))
    np.testing.assert_array_equal(r["dv"], 0.0)
    for t in range(5):
        np.testing.assert_allclose(r["dq"][0, t, 0], 0.5 * a[t] * h0[0, 0] @ do[0, t, 0], rtol=1e-12)
    want = sum(0.5 * a[t] * np.outer(q[0, t, 0], do[0, t, 0]) for t in range(5)) + a[-1] * dht[0, 0]
    np.testing.assert_allclose(r["dh0"][0, 0], want, rtol=1e-12)


def test_packed_sequences_are_independent():
    q, k, v, g, b, h0, do, dht = _inputs(B=1, T=10, H=2, D=3, seed=4)
    h0 = np.concatenate([h0, 0.5 * h0])
    dht = np.concatenate([dht, -dht])
    cu = [0, 4, 10]
    r = gdn_backward(q, k, v, g, b, 0.3, do, h0, dht, cu_seqlens=cu)
    s = gdn_backward(q[:, 4:], k[:, 4:], v[:, 4:], g[:, 4:], b[:, 4:], 0.3, do[:, 4:], h0[1:], dht[1:])
    np.testing.assert_allclose(r["dk"][:, 4:], s["dk"], rtol=1e-12)
    np.testing.assert_allclose(r["dh0"][1], s["dh0"][0], rtol=1e-12)
