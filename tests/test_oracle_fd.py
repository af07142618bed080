"""Pins the oracle's hand-derived adjoints to brute force: central finite
differences of L = sum <dO, o> + <dS_out, S_out> in fp64, on tiny inputs.

Every input (q, k, v, g, beta, S_in) is perturbed element by element, so a
dropped term, wrong sign, wrong index or transposed operand in any adjoint
fails here.  T = 70 crosses the oracle's 64-token checkpoint boundary."""
import numpy as np
import pytest

from oracle import oracle


def _loss_gdn(x, dO, dS_out):
    o, S = oracle.gdn_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"])
    return float(np.sum(o * dO) + np.sum(S * dS_out))


def _loss_gla(x, dO, dS_out):
    o, S = oracle.gla_fwd(x["q"], x["k"], x["v"], x["g"], x["S_in"])
    return float(np.sum(o * dO) + np.sum(S * dS_out))


def _fd(loss, x, key, dO, dS_out, h=1e-6):
    out = np.zeros_like(x[key])
    flat = x[key].reshape(-1)
    for i in range(flat.size):
        old = flat[i]
        flat[i] = old + h
        lp = loss(x, dO, dS_out)
        flat[i] = old - h
        lm = loss(x, dO, dS_out)
        flat[i] = old
        out.reshape(-1)[i] = (lp - lm) / (2 * h)
    return out


def _rand_gdn(rng, B, T, H, dk, dv):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    return dict(q=q, k=k, v=rng.standard_normal((B, T, H, dv)),
                g=-np.log1p(np.exp(rng.standard_normal((B, T, H)))) * 0.3,
                beta=1 / (1 + np.exp(-rng.standard_normal((B, T, H)))),
                S_in=0.5 * rng.standard_normal((B, H, dk, dv)))


def _rand_gla(rng, B, T, H, dk, dv):
    return dict(q=rng.standard_normal((B, T, H, dk)), k=rng.standard_normal((B, T, H, dk)),
                v=rng.standard_normal((B, T, H, dv)),
                g=-np.log1p(np.exp(-rng.standard_normal((B, T, H, dk)))) * 0.3,
                S_in=0.5 * rng.standard_normal((B, H, dk, dv)))


def _check(fd, an, name):
    scale = max(np.max(np.abs(fd)), 1e-3)
    err = np.max(np.abs(fd - an)) / scale
    assert err < 2e-7, (name, err)


@pytest.mark.parametrize("shape", [(1, 5, 1, 3, 2), (2, 9, 2, 4, 3), (1, 70, 1, 2, 2)])
def test_gdn_adjoints_match_finite_differences(shape):
    rng = np.random.default_rng(sum(shape))
    B, T, H, dk, dv = shape
    x = _rand_gdn(rng, *shape)
    dO = rng.standard_normal((B, T, H, dv))
    dS_out = rng.standard_normal((B, H, dk, dv))
    r = oracle.gdn_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"], dO, dS_out)
    names = dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", S_in="dS_in")
    for key, gname in names.items():
        _check(_fd(_loss_gdn, x, key, dO, dS_out), r[gname], gname)


@pytest.mark.parametrize("shape", [(1, 5, 1, 3, 2), (2, 9, 2, 4, 3), (1, 70, 1, 2, 2)])
def test_gla_adjoints_match_finite_differences(shape):
    rng = np.random.default_rng(100 + sum(shape))
    B, T, H, dk, dv = shape
    x = _rand_gla(rng, *shape)
    dO = rng.standard_normal((B, T, H, dv))
    dS_out = rng.standard_normal((B, H, dk, dv))
    r = oracle.gla_bwd(x["q"], x["k"], x["v"], x["g"], x["S_in"], dO, dS_out)
    names = dict(q="dq", k="dk", v="dv", g="dg", S_in="dS_in")
    for key, gname in names.items():
        _check(_fd(_loss_gla, x, key, dO, dS_out), r[gname], gname)


def test_null_state_and_null_upstream_mean_zero():
    rng = np.random.default_rng(7)
    x = _rand_gdn(rng, 1, 6, 2, 3, 4)
    z = np.zeros((1, 2, 3, 4))
    dO = rng.standard_normal((1, 6, 2, 4))
    o1, s1 = oracle.gdn_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], None)
    o2, s2 = oracle.gdn_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], z)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
    r1 = oracle.gdn_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], None, dO, None)
    r2 = oracle.gdn_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], z, dO, z)
    for key in r1:
        assert np.array_equal(r1[key], r2[key]), key
