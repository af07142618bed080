"""Pins the scalar-gate (Mamba-2) oracle, S_t = alpha_t S_{t-1} + k_t v_t^T,
o_t = S_t^T q_t (the scalar-identity transition of the StateFlow paper,
Sec. 2.1, Eq. 1), to things other than itself:

* brute force: central finite differences of every gradient, including dS_in,
  on tiny inputs (T = 70 crosses the 64-token checkpoint);
* closed forms: zero gate is causal linear attention; the general case equals
  the quadratic "attention" form with decay exp(sum of g over (s, t]);
* invariants that hold at any size: q.dq = o.dO and k.dk = v.dv per token,
  and dg_t = sum_{tau >= t} (q.dq - k.dk) + <S_out, dS_out>;
* reduction: it is the GLA map with the gate broadcast over key channels,
  and its dg is the channel sum of the GLA dg;
* the chunk-split invariant, bit-exactly."""
import numpy as np
import pytest

from oracle import oracle
from tests.test_oracle_fd import _check, _fd


def _rand(rng, B, T, H, dk, dv, gscale=0.3):
    return dict(q=rng.standard_normal((B, T, H, dk)), k=rng.standard_normal((B, T, H, dk)),
                v=rng.standard_normal((B, T, H, dv)),
                g=-np.log1p(np.exp(rng.standard_normal((B, T, H)))) * gscale,
                S_in=0.5 * rng.standard_normal((B, H, dk, dv)))


def _loss(x, dO, dS_out):
    o, S = oracle.mamba2_fwd(x["q"], x["k"], x["v"], x["g"], x["S_in"])
    return float(np.sum(o * dO) + np.sum(S * dS_out))


@pytest.mark.parametrize("shape", [(1, 5, 1, 3, 2), (2, 9, 2, 4, 3), (1, 70, 1, 2, 2)])
def test_adjoints_match_finite_differences(shape):
    rng = np.random.default_rng(200 + sum(shape))
    B, T, H, dk, dv = shape
    x = _rand(rng, *shape)
    dO = rng.standard_normal((B, T, H, dv))
    dS_out = rng.standard_normal((B, H, dk, dv))
    r = oracle.mamba2_bwd(x["q"], x["k"], x["v"], x["g"], x["S_in"], dO, dS_out)
    for key, gname in dict(q="dq", k="dk", v="dv", g="dg", S_in="dS_in").items():
        _check(_fd(_loss, x, key, dO, dS_out), r[gname], gname)


def test_zero_gate_is_causal_linear_attention():
    rng = np.random.default_rng(5)
    x = _rand(rng, 1, 11, 1, 4, 3)
    o, S = oracle.mamba2_fwd(x["q"], x["k"], x["v"], np.zeros((1, 11, 1)), x["S_in"])
    Q, K, V, S0 = x["q"][0, :, 0], x["k"][0, :, 0], x["v"][0, :, 0], x["S_in"][0, 0]
    assert np.allclose(o[0, :, 0], np.tril(Q @ K.T) @ V + Q @ S0, atol=1e-12)
    assert np.allclose(S[0, 0], S0 + K.T @ V, atol=1e-12)


def test_quadratic_form():
    """o_t = e^{c_t} S_in^T q_t + sum_{s<=t} e^{c_t - c_s} (q_t.k_s) v_s, c = cumsum(g)."""
    rng = np.random.default_rng(6)
    T, dk, dv = 23, 5, 4
    x = _rand(rng, 1, T, 1, dk, dv, gscale=1.0)
    o, S = oracle.mamba2_fwd(x["q"], x["k"], x["v"], x["g"], x["S_in"])
    Q, K, V, S0 = x["q"][0, :, 0], x["k"][0, :, 0], x["v"][0, :, 0], x["S_in"][0, 0]
    c = np.cumsum(x["g"][0, :, 0])
    D = np.tril(np.exp(c[:, None] - c[None, :]))
    ref = ((Q @ K.T) * D) @ V + np.exp(c)[:, None] * (Q @ S0)
    assert np.allclose(o[0, :, 0], ref, atol=1e-11)
    Sref = np.exp(c[-1]) * S0 + (K * np.exp(c[-1] - c)[:, None]).T @ V
    assert np.allclose(S[0, 0], Sref, atol=1e-11)


def test_identities():
    rng = np.random.default_rng(8)
    B, T, H, dk, dv = 2, 37, 2, 4, 3
    x = _rand(rng, B, T, H, dk, dv)
    dO = rng.standard_normal((B, T, H, dv))
    dS_out = rng.standard_normal((B, H, dk, dv))
    o, S_out = oracle.mamba2_fwd(x["q"], x["k"], x["v"], x["g"], x["S_in"])
    r = oracle.mamba2_bwd(x["q"], x["k"], x["v"], x["g"], x["S_in"], dO, dS_out)
    qdq = np.sum(x["q"] * r["dq"], -1)
    kdk = np.sum(x["k"] * r["dk"], -1)
    assert np.allclose(qdq, np.sum(o * dO, -1), atol=1e-10)
    assert np.allclose(kdk, np.sum(x["v"] * r["dv"], -1), atol=1e-10)
    suffix = np.flip(np.cumsum(np.flip(qdq - kdk, 1), 1), 1)
    gate = suffix + np.sum(S_out * dS_out, axis=(2, 3))[:, None, :]
    assert np.allclose(r["dg"], gate, atol=1e-10)


def test_is_gla_with_a_broadcast_gate():
    rng = np.random.default_rng(9)
    B, T, H, dk, dv = 1, 29, 2, 4, 3
    x = _rand(rng, B, T, H, dk, dv)
    dO = rng.standard_normal((B, T, H, dv))
    dS_out = rng.standard_normal((B, H, dk, dv))
    gb = np.repeat(x["g"][..., None], dk, axis=-1)
    o1, S1 = oracle.mamba2_fwd(x["q"], x["k"], x["v"], x["g"], x["S_in"])
    o2, S2 = oracle.gla_fwd(x["q"], x["k"], x["v"], gb, x["S_in"])
    assert np.allclose(o1, o2, atol=1e-12) and np.allclose(S1, S2, atol=1e-12)
    r1 = oracle.mamba2_bwd(x["q"], x["k"], x["v"], x["g"], x["S_in"], dO, dS_out)
    r2 = oracle.gla_bwd(x["q"], x["k"], x["v"], gb, x["S_in"], dO, dS_out)
    for key in ("dq", "dk", "dv", "dS_in"):
        assert np.allclose(r1[key], r2[key], atol=1e-11), key
    assert np.allclose(r1["dg"], r2["dg"].sum(-1), atol=1e-11)


@pytest.mark.parametrize("N", [2, 5])
def test_chunk_split_is_bit_exact(N):
    rng = np.random.default_rng(10 + N)
    B, T, H, dk, dv = 1, 130, 2, 3, 2
    T = T - T % N
    x = _rand(rng, B, T, H, dk, dv)
    dO = rng.standard_normal((B, T, H, dv))
    dS_out = rng.standard_normal((B, H, dk, dv))
    o1, S1, g1 = oracle.mamba2_chunked(x["q"], x["k"], x["v"], x["g"], x["S_in"], dO, dS_out, 1)
    oN, SN, gN = oracle.mamba2_chunked(x["q"], x["k"], x["v"], x["g"], x["S_in"], dO, dS_out, N)
    assert np.array_equal(o1, oN) and np.array_equal(S1, SN)
    for key in g1:
        assert np.array_equal(g1[key], gN[key]), key
