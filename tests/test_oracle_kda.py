"""Pins the KDA oracle (per-key-channel decay with the delta rule's erase and
write, S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T, the
diagonal-plus-low-rank transition of the StateFlow paper, Sec. 2.1, Eq. 1)
to things other than itself: finite differences of every gradient; the
reduction to the Gated DeltaNet oracle when the decay is the same on every
channel; the pure-decay closed form at beta = 0; the one-token matrix form;
the chunk split; and the chunk (WY) form that the GPU forward computes,
written out in numpy from its derivation."""
import numpy as np
import pytest

from oracle import oracle
from tests.test_oracle_fd import _check, _fd


def _rand(rng, B, T, H, dk, dv, gscale=0.3):
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    return dict(q=rng.standard_normal((B, T, H, dk)), k=k, v=rng.standard_normal((B, T, H, dv)),
                g=-np.log1p(np.exp(rng.standard_normal((B, T, H, dk)))) * gscale,
                beta=1 / (1 + np.exp(-rng.standard_normal((B, T, H)))),
                S_in=0.5 * rng.standard_normal((B, H, dk, dv)))


def _loss(x, dO, dS):
    o, S = oracle.kda_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"])
    return float(np.sum(o * dO) + np.sum(S * dS))


@pytest.mark.parametrize("shape", [(1, 5, 1, 3, 2), (2, 9, 2, 4, 3), (1, 70, 1, 2, 2)])
def test_adjoints_match_finite_differences(shape):
    rng = np.random.default_rng(300 + sum(shape))
    B, T, H, dk, dv = shape
    x = _rand(rng, *shape)
    dO = rng.standard_normal((B, T, H, dv))
    dS = rng.standard_normal((B, H, dk, dv))
    r = oracle.kda_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"], dO, dS)
    for key, gname in dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", S_in="dS_in").items():
        _check(_fd(_loss, x, key, dO, dS), r[gname], gname)


def test_uniform_decay_is_gated_deltanet():
    rng = np.random.default_rng(31)
    B, T, H, dk, dv = 1, 37, 2, 4, 3
    x = _rand(rng, B, T, H, dk, dv)
    gs = x["g"][..., 0].copy()
    gb = np.repeat(gs[..., None], dk, -1)
    dO = rng.standard_normal((B, T, H, dv))
    dS = rng.standard_normal((B, H, dk, dv))
    o1, S1 = oracle.kda_fwd(x["q"], x["k"], x["v"], gb, x["beta"], x["S_in"])
    o2, S2 = oracle.gdn_fwd(x["q"], x["k"], x["v"], gs, x["beta"], x["S_in"])
    assert np.allclose(o1, o2, atol=1e-12) and np.allclose(S1, S2, atol=1e-12)
    r1 = oracle.kda_bwd(x["q"], x["k"], x["v"], gb, x["beta"], x["S_in"], dO, dS)
    r2 = oracle.gdn_bwd(x["q"], x["k"], x["v"], gs, x["beta"], x["S_in"], dO, dS)
    for key in ("dq", "dk", "dv", "dbeta", "dS_in"):
        assert np.allclose(r1[key], r2[key], atol=1e-11), key
    assert np.allclose(r1["dg"].sum(-1), r2["dg"], atol=1e-11)


def test_zero_beta_is_pure_channel_decay():
    rng = np.random.default_rng(32)
    B, T, H, dk, dv = 1, 19, 1, 5, 3
    x = _rand(rng, B, T, H, dk, dv, gscale=1.0)
    o, S = oracle.kda_fwd(x["q"], x["k"], x["v"], x["g"], np.zeros((B, T, H)), x["S_in"])
    b = np.cumsum(x["g"][0, :, 0], 0)  # [T, dk]
    S0 = x["S_in"][0, 0]
    for t in range(T):
        St = np.exp(b[t])[:, None] * S0
        assert np.allclose(o[0, t, 0], St.T @ x["q"][0, t, 0], atol=1e-12)
    assert np.allclose(S[0, 0], np.exp(b[-1])[:, None] * S0, atol=1e-12)


def test_one_token_transition_matrix():
    rng = np.random.default_rng(33)
    dk, dv = 5, 3
    x = _rand(rng, 1, 1, 1, dk, dv)
    o, S = oracle.kda_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"])
    k, v, bt = x["k"][0, 0, 0], x["v"][0, 0, 0], x["beta"][0, 0, 0]
    ref = (np.eye(dk) - bt * np.outer(k, k)) @ np.diag(np.exp(x["g"][0, 0, 0])) @ x["S_in"][0, 0] + bt * np.outer(k, v)
    assert np.allclose(S[0, 0], ref, atol=1e-13) and np.allclose(o[0, 0, 0], ref.T @ x["q"][0, 0, 0], atol=1e-13)


def chunk_form(q, k, v, g, beta, S0, C):
    """The block (WY) form of one head, blocks of C tokens: with b the
    in-block cumulative log decay per channel,
      M[t][s] = sum_d k_t[d] k_s[d] e^{b_t[d] - b_s[d]}   (s < t)
      T = (I + Diag(beta) M)^-1,  W = T Diag(beta) (K * e^b),  Ut = T Diag(beta) V
      U = Ut - W S,  O = (Q * e^b) S + (P * tril) U,
      P[t][s] = sum_d q_t[d] k_s[d] e^{b_t[d] - b_s[d]}   (s <= t)
      S <- Diag(e^{b_C}) S + (K * e^{b_C - b})^T U."""
    T, dk = q.shape
    S = S0.copy()
    out = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, C):
        sl = slice(c0, min(c0 + C, T))
        Q, K, V, G, Bt = q[sl], k[sl], v[sl], g[sl], beta[sl]
        b = np.cumsum(G, 0)
        n = Q.shape[0]
        D = np.exp(b[:, None, :] - b[None, :, :])          # [t, s, d], e^{b_t - b_s}
        M = np.einsum("td,sd,tsd->ts", K, K, D) * np.tril(np.ones((n, n)), -1)
        P = np.einsum("td,sd,tsd->ts", Q, K, D) * np.tril(np.ones((n, n)))
        Tm = np.linalg.inv(np.eye(n) + Bt[:, None] * M)
        Wm = Tm @ (Bt[:, None] * K * np.exp(b))
        Ut = Tm @ (Bt[:, None] * V)
        U = Ut - Wm @ S
        out[sl] = (Q * np.exp(b)) @ S + P @ U
        S = np.exp(b[-1])[:, None] * S + (K * np.exp(b[-1] - b)).T @ U
    return out, S


@pytest.mark.parametrize("C", [4, 16, 64])
def test_chunk_form_equals_the_recurrence(C):
    rng = np.random.default_rng(34 + C)
    T, dk, dv = 150, 6, 5
    x = _rand(rng, 1, T, 1, dk, dv)
    o, S = oracle.kda_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"])
    oc, Sc = chunk_form(x["q"][0, :, 0], x["k"][0, :, 0], x["v"][0, :, 0], x["g"][0, :, 0],
                        x["beta"][0, :, 0], x["S_in"][0, 0], C)
    assert np.allclose(oc, o[0, :, 0], atol=1e-10) and np.allclose(Sc, S[0, 0], atol=1e-10)


@pytest.mark.parametrize("N", [2, 5])
def test_chunk_split_is_bit_exact(N):
    rng = np.random.default_rng(40 + N)
    B, T, H, dk, dv = 1, 130, 2, 3, 2
    x = _rand(rng, B, T, H, dk, dv)
    dO = rng.standard_normal((B, T, H, dv))
    dS = rng.standard_normal((B, H, dk, dv))
    o1, S1 = oracle.kda_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"])
    r1 = oracle.kda_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"], dO, dS)
    L = T // N
    S, states, outs = x["S_in"], [], []
    for i in range(N):
        sl = slice(i * L, (i + 1) * L)
        states.append(S)
        oi, S = oracle.kda_fwd(x["q"][:, sl], x["k"][:, sl], x["v"][:, sl], x["g"][:, sl], x["beta"][:, sl], S)
        outs.append(oi)
    assert np.array_equal(np.concatenate(outs, 1), o1) and np.array_equal(S, S1)
    ds, parts = dS, [None] * N
    for i in reversed(range(N)):
        sl = slice(i * L, (i + 1) * L)
        parts[i] = oracle.kda_bwd(x["q"][:, sl], x["k"][:, sl], x["v"][:, sl], x["g"][:, sl], x["beta"][:, sl],
                                  states[i], dO[:, sl], ds)
        ds = parts[i]["dS_in"]
    for key in ("dq", "dk", "dv", "dg", "dbeta"):
        assert np.array_equal(np.concatenate([p[key] for p in parts], 1), r1[key]), key
    assert np.array_equal(ds, r1["dS_in"])


@pytest.mark.parametrize("C", [4, 16, 64])
def test_chunk_form_backward_equals_the_oracle(C):
    """The block adjoints the GPU backward implements (tests/kda_chunk_bwd.py)
    against the oracle's per-token adjoints."""
    from tests.kda_chunk_bwd import kda_chunk_bwd
    rng = np.random.default_rng(50 + C)
    T, dk, dv = 150, 6, 5
    x = _rand(rng, 1, T, 1, dk, dv)
    dO = rng.standard_normal((1, T, 1, dv))
    dS = rng.standard_normal((1, 1, dk, dv))
    ref = oracle.kda_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"], dO, dS)
    got = kda_chunk_bwd(x["q"][0, :, 0], x["k"][0, :, 0], x["v"][0, :, 0], x["g"][0, :, 0], x["beta"][0, :, 0],
                        x["S_in"][0, 0], dO[0, :, 0], dS[0, 0], C)
    for key in ("dq", "dk", "dv", "dg", "dbeta"):
        r = ref[key][0, :, 0]
        assert np.allclose(got[key], r, atol=1e-9 * max(1.0, np.max(np.abs(r)))), key
    assert np.allclose(got["dS_in"], ref["dS_in"][0, 0], atol=1e-9)
