"""Pins the oracle's forward (and, through identities, its backward) to
closed forms and textbook special cases that do not use the oracle's
per-token delta-form code path:

  * one token: S_out = alpha (I - beta k k^T) S_in + beta k v^T, built as an
    explicit dk x dk transition matrix (numpy matmul);
  * GDN with beta = 0: o_t = exp(sum_{s<=t} g_s) S_in^T q_t, S_out = exp(sum g) S_in;
  * GDN with g = 0, beta = 1 and keys that are distinct standard basis vectors:
    the delta rule overwrites row pi(t) of S with v_t (associative memory);
  * GDN general: product-of-transition-matrices form
    S_t = A_t S_{t-1} + beta_t k_t v_t^T with A_t = alpha_t (I - beta_t k_t k_t^T)
    as explicit matrices;
  * GLA with g = 0: O = tril(Q K^T) V + Q S_in, S_out = S_in + K^T V;
  * GLA general: the O(T^2) parallel form
    o_t = S_in^T (exp(b_t) * q_t) + sum_{s<=t} ((q_t * exp(b_t - b_s)) . k_s) v_s,
    with b_t = sum_{s<=t} g_s per channel.
The layer family and its transitions are those of the StateFlow paper, Sec. 2.1."""
import numpy as np

from oracle import oracle


def _rng(s):
    return np.random.default_rng(s)


def test_single_token_transition_matrix():
    r = _rng(1)
    dk, dv = 5, 3
    q = r.standard_normal((1, 1, 1, dk))
    k = r.standard_normal((1, 1, 1, dk))
    v = r.standard_normal((1, 1, 1, dv))
    g = np.array([[[-0.3]]])
    beta = np.array([[[0.7]]])
    S0 = r.standard_normal((1, 1, dk, dv))
    o, S1 = oracle.gdn_fwd(q, k, v, g, beta, S0)
    kk = k[0, 0, 0]
    A = np.exp(-0.3) * (np.eye(dk) - 0.7 * np.outer(kk, kk))
    S_ref = A @ S0[0, 0] + 0.7 * np.outer(kk, v[0, 0, 0])
    np.testing.assert_allclose(S1[0, 0], S_ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(o[0, 0, 0], S_ref.T @ q[0, 0, 0], rtol=1e-13, atol=1e-13)


def test_gdn_beta_zero_is_pure_decay():
    r = _rng(2)
    B, T, H, dk, dv = 2, 11, 3, 4, 6
    q = r.standard_normal((B, T, H, dk))
    k = r.standard_normal((B, T, H, dk))
    v = r.standard_normal((B, T, H, dv))
    g = -np.abs(r.standard_normal((B, T, H)))
    S0 = r.standard_normal((B, H, dk, dv))
    o, S1 = oracle.gdn_fwd(q, k, v, g, np.zeros((B, T, H)), S0)
    cg = np.cumsum(g, axis=1)
    o_ref = np.exp(cg)[..., None] * np.einsum("bhkv,bthk->bthv", S0, q)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S1, np.exp(cg[:, -1])[:, :, None, None] * S0, rtol=1e-12)


def test_gdn_delta_rule_overwrites_basis_rows():
    r = _rng(3)
    dk, dv, T = 8, 5, 8
    perm = r.permutation(dk)
    k = np.zeros((1, T, 1, dk))
    for t in range(T):
        k[0, t, 0, perm[t]] = 1.0
    v = r.standard_normal((1, T, 1, dv))
    q = r.standard_normal((1, T, 1, dk))
    S0 = r.standard_normal((1, 1, dk, dv))
    o, S1 = oracle.gdn_fwd(q, k, v, np.zeros((1, T, 1)), np.ones((1, T, 1)), S0)
    S = S0[0, 0].copy()
    for t in range(T):
        S[perm[t]] = v[0, t, 0]        # row pi(t) replaced by v_t
        np.testing.assert_allclose(o[0, t, 0], S.T @ q[0, t, 0], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S1[0, 0], S, rtol=0, atol=1e-14)


def test_gdn_transition_matrix_product_form():
    r = _rng(4)
    B, T, H, dk, dv = 1, 37, 2, 6, 4
    q = r.standard_normal((B, T, H, dk))
    k = r.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, T, H, dv))
    g = -np.abs(r.standard_normal((B, T, H))) * 0.2
    beta = r.uniform(0, 1, (B, T, H))
    S0 = r.standard_normal((B, H, dk, dv))
    o, S1 = oracle.gdn_fwd(q, k, v, g, beta, S0)
    for h in range(H):
        S = S0[0, h]
        for t in range(T):
            kt = k[0, t, h]
            A = np.exp(g[0, t, h]) * (np.eye(dk) - beta[0, t, h] * np.outer(kt, kt))
            S = A @ S + beta[0, t, h] * np.outer(kt, v[0, t, h])
            np.testing.assert_allclose(o[0, t, h], S.T @ q[0, t, h], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(S1[0, h], S, rtol=1e-11, atol=1e-12)


def test_gla_zero_gate_is_causal_linear_attention():
    r = _rng(5)
    B, T, H, dk, dv = 2, 13, 2, 5, 7
    q = r.standard_normal((B, T, H, dk))
    k = r.standard_normal((B, T, H, dk))
    v = r.standard_normal((B, T, H, dv))
    S0 = r.standard_normal((B, H, dk, dv))
    o, S1 = oracle.gla_fwd(q, k, v, np.zeros((B, T, H, dk)), S0)
    for b in range(B):
        for h in range(H):
            Q, K, V = q[b, :, h], k[b, :, h], v[b, :, h]
            ref = np.tril(Q @ K.T) @ V + Q @ S0[b, h]
            np.testing.assert_allclose(o[b, :, h], ref, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(S1[b, h], S0[b, h] + K.T @ V, rtol=1e-12, atol=1e-12)


def test_gla_parallel_form():
    r = _rng(6)
    B, T, H, dk, dv = 1, 29, 2, 6, 5
    q = r.standard_normal((B, T, H, dk))
    k = r.standard_normal((B, T, H, dk))
    v = r.standard_normal((B, T, H, dv))
    g = -np.abs(r.standard_normal((B, T, H, dk))) * 0.3
    S0 = r.standard_normal((B, H, dk, dv))
    o, S1 = oracle.gla_fwd(q, k, v, g, S0)
    bcum = np.cumsum(g, axis=1)
    for h in range(H):
        for t in range(T):
            ref = S0[0, h].T @ (np.exp(bcum[0, t, h]) * q[0, t, h])
            for s in range(t + 1):
                w = np.sum(q[0, t, h] * np.exp(bcum[0, t, h] - bcum[0, s, h]) * k[0, s, h])
                ref = ref + w * v[0, s, h]
            np.testing.assert_allclose(o[0, t, h], ref, rtol=1e-11, atol=1e-12)
        Sref = np.exp(bcum[0, -1, h])[:, None] * S0[0, h]
        for s in range(T):
            Sref += np.outer(np.exp(bcum[0, -1, h] - bcum[0, s, h]) * k[0, s, h], v[0, s, h])
        np.testing.assert_allclose(S1[0, h], Sref, rtol=1e-11, atol=1e-12)


def test_gradients_against_torch_autograd_of_matrix_form():
    """A third opinion for every gradient: torch fp64 autograd of the explicit
    transition-matrix form (a different code path and mechanism)."""
    import torch
    r = _rng(8)
    B, T, H, dk, dv = 1, 12, 2, 4, 3
    q = r.standard_normal((B, T, H, dk))
    k = r.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, T, H, dv))
    g = -np.abs(r.standard_normal((B, T, H))) * 0.3
    beta = r.uniform(0.1, 0.9, (B, T, H))
    S0 = r.standard_normal((B, H, dk, dv))
    dO = r.standard_normal((B, T, H, dv))
    dS = r.standard_normal((B, H, dk, dv))
    ts = [torch.tensor(a, requires_grad=True) for a in (q, k, v, g, beta, S0)]
    tq, tk, tv, tg, tb, tS = ts
    L = 0
    for h in range(H):
        S = tS[0, h]
        for t in range(T):
            kt = tk[0, t, h]
            A = torch.exp(tg[0, t, h]) * (torch.eye(dk, dtype=torch.float64) - tb[0, t, h] * torch.outer(kt, kt))
            S = A @ S + tb[0, t, h] * torch.outer(kt, tv[0, t, h])
            L = L + (S.T @ tq[0, t, h] * torch.tensor(dO[0, t, h])).sum()
        L = L + (S * torch.tensor(dS[0, h])).sum()
    L.backward()
    ro = oracle.gdn_bwd(q, k, v, g, beta, S0, dO, dS)
    for t, name in zip(ts, ("dq", "dk", "dv", "dg", "dbeta", "dS_in")):
        np.testing.assert_allclose(ro[name], t.grad.numpy(), rtol=1e-10, atol=1e-11, err_msg=name)

    # GLA
    g2 = -np.abs(r.standard_normal((B, T, H, dk))) * 0.3
    ts = [torch.tensor(a, requires_grad=True) for a in (q, k, v, g2, S0)]
    tq, tk, tv, tg, tS = ts
    L = 0
    for h in range(H):
        S = tS[0, h]
        for t in range(T):
            S = torch.diag(torch.exp(tg[0, t, h])) @ S + torch.outer(tk[0, t, h], tv[0, t, h])
            L = L + (S.T @ tq[0, t, h] * torch.tensor(dO[0, t, h])).sum()
        L = L + (S * torch.tensor(dS[0, h])).sum()
    L.backward()
    ro = oracle.gla_bwd(q, k, v, g2, S0, dO, dS)
    for t, name in zip(ts, ("dq", "dk", "dv", "dg", "dS_in")):
        np.testing.assert_allclose(ro[name], t.grad.numpy(), rtol=1e-10, atol=1e-11, err_msg=name)
