"""fp64 numpy model of the chunkwise (64-token block) algorithm that the HIP
kernels implement.  It is a design check, not the oracle and not the product:
it validates, at fp64, that the block algebra below reproduces the per-token
recurrence (checked against the oracle in test_chunk_algebra.py) before any
of it is written as GPU code.

Gated DeltaNet, key-major state S (dk x dv), one block of C tokens, S0 = state
entering the block.  With gamma = cumsum(g) inside the block, Gam = exp(gamma),
G[r,s] = exp(gamma_r - gamma_s):
  A   = Diag(beta) strict_lower(K K^T * G)          (UT transform input)
  T   = (I + A)^-1
  W   = T Diag(beta Gam) K ,  Ut = T Diag(beta) V   (WY pair, independent of S0)
  U   = Ut - W S0                                   (the "new values")
  O   = Diag(Gam) Q S0 + (Q K^T * G * tril) U
  S1  = Gam_C S0 + Kh^T U ,  Kh = Diag(exp(gamma_C - gamma)) K
This is the Pre / state-transition / Out split of the StateFlow paper,
Sec. 2.2 (Eq. 2), with U playing the role of V^new.

Backward of one block given dO and dS1 (gradient w.r.t. the state leaving the
block):
  dU  = (Q K^T * G * tril)^T dO + Kh dS1
  dS0 = Gam_C dS1 + (Diag(Gam) Q)^T dO - W^T dU
and the per-block input gradients listed in block_bwd.  The gate gradient
uses the scaling identity  dg_r = sum_{tau>=r in block}(q.dq - v.dv) + <S1, dS1>.
"""
import numpy as np


def block_fwd(Q, K, V, g, beta, S0):
    C = Q.shape[0]
    gam = np.cumsum(g)
    Gam = np.exp(gam)
    G = np.exp(gam[:, None] - gam[None, :])
    L = np.tril(np.ones((C, C)))
    Ls = np.tril(np.ones((C, C)), -1)
    A = beta[:, None] * (K @ K.T) * G * Ls
    T = np.linalg.inv(np.eye(C) + A)
    W = T @ ((beta * Gam)[:, None] * K)
    Ut = T @ (beta[:, None] * V)
    U = Ut - W @ S0
    P = (Q @ K.T) * G * L
    O = Gam[:, None] * (Q @ S0) + P @ U
    Kh = np.exp(gam[-1] - gam)[:, None] * K
    S1 = Gam[-1] * S0 + Kh.T @ U
    return O, S1, dict(gam=gam, Gam=Gam, G=G, T=T, W=W, U=U, P=P, Kh=Kh, A=A)


def block_bwd(Q, K, V, g, beta, S0, S1, dO, dS1, c):
    """Returns dQ, dK, dV, dg, dbeta, dS0 for one block (c = block_fwd cache)."""
    C = Q.shape[0]
    gam, Gam, G, T, W, U, P, Kh = (c[k] for k in ("gam", "Gam", "G", "T", "W", "U", "P", "Kh"))
    L = np.tril(np.ones((C, C)))
    Ls = np.tril(np.ones((C, C)), -1)
    # reverse state step
    dU = P.T @ dO + Kh @ dS1
    dS0 = Gam[-1] * dS1 + (Gam[:, None] * Q).T @ dO - W.T @ dU
    # output path
    dPm = (dO @ U.T) * G * L
    dQ = Gam[:, None] * (dO @ S0.T) + dPm @ K
    dK = dPm.T @ Q
    # state-update path: S1 = ... + Kh^T U
    dK += np.exp(gam[-1] - gam)[:, None] * (U @ dS1.T)
    # U = Ut - W S0, Ut = T Diag(beta) V, W = T Diag(beta Gam) K
    dW = -dU @ S0.T
    dT = dU @ (beta[:, None] * V).T + dW @ ((beta * Gam)[:, None] * K).T
    TdU = T.T @ dU
    TdW = T.T @ dW
    dV = beta[:, None] * TdU
    dK += (beta * Gam)[:, None] * TdW
    dbeta = np.sum(TdU * V, 1) + Gam * np.sum(TdW * K, 1)
    # T = (I + A)^-1  ->  dA = -T^T dT T^T on the strictly-lower part
    dA = -(T.T @ dT @ T.T) * Ls
    KK = K @ K.T
    dbeta += np.sum(dA * KK * G, 1)
    M = dA * beta[:, None] * G
    dK += M @ K + M.T @ K
    # gate gradient by the scaling identity (o.do = q.dq per token)
    qdq = np.sum(Q * dQ, 1)
    vdv = np.sum(V * dV, 1)
    end = np.sum(S1 * dS1)
    dg = np.flip(np.cumsum(np.flip(qdq - vdv))) + end
    return dQ, dK, dV, dg, dbeta, dS0


def gdn_chunked_fwd_bwd(q, k, v, g, beta, S_in, dO, dS_out, C=64):
    """One (b, h) sequence: q [T,dk], ... Returns o, S_out, grads dict."""
    T_ = q.shape[0]
    nb = T_ // C
    S = S_in.copy()
    hs, caches, outs = [], [], []
    for n in range(nb):
        sl = slice(n * C, (n + 1) * C)
        O, S1, c = block_fwd(q[sl], k[sl], v[sl], g[sl], beta[sl], S)
        hs.append(S)
        caches.append((c, S1))
        outs.append(O)
        S = S1
    S_out = S
    dS = dS_out.copy()
    gr = {key: [None] * nb for key in ("dq", "dk", "dv", "dg", "dbeta")}
    for n in reversed(range(nb)):
        sl = slice(n * C, (n + 1) * C)
        c, S1 = caches[n]
        r = block_bwd(q[sl], k[sl], v[sl], g[sl], beta[sl], hs[n], S1, dO[sl], dS, c)
        for key, val in zip(("dq", "dk", "dv", "dg", "dbeta"), r[:5]):
            gr[key][n] = val
        dS = r[5]
    out = {key: np.concatenate(val) for key, val in gr.items()}
    out["dS_in"] = dS
    return np.concatenate(outs), S_out, out


# ---------------------------------------------------------------------------
# GLA (per-channel gate b = cumsum(g) inside the block, no delta term)
#   O  = (Q * exp(b)) S0 + (Q~ K~^T * tril) V,   Q~ = Q*exp(b - ref), K~ = K*exp(ref - b)
#   S1 = Diag(exp(b_C)) S0 + (K * exp(b_C - b))^T V
# Backward: dS0 = Diag(exp(b_C)) dS1 + (Q*exp(b))^T dO,
#   dq, dk, dv by the same products, dg by the per-channel scaling identity
#   dg_r[i] = sum_{tau>=r}(q dq - k dk)[i] + rowsum(S1 * dS1)[i].
# ---------------------------------------------------------------------------

def gla_block_fwd(Q, K, V, g, S0):
    C = Q.shape[0]
    b = np.cumsum(g, 0)
    L = np.tril(np.ones((C, C)))
    E = np.exp(b[:, None, :] - b[None, :, :])            # [r, s, i]
    P = np.einsum("ri,si,rsi->rs", Q, K, E) * L
    O = (Q * np.exp(b)) @ S0 + P @ V
    S1 = np.exp(b[-1])[:, None] * S0 + (K * np.exp(b[-1] - b)).T @ V
    return O, S1, dict(b=b, P=P, E=E)


def gla_block_bwd(Q, K, V, g, S0, S1, dO, dS1, c):
    C = Q.shape[0]
    b, P, E = c["b"], c["P"], c["E"]
    L = np.tril(np.ones((C, C)))
    Kh = K * np.exp(b[-1] - b)
    dS0 = np.exp(b[-1])[:, None] * dS1 + (Q * np.exp(b)).T @ dO
    dP = (dO @ V.T) * L
    dQ = np.exp(b) * (dO @ S0.T) + np.einsum("rs,si,rsi->ri", dP, K, E)
    dK = np.einsum("rs,ri,rsi->si", dP, Q, E) + np.exp(b[-1] - b) * (V @ dS1.T)
    dV = P.T @ dO + Kh @ dS1
    end = np.sum(S1 * dS1, 1)
    term = Q * dQ - K * dK
    dg = np.flip(np.cumsum(np.flip(term, 0), 0), 0) + end[None, :]
    return dQ, dK, dV, dg, dS0


def gla_chunked_fwd_bwd(q, k, v, g, S_in, dO, dS_out, C=64):
    T_ = q.shape[0]
    nb = T_ // C
    S = S_in.copy()
    hs, caches, outs = [], [], []
    for n in range(nb):
        sl = slice(n * C, (n + 1) * C)
        O, S1, c = gla_block_fwd(q[sl], k[sl], v[sl], g[sl], S)
        hs.append(S)
        caches.append((c, S1))
        outs.append(O)
        S = S1
    S_out = S
    dS = dS_out.copy()
    gr = {key: [None] * nb for key in ("dq", "dk", "dv", "dg")}
    for n in reversed(range(nb)):
        sl = slice(n * C, (n + 1) * C)
        c, S1 = caches[n]
        r = gla_block_bwd(q[sl], k[sl], v[sl], g[sl], hs[n], S1, dO[sl], dS, c)
        for key, val in zip(("dq", "dk", "dv", "dg"), r[:4]):
            gr[key][n] = val
        dS = r[4]
    out = {key: np.concatenate(val) for key, val in gr.items()}
    out["dS_in"] = dS
    return np.concatenate(outs), S_out, out
