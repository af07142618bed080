"""The block (WY) form of the KDA backward in fp64 numpy: a design check of
the adjoints the GPU backward implements, compared with the oracle's
per-token adjoints in tests/test_oracle_kda.py.  Shares nothing with the
kernels.

Per block of C tokens, with S0 the state entering the block and dS1 the
gradient of the state leaving it, b = cumsum(g) per channel,
E[t][s] = e^{b_t - b_s} per channel, and the forward quantities
  M = sum_d K K E (s < t), A = Diag(beta) M, T = (I + A)^-1,
  Kt = K e^b, X = Diag(beta) Kt, Y = Diag(beta) V, W = T X, Ut = T Y,
  U = Ut - W S0, P = sum_d Q K E (s <= t), Qt = Q e^b, Kh = K e^{b_C - b}:
  dU   = P^T dO + Kh dS1
  dS0  = Qt^T dO + Diag(e^{b_C}) dS1 - W^T dU
  dQt  = dO S0^T,  dP = (dO U^T) * tril,  dKh = U dS1^T
  dW   = -dU S0^T,  dT = dW X^T + dU Y^T,  dX = T^T dW,  dY = T^T dU
  dA   = -T^T dT T^T (strictly lower),  dM = Diag(beta) dA
  dq_t = dQt_t e^{b_t} + sum_s dP_ts k_s E_ts
  dk_s = sum_t dP_ts q_t E_ts                         (P, column side)
       + sum_{s'} dM_{s s'} k_{s'} E_{s s'} + sum_t dM_ts k_t E_ts   (M, both sides)
       + beta_s dX_s e^{b_s} + dKh_s e^{b_C - b_s}
  dv_s = beta_s dY_s,  dbeta_t = sum(dX_t Kt_t) + sum(dY_t V_t) + sum_s dA_ts M_ts
  db_t = q_t (P row side + Qt part) + k_t (M row side + X part)
         - k_t (P col side + M col side + Kh part);  db_C += sum_t k_t dKh_t e^{b_C - b_t}
         + e^{b_C} rowsum(S0 dS1);  dg = reverse cumsum of db within the block."""
import numpy as np


def kda_chunk_bwd(q, k, v, g, beta, S_in, dO, dS_out, C):
    """One head: q, k, g [T, dk]; v, dO [T, dv]; beta [T]; states [dk, dv].
    Returns dict dq, dk, dv, dg, dbeta, dS_in."""
    T, dk = q.shape
    blocks = [(c0, min(c0 + C, T)) for c0 in range(0, T, C)]
    # forward: states entering each block
    S = S_in.copy()
    states, fw = [], []
    for c0, c1 in blocks:
        Q, K, V, G, Bt = q[c0:c1], k[c0:c1], v[c0:c1], g[c0:c1], beta[c0:c1]
        n = c1 - c0
        b = np.cumsum(G, 0)
        E = np.exp(b[:, None, :] - b[None, :, :])
        lo, lo1 = np.tril(np.ones((n, n)), -1), np.tril(np.ones((n, n)))
        M = np.einsum("td,sd,tsd->ts", K, K, E) * lo
        P = np.einsum("td,sd,tsd->ts", Q, K, E) * lo1
        Tm = np.linalg.inv(np.eye(n) + Bt[:, None] * M)
        Kt = K * np.exp(b)
        X, Y = Bt[:, None] * Kt, Bt[:, None] * V
        W, Ut = Tm @ X, Tm @ Y
        U = Ut - W @ S
        Kh = K * np.exp(b[-1] - b)
        states.append(S.copy())
        fw.append(dict(b=b, E=E, M=M, P=P, Tm=Tm, Kt=Kt, X=X, Y=Y, W=W, U=U, Kh=Kh))
        S = np.exp(b[-1])[:, None] * S + Kh.T @ U
    out = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v), dg=np.zeros_like(g),
               dbeta=np.zeros_like(beta))
    dS = dS_out.copy()
    for (c0, c1), S0, f in reversed(list(zip(blocks, states, fw))):
        Q, K, V, Bt, dOb = q[c0:c1], k[c0:c1], v[c0:c1], beta[c0:c1], dO[c0:c1]
        b, E, M, P, Tm, Kt, X, Y, W, U, Kh = (f[x] for x in ("b", "E", "M", "P", "Tm", "Kt", "X", "Y", "W", "U", "Kh"))
        n = c1 - c0
        lo, lo1 = np.tril(np.ones((n, n)), -1), np.tril(np.ones((n, n)))
        dU = P.T @ dOb + Kh @ dS
        dQt = dOb @ S0.T
        dP = (dOb @ U.T) * lo1
        dKh = U @ dS.T
        dW = -dU @ S0.T
        dT = dW @ X.T + dU @ Y.T
        dX, dY = Tm.T @ dW, Tm.T @ dU
        dA = -(Tm.T @ dT @ Tm.T) * lo
        dM = Bt[:, None] * dA
        a_row = np.einsum("ts,sd,tsd->td", dP, K, E)      # P, row side (-> dq_t)
        c_col = np.einsum("ts,td,tsd->sd", dP, Q, E)      # P, column side (-> dk_s)
        e_row = np.einsum("ts,sd,tsd->td", dM, K, E)      # M, row side (-> dk_t)
        f_col = np.einsum("ts,td,tsd->sd", dM, K, E)      # M, column side (-> dk_s)
        dq_qt = dQt * np.exp(b)
        dk_x = Bt[:, None] * dX * np.exp(b)
        dk_kh = dKh * np.exp(b[-1] - b)
        out["dq"][c0:c1] = dq_qt + a_row
        out["dk"][c0:c1] = c_col + e_row + f_col + dk_x + dk_kh
        out["dv"][c0:c1] = Bt[:, None] * dY
        out["dbeta"][c0:c1] = np.sum(dX * Kt, 1) + np.sum(dY * V, 1) + np.sum(dA * M, 1)
        db = Q * (dq_qt + a_row) + K * (e_row + dk_x) - K * (c_col + f_col + dk_kh)
        db[-1] += np.sum(K * dk_kh, 0) + np.exp(b[-1]) * np.sum(S0 * dS, 1)
        out["dg"][c0:c1] = np.flip(np.cumsum(np.flip(db, 0), 0), 0)
        dS = (Q * np.exp(b)).T @ dOb + np.exp(b[-1])[:, None] * dS - W.T @ dU
    out["dS_in"] = dS
    return out
