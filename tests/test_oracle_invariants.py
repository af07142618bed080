"""Pins the oracle with identities that hold for the exact layer at any size
(derivable from the update rule of the StateFlow paper, Sec. 2.1), and with
the sequence-chunk exactness of Sec. 3.1 (Eqs. 3-7: chaining S_out -> S_in
forward and dS_in -> dS_out backward reproduces the unchunked run):

  (i)   q_t . dq_t = o_t . do_t                      (o_t linear in q_t)
  (ii)  GDN: k_t.dk_t + v_t.dv_t = 2 beta_t dbeta_t  (k->ck, beta->beta/c^2, v->cv)
  (iii) GLA: k_t.dk_t = v_t.dv_t                     (k->ck, v->v/c)
  (iv)  sum v.dv + <S_in,dS_in> = sum o.do + <S_out,dS_out>   (joint linearity)
  (v)   GDN: dg_t = sum_{tau>=t}(o.do - v.dv) + <S_out,dS_out>
        GLA: dg_t[i] = sum_{tau>=t}(q[i]dq[i] - k[i]dk[i]) + rowsum(S_out*dS_out)[i]
  (vi)  GLA: sum_t k*dk - sum_t q*dq + rowsum(S_in*dS_in) = rowsum(S_out*dS_out)
"""
import numpy as np
import pytest

from chunked_linear_recurrence_chunk_amd import inputs
from oracle import oracle


def _gdn_case(seed=11, B=2, T=150, H=3, dk=8, dv=6, slow=True):
    x = inputs.make_gdn(B, T, H, dk, dv, "fp32", seed, slow_decay=slow)
    return {k: v.astype(np.float64) for k, v in x.items()}


def _gla_case(seed=12, B=2, T=150, H=2, dk=8, dv=6):
    x = inputs.make_gla(B, T, H, dk, dv, "fp32", seed)
    return {k: v.astype(np.float64) for k, v in x.items()}


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30)


def test_gdn_identities():
    x = _gdn_case()
    o, S_out = oracle.gdn_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"])
    r = oracle.gdn_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"], x["dO"], x["dS_out"])
    qdq = np.sum(x["q"] * r["dq"], -1)
    odo = np.sum(o * x["dO"], -1)
    assert _rel(qdq, odo) < 1e-12
    kdk = np.sum(x["k"] * r["dk"], -1)
    vdv = np.sum(x["v"] * r["dv"], -1)
    assert _rel(kdk + vdv, 2 * x["beta"] * r["dbeta"]) < 1e-11
    lhs = vdv.sum((1,)) + np.sum(x["S_in"] * r["dS_in"], (2, 3))
    rhs = odo.sum((1,)) + np.sum(S_out * x["dS_out"], (2, 3))
    assert _rel(lhs, rhs) < 1e-11
    tail = np.flip(np.cumsum(np.flip(odo - vdv, 1), 1), 1)
    dg_ref = tail + np.sum(S_out * x["dS_out"], (2, 3))[:, None, :]
    assert _rel(r["dg"], dg_ref) < 1e-10


def test_gla_identities():
    x = _gla_case()
    o, S_out = oracle.gla_fwd(x["q"], x["k"], x["v"], x["g"], x["S_in"])
    r = oracle.gla_bwd(x["q"], x["k"], x["v"], x["g"], x["S_in"], x["dO"], x["dS_out"])
    assert _rel(np.sum(x["q"] * r["dq"], -1), np.sum(o * x["dO"], -1)) < 1e-12
    assert _rel(np.sum(x["k"] * r["dk"], -1), np.sum(x["v"] * r["dv"], -1)) < 1e-11
    vdv = np.sum(x["v"] * r["dv"], -1).sum(1)
    odo = np.sum(o * x["dO"], -1).sum(1)
    lhs = vdv + np.sum(x["S_in"] * r["dS_in"], (2, 3))
    rhs = odo + np.sum(S_out * x["dS_out"], (2, 3))
    assert _rel(lhs, rhs) < 1e-11
    end = np.sum(S_out * x["dS_out"], 3)                      # [B,H,dk]
    term = x["q"] * r["dq"] - x["k"] * r["dk"]               # [B,T,H,dk]
    dg_ref = np.flip(np.cumsum(np.flip(term, 1), 1), 1) + end[:, None]
    assert _rel(r["dg"], dg_ref) < 1e-10
    lhs = (x["k"] * r["dk"]).sum(1) - (x["q"] * r["dq"]).sum(1) + np.sum(x["S_in"] * r["dS_in"], 3)
    assert _rel(lhs, end) < 1e-10


@pytest.mark.parametrize("N", [2, 3, 4, 8, 16])
def test_gdn_chunk_split_is_bit_exact(N):
    x = _gdn_case(seed=20 + N, B=1, T=192, H=2, dk=5, dv=4)
    o1, S1 = oracle.gdn_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"])
    r1 = oracle.gdn_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"], x["dO"], x["dS_out"])
    if 192 % N:
        pytest.skip("uneven split")
    oN, SN, rN = oracle.gdn_chunked(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"],
                                    x["dO"], x["dS_out"], N)
    assert np.array_equal(o1, oN) and np.array_equal(S1, SN)
    for key in r1:
        assert np.array_equal(r1[key], rN[key]), key


@pytest.mark.parametrize("N", [2, 4, 8, 16])
def test_gla_chunk_split_is_bit_exact(N):
    x = _gla_case(seed=40 + N, B=1, T=128, H=2, dk=4, dv=5)
    o1, S1 = oracle.gla_fwd(x["q"], x["k"], x["v"], x["g"], x["S_in"])
    r1 = oracle.gla_bwd(x["q"], x["k"], x["v"], x["g"], x["S_in"], x["dO"], x["dS_out"])
    oN, SN, rN = oracle.gla_chunked(x["q"], x["k"], x["v"], x["g"], x["S_in"], x["dO"], x["dS_out"], N)
    assert np.array_equal(o1, oN) and np.array_equal(S1, SN)
    for key in r1:
        assert np.array_equal(r1[key], rN[key]), key
