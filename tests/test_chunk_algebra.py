"""The block (64-token) algebra the kernels implement reproduces the fp64
oracle's per-token recurrence, forward and backward, including across
several blocks with a boundary state (design check at fp64)."""
import numpy as np
import pytest

from chunked_linear_recurrence_chunk_amd import inputs
from oracle import oracle
from tests import chunk_algebra as ca


@pytest.mark.parametrize("C", [8, 64])
def test_gdn_block_algebra_matches_oracle(C):
    x = inputs.make_gdn(1, 4 * C, 2, 16, 8, "fp32", seed=5, slow_decay=True)
    x = {k: v.astype(np.float64) for k, v in x.items()}
    o_ref, S_ref = oracle.gdn_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"])
    r = oracle.gdn_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"], x["dO"], x["dS_out"])
    for h in range(2):
        o, S, gr = ca.gdn_chunked_fwd_bwd(x["q"][0, :, h], x["k"][0, :, h], x["v"][0, :, h],
                                          x["g"][0, :, h], x["beta"][0, :, h], x["S_in"][0, h],
                                          x["dO"][0, :, h], x["dS_out"][0, h], C=C)
        np.testing.assert_allclose(o, o_ref[0, :, h], rtol=1e-10, atol=1e-11)
        np.testing.assert_allclose(S, S_ref[0, h], rtol=1e-10, atol=1e-11)
        for key in ("dq", "dk", "dv", "dg", "dbeta"):
            np.testing.assert_allclose(gr[key], r[key][0, :, h], rtol=1e-9, atol=1e-10, err_msg=key)
        np.testing.assert_allclose(gr["dS_in"], r["dS_in"][0, h], rtol=1e-9, atol=1e-10)


@pytest.mark.parametrize("C", [16, 64])
def test_gla_block_algebra_matches_oracle(C):
    x = inputs.make_gla(1, 3 * C, 2, 8, 12, "fp32", seed=6)
    x = {k: v.astype(np.float64) for k, v in x.items()}
    o_ref, S_ref = oracle.gla_fwd(x["q"], x["k"], x["v"], x["g"], x["S_in"])
    r = oracle.gla_bwd(x["q"], x["k"], x["v"], x["g"], x["S_in"], x["dO"], x["dS_out"])
    for h in range(2):
        o, S, gr = ca.gla_chunked_fwd_bwd(x["q"][0, :, h], x["k"][0, :, h], x["v"][0, :, h],
                                          x["g"][0, :, h], x["S_in"][0, h], x["dO"][0, :, h],
                                          x["dS_out"][0, h], C=C)
        np.testing.assert_allclose(o, o_ref[0, :, h], rtol=1e-10, atol=1e-10)
        np.testing.assert_allclose(S, S_ref[0, h], rtol=1e-10, atol=1e-10)
        for key in ("dq", "dk", "dv", "dg"):
            np.testing.assert_allclose(gr[key], r[key][0, :, h], rtol=1e-9, atol=1e-9, err_msg=key)
        np.testing.assert_allclose(gr["dS_in"], r["dS_in"][0, h], rtol=1e-9, atol=1e-9)
