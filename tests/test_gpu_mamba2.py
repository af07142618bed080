"""GPU parity of the scalar-gate (Mamba-2 member) path against the fp64
oracle, through the C ABI (mamba2_fwd / mamba2_bwd), plus sequence-chunk
exactness and agreement with the GLA path given the same gate broadcast over
the key channels."""
import numpy as np
import pytest

from tests.conftest import gpu_available
from tests.gpu_util import rel_err, to_dev, to_np, tol

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

CASES = [
    # (B, T, H, dk, dv, dtype, seed, gate_scale)
    (1, 256, 1, 32, 32, "fp32", 61, 1 / 16),
    (2, 200, 2, 32, 32, "fp32", 62, 1.0),        # ragged tail, strong gates
    (1, 192, 2, 64, 64, "fp32", 67, 1 / 16),
    (2, 256, 2, 128, 256, "bf16", 63, 1 / 16),   # the measured workload's head shape
    (1, 320, 2, 64, 64, "bf16", 64, 1 / 16),
    (1, 100, 3, 128, 128, "bf16", 65, 1 / 16),   # ragged, < 2 blocks
    (1, 512, 2, 128, 256, "bf16", 66, 1.0),      # strong gates
]


def _ids(c):
    return f"B{c[0]}T{c[1]}H{c[2]}dk{c[3]}dv{c[4]}-{c[5]}-g{c[7]:.3g}"


def _dev(x, dtype):
    d = {k: to_dev(x[k], dtype) for k in ("q", "k", "v", "g", "dO")}
    return d, to_dev(x["S_in"], "fp32"), to_dev(x["dS_out"], "fp32")


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_mamba2_fwd_bwd_matches_oracle(case):
    import torch
    from chunked_linear_recurrence_chunk_amd import inputs, ops
    from oracle import oracle
    B, T, H, dk, dv, dtype, seed, gs = case
    print(f"[mamba2] case {case}", flush=True)
    x = inputs.make_mamba2(B, T, H, dk, dv, dtype, seed, gate_scale=gs)
    d, S_in, dS_out = _dev(x, dtype)
    o, S = ops.mamba2_fwd(d["q"], d["k"], d["v"], d["g"], S_in)
    gr = ops.mamba2_bwd(d["q"], d["k"], d["v"], d["g"], S_in, d["dO"], dS_out)
    torch.cuda.synchronize()
    assert gr["dg"].shape == (B, T, H)
    o_ref, S_ref = oracle.mamba2_fwd(x["q"], x["k"], x["v"], x["g"], x["S_in"])
    ref = oracle.mamba2_bwd(x["q"], x["k"], x["v"], x["g"], x["S_in"], x["dO"], x["dS_out"])
    ref.update(o=o_ref, S_out=S_ref)
    got = dict(o=o, S_out=S, **gr)
    errs = {k: rel_err(to_np(got[k]), ref[k]) for k in ref}
    print("  errors", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for k, e in errs.items():
        assert e < tol(dtype, k), (k, e)


def test_mamba2_chunked_equals_unchunked():
    import torch
    from chunked_linear_recurrence_chunk_amd import inputs, stateflow
    x = inputs.make_mamba2(1, 1024, 2, 128, 256, "bf16", 67)
    d, S_in, dS_out = _dev(x, "bf16")
    res = []
    for N in (1, 4):
        drv = stateflow.Mamba2Chunked(d["q"], d["k"], d["v"], d["g"], N)
        o, S = drv.forward(S_in)
        gr = drv.backward(d["dO"], dS_out)
        torch.cuda.synchronize()
        res.append(dict(o=o, S_out=S, **gr))
    for key in res[0]:
        assert torch.equal(res[0][key], res[1][key]), key


def test_mamba2_is_gla_with_a_broadcast_gate():
    """Same bits as the GLA path fed the broadcast gate, except dg, which is
    the channel sum (compared within the bf16 tolerance: the GLA dg is rounded
    per channel before the sum)."""
    import torch
    from chunked_linear_recurrence_chunk_amd import inputs, ops
    x = inputs.make_mamba2(2, 300, 2, 128, 256, "bf16", 68)
    d, S_in, dS_out = _dev(x, "bf16")
    gb = d["g"][..., None].expand(*d["g"].shape, 128).contiguous()
    o1, S1 = ops.mamba2_fwd(d["q"], d["k"], d["v"], d["g"], S_in)
    r1 = ops.mamba2_bwd(d["q"], d["k"], d["v"], d["g"], S_in, d["dO"], dS_out)
    o2, S2 = ops.gla_fwd(d["q"], d["k"], d["v"], gb, S_in)
    r2 = ops.gla_bwd(d["q"], d["k"], d["v"], gb, S_in, d["dO"], dS_out)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    for key in ("dq", "dk", "dv", "dS_in"):
        assert torch.equal(r1[key], r2[key]), key
    assert rel_err(to_np(r1["dg"]), to_np(r2["dg"]).sum(-1)) < 2e-2
