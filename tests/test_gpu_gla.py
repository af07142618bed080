"""GPU parity of the GLA (per-channel gate) path against the fp64 oracle,
through the C ABI, plus sequence-chunk exactness."""
import numpy as np
import pytest

from tests.conftest import gpu_available
from tests.gpu_util import rel_err, to_dev, to_np, tol

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

CASES = [
    # (B, T, H, dk, dv, dtype, seed, gate_scale)
    (1, 256, 1, 32, 32, "fp32", 41, 1 / 16),
    (2, 200, 2, 32, 32, "fp32", 42, 1.0),        # ragged tail, strong gates
    (1, 192, 2, 64, 64, "fp32", 47, 1 / 16),
    (2, 256, 2, 128, 256, "bf16", 43, 1 / 16),   # the GLA workload's head shape
    (1, 320, 2, 64, 64, "bf16", 44, 1 / 16),
    (1, 100, 3, 128, 128, "bf16", 45, 1 / 16),  # ragged, < 2 blocks
    (1, 512, 2, 128, 256, "bf16", 46, 1.0),      # strong gates (logsigmoid(N(0,1)) per token)
]


def _ids(c):
    return f"B{c[0]}T{c[1]}H{c[2]}dk{c[3]}dv{c[4]}-{c[5]}-g{c[7]:.3g}"


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_gla_fwd_bwd_matches_oracle(case):
    import torch
    from chunked_linear_recurrence_chunk_amd import inputs, ops
    from oracle import oracle
    B, T, H, dk, dv, dtype, seed, gs = case
    print(f"[gla] case {case}", flush=True)
    x = inputs.make_gla(B, T, H, dk, dv, dtype, seed, gate_scale=gs)
    d = {k: to_dev(x[k], dtype) for k in ("q", "k", "v", "g", "dO")}
    S_in = to_dev(x["S_in"], "fp32")
    dS_out = to_dev(x["dS_out"], "fp32")
    o, S = ops.gla_fwd(d["q"], d["k"], d["v"], d["g"], S_in)
    gr = ops.gla_bwd(d["q"], d["k"], d["v"], d["g"], S_in, d["dO"], dS_out)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.gla_fwd(x["q"], x["k"], x["v"], x["g"], x["S_in"])
    ref = oracle.gla_bwd(x["q"], x["k"], x["v"], x["g"], x["S_in"], x["dO"], x["dS_out"])
    ref.update(o=o_ref, S_out=S_ref)
    got = dict(o=o, S_out=S, **gr)
    errs = {k: rel_err(to_np(got[k]), ref[k]) for k in ref}
    print("  errors", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for k, e in errs.items():
        assert e < tol(dtype, k), (k, e)


def test_gla_chunked_equals_unchunked():
    import torch
    from chunked_linear_recurrence_chunk_amd import inputs, stateflow
    x = inputs.make_gla(1, 1024, 2, 128, 256, "bf16", 47)
    d = {k: to_dev(x[k], "bf16") for k in ("q", "k", "v", "g", "dO")}
    S_in = to_dev(x["S_in"], "fp32")
    dS_out = to_dev(x["dS_out"], "fp32")
    res = []
    for N in (1, 4):
        drv = stateflow.GlaChunked(d["q"], d["k"], d["v"], d["g"], N)
        o, S = drv.forward(S_in)
        gr = drv.backward(d["dO"], dS_out)
        torch.cuda.synchronize()
        res.append(dict(o=o, S_out=S, **gr))
    for key in res[0]:
        assert torch.equal(res[0][key], res[1][key]), key
