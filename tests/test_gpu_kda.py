"""GPU parity of the KDA forward and backward (per-key-channel decay with
the delta rule, kda_fwd / kda_bwd) against the fp64 oracle, through the C
ABI, and sequence-chunk exactness (the full workload: test_gpu_fullsize)."""
import pytest

from tests.conftest import gpu_available
from tests.gpu_util import rel_err, to_dev, to_np, tol

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

CASES = [
    # (B, T, H, dk, dv, dtype, seed, gate_scale)
    (1, 256, 1, 32, 32, "fp32", 71, 1 / 16),
    (2, 200, 2, 32, 32, "fp32", 72, 1.0),        # ragged tail, strong gates
    (1, 192, 2, 64, 64, "fp32", 73, 1 / 16),
    (1, 512, 2, 128, 128, "bf16", 74, 1 / 16),
    (2, 320, 2, 64, 64, "bf16", 75, 1 / 16),
    (1, 100, 3, 128, 128, "bf16", 76, 1 / 16),   # ragged, < 2 blocks
    (1, 256, 2, 128, 128, "bf16", 77, 1.0),      # strong gates
]


def _ids(c):
    return f"B{c[0]}T{c[1]}H{c[2]}d{c[3]}-{c[5]}-g{c[7]:.3g}"


def _dev(x, dtype):
    return {k: to_dev(x[k], dtype) for k in ("q", "k", "v", "g", "beta")}, to_dev(x["S_in"], "fp32")


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_kda_fwd_matches_oracle(case):
    import torch
    from chunked_linear_recurrence_chunk_amd import inputs, ops
    from oracle import oracle
    B, T, H, dk, dv, dtype, seed, gs = case
    print(f"[kda] case {case}", flush=True)
    x = inputs.make_kda(B, T, H, dk, dv, dtype, seed, gate_scale=gs)
    d, S_in = _dev(x, dtype)
    o, S = ops.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S_in)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.kda_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"])
    eo, es = rel_err(to_np(o), o_ref), rel_err(to_np(S), S_ref)
    print(f"  errors o {eo:.2e} S_out {es:.2e}", flush=True)
    assert eo < tol(dtype, "o") and es < tol(dtype, "S_out"), (eo, es)


def test_kda_chunked_equals_unchunked():
    import torch
    from chunked_linear_recurrence_chunk_amd import inputs, stateflow
    x = inputs.make_kda(1, 1024, 2, 128, 128, "bf16", 78)
    d, S_in = _dev(x, "bf16")
    dO, dS_out = to_dev(x["dO"], "bf16"), to_dev(x["dS_out"], "fp32")
    res = []
    for N in (1, 4):
        drv = stateflow.KdaChunked(d["q"], d["k"], d["v"], d["g"], d["beta"], N)
        o, S = drv.forward(S_in)
        gr = drv.backward(dO, dS_out)
        torch.cuda.synchronize()
        res.append(dict(o=o, S_out=S, **gr))
    for key in res[0]:
        assert torch.equal(res[0][key], res[1][key]), key


BWD_CASES = [
    (1, 256, 1, 32, 32, "fp32", 81, 1 / 16),
    (2, 200, 2, 32, 32, "fp32", 82, 1.0),        # ragged tail, strong gates
    (1, 200, 2, 64, 64, "fp32", 88, 1 / 16),     # ragged tail
    (1, 192, 2, 32, 32, "bf16", 83, 1 / 16),
    (2, 320, 2, 64, 64, "bf16", 84, 1 / 16),
    (1, 512, 2, 128, 128, "bf16", 85, 1 / 16),
    (1, 100, 3, 128, 128, "bf16", 86, 1 / 16),   # ragged, < 2 blocks
    (1, 256, 2, 128, 128, "bf16", 87, 1.0),      # strong gates
]


@pytest.mark.parametrize("case", BWD_CASES, ids=[_ids(c) for c in BWD_CASES])
def test_kda_bwd_matches_oracle(case):
    import torch
    from chunked_linear_recurrence_chunk_amd import inputs, ops
    from oracle import oracle
    B, T, H, dk, dv, dtype, seed, gs = case
    print(f"[kda bwd] case {case}", flush=True)
    x = inputs.make_kda(B, T, H, dk, dv, dtype, seed, gate_scale=gs)
    d, S_in = _dev(x, dtype)
    dO, dS_out = to_dev(x["dO"], dtype), to_dev(x["dS_out"], "fp32")
    gr = ops.kda_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S_in, dO, dS_out)
    torch.cuda.synchronize()
    ref = oracle.kda_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"], x["dO"], x["dS_out"])
    errs = {k: rel_err(to_np(gr[k]), ref[k]) for k in ref}
    print("  errors", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for k, e in errs.items():
        assert e < tol(dtype, k), (k, e)
