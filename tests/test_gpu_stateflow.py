"""Sequence-chunk (StateFlow) exactness on the GPU: the N-chunk state-passed
run equals the unchunked run bit for bit (same kernels on the same 64-token
blocks, fp32 boundary states), and both match the fp64 oracle."""
import numpy as np
import pytest

from tests.conftest import gpu_available
from tests.gpu_util import rel_err, to_dev, to_np, tol

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _gdn_run(x, dtype, N):
    import torch
    from chunked_linear_recurrence_chunk_amd import stateflow
    d = {k: to_dev(x[k], dtype) for k in ("q", "k", "v", "g", "beta", "dO")}
    S_in = to_dev(x["S_in"], "fp32")
    dS_out = to_dev(x["dS_out"], "fp32")
    drv = stateflow.GdnChunked(d["q"], d["k"], d["v"], d["g"], d["beta"], N)
    o, S = drv.forward(S_in)
    gr = drv.backward(d["dO"], dS_out)
    torch.cuda.synchronize()
    return dict(o=o, S_out=S, **gr)


@pytest.mark.parametrize("case", [
    (1, 256, 1, 32, 32, "fp32", 4, 31),      # the fp32 d=32 workload as 4 chunks of 64
    (1, 2048, 4, 128, 128, "bf16", 4, 32),
    (1, 1536, 2, 64, 64, "bf16", 3, 33),
    (2, 512, 2, 32, 32, "fp32", 2, 34),      # B > 1: chunk slices are copies
])
def test_gdn_chunked_equals_unchunked_and_oracle(case):
    import torch
    from chunked_linear_recurrence_chunk_amd import inputs
    from oracle import oracle
    B, T, H, dk, dv, dtype, N, seed = case
    print(f"[stateflow gdn] case {case}", flush=True)
    x = inputs.make_gdn(B, T, H, dk, dv, dtype, seed)
    one = _gdn_run(x, dtype, 1)
    many = _gdn_run(x, dtype, N)
    for key in one:
        assert torch.equal(one[key], many[key]), key
    o_ref, S_ref = oracle.gdn_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"])
    ref = oracle.gdn_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"], x["dO"], x["dS_out"])
    ref.update(o=o_ref, S_out=S_ref)
    for key, r in ref.items():
        e = rel_err(to_np(many[key]), r)
        assert e < tol(dtype, key), (key, e)


def test_resume_from_host_copy_of_boundary_state():
    """Stopping after a chunk and resuming from a host copy of S_out gives the
    same result as the uninterrupted chain (the boundary state is the resume
    point)."""
    import torch
    from chunked_linear_recurrence_chunk_amd import inputs, ops
    x = inputs.make_gdn(1, 1024, 2, 128, 128, "bf16", 35)
    d = {k: to_dev(x[k], "bf16") for k in ("q", "k", "v", "g", "beta")}
    S_in = to_dev(x["S_in"], "fp32")
    o_full, S_full = ops.gdn_fwd(*(d[k] for k in ("q", "k", "v", "g", "beta")), S_in)
    h = [t[:, :512].contiguous() for t in (d["q"], d["k"], d["v"], d["g"], d["beta"])]
    t2 = [t[:, 512:].contiguous() for t in (d["q"], d["k"], d["v"], d["g"], d["beta"])]
    o1, S_mid = ops.gdn_fwd(*h, S_in)
    S_host = S_mid.cpu()
    o2, S_end = ops.gdn_fwd(*t2, S_host.cuda())
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([o1, o2], 1), o_full)
    assert torch.equal(S_end, S_full)
