"""The allocation-free Gated DeltaNet forward (gdn_fwd_noalloc, through the C
ABI) against the workspace entry point gdn_fwd: the same kernels on the same
inputs, so the outputs must be equal bit for bit.  Two calls in a row share
the library's static scratch, the second with a smaller input (the first
call's leftovers must not leak into it); one case is also checked against the
fp64 oracle at the stated tolerances."""
import numpy as np
import pytest

from tests.conftest import gpu_available
from tests.gpu_util import rel_err, to_dev, to_np, tol

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _dev(x, dtype):
    return [to_dev(x[key], dtype) for key in ("q", "k", "v", "g", "beta")], to_dev(x["S_in"], "fp32")


def _both(x, dtype):
    import torch
    from chunked_linear_recurrence_chunk_amd import ops
    t, S_in = _dev(x, dtype)
    o_ref, S_ref = ops.gdn_fwd(*t, S_in)
    o, S = ops.gdn_fwd_noalloc(*t, S_in)
    torch.cuda.synchronize()
    return (o, S), (o_ref, S_ref)


@pytest.mark.parametrize("cases", [
    # (B, T, H, d, dtype, seed): the first call near the scratch limit, the second smaller
    [(1, 2240, 16, 128, "bf16", 401), (2, 200, 3, 64, "bf16", 402)],
    [(1, 1024, 4, 128, "bf16", 403), (1, 256, 1, 32, "fp32", 404)],
])
def test_noalloc_forward_equals_workspace_forward(cases):
    import torch
    from chunked_linear_recurrence_chunk_amd import inputs
    for (B, T, H, d, dtype, seed) in cases:
        print(f"[noalloc] case {(B, T, H, d, dtype, seed)}", flush=True)
        x = inputs.make_gdn(B, T, H, d, d, dtype, seed)
        (o, S), (o_ref, S_ref) = _both(x, dtype)
        assert torch.equal(o, o_ref)
        assert torch.equal(S, S_ref)


def test_noalloc_forward_matches_oracle():
    from chunked_linear_recurrence_chunk_amd import inputs
    from oracle import oracle
    x = inputs.make_gdn(1, 320, 2, 128, 128, "bf16", 405)
    (o, S), _ = _both(x, "bf16")
    o_ref, S_ref = oracle.gdn_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"])
    assert rel_err(to_np(o), o_ref) < tol("bf16", "o")
    assert rel_err(to_np(S), S_ref) < tol("bf16", "S_out")


def test_noalloc_rejects_a_shape_beyond_the_scratch():
    from chunked_linear_recurrence_chunk_amd import inputs, ops
    x = inputs.make_gdn(1, 2304, 16, 128, 128, "bf16", 406)
    t, S_in = _dev(x, "bf16")
    with pytest.raises(ops.ClrError) as e:
        ops.gdn_fwd_noalloc(*t, S_in)
    assert e.value.status == ops.CLR_ESCRATCH
