"""GPU parity of the Gated DeltaNet path against the fp64 oracle, through the
C ABI (include/clr.h) via the ctypes binding."""
import numpy as np
import pytest

from tests.conftest import gpu_available
from tests.gpu_util import rel_err, to_dev, to_np, tol

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _ops():
    from chunked_linear_recurrence_chunk_amd import ops
    return ops


def test_probe_mma_layout():
    import torch
    ops = _ops()
    rng = np.random.default_rng(0)
    A = rng.standard_normal((16, 32)).astype(np.float32)
    Bt = rng.standard_normal((16, 32)).astype(np.float32)
    for dt in ("fp32", "bf16"):
        from chunked_linear_recurrence_chunk_amd import inputs
        a = inputs.bf16_round(A) if dt == "bf16" else A
        b = inputs.bf16_round(Bt) if dt == "bf16" else Bt
        C = to_np(ops.probe_mma(to_dev(a, dt), to_dev(b, dt)))
        ref = a.astype(np.float64) @ b.astype(np.float64).T
        assert rel_err(C[:16], ref) < 1e-5, dt
        assert rel_err(C[16:], ref) < 1e-5, dt
    torch.cuda.synchronize()


def _run_fwd(x, dtype, with_state=True):
    ops = _ops()
    d = {k: to_dev(x[k], dtype) for k in ("q", "k", "v", "g", "beta")}
    S_in = to_dev(x["S_in"], "fp32") if with_state else None
    o, S_out = ops.gdn_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S_in)
    return to_np(o), to_np(S_out)


CASES = [
    # (B, T, H, dk, dv, dtype, seed)
    (1, 256, 1, 32, 32, "fp32", 1),
    (2, 200, 3, 32, 32, "fp32", 2),     # ragged tail
    (1, 192, 2, 64, 64, "fp32", 3),
    (1, 256, 2, 128, 128, "fp32", 4),
    (1, 512, 2, 128, 128, "bf16", 5),
    (2, 320, 2, 64, 64, "bf16", 6),
    (1, 100, 2, 128, 128, "bf16", 7),   # ragged, < 2 blocks
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}T{c[1]}H{c[2]}d{c[3]}-{c[5]}" for c in CASES])
def test_gdn_fwd_matches_oracle(case):
    from chunked_linear_recurrence_chunk_amd import inputs
    from oracle import oracle
    B, T, H, dk, dv, dtype, seed = case
    print(f"[gdn fwd] case {case}", flush=True)
    x = inputs.make_gdn(B, T, H, dk, dv, dtype, seed)
    o, S = _run_fwd(x, dtype)
    o_ref, S_ref = oracle.gdn_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"])
    assert rel_err(o, o_ref) < tol(dtype, "o"), rel_err(o, o_ref)
    assert rel_err(S, S_ref) < tol(dtype, "S_out"), rel_err(S, S_ref)


def test_gdn_fwd_slow_decay_bf16():
    from chunked_linear_recurrence_chunk_amd import inputs
    from oracle import oracle
    x = inputs.make_gdn(1, 1024, 2, 128, 128, "bf16", 11, slow_decay=True)
    o, S = _run_fwd(x, "bf16")
    o_ref, S_ref = oracle.gdn_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"])
    print("slow decay errors", rel_err(o, o_ref), rel_err(S, S_ref))
    assert rel_err(o, o_ref) < tol("bf16", "o")
    assert rel_err(S, S_ref) < tol("bf16", "S_out")


SPLIT_CASES = [
    # (B, T, H, dk, dv, dtype, seed, split per mille)
    (1, 1024, 2, 128, 128, "bf16", 21, 500),   # 16 blocks: the smallest split
    (2, 1500, 3, 64, 64, "bf16", 22, 500),     # ragged last block in part 2
    (1, 2048, 16, 128, 128, "bf16", 23, 250),
    (1, 2048, 16, 128, 128, "bf16", 23, 750),
    (1, 1100, 2, 32, 32, "fp32", 24, 500),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[f"B{c[0]}T{c[1]}H{c[2]}d{c[3]}-{c[5]}-s{c[7]}" for c in SPLIT_CASES])
def test_gdn_fwd_split_is_bit_identical(case):
    """The split-and-overlap forward gives the unsplit forward's bits."""
    import torch
    from chunked_linear_recurrence_chunk_amd import inputs
    ops = _ops()
    B, T, H, dk, dv, dtype, seed, pm = case
    print(f"[gdn fwd split] case {case}", flush=True)
    x = inputs.make_gdn(B, T, H, dk, dv, dtype, seed)
    old = ops.get_fwd_split()
    try:
        ops.set_fwd_split(0)
        o0, S0 = _run_fwd(x, dtype)
        ops.set_fwd_split(pm)
        o1, S1 = _run_fwd(x, dtype)
        o2, S2 = _run_fwd(x, dtype)  # again: the auxiliary stream is reused
    finally:
        ops.set_fwd_split(old)
    torch.cuda.synchronize()
    assert np.array_equal(o0, o1) and np.array_equal(S0, S1)
    assert np.array_equal(o0, o2) and np.array_equal(S0, S2)


BV_CASES = [
    # (B, T, H, dk, dv, dtype, seed)
    (1, 2048, 16, 128, 128, "bf16", 26),
    (2, 1500, 3, 64, 64, "bf16", 27),     # ragged last block, H not a multiple of 8
    (1, 200, 2, 32, 32, "fp32", 28),
]


@pytest.mark.parametrize("case", BV_CASES, ids=[f"B{c[0]}T{c[1]}H{c[2]}d{c[3]}-{c[5]}" for c in BV_CASES])
def test_gdn_fwd_scan_bv32_is_bit_identical(case):
    """The forward scan with 32 value columns per work-group (two slices
    sharing the W / K^T stream) gives the 16-column scan's bits, alone and
    under the split-and-overlap schedule."""
    import torch
    from chunked_linear_recurrence_chunk_amd import inputs
    ops = _ops()
    B, T, H, dk, dv, dtype, seed = case
    print(f"[gdn fwd bv32] case {case}", flush=True)
    x = inputs.make_gdn(B, T, H, dk, dv, dtype, seed)
    old_bv, old_split = ops.get_scan_bv(), ops.get_fwd_split()
    try:
        ops.set_fwd_split(0)
        ops.set_scan_bv(16)
        o0, S0 = _run_fwd(x, dtype)
        ops.set_scan_bv(32)
        o1, S1 = _run_fwd(x, dtype)
        ops.set_fwd_split(500)
        o2, S2 = _run_fwd(x, dtype)
    finally:
        ops.set_scan_bv(old_bv)
        ops.set_fwd_split(old_split)
    torch.cuda.synchronize()
    assert np.array_equal(o0, o1) and np.array_equal(S0, S1)
    assert np.array_equal(o0, o2) and np.array_equal(S0, S2)


def test_gdn_fwd_split_matches_oracle():
    from chunked_linear_recurrence_chunk_amd import inputs
    from oracle import oracle
    ops = _ops()
    x = inputs.make_gdn(2, 1500, 3, 64, 64, "bf16", 25)
    old = ops.get_fwd_split()
    try:
        ops.set_fwd_split(400)
        o, S = _run_fwd(x, "bf16")
    finally:
        ops.set_fwd_split(old)
    o_ref, S_ref = oracle.gdn_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"])
    assert rel_err(o, o_ref) < tol("bf16", "o"), rel_err(o, o_ref)
    assert rel_err(S, S_ref) < tol("bf16", "S_out"), rel_err(S, S_ref)


def _run_bwd(x, dtype, with_dS=True):
    ops = _ops()
    d = {k: to_dev(x[k], dtype) for k in ("q", "k", "v", "g", "beta", "dO")}
    S_in = to_dev(x["S_in"], "fp32")
    dS_out = to_dev(x["dS_out"], "fp32") if with_dS else None
    r = ops.gdn_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S_in, d["dO"], dS_out)
    return {k: to_np(v) for k, v in r.items()}


BWD_CASES = [
    (1, 256, 1, 32, 32, "fp32", 21),
    (2, 200, 3, 32, 32, "fp32", 22),    # ragged tail
    (1, 192, 2, 64, 64, "fp32", 27),
    (1, 512, 2, 128, 128, "bf16", 23),
    (2, 320, 2, 64, 64, "bf16", 24),
    (1, 100, 2, 128, 128, "bf16", 25),  # ragged, < 2 blocks
    (1, 256, 3, 32, 32, "bf16", 26),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=[f"B{c[0]}T{c[1]}H{c[2]}d{c[3]}-{c[5]}" for c in BWD_CASES])
def test_gdn_bwd_matches_oracle(case):
    from chunked_linear_recurrence_chunk_amd import inputs
    from oracle import oracle
    B, T, H, dk, dv, dtype, seed = case
    print(f"[gdn bwd] case {case}", flush=True)
    x = inputs.make_gdn(B, T, H, dk, dv, dtype, seed)
    got = _run_bwd(x, dtype)
    ref = oracle.gdn_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"], x["dO"], x["dS_out"])
    errs = {k: rel_err(got[k], ref[k]) for k in ref}
    print("  errors", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for k, e in errs.items():
        assert e < tol(dtype, k), (k, e)


def test_gdn_bwd_slow_decay_and_null_dS_out():
    from chunked_linear_recurrence_chunk_amd import inputs
    from oracle import oracle
    x = inputs.make_gdn(1, 1024, 2, 128, 128, "bf16", 27, slow_decay=True)
    got = _run_bwd(x, "bf16", with_dS=False)
    ref = oracle.gdn_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"], x["dO"], None)
    errs = {k: rel_err(got[k], ref[k]) for k in ref}
    print("  errors", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for k, e in errs.items():
        assert e < tol("bf16", k), (k, e)
