"""The diagonal tiles' decay bound of the per-channel and scalar-gate members
(GLA, KDA, Mamba-2).  Gates of -9 to -9.75 on every token for a quarter of the
key channels (the even heads for the scalar gate) stay within the bound: the
results match the fp64 oracle at the usual tolerances and clr_range_status
reports CLR_OK.  Gates of -11 to -12 leave it: the forward and backward report
CLR_ERANGE and every output stays finite."""
import numpy as np
import pytest

from tests.conftest import gpu_available
from tests.gpu_util import rel_err, to_dev, to_np, tol

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

CASES = [
    # (kind, B, T, H, dk, dv, dtype, seed)
    ("gla", 1, 200, 2, 32, 32, "fp32", 501),
    ("gla", 1, 256, 2, 128, 256, "bf16", 502),
    ("mamba2", 1, 200, 2, 32, 32, "fp32", 503),
    ("mamba2", 1, 256, 2, 128, 256, "bf16", 504),
    ("kda", 1, 200, 2, 32, 32, "fp32", 505),
    ("kda", 1, 256, 2, 128, 128, "bf16", 506),
]
OPS = {"gla": (2, 3), "mamba2": (4, 5), "kda": (6, 7)}


def _ids(c):
    return f"{c[0]}-T{c[2]}H{c[3]}dk{c[4]}dv{c[5]}-{c[6]}"


def _run(kind, x, dtype):
    import torch
    from chunked_linear_recurrence_chunk_amd import ops
    keys = ("q", "k", "v", "g", "beta", "dO") if kind == "kda" else ("q", "k", "v", "g", "dO")
    d = {key: to_dev(x[key], dtype) for key in keys}
    S_in, dS_out = to_dev(x["S_in"], "fp32"), to_dev(x["dS_out"], "fp32")
    shape = ops.make_shape(d["q"], d["v"])
    op_f, op_b = OPS[kind]
    ws_f = torch.empty(max(ops.workspace_bytes(shape, op_f), 256), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(max(ops.workspace_bytes(shape, op_b), 256), dtype=torch.uint8, device="cuda")
    if kind == "kda":
        o, S = ops.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S_in, ws=ws_f)
        st_f = ops.range_status(shape, op_f, ws_f)
        gr = ops.kda_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S_in, d["dO"], dS_out, ws=ws_b)
    else:
        fwd, bwd = (ops.gla_fwd, ops.gla_bwd) if kind == "gla" else (ops.mamba2_fwd, ops.mamba2_bwd)
        o, S = fwd(d["q"], d["k"], d["v"], d["g"], S_in, ws=ws_f)
        st_f = ops.range_status(shape, op_f, ws_f)
        gr = bwd(d["q"], d["k"], d["v"], d["g"], S_in, d["dO"], dS_out, ws=ws_b)
    st_b = ops.range_status(shape, op_b, ws_b)
    torch.cuda.synchronize()
    return dict(o=o, S_out=S, **gr), st_f, st_b


def _oracle(kind, x):
    from oracle import oracle
    if kind == "kda":
        args = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"])
        o, S = oracle.kda_fwd(*args)
        ref = oracle.kda_bwd(*args, x["dO"], x["dS_out"])
    else:
        fwd, bwd = (oracle.gla_fwd, oracle.gla_bwd) if kind == "gla" else (oracle.mamba2_fwd, oracle.mamba2_bwd)
        args = (x["q"], x["k"], x["v"], x["g"], x["S_in"])
        o, S = fwd(*args)
        ref = bwd(*args, x["dO"], x["dS_out"])
    ref.update(o=o, S_out=S)
    return ref


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_gates_within_the_bound_match_the_oracle(case):
    from chunked_linear_recurrence_chunk_amd import inputs, ops
    kind, B, T, H, dk, dv, dtype, seed = case
    print(f"[range] within bound {case}", flush=True)
    x = inputs.make_strong_decay(kind, B, T, H, dk, dv, dtype, seed, lo=9.0, hi=9.75)
    got, st_f, st_b = _run(kind, x, dtype)
    assert st_f == ops.CLR_OK and st_b == ops.CLR_OK, (st_f, st_b)
    ref = _oracle(kind, x)
    errs = {key: rel_err(to_np(got[key]), r) for key, r in ref.items()}
    print("  errors", {key: f"{e:.2e}" for key, e in errs.items()}, flush=True)
    bad = {key: e for key, e in errs.items() if not e < tol(dtype, key)}
    assert not bad, bad


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_gates_beyond_the_bound_are_reported(case):
    from chunked_linear_recurrence_chunk_amd import inputs, ops
    kind, B, T, H, dk, dv, dtype, seed = case
    print(f"[range] beyond bound {case}", flush=True)
    x = inputs.make_strong_decay(kind, B, T, H, dk, dv, dtype, seed, lo=11.0, hi=12.0)
    got, st_f, st_b = _run(kind, x, dtype)
    assert st_f == ops.CLR_ERANGE and st_b == ops.CLR_ERANGE, (st_f, st_b)
    for key, t in got.items():
        assert np.isfinite(to_np(t)).all(), key
