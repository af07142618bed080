"""GPU parity of the GLA and Mamba-2 pairs with saved activations
(gla_fwd_save / gla_bwd_saved, mamba2_fwd_save / mamba2_bwd_saved), through
the C ABI.

The forward that saves must return what the plain forward returns, bit for
bit.  The states it keeps are formed by the same scan arithmetic as the
backward's recompute, so the backward that reads them returns what gla_bwd /
mamba2_bwd return, bit for bit, and both match the fp64 oracle within the
tolerances.  Sequence chunking with saved activations reproduces the
unchunked run bit for bit."""
import pytest

from tests.conftest import gpu_available
from tests.gpu_util import rel_err, to_dev, to_np, tol

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

CASES = [
    # (member, B, T, H, dk, dv, dtype, seed)
    ("gla", 1, 256, 1, 32, 32, "fp32", 51),
    ("gla", 2, 200, 3, 32, 32, "fp32", 52),      # ragged tail
    ("gla", 1, 192, 2, 64, 64, "bf16", 53),
    ("gla", 2, 256, 2, 128, 256, "bf16", 54),    # the GLA workload's head shape
    ("gla", 1, 100, 2, 128, 128, "bf16", 55),    # ragged, < 2 blocks
    ("gla", 1, 1024, 8, 128, 256, "bf16", 56),
    ("mamba2", 1, 256, 1, 32, 32, "fp32", 57),
    ("mamba2", 2, 300, 2, 128, 256, "bf16", 58),  # ragged
    ("mamba2", 1, 1024, 8, 128, 256, "bf16", 59),
    ("gla", 1, 192, 2, 64, 64, "fp32", 63),
    ("mamba2", 2, 130, 2, 64, 64, "fp32", 64),   # ragged
]


def _make(member, B, T, H, dk, dv, dtype, seed):
    from chunked_linear_recurrence_chunk_amd import inputs
    if member == "gla":
        return inputs.make_gla(B, T, H, dk, dv, dtype, seed, gate_scale=1 / 16)
    return inputs.make_mamba2(B, T, H, dk, dv, dtype, seed)


def _dev(x, dtype):
    d = {k: to_dev(x[k], dtype) for k in ("q", "k", "v", "g", "dO")}
    return d, to_dev(x["S_in"], "fp32"), to_dev(x["dS_out"], "fp32")


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-B{c[1]}T{c[2]}H{c[3]}dk{c[4]}dv{c[5]}-{c[6]}" for c in CASES])
def test_saved_pair_equals_plain_pair_and_matches_oracle(case):
    import torch
    from chunked_linear_recurrence_chunk_amd import ops
    from oracle import oracle
    member, B, T, H, dk, dv, dtype, seed = case
    print(f"[{member} saved] case {case}", flush=True)
    x = _make(member, B, T, H, dk, dv, dtype, seed)
    d, S_in, dS = _dev(x, dtype)
    fwd, bwd = getattr(ops, f"{member}_fwd"), getattr(ops, f"{member}_bwd")
    fwd_s, bwd_s = getattr(ops, f"{member}_fwd_save"), getattr(ops, f"{member}_bwd_saved")
    args = (d["q"], d["k"], d["v"], d["g"])
    o0, S0 = fwd(*args, S_in)
    o1, S1, saved = fwd_s(*args, S_in)
    g0 = bwd(*args, S_in, d["dO"], dS)
    g1 = bwd_s(*args, None, d["dO"], dS, saved)  # S_in is not read by the saved backward
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(S0, S1)
    for key in g0:
        assert torch.equal(g0[key], g1[key]), key
    xo = (x["q"], x["k"], x["v"], x["g"], x["S_in"])
    o_ref, S_ref = getattr(oracle, f"{member}_fwd")(*xo)
    ref = getattr(oracle, f"{member}_bwd")(*xo, x["dO"], x["dS_out"])
    ref.update(o=o_ref, S_out=S_ref)
    got = dict(o=o1, S_out=S1, **g1)
    for key, r in ref.items():
        e = rel_err(to_np(got[key]), r)
        assert e < tol(dtype, key), (key, e)


@pytest.mark.parametrize("member", ["gla", "mamba2"])
def test_saved_chunked_equals_unchunked_and_plain(member):
    import torch
    from chunked_linear_recurrence_chunk_amd import stateflow
    B, T, H, dk, dv = 1, 1024, 4, 128, 256
    print(f"[{member} saved] stateflow 4 chunks", flush=True)
    x = _make(member, B, T, H, dk, dv, "bf16", 60)
    d, S_in, dS = _dev(x, "bf16")
    Drv = stateflow.GlaChunked if member == "gla" else stateflow.Mamba2Chunked
    res = []
    for N, save in ((4, False), (1, True), (4, True)):
        drv = Drv(d["q"], d["k"], d["v"], d["g"], N, save=save)
        o, S = drv.forward(S_in)
        gr = drv.backward(d["dO"], dS)
        torch.cuda.synchronize()
        assert all(a is None for a in drv.acts)  # released after each chunk's backward
        res.append(dict(o=o.clone(), S_out=S.clone(), **{k: v.clone() for k, v in gr.items()}))
    for key in res[0]:
        assert torch.equal(res[0][key], res[1][key]), key
        assert torch.equal(res[0][key], res[2][key]), key


@pytest.mark.parametrize("member", ["gla", "mamba2"])
def test_saved_forward_without_output(member):
    """A saving forward with no output o: the scan stores the states for the
    backward itself (the out kernel, which stores them otherwise, does not
    run).  The backward that reads them equals the recomputing one."""
    import torch
    from chunked_linear_recurrence_chunk_amd import ops
    print(f"[{member} saved] forward without o", flush=True)
    B, T, H, dk, dv = 1, 320, 2, 128, 256
    x = _make(member, B, T, H, dk, dv, "bf16", 65)
    d, S_in, dS = _dev(x, "bf16")
    args = (d["q"], d["k"], d["v"], d["g"])
    shape = ops.make_shape(d["q"], d["v"])
    op_f, op_b = (ops.OP_GLA_FWD, ops.OP_GLA_BWD) if member == "gla" else (ops.OP_M2_FWD, ops.OP_M2_BWD)
    saved = torch.empty(ops.saved_bytes(shape, op_f), dtype=torch.uint8, device="cuda")
    ws = torch.empty(max(ops.workspace_bytes(shape, op) for op in (op_f, op_b)), dtype=torch.uint8, device="cuda")
    S_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
    lib = ops.load()
    rc = getattr(lib, f"{member}_fwd_save")(ops.ctypes.byref(shape), ops._ptr(d["q"]), ops._ptr(d["k"]),
                                            ops._ptr(d["v"]), ops._ptr(d["g"]), None, ops._ptr(S_in), None,
                                            ops._ptr(S_out), ops._ptr(saved), saved.numel(), ops._ptr(ws),
                                            ws.numel(), ops._stream())
    assert rc == 0, rc
    g1 = getattr(ops, f"{member}_bwd_saved")(*args, None, d["dO"], dS, saved)
    o0, S0 = getattr(ops, f"{member}_fwd")(*args, S_in)
    g0 = getattr(ops, f"{member}_bwd")(*args, S_in, d["dO"], dS)
    torch.cuda.synchronize()
    assert torch.equal(S0, S_out)
    for key in g0:
        assert torch.equal(g0[key], g1[key]), key


def test_saved_buffer_reused_across_members():
    """One saved buffer and one workspace through a GLA chunk, then a Mamba-2
    chunk: the second call's results do not depend on what the first left."""
    import torch
    from chunked_linear_recurrence_chunk_amd import ops
    print("[gla saved] buffer reuse", flush=True)
    xa = _make("gla", 1, 512, 2, 128, 256, "bf16", 61)
    xb = _make("mamba2", 1, 384, 2, 128, 256, "bf16", 62)
    shape = ops.ClrShape(1, 512, 2, 128, 256, 1)
    saved = torch.empty(ops.saved_bytes(shape, ops.OP_GLA_BWD), dtype=torch.uint8, device="cuda")
    nws = max(ops.workspace_bytes(shape, op) for op in (ops.OP_GLA_FWD, ops.OP_GLA_BWD))
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    d, S_in, dS = _dev(xa, "bf16")
    ops.gla_fwd_save(d["q"], d["k"], d["v"], d["g"], S_in, saved=saved, ws=ws)
    ops.gla_bwd_saved(d["q"], d["k"], d["v"], d["g"], S_in, d["dO"], dS, saved, ws=ws)
    d, S_in, dS = _dev(xb, "bf16")
    args = (d["q"], d["k"], d["v"], d["g"])
    o1, S1, _ = ops.mamba2_fwd_save(*args, S_in, saved=saved, ws=ws)
    g1 = ops.mamba2_bwd_saved(*args, S_in, d["dO"], dS, saved, ws=ws)
    o0, S0 = ops.mamba2_fwd(*args, S_in)
    g0 = ops.mamba2_bwd(*args, S_in, d["dO"], dS)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(S0, S1)
    for key in g0:
        assert torch.equal(g0[key], g1[key]), key
