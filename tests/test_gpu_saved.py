"""GPU parity of the Gated DeltaNet pair with saved activations
(gdn_fwd_save / gdn_bwd_saved), through the C ABI.

gdn_fwd_save must return what gdn_fwd returns, bit for bit, and the backward
that reads its saved states and U must match the fp64 oracle within the
tolerances.  Where gdn_bwd's forward recompute runs one consumer wave per
value slice (fp32, and d = 32), its states are the forward's own, so the two
backwards agree bit for bit; with two consumers (bf16, d >= 64) the
recompute sums each block's products over key halves in another order, and
the two agree to rounding.  Sequence chunking with saved activations
reproduces the unchunked run bit for bit.
"""
import numpy as np
import pytest

from tests.conftest import gpu_available
from tests.gpu_util import rel_err, to_dev, to_np, tol

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

CASES = [
    # (B, T, H, dk, dv, dtype, seed)
    (1, 256, 1, 32, 32, "fp32", 31),
    (2, 200, 3, 32, 32, "fp32", 32),   # ragged tail
    (1, 192, 2, 64, 64, "fp32", 33),
    (1, 512, 2, 128, 128, "bf16", 34),
    (2, 320, 2, 64, 64, "bf16", 35),
    (1, 100, 2, 128, 128, "bf16", 36),  # ragged, < 2 blocks
    (1, 2048, 16, 128, 128, "bf16", 37),
]


def _dev(x, dtype):
    d = {k: to_dev(x[k], dtype) for k in ("q", "k", "v", "g", "beta", "dO")}
    return d, to_dev(x["S_in"], "fp32"), to_dev(x["dS_out"], "fp32")


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}T{c[1]}H{c[2]}d{c[3]}-{c[5]}" for c in CASES])
def test_saved_pair_matches_oracle_and_plain_pair(case):
    import torch
    from chunked_linear_recurrence_chunk_amd import inputs, ops
    from oracle import oracle
    B, T, H, dk, dv, dtype, seed = case
    print(f"[gdn saved] case {case}", flush=True)
    x = inputs.make_gdn(B, T, H, dk, dv, dtype, seed)
    d, S_in, dS = _dev(x, dtype)
    o0, S0 = ops.gdn_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S_in)
    o1, S1, saved = ops.gdn_fwd_save(d["q"], d["k"], d["v"], d["g"], d["beta"], S_in)
    g0 = ops.gdn_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S_in, d["dO"], dS)
    # S_in is not read by the saved backward
    g1 = ops.gdn_bwd_saved(d["q"], d["k"], d["v"], d["g"], d["beta"], None, d["dO"], dS, saved)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(S0, S1)
    one_consumer = dtype == "fp32" or dk == 32
    for key in g0:
        if one_consumer:
            assert torch.equal(g0[key], g1[key]), key
        else:
            assert rel_err(to_np(g1[key]), to_np(g0[key])) < 1e-2, key
    ref = oracle.gdn_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"], x["dO"], x["dS_out"])
    for key, r in ref.items():
        e = rel_err(to_np(g1[key]), r)
        assert e < tol(dtype, key), (key, e)


def test_saved_chunked_equals_unchunked_and_oracle():
    import torch
    from chunked_linear_recurrence_chunk_amd import inputs, stateflow
    from oracle import oracle
    B, T, H, dk, dv = 1, 1024, 4, 128, 128
    print("[gdn saved] stateflow 4 chunks", flush=True)
    x = inputs.make_gdn(B, T, H, dk, dv, "bf16", 38)
    d, S_in, dS = _dev(x, "bf16")
    res = []
    for N in (1, 4):
        drv = stateflow.GdnChunked(d["q"], d["k"], d["v"], d["g"], d["beta"], N, save=True)
        o, S = drv.forward(S_in)
        gr = drv.backward(d["dO"], dS)
        torch.cuda.synchronize()
        assert all(a is None for a in drv.acts)  # released after each chunk's backward
        res.append(dict(o=o.clone(), S_out=S.clone(), **{k: v.clone() for k, v in gr.items()}))
    for key in res[0]:
        assert torch.equal(res[0][key], res[1][key]), key
    o_ref, S_ref = oracle.gdn_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"])
    ref = oracle.gdn_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"], x["dO"], x["dS_out"])
    ref.update(o=o_ref, S_out=S_ref)
    for key, r in ref.items():
        e = rel_err(to_np(res[1][key]), r)
        assert e < tol("bf16", key), (key, e)


def test_saved_buffer_reused_for_a_second_chunk():
    """Two chunks in a row through one saved buffer and one workspace: the
    second call's results do not depend on what the first left in them."""
    import torch
    from chunked_linear_recurrence_chunk_amd import inputs, ops
    print("[gdn saved] buffer reuse", flush=True)
    xs = [inputs.make_gdn(1, 512, 2, 128, 128, "bf16", s) for s in (39, 40)]
    outs = []
    saved = None
    for x in xs:
        d, S_in, dS = _dev(x, "bf16")
        o, S, saved = ops.gdn_fwd_save(d["q"], d["k"], d["v"], d["g"], d["beta"], S_in, saved=saved)
        g = ops.gdn_bwd_saved(d["q"], d["k"], d["v"], d["g"], d["beta"], S_in, d["dO"], dS, saved)
        torch.cuda.synchronize()
        outs.append((o.clone(), {k: v.clone() for k, v in g.items()}))
    d, S_in, dS = _dev(xs[1], "bf16")
    o, S, fresh = ops.gdn_fwd_save(d["q"], d["k"], d["v"], d["g"], d["beta"], S_in)
    g = ops.gdn_bwd_saved(d["q"], d["k"], d["v"], d["g"], d["beta"], S_in, d["dO"], dS, fresh)
    torch.cuda.synchronize()
    assert torch.equal(o, outs[1][0])
    for key in g:
        assert torch.equal(g[key], outs[1][1][key]), key


STRESS = [
    # (T, H, d, dtype, N, gate, seed): the delta-rule stress input (almost no
    # decay, beta = 0.99, keys repeated from 8 L2-normalised vectors)
    (256, 2, 32, "fp32", 4, "slow", 321),
    (2048, 4, 128, "bf16", 1, "zero", 322),
    (8192, 4, 128, "bf16", 4, "slow", 323),
]


@pytest.mark.parametrize("case", STRESS, ids=[f"T{c[0]}H{c[1]}d{c[2]}-{c[3]}-N{c[4]}-{c[5]}" for c in STRESS])
def test_saved_stress_matches_oracle(case):
    import torch
    from chunked_linear_recurrence_chunk_amd import inputs, stateflow
    from oracle import oracle
    T, H, d, dtype, N, gate, seed = case
    print(f"[gdn saved] stress {case}", flush=True)
    x = inputs.make_delta_stress("gdn", 1, T, H, d, d, dtype, seed, gate=gate)
    dv, S_in, dS = _dev(x, dtype)
    drv = stateflow.GdnChunked(dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"], N, save=True)
    o, S = drv.forward(S_in)
    gr = drv.backward(dv["dO"], dS)
    torch.cuda.synchronize()
    got = dict(o=o, S_out=S, **gr)
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"])
    o_ref, S_ref = oracle.gdn_fwd(*args)
    ref = oracle.gdn_bwd(*args, x["dO"], x["dS_out"])
    ref.update(o=o_ref, S_out=S_ref)
    errs = {key: rel_err(to_np(got[key]), r) for key, r in ref.items()}
    print("  errors", {key: f"{e:.2e}" for key, e in errs.items()}, flush=True)
    bad = {key: e for key, e in errs.items() if not e < tol(dtype, key)}
    assert not bad, bad


KDA_CASES = [
    # (B, T, H, d, dtype, seed)
    (1, 256, 1, 32, "fp32", 71),
    (2, 200, 3, 64, "fp32", 72),    # ragged tail
    (1, 512, 2, 128, "bf16", 73),
    (1, 100, 2, 128, "bf16", 74),   # ragged, < 2 blocks
    (1, 2048, 16, 128, "bf16", 75),
]


@pytest.mark.parametrize("case", KDA_CASES, ids=[f"kda-B{c[0]}T{c[1]}H{c[2]}d{c[3]}-{c[4]}" for c in KDA_CASES])
def test_kda_saved_pair_equals_plain_pair_and_matches_oracle(case):
    """kda_fwd_save / kda_bwd_saved: the forward keeps the states and U its
    scan forms (with one consumer wave, the values the backward's recompute
    forms), so both halves equal kda_fwd / kda_bwd bit for bit."""
    import torch
    from chunked_linear_recurrence_chunk_amd import inputs, ops
    from oracle import oracle
    B, T, H, d, dtype, seed = case
    print(f"[kda saved] case {case}", flush=True)
    x = inputs.make_kda(B, T, H, d, d, dtype, seed)
    dv_, S_in, dS = _dev(x, dtype)
    args = (dv_["q"], dv_["k"], dv_["v"], dv_["g"], dv_["beta"])
    o0, S0 = ops.kda_fwd(*args, S_in)
    o1, S1, saved = ops.kda_fwd_save(*args, S_in)
    g0 = ops.kda_bwd(*args, S_in, dv_["dO"], dS)
    g1 = ops.kda_bwd_saved(*args, None, dv_["dO"], dS, saved)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(S0, S1)
    for key in g0:
        assert torch.equal(g0[key], g1[key]), key
    xo = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"])
    ref = oracle.kda_bwd(*xo, x["dO"], x["dS_out"])
    for key, r in ref.items():
        e = rel_err(to_np(g1[key]), r)
        assert e < tol(dtype, key), (key, e)


def test_kda_saved_chunked_equals_plain():
    import torch
    from chunked_linear_recurrence_chunk_amd import inputs, stateflow
    print("[kda saved] stateflow 4 chunks", flush=True)
    x = inputs.make_kda(1, 1024, 4, 128, 128, "bf16", 76)
    d, S_in, dS = _dev(x, "bf16")
    res = []
    for N, save in ((4, False), (4, True), (1, True)):
        drv = stateflow.KdaChunked(d["q"], d["k"], d["v"], d["g"], d["beta"], N, save=save)
        o, S = drv.forward(S_in)
        gr = drv.backward(d["dO"], dS)
        torch.cuda.synchronize()
        assert all(a is None for a in drv.acts)
        res.append(dict(o=o.clone(), S_out=S.clone(), **{k: v.clone() for k, v in gr.items()}))
    for key in res[0]:
        assert torch.equal(res[0][key], res[1][key]), key
        assert torch.equal(res[0][key], res[2][key]), key
