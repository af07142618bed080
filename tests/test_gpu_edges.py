"""Edge cases of every entry point on the GPU against the oracle: empty
sequences (T = 0: the state passes through, NULL per-token tensors), a
single token, one token short of a block, one token past it, zero boundary
states (NULL S_in / dS_out), B > 1 with H = 1."""
import numpy as np
import pytest

from tests.conftest import gpu_available
from tests.gpu_util import rel_err, to_dev, to_np, tol

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

FAMILIES = ["gdn", "gla", "mamba2", "kda"]


def _make(fam, B, T, H, d, dtype, seed):
    from chunked_linear_recurrence_chunk_amd import inputs
    return {"gdn": inputs.make_gdn, "gla": inputs.make_gla, "mamba2": inputs.make_mamba2,
            "kda": inputs.make_kda}[fam](B, T, H, d, d, dtype, seed)


def _gpu(fam, x, dtype, S_in, dS_out):
    from chunked_linear_recurrence_chunk_amd import ops
    delta = fam in ("gdn", "kda")
    keys = ("q", "k", "v", "g", "beta", "dO") if delta else ("q", "k", "v", "g", "dO")
    d = {k: to_dev(x[k], dtype) for k in keys}
    args = [d[k] for k in keys[:-1]]
    fwd, bwd = {"gdn": (ops.gdn_fwd, ops.gdn_bwd), "gla": (ops.gla_fwd, ops.gla_bwd),
                "mamba2": (ops.mamba2_fwd, ops.mamba2_bwd), "kda": (ops.kda_fwd, ops.kda_bwd)}[fam]
    o, S = fwd(*args, S_in)
    gr = bwd(*args, S_in, d["dO"], dS_out)
    return dict(o=o, S_out=S, **gr)


def _oracle(fam, x, S_in, dS_out):
    from oracle import oracle
    delta = fam in ("gdn", "kda")
    fwd, bwd = {"gdn": (oracle.gdn_fwd, oracle.gdn_bwd), "gla": (oracle.gla_fwd, oracle.gla_bwd),
                "mamba2": (oracle.mamba2_fwd, oracle.mamba2_bwd), "kda": (oracle.kda_fwd, oracle.kda_bwd)}[fam]
    args = [x[k] for k in (("q", "k", "v", "g", "beta") if delta else ("q", "k", "v", "g"))]
    o, S = fwd(*args, S_in)
    r = bwd(*args, S_in, x["dO"], dS_out)
    r.update(o=o, S_out=S)
    return r


@pytest.mark.parametrize("fam", FAMILIES)
@pytest.mark.parametrize("T", [1, 63, 65])
def test_short_and_ragged_sequences(fam, T):
    import torch
    B, H, d, dtype = 3, 1, 64, "bf16"
    print(f"[edges] {fam} T={T}", flush=True)
    x = _make(fam, B, T, H, d, dtype, 500 + T)
    with_s = T != 63                       # T = 63: zero S_in and dS_out (NULL)
    S_in = to_dev(x["S_in"], "fp32") if with_s else None
    dS_out = to_dev(x["dS_out"], "fp32") if with_s else None
    got = _gpu(fam, x, dtype, S_in, dS_out)
    torch.cuda.synchronize()
    ref = _oracle(fam, x, x["S_in"] if with_s else None, x["dS_out"] if with_s else None)
    for key, r in ref.items():
        e = rel_err(to_np(got[key]), r)
        assert e < tol(dtype, key), (key, e)


@pytest.mark.parametrize("fam", FAMILIES)
def test_empty_sequence_passes_the_state_through(fam):
    import torch
    B, H, d = 2, 2, 32
    x = _make(fam, B, 0, H, d, "bf16", 600)
    S_in, dS_out = to_dev(x["S_in"], "fp32"), to_dev(x["dS_out"], "fp32")
    got = _gpu(fam, x, "bf16", S_in, dS_out)
    nul = _gpu(fam, x, "bf16", None, None)
    torch.cuda.synchronize()
    assert got["o"].shape[1] == 0 and got["dq"].shape[1] == 0
    assert torch.equal(got["S_out"], S_in) and torch.equal(got["dS_in"], dS_out)
    assert not nul["S_out"].any() and not nul["dS_in"].any()


def test_shortconv_empty_and_single_token():
    import torch
    from chunked_linear_recurrence_chunk_amd import inputs, ops
    from oracle import oracle
    for T in (0, 1, 2):
        x = inputs.make_shortconv(2, T, 64, 4, "bf16", 700 + T)
        d = {k: to_dev(x[k], "bf16") for k in ("x", "state_in", "dy")}
        w, bias = to_dev(x["w"], "fp32"), to_dev(x["bias"], "fp32")
        dso = to_dev(x["dstate_out"], "fp32")
        y, so = ops.shortconv_fwd(d["x"], w, bias, d["state_in"], act=1)
        g = ops.shortconv_bwd(d["x"], w, bias, d["state_in"], d["dy"], dso, act=1)
        torch.cuda.synchronize()
        xs = {k: np.asarray(v, dtype=np.float64) for k, v in x.items()}
        y_ref, so_ref = oracle.conv_fwd(xs["x"], xs["w"], xs["bias"], xs["state_in"], 1)
        r = oracle.conv_bwd(xs["x"], xs["w"], xs["bias"], xs["state_in"], xs["dy"], xs["dstate_out"], 1)
        assert rel_err(to_np(so), so_ref) == 0.0, T               # copies of input rows
        if T:
            assert rel_err(to_np(y), y_ref) < 2e-2
            assert rel_err(to_np(g["dx"]), r["dx"]) < 2e-2
        assert rel_err(to_np(g["dstate_in"]), r["dstate_in"]) < 2e-2
        assert rel_err(to_np(g["dw"]), r["dw"]) < 2e-2 or T == 0
