"""The C ABI from a plain C program (tests/c_consumer/clr_c_driver.c): no
PyTorch, no C++, only include/clr.h and the HIP runtime API.

CPU: the program compiles as C11 against the public header and the library,
and every host-side rejection it exercises returns the documented status.
GPU: it runs one Gated DeltaNet layer over N sequence chunks in the StateFlow
order (StateFlow paper, Sec. 3.1, Eqs. 5 and 7) on its own device buffers,
recomputing each chunk's forward in its backward and, in a second run,
keeping the activations instead (gdn_fwd_save / gdn_bwd_saved); its outputs
match the fp64 oracle within the tolerances, and equal bit for bit what the
Python binding's chunk driver returns for the same inputs in the same mode.
"""
import os
import subprocess

import numpy as np
import pytest

from tests.conftest import gpu_available

MAGIC = 0x434C5231


def _driver():
    from tests.c_consumer import build_driver
    return build_driver.path()


def test_c_program_builds_and_host_checks_pass():
    from tests.c_consumer import build_driver
    exe = build_driver.build()
    p = subprocess.run([exe, "check"], capture_output=True, text=True, timeout=60)
    assert p.returncode == 0, p.stderr


def _write_inputs(path, x, B, T, H, dk, dv, dtype, N):
    from chunked_linear_recurrence_chunk_amd import inputs
    code = 1 if dtype == "bf16" else 0
    with open(path, "wb") as f:
        f.write(np.array([MAGIC, B, T, H, dk, dv, code, N], dtype=np.int32).tobytes())
        for key in ("q", "k", "v", "g", "beta", "dO"):
            a = np.ascontiguousarray(x[key], dtype=np.float32)
            f.write((inputs.bf16_bits(a) if dtype == "bf16" else a).tobytes())
        for key in ("S_in", "dS_out"):
            f.write(np.ascontiguousarray(x[key], dtype=np.float32).tobytes())


def _read_outputs(path, B, T, H, dk, dv, dtype):
    from chunked_linear_recurrence_chunk_amd import inputs
    raw = open(path, "rb").read()
    es = 2 if dtype == "bf16" else 4
    shapes = [("o", (B, T, H, dv)), ("dq", (B, T, H, dk)), ("dk", (B, T, H, dk)), ("dv", (B, T, H, dv)),
              ("dg", (B, T, H)), ("dbeta", (B, T, H))]
    out, off = {}, 0
    for key, shp in shapes:
        n = int(np.prod(shp))
        if dtype == "bf16":
            bits = np.frombuffer(raw, dtype=np.uint16, count=n, offset=off)
            out[key] = inputs.bf16_value(bits).reshape(shp)
        else:
            out[key] = np.frombuffer(raw, dtype=np.float32, count=n, offset=off).reshape(shp)
        off += n * es
    for key in ("S_out", "dS_in"):
        n = B * H * dk * dv
        out[key] = np.frombuffer(raw, dtype=np.float32, count=n, offset=off).reshape(B, H, dk, dv)
        off += n * 4
    assert off == len(raw), (off, len(raw))
    return out


CASES = [
    # (T, H, dk, dv, dtype, N, seed)
    (512, 4, 128, 128, "bf16", 4, 41),
    (320, 2, 64, 64, "bf16", 5, 42),
    (256, 1, 32, 32, "fp32", 4, 43),
]


@pytest.mark.gpu
@pytest.mark.skipif(not gpu_available(), reason="needs a GPU")
@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}H{c[1]}d{c[2]}-{c[4]}-N{c[5]}" for c in CASES])
def test_c_program_chunk_chain_matches_oracle_and_binding(case, tmp_path):
    import torch
    from chunked_linear_recurrence_chunk_amd import inputs, stateflow
    from oracle import oracle
    from tests.gpu_util import rel_err, to_dev, tol
    T, H, dk, dv, dtype, N, seed = case
    B = 1
    print(f"[c consumer] case {case}", flush=True)
    x = inputs.make_gdn(B, T, H, dk, dv, dtype, seed)
    fin, fout = os.path.join(tmp_path, "in.bin"), os.path.join(tmp_path, "out.bin")
    _write_inputs(fin, x, B, T, H, dk, dv, dtype, N)
    p = subprocess.run([_driver(), "run", fin, fout], capture_output=True, text=True, timeout=120)
    assert p.returncode == 0, p.stderr
    got = _read_outputs(fout, B, T, H, dk, dv, dtype)

    o_ref, S_ref = oracle.gdn_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"])
    ref = oracle.gdn_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S_in"], x["dO"], x["dS_out"])
    ref.update(o=o_ref, S_out=S_ref)
    for key, r in ref.items():
        e = rel_err(got[key], r)
        assert e < tol(dtype, key), (key, e)

    # the same chunk chain through the Python binding: identical bits
    d = {k: to_dev(x[k], dtype) for k in ("q", "k", "v", "g", "beta", "dO")}
    drv = stateflow.GdnChunked(d["q"], d["k"], d["v"], d["g"], d["beta"], N)
    o, S = drv.forward(to_dev(x["S_in"], "fp32"))
    gr = drv.backward(d["dO"], to_dev(x["dS_out"], "fp32"))
    torch.cuda.synchronize()
    py = dict(o=o, S_out=S, **gr)
    for key in ref:
        a = py[key].float().cpu().numpy()
        assert np.array_equal(a, got[key].astype(np.float32)), key

    # and with saved activations (gdn_fwd_save / gdn_bwd_saved), against the
    # oracle and the binding's chunk driver in the same mode
    fsv = os.path.join(tmp_path, "out_saved.bin")
    p = subprocess.run([_driver(), "run-saved", fin, fsv], capture_output=True, text=True, timeout=120)
    assert p.returncode == 0, p.stderr
    got_s = _read_outputs(fsv, B, T, H, dk, dv, dtype)
    for key, r in ref.items():
        e = rel_err(got_s[key], r)
        assert e < tol(dtype, key), (key, e)
    drv = stateflow.GdnChunked(d["q"], d["k"], d["v"], d["g"], d["beta"], N, save=True)
    o, S = drv.forward(to_dev(x["S_in"], "fp32"))
    gr = drv.backward(d["dO"], to_dev(x["dS_out"], "fp32"))
    torch.cuda.synchronize()
    py = dict(o=o, S_out=S, **gr)
    for key in ref:
        assert np.array_equal(py[key].float().cpu().numpy(), got_s[key].astype(np.float32)), key
