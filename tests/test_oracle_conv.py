"""Pins the short-convolution oracle (oracle/conv_oracle.c) to things other
than itself: numpy.convolve per channel, the pointwise W = 1 case, the SiLU
closed form, central finite differences of every gradient (including the
boundary state), the state hand-off over sequence chunks, and planted
mistakes that these pins must catch."""
import os

import numpy as np
import pytest

from oracle import oracle


def _rand(rng, B, T, C, W):
    return dict(x=rng.standard_normal((B, T, C)), w=rng.standard_normal((C, W)) * 0.5,
                bias=rng.standard_normal(C) * 0.3, state_in=rng.standard_normal((B, W - 1, C)))


def test_matches_numpy_convolve():
    rng = np.random.default_rng(1)
    B, T, C, W = 2, 17, 5, 4
    d = _rand(rng, B, T, C, W)
    y, st = oracle.conv_fwd(d["x"], d["w"], None, d["state_in"], act=0)
    for b in range(B):
        xe = np.concatenate([d["state_in"][b], d["x"][b]], 0)
        for c in range(C):
            ref = np.convolve(xe[:, c], d["w"][c][::-1], mode="valid")
            assert np.allclose(y[b, :, c], ref, atol=1e-12)
        assert np.array_equal(st[b], xe[-(W - 1):])


def test_pointwise_width_one_and_silu():
    rng = np.random.default_rng(2)
    d = _rand(rng, 1, 9, 4, 1)
    y, st = oracle.conv_fwd(d["x"], d["w"], d["bias"], None, act=0)
    assert np.allclose(y, d["x"] * d["w"][:, 0] + d["bias"], atol=1e-14) and st.shape == (1, 0, 4)
    y1, _ = oracle.conv_fwd(d["x"], d["w"], d["bias"], None, act=1)
    assert np.allclose(y1, y / (1 + np.exp(-y)), atol=1e-14)


def test_short_chunk_keeps_the_state_tail():
    """T < W - 1: the outgoing state still holds the last W - 1 rows of
    [state_in ; x]; T = 0 passes the state through."""
    rng = np.random.default_rng(3)
    d = _rand(rng, 2, 2, 3, 4)
    _, st = oracle.conv_fwd(d["x"], d["w"], d["bias"], d["state_in"])
    assert np.array_equal(st, np.concatenate([d["state_in"], d["x"]], 1)[:, -3:])
    _, st0 = oracle.conv_fwd(d["x"][:, :0], d["w"], d["bias"], d["state_in"])
    assert np.array_equal(st0, d["state_in"])


def _fd(f, a, h=1e-6):
    out = np.zeros_like(a)
    flat = a.reshape(-1)
    for i in range(flat.size):
        old = flat[i]
        flat[i] = old + h
        lp = f()
        flat[i] = old - h
        lm = f()
        flat[i] = old
        out.reshape(-1)[i] = (lp - lm) / (2 * h)
    return out


@pytest.mark.parametrize("shape", [(1, 6, 3, 4), (2, 2, 2, 4), (1, 7, 2, 1), (2, 5, 3, 2)])
@pytest.mark.parametrize("act", [0, 1])
def test_gradients_match_finite_differences(shape, act):
    rng = np.random.default_rng(10 + sum(shape) + act)
    B, T, C, W = shape
    d = _rand(rng, B, T, C, W)
    dy = rng.standard_normal((B, T, C))
    dso = rng.standard_normal((B, W - 1, C))

    def loss():
        y, st = oracle.conv_fwd(d["x"], d["w"], d["bias"], d["state_in"], act)
        return float(np.sum(y * dy) + np.sum(st * dso))
    r = oracle.conv_bwd(d["x"], d["w"], d["bias"], d["state_in"], dy, dso, act)
    for key, g in (("x", "dx"), ("w", "dw"), ("bias", "dbias"), ("state_in", "dstate_in")):
        fd = _fd(loss, d[key])
        err = np.max(np.abs(fd - r[g])) / max(np.max(np.abs(fd)), 1e-3) if fd.size else 0.0
        assert err < 1e-7, (key, err)


@pytest.mark.parametrize("N", [2, 5])
def test_chunk_split(N):
    """Chunks with the state handed on give the unsplit y, state_out and dx
    bit for bit; dw and dbias are the sums of the chunks' parts."""
    rng = np.random.default_rng(20 + N)
    B, T, C, W = 2, 40, 3, 4
    d = _rand(rng, B, T, C, W)
    dy = rng.standard_normal((B, T, C))
    dso = rng.standard_normal((B, W - 1, C))
    y1, s1 = oracle.conv_fwd(d["x"], d["w"], d["bias"], d["state_in"], 1)
    r1 = oracle.conv_bwd(d["x"], d["w"], d["bias"], d["state_in"], dy, dso, 1)
    L = T // N
    st, states, ys = d["state_in"], [], []
    for i in range(N):
        states.append(st)
        yi, st = oracle.conv_fwd(d["x"][:, i * L:(i + 1) * L], d["w"], d["bias"], st, 1)
        ys.append(yi)
    assert np.array_equal(np.concatenate(ys, 1), y1) and np.array_equal(st, s1)
    ds, dxs, dw, db = dso, [None] * N, 0.0, 0.0
    for i in reversed(range(N)):
        r = oracle.conv_bwd(d["x"][:, i * L:(i + 1) * L], d["w"], d["bias"], states[i],
                            dy[:, i * L:(i + 1) * L], ds, 1)
        dxs[i], ds = r["dx"], r["dstate_in"]
        dw, db = dw + r["dw"], db + r["dbias"]
    assert np.array_equal(np.concatenate(dxs, 1), r1["dx"]) and np.array_equal(ds, r1["dstate_in"])
    assert np.allclose(dw, r1["dw"], atol=1e-12) and np.allclose(db, r1["dbias"], atol=1e-12)


CONV_SRC = os.path.join(os.path.dirname(oracle.__file__), "conv_oracle.c")
MUTANTS = [
    ("taps reversed", "z += w[(size_t)c * W + j] * xe_at(x, state_in, b, t + j, c, T, C, W);\n                y[",
     "z += w[(size_t)c * W + (W - 1 - j)] * xe_at(x, state_in, b, t + j, c, T, C, W);\n                y["),
    ("silu derivative drops a term", "return s * (1.0 + z * (1.0 - s));", "return s;"),
    ("dstate_out not added", "double acc = (dstate_out && r >= T) ?", "double acc = (dstate_out && r >= T + W) ?"),
    ("dw off by one row", "dw[(size_t)c * W + j] += dz[t] * xe_at(x, state_in, b, t + j, c, T, C, W);",
     "dw[(size_t)c * W + j] += dz[t] * xe_at(x, state_in, b, t + j - (t + j > 0), c, T, C, W);"),
    ("state_out one row early", "xe_at(x, state_in, b, T + i, c, T, C, W);",
     "xe_at(x, state_in, b, T + i - 1, c, T, C, W);"),
]


def _pins_pass(lib):
    rng = np.random.default_rng(4)
    ok = True
    for act in (0, 1):
        B, T, C, W = 1, 6, 2, 4
        d = _rand(rng, B, T, C, W)
        dy = rng.standard_normal((B, T, C))
        dso = rng.standard_normal((B, W - 1, C))
        y, st = oracle.conv_fwd(d["x"], d["w"], d["bias"], d["state_in"], act, lib=lib)
        xe = np.concatenate([d["state_in"][0], d["x"][0]], 0)
        for c in range(C):
            z = np.convolve(xe[:, c], d["w"][c][::-1], mode="valid") + d["bias"][c]
            ref = z / (1 + np.exp(-z)) if act else z
            ok &= np.allclose(y[0, :, c], ref, atol=1e-12)
        ok &= np.array_equal(st[0], xe[-(W - 1):])

        def loss():
            yy, ss = oracle.conv_fwd(d["x"], d["w"], d["bias"], d["state_in"], act, lib=lib)
            return float(np.sum(yy * dy) + np.sum(ss * dso))
        r = oracle.conv_bwd(d["x"], d["w"], d["bias"], d["state_in"], dy, dso, act, lib=lib)
        for key, g in (("x", "dx"), ("w", "dw"), ("bias", "dbias"), ("state_in", "dstate_in")):
            fd = _fd(loss, d[key])
            ok &= np.max(np.abs(fd - r[g])) < 1e-7 * max(np.max(np.abs(fd)), 1e-3)
    return bool(ok)


def test_pins_pass_on_the_oracle():
    assert _pins_pass(oracle.load_conv())


@pytest.mark.parametrize("desc,find,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(desc, find, repl, tmp_path):
    src = open(CONV_SRC).read()
    assert src.count(find) == 1, desc
    mut = tmp_path / "mut.c"
    mut.write_text(src.replace(find, repl))
    so = str(tmp_path / "libmut.so")
    oracle.build_conv(src=str(mut), out=so)
    assert not _pins_pass(oracle.load_conv(so)), "planted mistake not caught: " + desc
