"""fp64 CPU oracle for the gated linear recurrence layer -- Python binding.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the benchmark's CPU-baseline leg may import this module.  The product
package never imports it and must not fall back to it.

It wraps ``clr_oracle.c`` (plain per-token fp64 recurrences with hand-derived
adjoints; see that file's header for the definitions and their source in the
StateFlow paper, Sec. 2.1 Eq. 1 and Sec. 3.1).  All arrays are numpy float64,
contiguous, in the layouts

    q, k [B,T,H,dk]; v, o, dO [B,T,H,dv]; g: GDN and Mamba-2 [B,T,H],
    GLA [B,T,H,dk];
    beta [B,T,H]; states S_in, S_out, dS_in, dS_out [B,H,dk,dv].

``build()`` compiles the C file with gcc into ``oracle/_build``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "clr_oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD, "libclr_oracle.so")

# Portable x86-64 (AVX2/FMA level) so the library runs on any current host;
# no FP contraction so every multiply and add rounds as written.
CFLAGS = ["-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fopenmp",
          "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra"]


def build(src: str = _SRC, out: str = _LIB_PATH, extra=()) -> str:
    """Compile the oracle (always; cheap) and return the library path."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, out)
    return out


_lib = None
_conv_lib = None
_CONV_SRC = os.path.join(_HERE, "conv_oracle.c")
_CONV_LIB_PATH = os.path.join(_BUILD, "libconv_oracle.so")


def build_conv(src: str = _CONV_SRC, out: str = _CONV_LIB_PATH) -> str:
    """Compile the short-convolution oracle (conv_oracle.c)."""
    return build(src=src, out=out)


def load_conv(path: Optional[str] = None):
    """Load (building first if absent) the short-convolution oracle."""
    global _conv_lib
    if path is None and _conv_lib is not None:
        return _conv_lib
    p = path or _CONV_LIB_PATH
    if not os.path.exists(p):
        build_conv(out=p)
    lib = ctypes.CDLL(p)
    i, dp = ctypes.c_int, _dp()
    lib.ref_conv_fwd.argtypes = [i] * 5 + [dp] * 6
    lib.ref_conv_bwd.argtypes = [i] * 5 + [dp] * 10
    lib.ref_conv_fwd.restype = lib.ref_conv_bwd.restype = i
    if path is None:
        _conv_lib = lib
    return lib


def conv_fwd(x, w, bias=None, state_in=None, act=0, lib=None):
    """Causal short convolution with boundary state (conv_oracle.c).
    x [B,T,C], w [C,W], bias [C], state_in [B,W-1,C].  Returns (y, state_out)."""
    lib = lib or load_conv()
    x, w, bias, state_in = map(_c, (x, w, bias, state_in))
    B, T, C = x.shape
    W = w.shape[1]
    y = np.zeros((B, T, C))
    st = np.zeros((B, W - 1, C))
    if lib.ref_conv_fwd(B, T, C, W, int(act), _p(x), _p(w), _p(bias), _p(state_in), _p(y), _p(st)) != 0:
        raise RuntimeError("ref_conv_fwd failed")
    return y, st


def conv_bwd(x, w, bias, state_in, dy, dstate_out=None, act=0, lib=None):
    """Gradients of the short convolution: dict dx, dw, dbias, dstate_in."""
    lib = lib or load_conv()
    x, w, bias, state_in, dy, dstate_out = map(_c, (x, w, bias, state_in, dy, dstate_out))
    B, T, C = x.shape
    W = w.shape[1]
    r = dict(dx=np.zeros((B, T, C)), dw=np.zeros((C, W)), dbias=np.zeros(C),
             dstate_in=np.zeros((B, W - 1, C)))
    rc = lib.ref_conv_bwd(B, T, C, W, int(act), _p(x), _p(w), _p(bias), _p(state_in), _p(dy),
                          _p(dstate_out), _p(r["dx"]), _p(r["dw"]), _p(r["dbias"]), _p(r["dstate_in"]))
    if rc != 0:
        raise RuntimeError("ref_conv_bwd failed")
    return r


def _dp():
    return ctypes.POINTER(ctypes.c_double)


def load(path: Optional[str] = None):
    """Load (building first if absent) and return the ctypes library."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        build(out=p)
    lib = ctypes.CDLL(p)
    i, dp = ctypes.c_int, _dp()
    lib.ref_gdn_fwd.argtypes = [i] * 5 + [dp] * 8
    lib.ref_gdn_bwd.argtypes = [i] * 5 + [dp] * 14
    lib.ref_gla_fwd.argtypes = [i] * 5 + [dp] * 7
    lib.ref_gla_bwd.argtypes = [i] * 5 + [dp] * 12
    lib.ref_m2_fwd.argtypes = [i] * 5 + [dp] * 7
    lib.ref_m2_bwd.argtypes = [i] * 5 + [dp] * 12
    lib.ref_kda_fwd.argtypes = [i] * 5 + [dp] * 8
    lib.ref_kda_bwd.argtypes = [i] * 5 + [dp] * 14
    for f in (lib.ref_gdn_fwd, lib.ref_gdn_bwd, lib.ref_gla_fwd, lib.ref_gla_bwd,
              lib.ref_m2_fwd, lib.ref_m2_bwd, lib.ref_kda_fwd, lib.ref_kda_bwd):
        f.restype = ctypes.c_int
    lib.ref_set_threads.argtypes = [i]
    lib.ref_set_threads.restype = None
    lib.ref_get_max_threads.argtypes = []
    lib.ref_get_max_threads.restype = i
    if path is None:
        _lib = lib
    return lib


def set_threads(n: int) -> None:
    load().ref_set_threads(int(n))


def max_threads() -> int:
    return int(load().ref_get_max_threads())


def _c(x):
    """float64 C-contiguous copy/view, or None."""
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(x):
    if x is None:
        return None
    return x.ctypes.data_as(_dp())


def _dims(q, v):
    B, T, H, dk = q.shape
    dv = v.shape[3]
    return B, T, H, dk, dv


def gdn_fwd(q, k, v, g, beta, S_in=None, lib=None):
    """Gated DeltaNet chunk forward: returns (o, S_out)."""
    lib = lib or load()
    q, k, v, g, beta, S_in = map(_c, (q, k, v, g, beta, S_in))
    B, T, H, dk, dv = _dims(q, v)
    o = np.zeros((B, T, H, dv))
    S_out = np.zeros((B, H, dk, dv))
    rc = lib.ref_gdn_fwd(B, T, H, dk, dv, _p(q), _p(k), _p(v), _p(g), _p(beta),
                         _p(S_in), _p(o), _p(S_out))
    if rc != 0:
        raise RuntimeError("ref_gdn_fwd failed")
    return o, S_out


def gdn_bwd(q, k, v, g, beta, S_in, dO, dS_out=None, lib=None):
    """Gated DeltaNet chunk backward: returns dict dq, dk, dv, dg, dbeta, dS_in."""
    lib = lib or load()
    q, k, v, g, beta, S_in, dO, dS_out = map(_c, (q, k, v, g, beta, S_in, dO, dS_out))
    B, T, H, dk, dv = _dims(q, v)
    r = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v),
             dg=np.zeros((B, T, H)), dbeta=np.zeros((B, T, H)),
             dS_in=np.zeros((B, H, dk, dv)))
    rc = lib.ref_gdn_bwd(B, T, H, dk, dv, _p(q), _p(k), _p(v), _p(g), _p(beta),
                         _p(S_in), _p(dO), _p(dS_out), _p(r["dq"]), _p(r["dk"]),
                         _p(r["dv"]), _p(r["dg"]), _p(r["dbeta"]), _p(r["dS_in"]))
    if rc != 0:
        raise RuntimeError("ref_gdn_bwd failed")
    return r


def gla_fwd(q, k, v, g, S_in=None, lib=None):
    """GLA chunk forward: returns (o, S_out)."""
    lib = lib or load()
    q, k, v, g, S_in = map(_c, (q, k, v, g, S_in))
    B, T, H, dk, dv = _dims(q, v)
    o = np.zeros((B, T, H, dv))
    S_out = np.zeros((B, H, dk, dv))
    rc = lib.ref_gla_fwd(B, T, H, dk, dv, _p(q), _p(k), _p(v), _p(g), _p(S_in),
                         _p(o), _p(S_out))
    if rc != 0:
        raise RuntimeError("ref_gla_fwd failed")
    return o, S_out


def gla_bwd(q, k, v, g, S_in, dO, dS_out=None, lib=None):
    """GLA chunk backward: returns dict dq, dk, dv, dg, dS_in."""
    lib = lib or load()
    q, k, v, g, S_in, dO, dS_out = map(_c, (q, k, v, g, S_in, dO, dS_out))
    B, T, H, dk, dv = _dims(q, v)
    r = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v),
             dg=np.zeros_like(g), dS_in=np.zeros((B, H, dk, dv)))
    rc = lib.ref_gla_bwd(B, T, H, dk, dv, _p(q), _p(k), _p(v), _p(g), _p(S_in),
                         _p(dO), _p(dS_out), _p(r["dq"]), _p(r["dk"]), _p(r["dv"]),
                         _p(r["dg"]), _p(r["dS_in"]))
    if rc != 0:
        raise RuntimeError("ref_gla_bwd failed")
    return r


def mamba2_fwd(q, k, v, g, S_in=None, lib=None):
    """Scalar-gate (Mamba-2) chunk forward, g [B,T,H]: returns (o, S_out)."""
    lib = lib or load()
    q, k, v, g, S_in = map(_c, (q, k, v, g, S_in))
    B, T, H, dk, dv = _dims(q, v)
    o = np.zeros((B, T, H, dv))
    S_out = np.zeros((B, H, dk, dv))
    rc = lib.ref_m2_fwd(B, T, H, dk, dv, _p(q), _p(k), _p(v), _p(g), _p(S_in),
                        _p(o), _p(S_out))
    if rc != 0:
        raise RuntimeError("ref_m2_fwd failed")
    return o, S_out


def mamba2_bwd(q, k, v, g, S_in, dO, dS_out=None, lib=None):
    """Scalar-gate (Mamba-2) chunk backward: returns dict dq, dk, dv, dg, dS_in."""
    lib = lib or load()
    q, k, v, g, S_in, dO, dS_out = map(_c, (q, k, v, g, S_in, dO, dS_out))
    B, T, H, dk, dv = _dims(q, v)
    r = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v),
             dg=np.zeros((B, T, H)), dS_in=np.zeros((B, H, dk, dv)))
    rc = lib.ref_m2_bwd(B, T, H, dk, dv, _p(q), _p(k), _p(v), _p(g), _p(S_in),
                        _p(dO), _p(dS_out), _p(r["dq"]), _p(r["dk"]), _p(r["dv"]),
                        _p(r["dg"]), _p(r["dS_in"]))
    if rc != 0:
        raise RuntimeError("ref_m2_bwd failed")
    return r


def kda_fwd(q, k, v, g, beta, S_in=None, lib=None):
    """KDA chunk forward (per-channel gate g [B,T,H,dk], beta [B,T,H]):
    returns (o, S_out)."""
    lib = lib or load()
    q, k, v, g, beta, S_in = map(_c, (q, k, v, g, beta, S_in))
    B, T, H, dk, dv = _dims(q, v)
    o = np.zeros((B, T, H, dv))
    S_out = np.zeros((B, H, dk, dv))
    rc = lib.ref_kda_fwd(B, T, H, dk, dv, _p(q), _p(k), _p(v), _p(g), _p(beta),
                         _p(S_in), _p(o), _p(S_out))
    if rc != 0:
        raise RuntimeError("ref_kda_fwd failed")
    return o, S_out


def kda_bwd(q, k, v, g, beta, S_in, dO, dS_out=None, lib=None):
    """KDA chunk backward: returns dict dq, dk, dv, dg, dbeta, dS_in."""
    lib = lib or load()
    q, k, v, g, beta, S_in, dO, dS_out = map(_c, (q, k, v, g, beta, S_in, dO, dS_out))
    B, T, H, dk, dv = _dims(q, v)
    r = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v),
             dg=np.zeros_like(g), dbeta=np.zeros((B, T, H)), dS_in=np.zeros((B, H, dk, dv)))
    rc = lib.ref_kda_bwd(B, T, H, dk, dv, _p(q), _p(k), _p(v), _p(g), _p(beta),
                         _p(S_in), _p(dO), _p(dS_out), _p(r["dq"]), _p(r["dk"]),
                         _p(r["dv"]), _p(r["dg"]), _p(r["dbeta"]), _p(r["dS_in"]))
    if rc != 0:
        raise RuntimeError("ref_kda_bwd failed")
    return r


# ---------------------------------------------------------------------------
# Sequence-chunk chaining (StateFlow paper, Sec. 3.1, Eqs. 3, 4 and 6, with
# the chain rules S_{i+1}^in = S_i^out and dS_i^out = dS_{i+1}^in).
# ---------------------------------------------------------------------------

def _split_bounds(T, N):
    if T % N:
        raise ValueError("T must be divisible by N")
    L = T // N
    return [(i * L, (i + 1) * L) for i in range(N)]


def gdn_chunked(q, k, v, g, beta, S_in, dO, dS_out, N, lib=None):
    """Run fwd over N sequence chunks in order and bwd in reverse order,
    passing the boundary state and its gradient.  Returns (o, S_out, grads)."""
    B, T, H, dk, dv = _dims(q, v)
    bounds = _split_bounds(T, N)
    S = S_in
    states, outs = [], []
    for a, b in bounds:
        states.append(S)
        o_i, S = gdn_fwd(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b], S, lib=lib)
        outs.append(o_i)
    S_out = S
    dS = dS_out
    parts = [None] * N
    for i in reversed(range(N)):
        a, b = bounds[i]
        r = gdn_bwd(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b], states[i],
                    dO[:, a:b], dS, lib=lib)
        parts[i] = r
        dS = r["dS_in"]
    grads = {key: np.concatenate([p[key] for p in parts], axis=1)
             for key in ("dq", "dk", "dv", "dg", "dbeta")}
    grads["dS_in"] = dS
    return np.concatenate(outs, axis=1), S_out, grads


def gla_chunked(q, k, v, g, S_in, dO, dS_out, N, lib=None):
    B, T, H, dk, dv = _dims(q, v)
    bounds = _split_bounds(T, N)
    S = S_in
    states, outs = [], []
    for a, b in bounds:
        states.append(S)
        o_i, S = gla_fwd(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], S, lib=lib)
        outs.append(o_i)
    S_out = S
    dS = dS_out
    parts = [None] * N
    for i in reversed(range(N)):
        a, b = bounds[i]
        r = gla_bwd(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], states[i], dO[:, a:b], dS, lib=lib)
        parts[i] = r
        dS = r["dS_in"]
    grads = {key: np.concatenate([p[key] for p in parts], axis=1)
             for key in ("dq", "dk", "dv", "dg")}
    grads["dS_in"] = dS
    return np.concatenate(outs, axis=1), S_out, grads


def mamba2_chunked(q, k, v, g, S_in, dO, dS_out, N, lib=None):
    B, T, H, dk, dv = _dims(q, v)
    bounds = _split_bounds(T, N)
    S = S_in
    states, outs = [], []
    for a, b in bounds:
        states.append(S)
        o_i, S = mamba2_fwd(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], S, lib=lib)
        outs.append(o_i)
    S_out = S
    dS = dS_out
    parts = [None] * N
    for i in reversed(range(N)):
        a, b = bounds[i]
        r = mamba2_bwd(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], states[i], dO[:, a:b], dS, lib=lib)
        parts[i] = r
        dS = r["dS_in"]
    grads = {key: np.concatenate([p[key] for p in parts], axis=1)
             for key in ("dq", "dk", "dv", "dg")}
    grads["dS_in"] = dS
    return np.concatenate(outs, axis=1), S_out, grads


def kda_chunked(q, k, v, g, beta, S_in, dO, dS_out, N, lib=None):
    """KDA over N sequence chunks: forward in order, backward in reverse,
    with the boundary state and its gradient handed over (as gdn_chunked)."""
    B, T, H, dk, dv = _dims(q, v)
    bounds = _split_bounds(T, N)
    S = S_in
    states, outs = [], []
    for a, b in bounds:
        states.append(S)
        o_i, S = kda_fwd(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b], S, lib=lib)
        outs.append(o_i)
    S_out = S
    dS = dS_out
    parts = [None] * N
    for i in reversed(range(N)):
        a, b = bounds[i]
        r = kda_bwd(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b], states[i],
                    dO[:, a:b], dS, lib=lib)
        parts[i] = r
        dS = r["dS_in"]
    grads = {key: np.concatenate([p[key] for p in parts], axis=1)
             for key in ("dq", "dk", "dv", "dg", "dbeta")}
    grads["dS_in"] = dS
    return np.concatenate(outs, axis=1), S_out, grads
