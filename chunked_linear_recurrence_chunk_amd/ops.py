"""Thin ctypes binding of ``libclr.so`` (the C ABI declared in include/clr.h).

Argument marshalling only: every step of the layer runs in the HIP kernels.
Tensors are torch tensors on the GPU (torch supplies device memory and the
current stream); the functions allocate the outputs and the workspace and
enqueue one library call on ``torch.cuda.current_stream()``.

If the library is missing, loading raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libclr.so")

CLR_OK, CLR_EINVAL, CLR_ENOTSUP, CLR_EWORKSPACE, CLR_EHIP, CLR_ESCRATCH, CLR_ERANGE = range(7)
NOALLOC_SCRATCH_BYTES = 64 << 20  # CLR_NOALLOC_SCRATCH_BYTES
CLR_F32, CLR_BF16 = 0, 1
OP_GDN_FWD, OP_GDN_BWD, OP_GLA_FWD, OP_GLA_BWD, OP_M2_FWD, OP_M2_BWD, OP_KDA_FWD, OP_KDA_BWD = range(8)


class ClrShape(ctypes.Structure):
    # chunk: the kernel-level block (0 = the library's 64 tokens)
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("chunk", ctypes.c_int32)]


class ClrConvShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("C", ctypes.c_int32),
                ("W", ctypes.c_int32), ("dtype", ctypes.c_int32), ("act", ctypes.c_int32)]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int), ("total_ms", ctypes.c_double)]


class ClrError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: status {status} ({msg})")
        self.status = status


_lib = None


def load(path: Optional[str] = None):
    """Load libclr.so (raises OSError if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise OSError(f"{p} not found: build it with `python -m chunked_linear_recurrence_chunk_amd.build`")
    lib = ctypes.CDLL(p)
    vp, sz, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    sp = ctypes.POINTER(ClrShape)
    lib.clr_workspace_bytes.argtypes = [sp, i]
    lib.clr_workspace_bytes.restype = sz
    for name in ("gdn_fwd", "gla_fwd", "mamba2_fwd", "kda_fwd"):
        f = getattr(lib, name)
        f.argtypes = [sp] + [vp] * 9 + [sz, vp]
        f.restype = i
    lib.gdn_fwd_noalloc.argtypes = [sp] + [vp] * 9
    lib.gdn_fwd_noalloc.restype = i
    if hasattr(lib, "gdn_fwd_save"):  # saved-activation pair (absent from older builds)
        lib.clr_saved_bytes.argtypes = [sp]
        lib.clr_saved_bytes.restype = sz
        lib.gdn_fwd_save.argtypes = [sp] + [vp] * 9 + [sz, vp, sz, vp]
        lib.gdn_fwd_save.restype = i
        lib.gdn_bwd_saved.argtypes = [sp] + [vp] * 9 + [sz] + [vp] * 7 + [sz, vp]
        lib.gdn_bwd_saved.restype = i
    if hasattr(lib, "gla_fwd_save"):  # the GLA and Mamba-2 saved-activation pairs
        lib.clr_saved_bytes_op.argtypes = [sp, i]
        lib.clr_saved_bytes_op.restype = sz
        for name in ("gla_fwd_save", "mamba2_fwd_save", "kda_fwd_save"):
            getattr(lib, name).argtypes = [sp] + [vp] * 9 + [sz, vp, sz, vp]
            getattr(lib, name).restype = i
        for name in ("gla_bwd_saved", "mamba2_bwd_saved", "kda_bwd_saved"):
            getattr(lib, name).argtypes = [sp] + [vp] * 9 + [sz] + [vp] * 7 + [sz, vp]
            getattr(lib, name).restype = i
    for name in ("gdn_bwd", "gla_bwd", "mamba2_bwd", "kda_bwd"):
        f = getattr(lib, name)
        f.argtypes = [sp] + [vp] * 15 + [sz, vp]
        f.restype = i
    cp = ctypes.POINTER(ClrConvShape)
    lib.clr_range_status.argtypes = [sp, i, vp, vp]
    lib.clr_range_status.restype = i
    lib.clr_shortconv_workspace_bytes.argtypes = [cp]
    lib.clr_shortconv_workspace_bytes.restype = sz
    lib.shortconv_fwd.argtypes = [cp] + [vp] * 7
    lib.shortconv_fwd.restype = i
    lib.shortconv_bwd.argtypes = [cp] + [vp] * 10 + [i, vp, sz, vp]
    lib.shortconv_bwd.restype = i
    lib.clr_set_fwd_split.argtypes = [i]
    lib.clr_set_fwd_split.restype = i
    lib.clr_get_fwd_split.argtypes = []
    lib.clr_get_fwd_split.restype = i
    lib.clr_set_scan_bv.argtypes = [i]
    lib.clr_set_scan_bv.restype = i
    lib.clr_get_scan_bv.argtypes = []
    lib.clr_get_scan_bv.restype = i
    lib.clr_status_string.argtypes = [i]
    lib.clr_status_string.restype = ctypes.c_char_p
    lib.clr_version.argtypes = []
    lib.clr_version.restype = i
    lib.clr_probe_mma.argtypes = [i, vp, vp, vp, vp]
    lib.clr_probe_mma.restype = i
    lib.clr_timing_enable.argtypes = [i]
    lib.clr_timing_enable.restype = i
    lib.clr_timing_report.argtypes = [ctypes.POINTER(KernelTime), i]
    lib.clr_timing_report.restype = i
    if path is None:
        _lib = lib
    return lib


def status_string(s: int) -> str:
    return load().clr_status_string(int(s)).decode()


def _check(fn, rc):
    if rc != CLR_OK:
        raise ClrError(fn, rc, status_string(rc))


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return CLR_BF16
    if t.dtype == torch.float32:
        return CLR_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def make_shape(q, v, dtype_code=None) -> ClrShape:
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    return ClrShape(B, T, H, dk, dv, _dtype_code(q) if dtype_code is None else dtype_code)


def workspace_bytes(shape: ClrShape, op: int) -> int:
    return int(load().clr_workspace_bytes(ctypes.byref(shape), op))


def _workspace(shape, op, device):
    import torch
    n = workspace_bytes(shape, op)
    # torch's caching allocator returns 512-byte aligned blocks
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device), n


# gate layout per member: one value per (token, head), or one per key channel
_GATE_PER_CHANNEL = {"gdn": False, "mamba2": False, "gla": True, "kda": True}
_HAS_BETA = {"gdn": True, "kda": True, "gla": False, "mamba2": False}


def _validate(kind, q, k, v, g, beta, S_in, dO=None, dS_out=None):
    """Shapes and dtypes of a layer call against (B, T, H, dk, dv) from q and v
    (ValueError for a shape, TypeError for a dtype), before anything reaches
    the library: the C ABI takes bare pointers and cannot see a wrong size."""
    import torch
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q and v must be [B, T, H, d]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"unsupported dtype {q.dtype}")
    want = {"k": (k, (B, T, H, dk)), "v": (v, (B, T, H, dv)),
            "g": (g, (B, T, H, dk) if _GATE_PER_CHANNEL[kind] else (B, T, H))}
    if _HAS_BETA[kind]:
        want["beta"] = (beta, (B, T, H))
    elif beta is not None:
        raise ValueError(f"{kind} takes no beta")
    if dO is not None:
        want["dO"] = (dO, (B, T, H, dv))
    for name, (t, shp) in want.items():
        if t is None:
            raise ValueError(f"{name} is required")
        if tuple(t.shape) != shp:
            raise ValueError(f"{name} must have shape {shp}, got {tuple(t.shape)}")
        if t.dtype != q.dtype:
            raise TypeError(f"{name} must be {q.dtype} like q, got {t.dtype}")
    for name, t in (("S_in", S_in), ("dS_out", dS_out)):
        if t is None:
            continue
        if tuple(t.shape) != (B, H, dk, dv):
            raise ValueError(f"{name} must have shape {(B, H, dk, dv)}, got {tuple(t.shape)}")
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32 (states are fp32), got {t.dtype}")


def _check_inputs(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def set_fwd_split(permille: int) -> None:
    """Split point of the split-and-overlap GDN forward (per mille of the
    blocks in the first part; 0 disables the split)."""
    _check("clr_set_fwd_split", load().clr_set_fwd_split(int(permille)))


def get_fwd_split() -> int:
    return int(load().clr_get_fwd_split())


def set_scan_bv(bv: int) -> None:
    """Value-tile width of the Gated DeltaNet forward state scan: 16 or 32
    (clr_set_scan_bv)."""
    _check("clr_set_scan_bv", load().clr_set_scan_bv(int(bv)))


def get_scan_bv() -> int:
    return int(load().clr_get_scan_bv())


def timing_enable(on: bool = True) -> None:
    """Time every library kernel with start/stop events (profiling aid)."""
    load().clr_timing_enable(1 if on else 0)


def timing_report() -> dict:
    """Wait for the timed kernels and return {name: (launches, total_ms)}; clears."""
    buf = (KernelTime * 64)()
    n = load().clr_timing_report(buf, 64)
    if n < 0:
        raise ClrError("clr_timing_report", -n, status_string(-n))
    return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms) for i in range(n)}


def _out(t, shape, dtype, device):
    import torch
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"output tensor must be contiguous {dtype} of shape {shape}")
    return t


def range_status(shape: ClrShape, op: int, ws) -> int:
    """clr_range_status: CLR_OK if the gates of the last GLA / KDA / Mamba-2
    call of ``op`` at ``shape`` on workspace ``ws`` stayed within the diagonal
    tiles' decay bound, CLR_ERANGE if not (waits for the current stream).
    The GLA, KDA and Mamba-2 wrappers take ``check_range=True`` to raise
    ClrError with CLR_ERANGE after the call in that case."""
    return int(load().clr_range_status(ctypes.byref(shape), op, _ptr(ws), _stream()))


def _range_check(name, shape, op, ws, check_range):
    if check_range:
        _check(name, range_status(shape, op, ws))


def _fwd(name, op, q, k, v, g, beta, S_in, want_state, ws, o=None, S_out=None, check_range=False):
    import torch
    _validate(name.split("_")[0], q, k, v, g, beta, S_in)
    _check_inputs(q, k, v, g, beta, S_in)
    shape = make_shape(q, v)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = _out(o, (B, T, H, dv), q.dtype, q.device)
    if want_state or S_out is not None:
        S_out = _out(S_out, (B, H, dk, dv), torch.float32, q.device)
    if ws is None:
        ws, n = _workspace(shape, op, q.device)
    else:
        n = ws.numel()
    rc = getattr(load(), name)(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                               _ptr(S_in), _ptr(o), _ptr(S_out), _ptr(ws), n, _stream())
    _check(name, rc)
    _range_check(name, shape, op, ws, check_range)
    return o, S_out


def gdn_fwd(q, k, v, g, beta, S_in=None, want_state=True, ws=None, o=None, S_out=None):
    """Gated DeltaNet chunk forward.  Returns (o, S_out).  ``o`` / ``S_out``
    may be preallocated contiguous outputs (e.g. views of a larger tensor)."""
    return _fwd("gdn_fwd", OP_GDN_FWD, q, k, v, g, beta, S_in, want_state, ws, o, S_out)


def gdn_fwd_noalloc(q, k, v, g, beta, S_in=None, o=None, S_out=None):
    """gdn_fwd through the allocation-free entry point: the library's static
    scratch replaces the workspace, so the call itself allocates nothing on
    the device once ``o`` and ``S_out`` are given (they are allocated here
    otherwise).  Returns (o, S_out); raises ClrError with CLR_ESCRATCH when the
    shape needs more than NOALLOC_SCRATCH_BYTES of workspace."""
    import torch
    _validate("gdn", q, k, v, g, beta, S_in)
    _check_inputs(q, k, v, g, beta, S_in)
    shape = make_shape(q, v)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = _out(o, (B, T, H, dv), q.dtype, q.device)
    S_out = _out(S_out, (B, H, dk, dv), torch.float32, q.device)
    rc = load().gdn_fwd_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                _ptr(S_in), _ptr(o), _ptr(S_out), _stream())
    _check("gdn_fwd_noalloc", rc)
    return o, S_out


def saved_bytes(shape: ClrShape, op: int = None) -> int:
    """Bytes of one chunk call's saved activations: clr_saved_bytes (the Gated
    DeltaNet pair: the states entering its blocks and their U) or, with ``op``,
    clr_saved_bytes_op for the member that op names (GLA, Mamba-2: the
    states; KDA: the states and U)."""
    if op is None:
        return int(load().clr_saved_bytes(ctypes.byref(shape)))
    return int(load().clr_saved_bytes_op(ctypes.byref(shape), op))


def _fwd_save(name, op, q, k, v, g, beta, S_in, saved, ws, o, S_out, check_range=False):
    import torch
    _validate(name.split("_")[0], q, k, v, g, beta, S_in)
    _check_inputs(q, k, v, g, beta, S_in)
    shape = make_shape(q, v)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = _out(o, (B, T, H, dv), q.dtype, q.device)
    S_out = _out(S_out, (B, H, dk, dv), torch.float32, q.device)
    ns = saved_bytes(shape, op)
    if saved is None:
        saved = torch.empty(max(ns, 256), dtype=torch.uint8, device=q.device)
    if ws is None:
        ws, n = _workspace(shape, op, q.device)
    else:
        n = ws.numel()
    rc = getattr(load(), name)(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S_in),
                               _ptr(o), _ptr(S_out), _ptr(saved), saved.numel(), _ptr(ws), n, _stream())
    _check(name, rc)
    _range_check(name, shape, op, ws, check_range)
    return o, S_out, saved


def _bwd_saved(name, op, q, k, v, g, beta, S_in, dO, dS_out, saved, ws, out, check_range=False):
    import torch
    _validate(name.split("_")[0], q, k, v, g, beta, S_in, dO, dS_out)
    _check_inputs(q, k, v, g, beta, S_in, dO, dS_out, saved)
    shape = make_shape(q, v)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    out = out or {}
    dq = _out(out.get("dq"), q.shape, q.dtype, q.device)
    dk_ = _out(out.get("dk"), k.shape, k.dtype, k.device)
    dv_ = _out(out.get("dv"), v.shape, v.dtype, v.device)
    dg = _out(out.get("dg"), g.shape, g.dtype, g.device)
    dbeta = _out(out.get("dbeta"), beta.shape, beta.dtype, beta.device) if beta is not None else None
    dS_in = _out(out.get("dS_in"), (B, H, dk, dv), torch.float32, q.device)
    if ws is None:
        ws, n = _workspace(shape, op, q.device)
    else:
        n = ws.numel()
    rc = getattr(load(), name)(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S_in),
                               _ptr(dO), _ptr(dS_out), _ptr(saved), saved.numel(), _ptr(dq), _ptr(dk_), _ptr(dv_),
                               _ptr(dg), _ptr(dbeta), _ptr(dS_in), _ptr(ws), n, _stream())
    _check(name, rc)
    _range_check(name, shape, op, ws, check_range)
    r = dict(dq=dq, dk=dk_, dv=dv_, dg=dg, dS_in=dS_in)
    if dbeta is not None:
        r["dbeta"] = dbeta
    return r


def gdn_fwd_save(q, k, v, g, beta, S_in=None, saved=None, ws=None, o=None, S_out=None):
    """gdn_fwd that also keeps the activations the backward needs (gdn_fwd_save):
    returns (o, S_out, saved), ``saved`` a uint8 device tensor to hand to
    gdn_bwd_saved for the same chunk (allocated here unless given)."""
    return _fwd_save("gdn_fwd_save", OP_GDN_FWD, q, k, v, g, beta, S_in, saved, ws, o, S_out)


def gdn_bwd_saved(q, k, v, g, beta, S_in, dO, dS_out, saved, ws=None, out=None):
    """gdn_bwd reading the activations gdn_fwd_save kept for this chunk instead
    of recomputing the forward (S_in is not read and may be None).  Returns
    dict dq, dk, dv, dg, dbeta, dS_in."""
    return _bwd_saved("gdn_bwd_saved", OP_GDN_BWD, q, k, v, g, beta, S_in, dO, dS_out, saved, ws, out)


def gla_fwd_save(q, k, v, g, S_in=None, saved=None, ws=None, o=None, S_out=None, check_range=False):
    """gla_fwd that also keeps the states the backward needs (gla_fwd_save):
    returns (o, S_out, saved) for gla_bwd_saved of the same chunk."""
    return _fwd_save("gla_fwd_save", OP_GLA_FWD, q, k, v, g, None, S_in, saved, ws, o, S_out, check_range)


def gla_bwd_saved(q, k, v, g, S_in, dO, dS_out, saved, ws=None, out=None, check_range=False):
    """gla_bwd reading the states gla_fwd_save kept (S_in is not read and may
    be None).  Returns dict dq, dk, dv, dg, dS_in."""
    return _bwd_saved("gla_bwd_saved", OP_GLA_BWD, q, k, v, g, None, S_in, dO, dS_out, saved, ws, out,
                      check_range)


def kda_fwd_save(q, k, v, g, beta, S_in=None, saved=None, ws=None, o=None, S_out=None, check_range=False):
    """kda_fwd that also keeps the states and U the backward needs: returns
    (o, S_out, saved) for kda_bwd_saved of the same chunk."""
    return _fwd_save("kda_fwd_save", OP_KDA_FWD, q, k, v, g, beta, S_in, saved, ws, o, S_out, check_range)


def kda_bwd_saved(q, k, v, g, beta, S_in, dO, dS_out, saved, ws=None, out=None, check_range=False):
    """kda_bwd reading what kda_fwd_save kept (S_in is not read and may be
    None).  Returns dict dq, dk, dv, dg, dbeta, dS_in."""
    return _bwd_saved("kda_bwd_saved", OP_KDA_BWD, q, k, v, g, beta, S_in, dO, dS_out, saved, ws, out,
                      check_range)


def mamba2_fwd_save(q, k, v, g, S_in=None, saved=None, ws=None, o=None, S_out=None, check_range=False):
    """mamba2_fwd that also keeps the states the backward needs: returns
    (o, S_out, saved) for mamba2_bwd_saved of the same chunk."""
    return _fwd_save("mamba2_fwd_save", OP_M2_FWD, q, k, v, g, None, S_in, saved, ws, o, S_out, check_range)


def mamba2_bwd_saved(q, k, v, g, S_in, dO, dS_out, saved, ws=None, out=None, check_range=False):
    """mamba2_bwd reading the states mamba2_fwd_save kept (S_in is not read
    and may be None).  Returns dict dq, dk, dv, dg, dS_in."""
    return _bwd_saved("mamba2_bwd_saved", OP_M2_BWD, q, k, v, g, None, S_in, dO, dS_out, saved, ws, out,
                      check_range)


def gla_fwd(q, k, v, g, S_in=None, want_state=True, ws=None, o=None, S_out=None, check_range=False):
    """GLA chunk forward (per-key-channel gate g).  Returns (o, S_out)."""
    return _fwd("gla_fwd", OP_GLA_FWD, q, k, v, g, None, S_in, want_state, ws, o, S_out, check_range)


def _bwd(name, op, q, k, v, g, beta, S_in, dO, dS_out, ws, out=None, check_range=False):
    import torch
    _validate(name.split("_")[0], q, k, v, g, beta, S_in, dO, dS_out)
    _check_inputs(q, k, v, g, beta, S_in, dO, dS_out)
    shape = make_shape(q, v)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    out = out or {}
    dq = _out(out.get("dq"), q.shape, q.dtype, q.device)
    dk_ = _out(out.get("dk"), k.shape, k.dtype, k.device)
    dv_ = _out(out.get("dv"), v.shape, v.dtype, v.device)
    dg = _out(out.get("dg"), g.shape, g.dtype, g.device)
    dbeta = _out(out.get("dbeta"), beta.shape, beta.dtype, beta.device) if beta is not None else None
    dS_in = _out(out.get("dS_in"), (B, H, dk, dv), torch.float32, q.device)
    if ws is None:
        ws, n = _workspace(shape, op, q.device)
    else:
        n = ws.numel()
    rc = getattr(load(), name)(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                               _ptr(S_in), _ptr(dO), _ptr(dS_out), _ptr(dq), _ptr(dk_), _ptr(dv_),
                               _ptr(dg), _ptr(dbeta), _ptr(dS_in), _ptr(ws), n, _stream())
    _check(name, rc)
    _range_check(name, shape, op, ws, check_range)
    r = dict(dq=dq, dk=dk_, dv=dv_, dg=dg, dS_in=dS_in)
    if dbeta is not None:
        r["dbeta"] = dbeta
    return r


def gdn_bwd(q, k, v, g, beta, S_in, dO, dS_out=None, ws=None, out=None):
    """Gated DeltaNet chunk backward.  Returns dict dq, dk, dv, dg, dbeta, dS_in
    (``out`` may hold preallocated contiguous tensors under those names)."""
    return _bwd("gdn_bwd", OP_GDN_BWD, q, k, v, g, beta, S_in, dO, dS_out, ws, out)


def gla_bwd(q, k, v, g, S_in, dO, dS_out=None, ws=None, out=None, check_range=False):
    """GLA chunk backward.  Returns dict dq, dk, dv, dg, dS_in."""
    return _bwd("gla_bwd", OP_GLA_BWD, q, k, v, g, None, S_in, dO, dS_out, ws, out, check_range)


def kda_fwd(q, k, v, g, beta, S_in=None, want_state=True, ws=None, o=None, S_out=None, check_range=False):
    """KDA chunk forward (per-key-channel gate g [B,T,H,dk], beta [B,T,H]).
    Returns (o, S_out)."""
    return _fwd("kda_fwd", OP_KDA_FWD, q, k, v, g, beta, S_in, want_state, ws, o, S_out, check_range)


def kda_bwd(q, k, v, g, beta, S_in, dO, dS_out=None, ws=None, out=None, check_range=False):
    """KDA chunk backward.  Returns dict dq, dk, dv, dg, dbeta, dS_in."""
    return _bwd("kda_bwd", OP_KDA_BWD, q, k, v, g, beta, S_in, dO, dS_out, ws, out, check_range)


def mamba2_fwd(q, k, v, g, S_in=None, want_state=True, ws=None, o=None, S_out=None, check_range=False):
    """Scalar-gate (Mamba-2 member) chunk forward, g [B,T,H].  Returns (o, S_out)."""
    return _fwd("mamba2_fwd", OP_M2_FWD, q, k, v, g, None, S_in, want_state, ws, o, S_out, check_range)


def mamba2_bwd(q, k, v, g, S_in, dO, dS_out=None, ws=None, out=None, check_range=False):
    """Scalar-gate (Mamba-2 member) chunk backward.  Returns dict dq, dk, dv, dg, dS_in."""
    return _bwd("mamba2_bwd", OP_M2_BWD, q, k, v, g, None, S_in, dO, dS_out, ws, out, check_range)


def _conv_shape(x, w, act):
    B, T, C = x.shape
    return ClrConvShape(B, T, C, w.shape[1], _dtype_code(x), int(act))


def shortconv_workspace_bytes(shape: ClrConvShape) -> int:
    return int(load().clr_shortconv_workspace_bytes(ctypes.byref(shape)))


def shortconv_fwd(x, w, bias=None, state_in=None, act=0, want_state=True, y=None, state_out=None):
    """Causal short convolution with boundary state.  x [B,T,C] (bf16/fp32),
    w [C,W] and bias [C] float32, state_in [B,W-1,C].  Returns (y, state_out)."""
    import torch
    _check_inputs(x, w, bias, state_in)
    shape = _conv_shape(x, w, act)
    B, T, C = x.shape
    W = w.shape[1]
    if w.dtype != torch.float32 or (bias is not None and bias.dtype != torch.float32):
        raise TypeError("w and bias must be float32")
    y = _out(y, (B, T, C), x.dtype, x.device)
    if want_state or state_out is not None:
        state_out = _out(state_out, (B, W - 1, C), x.dtype, x.device)
    rc = load().shortconv_fwd(ctypes.byref(shape), _ptr(x), _ptr(w), _ptr(bias), _ptr(state_in), _ptr(y),
                              _ptr(state_out), _stream())
    _check("shortconv_fwd", rc)
    return y, state_out


def shortconv_bwd(x, w, bias, state_in, dy, dstate_out=None, act=0, accumulate=False, out=None, ws=None):
    """Gradients of shortconv_fwd: dict dx, dw, dbias (None without bias),
    dstate_in (float32; dstate_out is float32 too).  With accumulate=True,
    out["dw"] / out["dbias"] are added to."""
    import torch
    _check_inputs(x, w, bias, state_in, dy, dstate_out)
    shape = _conv_shape(x, w, act)
    B, T, C = x.shape
    W = w.shape[1]
    out = out or {}
    dx = _out(out.get("dx"), (B, T, C), x.dtype, x.device)
    dw = _out(out.get("dw"), (C, W), torch.float32, x.device)
    dbias = _out(out.get("dbias"), (C,), torch.float32, x.device) if bias is not None else None
    dstate_in = _out(out.get("dstate_in"), (B, W - 1, C), torch.float32, x.device)
    if dstate_out is not None and dstate_out.dtype != torch.float32:
        raise TypeError("dstate_out must be float32")
    n = shortconv_workspace_bytes(shape)
    if ws is None or ws.numel() < n:
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device=x.device)
    rc = load().shortconv_bwd(ctypes.byref(shape), _ptr(x), _ptr(w), _ptr(bias), _ptr(state_in), _ptr(dy),
                              _ptr(dstate_out), _ptr(dx), _ptr(dw), _ptr(dbias),
                              _ptr(dstate_in) if W > 1 else None, 1 if accumulate else 0, _ptr(ws),
                              ws.numel(), _stream())
    _check("shortconv_bwd", rc)
    return dict(dx=dx, dw=dw, dbias=dbias, dstate_in=dstate_in)


def probe_mma(A, Bt):
    """C = A @ Bt.T (16x32 each) through the kernels' fragment layout, plus the
    same product through the accumulator-chaining path (rows 16..31 of C)."""
    import torch
    _check_inputs(A, Bt)
    C = torch.empty((32, 16), dtype=torch.float32, device=A.device)
    rc = load().clr_probe_mma(_dtype_code(A), _ptr(A), _ptr(Bt), _ptr(C), _stream())
    _check("clr_probe_mma", rc)
    return C
