"""The C-ABI library loads without a GPU, exports every symbol declared in
include/clr.h, and rejects bad arguments on the host before launching
anything (so these run on the CPU: every call here fails validation)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "clr.h")


def _lib():
    from chunked_linear_recurrence_chunk_amd import ops
    return ops, ops.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("gdn_fwd", "gdn_bwd", "gla_fwd", "gla_bwd", "clr_workspace_bytes", "clr_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol():
    ops, lib = _lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    ops, lib = _lib()
    assert lib.clr_version() >= 100
    for s in range(7):
        assert ops.status_string(s) != "unknown status"
    assert ops.status_string(7) == "unknown status"


def _shape(ops, B=1, T=128, H=2, dk=128, dv=128, dtype=1):
    return ops.ClrShape(B, T, H, dk, dv, dtype)


def test_fwd_split_setting():
    ops, lib = _lib()
    old = ops.get_fwd_split()
    assert 0 <= old < 1000
    assert lib.clr_set_fwd_split(-1) == ops.CLR_EINVAL
    assert lib.clr_set_fwd_split(1000) == ops.CLR_EINVAL
    assert ops.get_fwd_split() == old
    try:
        ops.set_fwd_split(0)
        assert ops.get_fwd_split() == 0
        ops.set_fwd_split(250)
        assert ops.get_fwd_split() == 250
    finally:
        ops.set_fwd_split(old)


def test_scan_bv_setting():
    ops, lib = _lib()
    old = ops.get_scan_bv()
    assert old in (16, 32)
    for bad in (0, 8, 24, 64, -16):
        assert lib.clr_set_scan_bv(bad) == ops.CLR_EINVAL
    assert ops.get_scan_bv() == old
    try:
        ops.set_scan_bv(32)
        assert ops.get_scan_bv() == 32
        ops.set_scan_bv(16)
        assert ops.get_scan_bv() == 16
    finally:
        ops.set_scan_bv(old)


def test_workspace_sizes():
    ops, lib = _lib()
    s = _shape(ops)
    f = ops.workspace_bytes(s, ops.OP_GDN_FWD)
    b = ops.workspace_bytes(s, ops.OP_GDN_BWD)
    assert 0 < f < b
    assert ops.workspace_bytes(_shape(ops, dk=96, dv=96), ops.OP_GDN_FWD) == 0      # unsupported
    assert ops.workspace_bytes(_shape(ops, dk=128, dv=256), ops.OP_GDN_FWD) == 0    # GDN needs dk == dv
    assert ops.workspace_bytes(_shape(ops, dk=128, dv=256), ops.OP_GLA_FWD) > 0
    assert ops.workspace_bytes(_shape(ops, dtype=0), ops.OP_GDN_BWD) == 0          # fp32 bwd only d=32
    assert ops.workspace_bytes(_shape(ops, dk=32, dv=32, dtype=0), ops.OP_GDN_BWD) > 0
    # linear in the number of 64-token blocks
    assert ops.workspace_bytes(_shape(ops, T=256), ops.OP_GDN_FWD) < 2.1 * ops.workspace_bytes(_shape(ops, T=128), ops.OP_GDN_FWD)


P = ctypes.c_void_p


def _fake(addr):
    return P(addr)


def _fwd(lib, ops, s, q=0x10000, k=0x20000, v=0x30000, g=0x40000, beta=0x50000, S_in=None, o=0x60000,
         S_out=0x70000, ws=0x100000, nws=1 << 40, name="gdn_fwd"):
    f = getattr(lib, name)
    args = [ctypes.byref(s)] + [None if a is None else _fake(a) for a in (q, k, v, g, beta, S_in, o, S_out, ws)]
    return f(*args, nws, None)


def test_validation_errors_are_returned_before_any_launch():
    ops, lib = _lib()
    s = _shape(ops, T=64, H=1, dk=32, dv=32)
    # the fake device addresses are never dereferenced: each call fails validation
    assert _fwd(lib, ops, s, q=None) == ops.CLR_EINVAL                     # null input
    assert _fwd(lib, ops, s, beta=None) == ops.CLR_EINVAL                  # GDN needs beta
    assert _fwd(lib, ops, s, q=0x10008) == ops.CLR_EINVAL                  # misaligned
    assert _fwd(lib, ops, s, o=0x10000) == ops.CLR_EINVAL                  # output aliases q
    assert _fwd(lib, ops, s, ws=None) == ops.CLR_EWORKSPACE                # no workspace
    assert _fwd(lib, ops, s, nws=16) == ops.CLR_EWORKSPACE                 # too small
    assert _fwd(lib, ops, s, ws=0x100010) == ops.CLR_EWORKSPACE            # workspace misaligned
    assert _fwd(lib, ops, _shape(ops, dk=96, dv=96)) == ops.CLR_ENOTSUP
    assert _fwd(lib, ops, _shape(ops, dtype=7)) == ops.CLR_ENOTSUP
    assert _fwd(lib, ops, _shape(ops, B=0)) == ops.CLR_EINVAL
    assert _fwd(lib, ops, _shape(ops, T=-1)) == ops.CLR_EINVAL
    # GLA rejects beta
    assert _fwd(lib, ops, _shape(ops, dk=128, dv=256), name="gla_fwd") == ops.CLR_EINVAL
    assert lib.gdn_fwd(None, *([None] * 9), 0, None) == ops.CLR_EINVAL


def test_bwd_validation():
    ops, lib = _lib()
    s = _shape(ops, T=64, H=1, dk=32, dv=32)
    ptrs = [_fake(0x10000 * (i + 1)) for i in range(14)] + [_fake(0x1000000)]
    bad = list(ptrs)
    bad[8] = None  # dq missing
    assert lib.gdn_bwd(ctypes.byref(s), *bad, 1 << 40, None) == ops.CLR_EINVAL
    bad = list(ptrs)
    bad[12] = None  # dbeta missing for GDN
    assert lib.gdn_bwd(ctypes.byref(s), *bad, 1 << 40, None) == ops.CLR_EINVAL
    bad = list(ptrs)
    bad[13] = bad[0]  # dS_in aliases q
    assert lib.gdn_bwd(ctypes.byref(s), *bad, 1 << 40, None) == ops.CLR_EINVAL
    # GLA: beta / dbeta must be NULL
    sg = _shape(ops, T=64, H=1, dk=32, dv=32)
    assert lib.gla_bwd(ctypes.byref(sg), *ptrs, 1 << 40, None) == ops.CLR_EINVAL
    # fp32 backward at d = 128 is not supported (d <= 64 is)
    s128 = _shape(ops, T=64, H=1, dk=128, dv=128, dtype=0)
    assert lib.gdn_bwd(ctypes.byref(s128), *ptrs, 1 << 40, None) == ops.CLR_ENOTSUP
    assert lib.kda_bwd(ctypes.byref(s128), *ptrs, 1 << 40, None) == ops.CLR_ENOTSUP
    # KDA needs beta and dbeta; its workspace is larger than the forward's
    bad = list(ptrs)
    bad[4] = None
    assert lib.kda_bwd(ctypes.byref(s), *bad, 1 << 40, None) == ops.CLR_EINVAL
    assert ops.workspace_bytes(s, ops.OP_KDA_BWD) > ops.workspace_bytes(s, ops.OP_KDA_FWD) > 0
    assert ops.workspace_bytes(s128, ops.OP_KDA_BWD) == 0 and ops.workspace_bytes(s128, ops.OP_KDA_FWD) == 0
    s64 = _shape(ops, T=64, H=1, dk=64, dv=64, dtype=0)
    assert ops.workspace_bytes(s64, ops.OP_KDA_BWD) > ops.workspace_bytes(s64, ops.OP_KDA_FWD) > 0


def test_mamba2_and_shortconv_validation():
    ops, lib = _lib()
    s = _shape(ops, T=64, H=1, dk=32, dv=32)
    assert _fwd(lib, ops, s, name="mamba2_fwd") == ops.CLR_EINVAL               # beta must be NULL
    assert _fwd(lib, ops, _shape(ops, dk=96, dv=96), beta=None, name="mamba2_fwd") == ops.CLR_ENOTSUP
    assert ops.workspace_bytes(_shape(ops, dk=128, dv=256), ops.OP_M2_BWD) == \
        ops.workspace_bytes(_shape(ops, dk=128, dv=256), ops.OP_GLA_BWD)
    cs = ops.ClrConvShape(2, 100, 64, 4, 1, 1)
    assert ops.shortconv_workspace_bytes(cs) > 0
    for bad in (ops.ClrConvShape(2, 100, 60, 4, 1, 1),   # C not a multiple of 8
                ops.ClrConvShape(2, 100, 64, 5, 1, 1),   # W > 4
                ops.ClrConvShape(2, 100, 64, 4, 1, 2),   # unknown activation
                ops.ClrConvShape(2, 100, 64, 4, 7, 1)):  # dtype
        assert ops.shortconv_workspace_bytes(bad) == 0
        assert lib.shortconv_fwd(ctypes.byref(bad), *[_fake(0x10000 * (i + 1)) for i in range(6)], None) == \
            ops.CLR_ENOTSUP
    f = [_fake(0x100000 * (i + 1)) for i in range(6)]
    assert lib.shortconv_fwd(ctypes.byref(cs), None, *f[1:], None) == ops.CLR_EINVAL     # x missing
    al = list(f)
    al[4] = al[0]                                                                   # y aliases x
    assert lib.shortconv_fwd(ctypes.byref(cs), *al, None) == ops.CLR_EINVAL
    b = [_fake(0x1000000 * (i + 1)) for i in range(10)]
    nws = ops.shortconv_workspace_bytes(cs)
    assert lib.shortconv_bwd(ctypes.byref(cs), *b, 0, _fake(0x20000000), nws - 256, None) == ops.CLR_EWORKSPACE
    assert lib.shortconv_bwd(ctypes.byref(cs), *b, 2, _fake(0x20000000), nws, None) == ops.CLR_EINVAL
    nb = list(b)
    nb[9] = None                                                                    # dstate_in needed (W > 1)
    assert lib.shortconv_bwd(ctypes.byref(cs), *nb, 0, _fake(0x20000000), nws, None) == ops.CLR_EINVAL


def test_product_path_has_no_oracle_or_fallback():
    """The package never imports the oracle and the binding refuses to run
    without the built library."""
    pkg = os.path.join(ROOT, "chunked_linear_recurrence_chunk_amd")
    for fn in os.listdir(pkg):
        if fn.endswith(".py"):
            src = open(os.path.join(pkg, fn)).read()
            assert not re.search(r"^\s*(from|import)\s+oracle", src, flags=re.M), fn
            assert "clr_oracle" not in src, fn
    from chunked_linear_recurrence_chunk_amd import ops
    with pytest.raises(OSError):
        ops.load(os.path.join(ROOT, "does_not_exist.so"))


def test_noalloc_forward_rejects_on_the_host():
    """The allocation-free forward validates like gdn_fwd and refuses shapes
    whose workspace exceeds its static scratch, before touching the GPU."""
    ops, lib = _lib()
    big = _shape(ops, T=2304, H=16)
    assert ops.workspace_bytes(big, ops.OP_GDN_FWD) > ops.NOALLOC_SCRATCH_BYTES
    # distinct, aligned, never dereferenced addresses: validation stops at the size
    fake = [ctypes.c_void_p((i + 1) << 30) for i in range(8)]
    assert lib.gdn_fwd_noalloc(ctypes.byref(big), *fake, None) == ops.CLR_ESCRATCH
    assert lib.gdn_fwd_noalloc(ctypes.byref(big), *([None] * 9)) == ops.CLR_EINVAL  # null tensors first
    fits = _shape(ops, T=2240, H=16)
    assert ops.workspace_bytes(fits, ops.OP_GDN_FWD) <= ops.NOALLOC_SCRATCH_BYTES
    assert lib.gdn_fwd_noalloc(ctypes.byref(fits), *([None] * 9)) == ops.CLR_EINVAL
    assert lib.gdn_fwd_noalloc(ctypes.byref(_shape(ops, dk=96, dv=96)), *([None] * 9)) == ops.CLR_ENOTSUP
    assert lib.gdn_fwd_noalloc(None, *([None] * 9)) == ops.CLR_EINVAL


def test_range_status_rejects_on_the_host():
    """clr_range_status validates shape, op and workspace before reading, and
    answers CLR_OK for the Gated DeltaNet ops without touching the workspace
    (no device call on any of these paths)."""
    ops, lib = _lib()
    sh = _shape(ops)
    fake = ctypes.c_void_p(1 << 30)
    for op in (ops.OP_GDN_FWD, ops.OP_GDN_BWD):
        assert lib.clr_range_status(ctypes.byref(sh), op, None, None) == ops.CLR_OK
    for op in (ops.OP_GLA_FWD, ops.OP_GLA_BWD, ops.OP_M2_FWD, ops.OP_M2_BWD, ops.OP_KDA_FWD, ops.OP_KDA_BWD):
        assert lib.clr_range_status(ctypes.byref(sh), op, None, None) == ops.CLR_EWORKSPACE
        assert lib.clr_range_status(ctypes.byref(sh), op, ctypes.c_void_p((1 << 30) + 8), None) == \
            ops.CLR_EWORKSPACE
        assert lib.clr_range_status(None, op, fake, None) == ops.CLR_EINVAL
        assert lib.clr_range_status(ctypes.byref(_shape(ops, dk=96, dv=96)), op, fake, None) == ops.CLR_ENOTSUP
        assert lib.clr_range_status(ctypes.byref(_shape(ops, T=0)), op, fake, None) == ops.CLR_OK  # no blocks
    for op in (-1, 8):
        assert lib.clr_range_status(ctypes.byref(sh), op, fake, None) == ops.CLR_EINVAL
    # the fp32 KDA backward exists for d <= 64
    f32 = _shape(ops, dk=128, dv=128, dtype=0)
    assert lib.clr_range_status(ctypes.byref(f32), ops.OP_KDA_BWD, fake, None) == ops.CLR_ENOTSUP


def test_binding_checks_shapes_and_dtypes_before_the_library():
    """ops.py compares every tensor with (B, T, H, dk, dv) taken from q and v,
    per member, so a wrong gate layout or a bf16 state never reaches the
    kernels as a short buffer (CPU tensors: the checks run before the device
    check)."""
    import torch
    ops, _ = _lib()
    B, T, H, dk, dv = 1, 64, 2, 32, 32
    bf = torch.bfloat16
    q = torch.zeros(B, T, H, dk, dtype=bf)
    k = torch.zeros(B, T, H, dk, dtype=bf)
    v = torch.zeros(B, T, H, dv, dtype=bf)
    g_tok = torch.zeros(B, T, H, dtype=bf)
    g_ch = torch.zeros(B, T, H, dk, dtype=bf)
    beta = torch.zeros(B, T, H, dtype=bf)
    S = torch.zeros(B, H, dk, dv)
    dO = torch.zeros(B, T, H, dv, dtype=bf)
    on_gpu = "must be on the GPU"

    def raises(exc, text, fn, *a):
        with pytest.raises(exc) as e:
            fn(*a)
        assert text in str(e.value), str(e.value)

    # well-formed calls get as far as the device check
    raises(ValueError, on_gpu, ops.gdn_fwd, q, k, v, g_tok, beta, S)
    raises(ValueError, on_gpu, ops.gla_fwd, q, k, v, g_ch, S)
    raises(ValueError, on_gpu, ops.kda_bwd, q, k, v, g_ch, beta, S, dO, S)
    raises(ValueError, on_gpu, ops.mamba2_bwd, q, k, v, g_tok, S, dO, None)
    # gate layouts: per (token, head) for GDN and Mamba-2, per key channel for GLA and KDA
    raises(ValueError, "g must have shape", ops.gla_fwd, q, k, v, g_tok, S)
    raises(ValueError, "g must have shape", ops.kda_fwd, q, k, v, g_tok, beta, S)
    raises(ValueError, "g must have shape", ops.gdn_bwd, q, k, v, g_ch, beta, S, dO, None)
    raises(ValueError, "g must have shape", ops.mamba2_fwd, q, k, v, g_ch, S)
    # beta: required for the delta rule, refused otherwise; [B, T, H]
    raises(ValueError, "beta is required", ops.gdn_fwd, q, k, v, g_tok, None, S)
    raises(ValueError, "beta must have shape", ops.kda_fwd, q, k, v, g_ch, g_ch, S)
    # k, v, dO shapes
    raises(ValueError, "k must have shape", ops.gdn_fwd, q, k[:, :32], v, g_tok, beta, S)
    raises(ValueError, "dO must have shape", ops.gdn_bwd, q, k, v, g_tok, beta, S, dO[..., :16], None)
    # dtypes: per-token tensors like q, states fp32
    raises(TypeError, "must be", ops.gdn_fwd, q, k.float(), v, g_tok, beta, S)
    raises(TypeError, "S_in must be float32", ops.gdn_fwd, q, k, v, g_tok, beta, S.to(bf))
    raises(TypeError, "dS_out must be float32", ops.gdn_bwd, q, k, v, g_tok, beta, S, dO, S.to(bf))
    raises(ValueError, "S_in must have shape", ops.gla_fwd, q, k, v, g_ch, S[:, :, :16])
    raises(ValueError, "dS_out must have shape", ops.gdn_bwd, q, k, v, g_tok, beta, S, dO, S[:1, :1])
    raises(TypeError, "unsupported dtype", ops.gdn_fwd, q.half(), k.half(), v.half(), g_tok.half(), beta.half(), S)
    raises(ValueError, "gla takes no beta", ops._fwd, "gla_fwd", ops.OP_GLA_FWD, q, k, v, g_ch, beta, S, True, None)
    raises(ValueError, "g must have shape", ops.gdn_fwd_noalloc, q, k, v, g_ch, beta, S)


def test_shape_chunk_field_and_unsupported_sizes():
    """The kernel-level block is 64 tokens (chunk 0 or 64); Gated DeltaNet at
    dk = dv = 256 and the fp32 backward beyond d = 64 are not built."""
    ops, lib = _lib()
    base = ops.workspace_bytes(_shape(ops), ops.OP_GDN_FWD)
    s64 = _shape(ops)
    s64.chunk = 64
    assert ops.workspace_bytes(s64, ops.OP_GDN_FWD) == base
    for bad in (16, 32, 128, -1):
        s = _shape(ops)
        s.chunk = bad
        assert ops.workspace_bytes(s, ops.OP_GDN_FWD) == 0
        assert lib.gdn_fwd(ctypes.byref(s), *([None] * 9), 0, None) == ops.CLR_ENOTSUP
    for op in (ops.OP_GDN_FWD, ops.OP_GDN_BWD, ops.OP_KDA_FWD, ops.OP_KDA_BWD):
        assert ops.workspace_bytes(_shape(ops, dk=256, dv=256), op) == 0
    s256 = _shape(ops, dk=256, dv=256)
    assert lib.gdn_fwd(ctypes.byref(s256), *([None] * 9), 0, None) == ops.CLR_ENOTSUP
    assert lib.gdn_bwd(ctypes.byref(s256), *([None] * 15), 0, None) == ops.CLR_ENOTSUP
    assert ops.workspace_bytes(_shape(ops, dk=128, dv=128, dtype=0), ops.OP_GDN_BWD) == 0
    for d in (32, 64):
        assert ops.workspace_bytes(_shape(ops, dk=d, dv=d, dtype=0), ops.OP_GDN_BWD) > 0


def test_saved_activation_entry_points_reject_on_the_host():
    ops, lib = _lib()
    s = _shape(ops, T=64, H=1, dk=32, dv=32)
    n = ops.saved_bytes(s)
    # one 64-token block: a 32 x 32 state and 64 x 32 values, bf16, 256-byte aligned parts
    assert n == 2048 + 4096
    assert ops.saved_bytes(_shape(ops, T=0)) == 0
    assert ops.saved_bytes(_shape(ops, dk=128, dv=128, dtype=0)) == 0   # no fp32 backward at d = 128
    assert ops.saved_bytes(_shape(ops, dk=96, dv=96)) == 0
    P_ = _fake
    # fwd: q k v g beta S_in o S_out | saved, nsaved | ws, nws
    base = [P_(0x10000), P_(0x20000), P_(0x30000), P_(0x40000), P_(0x50000), None, P_(0x60000), P_(0x70000)]

    def fwd(saved, nsaved, ws=0x100000, nws=1 << 40):
        return lib.gdn_fwd_save(ctypes.byref(s), *base, None if saved is None else P_(saved), nsaved,
                                None if ws is None else P_(ws), nws, None)
    assert fwd(None, 0) == ops.CLR_EWORKSPACE                    # no saved buffer
    assert fwd(0xA0000, n - 256) == ops.CLR_EWORKSPACE           # too small
    assert fwd(0xA0010, n) == ops.CLR_EWORKSPACE                 # misaligned
    assert fwd(0x60000, n) == ops.CLR_EINVAL                     # overlaps the output o
    assert fwd(0xFF000, n) == ops.CLR_EINVAL                     # overlaps the workspace
    assert fwd(0xA0000, n, ws=None) == ops.CLR_EWORKSPACE        # no workspace
    # bwd: q k v g beta S_in dO dS_out | saved, nsaved | dq dk dv dg dbeta dS_in | ws, nws
    outs = [P_(0x80000 + 0x10000 * i) for i in range(6)]

    def bwd(saved, nsaved, o=outs):
        return lib.gdn_bwd_saved(ctypes.byref(s), *base[:6], P_(0x60000), P_(0x70000),
                                 None if saved is None else P_(saved), nsaved, *o, P_(0x100000), 1 << 40, None)
    assert bwd(None, 0) == ops.CLR_EWORKSPACE
    assert bwd(0xF0000, n - 256) == ops.CLR_EWORKSPACE
    assert bwd(0xF0010, n) == ops.CLR_EWORKSPACE
    assert bwd(0x80000, n) == ops.CLR_EINVAL                     # overlaps the output dq
    bad = list(outs)
    bad[0] = None
    assert bwd(0xF0000, n, bad) == ops.CLR_EINVAL                # dq missing


@pytest.mark.parametrize("member", ["gla", "mamba2"])
def test_gla_saved_activation_entry_points_reject_on_the_host(member):
    """gla_* / mamba2_* with saved states: size query and host-side rejections
    (every call below fails validation, so nothing is launched)."""
    ops, lib = _lib()
    op_f, op_b = (ops.OP_GLA_FWD, ops.OP_GLA_BWD) if member == "gla" else (ops.OP_M2_FWD, ops.OP_M2_BWD)
    s = _shape(ops, T=64, H=1, dk=32, dv=32)
    n = ops.saved_bytes(s, op_f)
    assert n == 32 * 32 * 2 == ops.saved_bytes(s, op_b)           # one block: a 32 x 32 bf16 state
    assert ops.saved_bytes(_shape(ops, T=130, H=3, dk=128, dv=256), op_f) == 3 * 3 * 128 * 256 * 2
    assert ops.saved_bytes(_shape(ops, T=0), op_f) == 0
    assert ops.saved_bytes(_shape(ops, dk=128, dv=128, dtype=0), op_b) == 0   # no fp32 backward at d = 128
    assert ops.saved_bytes(_shape(ops, dk=96, dv=96), op_f) == 0
    # KDA keeps the states and U: the Gated DeltaNet pair's size
    assert ops.saved_bytes(s, ops.OP_KDA_FWD) == ops.saved_bytes(s, ops.OP_KDA_BWD) == ops.saved_bytes(s)
    assert ops.saved_bytes(_shape(ops, dk=128, dv=128, dtype=0), ops.OP_KDA_BWD) == 0  # fp32 KDA: d <= 64
    assert ops.saved_bytes(s, 99) == 0
    g16 = ops.ClrShape(1, 64, 1, 128, 128, 1)
    assert ops.saved_bytes(g16, ops.OP_GDN_FWD) == ops.saved_bytes(g16)
    P_ = _fake
    # fwd: q k v g beta(NULL) S_in o S_out | saved, nsaved | ws, nws
    base = [P_(0x10000), P_(0x20000), P_(0x30000), P_(0x40000), None, None, P_(0x60000), P_(0x70000)]
    fwd_f = getattr(lib, f"{member}_fwd_save")

    def fwd(saved, nsaved, ws=0x100000, nws=1 << 40):
        return fwd_f(ctypes.byref(s), *base, None if saved is None else P_(saved), nsaved,
                     None if ws is None else P_(ws), nws, None)
    assert fwd(None, 0) == ops.CLR_EWORKSPACE                    # no saved buffer
    assert fwd(0xA0000, n - 256) == ops.CLR_EWORKSPACE           # too small
    assert fwd(0xA0010, n) == ops.CLR_EWORKSPACE                 # misaligned
    assert fwd(0x60000, n) == ops.CLR_EINVAL                     # overlaps the output o
    assert fwd(0x100000 - n // 2, n) == ops.CLR_EINVAL           # overlaps the workspace
    assert fwd(0xA0000, n, ws=None) == ops.CLR_EWORKSPACE        # no workspace
    base_b = list(base)
    base_b[4] = P_(0x50000)
    assert fwd_f(ctypes.byref(s), *base_b, P_(0xA0000), n, P_(0x100000), 1 << 40, None) == ops.CLR_EINVAL  # beta given
    # bwd: q k v g beta(NULL) S_in dO dS_out | saved, nsaved | dq dk dv dg dbeta(NULL) dS_in | ws, nws
    outs = [P_(0x80000 + 0x10000 * i) for i in range(6)]
    outs[4] = None
    bwd_f = getattr(lib, f"{member}_bwd_saved")

    def bwd(saved, nsaved, o=outs):
        return bwd_f(ctypes.byref(s), *base[:6], P_(0x60000), P_(0x70000),
                     None if saved is None else P_(saved), nsaved, *o, P_(0x100000), 1 << 40, None)
    assert bwd(None, 0) == ops.CLR_EWORKSPACE
    assert bwd(0xF0000, n - 256) == ops.CLR_EWORKSPACE
    assert bwd(0xF0010, n) == ops.CLR_EWORKSPACE
    assert bwd(0x80000, n) == ops.CLR_EINVAL                     # overlaps the output dq
    bad = list(outs)
    bad[0] = None
    assert bwd(0xF0000, n, bad) == ops.CLR_EINVAL                # dq missing
    bad = list(outs)
    bad[4] = P_(0xC0000)
    assert bwd(0xF0000, n, bad) == ops.CLR_EINVAL                # dbeta given


def test_kda_saved_activation_entry_points_reject_on_the_host():
    """kda_fwd_save / kda_bwd_saved: host-side rejections (every call below
    fails validation, so nothing is launched)."""
    ops, lib = _lib()
    s = _shape(ops, T=64, H=1, dk=32, dv=32)
    n = ops.saved_bytes(s, ops.OP_KDA_FWD)
    assert n == 2048 + 4096
    P_ = _fake
    # fwd: q k v g beta S_in o S_out | saved, nsaved | ws, nws
    base = [P_(0x10000), P_(0x20000), P_(0x30000), P_(0x40000), P_(0x50000), None, P_(0x60000), P_(0x70000)]

    def fwd(saved, nsaved, ws=0x100000):
        return lib.kda_fwd_save(ctypes.byref(s), *base, None if saved is None else P_(saved), nsaved,
                                None if ws is None else P_(ws), 1 << 40, None)
    assert fwd(None, 0) == ops.CLR_EWORKSPACE
    assert fwd(0xA0000, n - 256) == ops.CLR_EWORKSPACE
    assert fwd(0xA0010, n) == ops.CLR_EWORKSPACE
    assert fwd(0x60000, n) == ops.CLR_EINVAL                     # overlaps the output o
    assert fwd(0xA0000, n, ws=None) == ops.CLR_EWORKSPACE
    s128 = _shape(ops, T=64, H=1, dk=128, dv=128, dtype=0)        # fp32 KDA at d = 128: unsupported
    assert lib.kda_fwd_save(ctypes.byref(s128), *base, P_(0xA0000), 1 << 20, P_(0x100000), 1 << 40,
                            None) == ops.CLR_ENOTSUP
    outs = [P_(0x80000 + 0x10000 * i) for i in range(6)]

    def bwd(saved, nsaved, o=outs):
        return lib.kda_bwd_saved(ctypes.byref(s), *base[:6], P_(0x60000), P_(0x70000),
                                 None if saved is None else P_(saved), nsaved, *o, P_(0x100000), 1 << 40, None)
    assert bwd(None, 0) == ops.CLR_EWORKSPACE
    assert bwd(0xF0000, n - 256) == ops.CLR_EWORKSPACE
    assert bwd(0x80000, n) == ops.CLR_EINVAL                     # overlaps the output dq
    bad = list(outs)
    bad[4] = None
    assert bwd(0xF0000, n, bad) == ops.CLR_EINVAL                # dbeta missing
