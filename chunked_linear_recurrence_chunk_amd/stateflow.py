"""StateFlow-style sequence-chunk driver on one GPU.

A sequence X = C_0 || C_1 || ... || C_{N-1} (StateFlow paper, Sec. 3.1,
Eq. 3) is processed chunk by chunk: the forward runs i = 0..N-1 with
S_{i+1}^in = S_i^out, the backward runs i = N-1..0 with
dS_i^out = dS_{i+1}^in, and a chunk's saved state is released right after its
backward (the chunk-level activation release of the same section).  Only the
boundary state S_i^in (fp32, dk x dv per head) is kept per chunk; the backward
recomputes the chunk's internals from it.

Every chunk call goes through the C ABI (``ops``); this module only slices
tensors (views, no copies, when B == 1) and orders the calls on the current
stream.  One workspace sized for the chunk length is reused by all calls.
"""
from __future__ import annotations

from typing import Optional


def _bounds(T: int, N: int):
    if N < 1 or T % N:
        raise ValueError(f"sequence length {T} is not divisible into {N} chunks")
    L = T // N
    return [(i * L, (i + 1) * L) for i in range(N)]


def _sl(t, a, b):
    """Token slice [a, b) of a [B, T, ...] tensor (a view if B == 1)."""
    s = t[:, a:b]
    return s if s.is_contiguous() else s.contiguous()


class GdnChunked:
    """Forward/backward of one Gated DeltaNet layer over N sequence chunks.

    With ``save=True`` each chunk's forward also keeps the activations its
    backward needs (gdn_fwd_save), and the backward reads them (gdn_bwd_saved)
    instead of recomputing the chunk's forward from S^in: more device memory
    (clr_saved_bytes per chunk until its backward), less work.  The GLA,
    Mamba-2 and KDA drivers below take the same flag."""

    kind = "gdn"
    _names = ("gdn_fwd", "gdn_bwd", "OP_GDN_FWD", "OP_GDN_BWD")

    def __init__(self, q, k, v, g, beta, N: int, save: bool = False):
        from . import ops
        self.ops = ops
        self.q, self.k, self.v, self.g, self.beta = q, k, v, g, beta
        self.N = N
        self.bounds = _bounds(q.shape[1], N)
        L = self.bounds[0][1]
        B, _, H, dk = q.shape
        dv = v.shape[-1]
        import torch
        fwd, bwd, op_f, op_b = self._names
        self._fwd, self._bwd = getattr(ops, fwd), getattr(ops, bwd)
        shape = ops.ClrShape(B, L, H, dk, dv, ops._dtype_code(q))
        nbytes = max(ops.workspace_bytes(shape, getattr(ops, op_f)), ops.workspace_bytes(shape, getattr(ops, op_b)))
        self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
        self.saved = [None] * N
        self._fwd_save, self._bwd_saved = getattr(ops, fwd + "_save"), getattr(ops, bwd + "_saved")
        self.save = save
        self.acts = [None] * N  # per chunk: the activations gdn_fwd_save kept

    def _chunk(self, i):
        a, b = self.bounds[i]
        return tuple(_sl(t, a, b) for t in (self.q, self.k, self.v, self.g, self.beta))

    def forward(self, S_in=None, o=None):
        """Returns (o, S_out); keeps each chunk's S^in for the backward."""
        import torch
        B, T, H, dk = self.q.shape
        dv = self.v.shape[-1]
        if o is None:
            o = torch.empty((B, T, H, dv), dtype=self.q.dtype, device=self.q.device)
        S = S_in
        for i in range(self.N):
            a, b = self.bounds[i]
            self.saved[i] = S
            view = o[:, a:b]
            ov = view if view.is_contiguous() else None
            if self.save:
                oi, S, self.acts[i] = self._fwd_save(*self._chunk(i), S, ws=self.ws, o=ov)
            else:
                oi, S = self._fwd(*self._chunk(i), S, ws=self.ws, o=ov)
            if oi.data_ptr() != view.data_ptr():
                view.copy_(oi)
        return o, S

    def backward(self, dO, dS_out=None, grads: Optional[dict] = None):
        """Returns dict dq, dk, dv, dg, dbeta, dS_in; releases saved states."""
        import torch
        if grads is None:
            grads = dict(dq=torch.empty_like(self.q), dk=torch.empty_like(self.k),
                         dv=torch.empty_like(self.v), dg=torch.empty_like(self.g),
                         dbeta=torch.empty_like(self.beta))
        dS = dS_out
        for i in reversed(range(self.N)):
            a, b = self.bounds[i]
            views = {key: grads[key][:, a:b] for key in ("dq", "dk", "dv", "dg", "dbeta")}
            out = {key: t for key, t in views.items() if t.is_contiguous()}
            if self.save:
                r = self._bwd_saved(*self._chunk(i), self.saved[i], _sl(dO, a, b), dS, self.acts[i],
                                    ws=self.ws, out=out)
                self.acts[i] = None
            else:
                r = self._bwd(*self._chunk(i), self.saved[i], _sl(dO, a, b), dS, ws=self.ws, out=out)
            for key, t in views.items():
                if r[key].data_ptr() != t.data_ptr():
                    t.copy_(r[key])
            dS = r["dS_in"]
            self.saved[i] = None
        grads["dS_in"] = dS
        return grads


class GlaChunked(GdnChunked):
    """Forward/backward of one GLA layer over N sequence chunks (``save`` as
    for the Gated DeltaNet driver: gla_fwd_save / gla_bwd_saved)."""

    kind = "gla"

    def __init__(self, q, k, v, g, N: int, save: bool = False):
        self._init(q, k, v, g, N, save, "gla", "GLA")

    def _init(self, q, k, v, g, N, save, name, op):
        from . import ops
        self.ops = ops
        self.q, self.k, self.v, self.g, self.beta = q, k, v, g, None
        self.N = N
        self.bounds = _bounds(q.shape[1], N)
        L = self.bounds[0][1]
        B, _, H, dk = q.shape
        dv = v.shape[-1]
        import torch
        shape = ops.ClrShape(B, L, H, dk, dv, ops._dtype_code(q))
        nbytes = max(ops.workspace_bytes(shape, getattr(ops, f"OP_{op}_FWD")),
                     ops.workspace_bytes(shape, getattr(ops, f"OP_{op}_BWD")))
        self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
        self.saved = [None] * N
        self._fwd, self._bwd = getattr(ops, f"{name}_fwd"), getattr(ops, f"{name}_bwd")
        self._fwd_save, self._bwd_saved = getattr(ops, f"{name}_fwd_save"), getattr(ops, f"{name}_bwd_saved")
        self.save = save
        self.acts = [None] * N  # per chunk: the states the forward kept

    def _chunk(self, i):
        a, b = self.bounds[i]
        return tuple(_sl(t, a, b) for t in (self.q, self.k, self.v, self.g))

    def forward(self, S_in=None, o=None):
        import torch
        B, T, H, dk = self.q.shape
        dv = self.v.shape[-1]
        if o is None:
            o = torch.empty((B, T, H, dv), dtype=self.q.dtype, device=self.q.device)
        S = S_in
        for i in range(self.N):
            a, b = self.bounds[i]
            self.saved[i] = S
            view = o[:, a:b]
            ov = view if view.is_contiguous() else None
            if self.save:
                oi, S, self.acts[i] = self._fwd_save(*self._chunk(i), S, ws=self.ws, o=ov)
            else:
                oi, S = self._fwd(*self._chunk(i), S, ws=self.ws, o=ov)
            if oi.data_ptr() != view.data_ptr():
                view.copy_(oi)
        return o, S

    def backward(self, dO, dS_out=None, grads: Optional[dict] = None):
        import torch
        if grads is None:
            grads = dict(dq=torch.empty_like(self.q), dk=torch.empty_like(self.k),
                         dv=torch.empty_like(self.v), dg=torch.empty_like(self.g))
        dS = dS_out
        for i in reversed(range(self.N)):
            a, b = self.bounds[i]
            views = {key: grads[key][:, a:b] for key in ("dq", "dk", "dv", "dg")}
            out = {key: t for key, t in views.items() if t.is_contiguous()}
            if self.save:
                r = self._bwd_saved(*self._chunk(i), self.saved[i], _sl(dO, a, b), dS, self.acts[i],
                                    ws=self.ws, out=out)
                self.acts[i] = None
            else:
                r = self._bwd(*self._chunk(i), self.saved[i], _sl(dO, a, b), dS, ws=self.ws, out=out)
            for key, t in views.items():
                if r[key].data_ptr() != t.data_ptr():
                    t.copy_(r[key])
            dS = r["dS_in"]
            self.saved[i] = None
        grads["dS_in"] = dS
        return grads


class Mamba2Chunked(GlaChunked):
    """Forward/backward of one scalar-gate (Mamba-2 member) layer over N
    sequence chunks."""

    kind = "mamba2"

    def __init__(self, q, k, v, g, N: int, save: bool = False):
        self._init(q, k, v, g, N, save, "mamba2", "M2")


class ShortConvChunked:
    """Causal short convolution over N sequence chunks: the forward hands the
    last W - 1 input rows on as the next chunk's boundary state, the backward
    hands dstate_in back and accumulates dw / dbias over the chunks (the
    local-convolution boundary state of the StateFlow paper, Sec. 3.3)."""

    def __init__(self, x, w, bias, N: int, act: int = 1):
        from . import ops
        self.ops = ops
        self.x, self.w, self.bias, self.act, self.N = x, w, bias, act, N
        self.bounds = _bounds(x.shape[1], N)
        self.saved = [None] * N

    def _chunk(self, t, i):
        a, b = self.bounds[i]
        return _sl(t, a, b)

    def forward(self, state_in=None, y=None):
        import torch
        if y is None:
            y = torch.empty_like(self.x)
        st = state_in
        for i in range(self.N):
            a, b = self.bounds[i]
            self.saved[i] = st
            view = y[:, a:b]
            yi, st = self.ops.shortconv_fwd(self._chunk(self.x, i), self.w, self.bias, st, self.act,
                                            y=view if view.is_contiguous() else None)
            if yi.data_ptr() != view.data_ptr():
                view.copy_(yi)
        return y, st

    def backward(self, dy, dstate_out=None):
        import torch
        dx = torch.empty_like(self.x)
        grads = dict(dw=torch.empty_like(self.w),
                     dbias=torch.empty_like(self.bias) if self.bias is not None else None)
        ds = dstate_out
        for n, i in enumerate(reversed(range(self.N))):
            a, b = self.bounds[i]
            view = dx[:, a:b]
            out = dict(dw=grads["dw"], dbias=grads["dbias"])
            if view.is_contiguous():
                out["dx"] = view
            r = self.ops.shortconv_bwd(self._chunk(self.x, i), self.w, self.bias, self.saved[i],
                                       self._chunk(dy, i), ds, self.act, accumulate=n > 0, out=out)
            if r["dx"].data_ptr() != view.data_ptr():
                view.copy_(r["dx"])
            ds = r["dstate_in"]
            self.saved[i] = None
        return dict(dx=dx, dw=grads["dw"], dbias=grads["dbias"], dstate_in=ds)


class KdaChunked(GdnChunked):
    """Forward/backward of one KDA layer (per-key-channel decay with the delta
    rule) over N sequence chunks; g is [B, T, H, dk]."""

    kind = "kda"
    _names = ("kda_fwd", "kda_bwd", "OP_KDA_FWD", "OP_KDA_BWD")
