"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random tensors with the shapes and distributions of the
workloads; it contains none of the layer's arithmetic, so the GPU path and the
fp64 oracle can both be fed from it without sharing any computation.

Distributions (per-token tensors are [B,T,H,d], states [B,H,dk,dv]):
  Gated DeltaNet: q, k ~ N(0,1) then L2-normalised per (token, head);
                  v ~ N(0,1); beta = sigmoid(N(0,1)); g = log alpha = -softplus(N(0,1));
                  S_in = 0.1 * N(0,1); dO ~ N(0,1); dS_out ~ N(0,1).
  GLA:            q, k, v ~ N(0,1); g = logsigmoid(N(0,1)) / 16 per key channel;
                  S_in = 0.1 * N(0,1); dO ~ N(0,1); dS_out ~ N(0,1).
  Mamba-2:        as GLA, but one gate per (token, head): g [B,T,H].
  KDA:            q, k, v, beta, S_in as Gated DeltaNet; g = logsigmoid(N(0,1)) / 16
                  per key channel [B,T,H,dk] as GLA.
  Delta-rule stress (make_delta_stress): keys repeated from 8 L2-normalised
                  vectors per head, beta = 0.99, g = -softplus(N(0,1))/1024 or 0.
  Strong decay (make_strong_decay): the GLA / KDA / Mamba-2 recipe, then
                  g = -U(lo, hi) on key channels d = 0 mod 4 (scalar gate: even heads).
  Short conv:     x ~ N(0,1) [B,T,C]; w = 0.5 * N(0,1) [C,W]; bias = 0.1 * N(0,1);
                  state_in ~ N(0,1) [B,W-1,C]; dy ~ N(0,1); dstate_out ~ N(0,1)
                  (float32: state gradients are partial sums and stay fp32).
                  The workload has C = H * (2 dk + dv) = 6144 channels, the q, k
                  and v projections of the Gated DeltaNet workload, W = 4, SiLU.
Draw order: q, k, v, g, beta (GDN only), S_in, dO, dS_out, all float32 from a
numpy PCG64 generator.  For dtype "bf16" every per-token tensor (including dO)
is rounded to bfloat16 (round-to-nearest-even) and returned as the exact
float32 value of that bfloat16; states stay float32.
"""
from __future__ import annotations

import numpy as np

# Workloads (name -> parameters).  "N" is the number of sequence chunks the
# sequence is split into with boundary-state hand-off.
CONFIGS = {
    "gdn_fp32_T256_d32": dict(kind="gdn", dtype="fp32", B=1, H=1, T=256, dk=32, dv=32, N=4),
    "gdn_bf16_H16_T8192_d128": dict(kind="gdn", dtype="bf16", B=1, H=16, T=8192, dk=128, dv=128, N=4),
    "gla_bf16_B4_H16_T4096_dk128_dv256": dict(kind="gla", dtype="bf16", B=4, H=16, T=4096, dk=128, dv=256, N=1),
    "gdn_bf16_H32_T65536_d128": dict(kind="gdn", dtype="bf16", B=1, H=32, T=65536, dk=128, dv=128, N=16),
    "gdn_bf16_H16_T262144_d128": dict(kind="gdn", dtype="bf16", B=1, H=16, T=262144, dk=128, dv=128, N=64),
    # short convolution in front of the Gated DeltaNet workload (q, k, v channels)
    "shortconv_bf16_T8192_C6144_W4": dict(kind="shortconv", dtype="bf16", B=1, T=8192, C=6144, W=4, act=1, N=4),
    # per-channel-decay delta rule at the Gated DeltaNet workload's shape
    "kda_bf16_H16_T8192_d128": dict(kind="kda", dtype="bf16", B=1, H=16, T=8192, dk=128, dv=128, N=4),
    # scalar-gate member at the GLA workload's shape
    "mamba2_bf16_B4_H16_T4096_dk128_dv256": dict(kind="mamba2", dtype="bf16", B=4, H=16, T=4096, dk=128, dv=256, N=1),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.
    NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> exact float32 values."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    return bf16_value(bf16_bits(x))


def _sigmoid(x):
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _softplus(x):
    x = x.astype(np.float64)
    return (np.maximum(x, 0) + np.log1p(np.exp(-np.abs(x)))).astype(np.float32)


def _l2n(x):
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / np.maximum(n, 1e-12)).astype(np.float32)


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def make_gdn(B, T, H, dk, dv, dtype="fp32", seed=0, slow_decay=False):
    """Gated DeltaNet inputs.  slow_decay=True draws g = -softplus(N(0,1))/64
    (a stress case where the state survives for ~100 tokens)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _l2n(_normal(rng, (B, T, H, dk)))
    k = _l2n(_normal(rng, (B, T, H, dk)))
    v = _normal(rng, (B, T, H, dv))
    g = -_softplus(_normal(rng, (B, T, H)))
    if slow_decay:
        g = (g / 64.0).astype(np.float32)
    beta = _sigmoid(_normal(rng, (B, T, H)))
    S_in = (0.1 * _normal(rng, (B, H, dk, dv))).astype(np.float32)
    dO = _normal(rng, (B, T, H, dv))
    dS_out = _normal(rng, (B, H, dk, dv))
    d = dict(q=q, k=k, v=v, g=g, beta=beta, S_in=S_in, dO=dO, dS_out=dS_out)
    if dtype == "bf16":
        for key in ("q", "k", "v", "g", "beta", "dO"):
            d[key] = bf16_round(d[key])
    elif dtype != "fp32":
        raise ValueError(dtype)
    return d


def make_gla(B, T, H, dk, dv, dtype="bf16", seed=0, gate_scale=1.0 / 16.0):
    """GLA inputs.  gate_scale=1 gives the strong-gate stress case."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _normal(rng, (B, T, H, dk))
    k = _normal(rng, (B, T, H, dk))
    v = _normal(rng, (B, T, H, dv))
    z = _normal(rng, (B, T, H, dk)).astype(np.float64)
    logsig = -(np.maximum(-z, 0) + np.log1p(np.exp(-np.abs(z))))
    g = (logsig * gate_scale).astype(np.float32)
    S_in = (0.1 * _normal(rng, (B, H, dk, dv))).astype(np.float32)
    dO = _normal(rng, (B, T, H, dv))
    dS_out = _normal(rng, (B, H, dk, dv))
    d = dict(q=q, k=k, v=v, g=g, S_in=S_in, dO=dO, dS_out=dS_out)
    if dtype == "bf16":
        for key in ("q", "k", "v", "g", "dO"):
            d[key] = bf16_round(d[key])
    elif dtype != "fp32":
        raise ValueError(dtype)
    return d


def make_mamba2(B, T, H, dk, dv, dtype="bf16", seed=0, gate_scale=1.0 / 16.0):
    """Scalar-gate (Mamba-2 member) inputs: the GLA recipe with g [B,T,H]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _normal(rng, (B, T, H, dk))
    k = _normal(rng, (B, T, H, dk))
    v = _normal(rng, (B, T, H, dv))
    z = _normal(rng, (B, T, H)).astype(np.float64)
    logsig = -(np.maximum(-z, 0) + np.log1p(np.exp(-np.abs(z))))
    g = (logsig * gate_scale).astype(np.float32)
    S_in = (0.1 * _normal(rng, (B, H, dk, dv))).astype(np.float32)
    dO = _normal(rng, (B, T, H, dv))
    dS_out = _normal(rng, (B, H, dk, dv))
    d = dict(q=q, k=k, v=v, g=g, S_in=S_in, dO=dO, dS_out=dS_out)
    if dtype == "bf16":
        for key in ("q", "k", "v", "g", "dO"):
            d[key] = bf16_round(d[key])
    elif dtype != "fp32":
        raise ValueError(dtype)
    return d


def make_kda(B, T, H, dk, dv, dtype="bf16", seed=0, gate_scale=1.0 / 16.0):
    """KDA inputs: q, k L2-normalised, v, beta, S_in as Gated DeltaNet; the
    gate per key channel as GLA."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _l2n(_normal(rng, (B, T, H, dk)))
    k = _l2n(_normal(rng, (B, T, H, dk)))
    v = _normal(rng, (B, T, H, dv))
    z = _normal(rng, (B, T, H, dk)).astype(np.float64)
    logsig = -(np.maximum(-z, 0) + np.log1p(np.exp(-np.abs(z))))
    g = (logsig * gate_scale).astype(np.float32)
    beta = _sigmoid(_normal(rng, (B, T, H)))
    S_in = (0.1 * _normal(rng, (B, H, dk, dv))).astype(np.float32)
    dO = _normal(rng, (B, T, H, dv))
    dS_out = _normal(rng, (B, H, dk, dv))
    d = dict(q=q, k=k, v=v, g=g, beta=beta, S_in=S_in, dO=dO, dS_out=dS_out)
    if dtype == "bf16":
        for key in ("q", "k", "v", "g", "beta", "dO"):
            d[key] = bf16_round(d[key])
    elif dtype != "fp32":
        raise ValueError(dtype)
    return d


def make_delta_stress(kind, B, T, H, dk, dv, dtype="bf16", seed=0, gate="slow", beta=0.99, n_keys=8):
    """Stress inputs for the delta-rule members (kind "gdn" or "kda"): almost
    no decay, an almost complete erase, and keys repeated from a small set, so
    that the state is carried over the whole sequence and each block's writes
    nearly cancel one another.

      keys:   a pool of n_keys L2-normalised N(0,1) vectors per (batch, head);
              token t uses pool[b, h, j] with j uniform in [0, n_keys);
      gate:   "slow": g = -softplus(N(0,1)) / 1024; "zero": g = 0
              (per (token, head) for "gdn", per key channel for "kda");
      beta:   the constant `beta` (0.99);
      q, v, S_in, dO, dS_out as make_gdn.
    Draw order: q, key pool, key index, v, gate normals, S_in, dO, dS_out."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _l2n(_normal(rng, (B, T, H, dk)))
    pool = _l2n(_normal(rng, (B, H, n_keys, dk)))
    idx = rng.integers(0, n_keys, size=(B, T, H))
    bi = np.arange(B)[:, None, None]
    hi = np.arange(H)[None, None, :]
    k = np.ascontiguousarray(pool[bi, hi, idx])  # [B, T, H, dk]
    v = _normal(rng, (B, T, H, dv))
    gshape = (B, T, H) if kind == "gdn" else (B, T, H, dk)
    z = _normal(rng, gshape)
    if gate == "slow":
        g = (-_softplus(z) / 1024.0).astype(np.float32)
    elif gate == "zero":
        g = np.zeros(gshape, np.float32)
    else:
        raise ValueError(gate)
    b = np.full((B, T, H), beta, np.float32)
    S_in = (0.1 * _normal(rng, (B, H, dk, dv))).astype(np.float32)
    dO = _normal(rng, (B, T, H, dv))
    dS_out = _normal(rng, (B, H, dk, dv))
    d = dict(q=q, k=k, v=v, g=g, beta=b, S_in=S_in, dO=dO, dS_out=dS_out)
    if dtype == "bf16":
        for key in ("q", "k", "v", "g", "beta", "dO"):
            d[key] = bf16_round(d[key])
    elif dtype != "fp32":
        raise ValueError(dtype)
    return d


def make_strong_decay(kind, B, T, H, dk, dv, dtype="bf16", seed=0, lo=9.0, hi=9.75):
    """Inputs of the per-channel and scalar-gate members (kind "gla", "kda",
    "mamba2") with some gates near the diagonal tiles' decay bound: the
    member's own recipe (make_gla / make_kda / make_mamba2 with `seed`), then,
    from a second generator (seed + 7919), g = -U(lo, hi) on every token for
    the key channels d = 0 mod 4 (per-channel members) or the even heads
    (scalar gate).  With hi <= 10 no 8 consecutive gates sum below -80; with
    lo > 80 / 7 some 16-token sub-tile leaves that bound."""
    f = {"gla": make_gla, "kda": make_kda, "mamba2": make_mamba2}[kind]
    d = f(B, T, H, dk, dv, "fp32", seed)
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    g = d["g"].copy()
    if kind == "mamba2":
        g[:, :, 0::2] = -rng.uniform(lo, hi, size=g[:, :, 0::2].shape)
    else:
        g[..., 0::4] = -rng.uniform(lo, hi, size=g[..., 0::4].shape)
    d["g"] = g.astype(np.float32)
    if dtype == "bf16":
        for key in ("q", "k", "v", "g", "beta", "dO"):
            if key in d:
                d[key] = bf16_round(d[key])
    elif dtype != "fp32":
        raise ValueError(dtype)
    return d


def make_shortconv(B, T, C, W, dtype="bf16", seed=0):
    """Short-convolution inputs (x, w, bias, state_in, dy, dstate_out)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = _normal(rng, (B, T, C))
    w = (0.5 * _normal(rng, (C, W))).astype(np.float32)
    bias = (0.1 * _normal(rng, (C,))).astype(np.float32)
    state_in = _normal(rng, (B, W - 1, C))
    dy = _normal(rng, (B, T, C))
    dstate_out = _normal(rng, (B, W - 1, C))
    d = dict(x=x, w=w, bias=bias, state_in=state_in, dy=dy, dstate_out=dstate_out)
    if dtype == "bf16":
        for key in ("x", "state_in", "dy"):
            d[key] = bf16_round(d[key])
    elif dtype != "fp32":
        raise ValueError(dtype)
    return d


def make(cfg: dict, seed: int, **kw):
    if cfg["kind"] == "shortconv":
        return make_shortconv(cfg["B"], cfg["T"], cfg["C"], cfg["W"], cfg["dtype"], seed)
    f = {"gdn": make_gdn, "gla": make_gla, "mamba2": make_mamba2, "kda": make_kda}[cfg["kind"]]
    return f(cfg["B"], cfg["T"], cfg["H"], cfg["dk"], cfg["dv"], cfg["dtype"], seed, **kw)
