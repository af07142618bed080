"""Helpers shared by the GPU tests: move seeded numpy inputs to the GPU in the
kernel's element type, and compare against the oracle."""
import numpy as np

from chunked_linear_recurrence_chunk_amd import inputs


def to_dev(x: np.ndarray, dtype: str):
    """numpy float32 (already bf16-exact when dtype == 'bf16') -> cuda tensor."""
    import torch
    if dtype == "bf16":
        bits = inputs.bf16_bits(x)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def to_np(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| (per tensor)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.max(np.abs(ref)) if ref.size else 0.0
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref)) / max(scale, 1e-30))


# Tolerances (per-tensor max-abs error over max |ref|).
TOL_FP32 = 1e-4
TOL_BF16 = 2e-2          # o, dq, dk, dv, dg, dbeta
TOL_BF16_STATE = 1e-2    # S_out, dS_in


def tol(dtype, key):
    if dtype == "fp32":
        return TOL_FP32
    return TOL_BF16_STATE if key in ("S_out", "dS_in") else TOL_BF16
