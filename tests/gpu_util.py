"""Helpers for the GPU parity tests: device upload and the tolerance checks.

Tolerances (O against the fp64 oracle): bf16 inputs max-abs <= 2e-2 and
mean-abs <= 2e-3; fp32 inputs max-abs <= 1e-5; LSE abs <= 1e-3.  Fully masked
rows must be exactly O = 0 and LSE = -inf.
"""
from __future__ import annotations

import numpy as np

BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
F32_MAX_ABS = 1e-5
LSE_ABS = 1e-3


def torch():
    import torch as t
    return t


def dev(x: np.ndarray, dtype: str):
    """Host array (bf16 bits or fp32 / int) -> device tensor of the same bits."""
    t = torch()
    if dtype == "bf16":
        return t.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(t.bfloat16).cuda()
    return t.from_numpy(np.ascontiguousarray(x)).cuda()


def host_f64(x) -> np.ndarray:
    """Device tensor -> float64 numpy (bf16 widened exactly)."""
    t = torch()
    if x.dtype == t.bfloat16:
        bits = x.view(t.int16).cpu().numpy().view(np.uint16)
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.cpu().numpy().astype(np.float64)


def empty_out(shape, dtype: str):
    t = torch()
    return t.empty(shape, dtype=t.bfloat16 if dtype == "bf16" else t.float32, device="cuda")


def check(o, lse, o_ref, lse_ref, dtype: str, what: str = "") -> dict:
    """Compare GPU (o, lse) with the oracle (float64 arrays, same shape)."""
    o = np.asarray(o, np.float64).reshape(o_ref.shape)
    lse = np.asarray(lse, np.float64).reshape(lse_ref.shape)
    dead = np.isneginf(lse_ref)
    # fully masked rows: exact zero output and -inf LSE
    assert np.all(np.isneginf(lse[dead])), f"{what}: masked rows must have LSE = -inf"
    assert np.all(o[dead] == 0.0), f"{what}: masked rows must have O = 0"
    live = ~dead
    assert np.all(np.isfinite(lse[live])), f"{what}: non-finite LSE on a live row"
    err = np.abs(o[live] - o_ref[live])
    assert np.all(np.isfinite(err)), f"{what}: non-finite output"
    lerr = np.abs(lse[live] - lse_ref[live])
    stats = {"max_abs": float(err.max()) if err.size else 0.0,
             "mean_abs": float(err.mean()) if err.size else 0.0,
             "lse_max_abs": float(lerr.max()) if lerr.size else 0.0}
    if dtype == "bf16":
        assert stats["max_abs"] <= BF16_MAX_ABS, f"{what}: O max-abs {stats}"
        assert stats["mean_abs"] <= BF16_MEAN_ABS, f"{what}: O mean-abs {stats}"
    else:
        assert stats["max_abs"] <= F32_MAX_ABS, f"{what}: O max-abs {stats}"
    assert stats["lse_max_abs"] <= LSE_ABS, f"{what}: LSE {stats}"
    return stats
