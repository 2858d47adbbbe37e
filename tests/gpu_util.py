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


# Gradients (dQ, dK, dV against the fp64 oracle's exact gradient).  Each
# gradient element is a sum x = sum_t a_t b_t over bf16 operands with fp32
# accumulation; its error has three parts, with u = 2^-8 the bf16 unit roundoff:
#   - the final rounding of x to bf16: at most u |x|, about u/3 |x| on average;
#   - the rounding to bf16 of the recomputed operand (P for dV, dS for dQ and
#     dK), u/2 per term at most; the terms have random signs, so the sum's error
#     is about 0.4 u sqrt(sum_t (a_t b_t)^2), i.e. about 0.4 u |x|;
#   - D_i = rowsum(dO_i * O_i) taken from the forward's bf16 O rather than the
#     exact O: |dD_i| <= u sum_e |dO_ie O_ie|, which moves dS_ij by P_ij dD_i.
# Relative to the tensor's scale (max |x|, mean |x|) these stay under 2u for
# the largest element and under u/2 on average; the bounds below allow 4u and
# u.  Elements to which nothing contributes (fully masked rows, masked or
# never-seen keys) must be exactly zero.
GRAD_MAX_REL = 2.0 ** -6
GRAD_MEAN_REL = 2.0 ** -8


def check_grad(got, ref, what: str = "", zero_rows=None) -> dict:
    """Compare a gradient with the oracle's; ``zero_rows`` (bool over the rows of
    the last axis) marks rows no element contributes to, which must be exactly 0."""
    got = np.asarray(got, np.float64).reshape(ref.shape)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite gradient"
    if ref.size == 0:
        return {"max_rel": 0.0, "mean_rel": 0.0}
    if zero_rows is not None:
        zr = np.asarray(zero_rows, bool).reshape(-1)
        rows_got = got.reshape(-1, ref.shape[-1])
        assert np.all(ref.reshape(-1, ref.shape[-1])[zr] == 0.0), f"{what}: oracle disagrees on zero rows"
        assert np.all(rows_got[zr] == 0.0), f"{what}: rows with no contribution must be exactly 0"
    scale_max = float(np.abs(ref).max())
    scale_mean = float(np.abs(ref).mean())
    if scale_max == 0.0:
        assert np.all(got == 0.0), f"{what}: expected all zeros"
        return {"max_rel": 0.0, "mean_rel": 0.0}
    err = np.abs(got - ref)
    stats = {"max_rel": float(err.max()) / scale_max, "mean_rel": float(err.mean()) / scale_mean,
             "scale_max": scale_max}
    assert stats["max_rel"] <= GRAD_MAX_REL, f"{what}: max error {stats}"
    assert stats["mean_rel"] <= GRAD_MEAN_REL, f"{what}: mean error {stats}"
    return stats
