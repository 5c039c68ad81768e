"""Comparison helpers for the GPU parity tests (test code, not the oracle)."""
from __future__ import annotations

import math

import numpy as np
import torch

# Output tolerance against the fp64 oracle (max-abs and mean-abs), plus the
# stage checks that are tighter than it.
OUT_MAX_ABS = 2e-2
OUT_MEAN_ABS = 2e-3
OUT_C_RTOL = 1e-6
OUT_C_ATOL = 1e-12
SPARSE_REL_RMS = 1e-2  # rms(gpu - oracle) / rms(oracle) for the sparse stage


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def rms(x) -> float:
    x = np.asarray(x, dtype=np.float64)
    return math.sqrt(float(np.mean(x * x))) if x.size else 0.0


def check_out(gpu: np.ndarray, ref: np.ndarray, what: str = "out"):
    m = np.isfinite(ref)
    d = np.abs(gpu[m] - ref[m])
    assert d.size > 0, f"{what}: nothing to compare"
    assert np.isfinite(gpu[m]).all(), f"{what}: non-finite GPU values"
    mx, mean = float(d.max()), float(d.mean())
    assert mx <= OUT_MAX_ABS, f"{what}: max-abs {mx:.3e} > {OUT_MAX_ABS}"
    assert mean <= OUT_MEAN_ABS, f"{what}: mean-abs {mean:.3e} > {OUT_MEAN_ABS}"
    return mx, mean


def check_sparse(gpu: np.ndarray, ref: np.ndarray, what: str = "out_s"):
    m = np.isfinite(ref)
    mx, _ = check_out(gpu, ref, what)
    rel = rms(gpu[m] - ref[m]) / max(rms(ref[m]), 1e-30)
    assert rel <= SPARSE_REL_RMS, f"{what}: rms error / rms {rel:.3e} > {SPARSE_REL_RMS}"
    return rel


def check_fused(fused: np.ndarray, unfused: np.ndarray, out_s: np.ndarray, what: str = "fused"):
    """The fused combine rounds once (bf16(fma(out_c, g, O))) where the stage
    sequence rounds O to bf16 first: they may differ by the rounding of O
    (half a bf16 ulp, 2^-9 |O|) plus one rounding of the result each."""
    bound = 2.0 ** -8 * (np.abs(out_s) + np.abs(fused) + np.abs(unfused))
    m = np.isfinite(unfused)
    bad = np.abs(fused[m] - unfused[m]) > bound[m]
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond the double-rounding bound"


def check_out_c(gpu: np.ndarray, ref: np.ndarray):
    bad = ~np.isclose(gpu, ref, rtol=OUT_C_RTOL, atol=OUT_C_ATOL)
    assert not bad.any(), f"out_c: {int(bad.sum())} elements off, worst rel " \
        f"{float(np.max(np.abs(gpu - ref) / np.maximum(np.abs(ref), 1e-30))):.3e}"


# ---------------------------------------------------------------------------
# exact emulation of bf16(fp32 fma(a, b, c)) / bf16(fp32(a + c)) on the CPU
# ---------------------------------------------------------------------------

def _round_to_f32(hi: np.ndarray, lo: np.ndarray) -> np.ndarray:
    """Round the exact value hi + lo (hi = fl64(hi + lo), |lo| <= ulp64(hi)/2) to
    float32, ties to even, without double rounding."""
    f = hi.astype(np.float32)
    diff = hi - f.astype(np.float64)
    up = np.nextafter(f, np.float32(np.inf))
    dn = np.nextafter(f, np.float32(-np.inf))
    half_up = (up.astype(np.float64) - f.astype(np.float64)) / 2
    half_dn = (f.astype(np.float64) - dn.astype(np.float64)) / 2
    # hi sits exactly on a float32 midpoint, RNE went to the other side of
    # it than the one lo points to: move one float32 step towards lo
    fix_up = (diff == half_up) & (lo > 0)
    fix_dn = (diff == -half_dn) & (lo < 0)
    f = np.where(fix_up, up, f)
    f = np.where(fix_dn, dn, f)
    return f


def _two_sum(a: np.ndarray, b: np.ndarray):
    s = a + b
    bb = s - a
    e = (a - (s - bb)) + (b - bb)
    return s, e


def f32_to_bf16_bits(f: np.ndarray) -> np.ndarray:
    u = f.astype(np.float32).view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((u >> 16) & 1)
    return ((u + bias) >> 16).astype(np.uint16)


def fma_bf16_bits(a32: np.ndarray, b32: np.ndarray, c32: np.ndarray) -> np.ndarray:
    p = a32.astype(np.float64) * b32.astype(np.float64)  # exact: 24 + 24 bits
    s, e = _two_sum(p, c32.astype(np.float64))
    return f32_to_bf16_bits(_round_to_f32(s, e))


def add_bf16_bits(a32: np.ndarray, c32: np.ndarray) -> np.ndarray:
    s, e = _two_sum(a32.astype(np.float64), c32.astype(np.float64))
    return f32_to_bf16_bits(_round_to_f32(s, e))


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)
