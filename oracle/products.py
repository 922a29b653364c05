"""Reference products over the (decoded) bf16 weights (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Unweight: how we compressed an LLM 22% without sacrificing quality",
paragraph on the reconstructive matmul: the kernel rebuilds the original bf16
weights and feeds them to the multiply, so the product is exactly the one
over the uncompressed matrix.  Definitions used here:

  y = W x            W [rows, cols] bf16, x [cols]            (batch 1)
  Y = X W^T          X [batch, cols],      Y [batch, rows]

The ground truth is the fp64 product of the exactly widened operands (a bf16
or fp32 value is exact in fp64); an fp32 product is kept beside it for
reporting.  bf16 outputs are judged against the fp64 result rounded once to
bf16 (round to nearest, ties to even).
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening: the bf16 pattern is the top half of an fp32 pattern."""
    b = np.asarray(bits).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits).astype(np.uint32) << 16
    return b.view(np.float32)


def gemm_f64(w_bits: np.ndarray, x: np.ndarray) -> np.ndarray:
    """Y[b, n] = sum_k X[b, k] * W[n, k] in fp64.  x: [batch, cols] float array
    (any float dtype; it is widened exactly) or [cols] for a matvec."""
    W = bf16_to_f64(w_bits)
    X = np.asarray(x, dtype=np.float64)
    return X @ W.T


def gemm_f32(w_bits: np.ndarray, x: np.ndarray) -> np.ndarray:
    W = bf16_to_f32(w_bits)
    X = np.asarray(x, dtype=np.float32)
    return X @ W.T


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """fp64 values -> bf16 bit patterns, a single round to nearest even.

    A finite value v = m * 2^e (frexp, m in [0.5, 1)) is rounded at the
    quantum 2^(e-8) (8 significant bits), never finer than the subnormal
    quantum 2^-133; magnitudes that round to 2^128 or beyond become Inf.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros(v.shape, dtype=np.uint16)
    finite = np.isfinite(v)
    m, e = np.frexp(np.where(finite, v, 0.0))
    q = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(np.where(finite, v, 0.0), -q)), q)
    over = np.abs(r) >= 2.0 ** 128
    with np.errstate(over="ignore", invalid="ignore"):
        f32 = np.where(over, 0.0, r).astype(np.float32)  # exact: <= 8 significant bits, in range
    bits = (f32.view(np.uint32) >> 16).astype(np.uint16)
    bits = np.where(over, np.where(r > 0, 0x7F80, 0xFF80), bits)
    bits = np.where(np.isnan(v), 0x7FC0, bits)
    bits = np.where(np.isposinf(v), 0x7F80, bits)
    bits = np.where(np.isneginf(v), 0xFF80, bits)
    out[...] = bits
    return out


def bf16_order_key(bits: np.ndarray) -> np.ndarray:
    """Monotone integer key of bf16 patterns: adjacent representable values
    differ by 1 and +0 / -0 both map to 0."""
    b = np.asarray(bits).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    return np.abs(bf16_order_key(a_bits) - bf16_order_key(b_bits))


def rel_error_floored(y: np.ndarray, ref64: np.ndarray) -> float:
    """max_i |y_i - ref_i| / max(|ref_i|, rms(ref)) over finite reference entries.

    The rms floor keeps the measure meaningful for outputs near zero (a sum of
    thousands of random terms lands arbitrarily close to 0 now and then).
    """
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref64, dtype=np.float64)
    fin = np.isfinite(ref)
    if not fin.any():
        return 0.0
    rms = float(np.sqrt(np.mean(ref[fin] ** 2)))
    den = np.maximum(np.abs(ref[fin]), rms if rms > 0 else 1.0)
    return float(np.max(np.abs(y[fin] - ref[fin]) / den))


def nonfinite_match(y: np.ndarray, ref64: np.ndarray) -> bool:
    """NaN positions equal and +-Inf positions equal."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref64, dtype=np.float64)
    return bool(np.array_equal(np.isnan(y), np.isnan(ref))
                and np.array_equal(np.isposinf(y), np.isposinf(ref))
                and np.array_equal(np.isneginf(y), np.isneginf(ref)))
