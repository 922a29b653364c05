"""Parity checks of device outputs against the oracle's fp64 products.

fp32 outputs:  max |y - y64| / max(|y64|, rms(y64)) <= 1e-3 (the rms floor
keeps the measure meaningful for outputs that land near zero).

bf16 outputs:  every output is either within 2 bf16 ulp of RNE(y64), or it is
RNE of a value v with |v - y64| <= cols * 2^-24 * rms(y64).  The second
clause is the reading that a bf16 output is one rounding of an fp32 sum: the
fp32 sum itself differs from y64 by an accumulation error of order
sqrt(cols) * 2^-24 * rms for random data (any order; cols * 2^-24 * rms is
that times sqrt(cols) of margin), and for an output much smaller than rms
that error alone can exceed 2 ulp of the output's own magnitude.  Outputs
that pass only through this clause are counted and capped, and each call
reports the count and the largest ulp distance among the other outputs, so
a drift toward the band's edge shows in the log.
"""
from __future__ import annotations

import sys

import numpy as np

from oracle import products

TOL = 1e-3
U24 = 2.0 ** -24


def _say(msg):
    print(f"[parity] {msg}", flush=True)
    sys.stdout.flush()


def check_f32(y, ref64, what):
    y = y.detach().float().cpu().numpy().astype(np.float64) if hasattr(y, "detach") else np.asarray(y, np.float64)
    assert products.nonfinite_match(y, ref64), what + ": non-finite pattern differs"
    err = products.rel_error_floored(y, ref64)
    assert err <= TOL, f"{what}: rel err {err:.3e}"
    return err


def bf16_band_stats(got_bits, ref64, cols):
    """(fails, band_only, worst_ulp_rest, n) for bf16 outputs got_bits against
    the fp64 reference, under the rule in the module docstring."""
    got = np.asarray(got_bits).astype(np.uint16)
    ref = products.round_to_bf16(ref64)
    fin = np.isfinite(ref64)
    r = ref64[fin]
    g = got[fin]
    dist = products.bf16_ulp_distance(g, ref[fin])
    near = dist <= 2
    rms = float(np.sqrt(np.mean(r ** 2))) if r.size else 1.0
    eps = cols * U24 * (rms if rms > 0 else 1.0)
    k = products.bf16_order_key(g)
    band = (k >= products.bf16_order_key(products.round_to_bf16(r - eps))) & \
           (k <= products.bf16_order_key(products.round_to_bf16(r + eps)))
    fails = int((~(near | band)).sum())
    band_only = int((band & ~near).sum())
    worst = int(dist[near].max()) if near.any() else 0
    return fails, band_only, worst, int(r.size)


def check_bf16(y, ref64, what, cols):
    """y: a torch bf16 tensor (or uint16 bits); cols: the contraction length."""
    if hasattr(y, "detach"):
        import torch
        got = y.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    else:
        got = np.asarray(y).view(np.uint16)
    fails, band_only, worst, n = bf16_band_stats(got, ref64, cols)
    _say(f"{what}: bf16 {n} outputs, {band_only} within the fp32 band only, worst ulp of the rest {worst}")
    assert fails == 0, f"{what}: {fails} outputs outside 2 bf16 ulp and the fp32 band"
    assert band_only <= max(8, n // 1000), f"{what}: {band_only} of {n} outputs pass only through the fp32 band"
    assert np.array_equal(np.isnan(products.bf16_to_f64(got)), np.isnan(ref64)), what
    return band_only, worst
