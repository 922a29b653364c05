"""Pins of the oracle's reference products and its bf16 rounding against exact
arithmetic (fractions), one-hot and integer closed forms and torch's own
fp32 -> bf16 conversion."""
from fractions import Fraction

import numpy as np
import torch

import workloads
from oracle import products


def _f(bits):
    return Fraction(float(products.bf16_to_f64(np.array([bits]))[0]))


def test_widening_is_exact():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = products.bf16_to_f64(b)
    fin = np.isfinite(t)
    assert np.array_equal(got[fin], t[fin])
    assert np.array_equal(np.isnan(got), np.isnan(t))


def test_one_hot_selects_a_column_exactly():
    for rows, cols in ((48, 256), (64, 64)):
        w = workloads.weights("down", rows=rows, cols=cols, seed=2).numpy().view(np.uint16)
        for k in (0, 17, cols - 1):
            x = np.zeros(cols)
            x[k] = 1.0
            assert np.array_equal(products.gemm_f64(w, x), products.bf16_to_f64(w[:, k]))
            assert np.array_equal(products.gemm_f32(w, x.astype(np.float32)), products.bf16_to_f32(w[:, k]))


def test_integer_valued_products_are_exact():
    rng = np.random.default_rng(1)
    wi = rng.integers(-8, 9, size=(32, 192)).astype(np.float32)
    xi = rng.integers(-8, 9, size=(3, 192)).astype(np.float32)
    wb = (wi.view(np.uint32) >> 16).astype(np.uint16)  # small integers are exact in bf16
    y64 = products.gemm_f64(wb, xi)
    y32 = products.gemm_f32(wb, xi)
    exact = (xi.astype(np.int64) @ wi.astype(np.int64).T).astype(np.float64)
    assert np.array_equal(y64, exact) and np.array_equal(y32.astype(np.float64), exact)


def test_fp64_product_against_exact_fractions():
    w = workloads.weights("small", rows=6, cols=64, seed=3).numpy().view(np.uint16)
    x = workloads.activations(64, 2, seed=4, dtype=torch.float32).numpy()
    y = products.gemm_f64(w, x)
    for b in range(2):
        for n in range(6):
            exact = sum(_f(w[n, k]) * Fraction(float(x[b, k])) for k in range(64))
            assert abs(Fraction(float(y[b, n])) - exact) <= abs(exact) * Fraction(1, 2**45) + Fraction(1, 2**60)


def test_round_to_bf16_by_hand():
    cases = {
        1.0: 0x3F80,
        1.0 + 2.0 ** -8: 0x3F80,               # tie -> even (down)
        1.0 + 3 * 2.0 ** -8: 0x3F82,           # tie -> even (up)
        1.0 + 2.0 ** -8 + 2.0 ** -30: 0x3F81,  # just above the tie
        -2.5: 0xC020,
        0.0: 0x0000,
        2.0 ** -133: 0x0001,                   # smallest subnormal
        2.0 ** -134: 0x0000,                   # tie between 0 and it -> even (0)
        3 * 2.0 ** -134: 0x0002,               # tie 1.5 quanta -> 2
        3.3895313892515355e38: 0x7F7F,         # max finite
        2.0 ** 128: 0x7F80,
        -1e39: 0xFF80,
    }
    got = products.round_to_bf16(np.array(list(cases)))
    assert [int(v) for v in got] == list(cases.values())
    assert products.round_to_bf16(np.array([np.nan]))[0] & 0x7FC0 == 0x7FC0


def test_round_to_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    t = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(products.round_to_bf16(f.astype(np.float64)), t)


def test_ulp_distance():
    a = np.array([0x3F80, 0x3F80, 0x0000, 0x8000, 0x0001, 0x7F7F], dtype=np.uint16)
    b = np.array([0x3F81, 0x3F7F, 0x8000, 0x8001, 0x8001, 0x7F80], dtype=np.uint16)
    assert list(products.bf16_ulp_distance(a, b)) == [1, 1, 0, 1, 2, 1]


def test_rel_error_floor():
    ref = np.array([1.0, -1.0, 1e-9, 2.0])
    rms = np.sqrt(np.mean(ref ** 2))
    y = ref + np.array([0, 0, 1e-3, 0])
    assert abs(products.rel_error_floored(y, ref) - 1e-3 / rms) < 1e-12
    assert products.nonfinite_match(np.array([np.nan, 1, np.inf]), np.array([np.nan, 2, np.inf]))
    assert not products.nonfinite_match(np.array([1.0, np.inf]), np.array([np.nan, np.inf]))
