"""The bf16 output rule of the GPU parity checks (tests/parity.py), on
constructed outputs: a correctly rounded result passes, 3 ulp off fails, a
tiny output off by more than 2 ulp of itself but inside the fp32
accumulation band passes and is counted, and one just outside the band
fails."""
import numpy as np

from oracle import products
from tests.parity import U24, bf16_band_stats


def _case():
    rng = np.random.default_rng(3)
    ref = rng.standard_normal(2000) * 1.3
    return ref, products.round_to_bf16(ref)


def test_exact_rounding_passes():
    ref, got = _case()
    fails, band_only, worst, n = bf16_band_stats(got, ref, cols=4096)
    assert (fails, band_only, worst, n) == (0, 0, 0, 2000)


def test_three_ulp_off_a_large_output_fails():
    ref, got = _case()
    i = int(np.argmax(np.abs(ref)))
    got = got.copy()
    got[i] = products.round_to_bf16(np.array([ref[i] * (1 + 3 * 2.0 ** -7)]))[0]
    assert bf16_band_stats(got, ref, cols=4096)[0] == 1


def test_tiny_output_inside_the_band_passes_and_is_counted():
    ref, got = _case()
    rms = float(np.sqrt(np.mean(ref ** 2)))
    ref = ref.copy()
    ref[7] = 1e-6 * rms  # 2 ulp of this is ~1e-8 rms; the band is cols * 2^-24 * rms
    eps = 4096 * U24 * rms
    got = products.round_to_bf16(ref)
    got[7] = products.round_to_bf16(np.array([ref[7] + 0.5 * eps]))[0]
    fails, band_only, worst, _ = bf16_band_stats(got, ref, cols=4096)
    assert (fails, band_only) == (0, 1)
    got[7] = products.round_to_bf16(np.array([ref[7] + 3 * eps]))[0]
    assert bf16_band_stats(got, ref, cols=4096)[0] == 1
