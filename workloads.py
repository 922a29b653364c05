"""Seeded synthetic inputs shared by the tests, the bench and the oracle timing.

This module only draws numbers: it holds none of the compression method's
arithmetic (no exponent split, no coding, no products), so the CPU oracle and
the GPU library can both be fed from it without sharing any code.

The pages measured trained Llama-3.1-8B MLP weights ("Unweight: how we
compressed an LLM 22% without sacrificing quality", results paragraph); none
are available here, so seeded Gaussian bf16 matrices of the same shapes stand
in for them.  Recipes, one per workload:

  small     1024x1024, N(0, 0.02), x fp32 N(0, 1)               seed 1
  gate      14336x4096 (gate_proj shape), N(0, 0.02), x bf16      seed 2
  down      4096x14336 (down_proj shape), N(0, 0.02) with a
            Bernoulli(0.005) mask of entries replaced by N(0, 1)  seed 3
  stack     32 layers of {gate, up 14336x4096; down 4096x14336},
            per-layer sigma = 0.01 + 0.03*U (U from seed 999),
            layer l matrices from seed 1000 + l
  randbits  8192x8192 uniformly random 16-bit patterns           seed 5
  big       8192x8192, N(0, 0.02)                                 seed 6

Activations use seed + 100.  Weights are drawn in fp32 and rounded to bf16
with torch's round-to-nearest-even conversion.
"""
from __future__ import annotations

import torch

SIGMA = 0.02
OUTLIER_RATE = 0.005

SHAPES = {
    "small": (1024, 1024),
    "gate": (14336, 4096),
    "up": (14336, 4096),
    "down": (4096, 14336),
    "randbits": (8192, 8192),
    "big": (8192, 8192),
}
SEEDS = {"small": 1, "gate": 2, "down": 3, "randbits": 5, "big": 6}
STACK_LAYERS = 32
STACK_SIGMA_SEED = 999
STACK_LAYER_SEED0 = 1000


def _gen(seed: int) -> torch.Generator:
    return torch.Generator().manual_seed(int(seed))


def gaussian_bf16(rows: int, cols: int, sigma: float, seed: int) -> torch.Tensor:
    """N(0, sigma) weights rounded to bf16; returned as the raw uint16 bit patterns (int16 view)."""
    g = _gen(seed)
    w = (torch.randn(rows, cols, generator=g) * sigma).to(torch.bfloat16)
    return w.view(torch.int16)


def gaussian_with_outliers_bf16(rows: int, cols: int, sigma: float, rate: float, seed: int) -> torch.Tensor:
    g = _gen(seed)
    w = torch.randn(rows, cols, generator=g) * sigma
    mask = torch.rand(rows, cols, generator=g) < rate
    out = torch.randn(rows, cols, generator=g)
    w = torch.where(mask, out, w).to(torch.bfloat16)
    return w.view(torch.int16)


def random_bits_bf16(rows: int, cols: int, seed: int) -> torch.Tensor:
    g = _gen(seed)
    return torch.randint(-32768, 32768, (rows, cols), generator=g, dtype=torch.int32).to(torch.int16)


def stack_sigmas() -> list[float]:
    g = _gen(STACK_SIGMA_SEED)
    u = torch.rand(STACK_LAYERS, generator=g, dtype=torch.float64)
    return [0.01 + 0.03 * float(v) for v in u]


def stack_layer(layer: int) -> dict[str, torch.Tensor]:
    """The three MLP matrices of one layer of the 32-layer stack (int16 bit views)."""
    sigma = stack_sigmas()[layer]
    g = _gen(STACK_LAYER_SEED0 + layer)
    out = {}
    for name in ("gate", "up", "down"):
        r, c = SHAPES[name]
        out[name] = (torch.randn(r, c, generator=g) * sigma).to(torch.bfloat16).view(torch.int16)
    return out


def weights(name: str, rows: int | None = None, cols: int | None = None, seed: int | None = None) -> torch.Tensor:
    """Weights (int16 bit view, [rows, cols] row-major) of a named workload.

    rows/cols/seed override the named shape, so tests can draw the same
    distribution at sizes the oracle finishes quickly.
    """
    r0, c0 = SHAPES.get(name, (None, None))
    r = rows if rows is not None else r0
    c = cols if cols is not None else c0
    s = seed if seed is not None else SEEDS[name]
    if name in ("small", "gate", "up", "big"):
        return gaussian_bf16(r, c, SIGMA, s)
    if name == "down":
        return gaussian_with_outliers_bf16(r, c, SIGMA, OUTLIER_RATE, s)
    if name == "randbits":
        return random_bits_bf16(r, c, s)
    raise KeyError(name)


def activations(cols: int, batch: int, seed: int, dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """x / X ~ N(0, 1), shape [batch, cols], in fp32 or rounded to bf16."""
    g = _gen(seed)
    x = torch.randn(batch, cols, generator=g)
    return x.to(dtype)


def special_values_bf16() -> list[int]:
    """bf16 bit patterns that must round-trip exactly: +-0, subnormal extremes,
    the largest finite value, +-Inf and NaNs with payloads."""
    return [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x807F, 0x0080, 0x7F7F, 0xFF7F,
            0x7F80, 0xFF80, 0x7FC0, 0x7FC1, 0xFFFF, 0x7F81, 0x3F80, 0xBF80]


# Broad parity sweep: seeded random configurations over shape, weight recipe,
# encoder options and batch size, so that every kernel meets ragged rows,
# narrow and wide rows, every block size family and raw groups of every
# density.  Recipes:
#   gauss     N(0, sigma), sigma = 10^U(-4, 0.5)
#   outliers  N(0, 0.02) with a Bernoulli(rate) mask replaced by N(0, 1),
#             rate = 10^U(-3, -1)
#   randbits  uniformly random 16-bit patterns (decompression only)
#   finite    gauss with 1 % of entries replaced by finite special values
#             (+-0, subnormal extremes, +-1)
#   special   gauss with 1 % of entries replaced by any special value
#             (NaN and Inf included: decompression only)
SWEEP_SEED = 20261202
_SWEEP_ROWS = (1, 2, 3, 7, 16, 17, 31, 64, 65, 100, 128, 129, 200, 257)
_SWEEP_COLS64 = (1, 2, 3, 5, 8, 13, 16, 17, 31, 32, 48, 64, 80)
_SWEEP_G = (0, 16, 32, 48, 64, 112, 128, 224, 256, 512, 1024)  # 0: the encoder's default
_SWEEP_KL = ((0, 0), (16, 6), (8, 4), (1, 1), (32, 8), (24, 5), (12, 12), (4, 2))  # 0: default
_SWEEP_BATCH = (1, 2, 3, 5, 8, 16, 17, 33, 64)
_SWEEP_RECIPES = ("gauss", "outliers", "randbits", "finite", "special")


def sweep_cases(n: int = 32, seed: int = SWEEP_SEED) -> list[dict]:
    """n seeded random configurations for the parity sweep."""
    g = _gen(seed)

    def pick(seq):
        return seq[int(torch.randint(0, len(seq), (1,), generator=g))]

    cases = []
    for i in range(n):
        K, L = pick(_SWEEP_KL)
        # the first cases pin one recipe each so every recipe is present
        recipe = _SWEEP_RECIPES[i] if i < len(_SWEEP_RECIPES) else pick(_SWEEP_RECIPES)
        cases.append({
            "id": i, "rows": pick(_SWEEP_ROWS), "cols": 64 * pick(_SWEEP_COLS64), "recipe": recipe,
            "K": K, "L": L, "G": pick(_SWEEP_G), "batch": pick(_SWEEP_BATCH),
            "sigma": float(10.0 ** (torch.rand(1, generator=g) * 4.5 - 4.0)),
            "rate": float(10.0 ** (torch.rand(1, generator=g) * 2.0 - 3.0)),
            "seed": seed + 1 + i,
        })
    return cases


def sweep_weights(case: dict) -> torch.Tensor:
    """The weights (int16 bit view) of a sweep configuration."""
    r, c, s = case["rows"], case["cols"], case["seed"]
    rec = case["recipe"]
    if rec == "randbits":
        return random_bits_bf16(r, c, s)
    if rec == "outliers":
        return gaussian_with_outliers_bf16(r, c, SIGMA, case["rate"], s)
    w = gaussian_bf16(r, c, case["sigma"], s)
    if rec in ("finite", "special"):
        g = _gen(s + 7)
        vals = special_values_bf16()
        if rec == "finite":
            vals = [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x807F, 0x0080, 0x3F80, 0xBF80]
        table = torch.tensor([v - 65536 if v >= 32768 else v for v in vals], dtype=torch.int16)
        mask = torch.rand(r, c, generator=g) < 0.01
        pick = torch.randint(0, len(vals), (r, c), generator=g)
        w = torch.where(mask, table[pick], w)
    return w
