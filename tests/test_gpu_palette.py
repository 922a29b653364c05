"""GPU parity of the direct-palette pipeline (UWP1) through the C-ABI.

The blobs come from the library's host encoder, which the CPU tests hold
byte-identical to oracle/palette.py.  Decompression must give back the
original weights bit for bit (the form is lossless); the fused GEMV is checked
against the fp64 product of the original weights with the same bars as the
Huffman pipeline: max |y - y64| / max(|y64|, rms(y64)) <= 1e-3 for fp32
outputs, 2 bf16 ulp (or the fp32 band) for bf16 outputs.
"""
import sys

import numpy as np
import pytest
import torch

import workloads
from oracle import palette as opal
from oracle import products

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import decode_gemv_canonical_amd as uw  # noqa: E402

from tests.parity import check_bf16, check_f32  # noqa: E402

DEV = torch.device("cuda:0")


def _say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


_cache = {}


def wide_exponents(rows, cols, seed):
    # random sign and mantissa, exponents uniform over 64 values (2^-31 ..
    # 2^32): every 64-weight group holds exponents outside any palette of 16,
    # and no product overflows fp32 (random bit patterns would: their fp32
    # sums can reach Inf where the fp64 reference stays finite)
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 1 << 16, size=(rows, cols), dtype=np.uint32)
    e = rng.integers(96, 160, size=(rows, cols), dtype=np.uint32)
    return ((bits & 0x807F) | (e << 7)).astype(np.uint16)


def pmatrix(name, rows=None, cols=None, seed=None):
    key = (name, rows, cols, seed)
    if key not in _cache:
        if name == "wide_exponents":
            wb = wide_exponents(rows, cols, seed)
        else:
            wb = workloads.weights(name, rows=rows, cols=cols, seed=seed).numpy().view(np.uint16)
        _cache[key] = (wb, uw.PaletteMatrix.from_weights(wb, device="cuda:0"))
    return _cache[key]


CASES = [
    ("small", None, None, None),       # 1024 x 1024, one tile per row
    ("gate", None, None, None),        # 14336 x 4096 (0.5 % raw groups)
    ("down", None, None, None),        # 4096 x 14336, outliers (8 % raw groups)
    ("randbits", 2048, 8192, None),    # every group raw
    ("gate", 37, 3072, 21),            # ragged: rows not a multiple of the rows per wave
    ("down", 1, 1024, 22),             # one row
    ("down", 5, 7168, 23),             # a row of 7 tiles (chunks of 4 cross rows)
    ("down", 3, 67584, 24),            # 66 tiles per row: a wave re-reads its tile flags after 64
]


@pytest.mark.parametrize("name,rows,cols,seed", CASES)
def test_palette_decompress_bit_exact(name, rows, cols, seed):
    wb, m = pmatrix(name, rows, cols, seed)
    _say(f"palette decompress {name} {wb.shape}")
    out = m.decompress()
    torch.cuda.synchronize()
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), wb)


def test_palette_decompress_strided_output():
    wb, m = pmatrix("gate", 37, 3072, 21)
    _say("palette decompress strided")
    big = torch.full((37, 3072 + 64), -1, dtype=torch.int16, device=DEV)
    uw.uw_palette_decompress(m.handle, big, 3072 + 64)
    torch.cuda.synchronize()
    got = big.cpu().numpy().view(np.uint16)
    assert np.array_equal(got[:, :3072], wb)
    assert (got[:, 3072:] == 0xFFFF).all()


@pytest.mark.parametrize("xdt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("name,rows,cols,seed", CASES)
def test_palette_gemv(name, rows, cols, seed, xdt):
    wb, m = pmatrix(name, rows, cols, seed)
    x = workloads.activations(wb.shape[1], 1, seed=(seed or 0) + 300, dtype=xdt)[0]
    ref = products.gemm_f64(wb, x.float().numpy())
    _say(f"palette gemv {name} {wb.shape} x={xdt}")
    y = m.gemv(x.to(DEV))
    yb = m.gemv(x.to(DEV), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    check_f32(y, ref, f"palette gemv {name}")
    check_bf16(yb, ref, f"palette gemv bf16 {name}", wb.shape[1])


def test_palette_gemv_one_hot_is_exact():
    wb, m = pmatrix("down", 5, 7168, 23)
    for k in (0, 15, 16, 1023, 1024, 7167):
        x = torch.zeros(7168, dtype=torch.bfloat16)
        x[k] = 1.0
        _say(f"palette gemv one-hot k={k}")
        y = m.gemv(x.to(DEV))
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy(), products.bf16_to_f32(wb[:, k]))


def test_palette_matches_oracle_form_on_special_values():
    wb = workloads.weights("small", rows=8, cols=1024).numpy().view(np.uint16).copy()
    wb[3, :8] = [0x7FC1, 0xFF80, 0x7F80, 0x0001, 0x8001, 0x0000, 0x8000, 0xFFFF]
    blob = opal.encode(wb)  # the oracle's bytes, handed to the device path
    m = uw.PaletteMatrix(blob, device="cuda:0")
    _say("palette special values")
    out = m.decompress()
    torch.cuda.synchronize()
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), wb)


def test_palette_argument_errors():
    wb, m = pmatrix("small", None, None, None)
    x = torch.zeros(1025, dtype=torch.bfloat16, device=DEV)
    y = torch.empty(1024, device=DEV)
    with pytest.raises(uw.UwError):
        uw.uw_palette_gemv(m.handle, x[1:], y)  # misaligned x
    out = torch.empty(1024, 1028, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(uw.UwError):
        uw.uw_palette_decompress(m.handle, out, 1028)  # ld not a multiple of 8


# Matrix-core product over the palette form: 1, 2 and 4 blocks of 16 rows
# per workgroup and 2 to 8 waves splitting K (both set by the row count), one
# or two register sets (set by the batch tiles and row blocks); several
# passes, ragged batches and row counts, raw groups, every group raw.
GEMM_CASES = [
    ("down", 8192, 2048, 43, [2, 33]),          # 2 row blocks, 8 % raw groups, a partial batch tile
    ("wide_exponents", 8192, 1024, 44, [5]),   # every group raw (64 exponents, all finite)
    ("down", 3, 67584, 24, [3, 20]),           # 66 tiles per row
    ("down", 2072, 4096, 45, [7, 40]),         # 40 rows: two workgroups per 32 rows split K, the last group partial
    ("gate", None, None, None, [16, 32, 64]),   # 4 row blocks per workgroup, 8 waves split K
    ("down", None, None, None, [4, 64, 100]),  # 1 row block per workgroup, 8 waves; 100 = two passes
    ("gate", 28672, 1024, 31, [3]),            # 4 row blocks per workgroup, 4 waves split K
    ("gate", 14344, 1024, 42, [9, 40]),        # 4 row blocks per workgroup, the last one partial
    ("big", 8192, 1024, 41, [20]),             # 2 row blocks per workgroup
    ("gate", 37, 3072, 21, [1, 5, 17]),        # a partial row block
    ("randbits", 48, 2048, None, [7]),         # every group raw
    ("down", 1, 1024, 22, [2]),                # one row
]


@pytest.mark.parametrize("case", GEMM_CASES, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}")
def test_palette_gemm(case):
    name, rows, cols, seed, batches = case
    wb, m = pmatrix(name, rows, cols, seed)
    for batch in batches:
        X = workloads.activations(wb.shape[1], batch, seed=900 + batch, dtype=torch.bfloat16)
        ref = products.gemm_f64(wb, X.float().numpy())
        _say(f"palette gemm {name} {wb.shape} batch={batch}")
        Y = m.gemm(X.to(DEV))
        Yb = m.gemm(X.to(DEV), out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        check_f32(Y, ref, f"palette gemm {name} b={batch}")
        check_bf16(Yb, ref, f"palette gemm bf16 {name} b={batch}", wb.shape[1])


def test_palette_gemm_split_is_deterministic():
    # at 17..64 batch rows with fp32 Y, matrices with few row blocks run two
    # workgroups per group of rows, each adding half of K into Y: two partial
    # sums added to zero give the same bits in either order
    wb, m = pmatrix("down", 2072, 4096, 45)
    for batch in (17, 64):
        X = workloads.activations(wb.shape[1], batch, seed=950 + batch, dtype=torch.bfloat16).to(DEV)
        _say(f"palette gemm split determinism batch={batch}")
        ys = [m.gemm(X) for _ in range(3)]
        yb = m.gemm(X, out_dtype=torch.bfloat16)  # bf16 Y: one workgroup per group
        torch.cuda.synchronize()
        assert all(torch.equal(ys[0], y) for y in ys[1:])
        ref = products.gemm_f64(wb, X.float().cpu().numpy())
        check_f32(ys[0], ref, f"palette gemm split b={batch}")
        check_bf16(yb, ref, f"palette gemm split bf16 b={batch}", wb.shape[1])


def test_palette_gemm_strided_and_errors():
    wb, m = pmatrix("gate", 37, 3072, 21)
    X = workloads.activations(3072, 9, seed=77, dtype=torch.bfloat16)
    Xs = torch.zeros(9, 3072 + 64, dtype=torch.bfloat16)
    Xs[:, :3072] = X
    Ys = torch.full((9, 37 + 11), 7.0, device=DEV)
    _say("palette gemm strided")
    uw.uw_palette_gemm(m.handle, Xs.to(DEV)[:, :3072], Ys[:, :37])
    torch.cuda.synchronize()
    check_f32(Ys[:, :37], products.gemm_f64(wb, X.float().numpy()), "palette gemm strided")
    assert (Ys[:, 37:].cpu() == 7.0).all()
    with pytest.raises(uw.UwError):
        uw.uw_palette_gemm(m.handle, X.float().to(DEV), torch.empty(9, 37, device=DEV))  # fp32 X
