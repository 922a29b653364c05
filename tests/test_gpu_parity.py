"""GPU parity: the library's kernels against the CPU oracle, through the C-ABI.

Decompression is bit-exact against the original weights (the method is
lossless, so the oracle's decode is the identity).  Products use fp32
accumulation and are checked against the fp64 product of the original
weights: max |y - y64| / max(|y64|, rms(y64)) <= 1e-3 for fp32 outputs; bf16
outputs within 2 bf16 ulp of round-to-nearest-even(y64), or RNE of a value
inside the fp32 accumulation band (the rule and its cap are in tests/parity.py).  Inputs
are the seeded synthetic workloads of workloads.py, at full size for the
benchmarked configurations and at small, ragged sizes for the edge cases.
"""
import sys

import numpy as np
import pytest
import torch

import workloads
from oracle import blob as oblob
from oracle import products

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import decode_gemv_canonical_amd as uw  # noqa: E402
from tests.parity import TOL, check_bf16, check_f32  # noqa: E402,F401

DEV = torch.device("cuda:0")


def _say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


_cache = {}


def matrix(name, rows=None, cols=None, seed=None, **opts):
    key = (name, rows, cols, seed, tuple(sorted(opts.items())))
    if key not in _cache:
        w = workloads.weights(name, rows=rows, cols=cols, seed=seed)
        wb = w.numpy().view(np.uint16)
        m = uw.CompressedMatrix.from_weights(w, device="cuda:0", **opts)
        _cache[key] = (wb, m)
    return _cache[key]


DECOMP_CASES = [
    ("small", None, None, None, {}),
    ("gate", None, None, None, {}),
    ("down", None, None, None, {}),
    ("big", None, None, None, {}),
    ("randbits", 1024, 2048, None, {}),
    ("down", 13, 512, 7, {"G": 48}),
    ("down", 5, 1024, 8, {"G": 16}),
    ("gate", 67, 4096, 16, {"G": 224}),
    ("down", 24, 14336, 17, {"G": 256}),
    ("small", 50, 3072, 18, {"G": 80}),
    ("small", 37, 1600, 9, {"K": 32, "L": 8}),
    ("small", 21, 960, 10, {"K": 16, "L": 12}),
    ("small", 9, 128, 12, {"K": 1, "L": 1}),
]


@pytest.mark.parametrize("name,rows,cols,seed,opts", DECOMP_CASES)
def test_decompress_bit_exact(name, rows, cols, seed, opts):
    wb, m = matrix(name, rows, cols, seed, **opts)
    _say(f"decompress {name} {wb.shape} {opts}")
    out = m.decompress()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16).cpu(), torch.from_numpy(wb.view(np.int16)))


def test_decompress_strided_output():
    wb, m = matrix("down", 13, 512, 7, G=48)
    _say("decompress strided")
    out = torch.full((13, 520), 7, dtype=torch.int16, device=DEV)
    uw.uw_decompress(m.handle, out, 520)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.array_equal(o[:, :512].view(np.uint16), wb) and (o[:, 512:] == 7).all()


def test_decompress_special_values():
    sv = np.array(workloads.special_values_bf16(), dtype=np.uint16)
    base = workloads.weights("small", rows=32, cols=256, seed=9).numpy().view(np.uint16).copy()
    base.ravel()[::97][: len(sv)] = sv
    for w in (base, np.resize(sv, (8, 128))):
        m = uw.CompressedMatrix(uw.uw_encode(w, flags=uw.UW_ENC_NO_PLAIN), device="cuda:0")
        _say(f"decompress special {w.shape}")
        out = m.decompress()
        torch.cuda.synchronize()
        assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), w)


GEMV_CASES = [
    ("small", None, None, None, {}, torch.float32),
    ("gate", None, None, None, {}, torch.bfloat16),
    ("down", None, None, None, {}, torch.bfloat16),
    ("big", None, None, None, {}, torch.bfloat16),
    ("down", 13, 512, 7, {"G": 48}, torch.bfloat16),
    ("down", 5, 1024, 8, {"G": 16}, torch.float32),
    ("small", 37, 1600, 9, {"K": 32, "L": 8}, torch.bfloat16),
    ("small", 21, 960, 10, {"K": 16, "L": 12}, torch.float32),
    ("small", 9, 128, 12, {"K": 1, "L": 1}, torch.bfloat16),
    ("gate", 33, 4096, 13, {"G": 64}, torch.bfloat16),
    ("small", 7, 64 * 7, 14, {}, torch.bfloat16),
    # blocks that end mid-row (G above the groups per row, not a multiple):
    # one wave per block, the crossing rows summed from two waves' parts
    ("gate", 70, 4096, 15, {"G": 224}, torch.bfloat16),
    ("gate", 67, 4096, 16, {"G": 224}, torch.float32),
    ("down", 24, 14336, 17, {"G": 256}, torch.bfloat16),
    ("small", 50, 3072, 18, {"G": 80}, torch.float32),
    # work units of more than 64 rows (the lcm of G and a groups-per-row
    # count prime to it): the finished rows parked in lanes are stored every 64
    ("small", 200, 320, 19, {"G": 1024}, torch.bfloat16),
    ("down", 150, 448, 20, {"G": 512}, torch.float32),
]


@pytest.mark.parametrize("batch", [3, 8])
def test_gemm_fused_valu_long_units(batch):
    wb, m = matrix("small", 200, 320, 19, G=1024)
    X = workloads.activations(320, batch, seed=310 + batch, dtype=torch.bfloat16)
    ref = products.gemm_f64(wb, X.float().numpy())
    _say(f"gemm fused long units batch={batch}")
    Y = m.gemm(X.to(DEV), variant=uw.UW_VARIANT_FUSED)
    torch.cuda.synchronize()
    check_f32(Y, ref, f"gemm fused long units b={batch}")


@pytest.mark.parametrize("name,rows,cols,seed,opts,xdt", GEMV_CASES)
def test_gemv_fused(name, rows, cols, seed, opts, xdt):
    wb, m = matrix(name, rows, cols, seed, **opts)
    x = workloads.activations(wb.shape[1], 1, seed=(seed or 0) + 100, dtype=xdt)[0]
    ref = products.gemm_f64(wb, x.float().numpy())
    _say(f"gemv {name} {wb.shape} {opts} x={xdt}")
    y = m.gemv(x.to(DEV))
    yb = m.gemv(x.to(DEV), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    check_f32(y, ref, f"gemv {name}")
    check_bf16(yb, ref, f"gemv bf16 {name}", wb.shape[1])


def test_gemv_one_hot_is_exact():
    wb, m = matrix("gate", 33, 4096, 13, G=64)
    for k in (0, 63, 64, 4095):
        x = torch.zeros(4096, dtype=torch.bfloat16)
        x[k] = 1.0
        _say(f"gemv one-hot k={k}")
        y = m.gemv(x.to(DEV))
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy(), products.bf16_to_f32(wb[:, k]))


def test_gemv_scale_by_two_is_exact():
    wb, m = matrix("small", None, None, None)
    e, sm = oblob.huffman.split_bf16(wb)
    assert (e < 250).all()
    w2 = oblob.huffman.join_bf16(np.where(e > 0, e + 1, e), sm)
    keep = (e > 0).all(axis=1)
    m2 = uw.CompressedMatrix(uw.uw_encode(w2), device="cuda:0")
    x = workloads.activations(1024, 1, seed=5, dtype=torch.float32)[0].to(DEV)
    _say("gemv scale by two")
    y1, y2 = m.gemv(x), m2.gemv(x)
    torch.cuda.synchronize()
    assert torch.equal((2 * y1)[torch.from_numpy(keep).to(DEV)], y2[torch.from_numpy(keep).to(DEV)])


@pytest.mark.parametrize("batch", [1, 2, 3, 4, 5, 8, 11])
@pytest.mark.parametrize("G", [256, 224])
def test_gemm_fused_valu(batch, G):
    wb, m = matrix("gate", 96, 4096, 21, G=G)
    X = workloads.activations(4096, batch, seed=300 + batch, dtype=torch.bfloat16)
    ref = products.gemm_f64(wb, X.float().numpy())
    _say(f"gemm fused batch={batch}")
    Y = m.gemm(X.to(DEV), variant=uw.UW_VARIANT_FUSED)
    Yb = m.gemm(X.to(DEV), variant=uw.UW_VARIANT_FUSED, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    check_f32(Y, ref, f"gemm fused b={batch}")
    check_bf16(Yb, ref, f"gemm fused bf16 b={batch}", wb.shape[1])


@pytest.mark.parametrize("batch", [1, 4, 16, 64])
def test_gemm_down_both_variants(batch):
    wb, m = matrix("down", None, None, None)
    X = workloads.activations(14336, batch, seed=400 + batch, dtype=torch.bfloat16)
    ref = products.gemm_f64(wb, X.float().numpy())
    ws = m.workspace(batch)
    for v in (uw.UW_VARIANT_FUSED, uw.UW_VARIANT_DECOMPRESS_GEMM, uw.UW_VARIANT_FUSED_MFMA):
        _say(f"gemm down batch={batch} variant={v}")
        Y = m.gemm(X.to(DEV), variant=v, ws=ws)
        torch.cuda.synchronize()
        check_f32(Y, ref, f"gemm down b={batch} v={v}")


# Matrix-core path: every shape of work unit (G a multiple of the groups per
# row with 1, 2 or 4 rows per block; G dividing a row; units of several
# blocks and rows; a partial last block), raw groups, the single-code table (L > 6), partial
# batch tiles and more than one 64-row pass.
MFMA_CASES = [
    ("small", None, None, None, {}, (16, 17, 64)),
    ("gate", 64, 4096, 41, {"G": 256}, (32, 48)),
    ("down", 48, 14336, 42, {"G": 112}, (16, 33)),
    ("small", 13, 1024, 43, {"G": 64}, (16,)),
    ("small", 40, 2048, 44, {"K": 32, "L": 8}, (20,)),
    ("big", 96, 8192, 45, {}, (100,)),
    # work units of several blocks and rows (G neither divides nor is a
    # multiple of the groups per row), with a partial last unit
    ("gate", 67, 4096, 46, {"G": 224}, (16, 40)),
    ("down", 24, 14336, 47, {"G": 256}, (16,)),
    ("small", 50, 3072, 48, {"G": 80}, (20,)),
]


@pytest.mark.parametrize("case", MFMA_CASES, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}-{c[4]}")
def test_gemm_fused_mfma(case):
    name, rows, cols, seed, opts, batches = case
    wb, m = matrix(name, rows, cols, seed, **opts)
    C = wb.shape[1]
    for batch in batches:
        X = workloads.activations(C, batch, seed=700 + batch, dtype=torch.bfloat16)
        ref = products.gemm_f64(wb, X.float().numpy())
        _say(f"gemm mfma {name} {wb.shape} {opts} batch={batch}")
        Y = m.gemm(X.to(DEV), variant=uw.UW_VARIANT_FUSED_MFMA)
        Yb = m.gemm(X.to(DEV), variant=uw.UW_VARIANT_FUSED_MFMA, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        check_f32(Y, ref, f"gemm mfma b={batch}")
        check_bf16(Yb, ref, f"gemm mfma bf16 b={batch}", wb.shape[1])


def test_gemm_fused_mfma_full_sizes():
    # the 32-row batch of a gate projection, and the 256-row batch on the 8192 x 8192
    # matrix with outputs sampled on 384 rows (fp64 oracle per sampled row)
    wb, m = matrix("gate", None, None, None)
    X = workloads.activations(4096, 32, seed=801, dtype=torch.bfloat16)
    _say("gemm mfma gate 14336x4096 batch=32")
    Y = m.gemm(X.to(DEV), variant=uw.UW_VARIANT_FUSED_MFMA)
    torch.cuda.synchronize()
    check_f32(Y, products.gemm_f64(wb, X.float().numpy()), "gate b=32")
    wb, m = matrix("big", None, None, None)
    X = workloads.activations(8192, 256, seed=802, dtype=torch.bfloat16)
    _say("gemm mfma big 8192x8192 batch=256")
    Y = m.gemm(X.to(DEV), variant=uw.UW_VARIANT_FUSED_MFMA)
    torch.cuda.synchronize()
    rows = np.random.default_rng(5).choice(8192, size=384, replace=False)
    ref = products.gemm_f64(wb[rows], X.float().numpy())
    check_f32(Y[:, rows], ref, "big b=256 sampled rows")


def test_gemm_fused_mfma_is_deterministic_and_checks_support():
    wb, m = matrix("down", 48, 14336, 42, G=112)
    X = workloads.activations(14336, 24, seed=803, dtype=torch.bfloat16).to(DEV)
    Y1 = m.gemm(X, variant=uw.UW_VARIANT_FUSED_MFMA)
    Y2 = m.gemm(X, variant=uw.UW_VARIANT_FUSED_MFMA)
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int32), Y2.view(torch.int32))
    # fp32 activations, misaligned rows and cols that are not a multiple of 1024 are refused
    with pytest.raises(uw.UwError) as e:
        m.gemm(X.float(), variant=uw.UW_VARIANT_FUSED_MFMA)
    assert e.value.status == uw.UW_ERR_UNSUPPORTED
    Xs = torch.zeros(24, 14336 + 4, dtype=torch.bfloat16, device=DEV)[:, :14336]
    with pytest.raises(uw.UwError) as e:
        m.gemm(Xs, variant=uw.UW_VARIANT_FUSED_MFMA)
    assert e.value.status == uw.UW_ERR_UNSUPPORTED
    wb2, m2 = matrix("small", 37, 1600, 9, K=32, L=8)
    X2 = workloads.activations(1600, 16, seed=804, dtype=torch.bfloat16)
    with pytest.raises(uw.UwError) as e:
        m2.gemm(X2.to(DEV), variant=uw.UW_VARIANT_FUSED_MFMA)
    assert e.value.status == uw.UW_ERR_UNSUPPORTED
    # AUTO falls back to a path that can run it
    Y = m2.gemm(X2.to(DEV), variant=uw.UW_VARIANT_AUTO, ws=m2.workspace(16))
    torch.cuda.synchronize()
    check_f32(Y, products.gemm_f64(wb2, X2.float().numpy()), "auto fallback")


def test_gemm_fp32_input_strided():
    wb, m = matrix("down", 5, 1024, 8, G=16)
    X = workloads.activations(1100, 3, seed=7, dtype=torch.float32)
    ref = products.gemm_f64(wb, X[:, :1024].numpy())
    Xd = X.to(DEV)[:, :1024]
    Y = torch.zeros(3, 8, device=DEV)
    _say("gemm strided fp32")
    uw.uw_gemm_fused(m.handle, Xd, Y[:, :5], uw.UW_VARIANT_FUSED)
    torch.cuda.synchronize()
    check_f32(Y[:, :5], ref, "strided")
    assert (Y[:, 5:] == 0).all()


@pytest.mark.parametrize("batch", [3, 8])
def test_gemm_fused_valu_fp32_split_rows(batch):
    # fp32 activations (8 rows: the 8-wave workgroup) on blocks that end mid-row
    wb, m = matrix("gate", 67, 4096, 16, G=224)
    X = workloads.activations(4096, batch, seed=320 + batch, dtype=torch.float32)
    ref = products.gemm_f64(wb, X.numpy())
    _say(f"gemm fused fp32 split batch={batch}")
    Y = m.gemm(X.to(DEV), variant=uw.UW_VARIANT_FUSED)
    torch.cuda.synchronize()
    check_f32(Y, ref, f"gemm fused fp32 split b={batch}")


@pytest.mark.parametrize("batch", [2, 3, 8, 16, 40, 64])
def test_gemm_auto_without_plan(batch):
    # every heuristic branch of AUTO (VALU up to 8 rows, matrix cores, decompress
    # + GEMM with a workspace, matrix cores without one) against the fp64 product
    wb, m = matrix("gate", 70, 4096, 15, G=224)
    X = workloads.activations(4096, batch, seed=330 + batch, dtype=torch.bfloat16)
    ref = products.gemm_f64(wb, X.float().numpy())
    for ws in (m.workspace(batch), None):
        _say(f"gemm auto batch={batch} ws={ws is not None}")
        Y = m.gemm(X.to(DEV), variant=uw.UW_VARIANT_AUTO, ws=ws)
        torch.cuda.synchronize()
        check_f32(Y, ref, f"gemm auto b={batch}")


def test_gemm_batch_zero_is_noop():
    wb, m = matrix("small", None, None, None)
    X = torch.zeros(0, 1024, dtype=torch.bfloat16, device=DEV)
    Y = torch.zeros(0, 1024, device=DEV)
    uw.uw_gemm_fused(m.handle, X, Y, uw.UW_VARIANT_FUSED)


def test_bf16_gemm_uncompressed():
    wb, _ = matrix("gate", 96, 4096, 21)
    W = torch.from_numpy(wb.view(np.int16)).to(DEV).view(torch.bfloat16)
    # batch 1 (x fits the GEMV-style kernel's LDS) and fp32 X on the vector
    # ALU, every other aligned bf16 batch on the matrix cores
    for batch in (1, 2, 3, 8, 9, 40, 256):
        X = workloads.activations(4096, batch, seed=500 + batch, dtype=torch.bfloat16)
        ref = products.gemm_f64(wb, X.float().numpy())
        Y = torch.empty(batch, 96, device=DEV)
        _say(f"bf16 gemm batch={batch}")
        uw.uw_bf16_gemm(W, X.to(DEV), Y)
        torch.cuda.synchronize()
        check_f32(Y, ref, f"bf16 gemm b={batch}")
        Yb = torch.empty(batch, 96, device=DEV, dtype=torch.bfloat16)
        uw.uw_bf16_gemm(W, X.to(DEV), Yb)
        torch.cuda.synchronize()
        check_bf16(Yb, ref, f"bf16 gemm b={batch} bf16 out", wb.shape[1])
        if batch <= 8:
            Yf = torch.empty(batch, 96, device=DEV)
            uw.uw_bf16_gemm(W, X.float().to(DEV), Yf)  # fp32 X: the vector kernel's passes
            torch.cuda.synchronize()
            check_f32(Yf, products.gemm_f64(wb, X.float().numpy()), f"bf16 gemm b={batch} fp32 x")
    # one row of X wider than 8192 columns: the matrix cores
    wd, _ = matrix("down", 48, 14336, 22)
    Wd = torch.from_numpy(wd.view(np.int16)).to(DEV).view(torch.bfloat16)
    X = workloads.activations(14336, 1, seed=509, dtype=torch.bfloat16)
    Y = torch.empty(1, 48, device=DEV)
    uw.uw_bf16_gemm(Wd, X.to(DEV), Y)
    torch.cuda.synchronize()
    check_f32(Y, products.gemm_f64(wd, X.float().numpy()), "bf16 gemm b=1 cols=14336")


def test_bf16_gemm_every_shape_ragged():
    # rows not a multiple of 16 (or 64), cols not a multiple of 128, batch
    # not a multiple of 16, a row stride wider than cols
    rows, cols = 100, 1000
    wfull, _ = matrix("small", rows, 1024, 24)
    wb = np.ascontiguousarray(wfull[:, :cols])
    Wp = torch.from_numpy(wfull.view(np.int16)).to(DEV).view(torch.bfloat16)
    W = Wp[:, :cols]
    for batch in (1, 5, 9, 37, 100):
        X = workloads.activations(cols, batch, seed=520 + batch, dtype=torch.bfloat16)
        ref = products.gemm_f64(wb, X.float().numpy())
        Xd = X.to(DEV)
        for shape in range(1, uw.uw_bf16_gemm_shape_count()):
            for ks in (0, 1, 2, 8):
                Y = torch.full((batch, rows + 3), float("nan"), device=DEV)
                uw.uw_bf16_gemm_shaped(W, Xd, Y[:, :rows], shape, ks)
                torch.cuda.synchronize()
                check_f32(Y[:, :rows], ref, f"bf16 gemm shape={shape} ks={ks} b={batch}")
                assert torch.isnan(Y[:, rows:]).all(), "wrote past the rows"
    # cols a multiple of 128: the LDS-stage kernels (shapes 14, 15) run too
    w2, _ = matrix("small", 100, 1024, 25)
    W2 = torch.from_numpy(w2.view(np.int16)).to(DEV).view(torch.bfloat16)
    for batch in (9, 100, 200):
        X = workloads.activations(1024, batch, seed=540 + batch, dtype=torch.bfloat16)
        ref = products.gemm_f64(w2, X.float().numpy())
        for shape in range(1, uw.uw_bf16_gemm_shape_count()):
            Y = torch.full((batch, 103), float("nan"), device=DEV)
            uw.uw_bf16_gemm_shaped(W2, X.to(DEV), Y[:, :100], shape, 0)
            torch.cuda.synchronize()
            check_f32(Y[:, :100], ref, f"bf16 gemm 100x1024 shape={shape} b={batch}")
            assert torch.isnan(Y[:, 100:]).all(), "wrote past the rows"
    # the K-split shapes (17, 18): an odd number of k-blocks (9), fp32 and
    # bf16 Y (bf16 runs one workgroup per tile), the same result twice
    w3, _ = matrix("small", 200, 1152, 26)
    W3 = torch.from_numpy(w3.view(np.int16)).to(DEV).view(torch.bfloat16)
    for batch in (20, 64):
        X = workloads.activations(1152, batch, seed=560 + batch, dtype=torch.bfloat16).to(DEV)
        ref = products.gemm_f64(w3, X.float().cpu().numpy())
        for shape in (17, 18):
            Y = torch.full((batch, 205), float("nan"), device=DEV)
            uw.uw_bf16_gemm_shaped(W3, X, Y[:, :200], shape, 0)
            Y2 = torch.empty(batch, 200, device=DEV)
            uw.uw_bf16_gemm_shaped(W3, X, Y2, shape, 0)
            Yb = torch.empty(batch, 200, device=DEV, dtype=torch.bfloat16)
            uw.uw_bf16_gemm_shaped(W3, X, Yb, shape, 0)
            torch.cuda.synchronize()
            check_f32(Y[:, :200], ref, f"bf16 gemm split shape={shape} b={batch}")
            assert torch.isnan(Y[:, 200:]).all(), "wrote past the rows"
            assert torch.equal(Y[:, :200], Y2), "split product differs between two runs"
            check_bf16(Yb, ref, f"bf16 gemm split shape={shape} b={batch} bf16 out", 1152)
    # unaligned X (odd element offset): the VALU passes take it
    X = workloads.activations(cols + 1, 12, seed=530, dtype=torch.bfloat16).to(DEV)[:, 1:]
    Y = torch.empty(12, rows, device=DEV)
    uw.uw_bf16_gemm(W, X, Y)
    torch.cuda.synchronize()
    check_f32(Y, products.gemm_f64(wb, X.float().cpu().numpy()), "bf16 gemm unaligned X")


def test_decompress_gemm_bf16_out_strided():
    # decompress into the workspace, then the library GEMM, bf16 Y with a row stride
    wb, m = matrix("gate", 256, 4096, 23)
    batch = 24
    X = workloads.activations(4096, batch, seed=523, dtype=torch.bfloat16)
    ref = products.gemm_f64(wb, X.float().numpy())
    Ybig = torch.zeros(batch, 256 + 64, device=DEV, dtype=torch.bfloat16)
    _say(f"decompress+gemm bf16 out batch={batch}")
    Y = m.gemm(X.to(DEV), variant=uw.UW_VARIANT_DECOMPRESS_GEMM, ws=m.workspace(batch), Y=Ybig[:, :256])
    torch.cuda.synchronize()
    check_bf16(Y, ref, "decompress+gemm bf16 out", wb.shape[1])
    assert torch.all(Ybig[:, 256:] == 0)


def test_plain_mode_products():
    wb, m = matrix("randbits", 1024, 2048, None)
    assert m.info["plain"] == 1
    x = workloads.activations(2048, 1, seed=77, dtype=torch.bfloat16)[0]
    with np.errstate(all="ignore"):
        ref = products.gemm_f64(wb, x.float().numpy())
    _say("plain gemv")
    y = m.gemv(x.to(DEV))
    torch.cuda.synchronize()
    assert products.nonfinite_match(y.cpu().numpy(), ref)


def test_autotune_plan_and_auto_dispatch():
    wb, m = matrix("down", 64, 14336, 31)
    for batch in (1, 16):
        _say(f"autotune batch={batch}")
        plan = m.autotune(batch)
        assert plan["variant"] in (uw.UW_VARIANT_FUSED, uw.UW_VARIANT_DECOMPRESS_GEMM, uw.UW_VARIANT_FUSED_MFMA)
        assert plan["time_us"] == min(plan["candidate_us"].values())
        got = uw.uw_get_plan(m.handle, batch)
        assert (got["variant"], got["knob"]) == (plan["variant"], plan["knob"])
        X = workloads.activations(14336, batch, seed=600 + batch, dtype=torch.bfloat16)
        ref = products.gemm_f64(wb, X.float().numpy())
        X = X.to(DEV)
        ws = m.workspace(batch)
        Ya = m.gemm(X, variant=uw.UW_VARIANT_AUTO, ws=ws)
        torch.cuda.synchronize()
        check_f32(Ya, ref, f"auto after autotune b={batch}")
        # AUTO runs the plan's (variant, knob): the same bits
        Yv = torch.empty_like(Ya)
        uw.uw_gemm_with_plan(m.handle, plan["variant"], plan["knob"], X, Yv, ws)
        torch.cuda.synchronize()
        assert torch.equal(Ya, Yv)


def test_auto_falls_back_when_the_plan_cannot_run():
    # a plan tuned for bf16 X with a workspace must not break calls it cannot
    # serve: fp32 X, or no workspace
    wb, m = matrix("gate", 64, 4096, 32)
    for v, knob in ((uw.UW_VARIANT_DECOMPRESS_GEMM, 0), (uw.UW_VARIANT_FUSED_MFMA, 0)):
        uw.uw_set_plan(m.handle, 4, v, knob=knob)
        for xdt, ws in ((torch.float32, m.workspace(4)), (torch.bfloat16, None), (torch.float32, None)):
            X = workloads.activations(4096, 4, seed=640, dtype=xdt)
            ref = products.gemm_f64(wb, X.float().numpy())
            _say(f"auto fallback plan={v} x={xdt} ws={ws is not None}")
            Y = m.gemm(X.to(DEV), variant=uw.UW_VARIANT_AUTO, ws=ws)
            torch.cuda.synchronize()
            check_f32(Y, ref, f"auto fallback plan={v}")


def test_every_knob_matches_the_oracle():
    wb, m = matrix("gate", 96, 4096, 33)
    for batch in (1, 4, 20, 40, 72):
        X = workloads.activations(4096, batch, seed=650 + batch, dtype=torch.bfloat16)
        ref = products.gemm_f64(wb, X.float().numpy())
        X = X.to(DEV)
        ws = m.workspace(batch)
        knobs = [(uw.UW_VARIANT_FUSED, k) for k in (0, 2, 4, 2 + 8 * 8, 4 + 8 * 4) if batch <= 8]
        knobs += [(uw.UW_VARIANT_FUSED_MFMA, k) for k in (0, 8, 12, 16)]
        knobs += [(uw.UW_VARIANT_DECOMPRESS_GEMM, 0)]
        if batch > 8:
            knobs += [(uw.UW_VARIANT_DECOMPRESS_GEMM, sh + 32 * ks)
                      for sh in range(1, uw.uw_bf16_gemm_shape_count()) for ks in (0, 1, 4)]
        for v, k in knobs:
            Y = torch.full((batch, 96), float("nan"), device=DEV)
            try:
                uw.uw_gemm_with_plan(m.handle, v, k, X, Y, ws)
            except uw.UwError as e:
                assert e.status == uw.UW_ERR_UNSUPPORTED, str(e)
                continue
            torch.cuda.synchronize()
            check_f32(Y, ref, f"knob b={batch} v={v} k={k}")


def test_plan_save_load_round_trip():
    wb, m = matrix("gate", 64, 4096, 34)
    uw.uw_set_plan(m.handle, 4, uw.UW_VARIANT_FUSED_MFMA, time_us=12.5, knob=12)
    uw.uw_set_plan(m.handle, 64, uw.UW_VARIANT_DECOMPRESS_GEMM, time_us=40.0, knob=5 + 32 * 4)
    text = m.save_plans()
    import json
    doc = json.loads(text)
    assert doc["format"] == "uw-plan-1" and doc["rows"] == 64 and doc["cols"] == 4096
    assert [(p["batch"], p["variant"], p["knob"]) for p in doc["plans"]] == \
        [(4, "fused_mfma", 12), (64, "decompress_gemm", 133)]
    fresh = uw.CompressedMatrix.from_weights(workloads.weights("gate", rows=64, cols=4096, seed=34), device="cuda:0")
    fresh.load_plans(text)
    for b in (4, 64):
        a, c = uw.uw_get_plan(m.handle, b), uw.uw_get_plan(fresh.handle, b)
        assert (a["variant"], a["knob"]) == (c["variant"], c["knob"])
    # a plan file of another matrix, or a broken one, is rejected whole
    other = uw.CompressedMatrix.from_weights(workloads.weights("gate", rows=64, cols=4096, seed=35), device="cuda:0")
    for bad in (text, text.replace('"knob": 12', '"knob": 99'), text[:-3], '{"format": "uw-plan-1"}'):
        with pytest.raises(uw.UwError) as e:
            (other if bad == text else fresh).load_plans(bad)
        assert e.value.status == uw.UW_ERR_FORMAT
    with pytest.raises(uw.UwError):
        uw.uw_get_plan(other.handle, 4)
    fresh.close()
    other.close()


def test_device_argument_errors_are_caught_on_host():
    wb, m = matrix("small", None, None, None)
    lib = uw.library()
    out = torch.empty(1024, 1024, dtype=torch.int16, device=DEV)
    # the C-ABI's own checks
    assert lib.uw_decompress(m.handle, out.data_ptr(), 1000, None) == uw.UW_ERR_INVALID
    assert lib.uw_decompress(m.handle, out.data_ptr() + 2, 1024, None) == uw.UW_ERR_INVALID
    X = torch.zeros(4, 1024, dtype=torch.bfloat16, device=DEV)
    Y = torch.zeros(4, 1024, device=DEV)
    with pytest.raises(uw.UwError) as e:
        uw.uw_gemm_fused(m.handle, X, Y, uw.UW_VARIANT_DECOMPRESS_GEMM, None)
    assert e.value.status == uw.UW_ERR_NOSPACE
    # the binding's checks of shapes, strides and devices
    with pytest.raises(ValueError):
        uw.uw_decompress(m.handle, out, 1000)
    with pytest.raises(ValueError):
        uw.uw_decompress(m.handle, out[:512])
    with pytest.raises(TypeError):
        m.gemv(torch.zeros(1024, dtype=torch.float16, device=DEV))
    with pytest.raises(ValueError):
        m.gemv(torch.zeros(1000, dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError):
        uw.uw_gemv_fused(m.handle, torch.zeros(1024, dtype=torch.bfloat16, device=DEV), torch.zeros(512, device=DEV))
    with pytest.raises(ValueError):
        uw.uw_gemm_fused(m.handle, X.t(), Y)
    with pytest.raises(ValueError):
        uw.uw_gemm_fused(m.handle, X, Y[:, :100])
    with pytest.raises(ValueError):
        uw.uw_gemm_fused(m.handle, X.cpu(), Y)


def test_read_probe():
    src = torch.arange(1 << 20, dtype=torch.int32, device=DEV)
    sink = torch.zeros(uw.uw_read_probe_sink_size() // 4, dtype=torch.int32, device=DEV)
    _say("read probe")
    uw.uw_read_probe(src, sink)
    torch.cuda.synchronize()
    # xor of all words: every workgroup folds a disjoint share
    total = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert total == np.bitwise_xor.reduce(np.arange(1 << 20, dtype=np.uint32))
