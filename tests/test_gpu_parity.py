"""GPU parity: the library's kernels against the CPU oracle, through the C-ABI.

Decompression is bit-exact against the original weights (the method is
lossless, so the oracle's decode is the identity).  Products use fp32
accumulation and are checked against the fp64 product of the original
weights: max |y - y64| / max(|y64|, rms(y64)) <= 1e-3 for fp32 outputs and
<= 2 bf16 ulp against round-to-nearest-even(y64) for bf16 outputs.  Inputs
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

DEV = torch.device("cuda:0")
TOL = 1e-3


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


def check_f32(y, ref64, what):
    y = y.detach().float().cpu().numpy().astype(np.float64)
    assert products.nonfinite_match(y, ref64), what + ": non-finite pattern differs"
    err = products.rel_error_floored(y, ref64)
    assert err <= TOL, f"{what}: rel err {err:.3e}"
    return err


def check_bf16(y, ref64, what):
    """Within 2 bf16 ulp of RNE(y64), or RNE of a value inside the fp32
    tolerance band |v - y64| <= TOL * max(|y64|, rms): the fp32 sum's error
    scales with the row's rms, so an output near zero may sit more than 2 bf16
    ulp (of its own tiny magnitude) from RNE(y64)."""
    got = y.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    ref = products.round_to_bf16(ref64)
    fin = np.isfinite(ref64)
    r = ref64[fin]
    k = products.bf16_order_key(got[fin])
    near = products.bf16_ulp_distance(got[fin], ref[fin]) <= 2
    rms = float(np.sqrt(np.mean(r ** 2))) if r.size else 1.0
    eps = TOL * np.maximum(np.abs(r), rms if rms > 0 else 1.0)
    band = (k >= products.bf16_order_key(products.round_to_bf16(r - eps))) & \
           (k <= products.bf16_order_key(products.round_to_bf16(r + eps)))
    bad = ~(near | band)
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs outside 2 bf16 ulp and the fp32 band"
    assert np.array_equal(np.isnan(products.bf16_to_f64(got)), np.isnan(ref64)), what


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
]


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
    check_bf16(yb, ref, f"gemv bf16 {name}")


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
    check_bf16(Yb, ref, f"gemm fused bf16 b={batch}")


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
        check_bf16(Yb, ref, f"gemm mfma bf16 b={batch}")


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


@pytest.mark.parametrize("batch", [2, 3, 40, 64])
def test_gemm_auto_without_plan(batch):
    # every heuristic branch of AUTO (VALU, matrix cores, decompress + GEMM with
    # a workspace, matrix cores without one) against the fp64 product
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
    # up to batch 8 the GEMV-style kernel, above it the library GEMM
    for batch in (1, 3, 8, 9, 40):
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
        check_bf16(Yb, ref, f"bf16 gemm b={batch} bf16 out")


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
    check_bf16(Y, ref, "decompress+gemm bf16 out")
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
        assert uw.uw_get_plan(m.handle, batch)["variant"] == plan["variant"]
        X = workloads.activations(14336, batch, seed=600 + batch, dtype=torch.bfloat16).to(DEV)
        ws = m.workspace(batch)
        Ya = m.gemm(X, variant=uw.UW_VARIANT_AUTO, ws=ws)
        Yv = m.gemm(X, variant=plan["variant"], ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(Ya, Yv)


def test_device_argument_errors_are_caught_on_host():
    wb, m = matrix("small", None, None, None)
    out = torch.empty(1024, 1024, dtype=torch.int16, device=DEV)
    with pytest.raises(uw.UwError) as e:
        uw.uw_decompress(m.handle, out, 1000)
    assert e.value.status == uw.UW_ERR_INVALID
    with pytest.raises(uw.UwError):
        uw.uw_decompress(m.handle, out.view(-1)[1:].view(1, -1)[:, :1024 * 1023], 1024 * 1024)
    x = torch.zeros(1024, dtype=torch.float16, device=DEV)
    with pytest.raises(TypeError):
        m.gemv(x)
    with pytest.raises(uw.UwError) as e:
        uw.uw_gemm_fused(m.handle, torch.zeros(4, 1024, dtype=torch.bfloat16, device=DEV),
                         torch.zeros(4, 1024, device=DEV), uw.UW_VARIANT_DECOMPRESS_GEMM, None)
    assert e.value.status == uw.UW_ERR_NOSPACE


def test_read_probe():
    src = torch.arange(1 << 20, dtype=torch.int32, device=DEV)
    sink = torch.zeros(uw.uw_read_probe_sink_size() // 4, dtype=torch.int32, device=DEV)
    _say("read probe")
    uw.uw_read_probe(src, sink)
    torch.cuda.synchronize()
    # xor of all words: every workgroup folds a disjoint share
    total = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert total == np.bitwise_xor.reduce(np.arange(1 << 20, dtype=np.uint32))
