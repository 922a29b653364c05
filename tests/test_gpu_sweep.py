"""GPU parity over the seeded sweep (workloads.sweep_cases: random shapes,
weight recipes, K, L, G and batch sizes) through the C-ABI: decompression
bit-exact, every product variant that accepts the shape against the oracle's
fp64 product (fp32 outputs max |y - y64| / max(|y64|, rms) <= 1e-3; bf16
outputs under the rule of tests/parity.py), and the direct-palette form
transcoded on the device, equal to the host encoder's bytes for the page's
16-entry palette and decompressing to the original bits.  Random bit
patterns and the special-value recipe (NaN, Inf, values near the largest
bf16, whose fp32 sums overflow where the fp64 reference does not) are checked
for decompression only."""
import sys

import numpy as np
import pytest
import torch

import workloads
from oracle import products

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import decode_gemv_canonical_amd as uw  # noqa: E402
from tests.parity import check_bf16, check_f32  # noqa: E402

DEV = torch.device("cuda:0")
CASES = workloads.sweep_cases()
VARIANTS = (uw.UW_VARIANT_FUSED, uw.UW_VARIANT_FUSED_MFMA, uw.UW_VARIANT_DECOMPRESS_GEMM, uw.UW_VARIANT_AUTO)


def _say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def _id(c):
    return f"{c['id']}-{c['recipe']}-{c['rows']}x{c['cols']}-K{c['K']}L{c['L']}G{c['G']}-b{c['batch']}"


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_sweep(case):
    w = workloads.sweep_weights(case)
    wb = w.numpy().view(np.uint16)
    rows, cols, batch = case["rows"], case["cols"], case["batch"]
    _say(f"sweep {_id(case)}")
    m = uw.CompressedMatrix.from_weights(w, device="cuda:0", K=case["K"], L=case["L"], G=case["G"])
    out = m.decompress()
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out), wb), "decompress differs"
    finite = case["recipe"] in ("gauss", "outliers", "finite")
    if finite:
        x = workloads.activations(cols, 1, seed=case["seed"] + 100, dtype=torch.bfloat16)[0]
        xf = workloads.activations(cols, 1, seed=case["seed"] + 101, dtype=torch.float32)[0]
        y = m.gemv(x.to(DEV))
        yb = m.gemv(xf.to(DEV), out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        check_f32(y, products.gemm_f64(wb, x.float().numpy()), "gemv")
        check_bf16(yb, products.gemm_f64(wb, xf.numpy()), "gemv bf16 out, fp32 x", cols)
        X = workloads.activations(cols, batch, seed=case["seed"] + 200, dtype=torch.bfloat16)
        ref = products.gemm_f64(wb, X.float().numpy())
        ran = []
        for v in VARIANTS:
            for ws in ((m.workspace(batch, v), None) if v == uw.UW_VARIANT_AUTO else (m.workspace(batch, v),)):
                try:
                    Y = m.gemm(X.to(DEV), variant=v, ws=ws)
                except uw.UwError as e:
                    assert e.status == uw.UW_ERR_UNSUPPORTED, str(e)
                    continue
                torch.cuda.synchronize()
                check_f32(Y, ref, f"gemm variant {v} ws={ws is not None}")
                ran.append(v)
        assert uw.UW_VARIANT_AUTO in ran and len(ran) >= 2, ran
    if m.info["plain"] or cols % 1024 or uw.uw_palette_transcode_size(m.handle) == 0:
        m.close()
        return
    p = m.transcode_palette()
    if case["K"] in (0, 16):
        got = p.d_blob.cpu().numpy().tobytes()
        assert got == uw.uw_palette_encode(w), "transcoded bytes differ from the host encoder's"
    pout = p.decompress()
    torch.cuda.synchronize()
    assert np.array_equal(_bits(pout), wb), "palette decompress differs"
    if finite:
        Y = m.gemm(X.to(DEV), variant=uw.UW_VARIANT_PALETTE)
        yp = p.gemv(x.to(DEV))
        torch.cuda.synchronize()
        check_f32(Y, ref, "palette variant")
        check_f32(yp, products.gemm_f64(wb, x.float().numpy()), "palette gemv")
    m.attach_palette(None)
    p.close()
    m.close()
