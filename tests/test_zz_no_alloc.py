"""uw_gemm_fused_static, the entry point that allocates nothing, against
uw_gemm_fused with a workspace, through the C-ABI: two calls in a row, the
second on a smaller matrix and batch, each checked against the workspace
call's output (and both against the fp64 oracle) to the fp32 tolerance."""
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
from tests.parity import check_f32  # noqa: E402

DEV = torch.device("cuda:0")


def _say(msg):
    print(f"[gpu-static] {msg}", flush=True)
    sys.stdout.flush()


def _one(name, rows, cols, seed, batch, variant):
    w = workloads.weights(name, rows=rows, cols=cols, seed=seed)
    wb = w.numpy().view(np.uint16)
    m = uw.CompressedMatrix.from_weights(w, device="cuda:0")
    X = workloads.activations(cols, batch, seed=seed + 7, dtype=torch.bfloat16)
    ref = products.gemm_f64(wb, X.float().numpy())
    Xd = X.to(DEV)
    Yw = torch.full((batch, rows), float("nan"), device=DEV)
    uw.uw_gemm_fused(m.handle, Xd, Yw, uw.UW_VARIANT_DECOMPRESS_GEMM, m.workspace(batch))
    Ys = torch.full((batch, rows), float("nan"), device=DEV)
    _say(f"static {name} {rows}x{cols} batch={batch} variant={variant}")
    uw.uw_gemm_fused_static(m.handle, Xd, Ys, variant)
    torch.cuda.synchronize()
    check_f32(Yw, ref, f"workspace {name} b={batch}")
    check_f32(Ys, ref, f"static {name} b={batch}")
    check_f32(Ys, Yw.double().cpu().numpy(), f"static vs workspace {name} b={batch}")
    m.close()


def test_static_scratch_two_calls_second_smaller():
    # gate at batch 32: two bands of rows through the 64 MiB scratch; then a
    # smaller matrix and batch in one band, which reuses the same scratch
    _one("gate", 14336, 4096, 2, 32, uw.UW_VARIANT_DECOMPRESS_GEMM)
    _one("gate", 1000, 4096, 9, 4, uw.UW_VARIANT_DECOMPRESS_GEMM)


def test_static_auto_and_fused_variants():
    # AUTO at batch 64 takes decompress + GEMM (the scratch stands for the
    # workspace); the fused variants need no scratch and give the same bits
    w = workloads.weights("down", rows=512, cols=14336, seed=4)
    m = uw.CompressedMatrix.from_weights(w, device="cuda:0")
    X = workloads.activations(14336, 64, seed=11, dtype=torch.bfloat16).to(DEV)
    Ya = torch.empty(64, 512, device=DEV)
    Yw = torch.empty(64, 512, device=DEV)
    uw.uw_gemm_fused_static(m.handle, X, Ya, uw.UW_VARIANT_AUTO)
    uw.uw_gemm_fused(m.handle, X, Yw, uw.UW_VARIANT_AUTO, m.workspace(64))
    torch.cuda.synchronize()
    check_f32(Ya, Yw.double().cpu().numpy(), "static auto vs workspace auto")
    for v in (uw.UW_VARIANT_FUSED, uw.UW_VARIANT_FUSED_MFMA):
        X4 = X[:4].contiguous()
        Ys = torch.empty(4, 512, device=DEV)
        Yf = torch.empty(4, 512, device=DEV)
        uw.uw_gemm_fused_static(m.handle, X4, Ys, v)
        uw.uw_gemm_fused(m.handle, X4, Yf, v)
        torch.cuda.synchronize()
        assert torch.equal(Ys, Yf)
    m.close()
