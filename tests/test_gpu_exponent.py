"""GPU parity of the exponent-only pipeline (uw_exponent_gemm): the exponent
plane it decodes into the workspace is bit-exact against the exponent bytes
of the original weights in the documented tile order, and the reconstructive
matrix-core product matches the fp64 oracle (1e-3 relative, 2 bf16 ulp)."""
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


def _say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def _tile_order_exponents(wb):
    """Exponent bytes of wb [R, C] in tile order: tile T = weights 1024 T ..
    of the row-major matrix, byte q = column 64 (q % 16) + q / 16 of it."""
    e = ((wb >> 7) & 0xFF).astype(np.uint8).reshape(-1, 16, 64)  # [tile, group, lane]
    return e.transpose(0, 2, 1).reshape(-1)                       # byte 16 lane + group


CASES = [
    ("gate", None, None, None, {}, [16, 64]),          # G = 224: blocks end mid-row
    ("down", None, None, None, {}, [4, 100]),          # 8 % raw groups; 100 = two passes
    ("small", None, None, None, {}, [5]),              # G = 64
    ("gate", 37, 3072, 21, {"G": 48}, [17]),           # G = 48 with 48 groups per row: one row per block
    ("gate", 14344, 1024, 42, {}, [9, 40]),            # 4 row blocks per workgroup, the last partial
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}-{c[4]}")
def test_exponent_gemm(case):
    name, rows, cols, seed, opts, batches = case
    wb = workloads.weights(name, rows=rows, cols=cols, seed=seed).numpy().view(np.uint16)
    m = uw.CompressedMatrix.from_weights(wb, device="cuda:0", **opts)
    R, C = wb.shape
    for batch in batches:
        X = workloads.activations(C, batch, seed=500 + batch, dtype=torch.bfloat16)
        ref = products.gemm_f64(wb, X.float().numpy())
        ws = torch.empty(uw.uw_exponent_ws_size(m.handle, batch), dtype=torch.uint8, device=DEV)
        _say(f"exponent gemm {name} {wb.shape} {opts} batch={batch}")
        Y = torch.empty(batch, R, device=DEV)
        Yb = torch.empty(batch, R, dtype=torch.bfloat16, device=DEV)
        uw.uw_exponent_gemm(m.handle, X.to(DEV), Y, ws)
        torch.cuda.synchronize()
        plane = ws[:R * C].cpu().numpy()
        assert np.array_equal(plane, _tile_order_exponents(wb)), "exponent plane"
        uw.uw_exponent_gemm(m.handle, X.to(DEV), Yb, ws)
        torch.cuda.synchronize()
        check_f32(Y, ref, f"exponent gemm {name} b={batch}")
        check_bf16(Yb, ref, f"exponent gemm bf16 {name} b={batch}", wb.shape[1])
    m.close()


def test_exponent_gemm_unsupported_forms():
    X = torch.zeros(4, 1024, dtype=torch.bfloat16, device=DEV)
    Y = torch.empty(4, 8, device=DEV)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    plain = uw.CompressedMatrix.from_weights(workloads.weights("randbits", rows=8, cols=1024), device="cuda:0")
    assert plain.info["plain"]
    with pytest.raises(uw.UwError) as e:
        uw.uw_exponent_gemm(plain.handle, X, Y, ws)
    assert e.value.status == uw.UW_ERR_UNSUPPORTED
    # 13 groups per row: tiles cross rows
    Xs = torch.zeros(4, 832, dtype=torch.bfloat16, device=DEV)
    blockwalk = uw.CompressedMatrix.from_weights(workloads.weights("gate", rows=8, cols=832), device="cuda:0")
    with pytest.raises(uw.UwError) as e:
        uw.uw_exponent_gemm(blockwalk.handle, Xs, Y, ws)
    assert e.value.status == uw.UW_ERR_UNSUPPORTED
