"""GPU parity at the benchmark configurations' full sizes, through the C-ABI.

- down_proj 4096x14336 with 0.5 % N(0,1) outliers: uw_autotune at batch 1,
  4, 16 and 64, then AUTO, every output against the fp64 oracle;
- one layer of the 32-layer MLP stack (gate, up 14336x4096, down
  4096x14336 at the layer's jittered sigma) through AUTO at batch 1 and 32,
  every output of the three products;
- 8192x8192 uniformly random bit patterns (plain mode): decompressed bit for
  bit;
- 8192x8192 N(0, 0.02) at batch 256: AUTO with a workspace (decompress +
  the matrix-core GEMM), sampled rows against the oracle.
"""
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
    print(f"[gpu-full] {msg}", flush=True)
    sys.stdout.flush()


def test_down_autotune_then_auto_full_size():
    w = workloads.weights("down")
    wb = w.numpy().view(np.uint16)
    W64 = products.bf16_to_f64(wb)
    m = uw.CompressedMatrix.from_weights(w, device="cuda:0")
    for batch in (1, 4, 16, 64):
        _say(f"down 4096x14336 autotune batch={batch}")
        plan = m.autotune(batch)
        _say(f"  plan {plan['variant_name']} knob {plan['knob']}: {plan['candidate_us']}")
        assert plan["time_us"] == min(plan["candidate_us"].values())
        X = workloads.activations(14336, batch, seed=workloads.SEEDS["down"] + 200 + batch, dtype=torch.bfloat16)
        ref = X.double().numpy() @ W64.T
        Y = m.gemm(X.to(DEV), variant=uw.UW_VARIANT_AUTO, ws=m.workspace(batch))
        torch.cuda.synchronize()
        check_f32(Y, ref, f"down auto b={batch}")
    m.close()


@pytest.mark.parametrize("batch", [1, 32])
def test_stack_layer_through_auto(batch):
    layer = workloads.stack_layer(7)
    mats = {k: uw.CompressedMatrix.from_weights(v, device="cuda:0") for k, v in layer.items()}
    W64 = {k: products.bf16_to_f64(v.numpy().view(np.uint16)) for k, v in layer.items()}
    H, F = workloads.SHAPES["gate"][1], workloads.SHAPES["gate"][0]
    x = workloads.activations(H, batch, seed=workloads.STACK_LAYER_SEED0 + 100 + batch, dtype=torch.bfloat16)
    ws = torch.empty(max(m.workspace(batch).numel() for m in mats.values()), dtype=torch.uint8, device=DEV)
    _say(f"stack layer 7 batch={batch}: gate, up")
    g = mats["gate"].gemm(x.to(DEV), variant=uw.UW_VARIANT_AUTO, ws=ws)
    u = torch.empty(batch, F, dtype=torch.bfloat16, device=DEV)
    uw.uw_gemm_fused(mats["up"].handle, x.to(DEV), u, uw.UW_VARIANT_AUTO, ws)
    torch.cuda.synchronize()
    xd = x.double().numpy()
    check_f32(g, xd @ W64["gate"].T, f"stack gate b={batch}")
    check_bf16(u, xd @ W64["up"].T, f"stack up b={batch} (bf16 out)", H)
    h = (torch.nn.functional.silu(g) * u.float()).to(torch.bfloat16)
    _say(f"stack layer 7 batch={batch}: down")
    d = mats["down"].gemm(h, variant=uw.UW_VARIANT_AUTO, ws=ws)
    torch.cuda.synchronize()
    check_f32(d, h.double().cpu().numpy() @ W64["down"].T, f"stack down b={batch}")
    for m in mats.values():
        m.close()


def test_random_bits_8192_full_size_bit_exact():
    w = workloads.weights("randbits")
    wb = w.numpy().view(np.uint16)
    m = uw.CompressedMatrix.from_weights(w, device="cuda:0")
    assert m.info["plain"] == 1
    _say("randbits 8192x8192 decompress")
    out = m.decompress()
    torch.cuda.synchronize()
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), wb)
    m.close()


def test_big_b256_auto_with_workspace_sampled_rows():
    w = workloads.weights("big")
    wb = w.numpy().view(np.uint16)
    m = uw.CompressedMatrix.from_weights(w, device="cuda:0")
    X = workloads.activations(8192, 256, seed=workloads.SEEDS["big"] + 456, dtype=torch.bfloat16)
    _say("big 8192x8192 batch 256 AUTO")
    Y = m.gemm(X.to(DEV), variant=uw.UW_VARIANT_AUTO, ws=m.workspace(256))
    Yb = m.gemm(X.to(DEV), variant=uw.UW_VARIANT_AUTO, ws=m.workspace(256), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.random.default_rng(5).choice(8192, size=64, replace=False)
    ref = products.gemm_f64(wb[rows], X.float().numpy())
    check_f32(Y[:, torch.from_numpy(rows).to(DEV)], ref, "big b=256 auto sampled rows")
    check_bf16(Yb[:, torch.from_numpy(rows).to(DEV)].contiguous(), ref, "big b=256 auto bf16 sampled rows", 8192)
    m.close()
