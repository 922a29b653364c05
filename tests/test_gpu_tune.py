"""GPU check of the model-level tuner: coordinate descent over an MLP layer
picks runnable variants, the plan file written from it installs the same
choices on fresh handles, and AUTO then runs exactly the chosen kernels
(bit-identical outputs) with parity against the oracle."""
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
from decode_gemv_canonical_amd import tune  # noqa: E402

from tests.parity import check_f32  # noqa: E402

DEV = torch.device("cuda:0")


def _say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def _layer_mats():
    w = {"gate": workloads.weights("gate", rows=2048, cols=1024, seed=51),
         "up": workloads.weights("gate", rows=2048, cols=1024, seed=52),
         "down": workloads.weights("down", rows=1024, cols=2048, seed=53)}
    return w, {p: uw.CompressedMatrix.from_weights(w[p], device="cuda:0") for p in w}


def _mlp(mats, X, ws, choice):
    B = X.shape[0]
    g = torch.empty(B, 2048, device=DEV)
    u = torch.empty(B, 2048, device=DEV)
    y = torch.empty(B, 1024, device=DEV)

    def run():
        uw.uw_gemm_fused(mats["gate"].handle, X, g, choice["gate"], ws)
        uw.uw_gemm_fused(mats["up"].handle, X, u, choice["up"], ws)
        h = (torch.nn.functional.silu(g) * u).to(torch.bfloat16)
        uw.uw_gemm_fused(mats["down"].handle, h, y, choice["down"], ws)
    return run, y


@pytest.mark.parametrize("batch", [4, 32])
def test_coordinate_descent_plan_file(batch, tmp_path):
    w, mats = _layer_mats()
    X = workloads.activations(1024, batch, seed=60 + batch, dtype=torch.bfloat16).to(DEV)
    ws = torch.empty(max(m.workspace(batch).numel() for m in mats.values()), dtype=torch.uint8, device=DEV)
    _say(f"tune mlp batch={batch}")
    choice, best, hist = tune.coordinate_descent(
        ("gate", "up", "down"), lambda c: _mlp(mats, X, ws, c)[0],
        start={"gate": uw.UW_VARIANT_FUSED_MFMA, "up": uw.UW_VARIANT_FUSED_MFMA, "down": uw.UW_VARIANT_FUSED_MFMA},
        steps=50)
    assert best > 0 and len(hist) >= 7
    assert best == min(t for _, t in hist)
    path = tmp_path / "plan.json"
    tune.install_choice({p: m.handle for p, m in mats.items()}, batch, choice, best)
    tune.save_plan_file(str(path), "mlp-2048x1024", {p: m.handle for p, m in mats.items()})
    _, fresh = _layer_mats()
    tune.load_plan_file(str(path), {p: m.handle for p, m in fresh.items()})
    for p, m in fresh.items():
        assert uw.uw_get_plan(m.handle, batch)["variant"] == choice[p]
    # AUTO on the fresh handles runs the chosen kernels: identical bits
    run_auto, y_auto = _mlp(fresh, X, ws, {p: uw.UW_VARIANT_AUTO for p in fresh})
    run_pick, y_pick = _mlp(fresh, X, ws, choice)
    run_auto()
    a = y_auto.clone()
    run_pick()
    torch.cuda.synchronize()
    assert torch.equal(a, y_pick)
    # and the layer's first product agrees with the oracle
    gate = torch.empty(batch, 2048, device=DEV)
    uw.uw_gemm_fused(fresh["gate"].handle, X, gate, uw.UW_VARIANT_AUTO, ws)
    torch.cuda.synchronize()
    check_f32(gate, products.gemm_f64(w["gate"].numpy().view(np.uint16), X.float().cpu().numpy()), "tuned gate")
