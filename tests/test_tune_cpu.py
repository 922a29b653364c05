"""Host logic of the model-level tuner (no GPU): the coordinate-descent sweep
order and stopping rule on a known cost table, the plan file round trip and
its checks, and uw_set_plan's argument checks."""
import json

import pytest

uw = pytest.importorskip("decode_gemv_canonical_amd")
from decode_gemv_canonical_amd import tune  # noqa: E402

F, M, D = uw.UW_VARIANT_FUSED, uw.UW_VARIANT_FUSED_MFMA, uw.UW_VARIANT_DECOMPRESS_GEMM


def test_coordinate_descent_on_a_cost_table(monkeypatch):
    # separable costs plus one interaction: down=F costs 10 more unless up=F.
    # From (F, F, F) = 8 the sweep takes gate=M (6); up=D alone then costs 15
    # and down=M alone 7, so it stops at (M, F, F) = 6.  (M, D, M) also costs
    # 6, but reaching it changes two projections at once, which coordinate
    # descent never does.
    cost = {"gate": {F: 5, M: 3, D: 4}, "up": {F: 2, M: 3, D: 1}, "down": {F: 1, M: 2, D: 6}}

    def layer(choice):
        t = sum(cost[p][choice[p]] for p in choice)
        if choice["down"] == F and choice["up"] != F:
            t += 10
        if choice["down"] == D and choice["gate"] == M:
            raise uw.UwError(uw.UW_ERR_UNSUPPORTED, "layer", "not runnable")
        return t

    monkeypatch.setattr(tune, "time_layer_us", lambda run, steps=0, warmup=0: run)
    choice, best, hist = tune.coordinate_descent(("gate", "up", "down"), layer)
    assert choice == {"gate": M, "up": F, "down": F} and best == 6
    # start F,F,F = 8; gate sweep first (M then D), then up, then down
    assert hist[0] == ({"gate": F, "up": F, "down": F}, 8)
    assert [c["gate"] for c, _ in hist[1:3]] == [M, D]
    # the unrunnable choice was skipped, not recorded
    assert all(not (c["down"] == D and c["gate"] == M) for c, _ in hist)


def test_plan_file_round_trip(tmp_path):
    path = tmp_path / "plan.json"
    plans = {"gate": {4: (M, 80.5), 32: (D, 120.0)}, "down": {4: (F, 80.5)}}
    tune.save_plan_file(str(path), "mlp-test", plans)
    raw = json.loads(path.read_text())
    assert raw["model"] == "mlp-test" and raw["plans"]["gate"]["32"]["variant"] == D
    assert tune.read_plan_file(str(path)) == plans
    raw["plans"]["down"]["4"]["variant"] = uw.UW_VARIANT_AUTO
    path.write_text(json.dumps(raw))
    with pytest.raises(ValueError):
        tune.read_plan_file(str(path))


def test_set_plan_argument_checks_without_a_gpu():
    lib = uw.library()
    p = uw.uw_plan()
    p.batch, p.variant = 4, M
    assert lib.uw_set_plan(None, None) == uw.UW_ERR_INVALID
    assert lib.uw_set_plan(None, p) == uw.UW_ERR_INVALID


def test_exponent_entry_points_reject_null_without_a_gpu():
    lib = uw.library()
    assert lib.uw_exponent_ws_size(None, 4) == 0
    assert lib.uw_exponent_gemm(None, None, 1, 0, 1, None, 0, 0, None, 0, None) == uw.UW_ERR_INVALID
