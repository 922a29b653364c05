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
    choice, best, hist = tune.coordinate_descent(("gate", "up", "down"), layer, candidates=(F, M, D))
    assert choice == {"gate": M, "up": F, "down": F} and best == 6
    # start F,F,F = 8; gate sweep first (M then D), then up, then down
    assert hist[0] == ({"gate": F, "up": F, "down": F}, 8)
    assert [c["gate"] for c, _ in hist[1:3]] == [M, D]
    # the unrunnable choice was skipped, not recorded
    assert all(not (c["down"] == D and c["gate"] == M) for c, _ in hist)


def test_plan_file_round_trip(tmp_path, monkeypatch):
    # the per-matrix documents come from uw_plan_save and go back through
    # uw_plan_load (both need a device handle; stand-ins record the calls)
    docs = {1: {"format": "uw-plan-1", "rows": 8, "cols": 1024, "blob_crc32": 7,
                "plans": [{"batch": 4, "variant": "fused_mfma", "knob": 0, "time_us": 80.5}]},
            2: {"format": "uw-plan-1", "rows": 1024, "cols": 8, "blob_crc32": 9, "plans": []}}
    loaded = {}
    monkeypatch.setattr(tune.uw, "uw_plan_save", lambda h: json.dumps(docs[h]))
    monkeypatch.setattr(tune.uw, "uw_plan_load", lambda h, text: loaded.__setitem__(h, json.loads(text)))
    path = tmp_path / "plan.json"
    tune.save_plan_file(str(path), "mlp-test", {"gate": 1, "down": 2})
    raw = json.loads(path.read_text())
    assert raw["model"] == "mlp-test" and raw["projections"]["gate"]["plans"][0]["variant"] == "fused_mfma"
    tune.load_plan_file(str(path), {"gate": 11, "down": 12})
    assert loaded == {11: docs[1], 12: docs[2]}
    with pytest.raises(ValueError):
        tune.load_plan_file(str(path), {"gate": 11})  # a projection without a handle
    raw["projections"]["down"]["format"] = "something else"
    path.write_text(json.dumps(raw))
    with pytest.raises(ValueError):
        tune.read_plan_file(str(path))


def test_plan_entry_points_reject_null_without_a_gpu():
    lib = uw.library()
    import ctypes
    size = ctypes.c_size_t(0)
    assert lib.uw_plan_save(None, None, ctypes.byref(size)) == uw.UW_ERR_INVALID
    assert lib.uw_plan_load(None, b"{}") == uw.UW_ERR_INVALID
    assert lib.uw_gemm_with_plan(None, None, None, 1, 0, 1, None, 0, 0, None, 0, None) == uw.UW_ERR_INVALID
    assert lib.uw_matrix_attach_palette(None, None) == uw.UW_ERR_INVALID
    assert lib.uw_palette_transcode_size(None) == 0


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
