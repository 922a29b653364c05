"""Model-level tuning by coordinate descent, and the per-model plan file.

"Unweight: how we compressed an LLM 22% without sacrificing quality",
autotuner paragraph: the configuration space (pipelines x matmul variants) is
searched by measuring real end-to-end throughput on the target hardware; the
tuner sweeps the gate projection's options with up and down fixed, then up,
then down, and repeats until nothing improves; the result is a model-specific
configuration file that tells the runtime which variant each projection uses
at each batch size.

Here a "layer" is whatever callable the caller gives: it runs one pass of the
layer with one variant per projection (for the MLP: h = silu(W_gate x) *
(W_up x), y = W_down h).  Every product inside it is a library call; this
module only times the layer (a captured HIP graph, replayed) and records the
choice.  The plan file is JSON: {"model": name, "plans": {projection:
{batch: {"variant": v, "layer_us": t}}}}; load_plan_file installs the choices
with uw_set_plan so that UW_VARIANT_AUTO follows them.
"""
from __future__ import annotations

import json

from . import uw

CANDIDATES = (uw.UW_VARIANT_FUSED, uw.UW_VARIANT_FUSED_MFMA, uw.UW_VARIANT_DECOMPRESS_GEMM)


def time_layer_us(run, steps: int = 200, warmup: int = 200) -> float:
    """Mean time of one run() in microseconds: run() is captured once in a
    HIP graph and replayed (the first eager call loads the kernels)."""
    import torch
    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        g.replay()
    end.record()
    end.synchronize()
    return start.elapsed_time(end) * 1000.0 / steps


def coordinate_descent(projections, layer, start=None, candidates=CANDIDATES, max_rounds: int = 4,
                       steps: int = 200) -> tuple[dict, float, list]:
    """Minimise the time of layer(choice) over one variant per projection.

    projections: names in sweep order (e.g. ("gate", "up", "down")).
    layer(choice) returns a callable that runs the layer once with the variant
    choice[name] for each projection; a variant a projection cannot run raises
    uw.UwError and is skipped.  start: the first choice (default: the first
    candidate everywhere).  Returns (choice, layer_us, history) where history
    lists every (choice, layer_us) measured."""
    choice = dict(start) if start else {p: candidates[0] for p in projections}
    history = []

    def measure(c):
        try:
            t = time_layer_us(layer(c), steps=steps, warmup=steps)
        except uw.UwError:
            return None
        history.append((dict(c), t))
        return t

    best = measure(choice)
    if best is None:
        raise uw.UwError(uw.UW_ERR_UNSUPPORTED, "coordinate_descent", "the starting choice does not run")
    for _ in range(max_rounds):
        improved = False
        for p in projections:
            for v in candidates:
                if v == choice[p]:
                    continue
                trial = dict(choice)
                trial[p] = v
                t = measure(trial)
                if t is not None and t < best:
                    best, choice, improved = t, trial, True
        if not improved:
            break
    return choice, best, history


def save_plan_file(path: str, model: str, plans: dict) -> None:
    """plans: {projection: {batch: (variant, layer_us)}}."""
    out = {"model": model, "plans": {p: {str(b): {"variant": int(v), "layer_us": float(t)}
                                         for b, (v, t) in sorted(by_batch.items())}
                                     for p, by_batch in plans.items()}}
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)


def read_plan_file(path: str) -> dict:
    """{projection: {batch: (variant, layer_us)}}, checked."""
    with open(path) as f:
        raw = json.load(f)
    plans = {}
    for p, by_batch in raw["plans"].items():
        plans[p] = {}
        for b, rec in by_batch.items():
            v = int(rec["variant"])
            if v not in CANDIDATES or int(b) < 1:
                raise ValueError(f"plan file {path}: bad entry {p} batch {b}")
            plans[p][int(b)] = (v, float(rec["layer_us"]))
    return plans


def load_plan_file(path: str, handles: dict) -> dict:
    """Install every plan of the file on the handle of its projection
    (handles: {projection: uw_matrix handle}); returns the plans read."""
    plans = read_plan_file(path)
    for p, by_batch in plans.items():
        for b, (v, t) in by_batch.items():
            uw.uw_set_plan(handles[p], b, v, t)
    return plans
