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
choice.  install_choice stores the choice on each projection's handle
(uw_set_plan); the plan file is JSON {"format": "uw-model-plan-1", "model":
name, "projections": {projection: <that handle's uw_plan_save document>}},
and load_plan_file hands each document back to uw_plan_load, which checks
that it belongs to the same matrix, so that UW_VARIANT_AUTO follows it.
"""
from __future__ import annotations

import json

from . import uw

CANDIDATES = (uw.UW_VARIANT_FUSED, uw.UW_VARIANT_FUSED_MFMA, uw.UW_VARIANT_DECOMPRESS_GEMM, uw.UW_VARIANT_PALETTE)


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


def install_choice(handles: dict, batch: int, choice: dict, layer_us: float) -> None:
    """Store the chosen variant of every projection for this batch on its
    handle (handles: {projection: uw_matrix handle})."""
    for p, v in choice.items():
        uw.uw_set_plan(handles[p], batch, v, layer_us)


def save_plan_file(path: str, model: str, handles: dict) -> dict:
    """Write the plans stored on every projection's handle (uw_plan_save) as
    one per-model file; returns the document written."""
    doc = {"format": "uw-model-plan-1", "model": model,
           "projections": {p: json.loads(uw.uw_plan_save(h)) for p, h in sorted(handles.items())}}
    with open(path, "w") as f:
        json.dump(doc, f, indent=1, sort_keys=True)
    return doc


def read_plan_file(path: str) -> dict:
    """The per-model document, with its structure checked (each projection's
    entries are checked again by uw_plan_load)."""
    with open(path) as f:
        doc = json.load(f)
    if doc.get("format") != "uw-model-plan-1" or not isinstance(doc.get("projections"), dict):
        raise ValueError(f"plan file {path}: not a uw-model-plan-1 document")
    for p, entry in doc["projections"].items():
        if not isinstance(entry, dict) or entry.get("format") != "uw-plan-1":
            raise ValueError(f"plan file {path}: projection {p} is not a uw-plan-1 document")
    return doc


def load_plan_file(path: str, handles: dict) -> dict:
    """Install every projection's plans on its handle (handles: {projection:
    uw_matrix handle}) with uw_plan_load; returns the document read."""
    doc = read_plan_file(path)
    missing = set(doc["projections"]) - set(handles)
    if missing:
        raise ValueError(f"plan file {path}: no handle for {sorted(missing)}")
    for p, entry in doc["projections"].items():
        uw.uw_plan_load(handles[p], json.dumps(entry))
    return doc
