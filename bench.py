"""Benchmark: fused exponent-Huffman decode + batch-1 GEMV on MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gate]

One step = one fused decode+GEMV call (uw_gemv_fused) over a whole
compressed matrix with a fresh bf16 activation vector: the on-chip decode
front end, Huffman decode, bf16 reassembly and the fp32-accumulated
product all run in that one kernel.  The weights are synthetic
(workloads.py), shaped like Llama-3.1-8B MLP projections; the default
workload is gate_proj 14336x4096 at batch 1.

Timing: at least W untimed steps and at least 0.5 s of them (the clocks
settle at the level a continuous decode loop runs at only after ~10 ms of
back-to-back launches, whatever W the caller asks for), then exactly K timed
steps, all replayed from captured HIP graphs (launch overhead out of the
way); the timed steps are bracketed by synchronisation and by HIP events
recorded on the stream the kernels run on.  The steps rotate over 8 device
copies of the compressed matrix so the working set (8 x 80 MB) exceeds the
256 MB Infinity Cache and every step reads HBM.

The JSON line carries the metric (effective uncompressed-weight GB/s), the
roofline of the fused kernel (algorithmic bytes = every byte of the blob +
x + y, per launch, over the average launch time, against the 8 TB/s HBM
peak), the compression figures, the uncompressed comparators (our bf16 GEMV
and torch.matmul on the same rotation), a streaming-read probe and the CPU
oracle timed on a bounded sample on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
ROTATE = 8
WARMUP_FLOOR_S = 0.5
PARITY_TOL = 1e-3  # max |y - y64| / max(|y64|, rms(y64)) for fp32 outputs


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=2000)
    p.add_argument("--workload", default="gate", choices=["gate", "down", "big", "small"])
    p.add_argument("--no-extras", action="store_true", help="skip comparators, GEMM sweep and CPU baseline")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip the oracle timing (profiler passes: its worker processes would each load the profiler)")
    p.add_argument("--skip-gemm", action="store_true", help="skip the batched-product sweep")
    p.add_argument("--gemm-only", action="store_true", help="run only the batched-product sweep (prints its JSON)")
    p.add_argument("--stack", action="store_true",
                   help="run only the 32-layer MLP stack at batch 1 and 32 (prints its JSON; ~2 min of encoding)")
    p.add_argument("--stack-layers", type=int, default=None,
                   help="layers of the stack to run (default all 32; fewer for a profiled run)")
    p.add_argument("--stack-reps", type=int, default=10, help="timed tokens per stack schedule")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# The sources the fused GEMV is built from: a recorded traffic figure is
# valid only while these are unchanged.
TRAFFIC_SOURCES = ("uw_kernels.hip", "uw_device.h", "uw_internal.h", "uw_api.cpp")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "decode_gemv_canonical_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str):
    """HBM bytes per launch measured with rocprofv3 counters for this exact
    kernel source (profiles/traffic.json), or None when the kernels changed."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    entry = rec.get(workload)
    if not entry or entry.get("source_hash") != kernel_source_hash():
        return None
    return entry.get("bytes_per_launch")


def time_graph(fn_list, steps, warmup, torch, floor_s=WARMUP_FLOOR_S):
    """Time exactly `steps` launches of the rotation fn_list (launch i runs
    fn_list[i % n]).  One eager pass loads the kernels; a graph of the n
    launches and one of the steps % n remaining are captured; the rotation
    graph is replayed untimed for at least `warmup` launches and `floor_s`
    seconds, then the timed launches run between two events on the capture
    stream.  Returns (avg launch us from the events, wall seconds of the timed
    launches, launches timed, warm-up launches, warm-up seconds)."""
    stream = torch.cuda.Stream()
    n = len(fn_list)
    with torch.cuda.stream(stream):
        for fn in fn_list:
            fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for fn in fn_list:
            fn()
    rem = steps % n
    g_rem = None
    if rem:
        g_rem = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_rem, stream=stream):
            for fn in fn_list[:rem]:
                fn()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    warm = 0
    with torch.cuda.stream(stream):
        while warm < warmup or time.perf_counter() - w0 < floor_s:
            for _ in range(16):
                g.replay()
            warm += 16 * n
            torch.cuda.synchronize()
    warm_s = time.perf_counter() - w0
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps // n):
            g.replay()
        if g_rem is not None:
            g_rem.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    return e0.elapsed_time(e1) * 1000.0 / steps, (t1 - t0), steps, warm, warm_s


def _oracle_chunk(args):
    """One worker of the all-core baseline: the oracle's decode of one row
    chunk's blob and its fp32 matvec, `reps` times (single-threaded BLAS)."""
    blob_bytes, x, reps = args
    from threadpoolctl import threadpool_limits

    from oracle import blob as oblob
    from oracle import products
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for _ in range(reps):
            dec = oblob.decode(blob_bytes)
            y = products.gemm_f32(dec, x)
        return time.perf_counter() - t0, int(y.shape[0])


def cpu_baseline(workload: str, target_s: float):
    """The oracle (numpy decode of the same blob format + fp32 matvec) on this
    host, on a sample of rows of the same workload: on one thread, and on every
    core of the process's affinity mask (the rows split into one chunk per
    core, each chunk's blob decoded by its own process, BLAS on one thread per
    process)."""
    import multiprocessing as mp

    import workloads
    from oracle import blob as oblob
    from oracle import products
    from threadpoolctl import threadpool_info, threadpool_limits

    import decode_gemv_canonical_amd as uw
    r_full, c = workloads.SHAPES[workload]
    x = workloads.activations(c, 1, seed=workloads.SEEDS[workload] + 100).float().numpy()[0]
    affinity = len(os.sched_getaffinity(0))
    blas = [f"{i.get('internal_api')}:{i.get('num_threads')}" for i in threadpool_info()]

    def run(rows, reps=1):
        w = workloads.weights(workload, rows=rows).numpy().view(np.uint16)
        b = uw.uw_encode(w)  # byte-identical to the oracle's encoder (CPU tests); only the decode is timed
        t0 = time.perf_counter()
        for _ in range(reps):
            dec = oblob.decode(b)
            y = products.gemm_f32(dec, x)
        dt = time.perf_counter() - t0
        assert np.array_equal(dec, w) and y.shape == (rows,)
        return dt / reps, dt

    rows = 64
    with threadpool_limits(limits=1):
        dt, total = run(rows)
        while dt < target_s / 4 and rows < r_full:
            rows = min(r_full, int(rows * min(8.0, max(2.0, target_s / max(dt, 1e-3)))))
            dt, total = run(rows)
        reps = 1
        if rows == r_full and dt < target_s / 2:
            reps = max(1, int(target_s / dt))  # the whole matrix is less work than the target: repeat it
            dt, total = run(rows, reps)
    one = {"value": round(2.0 * rows * c / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"{rows} of {r_full} rows of the {workload} matrix, {reps} pass(es): numpy lane-lockstep decode of "
                     f"the blob + fp32 matvec, {dt:.2f} s per pass, {total:.1f} s in all, on 1 thread",
           "seconds": round(total, 3)}
    # all cores: the whole matrix in one row chunk per core, each its own blob
    # (at most the CPU share the job is given: OMP_NUM_THREADS when set)
    cores = max(1, min(affinity, int(os.environ.get("OMP_NUM_THREADS", affinity) or affinity)))
    w = workloads.weights(workload).numpy().view(np.uint16)
    bounds = np.linspace(0, r_full, cores + 1).astype(int)
    chunks = [uw.uw_encode(np.ascontiguousarray(w[a:b])) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
    per_chunk_s = dt / rows * (r_full / len(chunks))  # from the 1-thread rate
    creps = max(1, int(target_s / 2 / max(per_chunk_s, 1e-3)))
    with mp.get_context("spawn").Pool(len(chunks)) as pool:
        t0 = time.perf_counter()
        res = pool.map(_oracle_chunk, [(b, x, creps) for b in chunks])
        wall = time.perf_counter() - t0
    assert sum(r for _, r in res) == r_full
    allc = {"value": round(2.0 * r_full * c * creps / wall / 1e9, 4), "unit": "GB/s", "cores": len(chunks),
            "kind": "oracle",
            "sample": f"all {r_full} rows of the {workload} matrix in {len(chunks)} row chunks (one blob and one "
                      f"process each), {creps} pass(es), {wall:.1f} s wall",
            "seconds": round(wall, 3)}
    return {**allc, "one_thread": one, "host": {"os_cpu_count": os.cpu_count(), "affinity_cores": affinity,
                                              "blas_threads_outside_the_timing": blas,
                                              "blas_threads_timed": 1}}


def gemm_sweep(uw, workloads, torch, dev, steps):
    """Batched products on the scope's batch sizes: down_proj at 1/4/16/64,
    gate_proj at 32 and 64 (one layer of the 32-layer stack), 8192x8192 at
    256.  Every candidate variant, the palette form, plus torch.matmul on the
    uncompressed bf16 weights; every operand rotates over 8 copies (the
    compressed, palette and bf16 working sets each exceed twice the 256 MB
    Infinity Cache), so every call reads HBM."""
    cases = [("down", (1, 4, 16, 64)), ("gate", (32, 64)), ("big", (256,))]
    names = {uw.UW_VARIANT_FUSED: "fused_valu", uw.UW_VARIANT_FUSED_MFMA: "fused_mfma",
             uw.UW_VARIANT_DECOMPRESS_GEMM: "decompress_gemm"}
    out = {}
    for name, batches in cases:
        rows, cols = workloads.SHAPES[name]
        w = workloads.weights(name)
        blob = uw.uw_encode(w)
        mats = [uw.CompressedMatrix(blob, device="cuda:0") for _ in range(ROTATE)]
        pblob = uw.uw_palette_encode(w)
        pmats = [uw.PaletteMatrix(pblob, device="cuda:0") for _ in range(ROTATE)]
        Wb = [torch.from_numpy(w.numpy()).to(dev).view(torch.bfloat16) for _ in range(ROTATE)]
        for B in batches:
            X = workloads.activations(cols, B, seed=workloads.SEEDS[name] + 200 + B, dtype=torch.bfloat16).to(dev)
            Y = torch.empty(B, rows, dtype=torch.float32, device=dev)
            rec = {}
            for v, vn in names.items():
                if v == uw.UW_VARIANT_FUSED and B > 16:
                    continue  # one decode pass per 8 rows: not a candidate at this size
                ws = mats[0].workspace(B, v)
                try:
                    us = time_graph([(lambda m=m: uw.uw_gemm_fused(m.handle, X, Y, v, ws)) for m in mats],
                                    steps, steps, torch, floor_s=0.05)[0]
                except uw.UwError:
                    continue
                rec[vn + "_us"] = round(us, 2)
                del ws
            # the exponent-only pipeline: exponent bytes to HBM, then the
            # reconstructive product on the matrix cores
            wse = torch.empty(uw.uw_exponent_ws_size(mats[0].handle, B), dtype=torch.uint8, device=dev)
            us = time_graph([(lambda m=m: uw.uw_exponent_gemm(m.handle, X, Y, wse)) for m in mats], steps, steps,
                            torch, floor_s=0.05)[0]
            rec["exponent_gemm_us"] = round(us, 2)
            del wse
            # the direct-palette form on the matrix cores (larger blob, no entropy decode)
            us = time_graph([(lambda m=m: uw.uw_palette_gemm(m.handle, X, Y)) for m in pmats], steps, steps, torch,
                            floor_s=0.05)[0]
            rec["palette_mfma_us"] = round(us, 2)
            rec["palette_blob_GBs"] = round(len(pblob) / (us * 1e-6) / 1e9, 1)
            Yb = torch.empty(B, rows, dtype=torch.bfloat16, device=dev)
            us = time_graph([(lambda W=W: torch.matmul(X, W.t(), out=Yb)) for W in Wb], steps, steps, torch,
                            floor_s=0.05)[0]
            rec["torch_bf16_matmul_us"] = round(us, 2)
            # the library's own bf16 product on the uncompressed weights
            us = time_graph([(lambda W=W: uw.uw_bf16_gemm(W, X, Y)) for W in Wb], steps, steps, torch, floor_s=0.05)[0]
            rec["ours_bf16_gemm_us"] = round(us, 2)
            best = min(v for k, v in rec.items() if k.startswith(("fused", "decompress", "exponent")))
            rec["blob_GBs_best"] = round(len(blob) / (best * 1e-6) / 1e9, 1)
            out[f"{name}_{rows}x{cols}_b{B}"] = rec
            log(f"gemm {name} B={B}: {rec}")
        for m in mats + pmats:
            m.close()
        del Wb, mats, pmats
        torch.cuda.empty_cache()
    return out


def stack_run(uw, workloads, torch, dev, steps, warmup, n_layers=None):
    """The 32-layer MLP stack (Llama-3.1-8B MLP shapes, per-layer sigma): per
    token and layer h = silu(W_gate x) * (W_up x), x' = rmsnorm(W_down h), with
    no learned scale and no residual.  At batch 1 and 32 it times the 96 matrix
    calls of one token (the AUTO variant, replayed from a graph), the
    elementwise ops alone, and the same 96 products on the uncompressed bf16
    weights; every product of one token is checked on sampled rows against the
    fp64 product of the original weights.  A second layout encodes gate and up
    as one 28672x4096 matrix per layer (one launch for both, as a fused
    gate_up projection): its 64 calls per token are timed and checked the
    same way.  The decode-ahead schedule decompresses each layer's down
    projection on a side stream (all compute units, or 64 of them) while the
    previous down product and the gate and up products run, and multiplies it
    from its slot."""
    import numpy as np

    from oracle import products
    H, F = workloads.SHAPES["gate"][1], workloads.SHAPES["gate"][0]
    layers, bfw, blob_bytes, pal_bytes = [], [], 0, 0
    t0 = time.perf_counter()
    n_layers = n_layers or workloads.STACK_LAYERS
    for li in range(n_layers):
        L = workloads.stack_layer(li)
        mats = {}
        for k, v in L.items():
            b = uw.uw_encode(v)
            blob_bytes += len(b)
            mats[k] = uw.CompressedMatrix(b, device="cuda:0")
        mats["gate_up"] = uw.CompressedMatrix(uw.uw_encode(torch.cat([L["gate"], L["up"]])), device="cuda:0")
        for k, v in L.items():
            pb = uw.uw_palette_encode(v)
            pal_bytes += len(pb)
            mats["pal_" + k] = uw.PaletteMatrix(pb, device="cuda:0")
        layers.append(mats)
        bfw.append({k: v.to(dev).view(torch.bfloat16) for k, v in L.items()})
        log(f"stack layer {li} encoded and uploaded ({time.perf_counter() - t0:.0f} s)")
    out = {"layers": n_layers, "matrices": 3 * n_layers, "blob_bytes": blob_bytes,
           "palette_bytes": pal_bytes,
           "bf16_bytes": 3 * n_layers * 2 * H * F, "prep_s": round(time.perf_counter() - t0, 1)}
    rng = np.random.default_rng(7)
    for B in (1, 32):
        n = n_layers
        xs = [torch.empty(B, H, dtype=torch.bfloat16, device=dev) for _ in range(n + 1)]
        xs[0].copy_(workloads.activations(H, B, seed=workloads.STACK_LAYER_SEED0 + 100 + B, dtype=torch.bfloat16))
        g = [torch.empty(B, F, dtype=torch.float32, device=dev) for _ in range(n)]
        u = [torch.empty(B, F, dtype=torch.float32, device=dev) for _ in range(n)]
        h = [torch.empty(B, F, dtype=torch.bfloat16, device=dev) for _ in range(n)]
        d = [torch.empty(B, H, dtype=torch.float32, device=dev) for _ in range(n)]
        ws = torch.empty(max(layers[0][k].workspace(B).numel() for k in ("gate", "up", "down")), dtype=torch.uint8,
                         device=dev)

        def matrix_calls(li):
            m = layers[li]
            uw.uw_gemm_fused(m["gate"].handle, xs[li], g[li], uw.UW_VARIANT_AUTO, ws)
            uw.uw_gemm_fused(m["up"].handle, xs[li], u[li], uw.UW_VARIANT_AUTO, ws)
            uw.uw_gemm_fused(m["down"].handle, h[li], d[li], uw.UW_VARIANT_AUTO, ws)

        def elementwise(li):
            h[li].copy_(torch.nn.functional.silu(g[li]) * u[li])
            v = d[li]
            xs[li + 1].copy_(v * torch.rsqrt(v.pow(2).mean(dim=1, keepdim=True) + 1e-6))

        # one eager token fills every buffer; its products are the parity sample
        for li in range(n):
            uw.uw_gemm_fused(layers[li]["gate"].handle, xs[li], g[li], uw.UW_VARIANT_AUTO, ws)
            uw.uw_gemm_fused(layers[li]["up"].handle, xs[li], u[li], uw.UW_VARIANT_AUTO, ws)
            h[li].copy_(torch.nn.functional.silu(g[li]) * u[li])
            uw.uw_gemm_fused(layers[li]["down"].handle, h[li], d[li], uw.UW_VARIANT_AUTO, ws)
            v = d[li]
            xs[li + 1].copy_(v * torch.rsqrt(v.pow(2).mean(dim=1, keepdim=True) + 1e-6))
        torch.cuda.synchronize()
        worst = 0.0
        for li in range(n):
            for k, inp, res, r in (("gate", xs[li], g[li], F), ("up", xs[li], u[li], F), ("down", h[li], d[li], H)):
                rows = rng.choice(r, size=64, replace=False)
                wb = bfw[li][k][torch.from_numpy(rows).to(dev)].view(torch.int16).cpu().numpy().view(np.uint16)
                ref = products.gemm_f64(wb, inp.float().cpu().numpy())
                got = res[:, torch.from_numpy(rows).to(dev)].cpu().numpy().astype(np.float64)
                worst = max(worst, products.rel_error_floored(got, ref))
        reps = max(1, steps // 96)
        us_m = time_graph([lambda: [matrix_calls(li) for li in range(n)]], reps, reps, torch)[0]
        log(f"stack B={B} fused (AUTO): {us_m / 1e3:.3f} ms/token")
        us_e = time_graph([lambda: [elementwise(li) for li in range(n)]], reps, reps, torch)[0]
        gb = [torch.empty(B, F, dtype=torch.bfloat16, device=dev) for _ in range(2)]
        db = torch.empty(B, H, dtype=torch.bfloat16, device=dev)

        def bf16_calls():
            for li in range(n):
                torch.matmul(xs[li], bfw[li]["gate"].t(), out=gb[0])
                torch.matmul(xs[li], bfw[li]["up"].t(), out=gb[1])
                torch.matmul(h[li], bfw[li]["down"].t(), out=db)

        us_b = time_graph([bf16_calls], reps, reps, torch)[0]
        log(f"stack B={B} bf16 torch.matmul: {us_b / 1e3:.3f} ms/token")
        # gate and up as one matrix: 64 calls per token
        gu = [torch.empty(B, 2 * F, dtype=torch.float32, device=dev) for _ in range(n)]

        def fused_calls(li):
            uw.uw_gemm_fused(layers[li]["gate_up"].handle, xs[li], gu[li], uw.UW_VARIANT_AUTO, ws)
            uw.uw_gemm_fused(layers[li]["down"].handle, h[li], d[li], uw.UW_VARIANT_AUTO, ws)

        for li in range(n):
            fused_calls(li)
        torch.cuda.synchronize()
        worst_gu = 0.0
        for li in range(n):
            rows = rng.choice(2 * F, size=64, replace=False)
            wcat = torch.cat([bfw[li]["gate"], bfw[li]["up"]])
            wb = wcat[torch.from_numpy(rows).to(dev)].view(torch.int16).cpu().numpy().view(np.uint16)
            ref = products.gemm_f64(wb, xs[li].float().cpu().numpy())
            got = gu[li][:, torch.from_numpy(rows).to(dev)].cpu().numpy().astype(np.float64)
            worst_gu = max(worst_gu, products.rel_error_floored(got, ref))
            del wcat
        us_f = time_graph([lambda: [fused_calls(li) for li in range(n)]], reps, reps, torch)[0]
        log(f"stack B={B} gate+up as one matrix: {us_f / 1e3:.3f} ms/token")

        # the same 96 products over the direct-palette form (GEMV at batch 1,
        # matrix-core GEMM above), on the inputs of the eager token
        gp = [torch.empty(B, F, dtype=torch.float32, device=dev) for _ in range(n)]
        up_ = [torch.empty(B, F, dtype=torch.float32, device=dev) for _ in range(n)]
        dp = [torch.empty(B, H, dtype=torch.float32, device=dev) for _ in range(n)]

        def pal(m, X, Y):
            if B == 1:
                uw.uw_palette_gemv(m.handle, X[0], Y[0])
            else:
                uw.uw_palette_gemm(m.handle, X, Y)

        def palette_calls(li):
            m = layers[li]
            pal(m["pal_gate"], xs[li], gp[li])
            pal(m["pal_up"], xs[li], up_[li])
            pal(m["pal_down"], h[li], dp[li])

        for li in range(n):
            palette_calls(li)
        torch.cuda.synchronize()
        worst_p = 0.0
        for li in range(n):
            for k, inp, res, r in (("gate", xs[li], gp[li], F), ("up", xs[li], up_[li], F), ("down", h[li], dp[li], H)):
                rows = rng.choice(r, size=64, replace=False)
                wb = bfw[li][k][torch.from_numpy(rows).to(dev)].view(torch.int16).cpu().numpy().view(np.uint16)
                ref = products.gemm_f64(wb, inp.float().cpu().numpy())
                got = res[:, torch.from_numpy(rows).to(dev)].cpu().numpy().astype(np.float64)
                worst_p = max(worst_p, products.rel_error_floored(got, ref))
        us_p = time_graph([lambda: [palette_calls(li) for li in range(n)]], reps, reps, torch)[0]
        log(f"stack B={B} palette form: {us_p / 1e3:.3f} ms/token")

        # decode-ahead: down_l+1 is decompressed on the side stream while
        # down_l's product (from its slot) and gate_l+1 / up_l+1 run.  Graph
        # replay with the side stream on every compute unit; the split of the
        # compute units (side stream limited to 64 of them) is timed from eager
        # launches at batch 32, where the kernels, not the host, set the pace
        ahead = {}
        for cus in ((0, 64) if B > 1 else (0,)):
            sched = uw.DecodeAhead(slot_bytes=2 * H * F, n_slots=2, decode_cus=cus)
            do = [torch.empty(B, H, dtype=torch.float32, device=dev) for _ in range(n)]

            def ahead_calls(sched=sched, do=do):
                slot = sched.prefetch(layers[0]["down"])
                for li in range(n):
                    m = layers[li]
                    uw.uw_gemm_fused(m["gate"].handle, xs[li], g[li], uw.UW_VARIANT_AUTO, ws)
                    uw.uw_gemm_fused(m["up"].handle, xs[li], u[li], uw.UW_VARIANT_AUTO, ws)
                    nxt = sched.prefetch(layers[li + 1]["down"]) if li + 1 < n else None
                    sched.gemm(slot, m["down"], h[li], do[li])
                    slot = nxt

            ahead_calls()
            torch.cuda.synchronize()
            worst_a = 0.0
            for li in range(n):
                rows = rng.choice(H, size=64, replace=False)
                wb = bfw[li]["down"][torch.from_numpy(rows).to(dev)].view(torch.int16).cpu().numpy().view(np.uint16)
                ref = products.gemm_f64(wb, h[li].float().cpu().numpy())
                got = do[li][:, torch.from_numpy(rows).to(dev)].cpu().numpy().astype(np.float64)
                worst_a = max(worst_a, products.rel_error_floored(got, ref))
            rec = {"parity_max_rel_err_sampled_down": worst_a}
            if cus == 0:
                rec["matrix_ms_per_token"] = round(time_graph([ahead_calls], reps, reps, torch)[0] / 1e3, 4)
            if B > 1:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                for _ in range(3):
                    ahead_calls()
                torch.cuda.synchronize()
                e0.record()
                for _ in range(reps):
                    ahead_calls()
                e1.record()
                torch.cuda.synchronize()
                rec["eager_matrix_ms_per_token"] = round(e0.elapsed_time(e1) / reps, 4)
            ahead[f"decode_cus_{sched.decode_cus}"] = rec
            log(f"stack B={B} decode-ahead cus={sched.decode_cus}: {rec}")
            sched.close()
            del do
        if B > 1:
            # the fused schedule timed the same eager way, for the comparison
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            for _ in range(3):
                [matrix_calls(li) for li in range(n)]
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                [matrix_calls(li) for li in range(n)]
            e1.record()
            torch.cuda.synchronize()
            ahead["fused_eager_matrix_ms_per_token"] = round(e0.elapsed_time(e1) / reps, 4)
            log(f"stack B={B} fused eager: {ahead['fused_eager_matrix_ms_per_token']} ms/token")
        out[f"b{B}"] = {"matrix_ms_per_token": round(us_m / 1e3, 4), "elementwise_ms_per_token": round(us_e / 1e3, 4),
                        "gate_up_fused_matrix_ms_per_token": round(us_f / 1e3, 4),
                        "gate_up_fused_parity_max_rel_err_sampled": worst_gu,
                        "palette_matrix_ms_per_token": round(us_p / 1e3, 4),
                        "palette_parity_max_rel_err_sampled": worst_p,
                        "decode_ahead": ahead,
                        "bf16_matmul_ms_per_token": round(us_b / 1e3, 4),
                        "speedup_vs_bf16": round(us_b / us_m, 4),
                        "effective_weight_GBs": round(out["bf16_bytes"] / (us_m * 1e-6) / 1e9, 1),
                        "compressed_GBs": round(blob_bytes / (us_m * 1e-6) / 1e9, 1),
                        "parity_max_rel_err_sampled": worst, "parity_ok": worst <= PARITY_TOL}
        log(f"stack B={B}: {out[f'b{B}']}")
        del xs, g, u, h, d, ws, gb, db, gu, gp, up_, dp
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1 "
                                   "(the multi-GPU sharding is a design note only)"}))
        sys.exit(2)
    import torch

    import decode_gemv_canonical_amd as uw
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.gemm_only:
        print(json.dumps({"gemm": gemm_sweep(uw, workloads, torch, dev, 48)}), flush=True)
        return
    if args.stack:
        print(json.dumps({"stack": stack_run(uw, workloads, torch, dev, 96 * args.stack_reps, 96 * args.stack_reps,
                                             args.stack_layers)}), flush=True)
        return
    name = args.workload
    rows, cols = workloads.SHAPES[name]
    log(f"encoding {name} {rows}x{cols}")
    w = workloads.weights(name)
    t0 = time.perf_counter()
    blob = uw.uw_encode(w)
    t_encode = time.perf_counter() - t0
    info = uw.uw_blob_info(blob)
    mats = [uw.CompressedMatrix(blob, device="cuda:0") for _ in range(ROTATE)]
    xdt = torch.float32 if name == "small" else torch.bfloat16
    x = workloads.activations(cols, 1, seed=workloads.SEEDS[name] + 100, dtype=xdt)[0].to(dev)
    y = torch.empty(rows, dtype=torch.float32, device=dev)
    weights = rows * cols

    # the timed step
    fns = [(lambda m=m: uw.uw_gemv_fused(m.handle, x, y)) for m in mats]
    log(f"timing fused decode+GEMV: {args.steps} steps after {args.warmup} warm-up")
    us, wall, done, warm_done, warm_s = time_graph(fns, args.steps, args.warmup, torch)
    algo_bytes = info["total_bytes"] + cols * x.element_size() + rows * 4
    achieved = algo_bytes / (us * 1e-6) / 1e9
    value = 2.0 * weights * done / wall / 1e9

    # parity spot check of the timed configuration (every output, fp64 oracle)
    from oracle import products
    ref = products.gemm_f64(w.numpy().view(np.uint16), x.float().cpu().numpy())
    err = products.rel_error_floored(y.cpu().numpy(), ref)

    traffic = recorded_traffic(name)
    out = {
        "metric": "fused decode+GEMV effective weight GB/s & % HBM peak; compression ratio",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": done,
        "warmup": args.warmup,
        "warmup_done": {"launches": warm_done, "seconds": round(warm_s, 3), "floor_s": WARMUP_FLOOR_S},
        "ms_per_step": round(wall * 1000.0 / done, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{name}_proj {rows}x{cols} bf16 N(0,0.02), fused decode+GEMV, batch 1",
                   "batch": 1, "rows": rows, "cols": cols, "rotation_copies": ROTATE},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "kernel_us": round(us, 3),
        "effective_weight_GBs_kernel": round(2.0 * weights / (us * 1e-6) / 1e9, 1),
        "compression": {"ratio": round(info["ratio"], 5), "saved": round(1 - info["ratio"], 5),
                        "bits_per_weight": round(info["bits_per_weight"], 4),
                        "raw_group_frac": round(info["n_raw_groups"] / (weights // 64), 6),
                        "blob_bytes": info["total_bytes"], "bf16_bytes": 2 * weights,
                        "K": info["K"], "L": info["L"], "G": info["G"], "encode_s": round(t_encode, 3)},
        "parity": {"max_rel_err_vs_fp64": err, "tolerance": PARITY_TOL, "ok": bool(err <= PARITY_TOL)},
    }

    if not args.no_extras:
        extras = {}
        # uncompressed comparators on the same rotation
        Wb = [torch.from_numpy(w.numpy()).to(dev).view(torch.bfloat16) for _ in range(ROTATE)]
        yb = torch.empty(rows, dtype=torch.float32, device=dev)
        xr = x.reshape(1, cols)
        yr = yb.reshape(1, rows)
        log("timing uncompressed bf16 GEMV (ours)")
        us_b = time_graph([(lambda W=W: uw.uw_bf16_gemm(W, xr, yr)) for W in Wb], args.steps, args.warmup, torch)[0]
        ybf = torch.empty(rows, dtype=torch.bfloat16, device=dev)
        log("timing torch.matmul (hipBLASLt) comparator")
        us_t = time_graph([(lambda W=W: torch.mv(W, x if x.dtype == torch.bfloat16 else x.bfloat16(), out=ybf))
                           for W in Wb], args.steps, args.warmup, torch)[0]
        best_bf16 = min(us_b, us_t)
        extras["uncompressed"] = {
            "ours_bf16_gemv_us": round(us_b, 3), "torch_mv_us": round(us_t, 3),
            "ours_bf16_GBs": round(2.0 * weights / (us_b * 1e-6) / 1e9, 1),
            "torch_mv_GBs": round(2.0 * weights / (us_t * 1e-6) / 1e9, 1),
            "fused_speedup_vs_best_bf16": round(best_bf16 / us, 4),
        }
        del Wb
        torch.cuda.empty_cache()
        # code-length limit: L = 6 decodes two codes per lookup (4096-entry
        # pair table); L = 8 and 12 decode one code per lookup (2^L entries)
        ablation = {}
        for L in (8, 12):
            bl = uw.uw_encode(w, L=L)
            ml = [uw.CompressedMatrix(bl, device="cuda:0") for _ in range(ROTATE)]
            us_l = time_graph([(lambda m=m: uw.uw_gemv_fused(m.handle, x, y)) for m in ml], args.steps,
                              args.warmup, torch)[0]
            ablation[f"L{L}"] = {"us": round(us_l, 3), "bits_per_weight": round(uw.uw_blob_info(bl)["bits_per_weight"], 4)}
            for m in ml:
                m.close()
        ablation["L6"] = {"us": round(us, 3), "bits_per_weight": round(info["bits_per_weight"], 4)}
        extras["lut_ablation"] = ablation
        log(f"L ablation: {ablation}")
        # streaming-read probe over 1 GiB
        log("read probe")
        buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        sink = torch.empty(uw.uw_read_probe_sink_size(), dtype=torch.uint8, device=dev)
        us_p = time_graph([lambda: uw.uw_read_probe(buf, sink)], 20, 3, torch, floor_s=0.05)[0]
        probe = buf.numel() / (us_p * 1e-6) / 1e9
        extras["read_probe_GBs"] = round(probe, 1)
        extras["fused_frac_of_read_probe"] = round(achieved / probe, 4)
        del buf
        # the same probe at the blob's size, on rotated copies and timed like
        # the fused step: the streaming ceiling for a read of this length
        nbytes = (info["total_bytes"] + 255) // 256 * 256
        bufs = [torch.ones(nbytes, dtype=torch.uint8, device=dev) for _ in range(ROTATE)]
        us_ps = time_graph([(lambda b=b: uw.uw_read_probe(b, sink)) for b in bufs], args.steps, args.warmup, torch)[0]
        probe_same = nbytes / (us_ps * 1e-6) / 1e9
        extras["read_probe_blob_size"] = {"bytes": nbytes, "us": round(us_ps, 3), "GBs": round(probe_same, 1),
                                          "fused_frac": round(achieved / probe_same, 4)}
        log(f"read probe at the blob size: {extras['read_probe_blob_size']}")
        del bufs
        # decompress-to-HBM alternative (reads the blob, writes bf16)
        out_w = [torch.empty(rows, cols, dtype=torch.bfloat16, device=dev) for _ in range(2)]
        log("timing decompress")
        us_d = time_graph([(lambda m=m, o=out_w[i % 2]: uw.uw_decompress(m.handle, o, cols))
                           for i, m in enumerate(mats)], 400, 400, torch, floor_s=0.05)[0]
        dbytes = info["total_bytes"] + 2 * weights
        extras["decompress"] = {"us": round(us_d, 3), "GBs_read_plus_write": round(dbytes / (us_d * 1e-6) / 1e9, 1),
                                "frac_hbm_peak": round(dbytes / (us_d * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        del out_w
        torch.cuda.empty_cache()
        # direct-palette pipeline on the same weights: 4-bit index + sm byte,
        # no entropy decode (larger blob, lighter kernel)
        log("timing direct-palette GEMV")
        pblob = uw.uw_palette_encode(w)
        pinfo = uw.uw_palette_info(pblob)
        pmats = [uw.PaletteMatrix(pblob, device="cuda:0") for _ in range(ROTATE)]
        yp = torch.empty(rows, dtype=torch.float32, device=dev)
        us_pg = time_graph([(lambda m=m: uw.uw_palette_gemv(m.handle, x, yp)) for m in pmats], args.steps,
                           args.warmup, torch)[0]
        perr = products.rel_error_floored(yp.cpu().numpy(), ref)
        pbytes = pinfo["bytes"] + cols * x.element_size() + rows * 4
        out_pw = [torch.empty(rows, cols, dtype=torch.bfloat16, device=dev) for _ in range(2)]
        us_pd = time_graph([(lambda m=m, o=out_pw[i % 2]: uw.uw_palette_decompress(m.handle, o, cols))
                            for i, m in enumerate(pmats)], 400, 400, torch, floor_s=0.05)[0]
        extras["palette_pipeline"] = {
            "ratio": round(pinfo["ratio"], 5), "blob_bytes": pinfo["bytes"],
            "raw_group_frac": round(pinfo["n_raw"] / (weights // 64), 6),
            "gemv_us": round(us_pg, 3), "gemv_GBs": round(pbytes / (us_pg * 1e-6) / 1e9, 1),
            "gemv_frac_hbm_peak": round(pbytes / (us_pg * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "effective_weight_GBs": round(2.0 * weights / (us_pg * 1e-6) / 1e9, 1),
            "vs_huffman_fused": round(us / us_pg, 4), "vs_best_bf16": round(best_bf16 / us_pg, 4),
            "max_rel_err_vs_fp64": perr, "parity_ok": bool(perr <= PARITY_TOL),
            "decompress_us": round(us_pd, 3),
            "decompress_GBs_read_plus_write": round((pinfo["bytes"] + 2 * weights) / (us_pd * 1e-6) / 1e9, 1),
        }
        log(f"palette: {extras['palette_pipeline']}")
        for m in pmats:
            m.close()
        del out_pw, pmats
        torch.cuda.empty_cache()
        # plain copy of known size (random bits store in plain mode: the
        # decompress is one read and one write of 128 MiB); its counter
        # readings calibrate FETCH_SIZE / WRITE_SIZE for the traffic figure
        log("timing plain-mode copy (counter calibration)")
        wr = workloads.weights("randbits", rows=8192, cols=8192)
        mplain = uw.CompressedMatrix(uw.uw_encode(wr), device="cuda:0")
        del wr
        assert mplain.info["plain"], "random bits are expected to take plain mode"
        out_p = torch.empty(8192, 8192, dtype=torch.bfloat16, device=dev)
        us_c = time_graph([lambda: uw.uw_decompress(mplain.handle, out_p, 8192)], 16, 4, torch, floor_s=0.05)[0]
        extras["plain_copy"] = {"bytes_each_way": 2 * 8192 * 8192, "us": round(us_c, 3),
                                "GBs_read_plus_write": round(4 * 8192 * 8192 / (us_c * 1e-6) / 1e9, 1)}
        mplain.close()
        del out_p
        torch.cuda.empty_cache()
        if not args.skip_gemm:
            log("gemm sweep")
            extras["gemm"] = gemm_sweep(uw, workloads, torch, dev, 48)
        out["extras"] = extras
        if args.no_cpu_baseline:
            out["cpu_baseline"] = None
        else:
            log("cpu baseline (oracle)")
            out["cpu_baseline"] = cpu_baseline(name, args.cpu_seconds)
    for m in mats:
        m.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
