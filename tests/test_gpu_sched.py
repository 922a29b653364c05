"""GPU checks of decode-ahead scheduling (uw_sched_*): a small two-layer MLP
whose down projections are decompressed on the side stream while the gate
and up products run on the caller's stream, every down product against the
fp64 oracle; the same token captured in a HIP graph and replayed several
times, with eager work in between, each replay bit-identical to the eager
token; a side stream limited to part of the compute units; and the error
paths (no free slot, an empty slot)."""
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
H, F = 1024, 2048


def _say(msg):
    print(f"[gpu-sched] {msg}", flush=True)
    sys.stdout.flush()


def _layers(n=2):
    out = []
    for li in range(n):
        w = {"gate": workloads.weights("gate", rows=F, cols=H, seed=70 + 3 * li),
             "up": workloads.weights("gate", rows=F, cols=H, seed=71 + 3 * li),
             "down": workloads.weights("down", rows=H, cols=F, seed=72 + 3 * li)}
        out.append((w, {k: uw.CompressedMatrix.from_weights(v, device="cuda:0") for k, v in w.items()}))
    return out


def _token(layers, sched, x0, B):
    """One token: per layer prefetch(down), gate, up, h, down from the slot."""
    xs, hs, ds = [x0], [], []
    for _, m in layers:
        slot = sched.prefetch(m["down"])
        g = torch.empty(B, F, device=DEV)
        u = torch.empty(B, F, device=DEV)
        uw.uw_gemm_fused(m["gate"].handle, xs[-1], g, uw.UW_VARIANT_AUTO)
        uw.uw_gemm_fused(m["up"].handle, xs[-1], u, uw.UW_VARIANT_AUTO)
        h = (torch.nn.functional.silu(g) * u).to(torch.bfloat16)
        d = torch.empty(B, H, device=DEV)
        sched.gemm(slot, m["down"], h, d)
        hs.append(h)
        ds.append(d)
        xs.append((d * torch.rsqrt(d.pow(2).mean(dim=1, keepdim=True) + 1e-6)).to(torch.bfloat16))
    return xs, hs, ds


@pytest.mark.parametrize("B,decode_cus", [(1, 0), (16, 0), (16, 64)])
def test_decode_ahead_mlp_matches_the_oracle(B, decode_cus):
    layers = _layers()
    sched = uw.DecodeAhead(slot_bytes=H * F * 2, n_slots=2, decode_cus=decode_cus)
    assert sched.decode_cus == decode_cus
    x0 = workloads.activations(H, B, seed=90 + B, dtype=torch.bfloat16).to(DEV)
    _say(f"decode-ahead token B={B} decode_cus={decode_cus}")
    xs, hs, ds = _token(layers, sched, x0, B)
    torch.cuda.synchronize()
    for li, (w, _) in enumerate(layers):
        ref = products.gemm_f64(w["down"].numpy().view(np.uint16), hs[li].float().cpu().numpy())
        check_f32(ds[li], ref, f"down layer {li} from the slot B={B}")
    sched.close()


def test_decode_ahead_in_a_graph_replays_identically():
    layers = _layers()
    B = 8
    sched = uw.DecodeAhead(slot_bytes=H * F * 2, n_slots=2)
    x0 = workloads.activations(H, B, seed=95, dtype=torch.bfloat16).to(DEV)
    eager = [t.clone() for t in _token(layers, sched, x0, B)[2]]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        _token(layers, sched, x0, B)  # warm the capture stream
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        outs = _token(layers, sched, x0, B)[2]
    for r in range(3):
        _say(f"graph replay {r}")
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert torch.equal(a, b), f"replay {r} differs from the eager token"
        # eager work on the same matrices between replays
        _token(layers, sched, x0, B)
        torch.cuda.synchronize()
    sched.close()


def test_masked_scheduler_refuses_graph_capture():
    layers = _layers(1)
    _, m = layers[0]
    sched = uw.DecodeAhead(slot_bytes=H * F * 2, n_slots=1, decode_cus=64)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    refused = []
    with torch.cuda.graph(g, stream=s):
        try:
            sched.prefetch(m["down"])
        except uw.UwError as e:
            refused.append(e.status)
    assert refused == [uw.UW_ERR_UNSUPPORTED]
    sched.close()


def test_scheduler_errors():
    layers = _layers(1)
    _, m = layers[0]
    sched = uw.DecodeAhead(slot_bytes=H * F * 2, n_slots=1)
    sched.prefetch(m["down"])
    with pytest.raises(uw.UwError) as e:
        sched.prefetch(m["down"])  # the only slot is still held
    assert e.value.status == uw.UW_ERR_NOSPACE
    small = uw.DecodeAhead(slot_bytes=1024, n_slots=1)
    with pytest.raises(uw.UwError) as e:
        small.prefetch(m["down"])
    assert e.value.status == uw.UW_ERR_NOSPACE
    lib = uw.library()
    assert lib.uw_sched_gemm(small.handle, 0, None, 1, H, uw.UW_BF16, None, 1, uw.UW_F32, None) == uw.UW_ERR_INVALID
    torch.cuda.synchronize()
    sched.close()
    small.close()
