"""GPU checks of the Huffman-to-palette transcode and of the palette form as
a candidate of the Huffman matrix.

uw_palette_transcode decodes the Huffman form on the device and writes the
direct-palette (UWP1) form; its bytes must equal what the host encoder
uw_palette_encode writes from the original weights (itself byte-identical to
the oracle's palette encoder, tests/test_palette_cpu.py).  Once attached,
UW_VARIANT_PALETTE runs the transcoded copy; its products are checked
against the fp64 oracle, and the autotuner and the plan file handle it like
any other variant.
"""
import json
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
    print(f"[gpu-transcode] {msg}", flush=True)
    sys.stdout.flush()


CASES = [
    ("gate", None, None, None, {}),
    ("down", None, None, None, {}),
    ("small", None, None, None, {}),
    ("small", 37, 2048, 41, {}),            # ragged: the last block is short
    ("down", 50, 3072, 42, {"G": 48}),      # blocks of 3 tiles, raw groups
    ("small", 24, 1024, 43, {"L": 8}),      # single-code tables
    ("down", 16, 2048, 44, {"G": 48}),      # blocks that end mid-row (one wave per block)
]


@pytest.mark.parametrize("name,rows,cols,seed,opts", CASES)
def test_transcode_matches_host_encoder_bytes(name, rows, cols, seed, opts):
    w = workloads.weights(name, rows=rows, cols=cols, seed=seed)
    want = uw.uw_palette_encode(w)
    m = uw.CompressedMatrix.from_weights(w, device="cuda:0", **opts)
    assert uw.uw_palette_transcode_size(m.handle) == len(want)
    _say(f"transcode {name} {tuple(w.shape)} {opts}")
    # a dirty output buffer: every byte must be written
    out = torch.full((len(want) + 256,), 0xA5, dtype=torch.uint8, device=DEV)
    uw.uw_palette_transcode(m.handle, out)
    torch.cuda.synchronize()
    got = out[: len(want)].cpu().numpy().tobytes()
    if got != want:
        a, b = np.frombuffer(got, np.uint8), np.frombuffer(want, np.uint8)
        bad = np.nonzero(a != b)[0]
        raise AssertionError(f"{len(bad)} bytes differ, first at {bad[:8]} of {len(want)}")
    assert (out[len(want):] == 0xA5).all(), "wrote past the transcoded form"
    m.close()


def test_untranscodable_matrices_are_refused():
    for cols, opts, why in ((2048, {"K": 32}, "palette of 32"), (1536, {}, "cols not a multiple of 1024")):
        w = workloads.weights("down", rows=16, cols=cols, seed=44)
        m = uw.CompressedMatrix.from_weights(w, device="cuda:0", **opts)
        assert uw.uw_palette_transcode_size(m.handle) == 0, why
        with pytest.raises(uw.UwError) as e:
            m.transcode_palette()
        assert e.value.status == uw.UW_ERR_UNSUPPORTED
        m.close()
    m = uw.CompressedMatrix.from_weights(workloads.weights("randbits", rows=64, cols=1024, seed=45), device="cuda:0")
    assert m.info["plain"] and uw.uw_palette_transcode_size(m.handle) == 0
    m.close()


def test_palette_variant_products():
    w = workloads.weights("down", rows=256, cols=4096, seed=46)
    wb = w.numpy().view(np.uint16)
    m = uw.CompressedMatrix.from_weights(w, device="cuda:0")
    with pytest.raises(uw.UwError) as e:
        m.gemm(torch.zeros(4, 4096, dtype=torch.bfloat16, device=DEV), variant=uw.UW_VARIANT_PALETTE)
    assert e.value.status == uw.UW_ERR_UNSUPPORTED  # nothing attached yet
    p = m.transcode_palette()
    for batch in (1, 4, 32, 70):
        X = workloads.activations(4096, batch, seed=470 + batch, dtype=torch.bfloat16)
        ref = products.gemm_f64(wb, X.float().numpy())
        _say(f"palette variant batch={batch}")
        Y = m.gemm(X.to(DEV), variant=uw.UW_VARIANT_PALETTE)
        torch.cuda.synchronize()
        check_f32(Y, ref, f"palette variant b={batch}")
    m.attach_palette(None)
    with pytest.raises(uw.UwError):
        m.gemm(torch.zeros(4, 4096, dtype=torch.bfloat16, device=DEV), variant=uw.UW_VARIANT_PALETTE)
    p.close()
    m.close()


def test_gate_b32_autotune_with_palette_and_plan_file(tmp_path):
    w = workloads.weights("gate")
    wb = w.numpy().view(np.uint16)
    m = uw.CompressedMatrix.from_weights(w, device="cuda:0")
    p = m.transcode_palette()
    _say("gate 14336x4096 batch 32 autotune with the palette copy attached")
    plan = m.autotune(32)
    _say(f"  plan {plan['variant_name']} knob {plan['knob']}: {plan['candidate_us']}")
    assert "palette" in plan["candidate_us"]
    assert plan["time_us"] == min(plan["candidate_us"].values())
    X = workloads.activations(4096, 32, seed=480, dtype=torch.bfloat16)
    ref = products.gemm_f64(wb, X.float().numpy())
    Y = m.gemm(X.to(DEV), variant=uw.UW_VARIANT_AUTO, ws=m.workspace(32))
    torch.cuda.synchronize()
    check_f32(Y, ref, "gate b=32 auto after autotune")
    # the plan file carries the choice to a fresh handle of the same weights
    doc = json.loads(m.save_plans())
    assert doc["plans"][0]["variant"] == plan["variant_name"]
    fresh = uw.CompressedMatrix.from_weights(w, device="cuda:0")
    fp = fresh.transcode_palette()
    fresh.load_plans(json.dumps(doc))
    got = uw.uw_get_plan(fresh.handle, 32)
    assert (got["variant"], got["knob"]) == (plan["variant"], plan["knob"])
    Y2 = fresh.gemm(X.to(DEV), variant=uw.UW_VARIANT_AUTO, ws=fresh.workspace(32))
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2)
    for h in (fp, fresh, p, m):
        h.close()


def test_auto_without_a_plan_picks_valu_only_when_one_pass_has_16_waves():
    # 4096 columns: one pass of 4 rows keeps 16 waves per CU, so AUTO runs the
    # vector-ALU product; 14336 columns: 4 rows of x leave room for few waves,
    # so AUTO runs the matrix-core product (bit-identical to the explicit variant)
    for cols, want in ((4096, uw.UW_VARIANT_FUSED), (14336, uw.UW_VARIANT_FUSED_MFMA)):
        w = workloads.weights("down", rows=64, cols=cols, seed=95)
        wb = w.numpy().view(np.uint16)
        m = uw.CompressedMatrix.from_weights(w, device="cuda:0")
        X = workloads.activations(cols, 4, seed=705, dtype=torch.bfloat16).to(DEV)
        y_want = m.gemm(X, variant=want)
        y_auto = m.gemm(X, variant=uw.UW_VARIANT_AUTO)
        torch.cuda.synchronize()
        _say(f"auto small batch cols={cols}")
        assert torch.equal(y_auto, y_want)
        check_f32(y_auto, products.gemm_f64(wb, X.float().cpu().numpy()), f"auto b=4 cols={cols}")
        m.close()


def test_auto_without_a_plan_takes_the_attached_palette_copy():
    # with no plan stored, AUTO's heuristic runs the palette product for 1..64
    # batch rows once a palette copy is attached (bit-identical to the explicit
    # variant); with none, the fused vector-ALU product up to 8 rows (at 4096
    # columns one pass takes 8 rows with 16 waves per workgroup) and the fused
    # matrix-core product above
    w = workloads.weights("gate", rows=256, cols=4096, seed=91)
    wb = w.numpy().view(np.uint16)
    m = uw.CompressedMatrix.from_weights(w, device="cuda:0")
    for batch in (1, 2, 3, 16, 64):
        X = workloads.activations(4096, batch, seed=700 + batch, dtype=torch.bfloat16).to(DEV)
        ref = products.gemm_f64(wb, X.float().cpu().numpy())
        y_mfma = m.gemm(X, variant=uw.UW_VARIANT_FUSED if batch <= 8 else uw.UW_VARIANT_FUSED_MFMA)
        y_auto0 = m.gemm(X, variant=uw.UW_VARIANT_AUTO)
        p = m.transcode_palette()
        y_pal = m.gemm(X, variant=uw.UW_VARIANT_PALETTE)
        y_auto = m.gemm(X, variant=uw.UW_VARIANT_AUTO)
        torch.cuda.synchronize()
        _say(f"auto heuristic b={batch}")
        assert torch.equal(y_auto0, y_mfma)
        assert torch.equal(y_auto, y_pal)
        check_f32(y_auto, ref, f"auto with palette b={batch}")
        m.attach_palette(None)
        p.close()
    m.close()
