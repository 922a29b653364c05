"""Pins of the direct-palette oracle (oracle/palette.py) against values that
do not come from it: a hand-built matrix whose palette, nibbles, raw groups,
prefix counts and section offsets are worked out by hand; the exponent
statistics of the Huffman blob oracle (an independent implementation of the
same palette and raw-group rule); lossless round trips including NaN payloads,
infinities and subnormals; and a per-weight reader on tiny inputs.

Source: "Unweight: how we compressed an LLM 22% without sacrificing quality",
section on the four execution pipelines (direct palette: 4-bit indices built
at load time) and the paragraph on rare exponents (16-exponent palette, raw
64-weight groups).
"""
import numpy as np
import pytest

from oracle import blob, palette


def _bf16(e, sm):
    e = np.asarray(e, dtype=np.uint16)
    sm = np.asarray(sm, dtype=np.uint16)
    return ((sm & 0x80) << 8) | (e << 7) | (sm & 0x7F)


def _hand_matrix():
    """1 x 2048: exponent 127 on even columns, 126 on odd ones; columns
    192..247 (group 3) carry exponents 101..114, four consecutive columns
    each; column 131 (group 2, tile 0) has exponent 201 and column 1291
    (group 20, tile 1) exponent 200, each used once.  Counts: 127 -> 996,
    126 -> 994, 101..114 -> 4 each, 200 and 201 -> 1, so the palette is
    127, 126, 101..114 and groups 2 and 20 are raw."""
    n = 2048
    e = np.where(np.arange(n) % 2 == 0, 127, 126)
    for k, x in enumerate(range(101, 115)):
        for j in range(4):
            e[192 + 4 * k + j] = x
    e[131] = 201
    e[1291] = 200
    sm = (np.arange(n) * 37 + 11) % 256
    return e, sm, _bf16(e, sm).reshape(1, n)


def test_hand_layout():
    e, sm, w = _hand_matrix()
    b = palette.encode(w)
    # sections: header 64 -> 256; sm 2048 bytes; idx 1024; flags 32 groups = 1 word;
    # prefix 2 tiles = 8 bytes; raw 2 groups = 128 bytes
    assert palette.layout(1, 2048, 2) == {"sm": 256, "idx": 2304, "flags": 3328, "prefix": 3584, "raw": 3840,
                                          "total": 4096}
    assert len(b) == 4096 and b[0:4] == b"UWP1"
    p = palette.parse(b)
    assert p["palette"] == [127, 126] + list(range(101, 115))
    assert p["n_raw"] == 2
    assert int(p["flags"][0]) == (1 << 2) | (1 << 20)
    assert list(p["prefix"]) == [0, 1]
    # raw slot 0 is group 2, slot 1 is group 20, exponents verbatim
    assert list(p["raw"][:64]) == list(e[128:192])
    assert list(p["raw"][64:]) == list(e[1280:1344])
    # sm bytes verbatim
    assert list(p["sm"]) == list(sm)
    # columns 0, 1: indices 0 (127) and 1 (126) -> low nibble 0, high nibble 1
    assert p["idx"][0] == 0x10
    # columns 192, 193 hold 101 (index 2); columns 196, 197 hold 102 (index 3)
    assert p["idx"][96] == 0x22 and p["idx"][98] == 0x33
    # column 248 is back to 127 (index 0), column 249 to 126 (index 1)
    assert p["idx"][124] == 0x10
    # raw groups carry index 0 everywhere
    assert not p["idx"][64:96].any() and not p["idx"][640:672].any()


def test_hand_layout_decodes():
    _, _, w = _hand_matrix()
    b = palette.encode(w)
    assert np.array_equal(palette.decode(b), w)
    for c in (0, 1, 130, 131, 192, 193, 1291, 1343, 2047):
        assert palette.decode_one(b, 0, c) == int(w[0, c])


def _outliers(rows, cols, seed, frac=0.005):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((rows, cols)).astype(np.float32) * 0.02
    m = rng.random((rows, cols)) < frac
    v[m] = rng.standard_normal(int(m.sum())).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def test_palette_and_raw_groups_match_huffman_blob():
    w = _outliers(24, 2048, seed=5)
    hb = blob.parse_header(blob.encode(w))
    p = palette.parse(palette.encode(w))
    assert p["palette"] == list(hb.palette[:len(p["palette"])])
    assert p["n_raw"] == hb.n_raw_groups


@pytest.mark.parametrize("kind", ["normal", "outliers", "random_bits", "specials"])
def test_round_trip(kind):
    rng = np.random.default_rng(11)
    if kind == "normal":
        w = _outliers(7, 3072, seed=3, frac=0.0)
    elif kind == "outliers":
        w = _outliers(9, 1024, seed=4, frac=0.02)
    elif kind == "random_bits":
        w = rng.integers(0, 1 << 16, size=(3, 2048), dtype=np.uint16)
    else:
        w = _outliers(4, 1024, seed=6, frac=0.0)
        w[0, :8] = [0x7FC1, 0xFF80, 0x7F80, 0x0001, 0x8001, 0x0000, 0x8000, 0xFFFF]
    b = palette.encode(w)
    assert np.array_equal(palette.decode(b), w)
    assert len(b) == palette.layout(*w.shape, palette.parse(b)["n_raw"])["total"]


def test_random_bits_are_almost_all_raw():
    # 256 equally likely exponents: a 64-weight group avoids the 240 unlisted
    # ones with probability (16/256)^64, so every group is raw
    w = np.random.default_rng(2).integers(0, 1 << 16, size=(2, 1024), dtype=np.uint16)
    assert palette.parse(palette.encode(w))["n_raw"] == 32


def test_bytes_per_weight_closed_form():
    # 8 distinct exponents, so no raw groups: 1 + 1/2 bytes per weight plus
    # the flag and prefix words
    rng = np.random.default_rng(9)
    w = _bf16(rng.integers(120, 128, size=(16, 4096)), rng.integers(0, 256, size=(16, 4096)))
    p = palette.parse(palette.encode(w))
    assert p["n_raw"] == 0
    n = 16 * 4096
    # header 256, sm n, idx n/2, flags 32 words (128 bytes, padded to 256),
    # prefix 64 words (256 bytes)
    assert palette.layout(16, 4096, 0)["total"] == 256 + n + n // 2 + 256 + 256 == 99072


def test_rejects_unsupported_shapes():
    with pytest.raises(ValueError):
        palette.encode(np.zeros((2, 1536), dtype=np.uint16))
