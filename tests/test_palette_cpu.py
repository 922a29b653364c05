"""Host-side checks of the direct-palette form in libuw.so (no GPU): the
encoder writes the oracle's bytes, the validator accepts them and rejects
corruption, and the entry points refuse bad arguments before touching a
device."""
import numpy as np
import pytest

import workloads
from oracle import palette as opal

uw = pytest.importorskip("decode_gemv_canonical_amd")


@pytest.mark.parametrize("name,rows,cols", [
    ("small", 1024, 1024),
    ("gate", 40, 4096),
    ("down", 7, 14336),
    ("randbits", 5, 2048),
    ("small", 1, 1024),
])
def test_encoder_matches_oracle_bytes(name, rows, cols):
    w = workloads.weights(name, rows=rows, cols=cols).numpy().view(np.uint16)
    lib_blob = uw.uw_palette_encode(w)
    assert lib_blob == opal.encode(w)
    info = uw.uw_palette_info(lib_blob)
    assert (info["rows"], info["cols"], info["n_raw"]) == (rows, cols, opal.parse(lib_blob)["n_raw"])


def test_special_values_round_trip():
    w = workloads.weights("small", rows=4, cols=1024).numpy().view(np.uint16).copy()
    w[1, :8] = [0x7FC1, 0xFF80, 0x7F80, 0x0001, 0x8001, 0x0000, 0x8000, 0xFFFF]
    b = uw.uw_palette_encode(w)
    assert b == opal.encode(w)
    assert np.array_equal(opal.decode(b), w)


def test_validator_rejects_corruption():
    w = workloads.weights("down", rows=4, cols=2048).numpy().view(np.uint16)
    b = bytearray(uw.uw_palette_encode(w))
    p = opal.parse(bytes(b))
    assert p["n_raw"] > 0
    off = opal.layout(4, 2048, p["n_raw"])
    for mutate in (lambda x: x.__setitem__(0, ord("X")),               # magic
                   lambda x: x.__setitem__(off["prefix"] + 4, 99),      # a tile prefix
                   lambda x: x.__setitem__(off["flags"], x[off["flags"]] ^ 1),  # a raw flag
                   lambda x: x.__setitem__(48, 17)):                    # palette size
        bad = bytearray(b)
        mutate(bad)
        with pytest.raises(uw.UwError) as e:
            uw.uw_palette_info(bytes(bad))
        assert e.value.status == uw.UW_ERR_FORMAT
    with pytest.raises(uw.UwError):
        uw.uw_palette_info(bytes(b[:-256]))


def test_argument_errors_without_a_gpu():
    lib = uw.library()
    with pytest.raises(uw.UwError) as e:
        uw.uw_palette_encode(np.zeros((2, 1536), dtype=np.uint16))
    assert e.value.status == uw.UW_ERR_INVALID
    assert lib.uw_palette_gemv(None, None, 0, None, 0, None) == uw.UW_ERR_INVALID
    assert lib.uw_palette_decompress(None, None, 0, None) == uw.UW_ERR_INVALID
    assert lib.uw_palette_create(None, 0, None, None) == uw.UW_ERR_INVALID
    lib.uw_palette_destroy(None)
