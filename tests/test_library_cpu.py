"""Host-side checks of libuw.so that need no GPU: it loads, exports every
entry point include/uw.h declares, and its host encoder / validator agree
with the oracle (byte-identical blobs, cross decoding, rejected corruption)."""
import ctypes

import numpy as np
import pytest

import workloads
from oracle import blob as oblob

uw = pytest.importorskip("decode_gemv_canonical_amd")


def test_exports_every_declared_symbol():
    lib = uw.library()
    syms = uw.header_symbols()
    assert len(syms) >= 15
    for s in syms:
        assert hasattr(lib, s), s
    assert uw.uw_version() == 20000
    assert uw.uw_status_string(uw.UW_ERR_FORMAT) == "invalid blob format"


@pytest.mark.parametrize("name,rows,cols,kw", [
    ("small", 1024, 1024, {}),
    ("gate", 96, 4096, {}),
    ("down", 24, 14336, {}),
    ("down", 13, 512, {"G": 48}),
    ("small", 40, 320, {"K": 7, "L": 5}),
    ("small", 40, 320, {"K": 32, "L": 8}),
    ("small", 40, 320, {"K": 16, "L": 12}),
    ("small", 3, 64, {"K": 1, "L": 1}),
    ("randbits", 32, 1024, {}),
])
def test_encoder_matches_oracle_bytes(name, rows, cols, kw):
    w = workloads.weights(name, rows=rows, cols=cols).numpy().view(np.uint16)
    lib_blob = uw.uw_encode(w, K=kw.get("K", 0), L=kw.get("L", 0), G=kw.get("G", 0))
    ora_blob = oblob.encode(w, K=kw.get("K", 16), L=kw.get("L", 6), G=kw.get("G"))
    assert lib_blob == ora_blob
    assert np.array_equal(oblob.decode(lib_blob), w)


@pytest.mark.parametrize("rows,cols", [(14336, 4096), (4096, 14336), (8192, 8192), (11008, 4096), (4096, 11008),
                                       (28672, 4096), (3000, 3072), (96, 4096), (13, 512), (1024, 1024)])
def test_default_block_size_matches_oracle(rows, cols):
    # the two encoders implement the default G separately
    b = uw.uw_encode(np.zeros((rows, cols), np.uint16), flags=uw.UW_ENC_NO_PLAIN)
    assert uw.uw_blob_info(b)["G"] == oblob.choose_groups_per_block(rows, cols)


def test_no_plain_flag_and_special_values():
    sv = np.array(workloads.special_values_bf16(), dtype=np.uint16)
    w = np.resize(sv, (4, 128))
    a = uw.uw_encode(w, flags=uw.UW_ENC_NO_PLAIN)
    b = oblob.encode(w, allow_plain=False)
    assert a == b and np.array_equal(oblob.decode(a), w)
    assert uw.uw_blob_info(a)["plain"] == 0


def test_blob_info_fields():
    w = workloads.weights("gate", rows=64).numpy().view(np.uint16)
    b = uw.uw_encode(w)
    info = uw.uw_blob_info(b)
    h = oblob.parse_header(b)
    assert (info["rows"], info["cols"], info["K"], info["L"], info["G"]) == (64, 4096, h.K, h.L, h.G)
    assert info["n_raw_groups"] == h.n_raw_groups and info["total_bytes"] == len(b)
    assert abs(info["ratio"] - len(b) / (2 * w.size)) < 1e-12


def test_validator_rejects_corruption():
    w = workloads.weights("down", rows=8, cols=1024).numpy().view(np.uint16)
    b = bytearray(uw.uw_encode(w))
    for mutate in (lambda x: x.__setitem__(0, ord("X")),          # magic
                   lambda x: x.__setitem__(4, 9),                 # version
                   lambda x: x.__setitem__(len(x) - 1, x[-1] ^ 1),  # payload (CRC)
                   ):
        bad = bytearray(b)
        mutate(bad)
        with pytest.raises(uw.UwError) as e:
            uw.uw_blob_info(bytes(bad))
        assert e.value.status == uw.UW_ERR_FORMAT
    with pytest.raises(uw.UwError) as e:
        uw.uw_blob_info(bytes(b[:-256]))
    assert e.value.status == uw.UW_ERR_FORMAT
    with pytest.raises(uw.UwError):
        uw.uw_blob_info(bytes(b[:100]))


def test_validator_rejects_consistent_but_wrong_tables():
    """Corrupt a table and fix the CRC: the structural checks must still fire."""
    import struct
    import zlib
    w = workloads.weights("down", rows=8, cols=1024).numpy().view(np.uint16)
    b = bytearray(uw.uw_encode(w))
    h = oblob.parse_header(bytes(b))

    def refresh(x):
        struct.pack_into("<I", x, 64, zlib.crc32(bytes(x[256:])))

    bad = bytearray(b)
    struct.pack_into("<H", bad, h.off_queue, 4000)  # lane 0 of block 0: more words than its block can hold
    refresh(bad)
    with pytest.raises(uw.UwError):
        uw.uw_blob_info(bytes(bad))
    bad = bytearray(b)
    first = struct.unpack_from("<H", bad, h.off_seg)[0]
    struct.pack_into("<H", bad, h.off_seg, first + 1)  # tile 0's segment one word longer, tile 1's shorter
    refresh(bad)
    with pytest.raises(uw.UwError):
        uw.uw_blob_info(bytes(bad))
    bad = bytearray(b)
    struct.pack_into("<I", bad, h.off_block + 4, struct.unpack_from("<I", bad, h.off_block + 4)[0] + 4)
    refresh(bad)
    with pytest.raises(uw.UwError):
        uw.uw_blob_info(bytes(bad))
    bad = bytearray(b)
    bad[104] = 1  # code lengths no longer a complete prefix code
    bad[105] = 1
    refresh(bad)
    with pytest.raises(uw.UwError):
        uw.uw_blob_info(bytes(bad))


def test_encoder_argument_errors():
    w = np.zeros((4, 64), dtype=np.uint16)
    lib = uw.library()
    size = ctypes.c_size_t(0)
    assert lib.uw_encode(None, 4, 64, None, None, ctypes.byref(size)) == uw.UW_ERR_INVALID
    assert lib.uw_encode(w.ctypes.data, 4, 100, None, None, ctypes.byref(size)) == uw.UW_ERR_INVALID
    assert lib.uw_encode(w.ctypes.data, 0, 64, None, None, ctypes.byref(size)) == uw.UW_ERR_INVALID
    opts = uw.uw_encode_opts(33, 0, 0, 0)
    assert lib.uw_encode(w.ctypes.data, 4, 64, ctypes.byref(opts), None, ctypes.byref(size)) == uw.UW_ERR_INVALID
    opts = uw.uw_encode_opts(0, 0, 24, 0)
    assert lib.uw_encode(w.ctypes.data, 4, 64, ctypes.byref(opts), None, ctypes.byref(size)) == uw.UW_ERR_INVALID
    # two-call pattern and a too-small buffer
    assert lib.uw_encode(w.ctypes.data, 4, 64, None, None, ctypes.byref(size)) == uw.UW_OK
    need = size.value
    small = ctypes.c_size_t(need - 1)
    buf = np.zeros(need, dtype=np.uint8)
    assert lib.uw_encode(w.ctypes.data, 4, 64, None, buf.ctypes.data, ctypes.byref(small)) == uw.UW_ERR_NOSPACE
    assert small.value == need
    assert "too small" in uw.uw_last_error()


def test_null_arguments_are_errors_without_a_gpu():
    lib = uw.library()
    assert lib.uw_blob_info(None, 0, None) == uw.UW_ERR_INVALID
    assert lib.uw_decompress(None, None, 0, None) == uw.UW_ERR_INVALID
    assert lib.uw_gemv_fused(None, None, 0, None, 0, None) == uw.UW_ERR_INVALID
    assert lib.uw_workspace_size(None, 1, 0) == 0
