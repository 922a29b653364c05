"""The oracle's two decoders of the blob layout against each other and
against the original weights.

oracle/blob.decode_reference is the plain per-block, per-group, per-lane
loop written from the layout description; oracle/blob.decode is the
vectorised lane-lockstep decoder.  Both must return the original weights on
the hand-derived fixtures (tests/golden/blob_*_hand.json, whose bytes the
blob tests pin field by field) and on random matrices across palette sizes,
code-length limits, block sizes (ragged last blocks), raw groups, special
values and plain mode.  A decoder that reads a word from the wrong place,
takes words in the wrong lane order, skips a raw group's bytes or misplaces
a sign+mantissa byte fails these.
"""
import numpy as np
import pytest

import workloads
from oracle import blob
from tests.test_oracle_blob import _fixture_1x64, _fixture_1x128, _fixture_1x4096


@pytest.mark.parametrize("make,K,L", [(_fixture_1x64, 16, 6), (_fixture_1x128, 16, 6), (_fixture_1x4096, 16, 6)])
def test_reference_decoder_on_hand_fixtures(make, K, L):
    w = make()
    b = blob.encode(w, K=K, L=L, allow_plain=False)
    assert np.array_equal(blob.decode_reference(b), w)


@pytest.mark.parametrize("K,L,G", [(16, 6, None), (16, 6, 16), (16, 6, 48), (4, 3, 32), (32, 8, 64),
                                   (16, 12, 80), (1, 1, 16), (2, 2, 16)])
def test_reference_decoder_agrees_on_random_matrices(K, L, G):
    for name, rows, cols in (("down", 7, 640), ("small", 5, 1024)):
        w = workloads.weights(name, rows=rows, cols=cols, seed=rows * 31 + cols + K).numpy().view(np.uint16)
        b = blob.encode(w, K=K, L=L, G=G)
        ref = blob.decode_reference(b)
        assert np.array_equal(ref, w)
        assert np.array_equal(ref, blob.decode(b))


def test_reference_decoder_special_values_and_plain():
    sv = np.array(workloads.special_values_bf16(), dtype=np.uint16)
    w = workloads.weights("small", rows=4, cols=256, seed=9).numpy().view(np.uint16).copy()
    w.ravel()[::37][: len(sv)] = sv
    b = blob.encode(w, allow_plain=False)
    assert blob.stats(b)["raw_groups"] > 0
    assert np.array_equal(blob.decode_reference(b), w)
    r = workloads.weights("randbits", rows=3, cols=128, seed=10).numpy().view(np.uint16)
    bp = blob.encode(r)
    assert blob.stats(bp)["plain"]
    assert np.array_equal(blob.decode_reference(bp), r)


def test_reference_decoder_rejects_a_wrong_word_order():
    # swapping two taken words inside a segment must not decode to the input
    w = workloads.weights("small", rows=2, cols=1024, seed=12).numpy().view(np.uint16)
    b = bytearray(blob.encode(w, K=16, L=6, allow_plain=False))
    h = blob.parse_header(bytes(b))
    o = h.off_queue + 136  # the head's first words (lane order)
    k = next(k for k in range(1, 64) if bytes(b[o:o + 4]) != bytes(b[o + 4 * k:o + 4 * k + 4]))
    b[o:o + 4], b[o + 4 * k:o + 4 * k + 4] = b[o + 4 * k:o + 4 * k + 4], b[o:o + 4]
    import zlib
    import struct
    struct.pack_into("<I", b, 64, zlib.crc32(bytes(b[256:])))
    try:
        out = blob.decode_reference(bytes(b))
    except ValueError:
        return
    assert not np.array_equal(out, w)
