"""The direct-palette form of a bf16 matrix (oracle): 4-bit exponent index plus
the raw sign+mantissa byte per weight.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "Unweight: how we compressed an LLM 22% without sacrificing quality",
section on the four execution pipelines: the direct-palette pipeline converts
the weights to a compact 4-bit form when the model is loaded and the matmul
rebuilds bf16 on the fly from those indices, with no preprocessing pass.
The pages give the palette (the 16 most frequent exponents) and the escape of
64-weight groups that use another exponent (paragraph on rare exponents) but
not the byte layout, so the layout below is this library's (format UWP1):

    header, 64 bytes: "UWP1", u32 version 1, u64 rows, u64 cols, u64 n_raw,
        u8 palette[16] (index i -> exponent; unused entries 0), u32 n_pal,
        zero padding
    sm     rows*cols bytes: (sign << 7) | mantissa of each weight, row-major
    idx    rows*cols/2 bytes: the palette index of weight i in the low nibble
           of byte i/2 when i is even, the high nibble when odd; 0 for the
           weights of raw groups
    flags  u32 words: bit (g % 32) of word g/32 set when group g is raw
    prefix u32 per 1024-weight tile: raw groups in the tiles before it
    raw    64 exponent bytes per raw group, groups in order
Every section starts at a multiple of 256 bytes; the total is rounded up to
256.  cols must be a multiple of 1024, so no tile crosses a row.
"""
from __future__ import annotations

import numpy as np

from . import huffman

MAGIC = b"UWP1"
HEADER_BYTES = 64
PALETTE_SIZE = 16
TILE = 1024
GROUP = 64


def _align(n: int) -> int:
    return (n + 255) // 256 * 256


def layout(rows: int, cols: int, n_raw: int) -> dict:
    """Byte offsets of the sections and the total size."""
    n = rows * cols
    groups = n // GROUP
    off = {"sm": _align(HEADER_BYTES)}
    off["idx"] = _align(off["sm"] + n)
    off["flags"] = _align(off["idx"] + n // 2)
    off["prefix"] = _align(off["flags"] + 4 * ((groups + 31) // 32))
    off["raw"] = _align(off["prefix"] + 4 * (n // TILE))
    off["total"] = _align(off["raw"] + GROUP * n_raw)
    return off


def encode(bits: np.ndarray) -> bytes:
    """bf16 bit patterns [rows, cols] -> the UWP1 bytes."""
    w = np.asarray(bits).astype(np.uint16)
    rows, cols = w.shape
    if rows < 1 or cols < TILE or cols % TILE:
        raise ValueError("cols must be a positive multiple of 1024")
    e, sm = huffman.split_bf16(w.reshape(-1))
    pal = huffman.palette(huffman.histogram(e), PALETTE_SIZE)
    index_of = np.zeros(256, dtype=np.uint8)
    index_of[np.array(pal, dtype=np.int64)] = np.arange(len(pal), dtype=np.uint8)
    # a group is raw when any of its exponents is outside the palette
    in_pal = np.isin(e, np.array(pal, dtype=np.uint8))
    raw = ~in_pal.reshape(-1, GROUP).all(axis=1)
    idx = np.where(np.repeat(raw, GROUP), np.uint8(0), index_of[e]).astype(np.uint8)
    n_raw = int(raw.sum())
    off = layout(rows, cols, n_raw)
    out = bytearray(off["total"])
    hdr = bytearray(HEADER_BYTES)
    hdr[0:4] = MAGIC
    hdr[4:8] = (1).to_bytes(4, "little")
    hdr[8:16] = rows.to_bytes(8, "little")
    hdr[16:24] = cols.to_bytes(8, "little")
    hdr[24:32] = n_raw.to_bytes(8, "little")
    hdr[32:32 + len(pal)] = bytes(pal)
    hdr[48:52] = len(pal).to_bytes(4, "little")
    out[0:HEADER_BYTES] = hdr
    out[off["sm"]:off["sm"] + sm.size] = sm.tobytes()
    packed = (idx[0::2] | (idx[1::2] << 4)).astype(np.uint8)
    out[off["idx"]:off["idx"] + packed.size] = packed.tobytes()
    for g in map(int, np.flatnonzero(raw)):
        word = off["flags"] + 4 * (g // 32)
        v = int.from_bytes(out[word:word + 4], "little") | (1 << (g % 32))
        out[word:word + 4] = v.to_bytes(4, "little")
    before = 0
    for t in range(e.size // TILE):
        out[off["prefix"] + 4 * t:off["prefix"] + 4 * t + 4] = before.to_bytes(4, "little")
        before += int(raw[16 * t:16 * t + 16].sum())
    for k, g in enumerate(map(int, np.flatnonzero(raw))):
        out[off["raw"] + GROUP * k:off["raw"] + GROUP * (k + 1)] = e[GROUP * g:GROUP * (g + 1)].tobytes()
    return bytes(out)


def parse(blob: bytes) -> dict:
    """Header fields and section views of a UWP1 blob."""
    if blob[0:4] != MAGIC or int.from_bytes(blob[4:8], "little") != 1:
        raise ValueError("not a UWP1 blob")
    rows = int.from_bytes(blob[8:16], "little")
    cols = int.from_bytes(blob[16:24], "little")
    n_raw = int.from_bytes(blob[24:32], "little")
    n_pal = int.from_bytes(blob[48:52], "little")
    off = layout(rows, cols, n_raw)
    if len(blob) != off["total"]:
        raise ValueError("size does not match the header")
    n = rows * cols
    b = np.frombuffer(blob, dtype=np.uint8)
    return {
        "rows": rows, "cols": cols, "n_raw": n_raw, "palette": list(blob[32:32 + n_pal]),
        "sm": b[off["sm"]:off["sm"] + n],
        "idx": b[off["idx"]:off["idx"] + n // 2],
        "flags": b[off["flags"]:off["flags"] + 4 * ((n // GROUP + 31) // 32)].view(np.uint32),
        "prefix": b[off["prefix"]:off["prefix"] + 4 * (n // TILE)].view(np.uint32),
        "raw": b[off["raw"]:off["raw"] + GROUP * n_raw],
    }


def decode(blob: bytes) -> np.ndarray:
    """UWP1 bytes -> bf16 bit patterns [rows, cols]."""
    p = parse(blob)
    rows, cols = p["rows"], p["cols"]
    n = rows * cols
    g = np.arange(n) // GROUP
    raw = ((p["flags"][g // 32] >> (g % 32).astype(np.uint32)) & 1).astype(bool)
    nib = (p["idx"][np.arange(n) // 2] >> (4 * (np.arange(n) & 1)).astype(np.uint8)) & 0xF
    e = np.array(p["palette"] + [0] * (PALETTE_SIZE - len(p["palette"])), dtype=np.uint8)[nib]
    # the k-th raw group (counted from the tile's prefix) holds raw bytes k*64 ..
    raw_groups = np.flatnonzero(raw.reshape(-1, GROUP)[:, 0])
    for k, grp in enumerate(raw_groups):
        t = grp * GROUP // TILE
        in_tile = int(raw.reshape(-1, GROUP)[16 * t:grp, 0].sum())
        slot = int(p["prefix"][t]) + in_tile
        e[GROUP * grp:GROUP * (grp + 1)] = p["raw"][GROUP * slot:GROUP * (slot + 1)]
    return huffman.join_bf16(e, p["sm"]).reshape(rows, cols)


def decode_one(blob: bytes, r: int, c: int) -> int:
    """Weight (r, c) alone, read straight from the sections (tiny cases)."""
    p = parse(blob)
    i = r * p["cols"] + c
    grp = i // GROUP
    if (int(p["flags"][grp // 32]) >> (grp % 32)) & 1:
        t = i // TILE
        k = int(p["prefix"][t])
        for h in range(16 * t, grp):
            k += (int(p["flags"][h // 32]) >> (h % 32)) & 1
        e = int(p["raw"][GROUP * k + i % GROUP])
    else:
        e = p["palette"][(int(p["idx"][i // 2]) >> (4 * (i & 1))) & 0xF]
    return int(huffman.join_bf16(np.uint8(e), p["sm"][i]))
