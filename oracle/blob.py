"""Compressed-matrix blob: encoder and decoder (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows "Unweight: how we compressed an LLM 22% without sacrificing quality":
the sign+mantissa byte is kept verbatim and only the exponent byte is
Huffman coded (paragraph on Huffman coding of the exponent byte); a row of 64
weights holding an exponent outside the top-K palette is stored raw, decided
once per row (paragraph on rare exponents).  The pages give no byte layout;
the layout below is this project's, written out in full so that this module
and the library implement it independently.

Layout (all integers little-endian; every section starts 256-byte aligned):

  header, 256 bytes
     0 "UWB1"          4 u32 version=1      8 u32 header_bytes=256
    12 u32 flags (bit 0: plain mode)       16 i64 rows   24 i64 cols
    32 u32 K (palette entries)             36 u32 L (max code length)
    40 u32 G (groups of 64 per block)      44 u32 n_blocks
    48 u64 n_raw_groups                    56 u64 total_bytes
    64 u32 crc32 of bytes [256, total)     68 u32 max block stream bytes
    72 u8 palette[32]                     104 u8 code_len[32]
   136 u64 off_start_word  144 u64 off_first_raw  152 u64 off_raw_bits
   160 u64 off_lane_bits   168 u64 off_stream     176 u64 size_stream
   184 u64 off_raw         192 u64 size_raw       200 u64 off_sm
   208 u64 size_sm         216 u64 off_plain      224 u64 size_plain
  start_word  u32[n_blocks+1]  first 32-bit word of each block's stream
  first_raw   u32[n_blocks+1]  raw groups in all earlier blocks
  raw_bits    u32[n_blocks*W]  W = ceil(G/32); bit j (LSB first) = group j raw
  lane_bits   u16[n_blocks*64] bits in each lane's stream
  stream      per block: the 64 lane streams concatenated in lane order,
              codes bit-reversed and packed LSB-first, zero padded to 16 bytes
  raw         64 exponent bytes per raw group, groups in order
  sm          per block, ceil(G_b/16) tiles of 1024 bytes; byte
              (j>>4)*1024 + lane*16 + (j&15) is the sign+mantissa byte of
              weight 64*j + lane of the block (missing groups are zero)
  plain       (plain mode only) the bf16 bits, row-major

A group is 64 consecutive weights of the row-major matrix (cols % 64 == 0, so
it never straddles rows).  Block b holds groups [b*G, min((b+1)*G, total)).
Lane l of a block owns weight 64*j + l of each of its groups j.
"""
from __future__ import annotations

import struct
import zlib
from dataclasses import dataclass

import numpy as np

from . import huffman

MAGIC = b"UWB1"
VERSION = 1
HEADER_BYTES = 256
FLAG_PLAIN = 1
ALIGN = 256
MAX_K = 32


def _align(n: int) -> int:
    return (n + ALIGN - 1) // ALIGN * ALIGN


def choose_groups_per_block(rows: int, cols: int) -> int:
    """Default G: the largest multiple of 16 (<= 256) that keeps at least 2048
    blocks, preferring sizes that are a divisor or a multiple of the groups per
    row; a matrix too small for 2048 blocks takes the largest such G <= 64."""
    n = cols // 64
    total = rows * n
    cands = list(range(16, 257, 16))
    aligned = [g for g in cands if n % g == 0 or g % n == 0]
    pool = aligned or cands
    good = [g for g in pool if -(-total // g) >= 2048]
    if good:
        return max(good)
    small = [g for g in pool if g <= 64]
    return max(small) if small else min(pool)


@dataclass
class Header:
    rows: int
    cols: int
    flags: int
    K: int
    L: int
    G: int
    n_blocks: int
    n_raw_groups: int
    total_bytes: int
    crc32: int
    max_block_stream_bytes: int
    palette: list
    code_len: list
    off_start_word: int
    off_first_raw: int
    off_raw_bits: int
    off_lane_bits: int
    off_stream: int
    size_stream: int
    off_raw: int
    size_raw: int
    off_sm: int
    size_sm: int
    off_plain: int
    size_plain: int


_HDR = struct.Struct("<4sIIIqqIIIIQQII32s32sQQQQQQQQQQQQ")


def _pack_header(h: Header) -> bytes:
    pal = bytes(h.palette) + bytes(32 - len(h.palette))
    cl = bytes(h.code_len) + bytes(32 - len(h.code_len))
    raw = _HDR.pack(MAGIC, VERSION, HEADER_BYTES, h.flags, h.rows, h.cols, h.K, h.L, h.G,
                    h.n_blocks, h.n_raw_groups, h.total_bytes, h.crc32, h.max_block_stream_bytes,
                    pal, cl, h.off_start_word, h.off_first_raw, h.off_raw_bits, h.off_lane_bits,
                    h.off_stream, h.size_stream, h.off_raw, h.size_raw, h.off_sm, h.size_sm,
                    h.off_plain, h.size_plain)
    return raw + bytes(HEADER_BYTES - len(raw))


def parse_header(blob: bytes) -> Header:
    if len(blob) < HEADER_BYTES:
        raise ValueError("blob shorter than its header")
    f = _HDR.unpack_from(blob, 0)
    if f[0] != MAGIC or f[1] != VERSION or f[2] != HEADER_BYTES:
        raise ValueError("bad magic/version")
    K = f[6]
    h = Header(rows=f[4], cols=f[5], flags=f[3], K=K, L=f[7], G=f[8], n_blocks=f[9],
               n_raw_groups=f[10], total_bytes=f[11], crc32=f[12], max_block_stream_bytes=f[13],
               palette=list(f[14][:K]), code_len=list(f[15][:K]),
               off_start_word=f[16], off_first_raw=f[17], off_raw_bits=f[18], off_lane_bits=f[19],
               off_stream=f[20], size_stream=f[21], off_raw=f[22], size_raw=f[23],
               off_sm=f[24], size_sm=f[25], off_plain=f[26], size_plain=f[27])
    if h.total_bytes != len(blob):
        raise ValueError("size mismatch")
    if zlib.crc32(blob[HEADER_BYTES:]) != h.crc32:
        raise ValueError("crc mismatch")
    return h


def _emit_lane_streams(codes_rev, lens_of, sym_idx, nonraw):
    """Bit emission of one block: sym_idx[j, lane] (palette index), nonraw[j].

    Returns (lane_bits[64], stream bytes padded to 16 bytes).  Each lane's codes
    go LSB-first into its own stream in increasing j; lanes are concatenated in
    lane order with no padding between them.
    """
    codes_rev = np.asarray(codes_rev, dtype=np.int64)
    lens_of = np.asarray(lens_of, dtype=np.int64)
    s = sym_idx[np.asarray(nonraw, dtype=bool)].T  # [lane, j] in stream order
    lens = lens_of[s]
    lane_bits = lens.sum(axis=1)
    flat_len = lens.ravel()
    flat_code = codes_rev[s].ravel()
    offset = np.cumsum(flat_len) - flat_len  # first bit of each code
    nbits = int(flat_len.sum())
    padded = -(-nbits // 128) * 128
    arr = np.zeros(padded, dtype=np.uint8)
    for t in range(int(lens_of.max(initial=0))):
        m = flat_len > t
        arr[offset[m] + t] = (flat_code[m] >> t) & 1
    return lane_bits, np.packbits(arr, bitorder="little").tobytes()


def encode(w_bits, K: int = 16, L: int = 6, G: int | None = None, allow_plain: bool = True) -> bytes:
    """bf16 bit patterns [rows, cols] (cols % 64 == 0) -> blob bytes.

    Plain mode (the bf16 bits stored as they are) is taken when nothing can be
    coded or when the coded payload would not be smaller than 2*rows*cols
    bytes, unless allow_plain is False (then only an empty code forces it).
    """
    w = np.ascontiguousarray(np.asarray(w_bits).astype(np.uint16))
    if w.ndim != 2:
        raise ValueError("need a 2-D matrix")
    rows, cols = w.shape
    if rows < 1 or cols < 64 or cols % 64:
        raise ValueError("rows >= 1 and cols a positive multiple of 64 required")
    if not (1 <= K <= MAX_K) or not (1 <= L <= 12) or K > (1 << L):
        raise ValueError("K in [1,32], L in [1,12] and K <= 2^L")
    if G is None:
        G = choose_groups_per_block(rows, cols)
    if G < 16 or G % 16 or G > 1024:
        raise ValueError("G must be a multiple of 16 in [16, 1024]")

    e, sm = huffman.split_bf16(w.ravel())
    n_groups = rows * cols // 64
    eg = e.reshape(n_groups, 64)
    smg = sm.reshape(n_groups, 64)
    hist = huffman.histogram(e)
    pal = huffman.palette(hist, K)
    in_pal = np.isin(eg, np.array(pal, dtype=np.uint8))
    raw = ~in_pal.all(axis=1)
    chist = huffman.histogram(eg[~raw]) if (~raw).any() else np.zeros(256, dtype=np.int64)
    coded = [i for i, s in enumerate(pal) if chist[s] > 0]
    if len(coded) > (1 << L):
        raise ValueError("palette larger than 2^L")
    lens_coded = huffman.package_merge([int(chist[pal[i]]) for i in coded], L,
                                       keys=[pal[i] for i in coded])
    code_len = [0] * len(pal)
    for i, l in zip(coded, lens_coded):
        code_len[i] = l
    codes = huffman.canonical_codes(code_len, pal)
    codes_rev = [huffman.reverse_bits(c, l) if l else 0 for c, l in zip(codes, code_len)]

    plain_payload = 2 * rows * cols
    if not coded:
        return _plain_blob(w, rows, cols)

    # palette index of every exponent (only meaningful in non-raw groups)
    lut = np.zeros(256, dtype=np.int64)
    for i, s in enumerate(pal):
        lut[s] = i
    sym = lut[eg]

    n_blocks = -(-n_groups // G)
    W = -(-G // 32)
    start_word = np.zeros(n_blocks + 1, dtype=np.uint32)
    first_raw = np.zeros(n_blocks + 1, dtype=np.uint32)
    raw_bits = np.zeros(n_blocks * W, dtype=np.uint32)
    lane_bits = np.zeros(n_blocks * 64, dtype=np.uint16)
    streams = []
    sm_tiles = []
    words = 0
    nraw = 0
    max_stream = 0
    for b in range(n_blocks):
        g0, g1 = b * G, min((b + 1) * G, n_groups)
        nonraw = ~raw[g0:g1]
        lb, sbytes = _emit_lane_streams(codes_rev, code_len, sym[g0:g1], nonraw)
        lane_bits[b * 64:(b + 1) * 64] = lb
        start_word[b] = words
        first_raw[b] = nraw
        words += len(sbytes) // 4
        max_stream = max(max_stream, len(sbytes))
        streams.append(sbytes)
        for j in range(g1 - g0):
            if raw[g0 + j]:
                raw_bits[b * W + j // 32] |= np.uint32(1 << (j % 32))
                nraw += 1
        ntiles = -(-(g1 - g0) // 16)
        tile = np.zeros((ntiles * 16, 64), dtype=np.uint8)
        tile[: g1 - g0] = smg[g0:g1]
        # (j>>4)*1024 + lane*16 + (j&15): tiles of [lane][16 groups]
        sm_tiles.append(tile.reshape(ntiles, 16, 64).transpose(0, 2, 1).tobytes())
    start_word[n_blocks] = words
    first_raw[n_blocks] = nraw
    raw_bytes = eg[raw].tobytes()
    stream = b"".join(streams)
    smb = b"".join(sm_tiles)

    off = HEADER_BYTES
    sections = {}
    for name, payload in (("start_word", start_word.tobytes()), ("first_raw", first_raw.tobytes()),
                          ("raw_bits", raw_bits.tobytes()), ("lane_bits", lane_bits.tobytes()),
                          ("stream", stream), ("raw", raw_bytes), ("sm", smb)):
        off = _align(off)
        sections[name] = (off, payload)
        off += len(payload)
    total = off
    if allow_plain and total - HEADER_BYTES >= plain_payload:
        return _plain_blob(w, rows, cols)

    body = bytearray(total)
    for name, (o, payload) in sections.items():
        body[o:o + len(payload)] = payload
    h = Header(rows=rows, cols=cols, flags=0, K=len(pal), L=L, G=G, n_blocks=n_blocks,
               n_raw_groups=nraw, total_bytes=total, crc32=0, max_block_stream_bytes=max_stream,
               palette=pal, code_len=code_len,
               off_start_word=sections["start_word"][0], off_first_raw=sections["first_raw"][0],
               off_raw_bits=sections["raw_bits"][0], off_lane_bits=sections["lane_bits"][0],
               off_stream=sections["stream"][0], size_stream=len(stream),
               off_raw=sections["raw"][0], size_raw=len(raw_bytes),
               off_sm=sections["sm"][0], size_sm=len(smb), off_plain=0, size_plain=0)
    h.crc32 = zlib.crc32(bytes(body[HEADER_BYTES:]))
    body[:HEADER_BYTES] = _pack_header(h)
    return bytes(body)


def _plain_blob(w, rows, cols) -> bytes:
    payload = w.astype("<u2").tobytes()
    off = _align(HEADER_BYTES)
    total = off + len(payload)
    body = bytearray(total)
    body[off:] = payload
    h = Header(rows=rows, cols=cols, flags=FLAG_PLAIN, K=0, L=0, G=0, n_blocks=0, n_raw_groups=0,
               total_bytes=total, crc32=zlib.crc32(bytes(body[HEADER_BYTES:])),
               max_block_stream_bytes=0, palette=[], code_len=[],
               off_start_word=0, off_first_raw=0, off_raw_bits=0, off_lane_bits=0,
               off_stream=0, size_stream=0, off_raw=0, size_raw=0, off_sm=0, size_sm=0,
               off_plain=off, size_plain=len(payload))
    body[:HEADER_BYTES] = _pack_header(h)
    return bytes(body)


def _section(blob: bytes, off: int, count: int, dtype) -> np.ndarray:
    return np.frombuffer(blob, dtype=dtype, count=count, offset=off)


def decode(blob: bytes) -> np.ndarray:
    """blob -> bf16 bit patterns [rows, cols] (uint16).

    Lane-lockstep: every (block, lane) stream advances one symbol per group
    step, all streams at once; the loop runs over the group index j only.  A
    symbol is found by reading the next L bits of the stream and matching them
    against each code's bit-reversed pattern of its own length.
    """
    h = parse_header(blob)
    rows, cols = h.rows, h.cols
    if h.flags & FLAG_PLAIN:
        return _section(blob, h.off_plain, rows * cols, "<u2").reshape(rows, cols).astype(np.uint16)
    n_groups = rows * cols // 64
    nb, G, W = h.n_blocks, h.G, -(-h.G // 32)
    start_word = _section(blob, h.off_start_word, nb + 1, "<u4").astype(np.int64)
    first_raw = _section(blob, h.off_first_raw, nb + 1, "<u4").astype(np.int64)
    raw_bits = _section(blob, h.off_raw_bits, nb * W, "<u4").astype(np.int64).reshape(nb, W)
    lane_bits = _section(blob, h.off_lane_bits, nb * 64, "<u2").astype(np.int64).reshape(nb, 64)
    stream_bits = np.unpackbits(np.frombuffer(blob, dtype=np.uint8, count=h.size_stream,
                                              offset=h.off_stream), bitorder="little")
    stream_bits = np.concatenate([stream_bits, np.zeros(16, dtype=np.uint8)])
    raw = _section(blob, h.off_raw, h.size_raw, np.uint8)
    sm_all = _section(blob, h.off_sm, h.size_sm, np.uint8)

    codes = huffman.canonical_codes(h.code_len, h.palette)
    # table of the next L stream bits (bit t of the index = t-th next stream bit)
    sym_of = np.full(1 << h.L, -1, dtype=np.int64)
    len_of = np.zeros(1 << h.L, dtype=np.int64)
    for s, (c, l) in enumerate(zip(codes, h.code_len)):
        if l == 0:
            continue
        pat = huffman.reverse_bits(c, l)
        for idx in range(1 << h.L):
            if idx & ((1 << l) - 1) == pat:
                sym_of[idx] = s
                len_of[idx] = l
    pal = np.array(h.palette, dtype=np.uint8)

    # per (block, lane) bit position: block base + exclusive prefix of lane bits
    lane_start = np.cumsum(lane_bits, axis=1) - lane_bits
    pos = start_word[:nb, None] * 32 + lane_start  # [nb, 64]
    out_e = np.zeros((nb * G + 16, 64), dtype=np.uint8)
    raw_seen = np.zeros(nb, dtype=np.int64)
    weights_of_bit = (1 << np.arange(h.L, dtype=np.int64))
    lanes = np.arange(64)
    for j in range(G):
        gidx = np.arange(nb) * G + j
        valid = gidx < n_groups
        is_raw = ((raw_bits[:, j // 32] >> (j % 32)) & 1).astype(bool) & valid
        coded = valid & ~is_raw
        if coded.any():
            p = pos[coded]
            peek = (stream_bits[p[:, :, None] + np.arange(h.L)] * weights_of_bit).sum(axis=2)
            s = sym_of[peek]
            if (s < 0).any():
                raise ValueError("invalid code in stream")
            out_e[gidx[coded]] = pal[s]
            pos[coded] = p + len_of[peek]
        if is_raw.any():
            ridx = first_raw[:nb][is_raw] + raw_seen[is_raw]
            out_e[gidx[is_raw]] = raw[(ridx[:, None] * 64 + lanes[None, :])]
            raw_seen[is_raw] += 1
    # every lane must end exactly where the next lane starts
    if not np.array_equal(pos - start_word[:nb, None] * 32, lane_start + lane_bits):
        raise ValueError("lane stream length mismatch")
    e = out_e[:n_groups]
    # sm bytes: block b, group j, lane l at b*G*64 + (j>>4)*1024 + l*16 + (j&15)
    g = np.arange(n_groups)
    b, j = g // G, g % G
    base = b * G * 64 + (j >> 4) * 1024 + (j & 15)
    smg = sm_all[base[:, None] + lanes[None, :] * 16]
    return huffman.join_bf16(e, smg).reshape(rows, cols)


def stats(blob: bytes) -> dict:
    """Sizes and ratios of a blob, for reporting."""
    h = parse_header(blob)
    weights = h.rows * h.cols
    return {
        "rows": h.rows, "cols": h.cols, "plain": bool(h.flags & FLAG_PLAIN), "K": h.K, "L": h.L,
        "G": h.G, "n_blocks": h.n_blocks, "raw_groups": h.n_raw_groups,
        "raw_group_frac": h.n_raw_groups / (weights // 64),
        "bytes": h.total_bytes, "ratio": h.total_bytes / (2 * weights),
        "bits_per_weight": 8 * h.total_bytes / weights,
    }
