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
     0 "UWB2"          4 u32 version=2      8 u32 header_bytes=256
    12 u32 flags (bit 0: plain mode)       16 i64 rows   24 i64 cols
    32 u32 K (palette entries)             36 u32 L (max code length)
    40 u32 G (groups of 64 per block)      44 u32 n_blocks
    48 u64 n_raw_groups                    56 u64 total_bytes
    64 u32 crc32 of bytes [256, total)     68 u32 largest segment, bytes
    72 u8 palette[32]                     104 u8 code_len[32]
   136 u32 R (groups per refill check)    140 u32 zero
   144 u64 off_block   152 u64 off_seg     160 u64 off_queue  168 u64 size_queue
   176 u64 off_sm      184 u64 size_sm     192 u64 off_plain  200 u64 size_plain
  block   u32[n_blocks+1]  byte offset of each block's data in the queue section
  seg     u16[n_blocks*T]  T = ceil(G/16); entry t = end of tile t's segment,
                           in 4-byte words from the block's start (entries past
                           the block's last tile repeat its end)
  queue   per block, its segments back to back (each a whole number of words)
  sm      per block, ceil(G_b/16) tiles of 1024 bytes; byte
          (j>>4)*1024 + lane*16 + (j&15) is the sign+mantissa byte of weight
          64*j + lane of the block (missing groups are zero)
  plain   (plain mode only) the bf16 bits, row-major

A group is 64 consecutive weights of the row-major matrix (cols % 64 == 0, so
it never straddles rows).  Block b holds groups [b*G, min((b+1)*G, total)) =
G_b groups; tile t of a block is its groups [16t, 16t+16).  Lane l of a block
owns weight 64*j + l of each of its groups j.

Code streams.  Lane l's codes (groups that are not raw, in increasing j; the
codes bit-reversed and packed LSB-first) form a bit string of bits_l bits, cut
into n_l = ceil(bits_l / 32) little-endian 32-bit words.  The decoder of a
lane holds three words (w0, w1, w2) = words (s-1, s, s+1) after s shifts
(word -1 reads as 0, so does any word past n_l - 1) and qm, the bit offset of
(next code - 2) inside w0: at the block start s = 0 and qm = 30.  A code of
length len is decoded from bits qm+2 ... of (w0, w1) and adds len to qm.
After every R-th group of the block (group j with (j+1) % R == 0; raw groups
count) every lane with qm >= 32 shifts: qm -= 32, w0 = w1, w1 = w2, and w2
becomes the lane's next word, taken from the block's data, if the lane has
taken fewer than n_l words.  R = 4 for L <= 7 and 2 otherwise, so the codes
between two checks span at most 28 bits and always lie in (w0, w1).  The
words taken at one check are stored in lane order; the checks of tile t
store their words in tile t's segment.

Segments.  Tile t's segment is: (tile 0 only) lane_words u16[64] = n_l,
raw_bits u32[ceil(G/32)] (bit j, LSB first: group j is raw), word 0 of every
lane with n_l >= 1 in lane order, word 1 of every lane with n_l >= 2 in lane
order; then the 64 exponent bytes (lane order) of each raw group of the tile,
in group order; then the words taken at the tile's checks.
"""
from __future__ import annotations

import math
import struct
import zlib
from dataclasses import dataclass

import numpy as np

from . import huffman

MAGIC = b"UWB2"
VERSION = 2
HEADER_BYTES = 256
FLAG_PLAIN = 1
ALIGN = 256
MAX_K = 32


def _align(n: int) -> int:
    return (n + ALIGN - 1) // ALIGN * ALIGN


def choose_groups_per_block(rows: int, cols: int) -> int:
    """Default G (a layout choice; the pages fix no block size).

    Candidates are the multiples of 16 up to 256 that divide the groups per
    row or are a multiple of it, and, when the groups per row are a multiple
    of 16, every larger G whose work unit (lcm of G and the groups per row)
    holds at most 8 blocks: a row then spans at most two blocks.  Among those
    that keep at least 2048 blocks, the one whose blocks spread most evenly
    over the 1024 SIMDs of a 256-CU part, one block per wave and 4 waves per
    SIMD in a round, counting a block start as one more tile: with
    b = ceil(blocks / 1024) blocks per SIMD, the least
    ceil(b / 4) * 4 * (G/16 + 1) (a round costs as much as a full one), ties
    to the larger G.  A matrix too small for 2048 blocks takes the largest
    divisor or multiple of the groups per row that is <= 64."""
    n = cols // 64
    total = rows * n
    cands = list(range(16, 257, 16))
    aligned = [g for g in cands if n % g == 0 or g % n == 0]
    wide = aligned + [g for g in cands
                      if n % 16 == 0 and g > n and g not in aligned and n // math.gcd(g, n) <= 8]
    good = [g for g in (wide or cands) if -(-total // g) >= 2048]
    if good:
        def cost(g):
            per_simd = -(-(-(-total // g)) // 1024)
            return -(-per_simd // 4) * 4 * (g // 16 + 1)
        return min(good, key=lambda g: (cost(g), -g))
    pool = aligned or cands
    small = [g for g in pool if g <= 64]
    return max(small) if small else min(pool)


def check_groups(L: int) -> int:
    """R, the groups between two refill checks: the codes in between must fit
    in the 30 bits a lane can always see (4 codes of <= 7 bits, else 2)."""
    return 4 if L <= 7 else 2


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
    max_segment_bytes: int
    palette: list
    code_len: list
    R: int
    off_block: int
    off_seg: int
    off_queue: int
    size_queue: int
    off_sm: int
    size_sm: int
    off_plain: int
    size_plain: int


_HDR = struct.Struct("<4sIIIqqIIIIQQII32s32sIIQQQQQQQQ")


def _pack_header(h: Header) -> bytes:
    pal = bytes(h.palette) + bytes(32 - len(h.palette))
    cl = bytes(h.code_len) + bytes(32 - len(h.code_len))
    raw = _HDR.pack(MAGIC, VERSION, HEADER_BYTES, h.flags, h.rows, h.cols, h.K, h.L, h.G,
                    h.n_blocks, h.n_raw_groups, h.total_bytes, h.crc32, h.max_segment_bytes,
                    pal, cl, h.R, 0, h.off_block, h.off_seg, h.off_queue, h.size_queue,
                    h.off_sm, h.size_sm, h.off_plain, h.size_plain)
    return raw + bytes(HEADER_BYTES - len(raw))


def parse_header(blob: bytes) -> Header:
    if len(blob) < HEADER_BYTES:
        raise ValueError("blob shorter than its header")
    f = _HDR.unpack_from(blob, 0)
    if f[0] != MAGIC or f[1] != VERSION or f[2] != HEADER_BYTES:
        raise ValueError("bad magic/version")
    K = f[6]
    h = Header(rows=f[4], cols=f[5], flags=f[3], K=K, L=f[7], G=f[8], n_blocks=f[9],
               n_raw_groups=f[10], total_bytes=f[11], crc32=f[12], max_segment_bytes=f[13],
               palette=list(f[14][:K]), code_len=list(f[15][:K]), R=f[16],
               off_block=f[18], off_seg=f[19], off_queue=f[20], size_queue=f[21],
               off_sm=f[22], size_sm=f[23], off_plain=f[24], size_plain=f[25])
    if h.total_bytes != len(blob):
        raise ValueError("size mismatch")
    if zlib.crc32(blob[HEADER_BYTES:]) != h.crc32:
        raise ValueError("crc mismatch")
    return h


def _lane_streams(codes_rev, code_len, sym, coded):
    """Code streams of every (block, lane): sym[b, j, lane] palette indices,
    coded[b, j] (group exists and is not raw).  Each lane's codes go LSB-first
    into its own stream in increasing j.  Returns (words[b, lane, i] uint32,
    n[b, lane] = words used, lens[b, j, lane] code lengths, 0 where not coded)."""
    nb, G, _ = sym.shape
    lens_of = np.asarray(code_len, dtype=np.int32)
    rev = np.asarray(codes_rev, dtype=np.int64)
    lens = lens_of[sym] * coded[:, :, None]
    start = np.cumsum(lens, axis=1, dtype=np.int32) - lens  # first bit of each code in its lane stream
    bits = lens.sum(axis=1)  # [nb, 64]
    maxw = max(1, -(-int(bits.max(initial=0)) // 32)) + 1
    bi, ji, li = np.nonzero(lens)
    code = rev[sym[bi, ji, li]]
    st = start[bi, ji, li].astype(np.int64)
    # a code at stream bit st lands in word st // 32, its high part (if it
    # crosses the word end) in the next word; codes never overlap, so the
    # per-word sums of the shifted parts are the word values (exact in fp64)
    lo = (code << (st % 32)) & 0xFFFFFFFF
    hi = code >> (32 - st % 32)
    slot = (bi * 64 + li) * maxw + st // 32
    acc = np.bincount(slot, weights=lo.astype(np.float64), minlength=nb * 64 * maxw)
    acc += np.bincount(slot + 1, weights=hi.astype(np.float64), minlength=nb * 64 * maxw)[: nb * 64 * maxw]
    words = acc.astype(np.uint64).astype(np.uint32).reshape(nb, 64, maxw)
    return words, -(-bits // 32), lens


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
    R = check_groups(L)

    n_blocks = -(-n_groups // G)
    W = -(-G // 32)
    T = -(-G // 16)
    pad = n_blocks * G - n_groups
    symb = np.concatenate([sym.astype(np.int16), np.zeros((pad, 64), np.int16)]).reshape(n_blocks, G, 64)
    rawb = np.concatenate([raw, np.zeros(pad, bool)]).reshape(n_blocks, G)
    live = (np.arange(n_blocks)[:, None] * G + np.arange(G)[None, :]) < n_groups
    coded_g = live & ~rawb
    words, lane_n, lens = _lane_streams(codes_rev, code_len, symb, coded_g)
    gb = np.minimum(G, n_groups - np.arange(n_blocks) * G)

    # the decoder's refill checks, all blocks and lanes at once
    qm = np.full((n_blocks, 64), 30, dtype=np.int64)
    taken = np.minimum(lane_n, 2)
    checks = []  # (tile, need[b, lane], word[b, lane]) per check
    for j in range(G):
        qm += lens[:, j, :]
        if (j + 1) % R == 0:
            chk = live[:, j][:, None]
            assert (qm[chk[:, 0]] < 64).all()
            shift = chk & (qm >= 32)
            need = shift & (taken < lane_n)
            idx = np.minimum(taken, words.shape[2] - 1)
            val = np.take_along_axis(words, idx[:, :, None], axis=2)[:, :, 0]
            checks.append((j // 16, need, val))
            qm = np.where(shift, qm - 32, qm)
            taken = taken + need
    assert np.array_equal(taken, lane_n), "every word is taken exactly once"
    c_tile = np.array([c[0] for c in checks], dtype=np.int64)
    c_need = np.stack([c[1] for c in checks], axis=1) if checks else np.zeros((n_blocks, 0, 64), bool)
    c_val = np.stack([c[2] for c in checks], axis=1) if checks else np.zeros((n_blocks, 0, 64), np.uint32)
    raw_bits = np.zeros((n_blocks, W), dtype=np.uint32)
    for j in range(G):
        raw_bits[:, j // 32] |= (rawb[:, j].astype(np.uint32) << np.uint32(j % 32))
    lanes_has = [lane_n >= 1, lane_n >= 2]

    block_off = np.zeros(n_blocks + 1, dtype=np.uint32)
    seg = np.zeros(n_blocks * T, dtype=np.uint16)
    datas = []
    sm_tiles = []
    nbytes = 0
    max_seg = 0
    for b in range(n_blocks):
        g0, g1 = b * G, min((b + 1) * G, n_groups)
        ntiles = -(-(g1 - g0) // 16)
        head = (lane_n[b].astype("<u2").tobytes() + raw_bits[b].astype("<u4").tobytes()
                + words[b, lanes_has[0][b], 0].astype("<u4").tobytes()
                + words[b, lanes_has[1][b], 1].astype("<u4").tobytes())
        taken_vals = c_val[b][c_need[b]]  # (check, lane) order
        per_check = c_need[b].sum(axis=1)
        per_tile = np.bincount(c_tile, weights=per_check, minlength=T).astype(np.int64)
        cut = np.concatenate([[0], np.cumsum(per_tile)])
        end = 0
        parts = []
        for t in range(T):
            if t < ntiles:
                rj = [j for j in range(16 * t, min(16 * t + 16, g1 - g0)) if rawb[b, j]]
                segb = ((head if t == 0 else b"") + b"".join(eg[g0 + j].tobytes() for j in rj)
                        + taken_vals[cut[t]:cut[t + 1]].astype("<u4").tobytes())
                parts.append(segb)
                end += len(segb)
                max_seg = max(max_seg, len(segb))
            seg[b * T + t] = end // 4
        block_off[b] = nbytes
        data = b"".join(parts)
        datas.append(data)
        nbytes += len(data)
        tile = np.zeros((ntiles * 16, 64), dtype=np.uint8)
        tile[: g1 - g0] = smg[g0:g1]
        # (j>>4)*1024 + lane*16 + (j&15): tiles of [lane][16 groups]
        sm_tiles.append(tile.reshape(ntiles, 16, 64).transpose(0, 2, 1).tobytes())
    block_off[n_blocks] = nbytes
    queue = b"".join(datas)
    smb = b"".join(sm_tiles)

    off = HEADER_BYTES
    sections = {}
    for name, payload in (("block", block_off.tobytes()), ("seg", seg.tobytes()), ("queue", queue),
                          ("sm", smb)):
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
               n_raw_groups=int(raw.sum()), total_bytes=total, crc32=0, max_segment_bytes=max_seg,
               palette=pal, code_len=code_len, R=R,
               off_block=sections["block"][0], off_seg=sections["seg"][0],
               off_queue=sections["queue"][0], size_queue=len(queue),
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
               max_segment_bytes=0, palette=[], code_len=[], R=0,
               off_block=0, off_seg=0, off_queue=0, size_queue=0, off_sm=0, size_sm=0,
               off_plain=off, size_plain=len(payload))
    body[:HEADER_BYTES] = _pack_header(h)
    return bytes(body)


def _section(blob: bytes, off: int, count: int, dtype) -> np.ndarray:
    return np.frombuffer(blob, dtype=dtype, count=count, offset=off)


def decode(blob: bytes) -> np.ndarray:
    """blob -> bf16 bit patterns [rows, cols] (uint16).

    Lane-lockstep over all blocks at once: every (block, lane) decoder holds
    its three-word window and advances one group per step; the loop runs over
    the group index j only.  A code is found by reading the next L window bits
    and matching them against each code's bit-reversed pattern of its own
    length.  At each refill check the lanes that shift take their next words
    from the current tile's segment in lane order.
    """
    h = parse_header(blob)
    rows, cols = h.rows, h.cols
    if h.flags & FLAG_PLAIN:
        return _section(blob, h.off_plain, rows * cols, "<u2").reshape(rows, cols).astype(np.uint16)
    n_groups = rows * cols // 64
    nb, G, R = h.n_blocks, h.G, h.R
    W, T = -(-G // 32), -(-G // 16)
    if R != check_groups(h.L):
        raise ValueError("refill interval does not match L")
    block_off = _section(blob, h.off_block, nb + 1, "<u4").astype(np.int64)
    seg = _section(blob, h.off_seg, nb * T, "<u2").astype(np.int64).reshape(nb, T)
    queue = np.frombuffer(blob, dtype=np.uint8, count=h.size_queue, offset=h.off_queue)
    qwords = np.concatenate([queue, np.zeros(4, np.uint8)])
    sm_all = _section(blob, h.off_sm, h.size_sm, np.uint8)

    def word_at(byte_off):  # little-endian u32 at byte offsets (array)
        b = qwords[byte_off[..., None] + np.arange(4)].astype(np.int64)
        return b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16) | (b[..., 3] << 24)

    codes = huffman.canonical_codes(h.code_len, h.palette)
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
    lanes = np.arange(64)
    blocks = np.arange(nb)
    gb = np.minimum(G, n_groups - blocks * G)  # groups per block
    base = block_off[:nb]  # byte offset of each block's data

    # tile 0 head of every block
    lane_n = word_at(base[:, None] + 2 * lanes[None, :]) & 0xFFFF  # two bytes read as part of a word
    raw_bits = word_at(base[:, None] + 128 + 4 * np.arange(W)[None, :])
    pos = base + 128 + 4 * W  # byte position of the next word to take / raw bytes
    w0 = np.zeros((nb, 64), dtype=np.int64)
    w1 = np.zeros((nb, 64), dtype=np.int64)
    w2 = np.zeros((nb, 64), dtype=np.int64)
    for i, wr in ((0, w1), (1, w2)):
        has = lane_n > i
        rank = np.cumsum(has, axis=1) - has
        got = word_at(pos[:, None] + 4 * rank)
        wr[has] = got[has]
        pos = pos + 4 * has.sum(axis=1)
    taken = np.minimum(lane_n, 2)
    qm = np.full((nb, 64), 30, dtype=np.int64)
    out_e = np.zeros((nb * G + 16, 64), dtype=np.uint8)
    mask_l = (1 << h.L) - 1
    rpos = pos  # raw exponent bytes of the current tile
    for j in range(G):
        live = j < gb
        t = j // 16
        if j % 16 == 0:
            # a tile's segment: (tile 0: the head read above) its raw groups'
            # exponent bytes, then the words its checks take
            if j > 0:
                rpos = np.where(live, base + 4 * seg[:, t - 1], pos)
            n_raw_t = np.zeros(nb, dtype=np.int64)
            for jj in range(j, min(j + 16, G)):
                n_raw_t += ((raw_bits[:, jj // 32] >> (jj % 32)) & 1) * (jj < gb)
            pos = rpos + 64 * n_raw_t
        gidx = blocks * G + j
        is_raw = ((raw_bits[:, j // 32] >> (j % 32)) & 1).astype(bool) & live
        coded = live & ~is_raw
        if is_raw.any():
            out_e[gidx[is_raw]] = qwords[rpos[is_raw][:, None] + lanes[None, :]]
            rpos = rpos + 64 * is_raw
        if coded.any():
            win = (w0 | (w1 << 32)) >> (qm + 2)
            idx = win & mask_l
            s = sym_of[idx]
            if (s[coded] < 0).any():
                raise ValueError("invalid code in stream")
            out_e[gidx[coded]] = pal[s[coded]]
            qm = np.where(coded[:, None], qm + len_of[idx], qm)
        if (j + 1) % R == 0:
            chk = live[:, None]
            if (qm[live] >= 64).any():
                raise ValueError("window overrun")
            shift = chk & (qm >= 32)
            need = shift & (taken < lane_n)
            rank = np.cumsum(need, axis=1) - need
            got = word_at(pos[:, None] + 4 * rank)
            qm = np.where(shift, qm - 32, qm)
            w0 = np.where(shift, w1, w0)
            w1 = np.where(shift, w2, w1)
            w2 = np.where(shift, np.where(need, got, 0), w2)
            taken = taken + need
            pos = pos + 4 * need.sum(axis=1)
        if (j % 16 == 15) or (j == G - 1):
            # every tile's segment ends exactly where its words end
            end_t = base + 4 * seg[:, t]
            fin = live & ((j == gb - 1) | (j % 16 == 15))
            if not np.array_equal(pos[fin], end_t[fin]):
                raise ValueError("segment length mismatch")
    if not np.array_equal(taken, lane_n):
        raise ValueError("lane word count mismatch")
    if not np.array_equal(base + 4 * seg[np.arange(nb), (gb - 1) // 16], block_off[1:]):
        raise ValueError("block length mismatch")
    e = out_e[:n_groups]
    # sm bytes: block b, group j, lane l at b*G*64 + (j>>4)*1024 + l*16 + (j&15)
    g = np.arange(n_groups)
    b, j = g // G, g % G
    sbase = b * G * 64 + (j >> 4) * 1024 + (j & 15)
    smg = sm_all[sbase[:, None] + lanes[None, :] * 16]
    return huffman.join_bf16(e, smg).reshape(rows, cols)


def decode_reference(blob: bytes) -> np.ndarray:
    """blob -> bf16 bit patterns [rows, cols] (uint16), one weight at a time.

    A second decoder of the same layout, written as plain loops over blocks,
    groups and lanes so that each step can be checked by eye against the
    layout description at the top of this module; only meant for small
    matrices.  For every block: read the head (lane word counts, raw bits,
    the first two words of every lane), then for each group j of the block,
    and for each lane, either copy the raw exponent byte or decode one code
    from the lane's window; after every R-th group run the refill check,
    lanes in order 0..63.
    """
    h = parse_header(blob)
    rows, cols = h.rows, h.cols
    if h.flags & FLAG_PLAIN:
        out = []
        for i in range(rows * cols):
            o = h.off_plain + 2 * i
            out.append(blob[o] | (blob[o + 1] << 8))
        return np.array(out, dtype=np.uint16).reshape(rows, cols)

    def u16(o):
        return blob[o] | (blob[o + 1] << 8)

    def u32(o):
        return blob[o] | (blob[o + 1] << 8) | (blob[o + 2] << 16) | (blob[o + 3] << 24)

    # canonical code table: bit-reversed pattern and length of each palette entry
    codes = huffman.canonical_codes(h.code_len, h.palette)
    table = [(huffman.reverse_bits(c, l), l, h.palette[s]) for s, (c, l) in enumerate(zip(codes, h.code_len)) if l]
    n_groups = rows * cols // 64
    G, R = h.G, h.R
    W = -(-G // 32)
    T = -(-G // 16)
    exps = [0] * (n_groups * 64)
    for b in range(h.n_blocks):
        g0 = b * G
        gb = min(G, n_groups - g0)
        start = h.off_queue + u32(h.off_block + 4 * b)  # this block's data
        n = [u16(start + 2 * l) for l in range(64)]
        raw = [(u32(start + 128 + 4 * (j // 32)) >> (j % 32)) & 1 for j in range(gb)]
        p = start + 128 + 4 * W
        # window of each lane: words (s-1, s, s+1) as one integer, qm, words taken
        win = [0] * 64
        for k in range(2):  # word 0 of the lanes that have one, then word 1
            for l in range(64):
                if n[l] > k:
                    win[l] |= u32(p) << (32 * (k + 1))
                    p += 4
        qm = [30] * 64
        taken = [min(nl, 2) for nl in n]
        raw_p = p
        for j in range(gb):
            if j % 16 == 0:
                if j > 0:  # the next tile's segment starts where the last one ended
                    seg_end = start + 4 * u16(h.off_seg + 2 * (b * T + j // 16 - 1))
                    if p != seg_end:
                        raise ValueError("segment length mismatch")
                raw_p = p
                p += 64 * sum(raw[jj] for jj in range(j, min(j + 16, gb)))
            for l in range(64):
                idx = g0 * 64 + j * 64 + l
                if raw[j]:
                    exps[idx] = blob[raw_p + l]
                    continue
                bits = win[l] >> (qm[l] + 2)
                for pat, ln, e in table:
                    if bits & ((1 << ln) - 1) == pat:
                        exps[idx] = e
                        qm[l] += ln
                        break
                else:
                    raise ValueError("invalid code in stream")
            if raw[j]:
                raw_p += 64
            if (j + 1) % R == 0:
                for l in range(64):
                    if qm[l] >= 64:
                        raise ValueError("window overrun")
                    if qm[l] >= 32:
                        qm[l] -= 32
                        win[l] >>= 32
                        if taken[l] < n[l]:
                            win[l] |= u32(p) << 64
                            p += 4
                            taken[l] += 1
        if p != start + 4 * u16(h.off_seg + 2 * (b * T + (gb - 1) // 16)):
            raise ValueError("segment length mismatch")
        if taken != n:
            raise ValueError("lane word count mismatch")
    out = np.zeros(n_groups * 64, dtype=np.uint16)
    for g in range(n_groups):
        b, j = divmod(g, G)
        for l in range(64):
            sm = blob[h.off_sm + b * G * 64 + (j >> 4) * 1024 + l * 16 + (j & 15)]
            e = exps[g * 64 + l]
            out[g * 64 + l] = ((sm & 0x80) << 8) | (e << 7) | (sm & 0x7F)
    return out.reshape(rows, cols)


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
