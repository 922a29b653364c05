"""Exponent statistics and the length-limited canonical Huffman code (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources: "Unweight: how we compressed an LLM 22% without sacrificing quality"
- paragraph on the anatomy of a BF16 value (1 sign, 8 exponent, 7 mantissa bits;
  sign and mantissa look random), paragraph on exponent redundancy (top-16
  exponents, ~2.6 bits), paragraph on Huffman coding of the exponent byte.
The length limit uses the package-merge algorithm (Larmore and Hirschberg,
"A fast algorithm for optimal length-limited Huffman codes", JACM 1990); the
canonical code assignment is the one of RFC 1951 section 3.2.2.
"""
from __future__ import annotations

import math

import numpy as np


def split_bf16(bits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """bf16 bit patterns -> (exponent byte, sign+mantissa byte).

    bf16 = s(1) e(8) m(7), MSB first.  The sign+mantissa byte is (s << 7) | m.
    """
    b = np.asarray(bits).astype(np.uint16)
    e = ((b >> 7) & 0xFF).astype(np.uint8)
    sm = (((b >> 8) & 0x80) | (b & 0x7F)).astype(np.uint8)
    return e, sm


def join_bf16(e: np.ndarray, sm: np.ndarray) -> np.ndarray:
    """Inverse of split_bf16: sign from bit 7 of sm, then exponent, then mantissa."""
    e = np.asarray(e).astype(np.uint16)
    sm = np.asarray(sm).astype(np.uint16)
    return (((sm & 0x80) << 8) | (e << 7) | (sm & 0x7F)).astype(np.uint16)


def histogram(exponents: np.ndarray) -> np.ndarray:
    """Count of each of the 256 exponent values."""
    return np.bincount(np.asarray(exponents, dtype=np.uint8).ravel(), minlength=256).astype(np.int64)


def palette(hist: np.ndarray, k: int) -> list[int]:
    """The k most frequent exponents with a non-zero count, by count descending
    then exponent ascending."""
    present = [s for s in range(256) if hist[s] > 0]
    present.sort(key=lambda s: (-int(hist[s]), s))
    return present[:k]


def entropy_bits(counts) -> float:
    c = np.asarray([x for x in counts if x > 0], dtype=np.float64)
    if c.size == 0:
        return 0.0
    p = c / c.sum()
    return float(-(p * np.log2(p)).sum())


def package_merge(counts: list[int], max_len: int, keys: list[int] | None = None) -> list[int]:
    """Optimal code lengths <= max_len for the given positive counts.

    Coin-collector formulation: every symbol owns one coin of each width
    2^-1 .. 2^-max_len whose value is its count; the cheapest set of coins of
    total width n-1 gives the lengths (a symbol's length is the number of its
    coins taken).  The list of the narrowest width is the leaves; each step
    pairs neighbours of the current list into packages of the next width and
    merges them with a fresh copy of the leaves.  Ordering: leaves by
    (count, key) where key defaults to the symbol index (the blob encoder
    passes the exponent value); in a merge an item of smaller weight goes first and
    on equal weight a leaf goes before a package; packages keep the order in
    which they were formed.  The first 2n-2 items of the widest list are taken.

    One symbol gets length 1 (Kraft sum 1/2); no symbols give [].
    """
    n = len(counts)
    if n == 0:
        return []
    if any(c <= 0 for c in counts):
        raise ValueError("counts must be positive")
    if n == 1:
        return [1]
    if n > (1 << max_len):
        raise ValueError("too many symbols for the length limit")
    if keys is None:
        keys = list(range(n))
    leaves = sorted(((int(c), [i]) for i, c in enumerate(counts)), key=lambda t: (t[0], keys[t[1][0]]))
    current = list(leaves)
    for _ in range(max_len - 1):
        packages = []
        for a in range(0, len(current) - 1, 2):
            packages.append((current[a][0] + current[a + 1][0], current[a][1] + current[a + 1][1]))
        merged = []
        i = j = 0
        while i < len(leaves) or j < len(packages):
            if j >= len(packages) or (i < len(leaves) and leaves[i][0] <= packages[j][0]):
                merged.append(leaves[i])
                i += 1
            else:
                merged.append(packages[j])
                j += 1
        current = merged
    lengths = [0] * n
    for _, members in current[: 2 * n - 2]:
        for s in members:
            lengths[s] += 1
    return lengths


def canonical_codes(lengths: list[int], keys: list[int]) -> list[int]:
    """RFC 1951 3.2.2 canonical codes (MSB-first integers) for the given lengths.

    Symbols of equal length get consecutive codes in increasing order of their
    key (here: the exponent value).  Length 0 means "no code" (returns -1).
    """
    max_len = max(lengths) if lengths else 0
    bl_count = [0] * (max_len + 1)
    for l in lengths:
        if l:
            bl_count[l] += 1
    next_code = [0] * (max_len + 2)
    code = 0
    for bits in range(1, max_len + 1):
        code = (code + bl_count[bits - 1]) << 1
        next_code[bits] = code
    out = [-1] * len(lengths)
    for idx in sorted(range(len(lengths)), key=lambda i: keys[i]):
        l = lengths[idx]
        if l:
            out[idx] = next_code[l]
            next_code[l] += 1
    return out


def kraft_sum(lengths: list[int]) -> float:
    return math.fsum(2.0 ** -l for l in lengths if l)


def reverse_bits(value: int, width: int) -> int:
    r = 0
    for _ in range(width):
        r = (r << 1) | (value & 1)
        value >>= 1
    return r
