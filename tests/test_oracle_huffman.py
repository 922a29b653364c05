"""Pins of the oracle's code construction against facts that do not come from it:
closed forms, the RFC 1951 printed example, brute force over every length
vector, Kraft's equality and Shannon's bound."""
import itertools
import json
import math
import os
import random

import numpy as np
import pytest

from oracle import huffman


def test_split_fields_by_hand():
    # 1.0 = 0x3F80: s=0 e=127 m=0 ; -1.5 = 0xBFC0: s=1 e=127 m=0x40 ; 0x0001: smallest subnormal
    e, sm = huffman.split_bf16(np.array([0x3F80, 0xBFC0, 0x0001, 0xFF80, 0x7FC1], dtype=np.uint16))
    assert list(e) == [127, 127, 0, 255, 255]
    assert list(sm) == [0x00, 0xC0, 0x01, 0x80, 0x41]


def test_split_join_all_patterns():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    e, sm = huffman.split_bf16(b)
    assert np.array_equal(huffman.join_bf16(e, sm), b)
    # sign and mantissa never touch the exponent byte and vice versa
    assert np.array_equal(e, (b >> 7) & 0xFF)


def test_palette_order():
    h = np.zeros(256, dtype=np.int64)
    h[[5, 9, 3, 200]] = [10, 10, 30, 1]
    assert huffman.palette(h, 16) == [3, 5, 9, 200]
    assert huffman.palette(h, 2) == [3, 5]


@pytest.mark.parametrize("counts,lengths", [
    ([8, 4, 2, 2], [1, 2, 3, 3]),
    ([1] * 16, [4] * 16),
    ([5, 7], [1, 1]),
    ([100], [1]),
    ([1, 1, 1, 1, 1, 1, 1, 1], [3] * 8),
])
def test_package_merge_closed_forms(counts, lengths):
    assert huffman.package_merge(counts, 12) == lengths


def test_package_merge_limit_binds():
    # Fibonacci-like counts want a deep tree; the limit forces a flatter one.
    counts = [1, 1, 2, 3, 5, 8, 13, 21]
    free = huffman.package_merge(counts, 12)
    assert max(free) == 7
    lim = huffman.package_merge(counts, 4)
    assert max(lim) <= 4 and huffman.kraft_sum(lim) == 1.0


def _brute_min_cost(counts, L):
    best = None
    for lens in itertools.product(range(1, L + 1), repeat=len(counts)):
        if sum(2.0 ** -l for l in lens) <= 1.0:
            c = sum(a * b for a, b in zip(counts, lens))
            best = c if best is None else min(best, c)
    return best


def test_package_merge_optimal_by_brute_force():
    rng = random.Random(7)
    for _ in range(150):
        n = rng.randint(2, 6)
        L = rng.randint(max(1, math.ceil(math.log2(n))), 6)
        counts = [rng.choice([1, 2, 3, 5, 8, 40, 100, 1000]) for _ in range(n)]
        lens = huffman.package_merge(counts, L)
        assert max(lens) <= L
        assert sum(a * b for a, b in zip(counts, lens)) == _brute_min_cost(counts, L)


def test_kraft_equality_and_entropy_bound():
    rng = np.random.default_rng(3)
    for _ in range(60):
        n = int(rng.integers(2, 33))
        counts = [int(c) for c in rng.integers(1, 10_000, size=n)]
        lens = huffman.package_merge(counts, 32)
        assert huffman.kraft_sum(lens) == 1.0
        H = huffman.entropy_bits(counts)
        mean = sum(a * b for a, b in zip(counts, lens)) / sum(counts)
        assert H - 1e-12 <= mean < H + 1


def test_rfc1951_printed_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "rfc1951_canonical_example.json")))
    keys = list(range(len(g["lengths"])))
    codes = huffman.canonical_codes(g["lengths"], keys)
    got = [format(c, "0%db" % l) for c, l in zip(codes, g["lengths"])]
    assert got == g["codes"]


def test_canonical_codes_prefix_free():
    rng = np.random.default_rng(11)
    for _ in range(40):
        n = int(rng.integers(2, 33))
        counts = [int(c) for c in rng.integers(1, 5000, size=n)]
        lens = huffman.package_merge(counts, 8 if n <= 256 else 12)
        keys = list(rng.permutation(256)[:n])
        codes = huffman.canonical_codes(lens, keys)
        strs = [format(c, "0%db" % l) for c, l in zip(codes, lens)]
        for a, b in itertools.permutations(strs, 2):
            assert not b.startswith(a)
        # same length: codes increase with the key
        for l in set(lens):
            idx = sorted([i for i in range(n) if lens[i] == l], key=lambda i: keys[i])
            cs = [codes[i] for i in idx]
            assert cs == sorted(cs) and len(set(cs)) == len(cs)


def test_reverse_bits():
    assert huffman.reverse_bits(0b110, 3) == 0b011
    assert huffman.reverse_bits(0b1, 1) == 0b1
    assert huffman.reverse_bits(0b10, 2) == 0b01
    assert huffman.reverse_bits(0b100000, 6) == 0b000001
