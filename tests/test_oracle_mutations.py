"""Each test plants one plausible mistake in the oracle (on the CPU, through
monkeypatch) and checks that at least one pin catches it.  A pin that lets a
planted mistake through is too weak to trust the oracle with."""
import json
import os

import numpy as np
import pytest

from oracle import blob, huffman, products
import tests.test_oracle_blob as tb
import tests.test_oracle_huffman as th
import tests.test_oracle_products as tp


def _fails(fn, *args):
    try:
        fn(*args)
    except (AssertionError, ValueError, IndexError):
        return True
    return False


def test_bit_order_mistake_is_caught(monkeypatch, golden_dir):
    monkeypatch.setattr(huffman, "reverse_bits", lambda v, w: v)  # MSB-first packing
    assert _fails(tb.test_hand_fixture_1x64, golden_dir)


def test_canonical_tie_order_mistake_is_caught(monkeypatch, golden_dir):
    real = huffman.canonical_codes
    monkeypatch.setattr(huffman, "canonical_codes", lambda lens, keys: real(lens, [-k for k in keys]))
    assert _fails(th.test_rfc1951_printed_example, golden_dir)


def test_dropped_raw_escape_is_caught(monkeypatch, golden_dir):
    real_isin = np.isin
    monkeypatch.setattr(blob.np, "isin", lambda a, b: np.ones(np.shape(a), dtype=bool))
    assert _fails(tb.test_hand_fixture_raw_group, golden_dir)
    monkeypatch.setattr(blob.np, "isin", real_isin)


def test_sign_bit_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(huffman, "join_bf16",
                        lambda e, sm: (((np.asarray(sm).astype(np.uint16) & 0x80) << 7)
                                       | (np.asarray(e).astype(np.uint16) << 7)
                                       | (np.asarray(sm).astype(np.uint16) & 0x7F)).astype(np.uint16))
    assert _fails(th.test_split_join_all_patterns)


def test_double_rounding_mistake_is_caught(monkeypatch):
    real = products.round_to_bf16
    monkeypatch.setattr(products, "round_to_bf16",
                        lambda v: real(np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)))
    assert _fails(tp.test_round_to_bf16_by_hand)


def test_transposed_operand_is_caught(monkeypatch):
    monkeypatch.setattr(products, "gemm_f64",
                        lambda w, x: np.asarray(x, dtype=np.float64) @ products.bf16_to_f64(w))
    assert _fails(tp.test_one_hot_selects_a_column_exactly)


def test_short_length_limit_is_caught(monkeypatch):
    real = huffman.package_merge
    monkeypatch.setattr(huffman, "package_merge", lambda c, L, keys=None: real(c, max(1, L - 1), keys)
                        if len(c) <= (1 << max(1, L - 1)) else real(c, L, keys))
    assert _fails(th.test_package_merge_optimal_by_brute_force)
