"""Pins of the oracle's packed codes and of the W4A16 product that consumes them.

The packed format is the codes of a row as one little-endian bit stream in
32-bit words (the pages print no storage format; this is the plainest dense
one).  The product is Y = X' W_hat^T with 16-bit activations and the exactly
dequantized 4-bit weights (page "量化经典：LLM.int8 / GPTQ / AWQ", GPTQ
section: weight-only 4-bit, activations stay 16-bit; page "LLM 量化方法原理与
实现详解", §2.2 dequantization).
"""
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pack_examples.txt")


def _golden():
    for line in open(GOLDEN, encoding="utf-8"):
        if line.startswith("#") or not line.strip():
            continue
        b, c, w = (f.strip() for f in line.split("|"))
        yield int(b), np.array([[int(v) for v in c.split()]], dtype=np.uint8), [int(v, 16) for v in w.split()]


def test_pack_worked_examples(oracle_mod):
    n = 0
    for bits, codes, words in _golden():
        got = oracle_mod.pack_codes(codes, bits)
        assert got.dtype == np.uint32 and got.shape == (1, len(words))
        assert [int(v) for v in got[0]] == words, (bits, codes)
        n += 1
    assert n == 5


def _bigint_words(row, bits):
    """The same definition by integer arithmetic: sum of code_k << (bits k), cut into 32-bit words."""
    v = 0
    for k, c in enumerate(row):
        v |= int(c) << (bits * k)
    nw = (len(row) * bits + 31) // 32
    return [(v >> (32 * w)) & 0xFFFFFFFF for w in range(nw)]


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_pack_equals_integer_definition(oracle_mod, bits):
    rng = np.random.default_rng(bits)
    for d in (1, 7, 32, 45, 130):
        codes = rng.integers(0, 2 ** bits, size=(3, d), dtype=np.uint8)
        got = oracle_mod.pack_codes(codes, bits)
        for r in range(3):
            assert [int(v) for v in got[r]] == _bigint_words(codes[r], bits)
        assert np.array_equal(oracle_mod.unpack_codes(got, bits, d), codes)


def test_pack_with_order_and_width_checks(oracle_mod):
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 16, size=(4, 64), dtype=np.uint8)
    perm = rng.permutation(64)
    assert np.array_equal(oracle_mod.pack_codes(codes, 4, perm), oracle_mod.pack_codes(codes[:, perm], 4))
    # 8-bit codes are the bytes themselves, read as little-endian words
    c8 = rng.integers(0, 256, size=(2, 12), dtype=np.uint8)
    assert np.array_equal(oracle_mod.pack_codes(c8, 8), c8.view("<u4"))
    with pytest.raises(ValueError):
        oracle_mod.pack_codes(np.array([[16]], dtype=np.uint8), 4)


def _grid_layer(rng, d_out, d_in, group):
    g = group if group > 0 else d_in
    ng = d_in // g
    codes = rng.integers(0, 16, size=(d_out, d_in), dtype=np.uint8)
    scales = rng.uniform(1e-3, 2e-2, size=(d_out, ng)).astype(np.float32)
    zeros = rng.integers(0, 16, size=(d_out, ng)).astype(np.float32)
    return codes, scales, zeros


@pytest.mark.parametrize("group", [32, 0])
def test_identity_activations_give_the_dequantized_weights(oracle_mod, group):
    """X = I: Y = W_hat^T, the pinned dequantization of the stored codes (fp32 stored format, so
    equal within one fp32 rounding of each weight)."""
    rng = np.random.default_rng(2)
    d_out, d_in = 24, 64
    codes, scales, zeros = _grid_layer(rng, d_out, d_in, group)
    Y = oracle_mod.w4a16_matmul(np.eye(d_in), oracle_mod.pack_codes(codes, 4), scales, zeros, group)
    What = oracle_mod.dequant(codes, scales, zeros, group)
    assert Y.shape == (d_in, d_out)
    assert np.allclose(Y, What.T, rtol=2 ** -23, atol=0)


def test_act_order_packing_meets_the_column_order(oracle_mod):
    """Dynamic grids under act-order: groups run in processing order and g_idx scatters them over the
    original columns.  Packing the codes in processing order (perm) and gathering X's columns by the
    same perm gives X W_hat^T with W_hat the dequantization through g_idx."""
    rng = np.random.default_rng(3)
    d_out, d_in, group = 16, 96, 32
    perm = rng.permutation(d_in).astype(np.int32)
    codes, scales, zeros = _grid_layer(rng, d_out, d_in, group)  # scales in processing order
    g_idx = np.empty(d_in, dtype=np.int32)
    g_idx[perm] = np.arange(d_in) // group
    packed = oracle_mod.pack_codes(codes, 4, perm)
    What = oracle_mod.dequant(codes, scales, zeros, group, g_idx)
    Y = oracle_mod.w4a16_matmul(np.eye(d_in), packed, scales, zeros, group, kperm=perm)
    assert np.allclose(Y, What.T, rtol=2 ** -23, atol=0)
    X = rng.standard_normal((5, d_in)).astype(np.float16)
    Y = oracle_mod.w4a16_matmul(X, packed, scales, zeros, group, kperm=perm)
    ref = X.astype(np.float64) @ What.T  # What holds fp32-rounded weights: one rounding each
    assert np.abs(Y - ref).max() <= 2 ** -23 * (np.abs(X.astype(np.float64)) @ np.abs(What).T).max()
    # without the gather the columns meet the wrong weights
    Yw = oracle_mod.w4a16_matmul(X, packed, scales, zeros, group)
    assert not np.allclose(Yw, Y, rtol=1e-3)
