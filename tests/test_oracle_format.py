"""Pins of the oracle's number formats: FP16 / BF16 decoding, code fields,
dequantization and the quantized matrix-vector product.

The weight format is the pages' symmetric b-bit, INT32-packed, FP16-group-scale
WNA16 layout (model card "hampsonw/DeepSeek-V4-Flash-0731-WNA16", "What
changed"); field order and sign encoding follow the readings stated in
tests/golden/packed_words.txt.
"""
import os

import numpy as np
import pytest

from oracle import oracle as O
from tests import _brute as B

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "packed_words.txt")


def _golden_words():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            rows.append((int(parts[0]), int(parts[1], 16), [int(v) for v in parts[2:]]))
    return rows


def test_f16_decode_every_pattern():
    """All 65536 binary16 patterns against numpy's own float16 widening."""
    lib = O._load()
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([lib.oracle_f16_to_f64(int(p)) for p in pats])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zero and the extremes
    assert np.signbit(got[0x8000]) and got[0x7BFF] == 65504.0 and got[0x0001] == 2.0**-24


def test_bf16_decode_every_pattern():
    """All 65536 bfloat16 patterns against float32 with the low half zero."""
    lib = O._load()
    pats = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        ref = (pats << 16).view(np.float32).astype(np.float64)
    got = np.array([lib.oracle_bf16_to_f64(int(p)) for p in pats])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


@pytest.mark.parametrize("bits,word,codes", _golden_words())
def test_code_fields_hand_built(bits, word, codes):
    w = np.array([word], np.uint32)
    assert list(O.codes(w, 32 // bits, bits)) == codes
    assert list(B.unpack(w, 32 // bits, bits)) == codes


@pytest.mark.parametrize("bits", [2, 4])
def test_code_index_crosses_words(bits):
    """K index j*(32/b)+i reads field i of word j (not word i of field j)."""
    per = 32 // bits
    words = np.zeros(3, np.uint32)
    top = (1 << bits) - 1
    words[1] = np.uint32(top << (bits * 2))            # field 2 of word 1
    q = O.codes(words, 3 * per, bits)
    lo = -(1 << (bits - 1))
    expect = np.full(3 * per, lo)
    expect[per + 2] = (1 << (bits - 1)) - 1
    assert np.array_equal(q, expect)


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_unpack_round_trip(bits):
    rng = np.random.default_rng(7 + bits)
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1))
    q = rng.integers(lo, hi, size=(3, 64))
    words = B.pack(q, bits)
    for r in range(3):
        assert np.array_equal(O.codes(words[r], 64, bits), q[r])
    # and the other way: random words are a bijection of code vectors
    w = rng.integers(0, 2**32, size=(2, 4), dtype=np.uint32)
    K = 4 * (32 // bits)
    back = B.pack(np.stack([O.codes(w[r], K, bits) for r in range(2)]), bits)
    assert np.array_equal(back, w)


def test_weight_is_code_times_group_scale():
    """W[n][k] = q * s[n][k // g], exact in double, on a non-square matrix so
    that swapping the N and K roles of the scale index fails."""
    rng = np.random.default_rng(3)
    rows, K, bits, g = 6, 96, 4, 32
    words = rng.integers(0, 2**32, size=(rows, K * bits // 32), dtype=np.uint32)
    scales = rng.uniform(0.5, 2.0, size=(rows, K // g)).astype(np.float16)
    q = B.unpack(words, K, bits)
    for n in range(rows):
        for k in range(0, K, 7):
            s = float(scales[n, k // g])
            assert O.weight(words, scales, K, bits, g, n, k) == q[n, k] * s


@pytest.mark.parametrize("bits,group", [(2, 32), (2, 64), (4, 32), (4, 64), (4, 128)])
def test_qmatvec_one_hot_reads_one_column(bits, group):
    """x = e_c picks column c of the dequantized matrix: code times the scale of
    group c // g of that row.  K != rows, and every group scale differs."""
    rng = np.random.default_rng(bits * 1000 + group)
    rows, K = 40, 256
    words = rng.integers(0, 2**32, size=(rows, K * bits // 32), dtype=np.uint32)
    scales = (np.arange(rows * (K // group)).reshape(rows, K // group) / 64.0 + 0.25).astype(np.float16)
    q = B.unpack(words, K, bits)
    for c in [0, 1, group - 1, group, K - 1]:
        v = np.zeros(K)
        v[c] = 1.0
        y = O.qmatvec(words, scales, rows, K, bits, group, v)
        expect = q[:, c] * scales[:, c // group].astype(np.float64)
        assert np.array_equal(y, expect)


@pytest.mark.parametrize("bits", [2, 4])
def test_qmatvec_integer_exact(bits):
    """All scales 1 and integer activations: the product is integer arithmetic,
    so the oracle must equal Python's exact integer dot products."""
    rng = np.random.default_rng(11)
    rows, K, g = 24, 128, 64
    words = rng.integers(0, 2**32, size=(rows, K * bits // 32), dtype=np.uint32)
    scales = np.ones((rows, K // g), np.float16)
    xi = rng.integers(-50, 51, size=K)
    q = B.unpack(words, K, bits)
    y = O.qmatvec(words, scales, rows, K, bits, g, xi.astype(np.float64))
    exact = [sum(int(a) * int(b) for a, b in zip(q[n], xi)) for n in range(rows)]
    assert [int(v) for v in y] == exact and np.all(y == np.round(y))
