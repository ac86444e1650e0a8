"""Pins of the oracle's prepared code order (oracle_prepare; the layout is the
library's own, stated in include/moe_wna16.h).

Checked without re-typing its index arithmetic: every block is a permutation
of its 16 rows' words; decoding a slot's words with the already-pinned field
decoder gives exactly the codes of the K offsets the layout assigns to that
lane group; and a few slots worked out by hand from the layout's statement.
"""
import numpy as np
import pytest

from oracle import oracle as O

FORMATS = [(2, 32), (2, 64), (2, 128), (4, 32), (4, 64), (4, 128)]


def words(E, rows, K, bits, seed=0):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 2 ** 32, size=(E, rows, K * bits // 32), dtype=np.uint32)


@pytest.mark.parametrize("bits,group", FORMATS)
def test_every_block_is_a_permutation_of_its_rows_words(bits, group):
    E, rows, K = 2, 48, 1024
    w = np.arange(E * rows * K * bits // 32, dtype=np.uint32).reshape(E, rows, -1)
    p = O.prepare(w, bits, group)
    unit = 512 // bits
    nunits = K // unit
    blocks = p.reshape(E, rows // 16, nunits, 256)
    for e in range(E):
        for rb in range(rows // 16):
            for u in range(nunits):
                src = w[e, rb * 16:(rb + 1) * 16, u * 16:(u + 1) * 16].ravel()
                assert np.array_equal(np.sort(blocks[e, rb, u]), np.sort(src))


@pytest.mark.parametrize("bits,group", FORMATS)
def test_slots_decode_to_their_lane_groups_codes(bits, group):
    """A slot's words, group by group, decode to the codes at in-group K
    offsets [g*group/4, (g+1)*group/4) of its row (16h..16h+16 for 2-bit
    group 32, two lane groups per slot)."""
    E, rows, K = 1, 32, 512
    w = words(E, rows, K, bits, seed=bits + group)
    p = O.prepare(w, bits, group).reshape(E, rows // 16, -1, 256)
    unit = 512 // bits
    gpu = unit // group
    per_word = 32 // bits
    for rb in range(rows // 16):
        for r in range(16):
            codes_row = O.codes(w[0, rb * 16 + r], K, bits)
            for u in range(K // unit):
                blk = p[0, rb, u]
                if bits == 2 and group == 32:
                    for h in range(2):
                        slot = blk[(h * 16 + r) * 8:(h * 16 + r) * 8 + 8]
                        for gq in range(8):
                            got = O.codes(slot[gq:gq + 1], 16, 2)
                            k0 = u * unit + gq * 32 + 16 * h
                            assert np.array_equal(got, codes_row[k0:k0 + 16])
                    continue
                n = group // 4 // per_word          # words per lane group and group
                for g in range(4):
                    slot = blk[(g * 16 + r) * 4:(g * 16 + r) * 4 + 4]
                    for gq in range(gpu):
                        got = O.codes(slot[gq * n:(gq + 1) * n], n * per_word, bits)
                        k0 = u * unit + gq * group + g * group // 4
                        assert np.array_equal(got, codes_row[k0:k0 + group // 4])


def test_hand_worked_slots():
    """Row r's words numbered 100 r + w (one load unit per row)."""
    def numbered(bits):
        K = 512 // bits
        w = np.zeros((1, 16, 16), np.uint32)
        for r in range(16):
            w[0, r] = 100 * r + np.arange(16)
        return w, K

    # 4-bit, group 64: 2 groups of 8 words; lane group g owns 16 codes = words
    # 2g, 2g+1 of each group -> slot (g, r) = w(2g), w(2g+1), w(8+2g), w(9+2g)
    w, _ = numbered(4)
    p = O.prepare(w, 4, 64).reshape(256)
    assert list(p[(1 * 16 + 3) * 4:(1 * 16 + 3) * 4 + 4]) == [302, 303, 310, 311]
    # 4-bit, group 128: one group; lane group g owns words 4g..4g+3
    p = O.prepare(w, 4, 128).reshape(256)
    assert list(p[(3 * 16 + 0) * 4:(3 * 16 + 0) * 4 + 4]) == [12, 13, 14, 15]
    # 4-bit, group 32: 4 groups of 4 words; lane group g owns word g of each
    p = O.prepare(w, 4, 32).reshape(256)
    assert list(p[(2 * 16 + 5) * 4:(2 * 16 + 5) * 4 + 4]) == [502, 506, 510, 514]
    # 2-bit, group 64: 4 groups of 4 words; lane group g owns word g of each
    w, _ = numbered(2)
    p = O.prepare(w, 2, 64).reshape(256)
    assert list(p[(2 * 16 + 0) * 4:(2 * 16 + 0) * 4 + 4]) == [2, 6, 10, 14]
    # 2-bit, group 128: 2 groups of 8 words; lane group g owns words 2g, 2g+1
    p = O.prepare(w, 2, 128).reshape(256)
    assert list(p[(0 * 16 + 7) * 4:(0 * 16 + 7) * 4 + 4]) == [700, 701, 708, 709]
    # 2-bit, group 32: 8 groups of 2 words; half h = word h of each group
    p = O.prepare(w, 2, 32).reshape(256)
    assert list(p[(1 * 16 + 2) * 8:(1 * 16 + 2) * 8 + 8]) == [201 + 2 * i for i in range(8)]
    assert list(p[(0 * 16 + 2) * 8:(0 * 16 + 2) * 8 + 8]) == [200 + 2 * i for i in range(8)]


def test_rejects_partial_blocks():
    with pytest.raises(ValueError):
        O.prepare(words(1, 24, 256, 4), 4, 128)        # rows not a multiple of 16
    with pytest.raises(ValueError):
        O.prepare(words(1, 16, 384, 2), 2, 128)        # K not a multiple of 256 (2-bit unit)
