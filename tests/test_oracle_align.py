"""Pins of the oracle's expert-sorted tile layout of the (token, slot) pairs.

The pages' layer is an indexed MoE: every token carries top-k expert indices
(PR "Incubate DeepSeek V4 WNA16 runtime on SM86", "What this branch adds"
item 3).  Running it as per-expert GEMMs needs the pairs grouped by expert in
tiles of block_m rows; the contract (stable order, padding value P, offsets
rounded up to block_m) is this project's reading and is pinned here against
Python's stable sort.
"""
import numpy as np
import pytest

from oracle import oracle as O


def check_against_sorted(ids, E, bm):
    ids = np.asarray(ids, np.int32)
    T, k = ids.shape
    P = T * k
    flat = ids.reshape(-1)
    r = O.align(ids, E, bm)
    valid = [p for p in range(P) if 0 <= flat[p] < E]
    order = sorted(valid, key=lambda p: (int(flat[p]), p))        # textbook stable sort
    # strip padding: the real slots in slot order are exactly the stable order
    real = [int(s) for s in r["sorted_ids"] if s != P]
    assert real == order
    counts = np.bincount(flat[(flat >= 0) & (flat < E)], minlength=E)
    padded = (counts + bm - 1) // bm * bm
    assert np.array_equal(r["expert_offsets"], np.concatenate([[0], np.cumsum(padded)]))
    assert r["num_tiles"] * bm == r["expert_offsets"][-1]
    assert np.all(r["expert_offsets"] % bm == 0)
    assert int(np.sum(r["sorted_ids"] == P)) == int(np.sum(padded - counts))
    for e in range(E):
        lo, hi = r["expert_offsets"][e], r["expert_offsets"][e + 1]
        seg = r["sorted_ids"][lo:hi]
        assert np.all(seg[: counts[e]] != P) and np.all(seg[counts[e]:] == P)
        assert np.all(r["tile_expert"][lo // bm: hi // bm] == e)
        assert np.all(flat[seg[: counts[e]]] == e)
    for p in range(P):
        if 0 <= flat[p] < E:
            assert r["sorted_ids"][r["inv_perm"][p]] == p
        else:
            assert r["inv_perm"][p] == -1
    assert r["bad_ids"] == P - len(valid)
    return r


@pytest.mark.parametrize("bm", [1, 16, 64])
@pytest.mark.parametrize("seed", range(4))
def test_random_routing(bm, seed):
    rng = np.random.default_rng(seed)
    T, k, E = int(rng.integers(1, 60)), int(rng.integers(1, 7)), int(rng.integers(1, 40))
    check_against_sorted(rng.integers(0, E, size=(T, k)), E, bm)


def test_empty_experts_and_single_hot_expert():
    ids = np.full((33, 2), 5, np.int32)
    r = check_against_sorted(ids, 9, 16)
    assert r["num_tiles"] == 5 and list(r["tile_expert"]) == [5] * 5


def test_exact_multiples_and_off_by_one():
    for n in (15, 16, 17, 32):
        ids = np.zeros((n, 1), np.int32)
        r = check_against_sorted(ids, 2, 16)
        assert r["num_tiles"] == (n + 15) // 16


def test_out_of_range_ids_skipped_and_counted():
    ids = np.array([[0, -1], [7, 2], [2, 3]], np.int32)
    r = check_against_sorted(ids, 4, 4)
    assert r["bad_ids"] == 2


def test_no_pairs():
    r = O.align(np.zeros((0, 4), np.int32), 8, 16)
    assert r["num_tiles"] == 0 and np.all(r["expert_offsets"] == 0)


def test_known_small_layout():
    """Hand-worked: ids [[1,0],[1,1]], block 2 -> expert 0 gets pair 1 plus one
    pad; expert 1 gets pairs 0, 2, 3 plus one pad."""
    r = O.align(np.array([[1, 0], [1, 1]], np.int32), 2, 2)
    assert list(r["sorted_ids"]) == [1, 4, 0, 2, 3, 4]
    assert list(r["expert_offsets"]) == [0, 2, 6]
    assert list(r["tile_expert"]) == [0, 1, 1]
    assert list(r["inv_perm"]) == [2, 0, 3, 4]
