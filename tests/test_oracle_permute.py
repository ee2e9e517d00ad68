"""Pins of the oracle's expert permutation: Python ``sorted`` of (expert,
flat index) pairs and the invariants the padded layout must satisfy."""

import numpy as np
import pytest

import oracle as O


def _check(ids, E, n_sh, B):
    T, k = ids.shape
    p = O.permute_align(ids, E, n_sh, B)
    A = T * (k + n_sh)
    Ep = E + n_sh
    pairs = [(int(ids[t, j]), t * k + j) for t in range(T) for j in range(k)]
    pairs += [(E, T * k + t) for t in range(T)] if n_sh else []
    pairs.sort()
    # segment contents: flat indices of each expert in ascending order
    counts = [sum(1 for e, _ in pairs if e == x) for x in range(Ep)]
    assert list(p["counts"]) == counts
    offs = p["offsets"]
    assert offs[0] == 0
    for e in range(Ep):
        seg = p["sorted_ids"][offs[e]:offs[e + 1]]
        expect = [f for x, f in pairs if x == e]
        pad = -(-counts[e] // B) * B
        assert offs[e + 1] - offs[e] == pad
        assert list(seg[:counts[e]]) == expect
        assert np.all(seg[counts[e]:] == A)
        assert np.all(p["block_expert"][offs[e] // B: offs[e + 1] // B] == e)
    total = int(offs[-1])
    assert total <= p["max_rows"] == O.permute_max_rows(T, k, E, n_sh, B)
    assert np.all(p["sorted_ids"][total:] == A)
    assert np.all(p["block_expert"][total // B:] == -1)
    # inverse map and exactly-once
    srt = p["sorted_ids"]
    assert sorted(srt[srt < A].tolist()) == list(range(A))
    assert np.array_equal(srt[p["inv_perm"]], np.arange(A))
    assert int(np.sum(srt == A)) == p["max_rows"] - A
    return p


@pytest.mark.parametrize("seed,T,E,k,n_sh,B", [
    (0, 13, 8, 2, 0, 4), (1, 64, 8, 2, 0, 16), (2, 50, 16, 3, 1, 8),
    (3, 32, 128, 8, 0, 16), (4, 7, 5, 5, 1, 1), (5, 100, 64, 10, 1, 32)])
def test_permute_vs_sorted(seed, T, E, k, n_sh, B):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _check(ids, E, n_sh, B)


def test_permute_all_one_expert_and_empty_experts():
    T, E, k = 40, 8, 1
    ids = np.full((T, k), 5, np.int32)
    p = _check(ids, E, 0, 16)
    assert list(p["counts"]) == [0, 0, 0, 0, 0, 40, 0, 0]


def test_permute_empty_input():
    p = O.permute_align(np.zeros((0, 4), np.int32), 8, 1, 16)
    assert p["max_rows"] == 0 and np.all(p["offsets"] == 0) and len(p["inv_perm"]) == 0


def test_max_rows_bound_is_tight():
    # every expert gets exactly one row: each segment pads to a full block
    T, E, k, B = 16, 32, 2, 8
    ids = np.arange(T * k, dtype=np.int32).reshape(T, k) % E
    p = O.permute_align(ids, E, 0, B)
    assert p["offsets"][-1] == E * B == p["max_rows"]
    # block count can never exceed the row count
    assert O.permute_max_rows(2, 1, 64, 0, 16) == 2 * 16


@pytest.mark.parametrize("n_sh", [0, 1])
def test_permute_picks_outside_the_experts_get_no_row(n_sh):
    """Reading: a routed pick outside [0, E) gets no row.  Pinned against the
    sorted-pairs construction over the valid picks only, by brute force."""
    rng = np.random.default_rng(9)
    T, E, k, B = 30, 12, 3, 4
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    bad = [(2, 0, -1), (5, 2, E), (11, 1, E + 7), (29, 0, -40)]
    for t, j, v in bad:
        ids[t, j] = v
    p = O.permute_align(ids, E, n_sh, B)
    A = T * (k + n_sh)
    Ep = E + n_sh
    pairs = [(int(ids[t, j]), t * k + j) for t in range(T) for j in range(k) if 0 <= ids[t, j] < E]
    pairs += [(E, T * k + t) for t in range(T)] if n_sh else []
    pairs.sort()
    assert list(p["counts"]) == [sum(1 for e, _ in pairs if e == x) for x in range(Ep)]
    offs = p["offsets"]
    for e in range(Ep):
        c = int(p["counts"][e])
        seg = p["sorted_ids"][offs[e]:offs[e + 1]]
        assert offs[e + 1] - offs[e] == -(-c // B) * B
        assert list(seg[:c]) == [f for x, f in pairs if x == e]
        assert np.all(seg[c:] == A)
    inv = p["inv_perm"]
    for t, j, _ in bad:
        assert inv[t * k + j] == -1
    valid = [f for _, f in pairs]
    assert sorted(int(v) for v in p["sorted_ids"] if v < A) == sorted(valid)
    assert np.array_equal(p["sorted_ids"][inv[valid]], np.array(valid))
    assert int(np.sum(inv == -1)) == len(bad)
