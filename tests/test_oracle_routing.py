"""Pins of the oracle's routers: rank-counting brute force, the textbook
soft-max (scipy), closed forms of the weights and invariants."""

import itertools

import numpy as np
import pytest
import scipy.special

import oracle as O


def _beats(la, a, lb, b):
    """(value, index) order: a ranks before b."""
    return la > lb or (la == lb and a < b)


def _brute_topk(row, k):
    """Expert e is chosen iff fewer than k experts rank before it; the chosen
    ones are listed by rank."""
    E = len(row)
    rank = [sum(_beats(row[o], o, row[e], e) for o in range(E) if o != e) for e in range(E)]
    return [e for r in range(k) for e in range(E) if rank[e] == r]


@pytest.mark.parametrize("seed,E,k", [(0, 8, 2), (1, 16, 4), (2, 128, 8), (3, 7, 7), (4, 512, 10)])
def test_softmax_topk_ids_vs_rank_counting(seed, E, k):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((20, E)).astype(np.float32)
    ids, _ = O.route_softmax_topk(logits, k)
    for t in range(20):
        assert list(ids[t]) == _brute_topk(list(map(float, logits[t])), k)


def test_topk_exact_ties_and_signed_zero():
    rng = np.random.default_rng(5)
    logits = rng.integers(-2, 3, (200, 16)).astype(np.float32)      # many exact ties
    logits[0] = 0.0
    logits[0, 3] = -0.0
    logits[0, 1] = -0.0
    ids, _ = O.route_softmax_topk(logits, 6)
    for t in range(200):
        assert list(ids[t]) == _brute_topk(list(map(float, logits[t])), 6)
    assert list(ids[0]) == [0, 1, 2, 3, 4, 5]


def test_softmax_weights_closed_forms():
    rng = np.random.default_rng(6)
    logits = (rng.standard_normal((50, 32)) * 3).astype(np.float32)
    ids, w = O.route_softmax_topk(logits, 5)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)
    sel = np.take_along_axis(logits.astype(np.float64), ids.astype(np.int64), axis=1)
    # w_i / w_j = exp(l_i - l_j)
    assert np.allclose(w[:, 1:] / w[:, :1], np.exp(sel[:, 1:] - sel[:, :1]), rtol=1e-6)
    # weights descend with the key order
    assert np.all(np.diff(w, axis=1) <= 0)
    ids1, w1 = O.route_softmax_topk(logits, 1)
    assert np.all(w1 == 1.0)
    assert np.array_equal(ids1[:, 0], np.argmax(logits, axis=1))


def test_softmax_k_equals_E_is_textbook_softmax():
    rng = np.random.default_rng(7)
    logits = (rng.standard_normal((10, 12)) * 4).astype(np.float32)
    ids, w = O.route_softmax_topk(logits, 12)
    ref = scipy.special.softmax(logits.astype(np.float64), axis=1)
    got = np.zeros_like(ref)
    np.put_along_axis(got, ids.astype(np.int64), w.astype(np.float64), axis=1)
    assert np.allclose(got, ref, rtol=1e-6, atol=1e-9)
    _, wn = O.route_softmax_topk(logits, 3, renormalize=False)
    full = np.take_along_axis(ref, ids[:, :3].astype(np.int64), axis=1)
    assert np.allclose(wn, full, rtol=1e-6)


def test_topk_shift_invariance():
    rng = np.random.default_rng(8)
    logits = rng.integers(-8, 8, (64, 32)).astype(np.float32)
    a, wa = O.route_softmax_topk(logits, 8)
    b, wb = O.route_softmax_topk(logits + np.float32(3.0), 8)
    assert np.array_equal(a, b)
    assert np.allclose(wa, wb, rtol=1e-6)


def _brute_grouped(logits, k, G, tg, bias, scale):
    """Group ranks and expert ranks by counting, scores in fp32 as the oracle
    states them; weights from the unbiased sigmoid scores."""
    E = len(logits)
    gsz = E // G
    s = [np.float32(1.0 / (1.0 + np.exp(-float(v)))) for v in logits]
    key = [np.float32(s[e] + np.float32(bias[e])) for e in range(E)]
    gs = []
    for g in range(G):
        ks = sorted((float(key[e]) for e in range(g * gsz, (g + 1) * gsz)), reverse=True)
        gs.append(float(np.float32(np.float32(ks[0]) + np.float32(ks[1]))))
    grank = [sum(_beats(gs[o], o, gs[g], g) for o in range(G) if o != g) for g in range(G)]
    kept = [e for e in range(E) if grank[e // gsz] < tg]
    erank = {e: sum(_beats(float(key[o]), o, float(key[e]), e) for o in kept if o != e) for e in kept}
    ids = [e for r in range(k) for e in kept if erank[e] == r]
    ss = np.array([float(s[e]) for e in ids])
    return ids, ss / ss.sum() * scale


@pytest.mark.parametrize("seed,E,G,tg,k,use_bias", [(0, 16, 4, 2, 4, False), (1, 32, 8, 4, 8, True),
                                                    (2, 256, 8, 4, 8, False), (3, 24, 4, 1, 3, True)])
def test_sigmoid_grouped_vs_brute_force(seed, E, G, tg, k, use_bias):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((12, E)).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.1).astype(np.float32) if use_bias else np.zeros(E, np.float32)
    ids, w = O.route_sigmoid_grouped(logits, k, G, tg, bias, 2.5)
    for t in range(12):
        bi, bw = _brute_grouped(logits[t], k, G, tg, bias, 2.5)
        assert list(ids[t]) == bi
        assert np.allclose(w[t], bw, rtol=1e-6)
    assert np.allclose(w.sum(axis=1), 2.5, rtol=1e-6)


def test_sigmoid_grouped_kept_groups_are_best_subset():
    """Exhaustive over all C(G, tg) group subsets: the kept groups maximise the
    summed group score (scores distinct with probability one)."""
    rng = np.random.default_rng(11)
    E, G, tg, k = 16, 4, 2, 4
    logits = rng.standard_normal((30, E)).astype(np.float32)
    ids, _ = O.route_sigmoid_grouped(logits, k, G, tg, None, 1.0)
    s = 1.0 / (1.0 + np.exp(-logits.astype(np.float64)))
    for t in range(30):
        gsc = [np.sort(s[t, g * 4:(g + 1) * 4])[-2:].sum() for g in range(G)]
        best = max(itertools.combinations(range(G), tg), key=lambda c: sum(gsc[i] for i in c))
        assert set(int(e) // 4 for e in ids[t]) <= set(best)


def test_sigmoid_one_group_reduces_to_plain_topk():
    rng = np.random.default_rng(12)
    logits = rng.standard_normal((40, 64)).astype(np.float32)
    ids, w = O.route_sigmoid_grouped(logits, 6, 1, 1, None, 1.0)
    ids2, _ = O.route_softmax_topk(logits, 6)
    assert np.array_equal(ids, ids2)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=1e-6)


def test_router_logits_vs_loops():
    rng = np.random.default_rng(13)
    x = O.bf16_round(rng.standard_normal((3, 5)).astype(np.float32))
    wr = (rng.standard_normal((4, 5)) * 0.02).astype(np.float32)
    got = O.router_logits(x, wr)
    for t in range(3):
        for e in range(4):
            ref = sum(float(x[t, d]) * float(wr[e, d]) for d in range(5))
            assert got[t, e] == np.float32(ref)
