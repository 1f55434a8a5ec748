"""Pins of the oracle's top-k block selection (O2): hand-worked cases, brute
force over all subsets on tiny rows, structural invariants."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import topk_select_row, topk_select, check_selection_row

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_worked_cases():
    g = json.load(open(os.path.join(GOLD, "topk_hand.json")))
    for c in g["cases"]:
        got = topk_select_row(np.array(c["scores"], np.float64), c["local"], c["k"])
        assert got.tolist() == c["expect"], c


def _brute_force(scores, local, k):
    """Every (k-1)-subset (or all of them, if fewer) of the competing blocks
    whose smallest score is >= the largest score left out is a valid top set;
    among those, ties resolve to the lowest indices, i.e. the smallest index
    sum.  Returns the selection in output form."""
    R = min(k - 1, local)
    cand = list(range(local))
    best = None
    for sub in itertools.combinations(cand, R):
        inside = [scores[b] for b in sub]
        outside = [scores[b] for b in cand if b not in sub]
        if inside and outside and min(inside) < max(outside):
            continue
        key = sum(sub)
        if best is None or key < best[0]:
            best = (key, sub)
    sel = sorted(list(best[1]) + [local])
    return sel + [-1] * (k - len(sel))


@pytest.mark.parametrize("seed", range(40))
def test_brute_force_subsets(seed):
    rng = np.random.default_rng(seed)
    nb = int(rng.integers(1, 11))
    local = int(rng.integers(0, nb))
    k = int(rng.integers(1, 6))
    if seed % 2:
        scores = rng.integers(-2, 3, size=nb).astype(np.float64)   # many exact ties
    else:
        scores = rng.standard_normal(nb)
    got = topk_select_row(scores, local, k).tolist()
    assert got == _brute_force(scores, local, k), (scores, local, k)


def test_invariants_and_monotone_transform():
    rng = np.random.default_rng(1)
    for _ in range(200):
        nb = int(rng.integers(1, 300))
        local = int(rng.integers(0, nb))
        k = int(rng.integers(1, 20))
        s = rng.standard_normal(nb)
        sel = topk_select_row(s, local, k)
        v = sel[sel >= 0]
        assert v.size == min(k, local + 1)
        assert v[-1] == local and np.all(np.diff(v) > 0) and np.all(sel[v.size:] == -1)
        # selection depends only on the order of the scores
        assert np.array_equal(topk_select_row(np.exp(s) * 3 - 1, local, k), sel)
        # the local block's own score never matters
        s2 = s.copy()
        s2[local] = -1e9
        assert np.array_equal(topk_select_row(s2, local, k), sel)
        ok, why = check_selection_row(sel, s, local, k)
        assert ok, why


def test_acceptance_rule_rejects_wrong_sets_and_accepts_near_ties():
    s = np.array([0.0, 5.0, 4.0, 4.0005, 1.0, 0.0])
    local, k = 5, 3
    ref = topk_select_row(s, local, k)
    assert ref.tolist() == [1, 3, 5]
    # 4.0 vs 4.0005 lie within the 1e-3 band: either is acceptable
    assert check_selection_row(np.array([1, 2, 5]), s, local, k)[0]
    assert not check_selection_row(np.array([1, 4, 5]), s, local, k)[0]
    assert not check_selection_row(np.array([1, 3, 4]), s, local, k)[0]      # local missing
    assert not check_selection_row(np.array([3, 1, 5]), s, local, k)[0]      # order
    s2 = np.array([0.0, 5.0, 4.0, 4.5, 1.0, 0.0])                            # clear gap
    assert not check_selection_row(np.array([1, 2, 5]), s2, local, k)[0]


def test_topk_select_over_rows_uses_each_rows_local_block():
    qo, kv, B = [3, 2], [300, 2], 128
    ms = np.random.default_rng(2).standard_normal((5, 2, 3))
    out = topk_select(ms, qo, kv, B, 2)
    # rows of sequence 0 sit at positions 297..299 (local block 2); sequence 1 at 0..1 (block 0)
    assert out[:3, :, 1].tolist() == [[2, 2]] * 3
    assert out[3:, :, :].tolist() == [[[0, -1], [0, -1]]] * 2
