"""Pins of the oracle's greedy acceptance.

Checked against: brute force over every root path of small random trees
(with an argmax written as a sort), planted paths whose accepted length is
known by construction, and hand cases for ties, signed zeros and NaN.
"""

import math

import numpy as np
import pytest

import oracle
import synth


def brute_argmax(row):
    """Index of the largest value: NaN ranks below every number, -0 == +0,
    ties go to the smallest index."""
    keyed = sorted(range(len(row)), key=lambda v: (0 if math.isnan(row[v]) else 1,
                                                   -math.inf if math.isnan(row[v]) else float(row[v]) + 0.0,
                                                   -v))
    return keyed[-1]


def brute_accept(logits, parent, tokens):
    n = len(parent)
    a = [brute_argmax(logits[i]) for i in range(n)]
    best = None
    for i in range(n):
        path = [i]
        while parent[path[-1]] >= 0:
            path.append(int(parent[path[-1]]))
        path = path[::-1]
        if all(tokens[path[k + 1]] == a[path[k]] for k in range(len(path) - 1)):
            if best is None or (len(path), [-x for x in path]) > (len(best), [-x for x in best]):
                best = path
    n_acc = len(best) - 1
    bonus = a[best[-1]]
    res = [-1] * (2 + 2 * n)
    res[0] = n_acc
    res[1] = bonus
    res[2:2 + len(best)] = best
    emitted = [int(tokens[p]) for p in best[1:]] + [bonus]
    res[2 + n:2 + n + len(emitted)] = emitted
    return np.array(a, np.int32), np.array(res, np.int32)


def test_random_small_trees_match_brute_force():
    rng = np.random.default_rng(2024)
    for trial in range(3000):
        n = int(rng.integers(1, 13))
        parent = synth.draft_tree(rng, n, depth_cap=int(rng.integers(1, 8)), p_spine=float(rng.random()))
        V = int(rng.integers(2, 6))
        tokens = rng.integers(0, V, size=n).astype(np.int32)  # duplicates among siblings allowed
        logits = rng.integers(-2, 3, size=(n, V)).astype(np.float32)  # many ties
        if trial % 7 == 0:
            logits[rng.random((n, V)) < 0.2] = np.nan
        if trial % 5 == 0:
            logits[logits == 0] = -0.0
        am, res = oracle.accept(logits, parent, tokens)
        bam, bres = brute_accept(logits, parent, tokens)
        assert np.array_equal(am, bam), trial
        assert np.array_equal(res, bres), (trial, parent, tokens, logits)


def test_planted_paths_give_their_length():
    for seed in range(200):
        s = synth.streams(seed)
        parent = synth.draft_tree(s["tree"], 23, 16)
        tokens = synth.sibling_distinct_tokens(s["tokens"], parent, 1024)
        logits, L, path = synth.planted_logits(s["logits"], parent, tokens, 1024)
        am, res = oracle.accept(logits, parent, tokens)
        assert res[0] == L
        assert list(res[2:2 + L + 1]) == path
        assert list(res[2 + 23:2 + 23 + L]) == [int(tokens[p]) for p in path[1:]]
        assert res[2 + 23 + L] == am[path[-1]] == res[1]


@pytest.mark.parametrize("row,expect", [
    ([1.0, 3.0, 3.0, 2.0], 1),                 # tie -> smallest index
    ([-0.0, 0.0, -1.0], 0),                    # -0 == +0
    ([0.0, -0.0, -1.0], 0),
    ([-1.0, -0.0, 0.0], 1),
    ([math.nan, 1.0, 2.0], 2),                 # NaN never wins
    ([math.nan, -math.inf], 1),                # ... not even over -inf
    ([math.nan, math.nan, math.nan], 0),       # all NaN -> 0
    ([-math.inf, -math.inf], 0),
    ([math.inf, math.nan, math.inf], 0),
    ([-3.4e38, -1e-45, -0.0], 2),              # subnormal below zero
])
def test_argmax_hand_cases(row, expect):
    assert oracle.argmax_row(np.array(row, np.float32)) == expect == brute_argmax(row)


def test_duplicate_sibling_tokens_take_longest_then_smallest():
    # root has children 1 and 2, both with token 7; only 2 continues
    parent = np.array([-1, 0, 0, 2], np.int32)
    tokens = np.array([0, 7, 7, 5], np.int32)
    logits = np.zeros((4, 10), np.float32)
    logits[0, 7] = 1
    logits[2, 5] = 1
    logits[1, 3] = 1
    logits[3, 9] = 1
    _, res = oracle.accept(logits, parent, tokens)
    assert res[0] == 2 and list(res[2:5]) == [0, 2, 3] and res[1] == 9
    # equal lengths: the smaller child wins
    logits[2, 5] = 0
    logits[2, 1] = 1
    _, res = oracle.accept(logits, parent, tokens)
    assert res[0] == 1 and list(res[2:4]) == [0, 1] and res[1] == 3


def test_nothing_accepted_gives_bonus_only():
    parent = np.array([-1, 0, 0], np.int32)
    tokens = np.array([0, 1, 2], np.int32)
    logits = np.zeros((3, 5), np.float32)
    logits[0, 4] = 1.0
    _, res = oracle.accept(logits, parent, tokens)
    assert res[0] == 0 and res[1] == 4 and res[2] == 0 and res[3] == -1
    assert res[2 + 3] == 4 and res[2 + 3 + 1] == -1
