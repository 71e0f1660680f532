"""Pins of the shared-prefix oracle: hand-derived cases, the pages' threshold, the route the
page takes (the lexicographically smallest and largest sequences), brute force over planted
prefixes, and order invariance."""

import json
import os

import numpy as np
import pytest

from oracle.prefix import PREFIX_MIN_TOKENS, PrefixError, plan_prefix, shared_prefix_len

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "prefix_cases.json")


def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_golden(case):
    assert plan_prefix(case["seqs"], case["min_prefix_tokens"]) == (
        case["shared"], case["prefix_len"], case["prefill_tokens"])


def _planted(shared, tails, seed=0):
    rng = np.random.default_rng(seed)
    head = rng.integers(0, 50, size=shared).tolist()
    seqs = []
    for i, t in enumerate(tails):
        # the first own token differs between every pair of sequences
        seqs.append(head + [1000 + i] + rng.integers(0, 50, size=t - 1).tolist())
    return seqs


def test_the_pages_threshold():
    seqs = _planted(260, [40, 40, 40])
    assert PREFIX_MIN_TOKENS == 256
    assert plan_prefix(seqs) == (260, 260, 900 - 2 * 260)
    assert plan_prefix(seqs, 261) == (260, 0, 900)
    assert plan_prefix(_planted(255, [10, 20])) == (255, 0, 2 * 255 + 30)


def _lexicographic_route(seqs):
    """The page's computation: the common prefix of all sequences is the common prefix of the
    lexicographically smallest and largest one."""
    if len(seqs) < 2:
        return 0
    lo, hi = min(seqs), max(seqs)
    p = 0
    while p < min(len(lo), len(hi)) and lo[p] == hi[p]:
        p += 1
    return min(p, min(len(s) for s in seqs) - 1)


@pytest.mark.parametrize("seed", range(30))
def test_matches_the_lexicographic_route(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 8))
    base = rng.integers(0, 3, size=int(rng.integers(1, 12))).tolist()
    seqs = []
    for _ in range(n):
        cut = int(rng.integers(0, len(base) + 1))
        seqs.append(base[:cut] + rng.integers(0, 3, size=int(rng.integers(0, 4))).tolist())
    seqs = [s if s else [0] for s in seqs]
    assert shared_prefix_len(seqs) == _lexicographic_route(seqs)


@pytest.mark.parametrize("seed", range(10))
def test_planted_prefix_and_order(seed):
    rng = np.random.default_rng(50 + seed)
    shared = int(rng.integers(0, 400))
    tails = rng.integers(1, 30, size=int(rng.integers(2, 10))).tolist()
    seqs = _planted(shared, tails, seed)
    assert shared_prefix_len(seqs) == shared
    perm = rng.permutation(len(seqs))
    assert shared_prefix_len([seqs[i] for i in perm]) == shared
    got = plan_prefix(seqs, 1)
    if shared:
        assert got == (shared, shared, shared + sum(tails))
    else:
        assert got == (0, 0, sum(tails))


def test_refusals():
    with pytest.raises(PrefixError, match="at least 1"):
        plan_prefix([[1, 2], [1, 3]], 0)
    with pytest.raises(PrefixError, match="at least one token"):
        plan_prefix([[1, 2], []], 1)
