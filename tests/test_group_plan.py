"""Host side of the grouped scoring step (plan_group), without a GPU: each request of a group
is checked on its own and a refused request carries its own error while the others go ahead
("public entry point" section of the blink.py page, decide_many), and the accepted requests
are split, in order, into launches within the limits of one grouped launch (64 requests, 512
questions)."""

import numpy as np
import pytest

import pass_typed_decision_amd as blink
from pass_typed_decision_amd.group import plan_group


def _req(tails, base, k=3, prefix=0, pstart=0, ids=None):
    n = len(tails)
    off = np.arange(n + 1, dtype=np.int32) * k
    cand = np.asarray(ids if ids is not None else np.tile(np.arange(k), n), np.int32)
    return blink.GroupRequest(np.asarray(tails, np.int32), cand, off, base, pstart, prefix)


def test_refusals_stay_with_their_request():
    reqs = [
        _req([5, 7, 3], 0, prefix=100, pstart=0),           # accepted: rows [0, 21)
        _req([4], 21, k=256, ids=np.arange(256)),           # 256 options
        _req([200], 30, prefix=131000, pstart=0),           # context past 131072
        _req([2, 2], 10),                                   # rows [10, 14) overlap request 0
        _req([1, 1], 500),                                  # rows [500, 502) past 100 rows
        _req([3], 40, prefix=50, pstart=90),                # prefix rows [90, 140) past 120
        _req([1, 2], 60, ids=[0, 0, 1, 2, 3, 4]),            # ids collide in question 0
        _req([0, 2], 70),                                   # an empty tail
        _req([6, 6], 80, prefix=20, pstart=100),            # accepted: rows [80, 92)
    ]
    packs, results, launches = plan_group(reqs, t_rows=100, prefix_rows=120, vocab=1000)
    assert launches == [[0, 8]]
    assert results[0] is None and results[8] is None
    want = {1: "256 options", 2: "maximum context length", 3: "overlap another request",
            4: "outside the 100 packed rows", 5: "outside the 120 prefix rows",
            6: "collide", 7: "empty tail"}
    for r, msg in want.items():
        assert isinstance(results[r], blink.BlinkError), r
        assert msg in str(results[r]), (r, str(results[r]))
        assert packs[r] is None
    assert packs[0].total_padded_tokens == 21 and packs[8].total_padded_tokens == 12


def test_launches_respect_the_limits():
    # 70 one-question requests: at most 64 requests per launch.
    reqs = [_req([1], i) for i in range(70)]
    _, results, launches = plan_group(reqs, t_rows=70, prefix_rows=0, vocab=10)
    assert all(r is None for r in results)
    assert [len(l) for l in launches] == [64, 6]
    assert sum(launches, []) == list(range(70))
    # 9 requests of 60 questions: 512 questions at most per launch, requests kept whole.
    reqs = [_req([1] * 60, 60 * i) for i in range(9)]
    _, _, launches = plan_group(reqs, t_rows=540, prefix_rows=0, vocab=10)
    assert launches == [list(range(8)), [8]]
    # A refused request in the middle does not break the order of the others.
    reqs = [_req([1] * 300, 0), _req([1], 300, k=0), _req([1] * 300, 301), _req([1] * 200, 601)]
    _, results, launches = plan_group(reqs, t_rows=1000, prefix_rows=0, vocab=10)
    assert isinstance(results[1], blink.BlinkError)
    assert launches == [[0], [2, 3]]
