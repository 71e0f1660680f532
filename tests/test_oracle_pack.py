"""Pins of the oracle packer: hand-derived golden cases and the properties that fix the greedy
partition uniquely (visiting order, budget, maximality, layout arithmetic)."""

import json
import os

import numpy as np
import pytest

from oracle.pack import pack_ragged, PackError

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pack_cases.json")


def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_golden(case):
    pk = pack_ragged(case["tail_len"], case["budget"], case["max_rows"])
    for key in ("order", "batch_first", "batch_width", "batch_base", "token_offset",
                "last_row", "batch_of", "row_of"):
        assert pk[key] == case[key], key
    assert pk["n_batches"] == len(case["batch_width"])
    assert pk["total_padded_tokens"] == case["batch_base"][-1]


def check_pack_properties(lengths, budget, max_rows, pk):
    n = len(lengths)
    order = pk["order"]
    assert sorted(order) == list(range(n)), "every question exactly once"
    # visiting order: ascending length, ties by index
    keys = [(lengths[i], i) for i in order]
    assert keys == sorted(keys)
    nb = pk["n_batches"]
    bf, bw, bb = pk["batch_first"], pk["batch_width"], pk["batch_base"]
    assert bf[0] == 0 and bf[-1] == n and len(bf) == nb + 1
    assert bb[0] == 0 and len(bb) == nb + 1
    for b in range(nb):
        members = order[bf[b]:bf[b + 1]]
        assert members, "no empty batch"
        width = max(lengths[i] for i in members)
        assert bw[b] == width
        rows = len(members)
        if rows > 1:
            assert rows * width <= budget
        if max_rows:
            assert rows <= max_rows
        assert bb[b + 1] - bb[b] == rows * width
        for r, i in enumerate(members):
            assert pk["batch_of"][i] == b and pk["row_of"][i] == r
            assert pk["token_offset"][i] == bb[b] + r * width
            assert pk["last_row"][i] == pk["token_offset"][i] + lengths[i] - 1
        if b + 1 < nb:
            # maximality: the next question would not have fitted
            nxt = order[bf[b + 1]]
            grown = max(width, lengths[nxt])
            assert grown * (rows + 1) > budget or (max_rows and rows >= max_rows)
    assert pk["total_padded_tokens"] == bb[-1]
    assert pk["total_valid_tokens"] == sum(lengths)


@pytest.mark.parametrize("seed", range(200))
def test_random_properties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 80))
    hi = int(rng.choice([4, 50, 300, 3000]))
    lengths = [int(x) for x in rng.integers(1, hi + 1, size=n)]
    budget = int(rng.choice([1, 7, 64, 1000, 32768]))
    max_rows = int(rng.choice([0, 0, 1, 3, 17]))
    pk = pack_ragged(lengths, budget, max_rows)
    check_pack_properties(lengths, budget, max_rows, pk)


def test_padded_rows_never_overlap():
    lengths = [3, 1, 4, 1, 5, 9, 2, 6]
    pk = pack_ragged(lengths, 12)
    taken = np.zeros(pk["total_padded_tokens"], dtype=int)
    for i, n in enumerate(lengths):
        taken[pk["token_offset"][i]:pk["token_offset"][i] + n] += 1
    assert taken.max() == 1


@pytest.mark.parametrize("bad, msg", [
    ([], "questions; the limit is 1 to 512"),
    ([1] * 513, "request of 513 questions; the limit is 1 to 512"),
    ([3, 0], "empty tail"),
])
def test_refused(bad, msg):
    with pytest.raises(PackError, match=msg):
        pack_ragged(bad)


def test_context_limit():
    with pytest.raises(PackError, match="the maximum context length is 131072"):
        pack_ragged([5, 2], prefix_len=131068)
    pack_ragged([4, 2], prefix_len=131068)  # exactly at the limit is accepted
