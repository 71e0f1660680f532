"""Pins of the distinct-label-row table and the batched readout of the oracle: hand-derived
golden tables, the properties that fix the table uniquely, and equality of the batched and
per-question readouts."""

import json
import os

import numpy as np
import pytest

from oracle.readout import label_readout, label_readout_batched, label_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "label_rows_cases.json")


def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_golden(case):
    row_id, row_first, row_entry = label_rows(case["cand_ids"], case["cand_off"])
    assert row_id == case["row_id"]
    assert row_first == case["row_first"]
    assert row_entry == case["row_entry"]


def check_label_rows_properties(ids, row_id, row_first, row_entry):
    """Every property below holds for exactly one table, so together they fix it."""
    ids = [int(x) for x in ids]
    u = len(row_id)
    assert all(row_id[j] < row_id[j + 1] for j in range(u - 1)), "strictly ascending ids"
    assert len(row_first) == u + 1 and row_first[0] == 0 and row_first[-1] == len(ids)
    assert sorted(row_entry) == list(range(len(ids))), "each entry exactly once"
    for j in range(u):
        grp = row_entry[row_first[j]:row_first[j + 1]]
        assert grp, "no empty row"
        assert all(ids[e] == row_id[j] for e in grp), "entries carry their row's id"
        assert grp == sorted(grp), "ascending entries within a row"


def random_table(rng, n, vocab, kmax, shared=False):
    k = rng.integers(1, kmax + 1, size=n)
    if shared:
        table = rng.choice(vocab, size=int(k.max()), replace=False)
        ids = np.concatenate([table[:int(x)] for x in k])
    else:
        ids = np.concatenate([rng.choice(vocab, size=int(x), replace=False) for x in k])
    off = np.concatenate([[0], np.cumsum(k)])
    return ids.astype(np.int32), off.astype(np.int32)


@pytest.mark.parametrize("seed", range(20))
def test_properties_random(seed):
    rng = np.random.default_rng(seed)
    ids, off = random_table(rng, int(rng.integers(1, 40)), int(rng.integers(1, 60)) + 8,
                            8, shared=bool(seed % 2))
    row_id, row_first, row_entry = label_rows(ids, off)
    check_label_rows_properties(ids, row_id, row_first, row_entry)
    # brute force: the distinct ids are the values that occur, counted the long way
    occurs = [t for t in range(int(ids.max()) + 1) if any(int(x) == t for x in ids)]
    assert row_id == occurs


@pytest.mark.parametrize("seed", range(5))
def test_batched_equals_per_question(seed):
    rng = np.random.default_rng(100 + seed)
    n, d, vocab, t_pad = 9, 24, 40, 50
    hidden = rng.standard_normal((t_pad, d))
    w_u = rng.standard_normal((vocab, d)) * 0.3
    ids, off = random_table(rng, n, vocab, 12, shared=bool(seed % 2))
    last = rng.integers(0, t_pad, size=n)
    a = label_readout(hidden, last, w_u, ids, off, 0.9)
    b = label_readout_batched(hidden, last, w_u, ids, off, 0.9)
    np.testing.assert_allclose(b[0], a[0], atol=1e-13)
    np.testing.assert_allclose(b[1], a[1], atol=1e-14)
    np.testing.assert_array_equal(b[2], a[2])


def test_batched_reads_the_right_column():
    # Two questions share label 1 and 3 in different option positions.
    hidden = np.array([[1.0, 0.0], [0.0, 1.0]])
    w_u = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0], [7.0, 8.0]])
    logits, _, _ = label_readout_batched(hidden, [0, 1], w_u, [3, 1, 1, 3, 0], [0, 2, 5], 1.0)
    np.testing.assert_array_equal(logits, [7.0, 3.0, 4.0, 8.0, 2.0])
