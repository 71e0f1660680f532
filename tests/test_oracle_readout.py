"""Pins of the readout oracle: closed forms, a different library's dot and softmax, the
gather index, temperature, overflow safety, tie-break and the refusals."""

import math

import numpy as np
import pytest
import torch

from oracle.readout import label_readout, softmax_t, ReadoutError


def _case(seed, n=5, d=16, vocab=50, t_pad=30):
    rng = np.random.default_rng(seed)
    hidden = rng.standard_normal((t_pad, d))
    w_u = rng.standard_normal((vocab, d)) * 0.5
    k = rng.integers(1, 9, size=n)
    off = np.concatenate([[0], np.cumsum(k)])
    ids = np.concatenate([rng.choice(vocab, size=int(x), replace=False) for x in k])
    last = rng.integers(0, t_pad, size=n)
    return hidden, w_u, ids, off, last


def test_zero_scores_are_uniform():
    hidden = np.zeros((4, 8))
    w_u = np.ones((10, 8))
    logits, probs, arg = label_readout(hidden, [1, 3], w_u, [2, 5, 7, 1, 0], [0, 3, 5], 1.0)
    np.testing.assert_array_equal(logits, 0.0)
    np.testing.assert_allclose(probs, [1 / 3] * 3 + [0.5] * 2, atol=1e-16)
    assert list(arg) == [0, 0]


def test_log_three_gives_quarter_and_three_quarters():
    hidden = np.array([[1.0, 0.0]])
    w_u = np.array([[0.0, 5.0], [math.log(3.0), -2.0]])
    logits, probs, arg = label_readout(hidden, [0], w_u, [0, 1], [0, 2], 1.0)
    np.testing.assert_allclose(probs, [0.25, 0.75], atol=1e-15)
    assert arg[0] == 1


def test_temperature_divides_scores():
    hidden, w_u, ids, off, last = _case(1)
    _, p_t, _ = label_readout(hidden, last, w_u, ids, off, 0.7)
    _, p_1, _ = label_readout(hidden, last, w_u / 0.7, ids, off, 1.0)
    np.testing.assert_allclose(p_t, p_1, atol=1e-14)
    _, p_2, _ = label_readout(hidden, last, w_u, ids, off, 1.0)
    assert np.abs(p_t - p_2).max() > 1e-3


@pytest.mark.parametrize("seed", range(5))
def test_against_torch_float64(seed):
    hidden, w_u, ids, off, last = _case(seed)
    logits, probs, arg = label_readout(hidden, last, w_u, ids, off, 0.8)
    ht, wt = torch.from_numpy(hidden), torch.from_numpy(w_u)
    for i in range(len(last)):
        rows = wt[torch.from_numpy(ids[off[i]:off[i + 1]]).long()]
        z = torch.mv(rows, ht[int(last[i])])
        np.testing.assert_allclose(logits[off[i]:off[i + 1]], z.numpy(), atol=1e-13)
        np.testing.assert_allclose(probs[off[i]:off[i + 1]], torch.softmax(z / 0.8, 0).numpy(), atol=1e-15)
        assert abs(probs[off[i]:off[i + 1]].sum() - 1.0) < 1e-14
        assert arg[i] == int(torch.argmax(z))


def test_reads_the_last_valid_row():
    hidden = np.eye(4)
    w_u = np.diag([1.0, 2.0, 3.0, 4.0])
    logits, _, _ = label_readout(hidden, [2], w_u, [0, 1, 2, 3], [0, 4], 1.0)
    np.testing.assert_array_equal(logits, [0.0, 0.0, 3.0, 0.0])


def test_large_scores_do_not_overflow():
    hidden = np.array([[1.0]])
    w_u = np.array([[1000.0], [999.0], [-1000.0]])
    _, probs, arg = label_readout(hidden, [0], w_u, [0, 1, 2], [0, 3], 1.0)
    e = math.exp(-1.0)
    np.testing.assert_allclose(probs, [1 / (1 + e), e / (1 + e), 0.0], atol=1e-15)
    assert arg[0] == 0


def test_options_permute_with_their_probabilities():
    hidden, w_u, ids, off, last = _case(7, n=1)
    k = off[1]
    perm = np.random.default_rng(0).permutation(k)
    _, p, _ = label_readout(hidden, last, w_u, ids, off, 1.3)
    _, q, _ = label_readout(hidden, last, w_u, ids[perm], off, 1.3)
    np.testing.assert_allclose(q, p[perm], atol=1e-15)


def test_ties_go_to_the_first_option():
    hidden = np.array([[1.0, 1.0]])
    w_u = np.array([[0.5, 0.5], [1.0, 0.0], [0.0, 1.0], [0.2, 0.2]])
    _, probs, arg = label_readout(hidden, [0], w_u, [3, 1, 2, 0], [0, 4], 1.0)
    assert arg[0] == 1


def test_single_option_is_certain():
    hidden, w_u, ids, off, last = _case(3)
    logits, probs, arg = label_readout(hidden, [4], w_u, [7], [0, 1], 1.0)
    assert probs[0] == 1.0 and arg[0] == 0


@pytest.mark.parametrize("temperature", [0.0, -1.0, float("nan"), float("inf")])
def test_bad_temperature(temperature):
    with pytest.raises(ReadoutError, match="temperature is not a positive finite number"):
        softmax_t([1.0, 2.0], temperature)


def test_refusals():
    hidden = np.zeros((2, 2))
    w_u = np.zeros((300, 2))
    with pytest.raises(ReadoutError, match="question with 0 options"):
        label_readout(hidden, [0], w_u, [], [0, 0], 1.0)
    with pytest.raises(ReadoutError, match="question with 256 options; the limit is 1 to 255"):
        label_readout(hidden, [0], w_u, list(range(256)), [0, 256], 1.0)
    with pytest.raises(ReadoutError, match="collide"):
        label_readout(hidden, [0], w_u, [4, 4], [0, 2], 1.0)
