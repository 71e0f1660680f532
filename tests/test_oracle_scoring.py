"""Pins of the teacher-forced scoring oracle: the pages' row/target positions, closed forms,
brute force in plain Python on a tiny vocabulary, normalisation and shift invariance; and the
sensitivity of the GPU bar: a vocabulary tile dropped from the oracle's log-sum-exp moves the
result by more than the bar the GPU parity tests use."""

import math

import numpy as np
import pytest

import synth
from helpers import SCORE_TOL
from oracle.scoring import ScoringError, score_rows, teacher_forced_logprobs


def test_rows_and_targets():
    # 10 tokens, the last 3 scored: rows 6, 7, 8 predict positions 7, 8, 9.
    assert score_rows(10, 3) == ([6, 7, 8], [7, 8, 9])
    assert score_rows(2, 1) == ([0], [1])
    with pytest.raises(ScoringError):
        score_rows(5, 5)
    with pytest.raises(ScoringError):
        score_rows(5, 0)


def test_zero_logits_are_uniform():
    hidden = np.ones((3, 4))
    w_u = np.zeros((37, 4))
    lp = teacher_forced_logprobs(hidden, [0, 2], [5, 36], w_u)
    np.testing.assert_allclose(lp, -math.log(37), atol=1e-15)


def test_brute_force_tiny_vocab():
    rng = np.random.default_rng(0)
    hidden = rng.standard_normal((5, 3))
    w_u = rng.standard_normal((6, 3))
    rows, targets = [4, 1, 1], [0, 5, 2]
    lp = teacher_forced_logprobs(hidden, rows, targets, w_u)
    for j, (r, t) in enumerate(zip(rows, targets)):
        z = [sum(float(w_u[v, d]) * float(hidden[r, d]) for d in range(3)) for v in range(6)]
        ref = z[t] - math.log(sum(math.exp(x) for x in z))
        assert abs(lp[j] - ref) < 1e-12


def test_probabilities_sum_to_one_and_shift_invariance():
    rng = np.random.default_rng(1)
    hidden = rng.standard_normal((2, 8))
    w_u = rng.standard_normal((50, 8)) * 2
    lp = teacher_forced_logprobs(hidden, [1] * 50, list(range(50)), w_u)
    assert abs(np.exp(lp).sum() - 1.0) < 1e-12
    # adding one vector to every unembedding row adds the same logit to every token
    shifted = teacher_forced_logprobs(hidden, [1] * 50, list(range(50)), w_u + rng.standard_normal(8))
    np.testing.assert_allclose(shifted, lp, atol=1e-12)
    # large logits do not overflow
    big = teacher_forced_logprobs(hidden, [0], [3], w_u * 400)
    assert np.isfinite(big).all() and big[0] <= 0


def test_refusal():
    with pytest.raises(ScoringError, match="outside the vocabulary"):
        teacher_forced_logprobs(np.zeros((1, 2)), [0], [9], np.zeros((9, 2)))


@pytest.mark.parametrize("dropped", [32, 128])
def test_bar_sees_a_dropped_vocabulary_tile(dropped):
    # The readout workload's scale (W_U ~ N(0, 0.02) in bf16, hidden ~ N(0, 1)) at the full
    # vocabulary of 151936, on a narrower hidden width (256) to keep the oracle quick. Dropping
    # one tile of `dropped` vocabulary rows from the normaliser (a mistake planted in the
    # oracle's input, on the CPU) must move every log-probability by more than the bar.
    rng = np.random.default_rng(11)
    vocab, d = 151936, 256
    hidden = synth.f32_to_bf16_bits(rng.standard_normal((4, d)).astype(np.float32))
    w_u = synth.f32_to_bf16_bits((rng.standard_normal((vocab, d)) * 0.02).astype(np.float32))
    rows, targets = [0, 1, 2, 3], [5, 70000, 150000, 1000]
    full = teacher_forced_logprobs(hidden, rows, targets, w_u)
    for start in (256, 66560, vocab - dropped):  # targets lie outside every dropped tile
        keep = np.ones(vocab, bool)
        keep[start:start + dropped] = False
        remap = np.cumsum(keep) - 1
        cut = teacher_forced_logprobs(hidden, rows, [int(remap[t]) for t in targets], w_u[keep])
        shift = cut - full
        assert (shift > SCORE_TOL).all(), (start, shift)
