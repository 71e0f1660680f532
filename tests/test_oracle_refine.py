"""Pins of the answer-refinement oracle: closed forms of the log-softmax, rotations that must
agree, a prior equal to the pass itself, stable ranking and the minus-infinity scatter."""

import math

import numpy as np
import pytest

from oracle.refine import combine_rotations, log_softmax, scatter_finalists, two_stage_finalists


def test_one_pass_is_the_log_softmax():
    got = combine_rotations([2], [(0, [0, 1], [0.0, math.log(3.0)])])
    assert got[0] == pytest.approx([math.log(0.25), math.log(0.75)], abs=1e-15)


def test_rotations_of_the_same_scores_agree():
    # The same two options shown in both orders, each with the logit that belongs to it:
    # every pass gives each key the same log-probability, so the mean is that value.
    z = {0: 1.3, 1: -0.4, 2: 0.2}
    passes = [(0, [0, 1, 2], [z[0], z[1], z[2]]), (0, [2, 0, 1], [z[2], z[0], z[1]]),
              (0, [1, 2, 0], [z[1], z[2], z[0]])]
    got = combine_rotations([3], passes)[0]
    ref = log_softmax([z[0], z[1], z[2]])
    assert got == pytest.approx(ref, abs=1e-15)


def test_position_bias_cancels_in_the_mean():
    # A pass adds +b to whatever sits first: averaged over all rotations, each key is first once.
    z, b = [0.5, -1.0, 2.0], 0.9
    passes = []
    for r in range(3):
        keys = [(r + i) % 3 for i in range(3)]
        passes.append((0, keys, [z[k] + (b if i == 0 else 0.0) for i, k in enumerate(keys)]))
    biased = combine_rotations([3], passes)[0]
    # the ranking equals the unbiased one, and differences between keys are preserved exactly
    assert np.argsort(biased).tolist() == np.argsort(z).tolist()
    assert biased[2] - biased[0] == pytest.approx(z[2] - z[0], abs=1e-12)


def test_prior_equal_to_the_pass_gives_zero():
    logits = [0.1, 0.7, -2.0, 1.5]
    prior = [log_softmax(logits)]
    got = combine_rotations([4], [(0, [0, 1, 2, 3], logits)], priors=prior)[0]
    assert got == pytest.approx([0.0] * 4, abs=1e-15)


def test_unoffered_key_is_nan_and_questions_are_separate():
    got = combine_rotations([3, 2], [(0, [0, 2], [1.0, 1.0]), (1, [1, 0], [0.0, 0.0])])
    assert math.isnan(got[0][1])
    assert got[0][0] == pytest.approx(math.log(0.5)) and got[1] == pytest.approx([math.log(0.5)] * 2)


def test_two_stage_ranking_and_scatter():
    s1 = [0.2, 1.5, 1.5, -3.0, 0.9]
    assert two_stage_finalists(s1, 3) == [1, 2, 4]  # the tie keeps option 1 before 2
    assert two_stage_finalists(s1, 10) == [1, 2, 4, 0, 3]
    full = scatter_finalists(5, [1, 2, 4], [0.3, -0.1, 2.0])
    assert full[1] == 0.3 and full[2] == -0.1 and full[4] == 2.0
    assert full[0] == float("-inf") and full[3] == float("-inf")
    p = np.exp(np.array(full) - max(full))
    p /= p.sum()
    assert p[0] == 0.0 and p[3] == 0.0 and abs(p.sum() - 1.0) < 1e-15
