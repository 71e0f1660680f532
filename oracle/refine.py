"""Oracle for the answer refinements of the ruling page (test infrastructure only).

Follows the ruling distill/engine page:
  * _score_plain: a question is read in several passes, each presenting its options in some
    order (a rotation); every pass's label logits become log-probabilities (log-softmax over
    the pass's options), a content-free prior's log-probabilities for the same positions are
    subtracted when prior debiasing is on, and each option key's final score is the mean of its
    values over the passes that offered it;
  * TwoStageChoice: a choice wider than one pass allows is first scored per option; the
    options ranked by that score (highest first, earlier options first on ties) keep their
    first few as finalists, the final choice scores only those, and every other option gets a
    score of minus infinity.
Plain Python floats (float64).
"""

from __future__ import annotations

import math

import numpy as np


def log_softmax(z):
    z = [float(v) for v in z]
    m = max(z)
    s = sum(math.exp(v - m) for v in z)
    return [v - m - math.log(s) for v in z]


def combine_rotations(n_keys, passes, priors=None):
    """n_keys[q]: options of question q. passes: (question, key of each position, logits of
    each position). priors: None, or per pass the prior log-probability of each position.
    Returns one list per question: the mean over passes of each key's (debiased)
    log-probability, NaN for a key no pass offered."""
    sums = [[0.0] * k for k in n_keys]
    counts = [[0] * k for k in n_keys]
    for p, (q, keys, logits) in enumerate(passes):
        lp = log_softmax(logits)
        for pos, key in enumerate(keys):
            v = lp[pos] - (float(priors[p][pos]) if priors is not None else 0.0)
            sums[q][key] += v
            counts[q][key] += 1
    return [[s / c if c else float("nan") for s, c in zip(sq, cq)]
            for sq, cq in zip(sums, counts)]


def two_stage_finalists(stage_one, keep):
    """Indices of the options kept for the final choice: highest stage-one score first,
    earlier options first on ties, at most `keep` of them."""
    order = sorted(range(len(stage_one)), key=lambda i: -float(stage_one[i]))  # stable
    return order[:keep]


def scatter_finalists(n_options, finalists, final_logits):
    """Full-width logits: the finalists' final scores, minus infinity elsewhere."""
    full = [float("-inf")] * n_options
    for key, v in zip(finalists, final_logits):
        full[key] = float(v)
    return full
