"""Pins of the typed-answer oracle: hand-derived cases, closed forms and the refusals."""

import json
import os

import numpy as np
import pytest

from oracle.answers import CHOICE, NOUL, SCORE, AnswerError, answer_for, assemble

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "answer_cases.json")


def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_golden(case):
    choice, conf, value = answer_for(case["type"], case["probs"])
    assert choice == case["choice"]
    if case["confidence"] is None:
        assert conf is None
    else:
        assert conf == pytest.approx(case["confidence"], abs=1e-15)
    assert value == pytest.approx(case["value"], abs=1e-15)


@pytest.mark.parametrize("seed", range(10))
def test_closed_forms(seed):
    rng = np.random.default_rng(seed)
    k = int(rng.integers(2, 11))
    p = rng.dirichlet(np.ones(k))
    choice, conf, value = answer_for(SCORE, p)
    assert value == pytest.approx(float(np.dot(np.arange(k), p)), abs=1e-14)
    assert choice == int(np.argmax(p))
    assert 0.0 <= conf <= 1.0
    # a point mass on one level is a certain answer at that level
    e = np.zeros(k)
    e[k // 2] = 1.0
    assert answer_for(SCORE, e) == (k // 2, 1.0, float(k // 2))
    assert answer_for(CHOICE, e) == (k // 2, 1.0, 1.0)
    # scaling all probabilities does not change the answer
    c1, f1, v1 = answer_for(CHOICE, p)
    c2, f2, v2 = answer_for(CHOICE, p * 3.5)
    assert c1 == c2 and f1 == pytest.approx(f2, abs=1e-14) and v1 == pytest.approx(v2, abs=1e-14)


def test_zero_sum_divides_by_one():
    assert answer_for(NOUL, [0.0, 0.0]) == (-1, None, 0.0)


def test_assemble_walks_the_csr():
    got = assemble([CHOICE, NOUL, SCORE], np.array([0.2, 0.8, 0.6, 0.4, 0.5, 0.5]), [0, 2, 4, 6])
    assert got[0][0] == 1 and got[1] == (-1, None, 0.6) and got[2][2] == pytest.approx(0.5)


def test_refusals():
    with pytest.raises(AnswerError, match="yes and no"):
        answer_for(NOUL, [0.2, 0.3, 0.5])
    with pytest.raises(AnswerError, match="2 to 10 levels"):
        answer_for(SCORE, [1.0])
    with pytest.raises(AnswerError, match="2 to 10 levels"):
        answer_for(SCORE, [0.1] * 11)
    with pytest.raises(AnswerError, match="unknown question type"):
        answer_for(7, [1.0])
