"""Oracle for typed-answer assembly (test infrastructure only).

Follows the blink.py page (thegovind/blink-4b), "answer assembly" section, answer_for, and
"rendering" section, question_options (a "noul" question offers yes then no; a "score"
question offers its levels 0..K-1, 2 <= K <= 10): the question's option probabilities are
first renormalised to sum to one (a zero sum divides by one), then
  * choice: the most probable option, the earlier one on ties, and its confidence
    (p_best - 1/K) / (1 - 1/K), or 1 for a single option;
  * noul:   the probability of "yes";
  * score:  the expected level sum_k k p_k, the most probable level (the lower on ties) and the
            same confidence formula clipped to [0, 1].
Plain Python floats (float64), in the page's order of operations.
"""

from __future__ import annotations

CHOICE, NOUL, SCORE = 0, 1, 2


class AnswerError(ValueError):
    pass


def answer_for(qtype: int, probs):
    """Returns (choice index or -1, confidence or None, value or None) for one question."""
    p = [float(x) for x in probs]
    z = sum(p) or 1.0
    p = [v / z for v in p]
    k = len(p)
    if qtype == CHOICE:
        if k < 1:
            raise AnswerError("a choice needs at least one option")
        best = 0
        for i in range(1, k):
            if p[i] > p[best]:
                best = i
        conf = (p[best] - 1 / k) / (1 - 1 / k) if k > 1 else 1.0
        return best, conf, p[best]
    if qtype == NOUL:
        if k != 2:
            raise AnswerError("a noul question offers exactly yes and no")
        return -1, None, p[0]
    if qtype == SCORE:
        if not 2 <= k <= 10:
            raise AnswerError("a score takes 2 to 10 levels")
        ev = sum(i * p[i] for i in range(k))
        top = 0
        for i in range(1, k):
            if p[i] > p[top]:
                top = i
        conf = min(1.0, max(0.0, (p[top] - 1 / k) / (1 - 1 / k)))
        return top, conf, ev
    raise AnswerError(f"unknown question type {qtype}")


def assemble(qtypes, probs, cand_off):
    """answer_for over every question of a request (probabilities in CSR by question)."""
    return [answer_for(int(t), probs[int(cand_off[i]):int(cand_off[i + 1])])
            for i, t in enumerate(qtypes)]
