"""Oracle for teacher-forced multi-token scoring (test infrastructure only).

Follows the simit MoT engine page's teacher-forced scoring (its job option score_len and the
logits consumer): a sequence of n_prompt tokens whose last score_len tokens are scored takes
the rows at key positions n_prompt - score_len - 1 .. n_prompt - 2; the row at position i
predicts the token at position i + 1, and its score is the log-softmax of the row's logits
over the whole vocabulary, read at that token. Logits are the dot products of the row's
hidden state with every unembedding row, here in float64.
"""

from __future__ import annotations

import numpy as np

from .attention import bf16_to_f64


class ScoringError(ValueError):
    pass


def score_rows(n_prompt: int, score_len: int):
    """(row positions, target positions) of a sequence scored on its last score_len tokens."""
    if not 1 <= score_len < n_prompt:
        raise ScoringError("score_len must be at least 1 and below the sequence length")
    lo, hi = n_prompt - score_len - 1, n_prompt - 2
    rows = list(range(lo, hi + 1))
    return rows, [i + 1 for i in rows]


def teacher_forced_logprobs(hidden, rows, targets, w_u):
    """log p(target | row) = z[target] - log(sum_v exp(z[v])) with z = W_U h_row, float64.

    hidden [T, d_model], w_u [vocab, d_model] (bf16 bits as uint16, or float); rows and
    targets are index lists of the same length."""
    hidden = np.asarray(hidden)
    w_u = np.asarray(w_u)
    conv = bf16_to_f64 if hidden.dtype == np.uint16 else (lambda a: np.asarray(a, np.float64))
    convw = bf16_to_f64 if w_u.dtype == np.uint16 else (lambda a: np.asarray(a, np.float64))
    vocab = w_u.shape[0]
    out = np.zeros(len(rows))
    for j, (r, t) in enumerate(zip(rows, targets)):
        if not 0 <= int(t) < vocab:
            raise ScoringError(f"target {int(t)} outside the vocabulary")
        h = conv(hidden[int(r)])
        z = np.zeros(vocab)
        for v0 in range(0, vocab, 8192):  # the vocabulary in slices, to bound memory
            z[v0:v0 + 8192] = convw(w_u[v0:v0 + 8192]) @ h
        m = z.max()
        out[j] = z[int(t)] - (m + np.log(np.exp(z - m).sum()))
    return out
