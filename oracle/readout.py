"""Oracle for the label readout (test infrastructure only).

Follows the blink.py page (thegovind/blink-4b):
  * "torch engine" section, _read: for every question take the hidden row of its last valid
    token, take the unembedding rows of its offered labels, and score each label by the dot
    product of the two in FP32 (here: float64);
  * "answer assembly" section, softmax: divide the label scores by the temperature, subtract
    the largest, exponentiate and normalise; answer_for picks the most probable label and
    breaks ties toward the earlier option;
  * "rendering" section, question_options and "constants the deployment sets": 1 to 255
    options per question;
  * "public entry point" section, decide: a temperature that is not positive is refused.

The argmax is taken on the scores (the softmax is monotone in them), first index on ties.
"""

from __future__ import annotations

import math

import numpy as np

from .attention import bf16_to_f64

MAX_OPTIONS = 255


class ReadoutError(ValueError):
    pass


def softmax_t(z, temperature):
    """Temperature softmax of one question's label scores, float64."""
    if not temperature > 0 or not math.isfinite(temperature):
        raise ReadoutError("temperature is not a positive finite number")
    zt = np.asarray(z, dtype=np.float64) / float(temperature)
    e = np.exp(zt - zt.max())
    return e / e.sum()


def label_readout(hidden, last_row, w_u, cand_ids, cand_off, temperature):
    """Returns (logits [sum K], probs [sum K], argmax [n]) in float64 / int.

    hidden   [T_pad, d_model] bf16 bits (uint16) or float
    last_row [n]   token index of each question's last valid token
    w_u      [vocab, d_model] bf16 bits or float (only the candidate rows are read)
    cand_ids [sum K], cand_off [n + 1]: the offered labels' token ids, CSR by question
    """
    n = len(last_row)
    cand_off = [int(x) for x in cand_off]
    if len(cand_off) != n + 1:
        raise ReadoutError("candidate offsets must have n + 1 entries")
    hidden = np.asarray(hidden)
    w_u = np.asarray(w_u)
    conv = bf16_to_f64 if hidden.dtype == np.uint16 else (lambda a: np.asarray(a, np.float64))
    convw = bf16_to_f64 if w_u.dtype == np.uint16 else (lambda a: np.asarray(a, np.float64))
    total = cand_off[-1]
    logits = np.zeros(total)
    probs = np.zeros(total)
    argmax = np.zeros(n, dtype=np.int64)
    for i in range(n):
        lo, hi = cand_off[i], cand_off[i + 1]
        if not 1 <= hi - lo <= MAX_OPTIONS:
            raise ReadoutError(f"question with {hi - lo} options; the limit is 1 to {MAX_OPTIONS}")
        ids = [int(c) for c in cand_ids[lo:hi]]
        if len(set(ids)) != len(ids):
            raise ReadoutError("label token ids collide")
        h = conv(hidden[int(last_row[i])])
        rows = convw(w_u[ids])
        z = rows @ h
        logits[lo:hi] = z
        probs[lo:hi] = softmax_t(z, temperature)
        argmax[i] = int(np.argmax(z))  # first index of the maximum
    return logits, probs, argmax


def label_rows(cand_ids, cand_off):
    """Distinct unembedding rows of an option table and the entries that use each.

    Follows the blink.py page, "torch engine" section, _read_batched: the distinct label
    token ids over the questions, in ascending order, each gathered once. Returns
    (row_id, row_first, row_entry): row_id [U] the distinct ids ascending; the flat option
    entries (positions in cand_ids) with id row_id[j] are row_entry[row_first[j]:row_first[j+1]],
    in ascending entry order.
    """
    cand_off = [int(x) for x in cand_off]
    ids = [int(c) for c in cand_ids[:cand_off[-1]]]
    row_id = sorted(set(ids))
    users = {t: [] for t in row_id}
    for e, t in enumerate(ids):
        users[t].append(e)
    row_first, row_entry = [0], []
    for t in row_id:
        row_entry.extend(users[t])
        row_first.append(len(row_entry))
    return row_id, row_first, row_entry


def label_readout_batched(hidden, last_row, w_u, cand_ids, cand_off, temperature):
    """The batched form of label_readout (blink.py page, "torch engine" section,
    _read_batched): every question's hidden row is scored against the distinct label rows
    once, and each option takes the score in its label's column. In exact arithmetic it
    equals label_readout; returns (logits, probs, argmax) like it."""
    n = len(last_row)
    cand_off = [int(x) for x in cand_off]
    if len(cand_off) != n + 1:
        raise ReadoutError("candidate offsets must have n + 1 entries")
    hidden = np.asarray(hidden)
    w_u = np.asarray(w_u)
    conv = bf16_to_f64 if hidden.dtype == np.uint16 else (lambda a: np.asarray(a, np.float64))
    convw = bf16_to_f64 if w_u.dtype == np.uint16 else (lambda a: np.asarray(a, np.float64))
    row_id, _, _ = label_rows(cand_ids, cand_off)
    col = {t: j for j, t in enumerate(row_id)}
    hs = np.stack([conv(hidden[int(r)]) for r in last_row])
    z_all = hs @ convw(w_u[row_id]).T  # [n, U]
    total = cand_off[-1]
    logits = np.zeros(total)
    probs = np.zeros(total)
    argmax = np.zeros(n, dtype=np.int64)
    for i in range(n):
        lo, hi = cand_off[i], cand_off[i + 1]
        if not 1 <= hi - lo <= MAX_OPTIONS:
            raise ReadoutError(f"question with {hi - lo} options; the limit is 1 to {MAX_OPTIONS}")
        ids = [int(c) for c in cand_ids[lo:hi]]
        if len(set(ids)) != len(ids):
            raise ReadoutError("label token ids collide")
        z = np.array([z_all[i, col[t]] for t in ids])
        logits[lo:hi] = z
        probs[lo:hi] = softmax_t(z, temperature)
        argmax[i] = int(np.argmax(z))
    return logits, probs, argmax
