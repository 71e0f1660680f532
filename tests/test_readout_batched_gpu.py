"""GPU parity of blink_label_readout_batched (through the C ABI): the batched readout over
the distinct label rows, against the FP64 oracle's batched readout, and bitwise against the
per-option readout (each logit is the same FP32 dot product in the same order).

Bar: probabilities and logits within 1e-4 (max-abs), argmax exact wherever the oracle's
top-2 gap exceeds 1e-5 (else one of the tied maxima)."""

import numpy as np
import pytest

import synth
from helpers import LOGIT_TOL, PROB_TOL, Request, check_argmax, run_readout
from oracle.readout import label_readout_batched

pytestmark = pytest.mark.gpu

READOUT_PARTS = ("hidden", "w_u")


def _check(req, got, ids, off, temperature=None):
    logits, probs, arg = got
    last = req.pack["last_row"]
    t = req.cfg.temperature if temperature is None else temperature
    z, p, a = label_readout_batched(req.tensors["hidden"], last, req.tensors["w_u"], ids, off, t)
    assert np.abs(logits - z).max() <= LOGIT_TOL
    assert np.abs(probs - p).max() <= PROB_TOL
    for i in range(len(last)):
        assert abs(probs[off[i]:off[i + 1]].sum() - 1.0) <= 1e-5
    ties = check_argmax(z, off, a, arg)
    print(f"  logits err {np.abs(logits - z).max():.2e} probs err {np.abs(probs - p).max():.2e} "
          f"near-ties {ties}", flush=True)


def _same_as_per_option(req, got, **kw):
    ref = run_readout(req, **kw)
    for a, b in zip(got, ref):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("number", [1, 2, 3, 4, 5])
def test_full_size(number):
    cfg = synth.config(number)
    print(f"batched readout parity: config {number}", flush=True)
    req = Request(cfg, parts=READOUT_PARTS)
    got = run_readout(req, batched=True)
    _check(req, got, req.tables.cand_ids, req.tables.cand_off)
    _same_as_per_option(req, got)


@pytest.mark.parametrize("questions", [64, 512])
def test_shared_label_table(questions):
    # The pages' own layout: every question uses the first K_i entries of one label table, so
    # each distinct row is offered by many questions.
    cfg = synth.config(4, n_questions=questions)
    req = Request(cfg, parts=READOUT_PARTS)
    table = np.random.default_rng(9).choice(cfg.vocab, 255, replace=False).astype(np.int32)
    ids = np.concatenate([table[:x] for x in req.tables.n_options]).astype(np.int32)
    got = run_readout(req, cand_ids=ids, batched=True)
    _check(req, got, ids, req.tables.cand_off)
    _same_as_per_option(req, got, cand_ids=ids)


def test_one_and_255_options():
    cfg = synth.config(2, n_questions=90)
    req = Request(cfg, parts=READOUT_PARTS)
    rng = np.random.default_rng(5)
    ids, counts = [], []
    for _ in range(30):
        for k in (1, 255, 7):
            ids.append(rng.choice(cfg.vocab, k, replace=False))
            counts.append(k)
    ids = np.concatenate(ids).astype(np.int32)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    got = run_readout(req, cand_ids=ids, cand_off=off, batched=True)
    for i in range(0, len(counts), 3):
        assert got[1][off[i]] == 1.0 and got[2][i] == 0
    _check(req, got, ids, off)


@pytest.mark.parametrize("temperature", [0.05, 3.0])
def test_temperatures(temperature):
    req = Request(synth.config(4), parts=READOUT_PARTS)
    got = run_readout(req, temperature=temperature, batched=True)
    _check(req, got, req.tables.cand_ids, req.tables.cand_off, temperature=temperature)


def test_out_of_range_row_is_flagged():
    import pass_typed_decision_amd as blink

    cfg = synth.config(4, n_questions=64)
    req = Request(cfg, parts=READOUT_PARTS)
    ids, off = req.tables.cand_ids, req.tables.cand_off
    lr = blink.pack_labels(ids, off, cfg.vocab)
    row_id = lr.row_id.copy()
    bad_id = int(ids[off[3]])  # a row question 3 offers
    j = int(np.searchsorted(row_id, bad_id))
    row_id[j] = cfg.vocab + 11
    users = set(int(e) for e in lr.row_entry[lr.row_first[j]:lr.row_first[j + 1]])
    hit = sorted({int(np.searchsorted(off, e, side="right") - 1) for e in users})
    logits, probs, arg = run_readout(req, batched=True,
                                     row_tables=(row_id, lr.row_first, lr.row_entry))
    z, p, a = label_readout_batched(req.tensors["hidden"], req.pack["last_row"],
                                    req.tensors["w_u"], ids, off, cfg.temperature)
    for i in range(len(off) - 1):
        lo, hi = off[i], off[i + 1]
        if i in hit:
            assert arg[i] == -1 and np.isnan(probs[lo:hi]).all()
        else:
            np.testing.assert_allclose(probs[lo:hi], p[lo:hi], atol=PROB_TOL)
    assert 3 in hit
