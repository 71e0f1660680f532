"""GPU parity of blink_label_readout (through the C ABI) with the FP64 oracle.

Bar: label probabilities within 1e-4 (max-abs), logits within 1e-4, argmax exact wherever the
oracle's top-2 gap exceeds 1e-5 (else one of the tied maxima). All five workloads at full
size, plus edge cases (1 and 255 options, temperature, malformed tables), and the launch forms
against one another: small tables take one fused launch; large ones the streaming pair, or,
when questions number at least twice the compute units and none is longer than about one
unit's share of the rows (the plain max packing table on a 256-CU part), one ranked launch
that hands out the longest questions first. The forms give bitwise the same results."""

import numpy as np
import pytest

import synth
from helpers import LOGIT_TOL, PROB_TOL, Request, check_argmax, device_bf16, run_readout
from oracle.readout import label_readout

pytestmark = pytest.mark.gpu

READOUT_PARTS = ("hidden", "w_u")


def _check(req, logits, probs, arg, ids=None, off=None, last=None, temperature=None):
    ids = req.tables.cand_ids if ids is None else ids
    off = req.tables.cand_off if off is None else off
    last = req.pack["last_row"] if last is None else last
    t = req.cfg.temperature if temperature is None else temperature
    z, p, a = label_readout(req.tensors["hidden"], last, req.tensors["w_u"], ids, off, t)
    assert np.abs(logits - z).max() <= LOGIT_TOL
    assert np.abs(probs - p).max() <= PROB_TOL
    for i in range(len(last)):
        assert abs(probs[off[i]:off[i + 1]].sum() - 1.0) <= 1e-5
    ties = check_argmax(z, off, a, arg)
    print(f"  logits err {np.abs(logits - z).max():.2e} probs err {np.abs(probs - p).max():.2e} "
          f"near-ties {ties}", flush=True)


@pytest.mark.parametrize("number", [1, 2, 3, 4, 5])
def test_full_size(number):
    cfg = synth.config(number)
    print(f"readout parity: config {number}", flush=True)
    req = Request(cfg, parts=READOUT_PARTS)
    logits, probs, arg = run_readout(req)
    _check(req, logits, probs, arg)


# Small tables take the fused one-launch kernel; large ones (over 32 MiB of label rows) the
# streaming kernel plus a softmax kernel. Both must meet the same bar on the same edge cases.
@pytest.mark.parametrize("repeat", [1, 30], ids=["fused", "streaming"])
def test_one_and_255_options(repeat):
    cfg = synth.config(2, n_questions=3 * repeat)
    req = Request(cfg, parts=READOUT_PARTS)
    rng = np.random.default_rng(5)
    ids, counts = [], []
    for _ in range(repeat):
        for k in (1, 255, 7):
            ids.append(rng.choice(cfg.vocab, k, replace=False))
            counts.append(k)
    ids = np.concatenate(ids).astype(np.int32)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    assert (len(ids) * cfg.d_model * 2 > 32 << 20) == (repeat > 1)
    logits, probs, arg = run_readout(req, cand_ids=ids, cand_off=off)
    for i in range(0, len(counts), 3):
        assert probs[off[i]] == 1.0 and arg[i] == 0
    _check(req, logits, probs, arg, ids=ids, off=off)


@pytest.mark.parametrize("temperature", [0.05, 0.7, 3.0])
def test_temperatures(temperature):
    req = Request(synth.config(2), parts=READOUT_PARTS)
    logits, probs, arg = run_readout(req, temperature=temperature)
    _check(req, logits, probs, arg, temperature=temperature)


def test_shared_label_table():
    # The pages' own layout: every question uses the first K_i entries of one label table.
    cfg = synth.config(4, n_questions=64)
    req = Request(cfg, parts=READOUT_PARTS)
    table = np.random.default_rng(9).choice(cfg.vocab, 255, replace=False).astype(np.int32)
    k = req.tables.n_options
    ids = np.concatenate([table[:x] for x in k]).astype(np.int32)
    logits, probs, arg = run_readout(req, cand_ids=ids)
    _check(req, logits, probs, arg, ids=ids)


@pytest.mark.parametrize("number,n_questions", [(1, None), (4, None), (4, 300)],
                         ids=["fused", "ranked", "streaming"])
def test_malformed_entries_are_flagged(number, n_questions):
    cfg = synth.config(number) if n_questions is None else synth.config(number,
                                                                        n_questions=n_questions)
    req = Request(cfg, parts=READOUT_PARTS)
    ids = req.tables.cand_ids.copy()
    ids[req.tables.cand_off[1]] = cfg.vocab + 5  # question 1: id out of range
    last = np.asarray(req.pack["last_row"], np.int64).copy()
    last[2] = -3  # question 2: row out of range
    assert (len(ids) * cfg.d_model * 2 > 32 << 20) == (number == 4)
    logits, probs, arg = run_readout(req, cand_ids=ids, last_row=last)
    off = req.tables.cand_off
    assert arg[1] == -1 and arg[2] == -1
    assert np.isnan(probs[off[1]:off[2]]).all() and np.isnan(probs[off[2]:off[3]]).all()
    assert np.isnan(logits[off[1]:off[2]]).all() and np.isnan(logits[off[2]:off[3]]).all()
    z, p, a = label_readout(req.tensors["hidden"], req.pack["last_row"], req.tensors["w_u"],
                            req.tables.cand_ids, off, cfg.temperature)
    good = [0] + list(range(3, len(off) - 1))
    for i in good:
        np.testing.assert_allclose(probs[off[i]:off[i + 1]], p[off[i]:off[i + 1]], atol=PROB_TOL)
        np.testing.assert_allclose(logits[off[i]:off[i + 1]], z[off[i]:off[i + 1]], atol=LOGIT_TOL)
    sub_off = np.concatenate([[0], np.cumsum([off[i + 1] - off[i] for i in good])])
    sub = np.concatenate([np.arange(off[i], off[i + 1]) for i in good])
    check_argmax(z[sub], sub_off, a[good], arg[good])


def _read_in_parts(req, ids, off, parts):
    """The same questions read in `parts` calls of consecutive questions; results joined."""
    n = len(off) - 1
    last = np.asarray(req.pack["last_row"], np.int64)
    out = [[], [], []]
    for p in range(parts):
        q0, q1 = n * p // parts, n * (p + 1) // parts
        got = run_readout(req, last_row=last[q0:q1], cand_ids=ids[off[q0]:off[q1]],
                          cand_off=(off[q0:q1 + 1] - off[q0]).astype(np.int32))
        for acc, x in zip(out, got):
            acc.append(x)
    return [np.concatenate(x) for x in out]


@pytest.mark.parametrize("counts", ["mixed", "equal"])
def test_ranked_and_streaming_forms_agree_bitwise(counts):
    # 512 questions read whole (the ranked launch on a 256-CU part) and as two calls of 256
    # (the streaming pair there): each question's results depend on its own rows only, so
    # the two must agree bit for bit. "mixed": the workload's 2..255 options (many equal
    # counts, so the rank's ties by index are exercised); "equal": 200 options everywhere.
    cfg = synth.config(4)
    req = Request(cfg, parts=READOUT_PARTS)
    ids, off = req.tables.cand_ids, req.tables.cand_off
    if counts == "equal":
        n = cfg.n_questions
        rng = np.random.default_rng(21)
        ids = np.concatenate([rng.choice(cfg.vocab, 200, replace=False)
                              for _ in range(n)]).astype(np.int32)
        off = (np.arange(n + 1) * 200).astype(np.int32)
    assert len(ids) * cfg.d_model * 2 > 32 << 20
    whole = run_readout(req, cand_ids=ids, cand_off=off)
    halves = _read_in_parts(req, ids, off, 2)
    for a, b in zip(whole, halves):
        np.testing.assert_array_equal(a, b)
    if counts == "equal":
        _check(req, *whole, ids=ids, off=off)


def test_ranked_form_at_hidden_5120():
    # The plain max-packing option mix at hidden 5120: the ranked form's 8-wave workgroups (a
    # 5120-wide row leaves too few registers for 16 waves), bitwise against the streaming pair
    # and, on the longest and some other questions, against the oracle. Short tails and a
    # 16384-row vocabulary keep the inputs small; the table is still far above the one-launch
    # small-table size.
    cfg = synth.config(4, d_model=5120, vocab=16384)
    req = Request(cfg, parts=READOUT_PARTS, tail_len=np.full(cfg.n_questions, 8, np.int32))
    ids, off = req.tables.cand_ids, req.tables.cand_off
    assert len(ids) * cfg.d_model * 2 > 32 << 20
    whole = run_readout(req)
    halves = _read_in_parts(req, ids, off, 2)
    for a, b in zip(whole, halves):
        np.testing.assert_array_equal(a, b)
    k = np.diff(off)
    pick = sorted(set(np.argsort(-k, kind="stable")[:8].tolist()) | {0, 1, 255, 256, 510, 511})
    last = np.asarray(req.pack["last_row"], np.int64)
    sub_ids = np.concatenate([ids[off[i]:off[i + 1]] for i in pick])
    sub_off = np.concatenate([[0], np.cumsum([k[i] for i in pick])])
    z, p, o_arg = label_readout(req.tensors["hidden"], last[pick], req.tensors["w_u"], sub_ids,
                                sub_off, cfg.temperature)
    sub = np.concatenate([np.arange(off[i], off[i + 1]) for i in pick])
    logits, probs, arg = whole
    assert np.abs(logits[sub] - z).max() <= LOGIT_TOL
    assert np.abs(probs[sub] - p).max() <= PROB_TOL
    check_argmax(z, sub_off, o_arg, arg[pick])


def test_unusable_offsets_in_a_ranked_launch():
    # Questions whose offsets cannot be used (more options than max_options, none, or an end
    # past the table) rank last in the ranked launch, get argmax -1, and every other question
    # is still read once and matches the oracle.
    cfg = synth.config(4)
    req = Request(cfg, parts=READOUT_PARTS)
    ids = req.tables.cand_ids
    off = req.tables.cand_off.astype(np.int64).copy()
    k = np.diff(off)
    n, total = len(k), int(off[-1])
    a = int(np.nonzero(k[:-1] + k[1:] > 255)[0][0])
    off[a + 1] = off[a + 2]  # question a: over 255 options; question a + 1: none
    b = int(np.nonzero((k[a + 3:-2] + k[a + 4:-1]) <= 255)[0][0]) + a + 3
    off[b + 1] = off[b]  # question b: none; question b + 1 takes its rows
    off[n] = total + 1  # question n - 1 ends past the table
    bad = [a, a + 1, b, n - 1]
    d_off = off.astype(np.int32)
    d_off_ok = d_off.copy()
    d_off_ok[n] = total
    logits, probs, arg = run_readout(req, cand_off=d_off, max_options=255)
    assert (arg[bad] == -1).all()
    good = [i for i in range(n) if i not in bad]
    last = np.asarray(req.pack["last_row"], np.int64)
    z, p, o_arg = label_readout(req.tensors["hidden"], last[good], req.tensors["w_u"],
                                np.concatenate([ids[d_off_ok[i]:d_off_ok[i + 1]] for i in good]),
                                np.concatenate([[0], np.cumsum([d_off_ok[i + 1] - d_off_ok[i]
                                                                for i in good])]),
                                cfg.temperature)
    sub = np.concatenate([np.arange(d_off_ok[i], d_off_ok[i + 1]) for i in good])
    assert np.abs(logits[sub] - z).max() <= LOGIT_TOL
    assert np.abs(probs[sub] - p).max() <= PROB_TOL
    sub_off = np.concatenate([[0], np.cumsum([d_off_ok[i + 1] - d_off_ok[i] for i in good])])
    check_argmax(z, sub_off, o_arg, arg[good])


def test_every_question_unusable_in_a_ranked_launch():
    # Every question's offsets unusable (none with options, the last with them all): all rank
    # equal at 0 options, every workgroup still finds its own question, and each gets argmax -1
    # with nothing else written.
    import torch

    import pass_typed_decision_amd as blink

    cfg = synth.config(4)
    req = Request(cfg, parts=READOUT_PARTS)
    ids = req.tables.cand_ids
    n, total = cfg.n_questions, len(ids)
    off = np.zeros(n + 1, np.int32)
    off[n] = total
    hidden, w_u = device_bf16(req.tensors["hidden"]), device_bf16(req.tensors["w_u"])
    d_last = torch.as_tensor(np.asarray(req.pack["last_row"], np.int64)).cuda()
    logits = torch.full((total,), 7.0, device="cuda")
    probs = torch.full((total,), 7.0, device="cuda")
    arg = torch.zeros(n, dtype=torch.int32, device="cuda")
    blink.label_readout(hidden, d_last, w_u, torch.as_tensor(ids).cuda(),
                        torch.as_tensor(off).cuda(), cfg.temperature, 255, logits, probs, arg)
    torch.cuda.synchronize()
    assert (arg.cpu().numpy() == -1).all()
    assert (logits.cpu().numpy() == 7.0).all() and (probs.cpu().numpy() == 7.0).all()


def test_rotations_through_the_readout():
    # Each question is read in three rotations of its option order (each rotation a question
    # of its own in one readout call); the GPU logits, combined per key on the host, must
    # match the same combination of the FP64 oracle's logits.
    import pass_typed_decision_amd as blink
    from oracle.readout import label_readout as oracle_readout
    from oracle.refine import combine_rotations as oracle_combine

    cfg = synth.config(2)
    req = Request(cfg, parts=READOUT_PARTS)
    ids, off = req.tables.cand_ids, req.tables.cand_off
    last = np.asarray(req.pack["last_row"], np.int64)
    n = len(off) - 1
    r_ids, r_last, r_counts, passes_meta = [], [], [], []
    for i in range(n):
        k = int(off[i + 1] - off[i])
        for r in range(3):
            order = [(r + j) % k for j in range(k)]
            r_ids.extend(int(ids[off[i] + o]) for o in order)
            r_last.append(int(last[i]))
            r_counts.append(k)
            passes_meta.append((i, order))
    r_off = np.concatenate([[0], np.cumsum(r_counts)]).astype(np.int32)
    r_ids = np.asarray(r_ids, np.int32)
    logits, _, _ = run_readout(req, last_row=np.asarray(r_last, np.int64), cand_ids=r_ids,
                               cand_off=r_off)
    z, _, _ = oracle_readout(req.tensors["hidden"], r_last, req.tensors["w_u"], r_ids, r_off,
                             cfg.temperature)
    n_keys = np.diff(off).tolist()
    gpu_passes = [(q, order, logits[r_off[p]:r_off[p + 1]])
                  for p, (q, order) in enumerate(passes_meta)]
    ref_passes = [(q, order, z[r_off[p]:r_off[p + 1]]) for p, (q, order) in enumerate(passes_meta)]
    got = blink.combine_rotations(n_keys, gpu_passes)
    ref = oracle_combine(n_keys, ref_passes)
    err = max(float(np.abs(g - np.asarray(r)).max()) for g, r in zip(got, ref))
    print(f"  rotations of {n} questions: max abs err {err:.2e}", flush=True)
    assert err <= LOGIT_TOL
