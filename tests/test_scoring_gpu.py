"""GPU parity of blink_score_targets (teacher-forced scoring, through the C ABI) with the
FP64 oracle: log p(target | row) over the whole vocabulary.

Bar (derived; none is stated for this step): max-abs 1e-4 on the log-probabilities
(helpers.SCORE_TOL). Logits are FP32 sums of up to 5120 bf16 products (|z| ~ 1) and the
log-sum-exp over 151936 FP32 terms adds a relative error of about 1e-6, so the kernel stays
near 1e-6; a wrong row or target, or one 32-row vocabulary tile dropped from the log-sum-exp
(about 2e-4 at vocab 151936, shown on the oracle in test_oracle_scoring.py), exceeds the
bar."""

import numpy as np
import pytest

import synth
from helpers import SCORE_TOL as TOL
from helpers import device_bf16
from oracle.scoring import score_rows, teacher_forced_logprobs

pytestmark = pytest.mark.gpu


def _run(hidden_bits, w_bits, rows, targets):
    import torch

    import pass_typed_decision_amd as blink

    h, w = device_bf16(hidden_bits), device_bf16(w_bits)
    d_rows = torch.as_tensor(np.asarray(rows, np.int64)).cuda()
    d_t = torch.as_tensor(np.asarray(targets, np.int32)).cuda()
    sc = blink.TargetScorer(h, w, d_rows, d_t)
    out = sc.run()
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _case(seed, t_pad, d_model, vocab, n_seq, score_len):
    rng = np.random.default_rng(seed)
    hidden = synth.f32_to_bf16_bits(rng.standard_normal((t_pad, d_model)).astype(np.float32))
    w_u = synth.f32_to_bf16_bits((rng.standard_normal((vocab, d_model)) * 0.02).astype(np.float32))
    tokens = rng.integers(0, vocab, size=t_pad)
    rows, targets = [], []
    start = 0
    for _ in range(n_seq):  # sequences laid end to end, each scored on its last tokens
        n = int(rng.integers(score_len + 1, 3 * score_len + 3))
        if start + n > t_pad:
            break
        r, t = score_rows(n, score_len)
        rows += [start + i for i in r]
        targets += [int(tokens[start + i]) for i in t]
        start += n
    return hidden, w_u, rows, targets


@pytest.mark.parametrize("d_model, vocab, n_seq, score_len", [
    (256, 1000, 8, 4),      # vocabulary not a multiple of the 128-row slice
    (2560, 4096, 40, 8),    # more than one block of 256 scored rows
    (5120, 777, 5, 3),      # the 27B-like width
    (64, 129, 3, 1),        # one full slice and one row
])
def test_matches_oracle(d_model, vocab, n_seq, score_len):
    print(f"scoring parity: d_model {d_model}, vocab {vocab}", flush=True)
    hidden, w_u, rows, targets = _case(d_model + vocab, 2048, d_model, vocab, n_seq, score_len)
    got = _run(hidden, w_u, rows, targets)
    ref = teacher_forced_logprobs(hidden, rows, targets, w_u)
    err = float(np.abs(got - ref).max())
    print(f"  {len(rows)} rows, max abs err {err:.2e}", flush=True)
    assert np.isfinite(got).all() and err <= TOL


@pytest.mark.parametrize("d_model, n_seq", [
    (2560, 32),  # 4B-like width: 256 rows, the 256-row form
    (5120, 16),  # 27B-like width: 128 rows, the 128-row form
])
def test_full_vocabulary_sampled(d_model, n_seq):
    # vocab 151936; n_seq sequences scored on their last 8 tokens. The oracle checks the first
    # and last row of every 32-row tile of the call (every row group of 64 and both of its
    # tiles, both lane edges); the first two targets are the two ends of the vocabulary.
    hidden, w_u, rows, targets = _case(7, 8192, d_model, 151936, n_seq, 8)
    targets[0], targets[1] = 0, 151935
    got = _run(hidden, w_u, rows, targets)
    pick = sorted({1, *[i for k in range(0, len(rows), 32) for i in (k, min(k + 31, len(rows) - 1))]})
    ref = teacher_forced_logprobs(hidden, [rows[i] for i in pick], [targets[i] for i in pick], w_u)
    err = float(np.abs(got[pick] - ref).max())
    print(f"  {len(rows)} rows, {len(pick)} sampled, max abs err {err:.2e}", flush=True)
    assert np.isfinite(got).all() and err <= TOL
    assert (got <= 1e-6).all()  # log-probabilities of a distribution


def test_out_of_range_rows_and_targets_are_nan():
    hidden, w_u, rows, targets = _case(5, 512, 128, 300, 6, 2)
    rows[1] = 512  # past the hidden rows
    targets[2] = 300  # past the vocabulary
    targets[3] = -1
    got = _run(hidden, w_u, rows, targets)
    assert np.isnan(got[[1, 2, 3]]).all()
    good = [i for i in range(len(rows)) if i not in (1, 2, 3)]
    ref = teacher_forced_logprobs(hidden, [rows[i] for i in good], [targets[i] for i in good], w_u)
    assert np.abs(got[good] - ref).max() <= TOL
