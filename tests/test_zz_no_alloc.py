"""blink_score_targets_noalloc, the scoring entry point that allocates nothing (its scratch is
the library's static device array), against blink_score_targets, which takes the caller's
workspace: two calls in a row on the 4B-like readout shapes (hidden 2560, vocab 151936), the
second with fewer rows than the first, each checked element by element against the workspace
form (the same kernels in the same order, so bit for bit) and against the FP64 oracle within
the scoring bar."""

import numpy as np
import pytest

import synth
from helpers import SCORE_TOL, device_bf16
from oracle.scoring import teacher_forced_logprobs

pytestmark = pytest.mark.gpu


def test_noalloc_matches_workspace_form_twice():
    import torch

    import pass_typed_decision_amd as blink

    rng = np.random.default_rng(2026)
    t_pad, d_model, vocab = 4096, 2560, 151936
    hidden = synth.f32_to_bf16_bits(rng.standard_normal((t_pad, d_model)).astype(np.float32))
    w_u = synth.f32_to_bf16_bits(
        (rng.standard_normal((vocab, d_model)) * 0.02).astype(np.float32))
    h, w = device_bf16(hidden), device_bf16(w_u)
    for n_rows in (256, 40):  # the 8-wave kernel form, then the 4-wave one on a smaller input
        print(f"no-alloc scoring: {n_rows} rows, vocab {vocab}", flush=True)
        rows = np.sort(rng.choice(t_pad, size=n_rows, replace=False)).astype(np.int64)
        targets = rng.integers(0, vocab, size=n_rows).astype(np.int32)
        sc = blink.TargetScorer(h, w, torch.as_tensor(rows).cuda(),
                                torch.as_tensor(targets).cuda())
        sc.logprob.fill_(float("nan"))
        ref_ws = sc.run().clone()
        sc.logprob.fill_(float("nan"))
        got = sc.run_noalloc()
        torch.cuda.synchronize()
        a, b = ref_ws.cpu().numpy(), got.cpu().numpy()
        assert np.isfinite(b).all()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        pick = [0, n_rows // 2, n_rows - 1]
        ref = teacher_forced_logprobs(hidden, rows[pick], targets[pick], w_u)
        err = float(np.abs(b[pick] - ref).max())
        print(f"  bitwise equal to the workspace form; oracle err {err:.2e}", flush=True)
        assert err <= SCORE_TOL
