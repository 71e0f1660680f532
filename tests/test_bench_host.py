"""bench.py's host-side parts, without a GPU: the one-GPU refusal and the attention FLOP count
that its roofline figure divides by the measured time."""
import importlib.util
import os
import subprocess
import sys

import numpy as np

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    run = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert run.returncode == 2
    assert "measures one GPU; --gpus 2 is not supported" in run.stderr
    assert run.stdout == ""


def test_attention_flops_counts_every_visible_key():
    # Each real tail row of question i at tail position t sees the P prefix keys and its own
    # tail keys 0..t; each (query head, row, key) pair is a QK^T dot product and a PV product
    # of head_dim multiply-adds each, 4 * head_dim FLOPs in all.
    bench = _bench()
    for number, tails in [(1, [1, 2, 17, 48]), (2, [64, 100, 256]), (4, [32, 255, 1])]:
        cfg = synth.config(number)
        pairs = 0
        for n in tails:
            for t in range(n):
                pairs += cfg.prefix_len + (t + 1)
        want = 4.0 * cfg.head_dim * cfg.n_heads_q * pairs
        assert bench.attention_flops(cfg, np.asarray(tails)) == want
