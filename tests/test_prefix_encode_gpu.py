"""GPU parity of the shared prefix's own causal prefill (encode_prefix_attention, through the
C ABI) with the FP64 oracle, and of the shared path against the plain path.

The shared path encodes the prefix once and runs every tail against it; the plain path runs
each question's full sequence [prefix ; tail] on its own. The pages state that both see the
same tokens at the same positions and differ only in floating-point order: the tail rows of
the two paths must agree within the attention bar (max-abs 2e-2 against the oracle, and
against each other), and the prefix rows, which both compute over the same keys in the same
tile order, must agree bit for bit."""

from dataclasses import replace
from types import SimpleNamespace

import numpy as np
import pytest

import synth
from helpers import ATTN_TOL, Request, bf16_to_f32_host, device_bf16, run_attention
from oracle.attention import attention_full, attention_rows

pytestmark = pytest.mark.gpu


def _encode(q_bits, k_bits, v_bits, hq, scale):
    import torch

    import pass_typed_decision_amd as blink

    q, k, v = device_bf16(q_bits), device_bf16(k_bits), device_bf16(v_bits)
    out = torch.full_like(q, float("nan"))
    blink.encode_prefix_attention(q, k, v, out, scale)
    torch.cuda.synchronize()
    return bf16_to_f32_host(out)


def _prefix_inputs(cfg):
    req = Request(cfg, parts=("q", "k_tail", "v_tail", "k_prefix", "v_prefix"))
    return req, synth.draw_prefix_queries(cfg)


@pytest.mark.parametrize("number", [1, 2])
def test_encode_whole(number):
    cfg = synth.config(number)
    print(f"prefix encode parity, whole: config {number}, {cfg.prefix_len} tokens", flush=True)
    req, qp = _prefix_inputs(cfg)
    kp, vp = req.tensors["k_prefix"], req.tensors["v_prefix"]
    got = _encode(qp, kp, vp, cfg.n_heads_q, cfg.scale)
    ref = attention_full(qp, kp, vp, None, None, [0], [cfg.prefix_len], cfg.n_heads_q,
                         cfg.n_heads_kv, cfg.scale)
    err = np.abs(got - ref).max()
    print(f"  max abs err {err:.3e}", flush=True)
    assert np.isfinite(got).all() and err <= ATTN_TOL


@pytest.mark.parametrize("number", [3, 5])
def test_encode_sampled(number):
    cfg = synth.config(number, n_questions=1, tail_lo=1, tail_hi=1)
    print(f"prefix encode parity, sampled: config {number}, {cfg.prefix_len} tokens", flush=True)
    req, qp = _prefix_inputs(cfg)
    kp, vp = req.tensors["k_prefix"], req.tensors["v_prefix"]
    got = _encode(qp, kp, vp, cfg.n_heads_q, cfg.scale)
    rng = np.random.default_rng(number)
    p = cfg.prefix_len
    positions = sorted({0, 1, 63, 64, p - 1, *rng.integers(0, p, size=40).tolist()})
    samples = [(0, int(t), int(rng.integers(cfg.n_heads_q))) for t in positions]
    ref = attention_rows(qp, kp, vp, None, None, [0], [p], cfg.n_heads_q, cfg.n_heads_kv,
                         cfg.scale, samples)
    picked = np.stack([got[t, h] for _, t, h in samples])
    err = np.abs(picked - ref).max()
    print(f"  max abs err {err:.3e} over {len(samples)} sampled rows", flush=True)
    assert np.isfinite(got).all() and err <= ATTN_TOL


SHARED_VS_PLAIN = {
    "tiny": synth.config(1),
    "4b_like_small": synth.config(2, prefix_len=700, n_questions=5, tail_lo=30, tail_hi=140),
    "27b_like_small": synth.config(5, prefix_len=333, n_questions=3, tail_lo=50, tail_hi=200),
}


@pytest.mark.parametrize("name", sorted(SHARED_VS_PLAIN))
def test_shared_path_equals_plain_path(name):
    cfg = SHARED_VS_PLAIN[name]
    print(f"shared vs plain path: {name}", flush=True)
    req, qp = _prefix_inputs(cfg)
    ts, p = req.tensors, cfg.prefix_len
    # Shared path: the prefix once, then every tail against it.
    enc = _encode(qp, ts["k_prefix"], ts["v_prefix"], cfg.n_heads_q, cfg.scale)
    tails = run_attention(req)
    # Plain path: each question's whole sequence, no shared prefix.
    off, n_i = req.pack["token_offset"], req.tail_len
    full = {"q": [], "k_tail": [], "v_tail": []}
    for i in range(len(n_i)):
        rows = slice(int(off[i]), int(off[i]) + int(n_i[i]))
        full["q"].append(np.concatenate([qp, ts["q"][rows]]))
        full["k_tail"].append(np.concatenate([ts["k_prefix"], ts["k_tail"][rows]]))
        full["v_tail"].append(np.concatenate([ts["v_prefix"], ts["v_tail"][rows]]))
    full = {k: np.concatenate(v) for k, v in full.items()}
    lens = (n_i + p).astype(np.int32)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    plain_req = SimpleNamespace(cfg=replace(cfg, prefix_len=0), tensors=full, tail_len=lens,
                                pack={"token_offset": starts})
    plain = run_attention(plain_req)
    ref = attention_full(full["q"], full["k_tail"], full["v_tail"], None, None, starts, lens,
                         cfg.n_heads_q, cfg.n_heads_kv, cfg.scale)
    worst = 0.0
    for i in range(len(n_i)):
        s = int(starts[i])
        # prefix rows: the same keys in the same order on both paths
        np.testing.assert_array_equal(plain[s:s + p], enc)
        got_tail = tails[int(off[i]):int(off[i]) + int(n_i[i])]
        plain_tail = plain[s + p:s + p + int(n_i[i])]
        ref_tail = ref[s + p:s + p + int(n_i[i])]
        worst = max(worst, float(np.abs(got_tail - plain_tail).max()))
        assert np.abs(got_tail - ref_tail).max() <= ATTN_TOL
        assert np.abs(plain_tail - ref_tail).max() <= ATTN_TOL
        assert np.abs(got_tail - plain_tail).max() <= ATTN_TOL
    print(f"  shared vs plain tail rows: max abs diff {worst:.3e}", flush=True)
