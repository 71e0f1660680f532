"""GPU parity of blink_prefix_tail_attention (through the C ABI) with the FP64 oracle.

Bar: max-abs 2e-2 on the bf16 outputs of every real row. Reduced variants of all five
workloads run whole against the oracle (several tiles, ragged tails, GQA 4 and 5, with and
without a prefix), and reduced requests that take the key split of the last round; the full-size
workloads are launched exactly as the bench launches them and
checked whole (4B-like, plain max packing) or at the first and last row of every unit of work
of the launch (long document, 27B-like). Invariants (padding content, batch composition, head permutation)
must hold bit for bit."""

import numpy as np
import pytest

import synth
from helpers import (ATTN_TOL, Request, attention_split, run_attention, sample_rows, unit_samples,
                     valid_rows)
from oracle.attention import attention_full, attention_rows

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny_full": synth.config(1),
    "4b_like_small": synth.config(2, prefix_len=700, n_questions=6, tail_lo=30, tail_hi=140),
    "long_document_small": synth.config(3, prefix_len=1000, n_questions=5, tail_lo=100, tail_hi=300),
    "plain_small": synth.config(4, n_questions=40, tail_lo=1, tail_hi=70),
    "27b_like_small": synth.config(5, prefix_len=333, n_questions=3, tail_lo=50, tail_hi=200),
    "one_question_one_token": synth.config(1, prefix_len=1, n_questions=1, tail_lo=1, tail_hi=1),
    "plain_single_tokens": synth.config(4, n_questions=7, tail_lo=1, tail_hi=1),
    "prefix_one_tile": synth.config(2, prefix_len=64, n_questions=3, tail_lo=63, tail_hi=65),
    "d64_group1": synth.config(1, n_heads_q=2, n_heads_kv=2, prefix_len=129, n_questions=9,
                               tail_lo=1, tail_hi=40),
    "d128_group8": synth.config(2, n_heads_q=16, n_heads_kv=2, prefix_len=90, n_questions=5,
                                tail_lo=20, tail_hi=90),
    # No prefix at head_dim 64: the second build of the kernel (prefix-free short tails).
    "plain_d64": synth.config(1, prefix_len=0, n_questions=12, tail_lo=1, tail_hi=90),
}


def _oracle(req):
    cfg, ts = req.cfg, req.tensors
    return attention_full(ts["q"], ts["k_tail"], ts["v_tail"], ts.get("k_prefix"),
                          ts.get("v_prefix"), req.pack["token_offset"], req.tail_len,
                          cfg.n_heads_q, cfg.n_heads_kv, cfg.scale)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_matches_oracle_whole(name):
    cfg = SMALL[name]
    print(f"attention parity: {name} {cfg}", flush=True)
    req = Request(cfg, parts=("q", "k_tail", "v_tail", "k_prefix", "v_prefix"))
    got = run_attention(req)
    ref = _oracle(req)
    rows = valid_rows(req)
    assert np.isfinite(got[rows]).all()
    err = np.abs(got[rows] - ref[rows]).max()
    print(f"  max abs err {err:.3e} over {rows.size} rows", flush=True)
    assert err <= ATTN_TOL


def _max_err_by_question(req, got, ref):
    """Largest |got - ref| over every real row and head, one question at a time."""
    err = 0.0
    for i, n in enumerate(req.tail_len):
        o = int(req.pack["token_offset"][i])
        part = got[o:o + int(n)]
        assert np.isfinite(part).all(), f"question {i} has a row that was not written"
        err = max(err, float(np.abs(part - ref[o:o + int(n)]).max()))
    return err


@pytest.mark.parametrize("number", [2, 4])
def test_full_size_whole(number):
    # The 4B-like request (448 workgroups, more than one round) and plain max packing (6392
    # workgroups, re-cut last round, three packer batches), launched exactly as the bench
    # launches them, compared with the oracle on every real row and head.
    cfg = synth.config(number)
    print(f"attention full-size whole parity: config {number}", flush=True)
    req = Request(cfg, parts=("q", "k_tail", "v_tail", "k_prefix", "v_prefix"))
    got = run_attention(req)
    ref = _oracle(req)
    err = _max_err_by_question(req, got, ref)
    print(f"  max abs err {err:.3e} over {int(np.sum(req.tail_len))} tokens x "
          f"{cfg.n_heads_q} heads", flush=True)
    assert err <= ATTN_TOL


@pytest.mark.parametrize("number", [3, 5])
def test_full_size_every_unit(number):
    # The long-document and 27B-like requests are too large for a whole FP64 comparison, so
    # the oracle checks the first and last row of every unit of work of the launch (each KV
    # head), the re-cut last-round units included, plus both ends of every tail.
    import torch

    cfg = synth.config(number)
    print(f"attention full-size parity at every unit: config {number}", flush=True)
    req = Request(cfg, parts=("q", "k_tail", "v_tail", "k_prefix", "v_prefix"))
    got = run_attention(req)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    samples = unit_samples(req, cus)
    ts = req.tensors
    ref = attention_rows(ts["q"], ts["k_tail"], ts["v_tail"], ts.get("k_prefix"),
                         ts.get("v_prefix"), req.pack["token_offset"], req.tail_len,
                         cfg.n_heads_q, cfg.n_heads_kv, cfg.scale, samples)
    off = req.pack["token_offset"]
    picked = np.stack([got[off[i] + t, h] for i, t, h in samples])
    err = np.abs(picked - ref).max()
    print(f"  max abs err {err:.3e} over {len(samples)} rows ({cus} CUs)", flush=True)
    assert np.isfinite(picked).all() and err <= ATTN_TOL
    # every real row was written (the output starts as NaN)
    assert np.isfinite(got[valid_rows(req)]).all()


# Launches that take the key split of the last round (with a workspace): the 384-row units left
# after the full rounds run as 2, 4 or 5 pieces over runs of prefix tiles (ragged last tile, the
# tail in the last piece only), and a merge pass joins their partial results. Sized so that each
# lands in the split at 256 CUs; whole output against the oracle, and within the bar of the
# unsplit launch of the same request.
SPLIT = {
    "ways2_d128": synth.config(5, prefix_len=1000, n_questions=12, tail_lo=250, tail_hi=330),
    "ways4_d128": synth.config(5, prefix_len=900, n_questions=10, tail_lo=280, tail_hi=320),
    "ways5_d128": synth.config(5, prefix_len=1500, n_questions=10, tail_lo=265, tail_hi=300),
    "ways4_d64_group4": synth.config(1, n_heads_q=16, n_heads_kv=4, prefix_len=700,
                                     n_questions=200, tail_lo=30, tail_hi=45),
}


@pytest.mark.parametrize("name", sorted(SPLIT))
def test_key_split_matches_oracle_whole(name):
    import torch

    import pass_typed_decision_amd as blink

    cfg = SPLIT[name]
    req = Request(cfg, parts=("q", "k_tail", "v_tail", "k_prefix", "v_prefix"))
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tokens = int(np.sum(req.tail_len))
    group = cfg.n_heads_q // cfg.n_heads_kv
    plan = attention_split(tokens * group, cfg.n_heads_kv, cus, cfg.prefix_len)
    print(f"attention key split: {name} ({tokens} tokens, {cus} CUs) plan {plan}", flush=True)
    assert plan is not None, "the request no longer lands in the key split"
    assert blink.attention_workspace(tokens, cfg.n_heads_q, cfg.n_heads_kv, cfg.head_dim,
                                     cfg.prefix_len) is not None
    got = run_attention(req)
    ref = _oracle(req)
    err = _max_err_by_question(req, got, ref)
    plain = run_attention(req, workspace=None)
    rows = valid_rows(req)
    gap = float(np.abs(got[rows] - plain[rows]).max())
    print(f"  max abs err {err:.3e}; split vs unsplit {gap:.3e}", flush=True)
    assert err <= ATTN_TOL and gap <= ATTN_TOL


def test_workspace_query_matches_the_split_plan():
    # The library's workspace size is what the key split of the last round needs on this
    # device (none when it does not split): pieces x KV heads x 12 waves x 64 lanes x
    # (D / 2 + 2) floats.
    import torch

    import pass_typed_decision_amd as blink

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rng = np.random.default_rng(11)
    cases = [(10864, 40, 8, 128, 65536), (5338, 32, 8, 128, 2048), (3242, 40, 8, 128, 1500),
             (6258, 16, 4, 64, 2900), (74705, 32, 8, 128, 0)]
    for _ in range(200):
        hkv = int(rng.choice([1, 2, 4, 8]))
        hq = hkv * int(rng.integers(1, 9))
        cases.append((int(rng.integers(1, 60000)), hq, hkv, int(rng.choice([64, 128])),
                      int(rng.integers(0, 70000))))
    for tokens, hq, hkv, d, p in cases:
        plan = attention_split(tokens * (hq // hkv), hkv, cus, p)
        ws = blink.attention_workspace(tokens, hq, hkv, d, p)
        if plan is None:
            assert ws is None, (tokens, hq, hkv, d, p)
        else:
            _, left, ways, _ = plan
            assert ws is not None and ws.is_cuda
            assert ws.numel() == left * ways * hkv * 12 * 64 * (d // 2 + 2) * 4


def test_undersized_workspace_falls_back_to_the_row_split():
    # A workspace smaller than the query asks for is not used: the launch keeps the row
    # re-cut, exactly as with none.
    import torch

    import pass_typed_decision_amd as blink

    cfg = SPLIT["ways2_d128"]
    req = Request(cfg, parts=("q", "k_tail", "v_tail", "k_prefix", "v_prefix"))
    tokens = int(np.sum(req.tail_len))
    full = blink.attention_workspace(tokens, cfg.n_heads_q, cfg.n_heads_kv, cfg.head_dim,
                                     cfg.prefix_len)
    assert full is not None
    short = torch.zeros(full.numel() - 16, dtype=torch.uint8, device="cuda")
    got = run_attention(req, workspace=short)
    plain = run_attention(req, workspace=None)
    rows = valid_rows(req)
    np.testing.assert_array_equal(got[rows], plain[rows])


# The largest context the boundary accepts (prefix + tail = 131072 tokens): one question whose
# tail is the whole context with no prefix (2048 tiles of causal tail attention, as when the
# prefix itself is encoded), and the longest prefix with a one-token tail.
MAXIMUM = {
    "tail_131072_no_prefix": synth.config(4, n_questions=1, tail_lo=131072, tail_hi=131072),
    "prefix_131071_tail_1": synth.config(2, prefix_len=131071, n_questions=1, tail_lo=1,
                                         tail_hi=1),
}


@pytest.mark.parametrize("name", sorted(MAXIMUM))
def test_maximum_context_sampled(name):
    cfg = MAXIMUM[name]
    print(f"attention at the maximum context: {name}", flush=True)
    req = Request(cfg, parts=("q", "k_tail", "v_tail", "k_prefix", "v_prefix"))
    got = run_attention(req)
    samples = sample_rows(req, 24, seed=11)
    ts = req.tensors
    ref = attention_rows(ts["q"], ts["k_tail"], ts["v_tail"], ts.get("k_prefix"),
                         ts.get("v_prefix"), req.pack["token_offset"], req.tail_len,
                         cfg.n_heads_q, cfg.n_heads_kv, cfg.scale, samples)
    off = req.pack["token_offset"]
    picked = np.stack([got[off[i] + t, h] for i, t, h in samples])
    err = np.abs(picked - ref).max()
    print(f"  max abs err {err:.3e} over {len(samples)} sampled rows", flush=True)
    assert np.isfinite(picked).all() and err <= ATTN_TOL
    assert np.isfinite(got[valid_rows(req)]).all()


def test_padding_content_is_never_read():
    cfg = SMALL["4b_like_small"]
    req = Request(cfg, parts=("q", "k_tail", "v_tail", "k_prefix", "v_prefix"))
    a = run_attention(req)
    rows = valid_rows(req)
    pad = np.ones(req.pack["total_padded_tokens"], bool)
    pad[rows] = False
    assert pad.any()
    ts = {k: v.copy() for k, v in req.tensors.items()}
    big = synth.f32_to_bf16_bits(np.array([300.0], np.float32))[0]
    for name in ("q", "k_tail", "v_tail"):
        ts[name][pad] = big
    b = run_attention(req, tensors=ts)
    np.testing.assert_array_equal(a[rows], b[rows])


def test_question_alone_is_bitwise_identical():
    # Launches without a workspace: a row's result does not depend on the rest of the batch.
    # (With one, rows in key-split units are summed in another order: equal up to rounding.)
    cfg = SMALL["4b_like_small"]
    req = Request(cfg, parts=("q", "k_tail", "v_tail", "k_prefix", "v_prefix"))
    packed = run_attention(req, workspace=None)
    for i in range(len(req.tail_len)):
        off, n = req.pack["token_offset"][i], int(req.tail_len[i])
        alone_ts = dict(req.tensors)
        for name in ("q", "k_tail", "v_tail"):
            alone_ts[name] = np.ascontiguousarray(req.tensors[name][off:off + n])
        alone = run_attention(req, tensors=alone_ts, token_offset=[0], tail_len=[n],
                              workspace=None)
        np.testing.assert_array_equal(alone, packed[off:off + n])


def test_head_permutation_within_group():
    cfg = SMALL["27b_like_small"]
    req = Request(cfg, parts=("q", "k_tail", "v_tail", "k_prefix", "v_prefix"))
    a = run_attention(req)
    g = cfg.n_heads_q // cfg.n_heads_kv
    perm = np.concatenate([np.roll(np.arange(k * g, (k + 1) * g), 2) for k in range(cfg.n_heads_kv)])
    ts = dict(req.tensors, q=np.ascontiguousarray(req.tensors["q"][:, perm]))
    b = run_attention(req, tensors=ts)
    rows = valid_rows(req)
    np.testing.assert_array_equal(a[rows][:, perm], b[rows])


def test_out_of_range_offsets_are_skipped_not_faulted():
    cfg = SMALL["tiny_full"]
    req = Request(cfg, parts=("q", "k_tail", "v_tail", "k_prefix", "v_prefix"))
    good = run_attention(req)
    offs = np.asarray(req.pack["token_offset"], np.int64).copy()
    offs[1] = 10 ** 9  # far outside the buffer
    got = run_attention(req, token_offset=offs)
    for i in range(len(req.tail_len)):
        o, n = req.pack["token_offset"][i], int(req.tail_len[i])
        if i == 1:
            continue
        np.testing.assert_array_equal(got[o:o + n], good[o:o + n])


def _shift(bits, delta):
    return synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(bits) + np.float32(delta))


def _fill(value, shape):
    return synth.f32_to_bf16_bits(np.full(shape, value, np.float32))


# Score-range extremes. A question's queries of KV group 0 are shifted by +1 and one key of
# that group is set to a constant c, so that key's score is about c * D * scale above the
# typical ones (c = 6: ~68 nats, past what the kernel's fixed-reference softmax covers, so its
# exact two-pass recomputation must take over; c = 3: ~34 nats, inside it). The key sits late
# in the prefix, early in the prefix, or inside the question's own tail; only some questions are
# shifted, so shifted and plain rows share workgroups.
EXTREMES = {
    "prefix_late_past_headroom": (SMALL["4b_like_small"], "prefix", 650, 6.0),
    "prefix_late_within_headroom": (SMALL["4b_like_small"], "prefix", 650, 3.0),
    "prefix_early_peak": (SMALL["4b_like_small"], "prefix", 5, 6.0),
    "tail_past_headroom": (SMALL["4b_like_small"], "tail", 40, 6.0),
    "plain_tail_past_headroom": (synth.config(4, n_questions=12, tail_lo=100, tail_hi=200),
                                 "tail", 130, 6.0),
    "d64_prefix_past_headroom": (SMALL["d64_group1"], "prefix", 100, 8.0),
    # key split: only the first piece's rows recompute, so the merge joins pieces with
    # different references
    "split_first_piece_past_headroom": (SPLIT["ways4_d128"], "prefix", 100, 6.0),
    "split_last_piece_past_headroom": (SPLIT["ways2_d128"], "prefix", 990, 6.0),
}


@pytest.mark.parametrize("name", sorted(EXTREMES))
def test_score_range_extremes(name):
    cfg, where, pos, c = EXTREMES[name]
    print(f"attention score extremes: {name}", flush=True)
    req = Request(cfg, parts=("q", "k_tail", "v_tail", "k_prefix", "v_prefix"))
    ts = {k: v.copy() for k, v in req.tensors.items()}
    group = cfg.n_heads_q // cfg.n_heads_kv
    off = req.pack["token_offset"]
    shifted = [i for i in range(len(req.tail_len))
               if i % 2 == 0 and (where == "prefix" or req.tail_len[i] > pos)]
    assert shifted
    for i in shifted:
        rows = slice(off[i], off[i] + int(req.tail_len[i]))
        ts["q"][rows, :group] = _shift(ts["q"][rows, :group], 1.0)
        if where == "tail":
            ts["k_tail"][off[i] + pos, 0] = _fill(c, cfg.head_dim)
    if where == "prefix":
        ts["k_prefix"][pos, 0] = _fill(c, cfg.head_dim)
    got = run_attention(req, tensors=ts)
    ref = attention_full(ts["q"], ts["k_tail"], ts["v_tail"], ts.get("k_prefix"),
                         ts.get("v_prefix"), off, req.tail_len, cfg.n_heads_q, cfg.n_heads_kv,
                         cfg.scale)
    rows = valid_rows(req)
    assert np.isfinite(got[rows]).all()
    err = np.abs(got[rows] - ref[rows]).max()
    print(f"  max abs err {err:.3e} over {rows.size} rows", flush=True)
    assert err <= ATTN_TOL
