"""Pins of the attention oracle against things other than itself: torch's float64
scaled_dot_product_attention over the full causal sequence (library routine, GQA by the
library's own convention), closed forms, and invariants of the shared-prefix reordering."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle.attention import attention_full, attention_decomposed, attention_rows, bf16_to_f64
from oracle.pack import pack_ragged


def _random_case(seed, h_q=4, h_kv=2, d=16, p=7, lengths=(3, 5, 1, 4), budget=10):
    rng = np.random.default_rng(seed)
    pk = pack_ragged(list(lengths), budget)
    t = pk["total_padded_tokens"]
    tensors = {
        "q": rng.standard_normal((t, h_q, d)),
        "k_tail": rng.standard_normal((t, h_kv, d)),
        "v_tail": rng.standard_normal((t, h_kv, d)),
        "k_prefix": rng.standard_normal((p, h_kv, d)),
        "v_prefix": rng.standard_normal((p, h_kv, d)),
    }
    return pk, tensors


def _call(fn, pk, tensors, lengths, h_q, h_kv, scale):
    return fn(tensors["q"], tensors["k_tail"], tensors["v_tail"], tensors["k_prefix"],
              tensors["v_prefix"], pk["token_offset"], list(lengths), h_q, h_kv, scale)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("shape", [(4, 2, 16, 7), (4, 1, 8, 0), (5, 1, 8, 3), (3, 3, 4, 11)])
def test_against_torch_sdpa_full_sequence(seed, shape):
    h_q, h_kv, d, p = shape
    lengths = (3, 5, 1, 4)
    pk, ts = _random_case(seed, h_q, h_kv, d, p, lengths)
    scale = 1.0 / np.sqrt(d)
    got = _call(attention_full, pk, ts, lengths, h_q, h_kv, scale)
    rng = np.random.default_rng(100 + seed)
    for i, n in enumerate(lengths):
        off = pk["token_offset"][i]
        # Full sequence [prefix ; tail]; the prefix rows' own queries are arbitrary because
        # causal masking keeps them from influencing the tail rows that are compared.
        q_full = np.concatenate([rng.standard_normal((p, h_q, d)), ts["q"][off:off + n]], 0)
        k_full = np.concatenate([ts["k_prefix"], ts["k_tail"][off:off + n]], 0)
        v_full = np.concatenate([ts["v_prefix"], ts["v_tail"][off:off + n]], 0)
        qt = torch.from_numpy(q_full).permute(1, 0, 2)[None]
        kt = torch.from_numpy(k_full).permute(1, 0, 2)[None]
        vt = torch.from_numpy(v_full).permute(1, 0, 2)[None]
        ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, enable_gqa=True)
        ref = ref[0].permute(1, 0, 2).numpy()[p:]
        np.testing.assert_allclose(got[off:off + n], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(10))
def test_decomposed_equals_full(seed):
    rng = np.random.default_rng(seed)
    lengths = tuple(int(x) for x in rng.integers(1, 9, size=5))
    p = int(rng.integers(0, 20))
    pk, ts = _random_case(seed, 6, 2, 8, p, lengths, budget=16)
    full = _call(attention_full, pk, ts, lengths, 6, 2, 0.3)
    dec = _call(attention_decomposed, pk, ts, lengths, 6, 2, 0.3)
    valid = ~np.isnan(full[:, 0, 0])
    assert np.isnan(dec[~valid]).all()
    np.testing.assert_allclose(dec[valid], full[valid], rtol=0, atol=1e-12)


def test_rows_match_full():
    lengths = (3, 5, 1, 4)
    pk, ts = _random_case(3, 4, 2, 16, 7, lengths)
    full = _call(attention_full, pk, ts, lengths, 4, 2, 0.25)
    rows = [(0, 2, 3), (1, 0, 0), (1, 4, 1), (2, 0, 2), (3, 3, 3)]
    got = attention_rows(ts["q"], ts["k_tail"], ts["v_tail"], ts["k_prefix"], ts["v_prefix"],
                         pk["token_offset"], list(lengths), 4, 2, 0.25, rows)
    for r, (i, t, h) in enumerate(rows):
        np.testing.assert_allclose(got[r], full[pk["token_offset"][i] + t, h], rtol=0, atol=1e-13)


def test_first_tail_token_without_prefix_is_its_own_value():
    lengths = (4, 2)
    pk, ts = _random_case(1, 4, 2, 8, 0, lengths)
    out = _call(attention_full, pk, ts, lengths, 4, 2, 0.5)
    for i in range(2):
        off = pk["token_offset"][i]
        for h in range(4):
            np.testing.assert_array_equal(out[off, h], ts["v_tail"][off, h // 2])


def test_zero_query_gives_mean_of_visible_values():
    lengths = (3, 5)
    pk, ts = _random_case(2, 2, 1, 8, 6, lengths)
    ts["q"][:] = 0.0
    out = _call(attention_full, pk, ts, lengths, 2, 1, 0.7)
    for i, n in enumerate(lengths):
        off = pk["token_offset"][i]
        for t in range(n):
            visible = np.concatenate([ts["v_prefix"][:, 0], ts["v_tail"][off:off + t + 1, 0]])
            np.testing.assert_allclose(out[off + t, 1], visible.mean(0), atol=1e-13)


def test_dominant_prefix_key_selects_its_value():
    lengths = (3, 2)
    pk, ts = _random_case(4, 2, 1, 8, 5, lengths)
    direction = np.ones(8) / np.sqrt(8)
    ts["q"][:] = direction
    ts["k_prefix"][3, 0] = 40.0 * direction
    out = _call(attention_full, pk, ts, lengths, 2, 1, 1.0)
    for i, n in enumerate(lengths):
        off = pk["token_offset"][i]
        np.testing.assert_allclose(out[off:off + n, 0], np.repeat(ts["v_prefix"][3:4, 0], n, 0), atol=1e-9)


def test_dominant_future_key_is_masked():
    # A huge score on a later tail key must not reach an earlier row (causality, inclusive).
    lengths = (4,)
    pk, ts = _random_case(5, 1, 1, 8, 3, lengths)
    direction = np.ones(8) / np.sqrt(8)
    ts["q"][:] = direction
    ts["k_tail"][2, 0] = 40.0 * direction
    out = _call(attention_full, pk, ts, lengths, 1, 1, 1.0)
    assert np.abs(out[1, 0] - ts["v_tail"][2, 0]).max() > 1e-3
    np.testing.assert_allclose(out[2, 0], ts["v_tail"][2, 0], atol=1e-9)
    np.testing.assert_allclose(out[3, 0], ts["v_tail"][2, 0], atol=1e-9)


def test_query_scale_trade():
    lengths = (3, 4)
    pk, ts = _random_case(6, 4, 2, 8, 5, lengths)
    a = _call(attention_full, pk, ts, lengths, 4, 2, 0.5)
    ts2 = dict(ts, q=ts["q"] * 4.0)
    b = _call(attention_full, pk, ts2, lengths, 4, 2, 0.125)
    np.testing.assert_allclose(a, b, atol=1e-12, equal_nan=True)


def test_padding_content_does_not_matter():
    lengths = (3, 5, 1, 4)
    pk, ts = _random_case(7, 4, 2, 8, 4, lengths)
    a = _call(attention_full, pk, ts, lengths, 4, 2, 0.4)
    valid = np.zeros(pk["total_padded_tokens"], bool)
    for i, n in enumerate(lengths):
        valid[pk["token_offset"][i]:pk["token_offset"][i] + n] = True
    ts2 = {k: v.copy() for k, v in ts.items()}
    for name in ("q", "k_tail", "v_tail"):
        ts2[name][~valid] = 1e3
    b = _call(attention_full, pk, ts2, lengths, 4, 2, 0.4)
    np.testing.assert_array_equal(a[valid], b[valid])


def test_question_alone_equals_question_packed():
    lengths = (3, 5, 2)
    pk, ts = _random_case(8, 4, 2, 8, 6, lengths, budget=100)
    together = _call(attention_full, pk, ts, lengths, 4, 2, 0.4)
    i = 1
    off, n = pk["token_offset"][i], lengths[i]
    alone_ts = dict(ts, q=ts["q"][off:off + n], k_tail=ts["k_tail"][off:off + n],
                    v_tail=ts["v_tail"][off:off + n])
    alone = attention_full(alone_ts["q"], alone_ts["k_tail"], alone_ts["v_tail"],
                           ts["k_prefix"], ts["v_prefix"], [0], [n], 4, 2, 0.4)
    np.testing.assert_array_equal(alone, together[off:off + n])


def test_head_permutation_within_group():
    lengths = (3, 4)
    pk, ts = _random_case(9, 4, 2, 8, 5, lengths)
    a = _call(attention_full, pk, ts, lengths, 4, 2, 0.4)
    perm = [1, 0, 3, 2]  # swaps stay inside the groups {0,1} and {2,3}
    b = _call(attention_full, pk, dict(ts, q=ts["q"][:, perm]), lengths, 4, 2, 0.4)
    np.testing.assert_array_equal(a[:, perm], b)


def test_bf16_inputs_are_widened_exactly():
    bits = synth.f32_to_bf16_bits(np.array([1.0, -2.5, 3.140625, 0.0], np.float32))
    np.testing.assert_array_equal(bf16_to_f64(bits), [1.0, -2.5, 3.140625, 0.0])
    # round to nearest even at the halfway point between two bf16 values
    halfway = np.array([1.0 + 2.0 ** -8], np.float32)
    assert bf16_to_f64(synth.f32_to_bf16_bits(halfway))[0] == 1.0
    above = np.array([1.0 + 2.0 ** -8 + 2.0 ** -20], np.float32)
    assert bf16_to_f64(synth.f32_to_bf16_bits(above))[0] == 1.0 + 2.0 ** -7


def _grouped_case(seed, prefixes=(0, 5, 9), questions=(2, 1, 3), d=8, hq=4, hkv=2):
    rng = np.random.default_rng(seed)
    tails = [rng.integers(1, 7, size=n).tolist() for n in questions]
    lens = [t for ts in tails for t in ts]
    off = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    t_pad = int(sum(lens))
    q = rng.standard_normal((t_pad, hq, d))
    kt = rng.standard_normal((t_pad, hkv, d))
    vt = rng.standard_normal((t_pad, hkv, d))
    rows = max(1, sum(prefixes))
    kp = rng.standard_normal((rows, hkv, d))
    vp = rng.standard_normal((rows, hkv, d))
    first = np.concatenate([[0], np.cumsum(questions)]).astype(int)
    pstart = np.concatenate([[0], np.cumsum(prefixes)[:-1]]).astype(int)
    return q, kt, vt, kp, vp, off, lens, first, pstart, list(prefixes), hq, hkv


def test_grouped_with_one_request_is_the_plain_call():
    from oracle.attention import attention_grouped

    q, kt, vt, kp, vp, off, lens, _, _, _, hq, hkv = _grouped_case(1, prefixes=(7,),
                                                                    questions=(4,))
    got = attention_grouped(q, kt, vt, kp, vp, off, lens, [0, 4], [0], [7], hq, hkv, 0.3)
    ref = attention_full(q, kt, vt, kp[:7], vp[:7], off, lens, hq, hkv, 0.3)
    np.testing.assert_array_equal(got, ref)


def test_grouped_requests_see_only_their_own_prefix():
    from oracle.attention import attention_grouped

    q, kt, vt, kp, vp, off, lens, first, pstart, plen, hq, hkv = _grouped_case(2)
    got = attention_grouped(q, kt, vt, kp, vp, off, lens, first, pstart, plen, hq, hkv, 0.3)
    for r in range(3):
        for i in range(first[r], first[r + 1]):
            o, n = int(off[i]), lens[i]
            # the question alone, its request's prefix concatenated in front (plain causal)
            pre_k = kp[pstart[r]:pstart[r] + plen[r]]
            pre_v = vp[pstart[r]:pstart[r] + plen[r]]
            full_k = np.concatenate([pre_k, kt[o:o + n]])
            full_v = np.concatenate([pre_v, vt[o:o + n]])
            ref = attention_full(np.concatenate([np.zeros((plen[r], hq, q.shape[2])), q[o:o + n]]),
                                 full_k, full_v, None, None, [0], [plen[r] + n], hq, hkv, 0.3)
            np.testing.assert_allclose(got[o:o + n], ref[plen[r]:], atol=1e-12)
    # a wrong prefix (the next request's) changes the rows of a request that has a prefix
    bad = attention_grouped(q, kt, vt, kp, vp, off, lens, first, [pstart[2]] * 3, plen, hq,
                            hkv, 0.3)
    o1 = int(off[first[1]])
    assert np.abs(bad[o1] - got[o1]).max() > 1e-6


def test_grouped_requests_may_share_prefix_rows():
    from oracle.attention import attention_grouped

    q, kt, vt, kp, vp, off, lens, first, _, _, hq, hkv = _grouped_case(3, prefixes=(6, 6, 6))
    shared = attention_grouped(q, kt, vt, kp, vp, off, lens, first, [0, 0, 0], [6, 6, 6], hq,
                               hkv, 0.3)
    one = attention_full(q, kt, vt, kp[:6], vp[:6], off, lens, hq, hkv, 0.3)
    np.testing.assert_array_equal(shared, one)
