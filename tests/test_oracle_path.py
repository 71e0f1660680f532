"""Pins of oracle.path.score_request, the whole scoring step on the CPU that the bench's CPU
baseline times (blink.py page, "torch engine" section: _forward_shared packs the tails,
attends every tail to the shared prefix and reads each question's labels with _read).

What a mistake in it would break, and what catches it here:
  * the pack it uses must be the packer's (golden-pinned) pack of the same request;
  * every question's attention rows must be plain causal attention over [prefix ; tail],
    checked against torch's float64 scaled_dot_product_attention on the full sequence (a
    library routine, not the oracle's own code), with padded rows left undefined (NaN);
  * a subset of questions must give those questions' rows bit for bit as the whole request
    does, leave every other row undefined, and read exactly their own options: each
    question's logits are checked against a float64 dot product of its own hidden row with
    its own label rows, and its probabilities against torch's softmax of those logits over
    the temperature, so a wrong sub-table offset, a wrong last row or a question mixed up
    with another fails."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle.attention import bf16_to_f64
from oracle.pack import pack_ragged
from oracle.path import score_request

TINY = synth.config(1)
# A second shape: GQA groups of 5, a prefix shorter than one 64-key tile, a row cap.
SMALL_27B = synth.config(5, prefix_len=37, n_questions=6, tail_lo=3, tail_hi=20, d_model=64,
                         vocab=300, k_lo=1, k_hi=7, max_rows=4, temperature=0.7)


def _request(cfg, seed=None):
    rng = synth.rng_for(cfg, seed)
    tables = synth.draw_tables(cfg, rng)
    pk = pack_ragged(tables.tail_len, cfg.token_budget, cfg.max_rows, cfg.prefix_len)
    tensors = synth.draw_tensors(cfg, rng, pk["total_padded_tokens"])
    return tables, pk, tensors


def _sdpa_rows(cfg, tensors, off, n):
    """torch float64 SDPA over the full causal sequence [prefix ; tail]; the tail's n rows."""
    p = cfg.prefix_len
    d = cfg.head_dim
    q_tail = bf16_to_f64(tensors["q"][off:off + n])
    q_full = np.concatenate([np.zeros((p, cfg.n_heads_q, d)), q_tail], 0)
    k_full = np.concatenate([bf16_to_f64(tensors["k_prefix"]),
                             bf16_to_f64(tensors["k_tail"][off:off + n])], 0)
    v_full = np.concatenate([bf16_to_f64(tensors["v_prefix"]),
                             bf16_to_f64(tensors["v_tail"][off:off + n])], 0)
    qt, kt, vt = (torch.from_numpy(x).permute(1, 0, 2)[None] for x in (q_full, k_full, v_full))
    ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, enable_gqa=True,
                                         scale=cfg.scale)
    return ref[0].permute(1, 0, 2).numpy()[p:]


def _own_readout(cfg, tensors, last_row, ids):
    """Logits of one question by a float64 dot product, probabilities by torch's softmax."""
    h = bf16_to_f64(tensors["hidden"][last_row])
    w = bf16_to_f64(tensors["w_u"][np.asarray(ids, np.int64)])
    z = w @ h
    p = torch.softmax(torch.from_numpy(z) / cfg.temperature, dim=0).numpy()
    return z, p


@pytest.mark.parametrize("cfg", [TINY, SMALL_27B], ids=["tiny", "small_gqa5"])
def test_whole_request(cfg):
    tables, pk, tensors = _request(cfg)
    got_pk, out, (z, p, arg) = score_request(tables.tail_len, tensors, tables.cand_ids,
                                             tables.cand_off, cfg)
    for key in ("token_offset", "last_row", "total_padded_tokens"):
        assert np.array_equal(np.asarray(got_pk[key]), np.asarray(pk[key])), key
    real = np.zeros(out.shape[0], bool)
    for i, n in enumerate(tables.tail_len):
        off = int(pk["token_offset"][i])
        real[off:off + int(n)] = True
        np.testing.assert_allclose(out[off:off + int(n)], _sdpa_rows(cfg, tensors, off, int(n)),
                                   rtol=0, atol=1e-12)
    assert np.isnan(out[~real]).all()
    off = tables.cand_off
    for i in range(len(tables.tail_len)):
        ids = tables.cand_ids[off[i]:off[i + 1]]
        zi, pi = _own_readout(cfg, tensors, int(pk["last_row"][i]), ids)
        np.testing.assert_allclose(z[off[i]:off[i + 1]], zi, rtol=0, atol=1e-12)
        np.testing.assert_allclose(p[off[i]:off[i + 1]], pi, rtol=0, atol=1e-12)
        assert arg[i] == int(np.argmax(zi))


@pytest.mark.parametrize("cfg, subset", [(TINY, [2, 0]), (TINY, [3]), (SMALL_27B, [5, 1, 4])],
                         ids=["tiny_2_0", "tiny_3", "small_gqa5_5_1_4"])
def test_subset_reads_only_its_questions(cfg, subset):
    tables, pk, tensors = _request(cfg)
    _, whole, _ = score_request(tables.tail_len, tensors, tables.cand_ids, tables.cand_off, cfg)
    _, out, (z, p, arg) = score_request(tables.tail_len, tensors, tables.cand_ids,
                                        tables.cand_off, cfg, questions=subset)
    keep = np.zeros(out.shape[0], bool)
    for i in subset:
        o, n = int(pk["token_offset"][i]), int(tables.tail_len[i])
        keep[o:o + n] = True
    assert np.array_equal(out[keep], whole[keep])
    assert np.isnan(out[~keep]).all()
    # The sub-table: the subset's options in subset order, each read from its own row.
    off = tables.cand_off
    assert len(z) == sum(int(off[i + 1] - off[i]) for i in subset) and len(arg) == len(subset)
    pos = 0
    for j, i in enumerate(subset):
        ids = tables.cand_ids[off[i]:off[i + 1]]
        zi, pi = _own_readout(cfg, tensors, int(pk["last_row"][i]), ids)
        np.testing.assert_allclose(z[pos:pos + len(ids)], zi, rtol=0, atol=1e-12)
        np.testing.assert_allclose(p[pos:pos + len(ids)], pi, rtol=0, atol=1e-12)
        assert arg[j] == int(np.argmax(zi))
        pos += len(ids)
