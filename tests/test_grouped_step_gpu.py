"""GPU parity of the grouped scoring step (several requests, each with its own shared prefix,
through one grouped attention launch and one readout) with the FP64 oracle, request by
request ("public entry point" section of the blink.py page, decide_many: each request is
validated on its own and one request's failure never reaches another).

Requests of different shapes share the group: shared prefixes of several lengths, a plain
request (no prefix), GQA 4. Two malformed requests sit between them: one question offers 256
options, and one request's prefix plus tail passes the maximum context length. Their results
are their errors; every other request matches the oracle (attention on every real row,
probabilities, argmax) and is bitwise what the same group gives without the malformed ones."""

import numpy as np
import pytest

import synth
from helpers import ATTN_TOL, PROB_TOL, bf16_to_f32_host, check_argmax, device_bf16
from oracle.attention import attention_full
from oracle.pack import pack_ragged
from oracle.readout import label_readout

pytestmark = pytest.mark.gpu

SHAPES = [  # (prefix_len, questions, tail range), 4 q / 1 kv heads, head_dim 64
    (256, 4, (16, 48)),
    (0, 6, (1, 40)),
    (700, 3, (30, 140)),
    (64, 5, (60, 70)),
]


def _build(with_bad: bool, seed: int = 5):
    """The group's requests and host tensors: request r's packed tails at rows token_base[r],
    its prefix at prefix_start[r]; one unembedding matrix shared by all."""
    cfg0 = synth.config(1)
    rng = np.random.default_rng(seed)
    reqs, tails, prefixes, hidden, bases, pstarts = [], [], [], [], [], []
    base = pstart = 0
    for i, (p, n, (lo, hi)) in enumerate(SHAPES):
        cfg = synth.config(1, prefix_len=p, n_questions=n, tail_lo=lo, tail_hi=hi)
        srng = synth.rng_for(cfg, seed=100 + i)
        tables = synth.draw_tables(cfg, srng)
        pk = pack_ragged(tables.tail_len, cfg.token_budget, 0, p)
        t = synth.draw_tensors(cfg, srng, pk["total_padded_tokens"],
                               ("q", "k_tail", "v_tail", "k_prefix", "v_prefix", "hidden"))
        reqs.append(dict(cfg=cfg, tables=tables, pack=pk, base=base, pstart=pstart))
        tails.append(t)
        bases.append(base)
        pstarts.append(pstart)
        base += pk["total_padded_tokens"]
        pstart += p
    w_u = synth.f32_to_bf16_bits((rng.standard_normal((cfg0.vocab, cfg0.d_model)) * 0.02)
                                 .astype(np.float32))
    cat = {k: np.concatenate([t[k] for t in tails]) for k in ("q", "k_tail", "v_tail", "hidden")}
    cat["k_prefix"] = np.concatenate([t["k_prefix"] for t in tails])
    cat["v_prefix"] = np.concatenate([t["v_prefix"] for t in tails])
    cat["w_u"] = w_u
    return reqs, cat


def _group_requests(blink, reqs, with_bad: bool):
    out = []
    for i, r in enumerate(reqs):
        tb = r["tables"]
        out.append(blink.GroupRequest(tb.tail_len, tb.cand_ids, tb.cand_off, r["base"],
                                      r["pstart"], r["cfg"].prefix_len))
        if with_bad and i == 1:
            # a question with 256 options (rows of request 0: never launched, so no overlap)
            ids = np.arange(256, dtype=np.int32)
            out.append(blink.GroupRequest([5], ids, [0, 256], reqs[0]["base"], 0, 0))
        if with_bad and i == 2:
            # prefix plus tail past the maximum context length
            out.append(blink.GroupRequest([200], [1, 2], [0, 2], reqs[0]["base"], 0, 131000))
    return out


def test_grouped_step_matches_oracle_per_request():
    import torch

    import pass_typed_decision_amd as blink

    reqs, cat = _build(True)
    dev = {k: device_bf16(v) for k, v in cat.items()}
    cfg = reqs[0]["cfg"]
    print(f"grouped step: {len(reqs)} requests + 2 malformed", flush=True)
    group = blink.GroupedScoringStep(_group_requests(blink, reqs, True), dev, cfg.n_heads_q,
                                     cfg.n_heads_kv, cfg.temperature, cfg.scale)
    assert len(group.launches) == 1
    res = group.run()
    assert len(res) == len(reqs) + 2
    bad = [res[2], res[4]]
    assert isinstance(bad[0], blink.BlinkError) and "256 options" in str(bad[0])
    assert isinstance(bad[1], blink.BlinkError) and "maximum context length" in str(bad[1])
    good = [res[0], res[1], res[3], res[5]]
    out = bf16_to_f32_host(group.out)
    for r, (probs, arg) in zip(reqs, good):
        c, tb, pk = r["cfg"], r["tables"], r["pack"]
        offs = np.asarray(pk["token_offset"]) + r["base"]
        kp = cat["k_prefix"][r["pstart"]:r["pstart"] + c.prefix_len]
        vp = cat["v_prefix"][r["pstart"]:r["pstart"] + c.prefix_len]
        ref = attention_full(cat["q"], cat["k_tail"], cat["v_tail"], kp if c.prefix_len else None,
                             vp if c.prefix_len else None, offs, tb.tail_len, c.n_heads_q,
                             c.n_heads_kv, c.scale)
        rows = np.concatenate([np.arange(o, o + n) for o, n in zip(offs, tb.tail_len)])
        attn_err = float(np.abs(out[rows] - ref[rows]).max())
        last = np.asarray(pk["last_row"]) + r["base"]
        z, p, a = label_readout(cat["hidden"], last, cat["w_u"], tb.cand_ids, tb.cand_off,
                                c.temperature)
        prob_err = float(np.abs(np.concatenate(probs) - p).max())
        print(f"  prefix {c.prefix_len}: attention err {attn_err:.2e}, probs err {prob_err:.2e}",
              flush=True)
        assert attn_err <= ATTN_TOL and prob_err <= PROB_TOL
        check_argmax(z, tb.cand_off, a, arg)

    # The same group without the malformed requests: bitwise the same results.
    clean = blink.GroupedScoringStep(_group_requests(blink, reqs, False), dev, cfg.n_heads_q,
                                     cfg.n_heads_kv, cfg.temperature, cfg.scale)
    res2 = clean.run()
    for (p1, a1), (p2, a2) in zip(good, res2):
        assert all(np.array_equal(x, y) for x, y in zip(p1, p2)) and np.array_equal(a1, a2)
    torch.cuda.synchronize()
    rows_all = np.isfinite(out[:, 0, 0])
    assert torch.equal(clean.out.view(torch.int16)[torch.as_tensor(rows_all).cuda()],
                       group.out.view(torch.int16)[torch.as_tensor(rows_all).cuda()])


def test_group_splits_into_launches_at_the_limits():
    # 9 requests of 60 questions: 540 questions in all, more than one launch may take (512),
    # so the step splits them, in order, into launches within the limits.
    import pass_typed_decision_amd as blink

    cfg = synth.config(1, prefix_len=0, n_questions=60, tail_lo=1, tail_hi=4)
    reqs, parts, base = [], [], 0
    for i in range(9):
        srng = synth.rng_for(cfg, seed=300 + i)
        tb = synth.draw_tables(cfg, srng)
        pk = pack_ragged(tb.tail_len, cfg.token_budget, 0, 0)
        parts.append(synth.draw_tensors(cfg, srng, pk["total_padded_tokens"],
                                        ("q", "k_tail", "v_tail", "k_prefix", "v_prefix",
                                         "hidden", "w_u")))
        reqs.append((tb, pk, base))
        base += pk["total_padded_tokens"]
    cat = {k: np.concatenate([p[k] for p in parts]) for k in ("q", "k_tail", "v_tail", "hidden")}
    cat["w_u"] = parts[0]["w_u"]
    dev = {k: device_bf16(v) for k, v in cat.items()}
    group = blink.GroupedScoringStep(
        [blink.GroupRequest(tb.tail_len, tb.cand_ids, tb.cand_off, b) for tb, _, b in reqs],
        dev, cfg.n_heads_q, cfg.n_heads_kv, cfg.temperature, cfg.scale)
    assert [len(l.members) for l in group.launches] == [8, 1]
    res = group.run()
    for (tb, pk, b), (probs, arg) in zip(reqs, res):
        z, p, a = label_readout(cat["hidden"], np.asarray(pk["last_row"]) + b, cat["w_u"],
                                tb.cand_ids, tb.cand_off, cfg.temperature)
        assert float(np.abs(np.concatenate(probs) - p).max()) <= PROB_TOL
        check_argmax(z, tb.cand_off, a, arg)
