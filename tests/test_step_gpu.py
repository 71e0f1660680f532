"""GPU parity of a whole scoring step (ScoringStep: host pack, table upload, attention, and the
readout writing probabilities and argmax into pinned host memory) with the FP64 oracle.

The step queues its work on the stream the caller picks, so it is checked both on torch's
current stream and on a separate stream, and over several consecutive steps (buffers are
reused, and the host result buffer is poisoned with NaN before each step)."""

import numpy as np
import pytest

import synth
from helpers import ATTN_TOL, PROB_TOL, Request, bf16_to_f32_host, check_argmax, device_bf16
from helpers import unit_samples, valid_rows
from oracle.attention import attention_full, attention_rows
from oracle.pack import pack_ragged
from oracle.readout import label_readout

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("side_stream, readout", [(False, "per_option"), (True, "per_option"),
                                                   (False, "batched")],
                         ids=["current", "side", "batched"])
def test_step_matches_oracle(side_stream, readout):
    import torch

    import pass_typed_decision_amd as blink

    cfg = synth.config(1)
    print(f"scoring step: config 1, side stream {side_stream}, readout {readout}", flush=True)
    req = Request(cfg)
    ts = {k: device_bf16(v) for k, v in req.tensors.items() if v.size}
    stream = torch.cuda.Stream() if side_stream else None
    step = blink.ScoringStep(req.tail_len, req.tables.cand_ids, req.tables.cand_off, ts,
                             cfg.n_heads_q, cfg.n_heads_kv, cfg.prefix_len, cfg.temperature,
                             cfg.scale, cfg.token_budget, cfg.max_rows, stream=stream,
                             readout=readout)
    assert step.readout_form == readout
    h = req.tensors
    ref = attention_full(h["q"], h["k_tail"], h["v_tail"], h.get("k_prefix"), h.get("v_prefix"),
                         req.pack["token_offset"], req.tail_len, cfg.n_heads_q, cfg.n_heads_kv,
                         cfg.scale)
    z, p, a = label_readout(h["hidden"], req.pack["last_row"], h["w_u"], req.tables.cand_ids,
                            req.tables.cand_off, cfg.temperature)
    rows = valid_rows(req)
    for it in range(3):
        step.out.fill_(float("nan"))
        step.h_res.fill_(float("nan"))
        torch.cuda.synchronize()
        probs, arg = step.run()
        assert np.array_equal(step.h_token_offset, req.pack["token_offset"])
        assert np.array_equal(step.h_last_row, req.pack["last_row"])
        out = bf16_to_f32_host(step.out)
        attn_err = float(np.abs(out[rows] - ref[rows]).max())
        prob_err = float(np.abs(probs - p).max())
        print(f"  step {it}: attention err {attn_err:.2e} probs err {prob_err:.2e}", flush=True)
        assert attn_err <= ATTN_TOL
        assert prob_err <= PROB_TOL
        check_argmax(z, req.tables.cand_off, a, arg)


@pytest.mark.parametrize("number", [2, 5])
def test_full_size_step_matches_oracle(number):
    # One whole step at full size (the bench's step: host pack, table upload, attention,
    # readout into pinned host memory) against the oracle: the packer's offsets and last rows
    # bit for bit, the label probabilities and argmax of every question, and attention on
    # every real row (4B-like) or on the first and last row of every unit of work (27B-like).
    import torch

    import pass_typed_decision_amd as blink

    cfg = synth.config(number)
    print(f"full-size scoring step: config {number}", flush=True)
    req = Request(cfg)
    ts = {k: device_bf16(v) for k, v in req.tensors.items() if v.size}
    step = blink.ScoringStep(req.tail_len, req.tables.cand_ids, req.tables.cand_off, ts,
                             cfg.n_heads_q, cfg.n_heads_kv, cfg.prefix_len, cfg.temperature,
                             cfg.scale, cfg.token_budget, cfg.max_rows)
    step.out.fill_(float("nan"))
    step.h_res.fill_(float("nan"))
    torch.cuda.synchronize()
    probs, arg = step.run()
    pk = pack_ragged(req.tail_len, cfg.token_budget, cfg.max_rows, cfg.prefix_len)
    assert np.array_equal(step.h_token_offset, pk["token_offset"])
    assert np.array_equal(step.h_last_row, pk["last_row"])
    assert np.array_equal(step.h_valid_start, req.valid_start())
    h = req.tensors
    z, p, a = label_readout(h["hidden"], pk["last_row"], h["w_u"], req.tables.cand_ids,
                            req.tables.cand_off, cfg.temperature)
    prob_err = float(np.abs(probs - p).max())
    ties = check_argmax(z, req.tables.cand_off, a, arg)
    out = bf16_to_f32_host(step.out)
    assert np.isfinite(out[valid_rows(req)]).all()
    if number == 2:
        ref = attention_full(h["q"], h["k_tail"], h["v_tail"], h.get("k_prefix"),
                             h.get("v_prefix"), pk["token_offset"], req.tail_len, cfg.n_heads_q,
                             cfg.n_heads_kv, cfg.scale)
        rows = valid_rows(req)
        attn_err = float(np.abs(out[rows] - ref[rows]).max())
        what = "every real row"
    else:
        samples = unit_samples(req, torch.cuda.get_device_properties(0).multi_processor_count)
        ref = attention_rows(h["q"], h["k_tail"], h["v_tail"], h.get("k_prefix"),
                             h.get("v_prefix"), pk["token_offset"], req.tail_len, cfg.n_heads_q,
                             cfg.n_heads_kv, cfg.scale, samples)
        got = np.stack([out[pk["token_offset"][i] + t, hd] for i, t, hd in samples])
        attn_err = float(np.abs(got - ref).max())
        what = f"{len(samples)} rows at every unit"
    print(f"  attention err {attn_err:.2e} ({what}), probs err {prob_err:.2e}, "
          f"{ties} near-ties", flush=True)
    assert attn_err <= ATTN_TOL
    assert prob_err <= PROB_TOL


def test_typed_answers_from_the_step():
    # The step's GPU probabilities, assembled into typed answers on the host, against the
    # oracle's answers from its FP64 probabilities ("answer assembly" section, answer_for).
    import pass_typed_decision_amd as blink
    from oracle.answers import assemble

    cfg = synth.config(1)
    req = Request(cfg)
    ts = {k: device_bf16(v) for k, v in req.tensors.items() if v.size}
    step = blink.ScoringStep(req.tail_len, req.tables.cand_ids, req.tables.cand_off, ts,
                             cfg.n_heads_q, cfg.n_heads_kv, cfg.prefix_len, cfg.temperature,
                             cfg.scale, cfg.token_budget, cfg.max_rows)
    probs, _ = step.run()
    off = req.tables.cand_off
    k = np.diff(off)
    types = np.where(k == 2, blink.ANSWER_NOUL,
                     np.where(np.arange(len(k)) % 2 == 1, blink.ANSWER_SCORE,
                              blink.ANSWER_CHOICE)).astype(np.int32)
    choice, conf, value = blink.assemble_answers(probs, off, types)
    _, p, _ = label_readout(req.tensors["hidden"], req.pack["last_row"], req.tensors["w_u"],
                            req.tables.cand_ids, off, cfg.temperature)
    ref = assemble(types, p, off)
    print(f"  typed answers for types {types.tolist()}", flush=True)
    for i, (c, f, v) in enumerate(ref):
        assert abs(value[i] - v) <= 10 * PROB_TOL
        if f is None:
            assert choice[i] == -1 and np.isnan(conf[i])
            continue
        assert abs(conf[i] - f) <= 10 * PROB_TOL
        q = np.sort(p[off[i]:off[i + 1]])
        if len(q) == 1 or q[-1] - q[-2] > 1e-5:
            assert choice[i] == c


@pytest.mark.parametrize("readout", ["per_option", "batched"])
def test_pipelined_steps_match_oracle(readout):
    # Two steps in flight (the second slot on its own stream): every collected step must carry
    # its own complete results, checked against the oracle, with the result buffers poisoned.
    import torch

    import pass_typed_decision_amd as blink

    cfg = synth.config(1)
    req = Request(cfg)
    ts = {k: device_bf16(v) for k, v in req.tensors.items() if v.size}
    step = blink.ScoringStep(req.tail_len, req.tables.cand_ids, req.tables.cand_off, ts,
                             cfg.n_heads_q, cfg.n_heads_kv, cfg.prefix_len, cfg.temperature,
                             cfg.scale, cfg.token_budget, cfg.max_rows, depth=2,
                             readout=readout)
    z, p, a = label_readout(req.tensors["hidden"], req.pack["last_row"], req.tensors["w_u"],
                            req.tables.cand_ids, req.tables.cand_off, cfg.temperature)
    for slot in step._slots:
        slot.h_res.fill_(float("nan"))
    torch.cuda.synchronize()
    seen = 0
    for i in range(7):
        step.submit()
        if step.outstanding() == 2:
            probs, arg = step.collect()
            assert float(np.abs(probs - p).max()) <= PROB_TOL
            check_argmax(z, req.tables.cand_off, a, arg)
            probs[:] = np.nan  # the slot must be rewritten by its next step
            seen += 1
    with pytest.raises(blink.BlinkError):
        step.submit()
        step.submit()  # a third outstanding step has no free slot
    while step.outstanding():
        probs, arg = step.collect()
        assert float(np.abs(probs - p).max()) <= PROB_TOL
        seen += 1
    assert seen == 8  # 7 + 1 submitted, all collected
    step.submit()
    step.close()  # waits for the outstanding step, then releases the events
    assert step.outstanding() == 0
    with pytest.raises(blink.BlinkError, match="closed"):
        step.submit()


def test_pipelined_full_size_is_bitwise_sequential():
    # The 4B-like request two steps deep, the second slot on its own stream, so consecutive
    # steps' kernels overlap on the GPU: every collected result and both slots' attention
    # outputs must equal a synchronised step's bit for bit.
    import torch

    import pass_typed_decision_amd as blink

    cfg = synth.config(2)
    req = Request(cfg)
    ts = {k: device_bf16(v) for k, v in req.tensors.items() if v.size}
    step = blink.ScoringStep(req.tail_len, req.tables.cand_ids, req.tables.cand_off, ts,
                             cfg.n_heads_q, cfg.n_heads_kv, cfg.prefix_len, cfg.temperature,
                             cfg.scale, cfg.token_budget, cfg.max_rows, depth=2)
    probs0, arg0 = (x.copy() for x in step.run())
    out0 = step.out.clone()
    rows = torch.as_tensor(valid_rows(req)).cuda()
    for slot in step._slots:
        slot.h_res.fill_(float("nan"))
    step._slots[1].keep[1].fill_(float("nan"))
    step.out.fill_(float("nan"))
    torch.cuda.synchronize()
    collected = 0
    for i in range(6):
        step.submit()
        if step.outstanding() == 2:
            probs, arg = step.collect()
            assert np.array_equal(probs, probs0) and np.array_equal(arg, arg0)
            collected += 1
    while step.outstanding():
        probs, arg = step.collect()
        assert np.array_equal(probs, probs0) and np.array_equal(arg, arg0)
        collected += 1
    torch.cuda.synchronize()
    assert collected == 6
    for out in (step.out, step._slots[1].keep[1]):
        assert torch.equal(out[rows].view(torch.int16), out0[rows].view(torch.int16))
    print("  six overlapped steps bitwise equal to a synchronised one", flush=True)


def test_three_steps_in_flight():
    import pass_typed_decision_amd as blink

    cfg = synth.config(1)
    req = Request(cfg)
    ts = {k: device_bf16(v) for k, v in req.tensors.items() if v.size}
    step = blink.ScoringStep(req.tail_len, req.tables.cand_ids, req.tables.cand_off, ts,
                             cfg.n_heads_q, cfg.n_heads_kv, cfg.prefix_len, cfg.temperature,
                             cfg.scale, cfg.token_budget, cfg.max_rows, depth=3)
    z, p, a = label_readout(req.tensors["hidden"], req.pack["last_row"], req.tensors["w_u"],
                            req.tables.cand_ids, req.tables.cand_off, cfg.temperature)
    for _ in range(3):
        step.submit()
    with pytest.raises(blink.BlinkError):
        step.submit()
    for _ in range(3):
        probs, arg = step.collect()
        assert float(np.abs(probs - p).max()) <= PROB_TOL
        check_argmax(z, req.tables.cand_off, a, arg)
    step.close()
