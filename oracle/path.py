"""The whole scoring step on the CPU, for timing the oracle beside the GPU (test
infrastructure only).

One step follows the batch loop of the blink.py page (thegovind/blink-4b, "torch engine"
section, _forward_shared / _forward): pack the question tails, run every tail's attention
against the shared prefix, then read each question's label distribution. ``questions``
restricts the attention and readout to a subset, so that a bounded sample of a large
workload can be timed; packing always covers the whole request.
"""

from __future__ import annotations

from .pack import pack_ragged
from .attention import attention_full
from .readout import label_readout


def score_request(tail_len, tensors, cand_ids, cand_off, cfg, questions=None):
    """Returns (pack, attention output [T_pad, H_q, D] float64, (logits, probs, argmax))."""
    pk = pack_ragged(tail_len, cfg.token_budget, cfg.max_rows, cfg.prefix_len)
    qs = list(range(len(tail_len))) if questions is None else list(questions)
    out = attention_full(
        tensors["q"], tensors["k_tail"], tensors["v_tail"],
        tensors.get("k_prefix"), tensors.get("v_prefix"),
        pk["token_offset"], tail_len, cfg.n_heads_q, cfg.n_heads_kv, cfg.scale, questions=qs)
    sub_off = [0]
    sub_ids = []
    for i in qs:
        ids = list(cand_ids[cand_off[i]:cand_off[i + 1]])
        sub_ids.extend(ids)
        sub_off.append(sub_off[-1] + len(ids))
    readout = label_readout(tensors["hidden"], [pk["last_row"][i] for i in qs], tensors["w_u"],
                            sub_ids, sub_off, cfg.temperature)
    return pk, out, readout
