"""One scoring step of a request, chained through the C ABI.

A step is the hot path of the blink.py page (thegovind/blink-4b, "torch engine" section,
_forward_shared and _read, and "answer assembly" section, softmax): pack the question tails
(host), upload the small row tables, run the shared-prefix tail attention and the label
readout on the GPU, and bring the label probabilities and argmax back to the host. The
request's tensors stay resident on the device between steps.
"""

from __future__ import annotations

import itertools
import string

import numpy as np

from ._binding import (
    BlinkError,
    BLINK_E_INVALID,
    check_candidate_table,
    label_readout,
    pack_ragged,
    prefix_tail_attention,
    TOKEN_BUDGET,
)

# Option index -> label: A..Z, then AA..ZZ ("constants the deployment sets" section:
# LABEL_POOL), at most 255 of them.
_LABELS = list(string.ascii_uppercase) + [
    a + b for a, b in itertools.product(string.ascii_uppercase, repeat=2)]


def label_name(index: int) -> str:
    if not 0 <= index < 255:
        raise BlinkError(BLINK_E_INVALID, f"option index {index} outside 0-254")
    return _LABELS[index]


class ScoringStep:
    """Device-resident request plus reusable buffers; ``run()`` is one scoring step."""

    def __init__(self, tail_len, cand_ids, cand_off, tensors: dict, n_heads_q: int,
                 n_heads_kv: int, prefix_len: int, temperature: float, scale: float,
                 token_budget: int = TOKEN_BUDGET, max_rows: int = 0, stream=None):
        import torch

        self.torch = torch
        self.tail_len = np.ascontiguousarray(np.asarray(tail_len, np.int32))
        self.n = int(self.tail_len.shape[0])
        self.prefix_len = int(prefix_len)
        self.token_budget = int(token_budget)
        self.max_rows = int(max_rows)
        self.temperature = float(temperature)
        self.scale = float(scale)
        self.t = tensors
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        dev = tensors["q"].device
        vocab = int(tensors["w_u"].shape[0])
        self.max_options = check_candidate_table(cand_ids, cand_off, vocab)
        pk = pack_ragged(self.tail_len, self.prefix_len, self.token_budget, self.max_rows)
        if pk.total_padded_tokens != tensors["q"].shape[0]:
            raise BlinkError(BLINK_E_INVALID, "tensors were not laid out for this pack")
        self.pack = pk
        self.cand_ids = torch.as_tensor(np.asarray(cand_ids, np.int32)).to(dev)
        self.cand_off = torch.as_tensor(np.asarray(cand_off, np.int32)).to(dev)
        total = int(self.cand_ids.shape[0])
        pin = dict(pin_memory=True)
        self.h_token_offset = torch.zeros(self.n, dtype=torch.int64, **pin)
        self.h_last_row = torch.zeros(self.n, dtype=torch.int64, **pin)
        self.h_valid_start = torch.zeros(self.n + 1, dtype=torch.int32, **pin)
        self.d_token_offset = torch.zeros(self.n, dtype=torch.int64, device=dev)
        self.d_last_row = torch.zeros(self.n, dtype=torch.int64, device=dev)
        self.d_valid_start = torch.zeros(self.n + 1, dtype=torch.int32, device=dev)
        t_pad = pk.total_padded_tokens
        self.out = torch.empty(t_pad, n_heads_q, tensors["q"].shape[2], dtype=torch.bfloat16,
                               device=dev)
        self.logits = torch.empty(total, dtype=torch.float32, device=dev)
        self.probs = torch.empty(total, dtype=torch.float32, device=dev)
        self.argmax = torch.empty(self.n, dtype=torch.int32, device=dev)
        self.h_probs = torch.empty(total, dtype=torch.float32, **pin)
        self.h_argmax = torch.empty(self.n, dtype=torch.int32, **pin)

    def pack_and_upload(self):
        pk = pack_ragged(self.tail_len, self.prefix_len, self.token_budget, self.max_rows)
        self.h_token_offset.numpy()[:] = pk.token_offset
        self.h_last_row.numpy()[:] = pk.last_row
        self.h_valid_start.numpy()[:] = pk.valid_start
        with self.torch.cuda.stream(self.stream):
            self.d_token_offset.copy_(self.h_token_offset, non_blocking=True)
            self.d_last_row.copy_(self.h_last_row, non_blocking=True)
            self.d_valid_start.copy_(self.h_valid_start, non_blocking=True)
        return pk

    def attention(self, pk):
        t = self.t
        prefix_tail_attention(t["q"], t["k_tail"], t["v_tail"], t.get("k_prefix"),
                              t.get("v_prefix"), self.out, self.d_token_offset,
                              self.d_valid_start, pk.total_valid_tokens, self.scale,
                              stream=self.stream.cuda_stream)

    def readout(self):
        label_readout(self.t["hidden"], self.d_last_row, self.t["w_u"], self.cand_ids,
                      self.cand_off, self.temperature, self.max_options, self.logits,
                      self.probs, self.argmax, stream=self.stream.cuda_stream)

    def run(self, fetch: bool = True):
        """One step. With ``fetch`` the probabilities and argmax are copied to pinned host
        memory and the stream is synchronised; returns (probs, argmax) host arrays."""
        pk = self.pack_and_upload()
        self.attention(pk)
        self.readout()
        if not fetch:
            return None
        with self.torch.cuda.stream(self.stream):
            self.h_probs.copy_(self.probs, non_blocking=True)
            self.h_argmax.copy_(self.argmax, non_blocking=True)
        self.stream.synchronize()
        return self.h_probs.numpy(), self.h_argmax.numpy()
