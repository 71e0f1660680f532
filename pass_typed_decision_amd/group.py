"""Several requests scored in one pass, each with its own shared prefix.

The blink.py page's cross-request mode ("public entry point" section, decide_many; "torch
engine" section, logits_rendered): every question of several requests goes through the same
forwards, the rows are split back per request, each request is validated on its own, and a
request that fails is answered with its own error without reaching the others. Here the
accepted requests' questions run through one grouped attention launch (each question against
its own request's prefix) and one label readout, and the probabilities and argmax come back
per request. PyTorch supplies device memory and the stream; every step runs in libblink.so.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np

from ._binding import (
    BlinkError,
    BLINK_E_INVALID,
    GroupedAttention,
    MAX_QUESTIONS,
    MAX_REQUESTS,
    TOKEN_BUDGET,
    check_candidate_table,
    label_readout,
    load_library,
    pack_ragged,
)
from .path import _HIP_MEMCPY_H2D, _hip_memcpy_async


@dataclass
class GroupRequest:
    """One request of a group.

    tail_len      int [n]: each question's own tail length
    cand_ids      int [sum K], cand_off int [n + 1]: the offered labels' token ids (CSR)
    token_base    first row of this request's packed tails in the group's q / k_tail / v_tail
                  / hidden buffers (its rows are token_base + the packer's token offsets)
    prefix_start  first row of its prefix in the group's k_prefix / v_prefix buffers
    prefix_len    its prefix length (0: the plain path)
    """

    tail_len: object
    cand_ids: object
    cand_off: object
    token_base: int
    prefix_start: int = 0
    prefix_len: int = 0


@dataclass
class _Launch:
    """One grouped attention launch and one readout over consecutive accepted requests."""

    members: list  # request indices, in order
    first: np.ndarray  # int32 [R + 1]: first question of each member
    h_tab: object  # pinned int64: token_offset [n], last_row [n], valid_start int32 [n + 1]
    d_tab: object
    up_args: tuple
    attn: GroupedAttention
    read_args: list
    h_res: object  # pinned float32: probs [sum K], argmax int32 [n]
    probs: object
    argmax: object
    cand_off: np.ndarray
    keep: tuple


def plan_group(requests, t_rows: int, prefix_rows: int, vocab: int,
               token_budget: int = TOKEN_BUDGET, max_rows: int = 0):
    """Host side of a group: checks each request on its own and splits the accepted ones into
    launches. Returns (packs, results, launches): packs[r] is request r's pack (None if it was
    refused), results[r] its BlinkError (None if accepted), and launches lists the accepted
    request indices of each launch, consecutive in request order, each launch within 64
    requests and 512 questions.

    A request is refused when its tails or context lengths break the packer's limits, its
    option table is malformed (1-255 options, ids in the vocabulary and distinct within a
    question), its packed rows [token_base, token_base + padded tokens) leave the t_rows rows of
    the buffers or overlap an accepted request's rows, or its prefix rows leave the prefix
    buffers."""
    packs = [None] * len(requests)
    results = [None] * len(requests)
    accepted, taken = [], []
    for r, req in enumerate(requests):
        try:
            tail = np.ascontiguousarray(np.asarray(req.tail_len, np.int32))
            off = np.asarray(req.cand_off)
            if tail.ndim != 1 or off.ndim != 1 or off.shape[0] != tail.shape[0] + 1:
                raise BlinkError(BLINK_E_INVALID, "cand_off must have one entry per question "
                                 "plus one")
            plen, pstart = int(req.prefix_len), int(req.prefix_start)
            pk = pack_ragged(tail, plen, token_budget, max_rows)
            check_candidate_table(req.cand_ids, req.cand_off, vocab)
            lo, hi = int(req.token_base), int(req.token_base) + pk.total_padded_tokens
            if lo < 0 or hi > t_rows:
                raise BlinkError(BLINK_E_INVALID, f"rows [{lo}, {hi}) lie outside the {t_rows} "
                                 "packed rows")
            if plen < 0 or pstart < 0 or pstart + plen > prefix_rows:
                raise BlinkError(BLINK_E_INVALID, f"prefix rows [{pstart}, {pstart + plen}) lie "
                                 f"outside the {prefix_rows} prefix rows")
            for a, b in taken:
                if lo < b and a < hi:
                    raise BlinkError(BLINK_E_INVALID, f"rows [{lo}, {hi}) overlap another "
                                     "request's rows")
        except BlinkError as exc:
            results[r] = exc
            continue
        taken.append((lo, hi))
        packs[r] = pk
        accepted.append(r)
    launches, cur, cur_q = [], [], 0
    for r in accepted:
        n = int(packs[r].token_offset.shape[0])
        if cur and (len(cur) == MAX_REQUESTS or cur_q + n > MAX_QUESTIONS):
            launches.append(cur)
            cur, cur_q = [], 0
        cur.append(r)
        cur_q += n
    if cur:
        launches.append(cur)
    return packs, results, launches


class GroupedScoringStep:
    """Device-resident group of requests; ``run()`` scores all of them once.

    ``tensors``: q [T, H_q, D], k_tail / v_tail [T, H_kv, D], hidden [T, d_model] (bf16,
    device; every request's packed tails at its token_base), k_prefix / v_prefix [rows, H_kv,
    D] or absent (every request's prefix at its prefix_start) and w_u [vocab, d_model].

    Each request is checked on its own when the step is built: its tails and context lengths
    (the packer's limits), its option table, and that its rows lie inside the buffers without
    overlapping an accepted request's rows. A request that fails keeps its BlinkError as its
    result and is left out of every launch. The accepted requests run in launches of at most
    64 requests and 512 questions, in request order. ``run()`` returns one item per request:
    the BlinkError, or (probs, argmax) with probs a list of float32 arrays (one per question,
    over its options) and argmax an int32 array (one per question)."""

    def __init__(self, requests, tensors: dict, n_heads_q: int, n_heads_kv: int,
                 temperature: float, scale: float, token_budget: int = TOKEN_BUDGET,
                 max_rows: int = 0, stream=None):
        import torch

        self.torch = torch
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        self.t = tensors
        self.temperature = float(temperature)
        self.scale = float(scale)
        self.token_budget = int(token_budget)
        self.max_rows = int(max_rows)
        q = tensors["q"]
        dev = q.device
        t_rows = int(q.shape[0])
        if int(q.shape[1]) != int(n_heads_q) or int(tensors["k_tail"].shape[1]) != int(n_heads_kv):
            raise BlinkError(BLINK_E_INVALID, "head counts do not match the tensors")
        if int(tensors["hidden"].shape[0]) != t_rows:
            raise BlinkError(BLINK_E_INVALID, "hidden must have one row per packed token")
        vocab = int(tensors["w_u"].shape[0])
        kp = tensors.get("k_prefix")
        prefix_rows = 0 if kp is None else int(kp.shape[0])

        self.requests = list(requests)
        self.packs, self.results, groups = plan_group(self.requests, t_rows, prefix_rows, vocab,
                                                      self.token_budget, self.max_rows)

        self._copy_fn = _hip_memcpy_async()
        self._lib = load_library()
        self.out = torch.full_like(q, float("nan"))
        self.launches = [self._prepare(g, dev, prefix_rows) for g in groups]

    def _prepare(self, members, dev, prefix_rows) -> _Launch:
        torch = self.torch
        reqs = [self.requests[r] for r in members]
        packs = [self.packs[r] for r in members]
        counts = [int(p.token_offset.shape[0]) for p in packs]
        n = int(sum(counts))
        first = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        tail = np.concatenate([np.asarray(q.tail_len, np.int32) for q in reqs])
        vs = np.concatenate([[0], np.cumsum(tail)]).astype(np.int32)
        ids = np.concatenate([np.asarray(q.cand_ids, np.int32) for q in reqs])
        k_counts = np.concatenate([np.diff(np.asarray(q.cand_off, np.int64)) for q in reqs])
        cand_off = np.concatenate([[0], np.cumsum(k_counts)]).astype(np.int32)
        words = 2 * n + (n + 2) // 2
        h_tab = torch.zeros(words, dtype=torch.int64, pin_memory=True)
        d_tab = torch.zeros(words, dtype=torch.int64, device=dev)
        h_tab.numpy()[2 * n:].view(np.int32)[:n + 1] = vs
        d_off, d_last = d_tab[:n], d_tab[n:2 * n]
        d_vs = d_tab[2 * n:].view(torch.int32)[:n + 1]
        stream_handle = ctypes.c_void_p(self.stream.cuda_stream)
        up_args = (ctypes.c_void_p(d_tab.data_ptr()), ctypes.c_void_p(h_tab.data_ptr()),
                   ctypes.c_size_t(words * 8), _HIP_MEMCPY_H2D, stream_handle)
        t = self.t
        attn = GroupedAttention(
            t["q"], t["k_tail"], t["v_tail"], t.get("k_prefix") if prefix_rows else None,
            t.get("v_prefix") if prefix_rows else None, self.out, d_off, d_vs, vs, first,
            np.asarray([q.prefix_start for q in reqs], np.int64),
            np.asarray([q.prefix_len for q in reqs], np.int32), self.scale,
            stream=self.stream.cuda_stream)
        d_ids = torch.as_tensor(ids).to(dev)
        d_coff = torch.as_tensor(cand_off).to(dev)
        total = int(ids.shape[0])
        logits = torch.empty(total, dtype=torch.float32, device=dev)
        h_res = torch.empty(total + n, dtype=torch.float32, pin_memory=True)
        probs, argmax = h_res[:total], h_res[total:].view(torch.int32)
        read_args = label_readout(t["hidden"], d_last, t["w_u"], d_ids, d_coff, self.temperature,
                                  int(k_counts.max()), logits, probs, argmax,
                                  stream=self.stream.cuda_stream, launch=False)
        return _Launch(members, first, h_tab, d_tab, up_args, attn, read_args, h_res, probs,
                       argmax, cand_off, (d_ids, d_coff, logits))

    def _pack(self, launch: _Launch):
        """Host pack of every member into the launch's pinned tables."""
        n = int(launch.first[-1])
        tab = launch.h_tab.numpy()
        for j, r in enumerate(launch.members):
            req = self.requests[r]
            pk = pack_ragged(req.tail_len, int(req.prefix_len), self.token_budget, self.max_rows)
            a, b = int(launch.first[j]), int(launch.first[j + 1])
            tab[a:b] = pk.token_offset + int(req.token_base)
            tab[n + a:n + b] = pk.last_row + int(req.token_base)

    def run(self):
        """One pass over every accepted request: host pack, one table upload, one grouped
        attention launch and one readout per launch, then the wait for the results."""
        for launch in self.launches:
            self._pack(launch)
            rc = self._copy_fn(*launch.up_args)
            if rc != 0:
                raise RuntimeError(f"hipMemcpyAsync failed with HIP error {rc}")
            launch.attn.launch()
            rc = self._lib.blink_label_readout(*launch.read_args)
            if rc != 0:
                raise BlinkError(rc, self._lib.blink_last_error().decode("utf-8", "replace"))
        self.stream.synchronize()
        results = list(self.results)
        for launch in self.launches:
            probs = launch.probs.numpy()
            argmax = launch.argmax.numpy()
            for j, r in enumerate(launch.members):
                a, b = int(launch.first[j]), int(launch.first[j + 1])
                results[r] = ([probs[launch.cand_off[i]:launch.cand_off[i + 1]].copy()
                               for i in range(a, b)], argmax[a:b].copy())
        return results
