"""Shared test helpers: build seeded requests, move them to the device, compare with the oracle."""

from __future__ import annotations

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle.pack import pack_ragged as oracle_pack  # noqa: E402

ATTN_TOL = 2e-2  # max-abs on bf16 attention outputs
PROB_TOL = 1e-4  # max-abs on label probabilities
LOGIT_TOL = 1e-4
ARGMAX_GAP = 1e-5  # argmax must match exactly where the oracle's top-2 logit gap exceeds this
# max-abs on teacher-forced log-probabilities. Logits are FP32 sums of at most 5120 bf16
# products (|z| ~ 1, rounding ~1e-6) and the log-sum-exp over 151936 FP32 terms adds a
# relative ~1e-6, so the kernel's error is a few 1e-6 (2e-6 measured). 1e-4 leaves a wide
# margin, and a vocabulary tile dropped from the log-sum-exp (32 rows: about -2e-4; a
# 128-row slice: about -8.4e-4 at vocab 151936) fails it; test_oracle_scoring.py shows that
# on the oracle.
SCORE_TOL = 1e-4


class Request:
    """One seeded request: integer tables, the oracle's pack and bf16 bit tensors."""

    def __init__(self, cfg, seed=None, parts=synth.TENSOR_ORDER, tail_len=None):
        self.cfg = cfg
        rng = synth.rng_for(cfg, seed)
        self.tables = synth.draw_tables(cfg, rng)
        if tail_len is not None:
            self.tables.tail_len = np.asarray(tail_len, np.int32)
        self.pack = oracle_pack(self.tables.tail_len, cfg.token_budget, cfg.max_rows,
                                cfg.prefix_len)
        self.tensors = synth.draw_tensors(cfg, rng, self.pack["total_padded_tokens"], parts)

    @property
    def tail_len(self):
        return self.tables.tail_len

    def valid_start(self):
        vs = np.zeros(len(self.tail_len) + 1, np.int32)
        np.cumsum(self.tail_len, out=vs[1:])
        return vs


def device_bf16(bits):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def bf16_to_f32_host(t):
    import torch

    return synth.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))


def run_attention(req, tensors=None, token_offset=None, tail_len=None, workspace="auto"):
    """GPU attention through the C ABI; returns the output as float32 numpy [T_pad, H_q, D].
    ``workspace``: "auto" (what the library asks for: the bench's launch) or None (none)."""
    import torch

    import pass_typed_decision_amd as blink

    cfg = req.cfg
    ts = req.tensors if tensors is None else tensors
    tail = req.tail_len if tail_len is None else np.asarray(tail_len, np.int32)
    offs = req.pack["token_offset"] if token_offset is None else token_offset
    q = device_bf16(ts["q"])
    kt, vt = device_bf16(ts["k_tail"]), device_bf16(ts["v_tail"])
    kp = vp = None
    if cfg.prefix_len:
        kp, vp = device_bf16(ts["k_prefix"]), device_bf16(ts["v_prefix"])
    out = torch.full_like(q, float("nan"))
    vs = np.zeros(len(tail) + 1, np.int32)
    np.cumsum(tail, out=vs[1:])
    d_off = torch.as_tensor(np.asarray(offs, np.int64)).cuda()
    d_vs = torch.as_tensor(vs).cuda()
    blink.prefix_tail_attention(q, kt, vt, kp, vp, out, d_off, d_vs, int(vs[-1]), cfg.scale,
                                workspace=workspace)
    torch.cuda.synchronize()
    return bf16_to_f32_host(out)


def run_readout(req, last_row=None, cand_ids=None, cand_off=None, temperature=None,
                batched=False, row_tables=None, max_options=None):
    """Runs the readout through the C ABI: blink_label_readout, or with ``batched``
    blink_label_readout_batched over the distinct-row tables of blink_pack_labels (or the
    given ``row_tables`` = (row_id, row_first, row_entry)). ``max_options`` defaults to the
    table's largest option count."""
    import torch

    import pass_typed_decision_amd as blink

    cfg = req.cfg
    ids = req.tables.cand_ids if cand_ids is None else np.asarray(cand_ids, np.int32)
    off = req.tables.cand_off if cand_off is None else np.asarray(cand_off, np.int32)
    last = req.pack["last_row"] if last_row is None else last_row
    t = cfg.temperature if temperature is None else temperature
    hidden = device_bf16(req.tensors["hidden"])
    w_u = device_bf16(req.tensors["w_u"])
    n = len(last)
    d_last = torch.as_tensor(np.asarray(last, np.int64)).cuda()
    d_ids = torch.as_tensor(ids).cuda()
    d_off = torch.as_tensor(off).cuda()
    logits = torch.empty(len(ids), dtype=torch.float32, device="cuda")
    probs = torch.empty_like(logits)
    argmax = torch.empty(n, dtype=torch.int32, device="cuda")
    kmax = int(np.diff(off).max()) if max_options is None else int(max_options)
    if batched:
        if row_tables is None:
            lr = blink.pack_labels(ids, off, cfg.vocab)
            row_tables = (lr.row_id, lr.row_first, lr.row_entry)
        d_rows = [torch.as_tensor(np.asarray(a, np.int32)).cuda() for a in row_tables]
        blink.label_readout_batched(hidden, d_last, w_u, d_off, *d_rows, t, kmax, logits, probs,
                                    argmax)
    else:
        blink.label_readout(hidden, d_last, w_u, d_ids, d_off, t, kmax, logits, probs, argmax)
    torch.cuda.synchronize()
    return logits.cpu().numpy(), probs.cpu().numpy(), argmax.cpu().numpy()


def valid_rows(req):
    rows = []
    for i, n in enumerate(req.tail_len):
        off = req.pack["token_offset"][i]
        rows.extend(range(off, off + int(n)))
    return np.asarray(rows, np.int64)


def sample_rows(req, count, seed=0):
    """(question, position, head) samples: both ends of every tail plus random interior rows."""
    rng = np.random.default_rng(seed)
    cfg = req.cfg
    picks = set()
    for i, n in enumerate(req.tail_len):
        for t in {0, int(n) - 1}:
            picks.add((i, t, int(rng.integers(cfg.n_heads_q))))
    while len(picks) < count:
        i = int(rng.integers(len(req.tail_len)))
        picks.add((i, int(rng.integers(req.tail_len[i])), int(rng.integers(cfg.n_heads_q))))
    return sorted(picks)


def check_argmax(oracle_logits, cand_off, oracle_arg, got_arg):
    """Exact where the oracle's top-2 gap is clear; otherwise the pick must be one of the
    (near-)tied maxima. Returns the number of near-ties seen."""
    ties = 0
    for i in range(len(oracle_arg)):
        z = oracle_logits[cand_off[i]:cand_off[i + 1]]
        top = z.max()
        if len(z) > 1 and np.sort(z)[-2] > top - ARGMAX_GAP:
            ties += 1
            assert z[got_arg[i]] >= top - ARGMAX_GAP, (i, got_arg[i], oracle_arg[i])
        else:
            assert got_arg[i] == oracle_arg[i], (i, got_arg[i], oracle_arg[i])
    return ties


# The attention launch's work split, restated from the launcher's rule so that tests can put a
# sample in every unit of work: per KV head, `rows` query rows (real tail token x query head of
# the group, token-major) are cut into units of 384 rows; when that leaves the last round of
# workgroups partly empty (or the launch is less than one round), the rows beyond the last full
# round are re-cut into smaller units, a multiple of 128 rows (one 32-row wave per SIMD), that
# fill the round. tests/test_unit_plan.py checks this restatement against the launcher itself.
ROWS_PER_UNIT = 384
SIMD_ROWS = 128


def attention_split(rows, hkv, cus, prefix_len):
    """The launcher's key split of the last round, given a workspace: (full units, split base
    units, pieces per unit, prefix tiles per piece), or None. When a head's 384-row units need
    more than one round and the units left after the full rounds would leave CUs idle, each of
    them runs as several pieces over disjoint runs of 64-key prefix tiles."""
    units = -(-rows // ROWS_PER_UNIT)
    per_round = cus // hkv
    if per_round < 2 or units <= per_round:
        return None
    full = units // per_round * per_round
    left = units - full
    if left == 0:
        return None
    ways = per_round // left
    tiles = -(-prefix_len // 64)
    if ways < 2 or tiles < 2 * ways:
        return None
    per = -(-tiles // ways)
    return full, left, -(-tiles // per), per


def attention_units(rows, hkv, cus, prefix_len=0, split=False):
    """[(row0, row_end)] of every unit of one KV head, in unit order (with `split`: as launched
    with a workspace, where a key split keeps whole 384-row units)."""
    if split and attention_split(rows, hkv, cus, prefix_len):
        n = -(-rows // ROWS_PER_UNIT)
        return [(i * ROWS_PER_UNIT, min(rows, (i + 1) * ROWS_PER_UNIT)) for i in range(n)]
    units = -(-rows // ROWS_PER_UNIT)
    full, small = units, ROWS_PER_UNIT
    per_round = cus // hkv
    if per_round >= 1:
        if units * hkv <= cus:
            want = -(-rows // per_round)
            up = max(SIMD_ROWS, -(-want // SIMD_ROWS) * SIMD_ROWS)
            if up < ROWS_PER_UNIT:
                full, small = 0, up
        else:
            whole = units // per_round * per_round
            rem = rows - whole * ROWS_PER_UNIT
            if rem > 0:
                s = -(-rem // per_round)
                s_up = -(-s // SIMD_ROWS) * SIMD_ROWS
                if s_up < ROWS_PER_UNIT:
                    full, small = whole, s_up
    out = []
    r = 0
    while r < rows:
        size = ROWS_PER_UNIT if len(out) < full else small
        out.append((r, min(rows, r + size)))
        r += size
    return out


def unit_samples(req, cus, split=True):
    """(question, position, head) at the first and last row of every (unit, KV head) of the
    attention launch (with `split`: launched with a workspace), plus the first and last token
    of every tail."""
    cfg = req.cfg
    g_size = cfg.n_heads_q // cfg.n_heads_kv
    vs = req.valid_start()
    picks = set()
    for i, n in enumerate(req.tail_len):
        for t in {0, int(n) - 1}:
            picks.add((i, t, (i * 7 + t) % cfg.n_heads_q))
    for row0, row_end in attention_units(int(vs[-1]) * g_size, cfg.n_heads_kv, cus,
                                         cfg.prefix_len, split):
        for r in {row0, row_end - 1}:
            c, hl = divmod(r, g_size)
            q = int(np.searchsorted(vs, c, side="right") - 1)
            for g in range(cfg.n_heads_kv):
                picks.add((q, int(c - vs[q]), g * g_size + hl))
    return sorted(picks)
