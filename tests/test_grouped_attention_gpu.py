"""GPU parity of blink_prefix_tail_attention_grouped (through the C ABI): several requests,
each with its own shared prefix, in one launch. Against the FP64 oracle (max-abs 2e-2 on every
real row), and bit for bit against one blink_prefix_tail_attention launch per request (a
question's rows do not depend on what else shares the launch)."""

from dataclasses import replace

import numpy as np
import pytest

import synth
from helpers import ATTN_TOL, Request, bf16_to_f32_host, device_bf16, run_attention
from oracle.attention import attention_grouped, attention_rows

pytestmark = pytest.mark.gpu

PARTS = ("q", "k_tail", "v_tail", "k_prefix", "v_prefix")


class Group:
    """Requests laid out one after another: tails in one packed buffer, prefixes in one."""

    def __init__(self, cfgs, seeds):
        self.reqs = [Request(c, seed=s, parts=PARTS) for c, s in zip(cfgs, seeds)]
        c0 = cfgs[0]
        self.hq, self.hkv, self.d, self.scale = c0.n_heads_q, c0.n_heads_kv, c0.head_dim, c0.scale
        self.tail_len = np.concatenate([r.tail_len for r in self.reqs]).astype(np.int32)
        bases = np.cumsum([0] + [r.pack["total_padded_tokens"] for r in self.reqs])
        self.token_offset = np.concatenate(
            [np.asarray(r.pack["token_offset"], np.int64) + b for r, b in zip(self.reqs, bases)])
        self.tensors = {k: np.concatenate([r.tensors[k] for r in self.reqs])
                        for k in ("q", "k_tail", "v_tail")}
        self.prefix_len = np.array([c.prefix_len for c in cfgs], np.int32)
        self.prefix_start = np.concatenate([[0], np.cumsum(self.prefix_len)[:-1]]).astype(np.int64)
        pre = [r.tensors["k_prefix"] for r, c in zip(self.reqs, cfgs) if c.prefix_len]
        shape = (0, self.hkv, self.d)
        self.k_prefix = np.concatenate(pre) if pre else np.zeros(shape, np.uint16)
        pre = [r.tensors["v_prefix"] for r, c in zip(self.reqs, cfgs) if c.prefix_len]
        self.v_prefix = np.concatenate(pre) if pre else np.zeros(shape, np.uint16)
        self.request_first = np.concatenate(
            [[0], np.cumsum([len(r.tail_len) for r in self.reqs])]).astype(np.int32)
        self.valid_start = np.concatenate([[0], np.cumsum(self.tail_len)]).astype(np.int32)

    def run(self):
        import torch

        import pass_typed_decision_amd as blink

        q = device_bf16(self.tensors["q"])
        kt, vt = device_bf16(self.tensors["k_tail"]), device_bf16(self.tensors["v_tail"])
        rows = self.k_prefix.shape[0]
        kp = device_bf16(self.k_prefix) if rows else None
        vp = device_bf16(self.v_prefix) if rows else None
        out = torch.full_like(q, float("nan"))
        d_off = torch.as_tensor(self.token_offset).cuda()
        d_vs = torch.as_tensor(self.valid_start).cuda()
        ga = blink.GroupedAttention(q, kt, vt, kp, vp, out, d_off, d_vs, self.valid_start,
                                    self.request_first, self.prefix_start, self.prefix_len,
                                    self.scale)
        ga.launch()
        torch.cuda.synchronize()
        return bf16_to_f32_host(out)

    def rows_of(self, r):
        req, base = self.reqs[r], int(self.token_offset[self.request_first[r]] -
                                      self.reqs[r].pack["token_offset"][0])
        return [np.arange(base + o, base + o + n)
                for o, n in zip(req.pack["token_offset"], req.tail_len)]


def _check_bitwise_against_single(group, got, which):
    # against the single-request launch without a workspace (no key split), which sums every
    # row in the same order as the grouped launch
    for r in which:
        single = run_attention(group.reqs[r], workspace=None)
        req = group.reqs[r]
        for (o, n), rows in zip(zip(req.pack["token_offset"], req.tail_len), group.rows_of(r)):
            np.testing.assert_array_equal(got[rows], single[o:o + n])


SMALL = {
    "mixed_prefixes_d128": ([synth.config(2, prefix_len=700, n_questions=5, tail_lo=30, tail_hi=140),
                             synth.config(2, prefix_len=0, n_questions=7, tail_lo=1, tail_hi=90),
                             synth.config(2, prefix_len=64, n_questions=3, tail_lo=63, tail_hi=65),
                             synth.config(2, prefix_len=333, n_questions=2, tail_lo=200, tail_hi=260)],
                            [11, 12, 13, 14]),
    "tiny_like_d64": ([synth.config(1), synth.config(1, prefix_len=1, n_questions=3),
                       synth.config(1, prefix_len=0, n_questions=2)], [21, 22, 23]),
    "one_request": ([synth.config(5, prefix_len=333, n_questions=3, tail_lo=50, tail_hi=200)],
                    [31]),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_grouped_matches_oracle_whole(name):
    cfgs, seeds = SMALL[name]
    print(f"grouped attention parity: {name}, {len(cfgs)} requests", flush=True)
    group = Group(cfgs, seeds)
    got = group.run()
    ref = attention_grouped(group.tensors["q"], group.tensors["k_tail"], group.tensors["v_tail"],
                            group.k_prefix, group.v_prefix, group.token_offset, group.tail_len,
                            group.request_first, group.prefix_start, group.prefix_len, group.hq,
                            group.hkv, group.scale)
    rows = np.concatenate([np.arange(o, o + n) for o, n in zip(group.token_offset,
                                                                group.tail_len)])
    assert np.isfinite(got[rows]).all()
    err = np.abs(got[rows] - ref[rows]).max()
    print(f"  max abs err {err:.3e} over {rows.size} rows", flush=True)
    assert err <= ATTN_TOL
    _check_bitwise_against_single(group, got, range(len(cfgs)))


# Eight 4B-like requests fill whole rounds of workgroups on 256 CUs; with two or three, the
# units beyond the last full round are re-cut into smaller ones (256 and 128 rows).
@pytest.mark.parametrize("n_req", [8, 2, 3])
def test_4b_like_requests_in_one_launch(n_req):
    cfgs = [synth.config(2)] * n_req
    seeds = [1002 + 100 * r for r in range(n_req)]
    print(f"grouped attention: {n_req} 4B-like requests", flush=True)
    group = Group(cfgs, seeds)
    got = group.run()
    rng = np.random.default_rng(n_req)
    worst = 0.0
    for r in range(n_req):
        req = group.reqs[r]
        picks = sorted({(int(i), int(t), int(rng.integers(req.cfg.n_heads_q)))
                        for i in rng.integers(0, len(req.tail_len), size=12)
                        for t in [0, int(rng.integers(req.tail_len[i])), int(req.tail_len[i]) - 1]})
        ts = req.tensors
        ref = attention_rows(ts["q"], ts["k_tail"], ts["v_tail"], ts["k_prefix"], ts["v_prefix"],
                             req.pack["token_offset"], req.tail_len, req.cfg.n_heads_q,
                             req.cfg.n_heads_kv, req.cfg.scale, picks)
        rows = group.rows_of(r)
        picked = np.stack([got[rows[i][t], h] for i, t, h in picks])
        worst = max(worst, float(np.abs(picked - ref).max()))
    print(f"  max abs err {worst:.3e} over sampled rows of {n_req} requests", flush=True)
    assert worst <= ATTN_TOL
    _check_bitwise_against_single(group, got, [0, n_req - 1])


def test_prepared_launch_holds_its_tables():
    # A prepared grouped launch built from temporary device tables must still read them after
    # the caller has dropped its own references and the allocator has handed out new blocks.
    import torch

    import pass_typed_decision_amd as blink

    cfgs, seeds = SMALL["mixed_prefixes_d128"]
    group = Group(cfgs, seeds)
    q = device_bf16(group.tensors["q"])
    kt, vt = device_bf16(group.tensors["k_tail"]), device_bf16(group.tensors["v_tail"])
    out = torch.full_like(q, float("nan"))
    ga = blink.GroupedAttention(q, kt, vt, device_bf16(group.k_prefix),
                                device_bf16(group.v_prefix), out,
                                torch.as_tensor(group.token_offset).cuda(),
                                torch.as_tensor(group.valid_start).cuda(), group.valid_start,
                                group.request_first, group.prefix_start, group.prefix_len,
                                group.scale)
    clutter = [torch.full((len(group.valid_start) + 64,), 7, dtype=torch.int64, device="cuda")
               for _ in range(8)]
    ga.launch()
    torch.cuda.synchronize()
    del clutter
    got = bf16_to_f32_host(out)
    _check_bitwise_against_single(group, got, range(len(cfgs)))


def test_sixty_four_requests_of_512_questions():
    # The largest group: 64 requests (the whole request table) with 512 questions in all,
    # prefixes of 0..190 tokens (some within one tile, some several), short tails.
    cfgs = [synth.config(2, n_heads_q=8, n_heads_kv=2, prefix_len=(r * 37) % 191,
                         n_questions=8, tail_lo=1, tail_hi=40) for r in range(64)]
    print("grouped attention: 64 requests, 512 questions", flush=True)
    group = Group(cfgs, [500 + r for r in range(64)])
    assert len(group.tail_len) == 512
    got = group.run()
    ref = attention_grouped(group.tensors["q"], group.tensors["k_tail"], group.tensors["v_tail"],
                            group.k_prefix, group.v_prefix, group.token_offset, group.tail_len,
                            group.request_first, group.prefix_start, group.prefix_len, group.hq,
                            group.hkv, group.scale)
    rows = np.concatenate([np.arange(o, o + n) for o, n in zip(group.token_offset,
                                                                group.tail_len)])
    err = np.abs(got[rows] - ref[rows]).max()
    print(f"  max abs err {err:.3e} over {rows.size} rows", flush=True)
    assert np.isfinite(got[rows]).all() and err <= ATTN_TOL
    _check_bitwise_against_single(group, got, [0, 31, 63])
