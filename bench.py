"""Benchmark of one-pass typed-decision scoring on one MI355X.

A step is the whole hot path over one request: host pack of the question tails, upload of the
row tables, shared-prefix tail-prefill attention (HIP), label readout (HIP) writing the label
probabilities and argmax into pinned host memory, and the wait that hands them to the host.
Inputs stay resident in HBM between steps. `value` is the rate of that step run one at a
time, each synchronised before the next is packed; the same steps overlapped two deep (as a
serving loop runs them) are reported beside it.

Default workload: the 27B-like layer slice (40 query / 8 KV heads, head_dim 128, a
65536-token shared prefix, 16 questions with 256-1024-token tails, readout over vocab 151936
x hidden 5120 with 2-16 options per question, temperature 1.0), synthetic seeded data. The
line also carries the 4B-like request's attention (its other matrix-core target) and the
plain max-packing request's readout (the one workload whose readout is bound by HBM), each
timed the same way in the same run.

Prints ONE JSON line (see the "metric" key). The dominant kernel's roofline figure uses HIP
events (without the system-scope fence) recorded on the launch stream around every timed
attention launch; hardware counter figures (HBM bytes, matrix-core busy cycles) are the
rocprofv3 readings stored below for the kernel source they were taken on; the CPU baseline is
the FP64 oracle timed on a bounded sample of the same request.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E

# rocprofv3 readings of the attention per call, keyed by workload number, with the sha256 of
# what decides the attention's device code (its two sources and the build script with their
# flags) at the time they were taken; once any of those changes they read null until counted
# again, or until the device assembly of both builds is shown byte-identical to the counted
# one (a host-only or comment edit), when the key moves to the new sources. HBM bytes = FETCH_SIZE (x2, calibrated on a plain 1 GiB copy) + WRITE_SIZE (x1),
# summed over the call's dispatches (the 27B-like call is a main launch and a merge pass).
# Matrix-core busy = SQ_VALU_MFMA_BUSY_CYCLES over (GRBM_GUI_ACTIVE / 8 XCDs) x 1024 SIMDs, for
# the main launch: the share of the cycles the clock actually ran.
_SHA = "0c83c8613739873b5a62ad2f5433f3f3ddc0987cf35218dbfb3204f3e691c01f"
MEASURED_TRAFFIC = {
    5: (_SHA, 3939117653),
    2: (_SHA, 122346795),
    4: (_SHA, 1536620971),
    3: (_SHA, 1446226923),
}
MEASURED_MFMA_BUSY = {
    5: (_SHA, 0.677),
    2: (_SHA, 0.448),
    4: (_SHA, 0.119),
    3: (_SHA, 0.648),
}
ATTENTION_SOURCES = [os.path.join(ROOT, "pass_typed_decision_amd", *parts) for parts in (
    ("csrc", "blink_attention.hip"), ("csrc", "blink_attention_plain.hip"), ("build.py",))]


def _source_sha() -> str | None:
    import hashlib

    h = hashlib.sha256()
    for path in ATTENTION_SOURCES:
        if not os.path.exists(path):
            return None
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _stored(table: dict, number: int):
    entry = table.get(number)
    if entry is None:
        return None
    return entry[1] if _source_sha() == entry[0] else None


def measured_traffic(number: int):
    return _stored(MEASURED_TRAFFIC, number)


def measured_mfma_busy(number: int):
    return _stored(MEASURED_MFMA_BUSY, number)


def attention_flops(cfg, tail_len) -> float:
    n = np.asarray(tail_len, np.float64)
    return float(4.0 * cfg.head_dim * cfg.n_heads_q * np.sum(n * cfg.prefix_len + n * (n + 1) / 2))


def attention_bytes(cfg, tail_len) -> float:
    valid = float(np.sum(tail_len))
    d = cfg.head_dim
    return (valid * (cfg.n_heads_q + 2 * cfg.n_heads_kv) * d * 2
            + cfg.prefix_len * 2 * cfg.n_heads_kv * d * 2 + valid * cfg.n_heads_q * d * 2)


def readout_bytes(cfg, cand_ids, n) -> float:
    distinct = np.unique(cand_ids).shape[0]
    return float(distinct * cfg.d_model * 2 + n * cfg.d_model * 2 + len(cand_ids) * 12 + 4 * n)


def cpu_baseline(cfg, req_tables, tensors, budget_s: float):
    """The oracle (as it stands) on whole questions of the same request until ~budget_s."""
    from threadpoolctl import threadpool_info

    from oracle.path import score_request

    n = len(req_tables.tail_len)
    done, t0 = 0, time.perf_counter()
    while True:  # whole questions, cycling through the request, until the time budget is used
        score_request(req_tables.tail_len, tensors, req_tables.cand_ids, req_tables.cand_off, cfg,
                      questions=[done % n])
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    elapsed = time.perf_counter() - t0
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    blas_threads = max([i.get("num_threads", 1) for i in blas] or [1])
    cores = len(os.sched_getaffinity(0))
    return {
        "value": done / elapsed,
        "unit": "questions/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{done} questions (cycling over the request's {n}) scored whole (pack, all "
                  f"{cfg.n_heads_q} heads of attention against the {cfg.prefix_len}-token prefix, "
                  f"readout) in {elapsed:.1f} s; float64 numpy, "
                  f"{blas[0].get('internal_api', 'blas') if blas else 'blas'} with "
                  f"{blas_threads} threads on {cores} host cores",
    }


class TimingEvents:
    """HIP events recorded on the launch stream, created without the system-scope fence: a
    timing-only event then adds no cache write-back and invalidation between the kernels it
    brackets (the HIP runtime's own recommendation for events used only to time work)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, count: int, stream):
        import ctypes

        hip = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD)
        self.ctypes, self.hip = ctypes, hip
        self.stream = ctypes.c_void_p(stream.cuda_stream)
        self.events = []
        for _ in range(count):
            ev = ctypes.c_void_p()
            self._check(hip.hipEventCreateWithFlags(ctypes.byref(ev),
                                                    ctypes.c_uint(self.DISABLE_SYSTEM_FENCE)))
            self.events.append(ev)

    @staticmethod
    def _check(rc):
        if rc != 0:
            raise RuntimeError(f"HIP event call failed with error {rc}")

    def record(self, i: int):
        self._check(self.hip.hipEventRecord(self.events[i], self.stream))

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = self.ctypes.c_float()
        self._check(self.hip.hipEventElapsedTime(self.ctypes.byref(ms), self.events[a],
                                                 self.events[b]))
        return ms.value

    def close(self):
        for ev in self.events:
            self.hip.hipEventDestroy(ev)
        self.events = []


def prefix_encode(cfg, tables, tensors, stream, reps: int = 5) -> dict:
    """The request's one-off work before its steps: the shared-prefix plan (host) and the
    prefix's own causal prefill (attention of one question of prefix_len tokens, no prefix),
    timed with HIP events on the step stream. The step itself reads the cached prefix K/V."""
    import torch

    import pass_typed_decision_amd as blink
    import synth

    p = cfg.prefix_len
    # Token sequences of the request (synthetic ids): the shared prefix, then each
    # question's own tail, whose first token differs from every other question's.
    rng = np.random.Generator(np.random.PCG64(3000 + cfg.number))
    head = rng.integers(0, cfg.vocab, size=p).tolist()
    seqs = [head + [int(i)] + rng.integers(0, cfg.vocab, size=int(t) - 1).tolist()
            for i, t in enumerate(tables.tail_len)]
    t0 = time.perf_counter()
    plan = blink.plan_prefix(seqs)
    plan_ms = (time.perf_counter() - t0) * 1e3
    if plan.prefix_len != p:
        raise RuntimeError(f"prefix plan found {plan.prefix_len} shared tokens, expected {p}")
    q = torch.from_numpy(synth.draw_prefix_queries(cfg).view(np.int16)).view(
        torch.bfloat16).cuda()
    out = torch.empty_like(q)
    # Checked once against encode_prefix_attention's own launch, then launched from a prepared
    # argument list (one question: the whole prefix as its tail, no prefix) as the step does.
    tables = blink.encode_prefix_attention(q, tensors["k_prefix"], tensors["v_prefix"], out,
                                           cfg.scale, stream=stream.cuda_stream)
    lib = blink.load_library()
    args = blink.prefix_tail_attention(q, tensors["k_prefix"], tensors["v_prefix"], None, None,
                                       out, tables[0], tables[1], p, cfg.scale,
                                       stream=stream.cuda_stream, launch=False)

    def launch():
        rc = lib.blink_prefix_tail_attention(*args)
        if rc != 0:
            raise RuntimeError(lib.blink_last_error().decode())

    ev = TimingEvents(2 * reps, stream)
    launch()
    torch.cuda.synchronize()
    for i in range(reps):
        ev.record(2 * i)
        launch()
        ev.record(2 * i + 1)
    torch.cuda.synchronize()
    ms = float(np.mean([ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(reps)]))
    ev.close()
    flops = 4.0 * cfg.head_dim * cfg.n_heads_q * p * (p + 1) / 2
    return {"tokens": p, "attention_ms": ms, "tflops": flops / (ms * 1e-3) / 1e12,
            "mfma_frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "work_per_launch": f"{flops:.4e} FLOP", "plan_host_ms": plan_ms,
            "prefill_tokens_per_request": plan.prefill_tokens,
            "plain_path_tokens_per_request": int(sum(len(x) for x in seqs))}


def grouped_attention(cfg, n_req: int, stream, reps: int = 10) -> dict:
    """R requests of the workload's shape (seeds 1000 + workload + 100 r), each with its own
    prefix, in one blink_prefix_tail_attention_grouped launch, against R single launches."""
    import torch

    import pass_typed_decision_amd as blink
    import synth

    parts = ("q", "k_tail", "v_tail", "k_prefix", "v_prefix")
    tails, offs, tens, pre_k, pre_v = [], [], {k: [] for k in parts[:3]}, [], []
    base = 0
    flops = 0.0
    singles = []
    for r in range(n_req):
        rng = synth.rng_for(cfg, seed=1000 + cfg.number + 100 * r)
        tables = synth.draw_tables(cfg, rng)
        pk = blink.pack_ragged(tables.tail_len, cfg.prefix_len, cfg.token_budget, cfg.max_rows)
        host = synth.draw_tensors(cfg, rng, pk.total_padded_tokens, parts)
        tails.append(tables.tail_len)
        offs.append(pk.token_offset + base)
        base += pk.total_padded_tokens
        for k in parts[:3]:
            tens[k].append(host[k])
        if cfg.prefix_len:
            pre_k.append(host["k_prefix"])
            pre_v.append(host["v_prefix"])
        flops += attention_flops(cfg, tables.tail_len)
        singles.append((tables.tail_len, pk, host))

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).cuda()

    tail_len = np.concatenate(tails).astype(np.int32)
    vs = np.concatenate([[0], np.cumsum(tail_len)]).astype(np.int32)
    q, kt, vt = (dev(np.concatenate(tens[k])) for k in parts[:3])
    kp = dev(np.concatenate(pre_k)) if pre_k else None
    vp = dev(np.concatenate(pre_v)) if pre_v else None
    out = torch.empty_like(q)
    first = np.concatenate([[0], np.cumsum([len(t) for t in tails])]).astype(np.int32)
    plen = np.full(n_req, cfg.prefix_len, np.int32)
    pstart = (np.arange(n_req) * cfg.prefix_len).astype(np.int64)
    ga = blink.GroupedAttention(q, kt, vt, kp, vp, out,
                                torch.as_tensor(np.concatenate(offs).astype(np.int64)).cuda(),
                                torch.as_tensor(vs).cuda(), vs, first, pstart, plen, cfg.scale,
                                stream=stream.cuda_stream)
    # One request at a time, each its own launch over its own buffers.
    lib = blink.load_library()
    single_args = []
    keep = []
    for tl, pk, host in singles:
        t = {k: dev(host[k]) for k in parts if host[k].size}
        o = torch.empty_like(t["q"])
        d_off = torch.as_tensor(pk.token_offset.astype(np.int64)).cuda()
        d_vs = torch.as_tensor(pk.valid_start).cuda()
        keep.append((t, o, d_off, d_vs))
        single_args.append(blink.prefix_tail_attention(
            t["q"], t["k_tail"], t["v_tail"], t.get("k_prefix"), t.get("v_prefix"), o, d_off,
            d_vs, pk.total_valid_tokens, cfg.scale, stream=stream.cuda_stream, launch=False))

    def run_singles():
        for a in single_args:
            if lib.blink_prefix_tail_attention(*a) != 0:
                raise RuntimeError(lib.blink_last_error().decode())

    ev = TimingEvents(4 * reps, stream)
    ga.launch()
    run_singles()
    torch.cuda.synchronize()
    for i in range(reps):
        ev.record(4 * i)
        ga.launch()
        ev.record(4 * i + 1)
        ev.record(4 * i + 2)
        run_singles()
        ev.record(4 * i + 3)
    torch.cuda.synchronize()
    g_ms = float(np.mean([ev.elapsed_ms(4 * i, 4 * i + 1) for i in range(reps)]))
    s_ms = float(np.mean([ev.elapsed_ms(4 * i + 2, 4 * i + 3) for i in range(reps)]))
    ev.close()
    return {"requests": n_req, "questions": int(len(tail_len)), "attention_ms": g_ms,
            "tflops": flops / (g_ms * 1e-3) / 1e12,
            "mfma_frac": flops / (g_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "one_launch_per_request_ms": s_ms, "speedup": s_ms / g_ms,
            "work_per_launch": f"{flops:.4e} FLOP"}


def grouped_step(number: int, n_req: int, stream, steps: int = 20, warmup: int = 3) -> dict:
    """R requests of the numbered workload's shape (seeds 1000 + workload + 100 r), each with
    its own prefix, scored together by one GroupedScoringStep (one grouped attention launch and
    one readout), against the same R requests scored one ScoringStep after another. Both loops
    synchronise every step and bring the results to the host."""
    import torch

    import pass_typed_decision_amd as blink
    import synth

    cfg = synth.config(number)
    parts = ("q", "k_tail", "v_tail", "k_prefix", "v_prefix", "hidden")
    reqs, host, base, pstart = [], {k: [] for k in parts}, 0, 0
    for r in range(n_req):
        rng = synth.rng_for(cfg, seed=1000 + cfg.number + 100 * r)
        tables = synth.draw_tables(cfg, rng)
        pk = blink.pack_ragged(tables.tail_len, cfg.prefix_len, cfg.token_budget, cfg.max_rows)
        t = synth.draw_tensors(cfg, rng, pk.total_padded_tokens, parts)
        for k in parts:
            host[k].append(t[k])
        reqs.append((tables, pk, base, pstart))
        base += pk.total_padded_tokens
        pstart += cfg.prefix_len
    w_rng = np.random.Generator(np.random.PCG64(5000 + cfg.number))
    w_u = synth.f32_to_bf16_bits(
        (w_rng.standard_normal((cfg.vocab, cfg.d_model), dtype=np.float32) * cfg.w_u_std))
    dev = {k: _dev(np.concatenate(v)) for k, v in host.items() if sum(x.size for x in v)}
    dev["w_u"] = _dev(w_u)
    del host, w_u
    group = blink.GroupedScoringStep(
        [blink.GroupRequest(tb.tail_len, tb.cand_ids, tb.cand_off, b, ps, cfg.prefix_len)
         for tb, _, b, ps in reqs], dev, cfg.n_heads_q, cfg.n_heads_kv, cfg.temperature,
        cfg.scale, cfg.token_budget, cfg.max_rows, stream=stream)
    singles = []
    for tb, pk, b, ps in reqs:
        t = {k: dev[k][b:b + pk.total_padded_tokens] for k in ("q", "k_tail", "v_tail", "hidden")}
        if cfg.prefix_len:
            t["k_prefix"] = dev["k_prefix"][ps:ps + cfg.prefix_len]
            t["v_prefix"] = dev["v_prefix"][ps:ps + cfg.prefix_len]
        t["w_u"] = dev["w_u"]
        singles.append(blink.ScoringStep(tb.tail_len, tb.cand_ids, tb.cand_off, t,
                                         cfg.n_heads_q, cfg.n_heads_kv, cfg.prefix_len,
                                         cfg.temperature, cfg.scale, cfg.token_budget,
                                         cfg.max_rows, stream=stream))
    for _ in range(warmup):
        group.run()
        for st in singles:
            st.run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        res = group.run()
    t_group = time.perf_counter() - t0
    t0 = time.perf_counter()
    for _ in range(steps):
        for st in singles:
            st.run()
    t_single = time.perf_counter() - t0
    # The group gives each request exactly its single-request probabilities.
    for st, (probs, arg) in zip(singles, res):
        p1, a1 = st.run()
        if not (np.array_equal(np.concatenate(probs), p1) and np.array_equal(arg, a1)):
            raise RuntimeError("grouped step differs from single-request steps")
    n_q = sum(len(tb.tail_len) for tb, _, _, _ in reqs)
    for st in singles:
        st.close()
    del group, singles, dev
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {"workload": f"{n_req} requests of {cfg.name} (config {cfg.number}), each with its "
                        f"own {cfg.prefix_len}-token prefix", "questions": n_q,
            "grouped_questions_per_s": n_q * steps / t_group,
            "grouped_ms_per_step": t_group * 1e3 / steps,
            "one_step_per_request_questions_per_s": n_q * steps / t_single,
            "speedup": t_single / t_group, "checked_equal_to_single_requests": True}


def teacher_forced_scoring(cfg, tables, pk, tensors, stream, score_len: int = 8,
                           reps: int = 10) -> dict:
    """The request's questions scored teacher-forced on their last score_len tokens: the rows
    n_i - score_len - 1 .. n_i - 2 of each tail (shorter tails give what they have), each
    against a synthetic next token, log-softmax over the whole vocabulary (blink_score_targets)."""
    import torch

    import pass_typed_decision_amd as blink

    rng = np.random.Generator(np.random.PCG64(4000 + cfg.number))
    rows = []
    for off, n in zip(pk.token_offset, tables.tail_len):
        lo = max(0, int(n) - score_len - 1)
        rows.extend(int(off) + i for i in range(lo, int(n) - 1))
    targets = rng.integers(0, cfg.vocab, size=len(rows)).astype(np.int32)
    sc = blink.TargetScorer(tensors["hidden"], tensors["w_u"],
                            torch.as_tensor(np.asarray(rows, np.int64)).cuda(),
                            torch.as_tensor(targets).cuda(), stream=stream.cuda_stream)
    ev = TimingEvents(2 * reps, stream)
    sc.run()
    torch.cuda.synchronize()
    for i in range(reps):
        ev.record(2 * i)
        sc.run()
        ev.record(2 * i + 1)
    torch.cuda.synchronize()
    ms = float(np.mean([ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(reps)]))
    ev.close()
    # The library's product of the same shape, logits only (no log-softmax, bf16 logits
    # written out): W [vocab, d_model] times the scored rows' transpose, both contiguous.
    h_t = tensors["hidden"][torch.as_tensor(np.asarray(rows, np.int64)).cuda()].t().contiguous()
    w = tensors["w_u"]
    ev = TimingEvents(2 * reps, stream)
    torch.mm(w, h_t)
    torch.cuda.synchronize()
    for i in range(reps):
        ev.record(2 * i)
        torch.mm(w, h_t)
        ev.record(2 * i + 1)
    torch.cuda.synchronize()
    lib_ms = float(np.median([ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(reps)]))
    ev.close()
    del h_t
    m = len(rows)
    flops = 2.0 * m * cfg.vocab * cfg.d_model
    wbytes = float(cfg.vocab) * cfg.d_model * 2 + m * cfg.d_model * 2
    return {"rows": m, "score_len": score_len, "ms": ms,
            "tflops": flops / (ms * 1e-3) / 1e12,
            "mfma_frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "hbm_gbps": wbytes / (ms * 1e-3) / 1e9,
            "hbm_frac": wbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "work_per_call": f"{flops:.4e} FLOP, {wbytes:.4e} B",
            "library_logits_gemm_ms": lib_ms,
            "library_logits_gemm_hbm_frac": wbytes / (lib_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "frac_of_library_reference": lib_ms / ms,
            "library_what": "torch.mm(W_U, H^T) bf16, the same shape, logits only; median of "
                            f"{reps}"}


def library_references(stream, reps: int = 10) -> dict:
    """What the vendor libraries reach on this device, measured beside the vendor peaks: a
    large square bf16 matrix product (torch.matmul, i.e. hipBLASLt) and a 1 GiB streaming read
    (torch's sum over the buffer). They are practical reference points, not peaks: this path's
    kernels can exceed them."""
    import torch

    n = 8192
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    buf = torch.ones(1 << 28, device="cuda", dtype=torch.float32)  # 1 GiB
    ev = TimingEvents(4 * reps, stream)
    torch.matmul(a, b)
    buf.sum()
    torch.cuda.synchronize()
    for i in range(reps):
        ev.record(4 * i)
        torch.matmul(a, b)
        ev.record(4 * i + 1)
        ev.record(4 * i + 2)
        buf.sum()
        ev.record(4 * i + 3)
    torch.cuda.synchronize()
    gemm_ms = float(np.median([ev.elapsed_ms(4 * i, 4 * i + 1) for i in range(reps)]))
    read_ms = float(np.median([ev.elapsed_ms(4 * i + 2, 4 * i + 3) for i in range(reps)]))
    ev.close()
    del a, b, buf
    torch.cuda.empty_cache()
    return {"bf16_gemm_tflops": 2.0 * n ** 3 / (gemm_ms * 1e-3) / 1e12,
            "hbm_read_gbps": float(1 << 30) / (read_ms * 1e-3) / 1e9,
            "what": "torch.matmul 8192^3 bf16; sum over a 1 GiB float32 buffer; medians of "
                    f"{reps}"}


def _dev(bits):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def make_request(number: int, stream, readout: str = "per_option", depth: int = 1):
    """Seeded request of the numbered workload, resident on the device, and its scoring step."""
    import synth
    import pass_typed_decision_amd as blink

    cfg = synth.config(number)
    rng = synth.rng_for(cfg)
    tables = synth.draw_tables(cfg, rng)
    pk = blink.pack_ragged(tables.tail_len, cfg.prefix_len, cfg.token_budget, cfg.max_rows)
    host = synth.draw_tensors(cfg, rng, pk.total_padded_tokens)
    tensors = {k: _dev(v) for k, v in host.items() if v.size}
    if cfg.prefix_len == 0:
        tensors.pop("k_prefix", None)
        tensors.pop("v_prefix", None)
    step = blink.ScoringStep(tables.tail_len, tables.cand_ids, tables.cand_off, tensors,
                             cfg.n_heads_q, cfg.n_heads_kv, cfg.prefix_len, cfg.temperature,
                             cfg.scale, cfg.token_budget, cfg.max_rows, stream=stream,
                             readout=readout, depth=depth)
    return cfg, tables, pk, host, tensors, step


def time_sequential(step, steps: int, warmup: int, stream):
    """`steps` whole steps, each synchronised before the next is packed, with HIP events on
    the step's stream around its attention and its readout. Returns (per-step attention ms,
    per-step readout ms, wall seconds for all steps)."""
    import torch

    for _ in range(warmup):
        step.run()
    torch.cuda.synchronize()
    ev = TimingEvents(3 * steps, stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        total_valid = step.pack_and_upload()
        ev.record(3 * i)
        step.attention(total_valid)
        ev.record(3 * i + 1)
        step.readout()
        ev.record(3 * i + 2)
        stream.synchronize()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    attn = np.array([ev.elapsed_ms(3 * i, 3 * i + 1) for i in range(steps)])
    read = np.array([ev.elapsed_ms(3 * i + 1, 3 * i + 2) for i in range(steps)])
    ev.close()
    return attn, read, elapsed


def attention_dispatches(cfg, tail_len) -> int:
    """Kernel dispatches of one attention call: two when the launch takes the key split of the
    last round (main launch and merge pass), else one."""
    import pass_typed_decision_amd as blink

    ws = blink.attention_workspace(int(np.sum(tail_len)), cfg.n_heads_q, cfg.n_heads_kv,
                                   cfg.head_dim, cfg.prefix_len)
    return 1 if ws is None else 2


def attention_roofline(cfg, tail_len, attn_ms: float) -> dict:
    """The attention call against its roofline: algorithmic FLOPs (or bytes, for the plain path)
    over the event time of the whole call (all its dispatches)."""
    flops = attention_flops(cfg, tail_len)
    abytes = attention_bytes(cfg, tail_len)
    common = {"kernel": "prefix_tail_attention_kernel",
              "dispatches_per_call": attention_dispatches(cfg, tail_len)}
    if cfg.prefix_len > 0:
        achieved = flops / (attn_ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "work_per_launch": f"{flops:.4e} FLOP", **common}
    achieved = abytes / (attn_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBPS, "work_per_launch": f"{abytes:.4e} B", **common}


def secondary(number: int, stream, steps: int = 20, warmup: int = 5,
              readout: str = "per_option") -> dict:
    """Another workload's step, timed the same way (sequential steps, events around each
    kernel): its attention against the matrix-core or HBM peak and its readout against HBM."""
    import torch

    cfg, tables, pk, host, tensors, step = make_request(number, stream, readout=readout)
    del host
    attn, read, elapsed = time_sequential(step, steps, warmup, stream)
    attn_ms, read_ms = float(attn.mean()), float(read.mean())
    rbytes = readout_bytes(cfg, tables.cand_ids, cfg.n_questions)
    out = {
        "workload": f"{cfg.name} (config {cfg.number})",
        "questions_per_s": cfg.n_questions * steps / elapsed,
        "ms_per_step": elapsed * 1e3 / steps,
        "attention_ms": attn_ms,
        "attention": attention_roofline(cfg, tables.tail_len, attn_ms),
        "attention_hbm_bytes_counted": measured_traffic(number),
        "attention_mfma_busy_counted": measured_mfma_busy(number),
        "readout_ms": read_ms,
        "readout_form": step.readout_form,
        "readout_algorithmic_bytes": rbytes,
        "readout_gbps": rbytes / (read_ms * 1e-3) / 1e9,
        "readout_hbm_frac": rbytes / (read_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "steps": steps,
    }
    step.close()
    del step, tensors
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=5, help="workload number (1-5)")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--also", default="2,4",
                    help="other workloads whose attention and readout are timed in the same run "
                         "(comma-separated numbers, empty for none)")
    ap.add_argument("--depth", type=int, default=2,
                    help="steps in flight in the overlapped serving loop reported beside the "
                         "sequential rate (1-4)")
    ap.add_argument("--group", type=int, default=0, metavar="R",
                    help="also time R requests of the workload's shape, each with its own "
                         "prefix, in one grouped attention launch")
    ap.add_argument("--group-step", default="2:8", metavar="N:R",
                    help="also score R requests of workload N, each with its own prefix, in one "
                         "grouped step (empty for none)")
    ap.add_argument("--readout", default="per_option", choices=("per_option", "batched"),
                    help="readout form: per option (default), or batched over the distinct "
                         "label rows")
    ap.add_argument("--only-attention", type=int, default=0, metavar="REPS",
                    help="profiling aid: launch the workload's attention REPS times after one "
                         "step and exit without a bench line")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run one plain device copy of this many MiB (the known-size "
                         "reference for hardware byte counters) and exit after it")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the scoring path "
              "runs on a single device)", file=sys.stderr)
        sys.exit(2)

    import torch

    import pass_typed_decision_amd as blink

    if args.copy_calibration:
        n_bytes = args.copy_calibration << 20
        src = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n_bytes}), flush=True)
        return

    stream = torch.cuda.current_stream()
    cfg, tables, pk, host, tensors, step = make_request(args.config, stream,
                                                        readout=args.readout, depth=args.depth)
    if args.only_attention:
        step.run()
        for _ in range(args.only_attention):
            step.attention(pk.total_valid_tokens)
        torch.cuda.synchronize()
        print(json.dumps({"attention_launches": args.only_attention}), flush=True)
        return
    label_pack_ms = None
    if step.readout_form == "batched":
        # The distinct-row table is built once per request, with the option table's upload;
        # its host cost is reported beside the step, not inside it.
        reps = 20
        t_lp = time.perf_counter()
        for _ in range(reps):
            blink.pack_labels(tables.cand_ids, tables.cand_off, cfg.vocab)
        label_pack_ms = (time.perf_counter() - t_lp) * 1e3 / reps

    attn_each, read_each, elapsed = time_sequential(step, args.steps, args.warmup, stream)

    # The same K steps again as a serving loop runs them: step i + 1 is packed and queued
    # while step i runs (two slots of host buffers), and each step's results are collected
    # from pinned host memory once its completion event has fired. Every step still packs,
    # uploads, runs attention and readout and brings its results to the host.
    for _ in range(2):
        step.submit()
        step.collect()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step.submit()
        if step.outstanding() == args.depth:
            step.collect()
    while step.outstanding():
        step.collect()
    torch.cuda.synchronize()
    elapsed_pipelined = time.perf_counter() - t0

    # Untimed check: overlapped steps give bitwise the results of a synchronised step.
    ref_probs, ref_arg = (x.copy() for x in step.run())
    for i in range(2 * args.depth):
        step.submit()
        if step.outstanding() == args.depth or i == 2 * args.depth - 1:
            while step.outstanding():
                probs, arg = step.collect()
                if not (np.array_equal(probs, ref_probs) and np.array_equal(arg, ref_arg)):
                    raise RuntimeError("overlapped steps differ from a synchronised step")

    attn_ms, read_ms = float(attn_each.mean()), float(read_each.mean())
    flops = attention_flops(cfg, tables.tail_len)
    rbytes = readout_bytes(cfg, tables.cand_ids, cfg.n_questions)
    n = cfg.n_questions
    roof = attention_roofline(cfg, tables.tail_len, attn_ms)
    roof["traffic"] = measured_traffic(cfg.number)
    roof["traffic_unit"] = "HBM bytes per attention call (all its dispatches)"
    roof["mfma_busy_counted"] = measured_mfma_busy(cfg.number)
    roof["launch_ms"] = attn_ms

    prefix = prefix_encode(cfg, tables, tensors, stream) if cfg.prefix_len > 0 else None
    grouped = grouped_attention(cfg, args.group, stream) if args.group > 1 else None
    scoring = teacher_forced_scoring(cfg, tables, pk, tensors, stream)
    step.close()
    del step, tensors
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    others = {}
    for number in [int(x) for x in args.also.split(",") if x.strip()]:
        if number != cfg.number:
            others[synth_name(number)] = secondary(number, stream, readout=args.readout)

    group_step = None
    if args.group_step:
        g_num, g_req = (int(x) for x in args.group_step.split(":"))
        group_step = grouped_step(g_num, g_req, stream)

    refs = library_references(stream)
    roof["frac_of_library_reference"] = roof["achieved"] / (
        refs["bf16_gemm_tflops"] if roof["bound"] == "mfma" else refs["hbm_read_gbps"])

    baseline = None
    if not args.no_cpu_baseline:
        baseline = cpu_baseline(cfg, tables, host, args.cpu_budget)

    line = {
        "metric": "scored questions/s (one request = pack + tail-prefix attention + label readout)",
        "value": n * args.steps / elapsed,
        "unit": "questions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name} (config {cfg.number}): {cfg.n_heads_q} q / {cfg.n_heads_kv} kv "
                        f"heads, head_dim {cfg.head_dim}, prefix {cfg.prefix_len}, {n} questions "
                        f"with tails {cfg.tail_lo}-{cfg.tail_hi}, hidden {cfg.d_model}, vocab "
                        f"{cfg.vocab}, options {cfg.k_lo}-{cfg.k_hi}, T {cfg.temperature}",
            "questions": n,
            "valid_tail_tokens": int(np.sum(tables.tail_len)),
            "padded_tokens": pk.total_padded_tokens,
            "batches": pk.n_batches,
            "parallelism": "single GPU",
        },
        "roofline": roof,
        "kernels": {
            "attention_ms": attn_ms,
            "attention_tflops": flops / (attn_ms * 1e-3) / 1e12,
            # Algorithmic FLOPs over event time and the 2.5 PFLOP/s vendor peak (not a counter).
            "attention_algorithmic_mfma_frac": flops / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "readout_ms": read_ms,
            "readout_gbps": rbytes / (read_ms * 1e-3) / 1e9,
            "readout_hbm_frac": rbytes / (read_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "readout_algorithmic_bytes": rbytes,
            # Spread over the timed steps (median, 10th and 90th percentile, ms).
            "attention_ms_p50_p10_p90": [float(np.percentile(attn_each, q)) for q in (50, 10, 90)],
            "readout_ms_p50_p10_p90": [float(np.percentile(read_each, q)) for q in (50, 10, 90)],
            # Questions per second of GPU kernel time alone (attention + readout), without the
            # host pack, the table upload and the synchronisation that `value` includes.
            "kernel_only_questions_per_s": n / ((attn_ms + read_ms) * 1e-3),
            # The same steps overlapped `depth` deep (step i + 1 packed and queued while step i
            # runs on a second stream): a serving loop's rate, not a single step's.
            "overlapped_questions_per_s": n * args.steps / elapsed_pipelined,
            "overlapped_ms_per_step": elapsed_pipelined * 1e3 / args.steps,
            "overlapped_depth": args.depth,
            "overlapped_steps_checked_bitwise": True,
            "readout_form": args.readout,
            "label_pack_host_ms_once_per_request": label_pack_ms,
        },
        "secondary": others,
        "prefix_encode_once_per_request": prefix,
        "grouped_requests": grouped,
        "grouped_step": group_step,
        "teacher_forced_scoring": scoring,
        "library_references": refs,
        "cpu_baseline": baseline,
    }
    print(json.dumps(line), flush=True)


def synth_name(number: int) -> str:
    import synth

    return synth.config(number).name


if __name__ == "__main__":
    main()
