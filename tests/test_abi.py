"""The C ABI on the host (no GPU): the library loads, exports every symbol the header
declares, packs bit-exactly like the oracle, and refuses bad arguments before any launch."""

import ctypes
import os
import re

import numpy as np
import pytest

from helpers import ROOT
from oracle.pack import pack_ragged as oracle_pack
from oracle.readout import label_rows as oracle_label_rows
from oracle.prefix import plan_prefix as oracle_plan_prefix
from oracle.answers import assemble as oracle_assemble
from oracle import refine as oracle_refine

HEADER = os.path.join(ROOT, "include", "blink.h")


@pytest.fixture(scope="module")
def blink():
    import pass_typed_decision_amd as b
    from pass_typed_decision_amd import build

    if not os.path.exists(b.LIBRARY):
        build.build()
    b.load_library()
    return b


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(blink_\w+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(__import__("pass_typed_decision_amd").EXPORTS)


def test_library_exports_every_declared_symbol(blink):
    lib = ctypes.CDLL(blink.LIBRARY)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert blink.load_library().blink_abi_version() == 9


def _compare(pk, ref):
    for key in ("order", "batch_of", "row_of", "token_offset", "last_row", "batch_first",
                "batch_width", "batch_base"):
        np.testing.assert_array_equal(getattr(pk, key), ref[key], err_msg=key)
    assert pk.n_batches == ref["n_batches"]
    assert pk.total_padded_tokens == ref["total_padded_tokens"]
    assert pk.total_valid_tokens == ref["total_valid_tokens"]


def test_pack_matches_oracle_on_golden(blink):
    import json

    with open(os.path.join(ROOT, "tests", "golden", "pack_cases.json")) as f:
        for case in json.load(f)["cases"]:
            pk = blink.pack_ragged(case["tail_len"], 0, case["budget"], case["max_rows"])
            _compare(pk, oracle_pack(case["tail_len"], case["budget"], case["max_rows"]))


def test_pack_matches_oracle_random(blink):
    rng = np.random.default_rng(123)
    for _ in range(3000):
        n = int(rng.integers(1, 513))
        hi = int(rng.choice([3, 40, 600, 5000, 131072]))
        lengths = rng.integers(1, hi + 1, size=n)
        budget = int(rng.choice([1, 16, 500, 32768, 65536]))
        max_rows = int(rng.choice([0, 0, 1, 4, 56]))
        pk = blink.pack_ragged(lengths, 0, budget, max_rows)
        _compare(pk, oracle_pack(lengths.tolist(), budget, max_rows))
        vs = np.concatenate([[0], np.cumsum(lengths)])
        np.testing.assert_array_equal(pk.valid_start, vs)


def test_prepared_pack_call_matches_pack_ragged(blink):
    # The scoring step calls the packer through a prepared argument list that writes the
    # row tables into one shared buffer (int64 offsets, int64 last rows, int32 starts).
    import ctypes

    from pass_typed_decision_amd._binding import pack_ragged_args

    rng = np.random.default_rng(7)
    lib = blink.load_library()
    for _ in range(200):
        n = int(rng.integers(1, 513))
        lengths = rng.integers(1, int(rng.choice([5, 300, 4000])) + 1, size=n).astype(np.int32)
        budget, max_rows = int(rng.choice([64, 32768])), int(rng.choice([0, 3]))
        tab = np.full(2 * n + (n + 2) // 2, -7, np.int64)
        offs, last, vs = tab[:n], tab[n:2 * n], tab[2 * n:].view(np.int32)[:n + 1]
        extra = [np.zeros(n, np.int32) for _ in range(3)] + [
            np.zeros(n + 1, np.int32), np.zeros(n, np.int32), np.zeros(n + 1, np.int64)]
        nb, tp, tv = ctypes.c_int32(0), ctypes.c_int64(0), ctypes.c_int64(0)
        args = pack_ragged_args(lengths, 0, budget, max_rows, extra[0], extra[1], extra[2], offs,
                                last, vs, extra[3], extra[4], extra[5], nb, tp, tv)
        assert lib.blink_pack_ragged(*args) == 0
        pk = blink.pack_ragged(lengths, 0, budget, max_rows)
        np.testing.assert_array_equal(offs, pk.token_offset)
        np.testing.assert_array_equal(last, pk.last_row)
        np.testing.assert_array_equal(vs, pk.valid_start)
        np.testing.assert_array_equal(extra[0], pk.order)
        assert (nb.value, tp.value, tv.value) == (
            pk.n_batches, pk.total_padded_tokens, pk.total_valid_tokens)
    with pytest.raises(blink.BlinkError):
        pack_ragged_args(lengths, 0, budget, max_rows, extra[0], extra[1], extra[2],
                         offs.astype(np.int32), last, vs, extra[3], extra[4], extra[5], nb, tp, tv)


@pytest.mark.parametrize("lengths, prefix, code, msg", [
    ([], 0, -2, "request of 0 questions; the limit is 1 to 512"),
    ([1] * 513, 0, -2, "request of 513 questions; the limit is 1 to 512"),
    ([4, 0], 0, -1, "question 1 has an empty tail"),
    ([5, 2], 131068, -2, "question 0 needs 131073 tokens of context; the maximum context length is 131072"),
    ([3], -1, -1, "prefix length must be non-negative"),
])
def test_pack_refusals(blink, lengths, prefix, code, msg):
    with pytest.raises(blink.BlinkError) as e:
        blink.pack_ragged(lengths, prefix)
    assert e.value.code == code and msg in str(e.value)


def test_pack_limits_accepted(blink):
    pk = blink.pack_ragged([1] * 512, 131071)
    assert pk.n_batches == 1 and pk.total_padded_tokens == 512
    blink.pack_ragged([4, 2], 131068)


def _readout(lib, temperature=1.0, n=2, max_options=4, d_model=256, total=4):
    fake = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    return lib.blink_label_readout(fake, 10, d_model, fake, fake, 100, fake, fake, n, total,
                                   max_options, temperature, fake, fake, fake, None)


@pytest.mark.parametrize("kw, code, msg", [
    (dict(temperature=0.0), -1, "temperature is not a positive finite number"),
    (dict(temperature=-0.5), -1, "temperature is not a positive finite number"),
    (dict(temperature=float("nan")), -1, "temperature is not a positive finite number"),
    (dict(temperature=float("inf")), -1, "temperature is not a positive finite number"),
    (dict(n=0), -2, "request of 0 questions; the limit is 1 to 512"),
    (dict(n=513), -2, "request of 513 questions; the limit is 1 to 512"),
    (dict(max_options=256), -2, "question with 256 options; the limit is 1 to 255"),
    (dict(max_options=0), -2, "question with 0 options; the limit is 1 to 255"),
    (dict(d_model=100), -1, "d_model 100 must be a multiple of 8"),
    (dict(total=1), -1, "does not fit"),
])
def test_readout_refusals_before_launch(blink, kw, code, msg):
    lib = blink.load_library()
    rc = _readout(lib, **kw)
    assert rc == code
    assert msg in lib.blink_last_error().decode()


def _attention(lib, n=2, total=10, t_pad=12, prefix=0, hq=4, hkv=1, d=64, scale=0.125,
               null_prefix=True, workspace=None):
    fake = ctypes.c_void_p(256)
    pre = None if null_prefix else fake
    return lib.blink_prefix_tail_attention(fake, fake, fake, pre, pre, fake, fake, fake, n,
                                           total, t_pad, prefix, hq, hkv, d, scale, workspace,
                                           1 << 20 if workspace else 0, None)


@pytest.mark.parametrize("kw, code, msg", [
    (dict(n=0), -2, "request of 0 questions; the limit is 1 to 512"),
    (dict(d=96), -1, "head_dim 96 is not supported"),
    (dict(hq=6, hkv=4), -1, "head counts 6/4"),
    (dict(hq=34, hkv=2), -1, "group <= 16"),
    (dict(scale=0.0), -1, "scale must be finite and positive"),
    (dict(prefix=5), -1, "prefix K/V pointers are NULL"),
    (dict(prefix=131072, null_prefix=False), -2, "maximum context length is 131072"),
    (dict(total=20, t_pad=12), -1, "token totals do not fit"),
    (dict(total=1), -1, "token totals do not fit"),
    (dict(workspace=ctypes.c_void_p(264)), -1, "workspace must be 16-byte aligned"),
])
def test_attention_refusals_before_launch(blink, kw, code, msg):
    lib = blink.load_library()
    assert _attention(lib, **kw) == code
    assert msg in lib.blink_last_error().decode()


def test_attention_workspace_query_refuses_bad_sizes(blink):
    # Sizes the launch would refuse ask for no workspace (without a device every size gets 0).
    lib = blink.load_library()
    for args in [(0, 32, 8, 128, 2048), (5000, 6, 4, 128, 0), (5000, 32, 8, 96, 2048),
                 (5000, 32, 8, 128, -1), (512 * 131072 + 1, 32, 8, 128, 0)]:
        assert lib.blink_prefix_tail_attention_workspace(*args) == 0


def test_error_text_is_cleared_by_success(blink):
    lib = blink.load_library()
    assert _readout(lib, temperature=0.0) == -1
    blink.pack_ragged([3, 4])
    assert lib.blink_last_error() == b""


def test_label_names():
    from pass_typed_decision_amd import label_name

    assert [label_name(i) for i in (0, 1, 25, 26, 27, 51, 52, 254)] == \
        ["A", "B", "Z", "AA", "AB", "AZ", "BA", "IU"]
    with pytest.raises(ValueError):
        label_name(255)


def _compare_label_rows(lr, ids, off):
    row_id, row_first, row_entry = oracle_label_rows(ids, off)
    assert lr.n_rows == len(row_id)
    np.testing.assert_array_equal(lr.row_id, row_id)
    np.testing.assert_array_equal(lr.row_first, row_first)
    np.testing.assert_array_equal(lr.row_entry, row_entry)


def test_pack_labels_matches_oracle_on_golden(blink):
    import json

    with open(os.path.join(ROOT, "tests", "golden", "label_rows_cases.json")) as f:
        for case in json.load(f)["cases"]:
            lr = blink.pack_labels(case["cand_ids"], case["cand_off"], 1000)
            _compare_label_rows(lr, case["cand_ids"], case["cand_off"])


def test_pack_labels_matches_oracle_random(blink):
    rng = np.random.default_rng(321)
    for trial in range(300):
        n = int(rng.integers(1, 513))
        vocab = int(rng.choice([1, 7, 64, 65, 300, 151936]))
        kmax = int(rng.choice([1, 4, 26, 255]))
        k = rng.integers(1, kmax + 1, size=n)
        if trial % 3 == 0:  # the pages' form: one label table, first K per question
            table = rng.permutation(vocab)[:kmax] if vocab >= kmax else rng.integers(0, vocab, kmax)
            ids = np.concatenate([table[:int(x)] for x in k])
        else:
            ids = rng.integers(0, vocab, size=int(k.sum()))
        off = np.concatenate([[0], np.cumsum(k)]).astype(np.int32)
        ids = ids.astype(np.int32)
        _compare_label_rows(blink.pack_labels(ids, off, vocab), ids, off)


@pytest.mark.parametrize("ids, off, vocab, code, msg", [
    ([1, 2], [0, 2, 2], 10, -2, "question with 0 options; the limit is 1 to 255"),
    (list(range(256)), [0, 256], 300, -2, "question with 256 options; the limit is 1 to 255"),
    ([1, 12], [0, 2], 10, -1, "option entry 1 has token id 12 outside [0, 10)"),
    ([-1], [0, 1], 10, -1, "option entry 0 has token id -1"),
    ([1], [0, 1], 0, -1, "vocab 0 outside"),
    ([1], [0], 10, -2, "request of 0 questions; the limit is 1 to 512"),
])
def test_pack_labels_refusals(blink, ids, off, vocab, code, msg):
    with pytest.raises(blink.BlinkError) as e:
        blink.pack_labels(ids, off, vocab)
    assert e.value.code == code and msg in str(e.value)


def _readout_batched(lib, temperature=1.0, n=2, max_options=4, d_model=256, total=4, n_rows=3,
                     null_rows=False):
    fake = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    rows = None if null_rows else fake
    return lib.blink_label_readout_batched(fake, 10, d_model, fake, fake, 100, fake, n, total,
                                           max_options, rows, rows, rows, n_rows, temperature,
                                           fake, fake, fake, None)


@pytest.mark.parametrize("kw, code, msg", [
    (dict(temperature=0.0), -1, "temperature is not a positive finite number"),
    (dict(n=513), -2, "request of 513 questions; the limit is 1 to 512"),
    (dict(max_options=256), -2, "question with 256 options; the limit is 1 to 255"),
    (dict(d_model=12), -1, "d_model 12 must be a multiple of 8"),
    (dict(total=9), -1, "does not fit"),
    (dict(n_rows=0), -1, "n_rows 0 outside"),
    (dict(n_rows=5), -1, "n_rows 5 outside"),
    (dict(null_rows=True), -1, "a pointer argument is NULL"),
])
def test_readout_batched_refusals_before_launch(blink, kw, code, msg):
    lib = blink.load_library()
    assert _readout_batched(lib, **kw) == code
    assert msg in lib.blink_last_error().decode()


def test_plan_prefix_matches_oracle_on_golden(blink):
    import json

    with open(os.path.join(ROOT, "tests", "golden", "prefix_cases.json")) as f:
        for case in json.load(f)["cases"]:
            got = blink.plan_prefix(case["seqs"], case["min_prefix_tokens"])
            assert (got.shared_len, got.prefix_len, got.prefill_tokens) == (
                case["shared"], case["prefix_len"], case["prefill_tokens"]), case["name"]


def test_plan_prefix_matches_oracle_random(blink):
    rng = np.random.default_rng(77)
    for _ in range(500):
        n = int(rng.integers(1, 20))
        vocab = int(rng.choice([2, 5, 1000]))
        head = rng.integers(0, vocab, size=int(rng.integers(0, 600))).tolist()
        seqs = []
        for _ in range(n):
            cut = int(rng.integers(max(0, len(head) - 3), len(head) + 1))
            tail = rng.integers(0, vocab, size=int(rng.integers(0, 6))).tolist()
            seq = head[:cut] + tail
            seqs.append(seq if seq else [int(rng.integers(0, vocab))])
        m = int(rng.choice([1, 2, 256, 10**6]))
        got = blink.plan_prefix(seqs, m)
        assert (got.shared_len, got.prefix_len, got.prefill_tokens) == oracle_plan_prefix(seqs, m)


def test_plan_prefix_at_the_context_limit(blink):
    head = list(range(131071))
    got = blink.plan_prefix([head + [1], head + [2]])
    assert (got.shared_len, got.prefix_len, got.prefill_tokens) == (131071, 131071, 131073)


@pytest.mark.parametrize("seqs, m, code, msg", [
    ([], 256, -2, "request of 0 questions; the limit is 1 to 512"),
    ([[1]] * 513, 256, -2, "request of 513 questions; the limit is 1 to 512"),
    ([[1, 2], []], 256, -1, "sequence 1 needs at least one token"),
    ([[1, 2]], 0, -1, "the minimum shared prefix must be at least 1"),
    ([[0] * 131073], 256, -2, "question 0 needs 131073 tokens of context; the maximum context length"),
])
def test_plan_prefix_refusals(blink, seqs, m, code, msg):
    with pytest.raises(blink.BlinkError) as e:
        blink.plan_prefix(seqs, m)
    assert e.value.code == code and msg in str(e.value)


def _compare_answers(blink, probs, off, types):
    p32 = np.asarray(probs, np.float32)
    choice, conf, value = blink.assemble_answers(p32, off, types)
    ref = oracle_assemble(types, p32.astype(np.float64), off)
    for i, (c, f, v) in enumerate(ref):
        assert choice[i] == c, i
        if f is None:
            assert np.isnan(conf[i])
        else:
            assert abs(conf[i] - f) <= 1e-12, i
        assert abs(value[i] - v) <= 1e-12, i


def test_assemble_answers_matches_oracle_on_golden(blink):
    import json

    with open(os.path.join(ROOT, "tests", "golden", "answer_cases.json")) as f:
        for case in json.load(f)["cases"]:
            _compare_answers(blink, case["probs"], [0, len(case["probs"])], [case["type"]])


def test_assemble_answers_matches_oracle_random(blink):
    rng = np.random.default_rng(99)
    for _ in range(200):
        n = int(rng.integers(1, 513))
        types = rng.integers(0, 3, size=n)
        k = np.where(types == 1, 2, np.where(types == 2, rng.integers(2, 11, size=n),
                                             rng.integers(1, 256, size=n)))
        off = np.concatenate([[0], np.cumsum(k)]).astype(np.int32)
        probs = np.concatenate([rng.dirichlet(np.ones(int(x))) for x in k])
        if rng.random() < 0.3:  # exact ties in float32
            probs = np.round(probs * 4) / 4
        _compare_answers(blink, probs, off, types.astype(np.int32))


@pytest.mark.parametrize("probs, off, types, code, msg", [
    ([], [0], [], -2, "request of 0 questions; the limit is 1 to 512"),
    ([0.2, 0.3, 0.5], [0, 3], [1], -1, "a noul question offers exactly yes and no"),
    ([1.0], [0, 1], [2], -1, "a score takes 2 to 10 levels"),
    ([0.1] * 11, [0, 11], [2], -1, "a score takes 2 to 10 levels"),
    ([0.5, 0.5], [0, 2], [5], -1, "unknown question type 5"),
    ([0.5, 0.5], [0, 2, 2], [0, 0], -2, "question with 0 options"),
])
def test_assemble_answers_refusals(blink, probs, off, types, code, msg):
    with pytest.raises(blink.BlinkError) as e:
        blink.assemble_answers(probs, off, types)
    assert e.value.code == code and msg in str(e.value)


def _grouped(lib, n=3, total=9, t_pad=12, vs=(0, 3, 5, 9), first=(0, 2, 3), pstart=(0, 4),
             plen=(4, 2), rows=6, hq=4, hkv=1, d=64):
    fake = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    h_vs = np.asarray(vs, np.int32)
    fi = np.asarray(first, np.int32)
    ps = np.asarray(pstart, np.int64)
    pl = np.asarray(plen, np.int32)
    n_req = len(first) - 1
    return lib.blink_prefix_tail_attention_grouped(
        fake, fake, fake, fake if rows else None, fake if rows else None, fake, fake, fake,
        _ptr32(h_vs), n, total, t_pad, n_req, _ptr32(fi),
        ps.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _ptr32(pl), rows, hq, hkv, d, 0.125,
        None)


def _ptr32(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


@pytest.mark.parametrize("kw, code, msg", [
    (dict(first=(0,), pstart=(), plen=()), -2, "group of 0 requests; the limit is 1 to 64"),
    (dict(first=tuple(range(66)), pstart=(0,) * 65, plen=(0,) * 65, n=65, total=65, t_pad=65,
          vs=tuple(range(66))), -2, "group of 65 requests; the limit is 1 to 64"),
    (dict(first=(0, 2, 2)), -1, "request_first must run from 0 to n_questions"),
    (dict(first=(0, 3, 3)), -1, "request 1 has no questions"),
    (dict(first=(0, 0, 3)), -1, "request 0 has no questions"),
    (dict(pstart=(0, 5)), -1, "request 1: prefix rows [5, 7) outside the 6 prefix rows"),
    (dict(plen=(4, -1)), -1, "request 1: prefix rows"),
    (dict(vs=(0, 3, 3, 9)), -1, "question 1 has an empty tail"),
    (dict(vs=(0, 3, 5, 8)), -1, "valid_start must run from 0 to total_valid_tokens"),
    (dict(rows=0), -1, "prefix rows"),
    (dict(plen=(4, 131070), rows=131080, pstart=(0, 4)), -2,
     "question 2 needs 131074 tokens of context; the maximum context length is 131072"),
])
def test_grouped_attention_refusals_before_launch(blink, kw, code, msg):
    lib = blink.load_library()
    assert _grouped(lib, **kw) == code
    assert msg in lib.blink_last_error().decode()


def test_score_targets_workspace_size(blink):
    lib = blink.load_library()
    need = lib.blink_score_targets_workspace(256, 151936)
    # (max, sum) per row and vocabulary slice, plus one target logit per row
    assert need % 256 == 0 and need >= 256 * 4 + 256 * 8 * (151936 // 256)
    assert lib.blink_score_targets_workspace(512, 151936) >= 2 * need - 512
    assert lib.blink_score_targets_workspace(0, 100) == 0
    assert lib.blink_score_targets_workspace(5, 0) == 0


def _score(lib, n=4, d_model=128, vocab=1000, ws=1 << 20, null=False, rows=10):
    fake = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    return lib.blink_score_targets(fake, rows, d_model, fake, fake, n, None if null else fake,
                                   vocab, fake, fake, ws, None)


@pytest.mark.parametrize("kw, code, msg", [
    (dict(n=0), -2, "0 scored rows"),
    (dict(d_model=100), -1, "d_model 100 must be a multiple of 64"),
    (dict(d_model=32768), -1, "d_model 32768 must be a multiple of 64"),
    (dict(vocab=0), -1, "vocab in 1..2^31"),
    (dict(rows=0), -1, "hidden_rows must be positive"),
    (dict(ws=100), -1, "workspace of 100 bytes; 512 needed"),
    (dict(null=True), -1, "a pointer argument is NULL"),
])
def test_score_targets_refusals_before_launch(blink, kw, code, msg):
    lib = blink.load_library()
    assert _score(lib, **kw) == code
    assert msg in lib.blink_last_error().decode()


@pytest.mark.parametrize("kw, code, msg", [
    (dict(n=1767, vocab=151936), -2, "the library's static scratch holds 16777216"),
    (dict(n=0), -2, "0 scored rows"),
    (dict(d_model=100), -1, "d_model 100 must be a multiple of 64"),
    (dict(null=True), -1, "a pointer argument is NULL"),
])
def test_score_targets_noalloc_refusals_before_launch(blink, kw, code, msg):
    # The no-allocation form refuses sizes beyond its static scratch before any device call.
    lib = blink.load_library()
    fake = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    n, d_model, vocab = kw.get("n", 4), kw.get("d_model", 128), kw.get("vocab", 1000)
    assert lib.blink_score_targets_noalloc(fake, 10, d_model, fake, fake, n,
                                           None if kw.get("null") else fake, vocab, fake,
                                           None) == code
    assert msg in lib.blink_last_error().decode()
    # The largest call that fits: at vocab 151936, 1766 rows need exactly 16 MiB.
    assert lib.blink_score_targets_workspace(1766, 151936) <= 16 << 20
    assert lib.blink_score_targets_workspace(1767, 151936) > 16 << 20


def test_combine_rotations_matches_oracle_random(blink):
    rng = np.random.default_rng(11)
    for trial in range(100):
        nq = int(rng.integers(1, 20))
        n_keys = rng.integers(1, 30, size=nq).tolist()
        passes, priors = [], []
        for _ in range(int(rng.integers(1, 60))):
            q = int(rng.integers(nq))
            k = n_keys[q]
            shown = rng.permutation(k)[:int(rng.integers(1, k + 1))].tolist()
            logits = (rng.standard_normal(len(shown)) * 3).astype(np.float32)
            passes.append((q, shown, logits))
            priors.append(np.log(rng.dirichlet(np.ones(len(shown)))).astype(np.float32))
        use_prior = trial % 2 == 0
        got = blink.combine_rotations(n_keys, passes, priors if use_prior else None)
        ref = oracle_refine.combine_rotations(
            n_keys, [(q, keys, [float(v) for v in lg]) for q, keys, lg in passes],
            [[float(v) for v in p] for p in priors] if use_prior else None)
        for g, r in zip(got, ref):
            r = np.asarray(r)
            assert np.array_equal(np.isnan(g), np.isnan(r))
            np.testing.assert_allclose(g[~np.isnan(g)], r[~np.isnan(r)], rtol=0, atol=2e-6)


def test_two_stage_finalists_matches_oracle_random(blink):
    rng = np.random.default_rng(12)
    for _ in range(300):
        n = int(rng.integers(1, 256))
        s1 = np.round(rng.standard_normal(n) * 2, int(rng.integers(0, 3))).astype(np.float32)
        keep = int(rng.integers(1, 300))
        got = blink.two_stage_finalists(s1, keep)
        assert got.tolist() == oracle_refine.two_stage_finalists([float(v) for v in s1], keep)


@pytest.mark.parametrize("call, msg", [
    (lambda b: b.combine_rotations([2], [(1, [0, 1], [0.0, 0.0])]), "pass 0 names question 1"),
    (lambda b: b.combine_rotations([2], [(0, [0, 2], [0.0, 0.0])]), "names key 2"),
    (lambda b: b.combine_rotations([2], [(0, [0, 1, 0], [0.0, 0.0, 0.0])]), "offers 3 options"),
    (lambda b: b.combine_rotations([2], []), "0 passes"),
    (lambda b: b.combine_rotations([256], [(0, [0], [0.0])]), "question with 256 options"),
    (lambda b: b.two_stage_finalists([1.0, float("nan")], 1), "stage-one score 1 is NaN"),
    (lambda b: b.two_stage_finalists([1.0], 0), "keep must be at least 1"),
    (lambda b: b.two_stage_finalists([0.0] * 256, 3), "question with 256 options"),
])
def test_refinement_refusals(blink, call, msg):
    with pytest.raises(blink.BlinkError) as e:
        call(blink)
    assert msg in str(e.value)
