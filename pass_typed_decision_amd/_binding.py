"""ctypes binding of libblink.so (argument marshalling only).

Every computation happens in the library: the host packer in C++ and the attention and
readout in HIP kernels for gfx950. PyTorch tensors only supply device memory and the stream.
If the library is missing the binding raises; there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libblink.so")

BLINK_OK = 0
BLINK_E_INVALID = -1
BLINK_E_LIMIT = -2
BLINK_E_DEVICE = -3
MAX_QUESTIONS = 512
MAX_OPTIONS = 255
MAX_INPUT_TOKENS = 131072
TOKEN_BUDGET = 32768
PREFIX_MIN_TOKENS = 256
MAX_REQUESTS = 64

# Every symbol declared in include/blink.h.
EXPORTS = (
    "blink_last_error",
    "blink_abi_version",
    "blink_pack_ragged",
    "blink_prefix_tail_attention",
    "blink_prefix_tail_attention_workspace",
    "blink_label_readout",
    "blink_pack_labels",
    "blink_label_readout_batched",
    "blink_plan_prefix",
    "blink_assemble_answers",
    "blink_prefix_tail_attention_grouped",
    "blink_score_targets_workspace",
    "blink_score_targets",
    "blink_score_targets_noalloc",
    "blink_combine_rotations",
    "blink_two_stage_finalists",
)


class BlinkError(ValueError):
    """A call the library refused; ``code`` is the negative BLINK_E_* status."""

    def __init__(self, code: int, message: str):
        super().__init__(message)
        self.code = code


_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F32 = ctypes.c_float
_PI32 = ctypes.POINTER(ctypes.c_int32)
_PI64 = ctypes.POINTER(ctypes.c_int64)


def load_library(path: str = LIBRARY) -> ctypes.CDLL:
    """Loads libblink.so (once) and declares the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m pass_typed_decision_amd.build` "
            "(the scoring path has no non-HIP fallback)")
    lib = ctypes.CDLL(path)
    lib.blink_last_error.restype = ctypes.c_char_p
    lib.blink_last_error.argtypes = []
    lib.blink_abi_version.restype = ctypes.c_int
    lib.blink_abi_version.argtypes = []
    lib.blink_pack_ragged.restype = ctypes.c_int
    lib.blink_pack_ragged.argtypes = [
        _PI32, _I32, _I32, _I64, _I32,
        _PI32, _PI32, _PI32, _PI64, _PI64, _PI32,
        _PI32, _PI32, _PI64, _PI32, _PI64, _PI64,
    ]
    lib.blink_prefix_tail_attention.restype = ctypes.c_int
    lib.blink_prefix_tail_attention.argtypes = [
        _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I64, _I64, _I32, _I32, _I32, _I32, _F32, _P,
        ctypes.c_size_t, _P,
    ]
    lib.blink_prefix_tail_attention_workspace.restype = ctypes.c_size_t
    lib.blink_prefix_tail_attention_workspace.argtypes = [_I64, _I32, _I32, _I32, _I32]
    lib.blink_label_readout.restype = ctypes.c_int
    lib.blink_label_readout.argtypes = [
        _P, _I64, _I32, _P, _P, _I64, _P, _P, _I32, _I64, _I32, _F32, _P, _P, _P, _P,
    ]
    lib.blink_pack_labels.restype = ctypes.c_int
    lib.blink_pack_labels.argtypes = [_PI32, _PI32, _I32, _I64, _PI32, _PI32, _PI32, _PI32]
    lib.blink_label_readout_batched.restype = ctypes.c_int
    lib.blink_label_readout_batched.argtypes = [
        _P, _I64, _I32, _P, _P, _I64, _P, _I32, _I64, _I32, _P, _P, _P, _I32, _F32, _P, _P, _P,
        _P,
    ]
    lib.blink_assemble_answers.restype = ctypes.c_int
    lib.blink_assemble_answers.argtypes = [
        ctypes.POINTER(ctypes.c_float), _PI32, _PI32, _I32, _PI32,
        ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    lib.blink_prefix_tail_attention_grouped.restype = ctypes.c_int
    lib.blink_prefix_tail_attention_grouped.argtypes = [
        _P, _P, _P, _P, _P, _P, _P, _P, _PI32, _I32, _I64, _I64, _I32, _PI32, _PI64, _PI32, _I64,
        _I32, _I32, _I32, _F32, _P,
    ]
    lib.blink_score_targets_workspace.restype = ctypes.c_size_t
    lib.blink_score_targets_workspace.argtypes = [_I32, _I64]
    lib.blink_score_targets.restype = ctypes.c_int
    lib.blink_score_targets.argtypes = [_P, _I64, _I32, _P, _P, _I32, _P, _I64, _P, _P,
                                        ctypes.c_size_t, _P]
    lib.blink_score_targets_noalloc.restype = ctypes.c_int
    lib.blink_score_targets_noalloc.argtypes = [_P, _I64, _I32, _P, _P, _I32, _P, _I64, _P, _P]
    _PF = ctypes.POINTER(ctypes.c_float)
    lib.blink_combine_rotations.restype = ctypes.c_int
    lib.blink_combine_rotations.argtypes = [_PF, _PI32, _PI32, _PI32, _PF, _I32, _PI32, _I32,
                                            _PF]
    lib.blink_two_stage_finalists.restype = ctypes.c_int
    lib.blink_two_stage_finalists.argtypes = [_PF, _I32, _I32, _PI32, _PI32]
    lib.blink_plan_prefix.restype = ctypes.c_int
    lib.blink_plan_prefix.argtypes = [_PI32, _PI64, _I32, _I32, _PI32, _PI32, _PI64]
    _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != BLINK_OK:
        msg = load_library().blink_last_error().decode("utf-8", "replace")
        raise BlinkError(rc, msg)


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


@dataclass
class Pack:
    """Result of blink_pack_ragged (host arrays, question-indexed unless stated)."""

    order: np.ndarray
    batch_of: np.ndarray
    row_of: np.ndarray
    token_offset: np.ndarray
    last_row: np.ndarray
    valid_start: np.ndarray
    batch_first: np.ndarray  # [n_batches + 1]
    batch_width: np.ndarray  # [n_batches]
    batch_base: np.ndarray  # [n_batches + 1]
    n_batches: int
    total_padded_tokens: int
    total_valid_tokens: int


def pack_ragged_args(tail_len, prefix_len, token_budget, max_rows, order, batch_of, row_of,
                     token_offset, last_row, valid_start, batch_first, batch_width, batch_base,
                     n_batches, total_padded, total_valid) -> list:
    """Argument list of blink_pack_ragged over caller-owned arrays (which must stay alive
    and keep their sizes) and ctypes scalars for the three counts; for repeated calls."""
    t = tail_len
    n = int(t.shape[0])
    arrays = ((t, np.int32, n), (order, np.int32, n), (batch_of, np.int32, n),
              (row_of, np.int32, n), (token_offset, np.int64, n), (last_row, np.int64, n),
              (valid_start, np.int32, n + 1), (batch_first, np.int32, n + 1),
              (batch_width, np.int32, n), (batch_base, np.int64, n + 1))
    for a, dt, size in arrays:
        if a.dtype != dt or not a.flags["C_CONTIGUOUS"] or a.shape[0] < size:
            raise BlinkError(BLINK_E_INVALID, "pack buffers have the wrong type or size")
    c32, c64 = ctypes.c_int32, ctypes.c_int64
    return [_ptr(t, c32), n, int(prefix_len), int(token_budget), int(max_rows),
            _ptr(order, c32), _ptr(batch_of, c32), _ptr(row_of, c32), _ptr(token_offset, c64),
            _ptr(last_row, c64), _ptr(valid_start, c32), _ptr(batch_first, c32),
            _ptr(batch_width, c32), _ptr(batch_base, c64), ctypes.byref(n_batches),
            ctypes.byref(total_padded), ctypes.byref(total_valid)]


def pack_ragged(tail_len, prefix_len: int = 0, token_budget: int = TOKEN_BUDGET,
                max_rows: int = 0) -> Pack:
    """Host packer (blink_pack_ragged)."""
    lib = load_library()
    t = np.ascontiguousarray(np.asarray(tail_len, dtype=np.int32))
    n = int(t.shape[0])
    cap = max(n, 1)
    order = np.zeros(cap, np.int32)
    batch_of = np.zeros(cap, np.int32)
    row_of = np.zeros(cap, np.int32)
    token_offset = np.zeros(cap, np.int64)
    last_row = np.zeros(cap, np.int64)
    valid_start = np.zeros(cap + 1, np.int32)
    batch_first = np.zeros(cap + 1, np.int32)
    batch_width = np.zeros(cap, np.int32)
    batch_base = np.zeros(cap + 1, np.int64)
    nb = ctypes.c_int32(0)
    tp = ctypes.c_int64(0)
    tv = ctypes.c_int64(0)
    src = t if n else np.zeros(1, np.int32)
    _check(lib.blink_pack_ragged(
        _ptr(src, ctypes.c_int32), n, int(prefix_len), int(token_budget), int(max_rows),
        _ptr(order, ctypes.c_int32), _ptr(batch_of, ctypes.c_int32), _ptr(row_of, ctypes.c_int32),
        _ptr(token_offset, ctypes.c_int64), _ptr(last_row, ctypes.c_int64),
        _ptr(valid_start, ctypes.c_int32), _ptr(batch_first, ctypes.c_int32),
        _ptr(batch_width, ctypes.c_int32), _ptr(batch_base, ctypes.c_int64),
        ctypes.byref(nb), ctypes.byref(tp), ctypes.byref(tv)))
    k = nb.value
    return Pack(order[:n], batch_of[:n], row_of[:n], token_offset[:n], last_row[:n],
                valid_start[:n + 1], batch_first[:k + 1], batch_width[:k], batch_base[:k + 1],
                k, tp.value, tv.value)


@dataclass
class PrefixPlan:
    """Result of blink_plan_prefix."""

    shared_len: int  # leading tokens common to every sequence (each keeps one of its own)
    prefix_len: int  # shared_len on the shared path, 0 on the plain path
    prefill_tokens: int  # tokens the model computes


def plan_prefix(seqs, min_prefix_tokens: int = PREFIX_MIN_TOKENS) -> PrefixPlan:
    """Shared-prefix plan of a request's token sequences (blink_plan_prefix)."""
    lib = load_library()
    lens = [len(s) for s in seqs]
    off = np.zeros(len(lens) + 1, np.int64)
    off[1:] = np.cumsum(lens)
    flat = (np.concatenate([np.asarray(s, np.int32) for s in seqs]) if seqs and off[-1]
            else np.zeros(1, np.int32))
    flat = np.ascontiguousarray(flat, dtype=np.int32)
    shared, prefix = ctypes.c_int32(0), ctypes.c_int32(0)
    prefill = ctypes.c_int64(0)
    _check(lib.blink_plan_prefix(_ptr(flat, ctypes.c_int32), _ptr(off, ctypes.c_int64), len(lens),
                                 int(min_prefix_tokens), ctypes.byref(shared),
                                 ctypes.byref(prefix), ctypes.byref(prefill)))
    return PrefixPlan(shared.value, prefix.value, prefill.value)


ANSWER_CHOICE, ANSWER_NOUL, ANSWER_SCORE = 0, 1, 2


def assemble_answers(probs, cand_off, qtype):
    """Typed answers of a request (blink_assemble_answers): returns (choice int32 [n],
    confidence float64 [n], value float64 [n])."""
    lib = load_library()
    p = np.ascontiguousarray(np.asarray(probs, dtype=np.float32))
    off = np.ascontiguousarray(np.asarray(cand_off, dtype=np.int32))
    t = np.ascontiguousarray(np.asarray(qtype, dtype=np.int32))
    n = int(t.shape[0])
    if off.shape[0] != n + 1 or (n and int(off[-1]) != p.shape[0]):
        raise BlinkError(BLINK_E_INVALID, "offsets must have n + 1 entries ending at len(probs)")
    cap = max(n, 1)
    choice = np.zeros(cap, np.int32)
    conf = np.zeros(cap, np.float64)
    value = np.zeros(cap, np.float64)
    src_p = p if p.size else np.zeros(1, np.float32)
    src_t = t if n else np.zeros(1, np.int32)
    _check(lib.blink_assemble_answers(
        src_p.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), _ptr(off, ctypes.c_int32),
        _ptr(src_t, ctypes.c_int32), n, _ptr(choice, ctypes.c_int32),
        conf.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
        value.ctypes.data_as(ctypes.POINTER(ctypes.c_double))))
    return choice[:n], conf[:n], value[:n]


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, dtype, name):
    import torch

    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise BlinkError(BLINK_E_INVALID, f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise BlinkError(BLINK_E_INVALID, f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise BlinkError(BLINK_E_INVALID, f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _dev_or_pinned(t, dtype, name):
    """An output the device writes: a device tensor, or pinned host memory it can reach."""
    import torch

    if isinstance(t, torch.Tensor) and not t.is_cuda and t.is_pinned():
        if t.dtype != dtype or not t.is_contiguous():
            raise BlinkError(BLINK_E_INVALID, f"{name} must be contiguous {dtype}")
        return ctypes.c_void_p(t.data_ptr())
    return _dev(t, dtype, name)


class _ArgList(list):
    """A checked argument list that also holds the device memory its addresses point into."""

    keep = None


def attention_workspace(total_valid_tokens: int, n_heads_q: int, n_heads_kv: int,
                        head_dim: int, prefix_len: int, device=None):
    """Device workspace for blink_prefix_tail_attention at these sizes on the current device
    (a uint8 tensor), or None when its work split needs none."""
    import torch

    size = int(load_library().blink_prefix_tail_attention_workspace(
        int(total_valid_tokens), int(n_heads_q), int(n_heads_kv), int(head_dim), int(prefix_len)))
    if size == 0:
        return None
    if device is None:
        device = torch.device("cuda", torch.cuda.current_device())
    return torch.empty(size, dtype=torch.uint8, device=device)


def prefix_tail_attention(q, k_tail, v_tail, k_prefix, v_prefix, out, token_offset,
                          valid_start, total_valid_tokens: int, scale: float, stream=None,
                          launch: bool = True, workspace="auto"):
    """Launches blink_prefix_tail_attention. Shapes: q/out [T_pad, H_q, D], k/v_tail
    [T_pad, H_kv, D], k/v_prefix [P, H_kv, D] or None; token_offset int64 [n],
    valid_start int32 [n + 1] (device). ``workspace``: "auto" allocates what the library asks
    for on the current device (on the launch stream's order), None passes none, or a uint8
    device tensor. With ``launch=False`` returns the checked argument list instead (index 9 is
    total_valid_tokens) for repeated launches; it holds raw addresses, so the caller keeps every
    tensor alive while the list is in use (the list itself holds an automatic workspace)."""
    import torch

    bf = torch.bfloat16
    if q.dim() != 3 or k_tail.dim() != 3:
        raise BlinkError(BLINK_E_INVALID, "q and k_tail must be [tokens, heads, head_dim]")
    t_pad, hq, d = q.shape
    hkv = k_tail.shape[1]
    if tuple(k_tail.shape) != (t_pad, hkv, d) or tuple(v_tail.shape) != (t_pad, hkv, d):
        raise BlinkError(BLINK_E_INVALID, "k_tail/v_tail must be [T_pad, H_kv, D]")
    if tuple(out.shape) != (t_pad, hq, d):
        raise BlinkError(BLINK_E_INVALID, "out must be [T_pad, H_q, D]")
    p = 0 if k_prefix is None else int(k_prefix.shape[0])
    if p:
        if tuple(k_prefix.shape) != (p, hkv, d) or tuple(v_prefix.shape) != (p, hkv, d):
            raise BlinkError(BLINK_E_INVALID, "k_prefix/v_prefix must be [P, H_kv, D]")
        kp, vp = _dev(k_prefix, bf, "k_prefix"), _dev(v_prefix, bf, "v_prefix")
    else:
        kp = vp = ctypes.c_void_p(0)
    n = int(token_offset.shape[0])
    if int(valid_start.shape[0]) != n + 1:
        raise BlinkError(BLINK_E_INVALID, "valid_start must have n + 1 entries")
    lib = load_library()
    if isinstance(workspace, str):
        if workspace != "auto":
            raise BlinkError(BLINK_E_INVALID, "workspace must be 'auto', None or a tensor")
        if stream is not None and launch:
            # the allocator orders reuse on the current stream; the launch runs on `stream`
            torch.cuda.ExternalStream(int(stream)).wait_stream(torch.cuda.current_stream())
        workspace = attention_workspace(int(total_valid_tokens), int(hq), int(hkv), int(d), p,
                                        device=q.device)
        if workspace is not None and stream is not None and launch:
            workspace.record_stream(torch.cuda.ExternalStream(int(stream)))
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda:
            raise BlinkError(BLINK_E_INVALID, "workspace must be a device tensor")
        ws_ptr, ws_bytes = ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * \
            workspace.element_size()
    else:
        ws_ptr, ws_bytes = ctypes.c_void_p(0), 0
    args = _ArgList([
        _dev(q, bf, "q"), _dev(k_tail, bf, "k_tail"), _dev(v_tail, bf, "v_tail"), kp, vp,
        _dev(out, bf, "out"), _dev(token_offset, torch.int64, "token_offset"),
        _dev(valid_start, torch.int32, "valid_start"), n, int(total_valid_tokens), int(t_pad),
        p, int(hq), int(hkv), int(d), float(scale), ws_ptr, ctypes.c_size_t(ws_bytes),
        _stream(stream)])
    args.keep = workspace
    if not launch:
        return args
    _check(lib.blink_prefix_tail_attention(*args))


def combine_rotations(n_keys, passes, priors=None) -> list:
    """Rotation averaging (blink_combine_rotations). n_keys[q]: options of question q;
    passes: (question, key of each position, logits of each position); priors: None or per
    pass the prior log-probability of each position. Returns per question a float32 array of
    mean log-probabilities per key (NaN where no pass offered the key)."""
    lib = load_library()
    f32 = ctypes.POINTER(ctypes.c_float)
    key_off = np.concatenate([[0], np.cumsum(n_keys)]).astype(np.int32)
    pass_off = np.concatenate([[0], np.cumsum([len(p[1]) for p in passes])]).astype(np.int32)
    pq = np.asarray([p[0] for p in passes], np.int32)
    keys = np.ascontiguousarray(np.concatenate([np.asarray(p[1], np.int32) for p in passes])
                                if passes else np.zeros(1, np.int32))
    logits = np.ascontiguousarray(np.concatenate([np.asarray(p[2], np.float32) for p in passes])
                                  if passes else np.zeros(1, np.float32))
    prior = None
    if priors is not None:
        prior = np.ascontiguousarray(np.concatenate([np.asarray(x, np.float32) for x in priors]))
        if prior.shape[0] != logits.shape[0]:
            raise BlinkError(BLINK_E_INVALID, "priors must give one value per pass position")
    out = np.zeros(max(int(key_off[-1]), 1), np.float32)
    pq_src = pq if pq.size else np.zeros(1, np.int32)
    _check(lib.blink_combine_rotations(
        logits.ctypes.data_as(f32), _ptr(pass_off, ctypes.c_int32), _ptr(pq_src, ctypes.c_int32),
        _ptr(keys, ctypes.c_int32), None if prior is None else prior.ctypes.data_as(f32),
        len(passes), _ptr(key_off, ctypes.c_int32), len(n_keys), out.ctypes.data_as(f32)))
    return [out[key_off[q]:key_off[q + 1]] for q in range(len(n_keys))]


def two_stage_finalists(stage_one, keep: int) -> np.ndarray:
    """Finalists of a two-stage choice (blink_two_stage_finalists), best first."""
    lib = load_library()
    s1 = np.ascontiguousarray(np.asarray(stage_one, np.float32))
    out = np.zeros(max(int(s1.shape[0]), 1), np.int32)
    k = ctypes.c_int32(0)
    src = s1 if s1.size else np.zeros(1, np.float32)
    _check(lib.blink_two_stage_finalists(src.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                                         int(s1.shape[0]), int(keep),
                                         _ptr(out, ctypes.c_int32), ctypes.byref(k)))
    return out[:k.value]


class GroupedAttention:
    """Prepared launch of blink_prefix_tail_attention_grouped: several requests, each with
    its own prefix, in one launch. q/out [T_pad, H_q, D], k/v_tail [T_pad, H_kv, D],
    k/v_prefix [total prefix rows, H_kv, D] or None (device, bf16); token_offset int64 [n] and
    valid_start int32 [n + 1] on the device, with valid_start's host copy; request_first
    int32 [R + 1], prefix_start int64 [R], prefix_len int32 [R] on the host. The object holds
    every tensor and host array it was given, since ``launch()`` passes their addresses again
    on each call."""

    def __init__(self, q, k_tail, v_tail, k_prefix, v_prefix, out, token_offset, valid_start,
                 h_valid_start, request_first, prefix_start, prefix_len, scale: float,
                 stream=None):
        import torch

        bf = torch.bfloat16
        t_pad, hq, d = q.shape
        hkv = k_tail.shape[1]
        if tuple(k_tail.shape) != (t_pad, hkv, d) or tuple(v_tail.shape) != (t_pad, hkv, d):
            raise BlinkError(BLINK_E_INVALID, "k_tail/v_tail must be [T_pad, H_kv, D]")
        if tuple(out.shape) != (t_pad, hq, d):
            raise BlinkError(BLINK_E_INVALID, "out must be [T_pad, H_q, D]")
        rows = 0 if k_prefix is None else int(k_prefix.shape[0])
        if rows:
            if tuple(k_prefix.shape) != (rows, hkv, d) or tuple(v_prefix.shape) != (rows, hkv, d):
                raise BlinkError(BLINK_E_INVALID, "k_prefix/v_prefix must be [rows, H_kv, D]")
            kp, vp = _dev(k_prefix, bf, "k_prefix"), _dev(v_prefix, bf, "v_prefix")
        else:
            kp = vp = ctypes.c_void_p(0)
        self.h_vs = np.ascontiguousarray(np.asarray(h_valid_start, np.int32))
        self.first = np.ascontiguousarray(np.asarray(request_first, np.int32))
        self.pstart = np.ascontiguousarray(np.asarray(prefix_start, np.int64))
        self.plen = np.ascontiguousarray(np.asarray(prefix_len, np.int32))
        n = int(token_offset.shape[0])
        n_req = int(self.first.shape[0]) - 1
        if self.h_vs.shape[0] != n + 1 or int(valid_start.shape[0]) != n + 1:
            raise BlinkError(BLINK_E_INVALID, "valid_start must have n + 1 entries")
        if n_req < 0 or self.pstart.shape[0] != n_req or self.plen.shape[0] != n_req:
            raise BlinkError(BLINK_E_INVALID, "request tables must have R + 1, R and R entries")
        self._tensors = (q, k_tail, v_tail, k_prefix, v_prefix, out, token_offset, valid_start)
        self.lib = load_library()
        self.args = [
            _dev(q, bf, "q"), _dev(k_tail, bf, "k_tail"), _dev(v_tail, bf, "v_tail"), kp, vp,
            _dev(out, bf, "out"), _dev(token_offset, torch.int64, "token_offset"),
            _dev(valid_start, torch.int32, "valid_start"), _ptr(self.h_vs, ctypes.c_int32), n,
            int(self.h_vs[-1]), int(t_pad), n_req, _ptr(self.first, ctypes.c_int32),
            _ptr(self.pstart, ctypes.c_int64), _ptr(self.plen, ctypes.c_int32), rows, int(hq),
            int(hkv), int(d), float(scale), _stream(stream)]

    def launch(self):
        _check(self.lib.blink_prefix_tail_attention_grouped(*self.args))


class TargetScorer:
    """Prepared teacher-forced scoring (blink_score_targets): log p(target | row) over the full
    vocabulary for n scored rows. hidden [T, d_model] and w_u [vocab, d_model] bf16, rows int64
    [n] and targets int32 [n] (device). The workspace is allocated here, once; ``run()`` queues
    the two kernels and returns the float32 [n] device tensor of log-probabilities."""

    def __init__(self, hidden, w_u, rows, targets, stream=None):
        import torch

        bf = torch.bfloat16
        if hidden.dim() != 2 or w_u.dim() != 2 or hidden.shape[1] != w_u.shape[1]:
            raise BlinkError(BLINK_E_INVALID, "hidden and w_u must be 2-D with the same width")
        n = int(rows.shape[0])
        if int(targets.shape[0]) != n:
            raise BlinkError(BLINK_E_INVALID, "rows and targets must have the same length")
        self.lib = load_library()
        size = int(self.lib.blink_score_targets_workspace(n, int(w_u.shape[0])))
        if size == 0:
            raise BlinkError(BLINK_E_INVALID, "no workspace size for these sizes")
        self.workspace = torch.empty(size, dtype=torch.uint8, device=hidden.device)
        self.logprob = torch.empty(n, dtype=torch.float32, device=hidden.device)
        self._tensors = (hidden, w_u, rows, targets)
        self.args = [
            _dev(hidden, bf, "hidden"), int(hidden.shape[0]), int(hidden.shape[1]),
            _dev(rows, torch.int64, "rows"), _dev(targets, torch.int32, "targets"), n,
            _dev(w_u, bf, "w_u"), int(w_u.shape[0]), _dev(self.logprob, torch.float32, "logprob"),
            ctypes.c_void_p(self.workspace.data_ptr()), size, _stream(stream)]

    def run(self):
        _check(self.lib.blink_score_targets(*self.args))
        return self.logprob

    def run_noalloc(self):
        """The same scoring through blink_score_targets_noalloc (the library's static scratch
        instead of this object's workspace)."""
        a = self.args
        _check(self.lib.blink_score_targets_noalloc(*a[:9], a[11]))
        return self.logprob


def encode_prefix_attention(q, k, v, out, scale: float, stream=None):
    """Attention of the shared prefix's own causal prefill, encoded once per request
    ("torch engine" section, _forward_shared: the batch-1 forward over the prefix tokens).
    It is blink_prefix_tail_attention with no prefix and the whole prefix as the tail of a
    single question. q/out [L, H_q, D], k/v [L, H_kv, D] (bf16, device). Returns the two
    small device row tables the launch reads (keep them until the stream has finished)."""
    import torch

    length = int(q.shape[0])
    if length < 1:
        raise BlinkError(BLINK_E_INVALID, "the prefix needs at least one token")
    token_offset = torch.zeros(1, dtype=torch.int64, device=q.device)
    valid_start = torch.tensor([0, length], dtype=torch.int32, device=q.device)
    if stream is not None:
        s = torch.cuda.ExternalStream(int(stream)) if not isinstance(stream, torch.cuda.Stream) \
            else stream
        s.wait_stream(torch.cuda.current_stream())
        token_offset.record_stream(s)
        valid_start.record_stream(s)
        stream = s.cuda_stream
    prefix_tail_attention(q, k, v, None, None, out, token_offset, valid_start, length, scale,
                          stream=stream)
    return token_offset, valid_start


def label_readout(hidden, last_row, w_u, cand_ids, cand_off, temperature: float,
                  max_options: int, logits, probs, argmax, stream=None, launch: bool = True):
    """Launches blink_label_readout. hidden [T_pad, d_model] bf16, last_row int64 [n],
    w_u [vocab, d_model] bf16, cand_ids int32 [sum K], cand_off int32 [n + 1];
    outputs logits float32 [sum K] (device), probs float32 [sum K] and argmax int32 [n] (device,
    or pinned host memory, readable once the stream is synchronised). With ``launch=False``
    returns the checked argument list instead, for repeated launches; it holds raw addresses,
    so the caller keeps every tensor alive while the list is in use."""
    import torch

    bf = torch.bfloat16
    if hidden.dim() != 2 or w_u.dim() != 2 or hidden.shape[1] != w_u.shape[1]:
        raise BlinkError(BLINK_E_INVALID, "hidden and w_u must be 2-D with the same width")
    n = int(last_row.shape[0])
    total = int(cand_ids.shape[0])
    if int(cand_off.shape[0]) != n + 1:
        raise BlinkError(BLINK_E_INVALID, "cand_off must have n + 1 entries")
    if int(logits.shape[0]) != total or int(probs.shape[0]) != total or int(argmax.shape[0]) != n:
        raise BlinkError(BLINK_E_INVALID, "output sizes do not match the candidate table")
    lib = load_library()
    args = [
        _dev(hidden, bf, "hidden"), int(hidden.shape[0]), int(hidden.shape[1]),
        _dev(last_row, torch.int64, "last_row"), _dev(w_u, bf, "w_u"), int(w_u.shape[0]),
        _dev(cand_ids, torch.int32, "cand_ids"), _dev(cand_off, torch.int32, "cand_off"), n, total,
        int(max_options), float(temperature), _dev(logits, torch.float32, "logits"),
        _dev_or_pinned(probs, torch.float32, "probs"),
        _dev_or_pinned(argmax, torch.int32, "argmax"),
        _stream(stream)]
    if not launch:
        return args
    _check(lib.blink_label_readout(*args))


@dataclass
class LabelRows:
    """Result of blink_pack_labels (host arrays)."""

    row_id: np.ndarray  # [n_rows] distinct label ids, ascending
    row_first: np.ndarray  # [n_rows + 1]
    row_entry: np.ndarray  # [total] flat option entries grouped by row
    n_rows: int


def pack_labels(cand_ids, cand_off, vocab: int) -> LabelRows:
    """Distinct label rows of an option table (blink_pack_labels)."""
    lib = load_library()
    ids = np.ascontiguousarray(np.asarray(cand_ids, dtype=np.int32))
    off = np.ascontiguousarray(np.asarray(cand_off, dtype=np.int32))
    n = int(off.shape[0]) - 1
    total = int(ids.shape[0])
    if n < 0 or (n and int(off[-1]) != total):
        raise BlinkError(BLINK_E_INVALID, "candidate offsets must run from 0 to len(cand_ids)")
    cap = max(total, 1)
    row_id = np.zeros(cap, np.int32)
    row_first = np.zeros(cap + 1, np.int32)
    row_entry = np.zeros(cap, np.int32)
    u = ctypes.c_int32(0)
    src_ids = ids if total else np.zeros(1, np.int32)
    src_off = off if n >= 0 and off.shape[0] else np.zeros(1, np.int32)
    _check(lib.blink_pack_labels(_ptr(src_ids, ctypes.c_int32), _ptr(src_off, ctypes.c_int32), n,
                                 int(vocab), _ptr(row_id, ctypes.c_int32),
                                 _ptr(row_first, ctypes.c_int32), _ptr(row_entry, ctypes.c_int32),
                                 ctypes.byref(u)))
    k = u.value
    return LabelRows(row_id[:k], row_first[:k + 1], row_entry[:total], k)


def label_readout_batched(hidden, last_row, w_u, cand_off, row_id, row_first, row_entry,
                          temperature: float, max_options: int, logits, probs, argmax,
                          stream=None, launch: bool = True):
    """Launches blink_label_readout_batched: as label_readout, with the option table given
    by its CSR offsets and its distinct-row tables (row_id int32 [U], row_first int32 [U + 1],
    row_entry int32 [sum K], device; from pack_labels). With ``launch=False`` returns the
    checked argument list instead, for repeated launches; it holds raw addresses, so the
    caller keeps every tensor alive while the list is in use."""
    import torch

    bf = torch.bfloat16
    if hidden.dim() != 2 or w_u.dim() != 2 or hidden.shape[1] != w_u.shape[1]:
        raise BlinkError(BLINK_E_INVALID, "hidden and w_u must be 2-D with the same width")
    n = int(last_row.shape[0])
    total = int(row_entry.shape[0])
    u = int(row_id.shape[0])
    if int(cand_off.shape[0]) != n + 1:
        raise BlinkError(BLINK_E_INVALID, "cand_off must have n + 1 entries")
    if int(row_first.shape[0]) != u + 1:
        raise BlinkError(BLINK_E_INVALID, "row_first must have n_rows + 1 entries")
    if int(logits.shape[0]) != total or int(probs.shape[0]) != total or int(argmax.shape[0]) != n:
        raise BlinkError(BLINK_E_INVALID, "output sizes do not match the candidate table")
    lib = load_library()
    args = [
        _dev(hidden, bf, "hidden"), int(hidden.shape[0]), int(hidden.shape[1]),
        _dev(last_row, torch.int64, "last_row"), _dev(w_u, bf, "w_u"), int(w_u.shape[0]),
        _dev(cand_off, torch.int32, "cand_off"), n, total, int(max_options),
        _dev(row_id, torch.int32, "row_id"), _dev(row_first, torch.int32, "row_first"),
        _dev(row_entry, torch.int32, "row_entry"), u, float(temperature),
        _dev(logits, torch.float32, "logits"), _dev_or_pinned(probs, torch.float32, "probs"),
        _dev_or_pinned(argmax, torch.int32, "argmax"), _stream(stream)]
    if not launch:
        return args
    _check(lib.blink_label_readout_batched(*args))


def check_candidate_table(cand_ids, cand_off, vocab: int) -> int:
    """Host-side check of a candidate table before upload; returns max options per question.

    Mirrors the pages' rules ("rendering" section: 1-255 options; "torch engine" section:
    label token ids are distinct)."""
    ids = np.asarray(cand_ids)
    off = np.asarray(cand_off)
    if off.ndim != 1 or off.shape[0] < 2 or off[0] != 0 or off[-1] != ids.shape[0]:
        raise BlinkError(BLINK_E_INVALID, "candidate offsets must run from 0 to len(cand_ids)")
    k = np.diff(off)
    for i, ki in enumerate(k):
        if not 1 <= ki <= MAX_OPTIONS:
            raise BlinkError(BLINK_E_LIMIT, f"question with {int(ki)} options; the limit is 1 to {MAX_OPTIONS}")
        row = ids[off[i]:off[i + 1]]
        if row.min() < 0 or row.max() >= vocab:
            raise BlinkError(BLINK_E_INVALID, f"question {i}: label token id out of range")
        if np.unique(row).shape[0] != row.shape[0]:
            raise BlinkError(BLINK_E_INVALID, f"question {i}: label token ids collide")
    return int(k.max())
