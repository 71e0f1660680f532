"""One scoring step of a request, chained through the C ABI.

A step is the hot path of the blink.py page (thegovind/blink-4b, "torch engine" section,
_forward_shared and _read, and "answer assembly" section, softmax): pack the question tails
(host), upload the small row tables, run the shared-prefix tail attention and the label
readout on the GPU, and bring the label probabilities and argmax back to the host. The
request's tensors stay resident on the device between steps.
"""

from __future__ import annotations

import ctypes
import itertools
import os
import string

import numpy as np

from ._binding import (
    BlinkError,
    BLINK_E_INVALID,
    check_candidate_table,
    label_readout,
    label_readout_batched,
    load_library,
    pack_labels,
    pack_ragged,
    pack_ragged_args,
    prefix_tail_attention,
    TOKEN_BUDGET,
)

# Option index -> label: A..Z, then AA..ZZ ("constants the deployment sets" section:
# LABEL_POOL), at most 255 of them.
_LABELS = list(string.ascii_uppercase) + [
    a + b for a, b in itertools.product(string.ascii_uppercase, repeat=2)]


_HIP_MEMCPY_H2D = 1


def _hip_runtime():
    try:
        return ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)
    except OSError as exc:
        raise RuntimeError("the HIP runtime is not loaded in this process") from exc


def _hip_memcpy_async():
    """hipMemcpyAsync of the HIP runtime this process already runs (torch and libblink.so
    share one copy). Queuing a copy through it avoids torch's stream-context switch, which
    costs several microseconds per copy on the host."""
    try:
        hip = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)
    except OSError as exc:
        raise RuntimeError("the HIP runtime is not loaded in this process") from exc
    fn = hip.hipMemcpyAsync
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                   ctypes.c_void_p]
    return fn


def label_name(index: int) -> str:
    if not 0 <= index < 255:
        raise BlinkError(BLINK_E_INVALID, f"option index {index} outside 0-254")
    return _LABELS[index]


class ScoringStep:
    """Device-resident request plus reusable buffers; ``run()`` is one scoring step.

    Everything that does not change between steps is prepared once: the packer writes the
    row tables straight into one pinned buffer that a single copy uploads, the launches use
    argument lists validated at construction, and the readout writes the probabilities and
    argmax straight into one pinned host buffer. Those host buffers are reused, so a step
    queued with ``run(fetch=False)`` must be synchronised before the next step is packed.

    ``depth`` (1 to 4) is the number of steps that may be in flight. Each slot beyond the first
    has its own pinned row tables and results, its own device row tables, attention output and
    logits, and its own stream (default priority), so step k + 1 can be packed and queued with
    ``submit()`` while step k still runs, and its kernels can start on compute units that
    step k's last workgroups leave idle; ``collect()`` waits for the oldest step and returns its
    results. The request's inputs are shared and only read.

    ``readout``: "per_option" (blink_label_readout, the default) or "batched"
    (blink_label_readout_batched over the request's distinct label rows, built once here by
    blink_pack_labels). Both give bitwise the same results; on MI355X the per-option form is
    the faster one even where many questions share label rows."""

    def __init__(self, tail_len, cand_ids, cand_off, tensors: dict, n_heads_q: int,
                 n_heads_kv: int, prefix_len: int, temperature: float, scale: float,
                 token_budget: int = TOKEN_BUDGET, max_rows: int = 0, stream=None,
                 readout: str = "per_option", depth: int = 1):
        import ctypes

        import torch

        self.torch = torch
        if depth not in (1, 2, 3, 4):
            raise BlinkError(BLINK_E_INVALID, "depth must be 1 to 4")
        self.tail_len = np.ascontiguousarray(np.asarray(tail_len, np.int32))
        n = self.n = int(self.tail_len.shape[0])
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

        # Row tables, host (pinned) and device, in one buffer each: token_offset int64 [n],
        # last_row int64 [n], valid_start int32 [n + 1].
        words = 2 * n + (n + 2) // 2
        self.h_tab = torch.zeros(words, dtype=torch.int64, pin_memory=True)
        self.d_tab = torch.zeros(words, dtype=torch.int64, device=dev)
        tab = self.h_tab.numpy()
        self.h_token_offset, self.h_last_row = tab[:n], tab[n:2 * n]
        self.h_valid_start = tab[2 * n:].view(np.int32)[:n + 1]
        self.d_token_offset, self.d_last_row = self.d_tab[:n], self.d_tab[n:2 * n]
        self.d_valid_start = self.d_tab[2 * n:].view(torch.int32)[:n + 1]
        # The packer's other outputs (host only).
        self._order, self._batch_of, self._row_of = (np.zeros(n, np.int32) for _ in range(3))
        self._batch_first = np.zeros(n + 1, np.int32)
        self._batch_width = np.zeros(n, np.int32)
        self._batch_base = np.zeros(n + 1, np.int64)
        self._nb, self._tp, self._tv = ctypes.c_int32(0), ctypes.c_int64(0), ctypes.c_int64(0)

        t_pad = pk.total_padded_tokens
        self.out = torch.empty(t_pad, n_heads_q, tensors["q"].shape[2], dtype=torch.bfloat16,
                               device=dev)
        self.logits = torch.empty(total, dtype=torch.float32, device=dev)
        # Probabilities and argmax in one pinned host buffer (float32 [total] then int32 [n])
        # that the readout kernels write directly: no copy back.
        self.h_res = torch.empty(total + n, dtype=torch.float32, pin_memory=True)
        self.h_probs, self.h_argmax = self.h_res[:total], self.h_res[total:].view(torch.int32)

        # Argument lists checked once; every step reuses them.
        lib = load_library()
        self._copy_fn = _hip_memcpy_async()
        stream_handle = ctypes.c_void_p(self.stream.cuda_stream)
        self._up_args = (ctypes.c_void_p(self.d_tab.data_ptr()),
                         ctypes.c_void_p(self.h_tab.data_ptr()),
                         ctypes.c_size_t(self.h_tab.numel() * 8), _HIP_MEMCPY_H2D, stream_handle)
        self._pack_fn = lib.blink_pack_ragged
        self._pack_args = pack_ragged_args(
            self.tail_len, self.prefix_len, self.token_budget, self.max_rows, self._order,
            self._batch_of, self._row_of, self.h_token_offset, self.h_last_row,
            self.h_valid_start, self._batch_first, self._batch_width, self._batch_base,
            self._nb, self._tp, self._tv)
        t = tensors
        self._attn_fn = lib.blink_prefix_tail_attention
        self._attn_args = prefix_tail_attention(
            t["q"], t["k_tail"], t["v_tail"], t.get("k_prefix"), t.get("v_prefix"), self.out,
            self.d_token_offset, self.d_valid_start, pk.total_valid_tokens, self.scale,
            stream=self.stream.cuda_stream, launch=False)
        if readout not in ("batched", "per_option"):
            raise BlinkError(BLINK_E_INVALID, f"unknown readout form {readout!r}")
        self.readout_form = readout
        self.label_rows = None
        if readout == "batched":
            lr = self.label_rows = pack_labels(cand_ids, cand_off, vocab)
            self.d_rows = [torch.as_tensor(a).to(dev)
                           for a in (lr.row_id, lr.row_first, lr.row_entry)]
            self._read_fn = lib.blink_label_readout_batched
            self._read_args = label_readout_batched(
                t["hidden"], self.d_last_row, t["w_u"], self.cand_off, *self.d_rows,
                self.temperature, self.max_options, self.logits, self.h_probs, self.h_argmax,
                stream=self.stream.cuda_stream, launch=False)
        else:
            self._read_fn = lib.blink_label_readout
            self._read_args = label_readout(
                t["hidden"], self.d_last_row, t["w_u"], self.cand_ids, self.cand_off,
                self.temperature, self.max_options, self.logits, self.h_probs, self.h_argmax,
                stream=self.stream.cuda_stream, launch=False)

        # Slot 0 is the buffers above, on the caller's stream. A second slot gets its own host
        # and device buffers and its own stream (see the class docstring).
        hip = _hip_runtime()
        self._ev_record, self._ev_sync = hip.hipEventRecord, hip.hipEventSynchronize
        self._ev_record.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self._ev_sync.argtypes = [ctypes.c_void_p]
        self._stream_handle = stream_handle
        self._slots = [self._slot(hip, self.h_tab, self.h_res, self._pack_args, self._up_args,
                                  self._read_args)]
        self._slots[0].stream, self._slots[0].stream_handle = self.stream, stream_handle
        self._slots[0].attn_args = self._attn_args
        for _ in range(depth - 1):
            side = torch.cuda.Stream(device=dev)
            side.wait_stream(self.stream)  # the request's inputs, queued on the main stream
            side_handle = ctypes.c_void_p(side.cuda_stream)
            h_tab = torch.zeros_like(self.h_tab, pin_memory=True)
            h_res = torch.empty_like(self.h_res, pin_memory=True)
            d_tab = torch.zeros_like(self.d_tab)
            out = torch.empty_like(self.out)
            logits = torch.empty_like(self.logits)
            tab = h_tab.numpy()
            pack_args = pack_ragged_args(
                self.tail_len, self.prefix_len, self.token_budget, self.max_rows, self._order,
                self._batch_of, self._row_of, tab[:n], tab[n:2 * n],
                tab[2 * n:].view(np.int32)[:n + 1], self._batch_first, self._batch_width,
                self._batch_base, self._nb, self._tp, self._tv)
            up_args = (ctypes.c_void_p(d_tab.data_ptr()), ctypes.c_void_p(h_tab.data_ptr()),
                       self._up_args[2], _HIP_MEMCPY_H2D, side_handle)
            d_off, d_last = d_tab[:n], d_tab[n:2 * n]
            d_vs = d_tab[2 * n:].view(torch.int32)[:n + 1]
            attn_args = prefix_tail_attention(
                t["q"], t["k_tail"], t["v_tail"], t.get("k_prefix"), t.get("v_prefix"), out,
                d_off, d_vs, pk.total_valid_tokens, self.scale, stream=side.cuda_stream,
                launch=False)
            probs, argmax = h_res[:total], h_res[total:].view(torch.int32)
            if readout == "batched":
                read_args = label_readout_batched(
                    t["hidden"], d_last, t["w_u"], self.cand_off, *self.d_rows,
                    self.temperature, self.max_options, logits, probs, argmax,
                    stream=side.cuda_stream, launch=False)
            else:
                read_args = label_readout(
                    t["hidden"], d_last, t["w_u"], self.cand_ids, self.cand_off,
                    self.temperature, self.max_options, logits, probs, argmax,
                    stream=side.cuda_stream, launch=False)
            slot = self._slot(hip, h_tab, h_res, pack_args, up_args, read_args)
            slot.stream, slot.stream_handle, slot.attn_args = side, side_handle, attn_args
            slot.keep = (d_tab, out, logits)  # the argument lists hold their raw addresses
            self._slots.append(slot)
        self._next = 0
        self._queue = []

    def close(self):
        """Waits for outstanding steps and releases the slots' completion events."""
        while getattr(self, "_queue", None):
            self.collect()
        hip = _hip_runtime()
        for slot in getattr(self, "_slots", []):
            if slot.event:
                hip.hipEventDestroy(slot.event)
                slot.event = None
        self._slots = []

    def __del__(self):
        try:
            self.close()
        except Exception:  # interpreter shutdown: the runtime may already be gone
            pass

    def _slot(self, hip, h_tab, h_res, pack_args, up_args, read_args):
        from types import SimpleNamespace

        ev = ctypes.c_void_p()
        if hip.hipEventCreate(ctypes.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        total = int(self.logits.shape[0])
        return SimpleNamespace(h_tab=h_tab, h_res=h_res, pack_args=pack_args, up_args=up_args,
                               read_args=read_args, event=ev, busy=False,
                               probs=h_res[:total], argmax=h_res[total:].view(self.torch.int32))

    @staticmethod
    def _call(fn, args):
        rc = fn(*args)
        if rc != 0:
            raise BlinkError(rc, load_library().blink_last_error().decode("utf-8", "replace"))

    def _copy(self, args):
        if args[2].value == 0:
            return
        rc = self._copy_fn(*args)
        if rc != 0:
            raise RuntimeError(f"hipMemcpyAsync failed with HIP error {rc}")

    def pack_and_upload(self) -> int:
        """Packs the tails into the pinned tables and queues their upload (one copy);
        returns the number of real tail tokens."""
        self._call(self._pack_fn, self._pack_args)
        if self._tp.value != self.pack.total_padded_tokens:
            raise BlinkError(BLINK_E_INVALID, "tensors were not laid out for this pack")
        self._copy(self._up_args)
        return self._tv.value

    def attention(self, total_valid: int):
        self._attn_args[9] = int(total_valid)
        self._call(self._attn_fn, self._attn_args)

    def readout(self):
        """Queues the readout; it writes probabilities and argmax into pinned host memory,
        valid once the stream has been synchronised."""
        self._call(self._read_fn, self._read_args)

    def run(self, fetch: bool = True):
        """One step. With ``fetch`` the stream is synchronised and the (probs, argmax) host
        arrays are returned; without it the step is only queued."""
        total_valid = self.pack_and_upload()
        self.attention(total_valid)
        self.readout()
        if not fetch:
            return None
        self.stream.synchronize()
        return self.h_probs.numpy(), self.h_argmax.numpy()

    def submit(self):
        """Packs the next step into a free slot and queues it (upload, attention, readout and
        a completion event). At most ``depth`` steps may be outstanding."""
        if not self._slots:
            raise BlinkError(BLINK_E_INVALID, "the step was closed")
        slot = self._slots[self._next]
        if slot.busy:
            raise BlinkError(BLINK_E_INVALID, "every slot holds a step that was not collected")
        self._call(self._pack_fn, slot.pack_args)
        if self._tp.value != self.pack.total_padded_tokens:
            raise BlinkError(BLINK_E_INVALID, "tensors were not laid out for this pack")
        self._copy(slot.up_args)
        slot.attn_args[9] = int(self._tv.value)
        self._call(self._attn_fn, slot.attn_args)
        self._call(self._read_fn, slot.read_args)
        if self._ev_record(slot.event, slot.stream_handle) != 0:
            raise RuntimeError("hipEventRecord failed")
        slot.busy = True
        self._queue.append(slot)
        self._next = (self._next + 1) % len(self._slots)

    def outstanding(self) -> int:
        return len(self._queue)

    def collect(self):
        """Waits for the oldest submitted step; returns its (probs, argmax) host arrays, valid
        until that slot is submitted again."""
        if not self._queue:
            raise BlinkError(BLINK_E_INVALID, "no step to collect")
        slot = self._queue.pop(0)
        if self._ev_sync(slot.event) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        slot.busy = False
        return slot.probs.numpy(), slot.argmax.numpy()
