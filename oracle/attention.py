"""Oracle for shared-prefix tail-prefill attention (test infrastructure only).

What is computed (blink.py page, thegovind/blink-4b, "torch engine" section, _forward_shared
and _forward; PREFIX_CACHE comment in "constants the deployment sets"): the shared prefix is
encoded once, and each question's own tail then runs against that cached prefix. The pages
state that this keeps the same tokens and positions as running every question's full
sequence and only changes floating-point order, and that every layer is causal. So for
question i, query head h and tail position t (t < n_i), the result is plain causal softmax
attention over the full sequence [prefix ; tail_i] at row P + t:

    s_j = scale * <q_t, k_j>   for every prefix key and every tail key j <= t
    o   = sum_j exp(s_j - max s) v_j / sum_j exp(s_j - max s)

Readings where the pages are silent:
  * query head h reads KV head floor(h / (H_q / H_kv)) (contiguous groups);
  * inputs are already rotated (no RoPE here) and ``scale`` is given (1/sqrt(D) in the workloads);
  * padded rows (t >= n_i) are not part of the result; they are NaN here;
  * layouts are token-major: Q [T_pad, H_q, D], tail K/V [T_pad, H_kv, D], prefix K/V [P, H_kv, D].

Two independent forms are provided: ``attention_full`` (the definition above over the
concatenated sequence) and ``attention_decomposed`` (a prefix partial and a tail partial
merged through their log-sum-exp), which is the reordering the shared-prefix path relies on.
All arithmetic is float64; bf16 inputs are widened exactly.
"""

from __future__ import annotations

import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _as_f64(x):
    x = np.asarray(x)
    return bf16_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)


def _kv_head(h, n_heads_q, n_heads_kv):
    if n_heads_q % n_heads_kv:
        raise ValueError("query heads must be a multiple of KV heads")
    return h // (n_heads_q // n_heads_kv)


def _softmax_rows(s):
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    return w / w.sum(axis=1, keepdims=True)


def _question_full(q_rows, k_pre, v_pre, k_tail, v_tail, scale):
    """Plain causal attention of tail rows over [prefix ; tail], float64, one head."""
    n, p = q_rows.shape[0], k_pre.shape[0]
    keys = np.concatenate([k_pre, k_tail], axis=0)
    values = np.concatenate([v_pre, v_tail], axis=0)
    s = scale * (q_rows @ keys.T)
    # Row t of the tail sits at absolute position p + t and sees keys 0 .. p + t.
    visible = np.arange(p + n)[None, :] <= (p + np.arange(n))[:, None]
    s = np.where(visible, s, -np.inf)
    return _softmax_rows(s) @ values


def _partial(q_rows, keys, values, scale, visible=None):
    """Unnormalised softmax partial: (row max, row sum of weights, weighted value sum)."""
    s = scale * (q_rows @ keys.T)
    if visible is not None:
        s = np.where(visible, s, -np.inf)
    m = s.max(axis=1)
    w = np.exp(s - m[:, None])
    return m, w.sum(axis=1), w @ values


def _question_decomposed(q_rows, k_pre, v_pre, k_tail, v_tail, scale):
    n, p = q_rows.shape[0], k_pre.shape[0]
    causal = np.arange(n)[None, :] <= np.arange(n)[:, None]
    m_t, l_t, o_t = _partial(q_rows, k_tail, v_tail, scale, causal)
    if p == 0:
        return o_t / l_t[:, None]
    m_p, l_p, o_p = _partial(q_rows, k_pre, v_pre, scale)
    m = np.maximum(m_p, m_t)
    a_p, a_t = np.exp(m_p - m), np.exp(m_t - m)
    return (a_p[:, None] * o_p + a_t[:, None] * o_t) / (a_p * l_p + a_t * l_t)[:, None]


def _run(form, q, k_tail, v_tail, k_prefix, v_prefix, token_offset, tail_len,
         n_heads_q, n_heads_kv, scale, questions=None):
    q = _as_f64(q)
    k_tail, v_tail = _as_f64(k_tail), _as_f64(v_tail)
    t_pad, hq, d = q.shape
    hkv = k_tail.shape[1]
    if hq != n_heads_q or hkv != n_heads_kv:
        raise ValueError("head counts do not match the tensors")
    if k_prefix is None or np.asarray(k_prefix).size == 0:
        k_prefix = np.zeros((0, hkv, d))
        v_prefix = np.zeros((0, hkv, d))
    k_prefix, v_prefix = _as_f64(k_prefix), _as_f64(v_prefix)
    out = np.full((t_pad, hq, d), np.nan)
    qs = range(len(tail_len)) if questions is None else questions
    for i in qs:
        off, n = int(token_offset[i]), int(tail_len[i])
        for h in range(hq):
            g = _kv_head(h, hq, hkv)
            out[off:off + n, h, :] = form(
                q[off:off + n, h, :], k_prefix[:, g, :], v_prefix[:, g, :],
                k_tail[off:off + n, g, :], v_tail[off:off + n, g, :], scale)
    return out


def attention_full(q, k_tail, v_tail, k_prefix, v_prefix, token_offset, tail_len,
                   n_heads_q, n_heads_kv, scale, questions=None):
    """[T_pad, H_q, D] float64 output by the plain full-sequence definition; pad rows NaN."""
    return _run(_question_full, q, k_tail, v_tail, k_prefix, v_prefix, token_offset,
                tail_len, n_heads_q, n_heads_kv, scale, questions)


def attention_decomposed(q, k_tail, v_tail, k_prefix, v_prefix, token_offset, tail_len,
                         n_heads_q, n_heads_kv, scale, questions=None):
    """Same result through a prefix partial and a tail partial merged by log-sum-exp."""
    return _run(_question_decomposed, q, k_tail, v_tail, k_prefix, v_prefix, token_offset,
                tail_len, n_heads_q, n_heads_kv, scale, questions)


def attention_rows(q, k_tail, v_tail, k_prefix, v_prefix, token_offset, tail_len,
                   n_heads_q, n_heads_kv, scale, rows):
    """Plain definition for selected outputs only: ``rows`` is a list of
    (question, tail position, query head); returns float64 [len(rows), D]."""
    hq, hkv = n_heads_q, n_heads_kv
    d = np.asarray(q).shape[2]
    out = np.zeros((len(rows), d))
    p = 0 if k_prefix is None else np.asarray(k_prefix).shape[0]
    by_group = {}
    for r, (i, t, h) in enumerate(rows):
        if not 0 <= t < int(tail_len[i]):
            raise ValueError("sampled row is not a valid tail position")
        by_group.setdefault((int(i), _kv_head(int(h), hq, hkv)), []).append((r, int(t), int(h)))
    for (i, g), members in by_group.items():
        off, n = int(token_offset[i]), int(tail_len[i])
        k_pre = _as_f64(k_prefix[:, g, :]) if p else np.zeros((0, d))
        v_pre = _as_f64(v_prefix[:, g, :]) if p else np.zeros((0, d))
        keys = np.concatenate([k_pre, _as_f64(k_tail[off:off + n, g, :])], axis=0)
        values = np.concatenate([v_pre, _as_f64(v_tail[off:off + n, g, :])], axis=0)
        for r, t, h in members:
            qt = _as_f64(q[off + t, h, :])
            s = scale * (keys[: p + t + 1] @ qt)
            w = np.exp(s - s.max())
            out[r] = (w @ values[: p + t + 1]) / w.sum()
    return out


def attention_grouped(q, k_tail, v_tail, k_prefix, v_prefix, token_offset, tail_len,
                      request_first, prefix_start, prefix_len, n_heads_q, n_heads_kv, scale):
    """Several requests in one packed buffer, each question attending to its own request's
    prefix (rows prefix_start[r] .. prefix_start[r] + prefix_len[r] of k/v_prefix) and to its
    own tail: the plain full-sequence definition applied request by request ("public entry
    point" section of the blink.py page: the questions of several requests share one call)."""
    q = np.asarray(q)
    out = np.full((q.shape[0], n_heads_q, q.shape[2]), np.nan)
    for r in range(len(request_first) - 1):
        qs = range(int(request_first[r]), int(request_first[r + 1]))
        p0, pl = int(prefix_start[r]), int(prefix_len[r])
        kp = None if pl == 0 else np.asarray(k_prefix)[p0:p0 + pl]
        vp = None if pl == 0 else np.asarray(v_prefix)[p0:p0 + pl]
        part = attention_full(q, k_tail, v_tail, kp, vp, token_offset, tail_len, n_heads_q,
                              n_heads_kv, scale, questions=qs)
        for i in qs:
            off, n = int(token_offset[i]), int(tail_len[i])
            out[off:off + n] = part[off:off + n]
    return out
