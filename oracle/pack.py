"""Oracle for the ragged right-padded packer (test infrastructure only).

Follows the blink.py page (thegovind/blink-4b):
  * "constants the deployment sets": at most 512 questions per request, at most 131072
    rendered tokens per question, a budget of 32768 padded tokens per forward;
  * "torch engine" section, _batches: questions are visited shortest first; a batch is
    closed before a question joins it when the padded size (widest row times row count,
    counting the newcomer) would exceed the budget, or when an optional row cap is reached;
    a question longer than the budget therefore always runs in a batch of its own;
  * "torch engine" section, _padded: each batch is a [rows, width] block whose width is its
    longest member; every row is left-aligned and right-padded;
  * "torch engine" section, _forward_shared: with a shared prefix only the tails are packed,
    so the budget counts tail tokens.

Reading (the pages keep one tensor per forward and say nothing about a single buffer): the
batches are laid end to end in visiting order in one token-major buffer, so a question's
rows are addressed by a token offset into that buffer.
"""

from __future__ import annotations

MAX_QUESTIONS = 512
MAX_INPUT_TOKENS = 131072
TOKEN_BUDGET = 32768


class PackError(ValueError):
    """An input the packer refuses (the pages raise a ValueError subclass for these)."""


def _visit_order(lengths):
    # Shortest first; equal lengths keep their question index order.
    return sorted(range(len(lengths)), key=lambda i: (lengths[i], i))


def _group(lengths, budget, max_rows):
    """Greedy grouping of the visiting order into batches."""
    groups = []
    for i in _visit_order(lengths):
        if groups:
            current = groups[-1]
            width = max([lengths[j] for j in current] + [lengths[i]])
            within_budget = width * (len(current) + 1) <= budget
            below_cap = max_rows <= 0 or len(current) < max_rows
            if within_budget and below_cap:
                current.append(i)
                continue
        groups.append([i])
    return groups


def pack_ragged(tail_len, token_budget=TOKEN_BUDGET, max_rows=0, prefix_len=0,
                max_input_tokens=MAX_INPUT_TOKENS):
    """Pack question tails into right-padded batches laid end to end.

    Returns a dict of plain Python lists / ints:
      order          questions in visiting order (batch by batch, row by row)
      batch_of, row_of   per question (indexed by question)
      token_offset   per question: first token of its row in the concatenated buffer
      last_row       per question: token index of its last valid token
      batch_first    [n_batches + 1] start of each batch in ``order``
      batch_width    [n_batches] padded width
      batch_base     [n_batches + 1] first token of each batch; the last entry is the total
      n_batches, total_padded_tokens, total_valid_tokens
    """
    lengths = [int(x) for x in tail_len]
    n = len(lengths)
    if not 1 <= n <= MAX_QUESTIONS:
        raise PackError(f"request of {n} questions; the limit is 1 to {MAX_QUESTIONS}")
    if prefix_len < 0:
        raise PackError("prefix length must be non-negative")
    if token_budget < 1:
        raise PackError("token budget is below 1")
    if max_rows < 0:
        raise PackError("row cap must be non-negative")
    for i, length in enumerate(lengths):
        if length < 1:
            raise PackError(f"question {i} has an empty tail")
        if prefix_len + length > max_input_tokens:
            raise PackError(
                f"question {i} needs {prefix_len + length} tokens of context; the maximum "
                f"context length is {max_input_tokens}")

    groups = _group(lengths, token_budget, max_rows)
    order, batch_first, batch_width, batch_base = [], [0], [], [0]
    batch_of, row_of = [0] * n, [0] * n
    token_offset, last_row = [0] * n, [0] * n
    for b, members in enumerate(groups):
        width = max(lengths[i] for i in members)
        for r, i in enumerate(members):
            batch_of[i] = b
            row_of[i] = r
            token_offset[i] = batch_base[b] + r * width
            last_row[i] = token_offset[i] + lengths[i] - 1
            order.append(i)
        batch_width.append(width)
        batch_first.append(len(order))
        batch_base.append(batch_base[b] + len(members) * width)
    return {
        "order": order,
        "batch_of": batch_of,
        "row_of": row_of,
        "token_offset": token_offset,
        "last_row": last_row,
        "batch_first": batch_first,
        "batch_width": batch_width,
        "batch_base": batch_base,
        "n_batches": len(groups),
        "total_padded_tokens": batch_base[-1],
        "total_valid_tokens": sum(lengths),
    }
