"""Oracle for shared-prefix detection and prefill accounting (test infrastructure only).

Follows the blink.py page (thegovind/blink-4b):
  * "torch engine" section, _shared_prefix_len: the number of leading tokens that every
    question's full token sequence has in common, cut so that every sequence keeps at least
    one token of its own (its answer position must be computed in the per-question pass);
    none when there are fewer than two sequences;
  * "constants the deployment sets": PREFIX_MIN_TOKENS (256), the shared length below which
    the plain path is used because it is as fast;
  * "torch engine" section, _forward (the shared path only when the shared length is
    positive and at least PREFIX_MIN_TOKENS) and _prefill_tokens (tokens the model computes:
    the shared prefix once when it is reused, otherwise every token of every sequence).

The shared length is computed here column by column over all sequences, the plain
definition; the page reaches the same value through the lexicographically smallest and
largest sequences.
"""

from __future__ import annotations

PREFIX_MIN_TOKENS = 256


class PrefixError(ValueError):
    pass


def shared_prefix_len(seqs) -> int:
    """Length of the token prefix common to every sequence, at most (shortest length - 1);
    0 for fewer than two sequences."""
    seqs = [list(s) for s in seqs]
    if len(seqs) < 2:
        return 0
    shortest = min(len(s) for s in seqs)
    p = 0
    while p < shortest and all(s[p] == seqs[0][p] for s in seqs):
        p += 1
    return max(0, min(p, shortest - 1))


def plan_prefix(seqs, min_prefix_tokens: int = PREFIX_MIN_TOKENS):
    """Returns (shared, prefix_len, prefill_tokens): the shared length; the prefix the shared
    path encodes once (the shared length when it is at least min_prefix_tokens, else 0 for
    the plain path); and the tokens the model computes for these sequences."""
    if min_prefix_tokens < 1:
        raise PrefixError("the minimum shared prefix must be at least 1")
    seqs = [list(s) for s in seqs]
    if any(len(s) < 1 for s in seqs):
        raise PrefixError("every sequence needs at least one token")
    shared = shared_prefix_len(seqs)
    total = sum(len(s) for s in seqs)
    if shared > 0 and shared >= min_prefix_tokens:
        return shared, shared, total - (len(seqs) - 1) * shared
    return shared, 0, total
