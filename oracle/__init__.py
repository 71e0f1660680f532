"""Plain, slow CPU oracle of the one-pass typed-decision scoring hot path.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link this
package: only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` use it. It shares no code with the HIP library (no kernels, headers, tables or
helpers); both sides are fed the same seeded inputs from ``synth``.

It follows the blink.py page (thegovind/blink-4b):
  * ``pack``      -- the ragged right-padded packer ("torch engine" section: _batches, _padded,
                     and the batch loop of _forward / _forward_shared);
  * ``attention`` -- causal attention of each question's tail over one shared prefix, computed
                     as the plain full-sequence definition and, independently, as a prefix
                     partial merged with a tail partial ("torch engine" section: _forward_shared;
                     PREFIX_CACHE comment in "constants the deployment sets");
  * ``readout``   -- last-valid-row gather, FP64 dot against the offered labels' unembedding
                     rows, temperature softmax and first-index argmax ("torch engine" section:
                     _read; "answer assembly" section: softmax and answer_for), and its
                     batched form over the distinct label rows (_read_batched);
  * ``prefix``    -- shared-prefix detection, the minimum-length switch and the count of tokens
                     computed ("torch engine" section: _shared_prefix_len, _prefill_tokens,
                     _forward; PREFIX_MIN_TOKENS in "constants the deployment sets");
  * ``answers``   -- typed answers from the option probabilities ("answer assembly" section:
                     answer_for);
  * ``scoring``   -- teacher-forced scoring of a sequence's last tokens: full-vocabulary
                     log-softmax at each scored row, read at the next token (the simit MoT
                     engine page: score_len);
  * ``refine``    -- rotation averaging of label log-probabilities with an optional
                     content-free prior, and the two-stage choice's finalists (the ruling
                     page: _score_plain, TwoStageChoice).

Arithmetic is float64 throughout; bf16 inputs are widened exactly.
Every function is pinned by tests under ``tests/test_oracle_*.py``; none is "parity unpinned".
"""

from .pack import pack_ragged, MAX_QUESTIONS, MAX_INPUT_TOKENS, TOKEN_BUDGET
from .attention import (
    bf16_to_f64,
    attention_full,
    attention_decomposed,
    attention_rows,
    attention_grouped,
)
from .readout import label_readout, label_readout_batched, label_rows, softmax_t, MAX_OPTIONS
from .path import score_request
from .prefix import plan_prefix, shared_prefix_len, PREFIX_MIN_TOKENS
from .answers import answer_for, assemble
from .scoring import score_rows, teacher_forced_logprobs
from .refine import combine_rotations, scatter_finalists, two_stage_finalists

__all__ = [
    "pack_ragged",
    "MAX_QUESTIONS",
    "MAX_INPUT_TOKENS",
    "TOKEN_BUDGET",
    "MAX_OPTIONS",
    "bf16_to_f64",
    "attention_full",
    "attention_decomposed",
    "attention_rows",
    "attention_grouped",
    "label_readout",
    "label_readout_batched",
    "label_rows",
    "softmax_t",
    "score_request",
    "plan_prefix",
    "shared_prefix_len",
    "PREFIX_MIN_TOKENS",
    "answer_for",
    "assemble",
    "score_rows",
    "teacher_forced_logprobs",
    "combine_rotations",
    "scatter_finalists",
    "two_stage_finalists",
]
