"""One-pass typed-decision scoring hot path for MI355X (gfx950).

Three calls, each a thin binding of the C ABI in ``include/blink.h`` (libblink.so):

* ``pack_ragged``            -- host packer: question tails into right-padded batches;
* ``prefix_tail_attention``  -- HIP kernel: every tail attends to one cached prefix and
                                causally to itself (bf16 MFMA, FP32 online softmax);
* ``label_readout``          -- HIP kernel: last-real-row gather, FP32 dot with the offered
                                labels' unembedding rows, temperature softmax, argmax.

``ScoringStep`` chains them for one request (the hot path of one scoring step);
``GroupedScoringStep`` runs several requests, each with its own prefix, in one pass.
"""

from ._binding import (
    BlinkError,
    BLINK_OK,
    BLINK_E_INVALID,
    BLINK_E_LIMIT,
    BLINK_E_DEVICE,
    EXPORTS,
    LIBRARY,
    MAX_INPUT_TOKENS,
    MAX_OPTIONS,
    MAX_QUESTIONS,
    TOKEN_BUDGET,
    GroupedAttention,
    LabelRows,
    MAX_REQUESTS,
    Pack,
    PREFIX_MIN_TOKENS,
    PrefixPlan,
    TargetScorer,
    ANSWER_CHOICE,
    ANSWER_NOUL,
    ANSWER_SCORE,
    assemble_answers,
    check_candidate_table,
    combine_rotations,
    encode_prefix_attention,
    label_readout,
    label_readout_batched,
    load_library,
    pack_labels,
    pack_ragged,
    plan_prefix,
    two_stage_finalists,
    attention_workspace,
    prefix_tail_attention,
)
from .group import GroupRequest, GroupedScoringStep
from .path import ScoringStep, label_name

__all__ = [
    "BlinkError",
    "BLINK_OK",
    "BLINK_E_INVALID",
    "BLINK_E_LIMIT",
    "BLINK_E_DEVICE",
    "EXPORTS",
    "LIBRARY",
    "MAX_INPUT_TOKENS",
    "MAX_OPTIONS",
    "MAX_QUESTIONS",
    "TOKEN_BUDGET",
    "GroupedAttention",
    "LabelRows",
    "MAX_REQUESTS",
    "Pack",
    "PREFIX_MIN_TOKENS",
    "PrefixPlan",
    "TargetScorer",
    "plan_prefix",
    "ANSWER_CHOICE",
    "ANSWER_NOUL",
    "ANSWER_SCORE",
    "assemble_answers",
    "check_candidate_table",
    "combine_rotations",
    "two_stage_finalists",
    "encode_prefix_attention",
    "label_readout",
    "label_readout_batched",
    "load_library",
    "pack_labels",
    "pack_ragged",
    "attention_workspace",
    "prefix_tail_attention",
    "ScoringStep",
    "GroupRequest",
    "GroupedScoringStep",
    "label_name",
]
