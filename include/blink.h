/*
 * blink.h -- C ABI of the one-pass typed-decision scoring hot path on MI355X (gfx950).
 *
 * The method (blink.py page, thegovind/blink-4b, module docstring and "torch engine"
 * section): every question of a request is run as a right-padded prefill that generates no
 * token; question tails are packed into batches under a padded-token budget; with the shared
 * prefix opt-in, the prefix (system prompt plus evidence) is encoded once and every tail
 * attends to it; each question's answer is the next-token distribution over its offered
 * option labels, read from the hidden row of its last real token.
 *
 * Request model: one shared prefix of P >= 0 tokens plus 1..512 questions. A question has its
 * own tail of n_i >= 1 tokens (P + n_i <= 131072) and 1..255 options; option k is the label
 * A..Z, AA..ZZ with index k and maps to one token id, i.e. one unembedding row.
 *
 * Conventions shared by every entry point:
 *  - Return value: BLINK_OK (0) or a negative BLINK_E_* code. On error, blink_last_error()
 *    returns a message for the calling thread (the text stays valid until that thread's next
 *    call into the library); on success it returns "".
 *  - Every argument error is detected before anything is launched; a call that fails
 *    validation has no effect on device memory.
 *  - The caller owns all memory and the stream. The library allocates no device memory,
 *    keeps no global state between calls and may be called from several threads. Calls that
 *    need scratch memory take it from the caller as a workspace (blink_score_targets, and
 *    blink_prefix_tail_attention where its work split uses one); the variant
 *    blink_score_targets_noalloc uses a fixed static scratch array instead (the one exception
 *    to "no global state", described there). The library also remembers each device's
 *    compute-unit count after first reading it (a property of the hardware, not of a call).
 *  - Device entry points are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream). Device arrays must stay alive until the work on `stream` has finished.
 *  - bf16 means the 16-bit brain-float storage format. All tensors are dense and row-major
 *    with the last dimension contiguous; device tensors must be 16-byte aligned.
 *  - Tables that live on the device (offsets, ids) are read by the kernels without host
 *    checks. The kernels never access memory outside the sizes passed in, whatever the table
 *    contents: a malformed entry makes that question's outputs NaN / -1 (readout) or leaves
 *    its attention rows unwritten.
 */
#ifndef BLINK_H
#define BLINK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BLINK_OK 0
#define BLINK_E_INVALID (-1) /* malformed argument: null pointer, bad size, bad alignment */
#define BLINK_E_LIMIT (-2)   /* a limit of the method is exceeded (questions, options, context) */
#define BLINK_E_DEVICE (-3)  /* the HIP runtime refused a launch */

/* Limits of the method ("constants the deployment sets" section of the blink.py page). */
#define BLINK_MAX_QUESTIONS 512
#define BLINK_MAX_OPTIONS 255
#define BLINK_MAX_INPUT_TOKENS 131072
#define BLINK_TOKEN_BUDGET 32768
#define BLINK_MAX_REQUESTS 64 /* prefixes in one grouped attention launch */
#define BLINK_PREFIX_MIN_TOKENS 256 /* shared prefixes shorter than this take the plain path */

/* Message for the calling thread's last failed call; "" after a successful call. */
const char *blink_last_error(void);

/* ABI version of this header (incremented on any signature change). */
int blink_abi_version(void);
#define BLINK_ABI_VERSION 9

/*
 * blink_pack_ragged -- host, synchronous, integer only.
 *
 * Packs question tails into right-padded batches ("torch engine" section: _batches and
 * _padded, and the tail loop of _forward_shared). Questions are visited in ascending tail
 * length, equal lengths in question order. A question joins the current batch unless the
 * batch's padded size with it (widest row times rows, newcomer included) would exceed
 * `token_budget`, or the batch already holds `max_rows` rows (max_rows > 0); otherwise it
 * opens a new batch, so a question longer than the budget runs alone. A batch's width is its
 * longest tail; rows are left-aligned. Batches are laid end to end in visiting order in one
 * token-major buffer of `*total_padded_tokens` tokens (this single-buffer layout is this
 * library's reading; the pages keep one tensor per forward).
 *
 * Inputs (host):
 *   tail_len[n]       tokens of each question's own tail, >= 1
 *   n_questions       1..512                          (else BLINK_E_LIMIT)
 *   prefix_len        P >= 0; only checks P + tail_len[i] <= 131072 (else BLINK_E_LIMIT,
 *                     message names the question and "the maximum context length")
 *   token_budget      >= 1 (the pages use 32768)
 *   max_rows          0 = no row cap, else rows per batch at most max_rows
 * Outputs (host arrays the caller allocates; any may not be NULL):
 *   order[n]          questions in visiting order
 *   batch_of[n], row_of[n]      batch and row of each question
 *   token_offset[n]   first token of the question's row in the packed buffer
 *   last_row[n]       token index of the question's last real token (its readout row)
 *   valid_start[n+1]  exclusive prefix sum of tail_len in question order (valid_start[n] =
 *                     total real tokens); this is the row table the attention call takes
 *   batch_first[n+1]  start of each batch in order[]; entries past n_batches are unspecified
 *   batch_width[n]    padded width of each batch
 *   batch_base[n+1]   first token of each batch; batch_base[n_batches] = total padded tokens
 *   n_batches, total_padded_tokens, total_valid_tokens (scalars)
 */
int blink_pack_ragged(const int32_t *tail_len, int32_t n_questions, int32_t prefix_len,
                      int64_t token_budget, int32_t max_rows,
                      int32_t *order, int32_t *batch_of, int32_t *row_of,
                      int64_t *token_offset, int64_t *last_row, int32_t *valid_start,
                      int32_t *batch_first, int32_t *batch_width, int64_t *batch_base,
                      int32_t *n_batches, int64_t *total_padded_tokens,
                      int64_t *total_valid_tokens);

/*
 * blink_pack_labels -- host, synchronous, integer only.
 *
 * Distinct label rows of an option table ("torch engine" section, _read_batched: the
 * distinct label token ids of the questions, in ascending order, each gathered once). The
 * flat option entries are the positions 0..total-1 of cand_ids (total = cand_off[n]).
 *
 * Inputs (host):
 *   cand_ids[total]   token id of each offered label, each in [0, vocab) (else
 *                     BLINK_E_INVALID, naming the entry)
 *   cand_off[n+1]     CSR offsets: cand_off[0] = 0, 1 <= K_i <= 255 (else BLINK_E_LIMIT,
 *                     "question with K options; the limit is 1 to 255")
 *   n_questions       1..512 (else BLINK_E_LIMIT)
 *   vocab             1..2^31
 * Outputs (host arrays the caller allocates for the worst case, U = total):
 *   row_id[U]         the distinct ids, strictly ascending; the first *n_rows are written
 *   row_first[U+1]    the entries with id row_id[j] are row_entry[row_first[j] ..
 *                     row_first[j+1]); row_first[*n_rows] = total
 *   row_entry[total]  flat entry indices grouped by row, ascending within each row
 *   n_rows            number of distinct ids
 * Ids that repeat inside one question are allowed here (the readout's callers refuse them).
 */
int blink_pack_labels(const int32_t *cand_ids, const int32_t *cand_off, int32_t n_questions,
                      int64_t vocab, int32_t *row_id, int32_t *row_first, int32_t *row_entry,
                      int32_t *n_rows);

/*
 * blink_plan_prefix -- host, synchronous, integer only.
 *
 * Shared-prefix plan of a request ("torch engine" section: _shared_prefix_len, the switch in
 * _forward, _prefill_tokens; PREFIX_MIN_TOKENS in "constants the deployment sets"). The
 * shared length is the number of leading tokens every sequence has in common, cut so that
 * every sequence keeps at least one token of its own (its answer position is computed in the
 * per-question pass); it is 0 for a single sequence. The shared path encodes that prefix
 * once (a causal prefill: blink_prefix_tail_attention with prefix_len 0 and the prefix as the
 * one question's tail) and runs every question's remaining tail against it; it is taken only
 * when the shared length is at least min_prefix_tokens.
 *
 * Inputs (host):
 *   tokens[seq_off[n]]   every question's full token sequence, concatenated
 *   seq_off[n+1]         CSR offsets, seq_off[0] = 0; every sequence 1..131072 tokens
 *                        (else BLINK_E_INVALID / BLINK_E_LIMIT, "maximum context length")
 *   n_seqs               1..512 (else BLINK_E_LIMIT)
 *   min_prefix_tokens    >= 1 (BLINK_PREFIX_MIN_TOKENS = 256 on the pages)
 * Outputs (host scalars):
 *   shared_len           the shared length
 *   prefix_len           shared_len when the shared path is taken, else 0 (plain path)
 *   prefill_tokens       tokens the model computes: the prefix once plus every tail on the
 *                        shared path, every token of every sequence on the plain path
 */
int blink_plan_prefix(const int32_t *tokens, const int64_t *seq_off, int32_t n_seqs,
                      int32_t min_prefix_tokens, int32_t *shared_len, int32_t *prefix_len,
                      int64_t *prefill_tokens);

/*
 * blink_prefix_tail_attention -- device, asynchronous.
 *
 * Shared-prefix tail-prefill attention ("torch engine" section, _forward_shared; the
 * PREFIX_CACHE comment in "constants the deployment sets"). For question i, query head h
 * and tail position t < n_i:
 *     out[tok, h, :] = sum_j w_j v_j / sum_j w_j,  w_j = exp(scale * <q[tok,h,:], k_j> - max)
 * over the P prefix keys of KV head g = h / (H_q / H_kv) followed by the question's own tail
 * keys 0..t (tok = token_offset[i] + t). This equals plain causal attention over the full
 * sequence [prefix ; tail_i] at positions P..P+n_i-1; only the floating-point order differs.
 * Inputs are post-rotary; no positional encoding is applied. QK^T and PV use bf16 matrix cores
 * on the inputs as given; the scale multiplies the FP32 scores; softmax and accumulation are
 * FP32; out is rounded to bf16 (nearest even).
 *
 *   q        bf16 [T_pad, H_q, D]     device
 *   k_tail, v_tail  bf16 [T_pad, H_kv, D]   device
 *   k_prefix, v_prefix bf16 [P, H_kv, D]    device; may be NULL iff prefix_len == 0
 *   out      bf16 [T_pad, H_q, D]     device; rows of padding positions are not written
 *   d_token_offset  int64 [n]  device: first token of question i (from blink_pack_ragged)
 *   d_valid_start   int32 [n+1] device: exclusive prefix sum of tail lengths (question order)
 *   n_questions       1..512
 *   total_valid_tokens  must equal d_valid_start[n]; sizes the launch
 *   total_padded_tokens T_pad (>= every token_offset[i] + n_i)
 *   prefix_len        P, 0..131071
 *   n_heads_q, n_heads_kv  H_kv >= 1, H_q % H_kv == 0, H_q / H_kv <= 16
 *   head_dim          64 or 128
 *   scale             finite, > 0 (1/sqrt(D) for standard attention)
 *   workspace, workspace_bytes  optional device scratch (16-byte aligned; NULL / 0 for none),
 *                     owned by the caller, contents not preserved. When a request's query rows
 *                     need more than one round of the device's compute units and leave the
 *                     last round part-empty, the launch can split that round's units by prefix
 *                     keys (their partial sums go through the workspace and a merge pass adds
 *                     them); it does so when workspace_bytes is at least
 *                     blink_prefix_tail_attention_workspace(...) for the same sizes on the
 *                     current device, and otherwise cuts that round into smaller row units.
 *                     Either way the result is the same attention (rounding aside). Calls that
 *                     share one workspace on different streams race.
 * Without a workspace, rows of one question never depend on which other questions share the
 * launch: results are bitwise identical whether a question runs alone or packed with others.
 * With one, rows that fall in key-split units are summed in another order and agree with
 * those results up to rounding.
 */
int blink_prefix_tail_attention(const void *q, const void *k_tail, const void *v_tail,
                                const void *k_prefix, const void *v_prefix, void *out,
                                const int64_t *d_token_offset, const int32_t *d_valid_start,
                                int32_t n_questions, int64_t total_valid_tokens,
                                int64_t total_padded_tokens, int32_t prefix_len,
                                int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim,
                                float scale, void *workspace, size_t workspace_bytes,
                                void *stream);

/* Workspace bytes blink_prefix_tail_attention uses for these sizes on the current device
 * (0: its work split needs none; also 0 for sizes it would refuse). */
size_t blink_prefix_tail_attention_workspace(int64_t total_valid_tokens, int32_t n_heads_q,
                                             int32_t n_heads_kv, int32_t head_dim,
                                             int32_t prefix_len);

/*
 * blink_prefix_tail_attention_grouped -- device, asynchronous.
 *
 * Several requests, each with its own shared prefix, in one launch (the cross-request group
 * of the "public entry point" section: the questions of several requests share the forwards
 * of one call). Every question attends to its own request's prefix exactly as in
 * blink_prefix_tail_attention; results are bitwise those of one blink_prefix_tail_attention
 * call per request made without a workspace (with one, that call's key-split rows differ by
 * rounding). The requests' questions are laid out one request after another.
 *
 *   q, k_tail, v_tail, out, d_token_offset, d_valid_start: as in blink_prefix_tail_attention,
 *                     over the questions of every request (1..512 questions in total)
 *   h_valid_start[n+1]  host copy of d_valid_start (sizes the launch; must match it)
 *   n_requests        1..64 (BLINK_MAX_REQUESTS; else BLINK_E_LIMIT)
 *   h_request_first[n_requests+1]  host: first question of each request; [0] = 0,
 *                     [n_requests] = n_questions, every request at least one question
 *   h_prefix_start[n_requests]     host: first row of the request's prefix in k/v_prefix
 *   h_prefix_len[n_requests]       host: the request's prefix length P_r >= 0
 *                     (P_r + tail <= 131072 for each of its questions, else BLINK_E_LIMIT)
 *   k_prefix, v_prefix  bf16 [total_prefix_rows, H_kv, D] device: every request's prefix
 *                     K/V (requests may share rows); NULL iff total_prefix_rows == 0
 *   n_heads_q, n_heads_kv, head_dim, scale: as in blink_prefix_tail_attention
 */
int blink_prefix_tail_attention_grouped(
    const void *q, const void *k_tail, const void *v_tail, const void *k_prefix,
    const void *v_prefix, void *out, const int64_t *d_token_offset, const int32_t *d_valid_start,
    const int32_t *h_valid_start, int32_t n_questions, int64_t total_valid_tokens,
    int64_t total_padded_tokens, int32_t n_requests, const int32_t *h_request_first,
    const int64_t *h_prefix_start, const int32_t *h_prefix_len, int64_t total_prefix_rows,
    int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim, float scale, void *stream);

/*
 * blink_label_readout -- device, asynchronous.
 *
 * Label readout ("torch engine" section, _read; "answer assembly" section, softmax and
 * answer_for): for question i, h = hidden[last_row[i]] widened to FP32; for each offered
 * option k < K_i, logits[off_i + k] = sum_d W_U[cand_ids[off_i + k], d] * h[d] with FP32
 * accumulation; probs = softmax(logits / temperature) over the question's own options;
 * argmax[i] = the first option index with the largest logit.
 *
 *   hidden      bf16 [hidden_rows, d_model]  device (hidden_rows = T_pad)
 *   d_last_row  int64 [n]   device: row of each question's last real token
 *   w_u         bf16 [vocab, d_model]        device (unembedding / lm_head weight)
 *   d_cand_ids  int32 [total_candidates]     device: token id of each offered label
 *   d_cand_off  int32 [n+1] device: CSR offsets, cand_off[0] = 0, 1 <= K_i <= max_options
 *   n_questions 1..512, total_candidates = cand_off[n] (host copy, sizes checks)
 *   max_options 1..255: upper bound of every K_i
 *   d_model     multiple of 8, 8..8192
 *   temperature finite and > 0 (else BLINK_E_INVALID, "temperature is not a positive finite number")
 *   d_logits    float32 [total_candidates] device output
 *   d_probs     float32 [total_candidates] output
 *   d_argmax    int32 [n] output; -1 (with NaN logits/probs) marks a question whose
 *               table entries were out of range; -1 alone (nothing else written) a question
 *               whose offsets cannot be used (K_i outside 1..max_options, or past the table)
 *               d_probs and d_argmax are only written, never read: each may be device memory
 *               or pinned host memory the device can access (hipHostMalloc), which the host
 *               may read once the stream has been synchronised.
 * Launch form, chosen from the sizes and the current device's compute-unit count (read once
 * per device); every form gives bitwise the same results. Tables of at most 32 MiB of label
 * rows: one launch, a workgroup per question. Larger tables with n >= 2 x compute units and
 * max_options * compute units <= 9/8 * total_candidates: one launch, workgroup b taking the
 * question with the b-th most options (ties by index), so the longest start first. Otherwise
 * two launches: logits over the flat option list, then one wave per question for the softmax.
 */
int blink_label_readout(const void *hidden, int64_t hidden_rows, int32_t d_model,
                        const int64_t *d_last_row, const void *w_u, int64_t vocab,
                        const int32_t *d_cand_ids, const int32_t *d_cand_off,
                        int32_t n_questions, int64_t total_candidates, int32_t max_options,
                        float temperature, float *d_logits, float *d_probs,
                        int32_t *d_argmax, void *stream);

/*
 * blink_label_readout_batched -- device, asynchronous.
 *
 * The same readout as blink_label_readout in its batched form ("torch engine" section,
 * _read_batched): each distinct label row of the request is read from memory once and
 * scored against the hidden row of every question that offers it, instead of once per
 * offering question. Outputs, their meaning and the error behaviour are those of
 * blink_label_readout, and every logit is the same FP32 dot product accumulated in the same
 * order, so the results are bitwise those of blink_label_readout.
 *
 *   hidden, d_last_row, w_u, vocab, d_model, d_cand_off, n_questions, total_candidates,
 *   max_options, temperature, d_logits, d_probs, d_argmax: as in blink_label_readout
 *   d_row_id     int32 [n_rows]   device: distinct ids (blink_pack_labels row_id)
 *   d_row_first  int32 [n_rows+1] device: CSR offsets into d_row_entry (row_first)
 *   d_row_entry  int32 [total_candidates] device: flat entries grouped by row (row_entry)
 *   n_rows       1..total_candidates
 * The three row tables must be blink_pack_labels' output for the same option table; for
 * other contents every access still stays inside the sizes passed in, an out-of-range id
 * gives NaN logits for its entries, and entries no row lists are left with unspecified
 * results.
 */
int blink_label_readout_batched(const void *hidden, int64_t hidden_rows, int32_t d_model,
                                const int64_t *d_last_row, const void *w_u, int64_t vocab,
                                const int32_t *d_cand_off, int32_t n_questions,
                                int64_t total_candidates, int32_t max_options,
                                const int32_t *d_row_id, const int32_t *d_row_first,
                                const int32_t *d_row_entry, int32_t n_rows, float temperature,
                                float *d_logits, float *d_probs, int32_t *d_argmax,
                                void *stream);

/*
 * blink_assemble_answers -- host, synchronous.
 *
 * Typed answers from the readout's probabilities ("answer assembly" section, answer_for;
 * "rendering" section, question_options). Each question's probabilities are renormalised to
 * sum to one (a zero sum divides by one), in double precision, then by question type:
 *   BLINK_ANSWER_CHOICE  choice = the first most probable option; value = its probability;
 *                        confidence = (p_best - 1/K) / (1 - 1/K), 1 for K = 1
 *   BLINK_ANSWER_NOUL    options are (yes, no), K = 2; value = p(yes); choice = -1;
 *                        confidence = NaN (the pages give none)
 *   BLINK_ANSWER_SCORE   options are the levels 0..K-1, 2 <= K <= 10; value = sum_k k p_k;
 *                        choice = the first most probable level; confidence as for a choice,
 *                        clipped to [0, 1]
 *
 *   probs[total]      host copy of the readout's probabilities (CSR by question)
 *   cand_off[n+1]     CSR offsets (cand_off[0] = 0, 1 <= K_i <= 255)
 *   qtype[n]          BLINK_ANSWER_* of each question (else BLINK_E_INVALID; a noul question
 *                     with K != 2 or a score with K outside 2..10 is BLINK_E_INVALID)
 *   n_questions       1..512
 *   choice[n], confidence[n], value[n]   outputs (host)
 */
#define BLINK_ANSWER_CHOICE 0
#define BLINK_ANSWER_NOUL 1
#define BLINK_ANSWER_SCORE 2
int blink_assemble_answers(const float *probs, const int32_t *cand_off, const int32_t *qtype,
                           int32_t n_questions, int32_t *choice, double *confidence,
                           double *value);

/*
 * blink_score_targets -- device, asynchronous.
 *
 * Teacher-forced scoring (the simit MoT engine page: score_len and its logits consumer): for
 * scored row j, h = hidden[rows[j]]; z_v = sum_d W_U[v, d] * h[d] over the whole vocabulary
 * (bf16 products, FP32 accumulation, bf16 matrix cores); logprob[j] = z_{targets[j]} -
 * log(sum_v exp(z_v)). A sequence of n tokens scored on its last S tokens uses the rows at
 * positions n - S - 1 .. n - 2, each with the next position's token as its target.
 *
 *   hidden      bf16 [hidden_rows, d_model] device; d_model a multiple of 64, 64..16384
 *   d_rows      int64 [n_rows] device: hidden row of each scored row
 *   d_targets   int32 [n_rows] device: target token of each scored row
 *   n_rows      1..2^20
 *   w_u         bf16 [vocab, d_model] device, vocab 1..2^31
 *   d_logprob   float32 [n_rows] device output; NaN for a row whose index or target is out
 *               of range
 *   workspace   device scratch of at least blink_score_targets_workspace(n_rows, vocab)
 *               bytes, 16-byte aligned; owned by the caller, its contents are not preserved
 *               (else BLINK_E_INVALID)
 * Calls that share one workspace on different streams race.
 */
size_t blink_score_targets_workspace(int32_t n_rows, int64_t vocab); /* 0 for bad sizes */
int blink_score_targets(const void *hidden, int64_t hidden_rows, int32_t d_model,
                        const int64_t *d_rows, const int32_t *d_targets, int32_t n_rows,
                        const void *w_u, int64_t vocab, float *d_logprob, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * blink_score_targets_noalloc -- device, asynchronous; allocates nothing.
 *
 * For callers that cannot allocate device memory (code under HIP graph capture, serving loops
 * that forbid hipMalloc): blink_score_targets with the same arguments, meaning, layout, error
 * behaviour and results, minus the workspace. The scratch lives in a static device array of
 * BLINK_SCORE_SCRATCH_BYTES (16 MiB) that the library holds on every GPU it runs on until the
 * process ends; its address is looked up once per device (the first call on a device, with
 * that device current). A call needing more scratch than that, blink_score_targets_workspace
 * (n_rows, vocab) > BLINK_SCORE_SCRATCH_BYTES (at vocab 151936: more than 1766 scored
 * rows), returns BLINK_E_LIMIT before anything is launched. Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (on different streams, or from several threads
 * without ordering) race and give unspecified results. Nothing in the array needs clearing
 * between calls; each call overwrites what it reads.
 */
#define BLINK_SCORE_SCRATCH_BYTES (16u << 20)
int blink_score_targets_noalloc(const void *hidden, int64_t hidden_rows, int32_t d_model,
                                const int64_t *d_rows, const int32_t *d_targets, int32_t n_rows,
                                const void *w_u, int64_t vocab, float *d_logprob, void *stream);

/*
 * blink_combine_rotations -- host, synchronous.
 *
 * Rotation averaging of label log-probabilities (the ruling page, _score_plain): a question
 * may be read in several passes, each presenting its options in another order. For every pass
 * the label logits become log-probabilities over that pass's options (log-softmax, double
 * precision); when `prior` is given, the content-free prior's log-probability of each position
 * is subtracted; each option key's result is the mean over the passes that offered it.
 *
 *   pass_logits[sum], pass_off[n_passes+1]  each pass's logits by position (CSR)
 *   pass_question[n_passes]   the question each pass reads (0..n_questions-1)
 *   pass_key[sum]             the option key each position presents (0..K_q-1)
 *   prior[sum]                NULL, or the prior log-probability of each position
 *   key_off[n_questions+1]    CSR of the questions' option keys (1..255 each)
 *   mean_logprob[key_off[n]]  output: mean log-probability per key; NaN if no pass offered it
 * Malformed tables are BLINK_E_INVALID / BLINK_E_LIMIT, naming the pass or position.
 */
int blink_combine_rotations(const float *pass_logits, const int32_t *pass_off,
                            const int32_t *pass_question, const int32_t *pass_key,
                            const float *prior, int32_t n_passes, const int32_t *key_off,
                            int32_t n_questions, float *mean_logprob);

/*
 * blink_two_stage_finalists -- host, synchronous.
 *
 * The two-stage choice for option lists wider than one pass (the ruling page,
 * TwoStageChoice): options ranked by their stage-one score, highest first and earlier options
 * first on ties, keep their first `keep` (at least 1) as finalists. The final choice then
 * scores only the finalists; every other option gets a score of minus infinity.
 *
 *   stage_one[n_options]   1..255 scores, none NaN
 *   finalists[min(keep, n_options)]   output option indices, best first; n_finalists output
 */
int blink_two_stage_finalists(const float *stage_one, int32_t n_options, int32_t keep,
                              int32_t *finalists, int32_t *n_finalists);

#ifdef __cplusplus
}
#endif

#endif /* BLINK_H */
