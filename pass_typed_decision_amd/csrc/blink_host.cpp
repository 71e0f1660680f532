// Host half of the library: per-thread error text and the ragged right-padded packer.
//
// Packing rule (blink.py page, thegovind/blink-4b, "torch engine" section: _batches, _padded
// and the tail loop of _forward_shared): visit questions from the shortest tail to the
// longest (ties in question order); keep adding them to the open batch while the padded size
// of the batch with the newcomer, widest row times row count, stays within the budget and
// the optional row cap is not reached; otherwise open a new batch. Batch width is its
// longest row. Batches are laid end to end in one token-major buffer.
#include <hip/hip_runtime_api.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <numeric>
#include <string>
#include <vector>

#include "blink_internal.h"

namespace blink {

static thread_local std::string g_error;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error.assign(buf);
  return code;
}

int ok() {
  g_error.clear();
  return BLINK_OK;
}

int device_cus(int &cus, const char *who) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> known[kMaxDevices] = {};
  int device = -1;
  cus = 0;
  if (hipGetDevice(&device) != hipSuccess || device < 0)
    return fail(BLINK_E_DEVICE, "%s: no device", who);
  if (device < kMaxDevices) cus = known[device].load(std::memory_order_relaxed);
  if (cus > 0) return BLINK_OK;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
      cus < 1)
    return fail(BLINK_E_DEVICE, "%s: no device", who);
  if (device < kMaxDevices) known[device].store(cus, std::memory_order_relaxed);
  return BLINK_OK;
}

}  // namespace blink

extern "C" const char *blink_last_error(void) { return blink::g_error.c_str(); }

extern "C" int blink_abi_version(void) { return BLINK_ABI_VERSION; }

extern "C" int blink_pack_ragged(const int32_t *tail_len, int32_t n_questions, int32_t prefix_len,
                                 int64_t token_budget, int32_t max_rows, int32_t *order,
                                 int32_t *batch_of, int32_t *row_of, int64_t *token_offset,
                                 int64_t *last_row, int32_t *valid_start, int32_t *batch_first,
                                 int32_t *batch_width, int64_t *batch_base, int32_t *n_batches,
                                 int64_t *total_padded_tokens, int64_t *total_valid_tokens) {
  using blink::fail;
  if (!tail_len || !order || !batch_of || !row_of || !token_offset || !last_row ||
      !valid_start || !batch_first || !batch_width || !batch_base || !n_batches ||
      !total_padded_tokens || !total_valid_tokens)
    return fail(BLINK_E_INVALID, "blink_pack_ragged: a pointer argument is NULL");
  if (n_questions < 1 || n_questions > BLINK_MAX_QUESTIONS)
    return fail(BLINK_E_LIMIT, "request of %d questions; the limit is 1 to %d", n_questions, BLINK_MAX_QUESTIONS);
  if (prefix_len < 0) return fail(BLINK_E_INVALID, "prefix length must be non-negative");
  if (token_budget < 1) return fail(BLINK_E_INVALID, "token budget is below 1");
  if (max_rows < 0) return fail(BLINK_E_INVALID, "row cap must be non-negative");
  const int n = n_questions;
  for (int i = 0; i < n; ++i) {
    if (tail_len[i] < 1) return fail(BLINK_E_INVALID, "question %d has an empty tail", i);
    const int64_t total = int64_t(prefix_len) + tail_len[i];
    if (total > BLINK_MAX_INPUT_TOKENS)
      return fail(BLINK_E_LIMIT,
                  "question %d needs %lld tokens of context; the maximum context length is %d", i,
                  (long long)total, BLINK_MAX_INPUT_TOKENS);
  }

  // Visiting order: a stable sort by length keeps equal lengths in question order.
  std::vector<int32_t> walk(n);
  std::iota(walk.begin(), walk.end(), 0);
  std::stable_sort(walk.begin(), walk.end(),
                   [&](int32_t a, int32_t b) { return tail_len[a] < tail_len[b]; });

  // Cut the walk into batches: [cut[b], cut[b+1]).
  std::vector<int32_t> cut{0};
  int64_t widest = tail_len[walk[0]];
  for (int k = 1; k < n; ++k) {
    const int64_t rows = k - cut.back();
    const int64_t grown = std::max<int64_t>(widest, tail_len[walk[k]]);
    const bool over_budget = grown * (rows + 1) > token_budget;
    const bool at_cap = max_rows > 0 && rows >= max_rows;
    if (over_budget || at_cap) {
      cut.push_back(k);
      widest = tail_len[walk[k]];
    } else {
      widest = grown;
    }
  }
  cut.push_back(n);

  const int nb = int(cut.size()) - 1;
  int64_t base = 0;
  for (int b = 0; b < nb; ++b) {
    int32_t width = 0;
    for (int k = cut[b]; k < cut[b + 1]; ++k) width = std::max(width, tail_len[walk[k]]);
    batch_first[b] = cut[b];
    batch_width[b] = width;
    batch_base[b] = base;
    for (int k = cut[b]; k < cut[b + 1]; ++k) {
      const int32_t q = walk[k];
      const int32_t r = k - cut[b];
      order[k] = q;
      batch_of[q] = b;
      row_of[q] = r;
      token_offset[q] = base + int64_t(r) * width;
      last_row[q] = token_offset[q] + tail_len[q] - 1;
    }
    base += int64_t(cut[b + 1] - cut[b]) * width;
  }
  batch_first[nb] = n;
  batch_base[nb] = base;
  int64_t running = 0;
  for (int i = 0; i < n; ++i) {
    valid_start[i] = int32_t(running);
    running += tail_len[i];
  }
  valid_start[n] = int32_t(running);
  *n_batches = nb;
  *total_padded_tokens = base;
  *total_valid_tokens = running;
  return blink::ok();
}

// Distinct label rows of an option table (blink.py page, "torch engine" section,
// _read_batched: the distinct label ids of the questions, ascending, each gathered once).
// One bit per vocabulary id marks the ids in use; a scan of the bit words lists them in
// ascending order and gives each id its column; a stable counting sort by column then
// groups the flat option entries under their row, in ascending entry order.
extern "C" int blink_pack_labels(const int32_t *cand_ids, const int32_t *cand_off,
                                 int32_t n_questions, int64_t vocab, int32_t *row_id,
                                 int32_t *row_first, int32_t *row_entry, int32_t *n_rows) {
  using blink::fail;
  if (!cand_ids || !cand_off || !row_id || !row_first || !row_entry || !n_rows)
    return fail(BLINK_E_INVALID, "blink_pack_labels: a pointer argument is NULL");
  if (n_questions < 1 || n_questions > BLINK_MAX_QUESTIONS)
    return fail(BLINK_E_LIMIT, "request of %d questions; the limit is 1 to %d", n_questions, BLINK_MAX_QUESTIONS);
  if (vocab < 1 || vocab > (int64_t(1) << 31))
    return fail(BLINK_E_INVALID, "vocab %lld outside 1..2^31", (long long)vocab);
  if (cand_off[0] != 0) return fail(BLINK_E_INVALID, "candidate offsets must start at 0");
  for (int i = 0; i < n_questions; ++i) {
    const int64_t k = int64_t(cand_off[i + 1]) - cand_off[i];
    if (k < 1 || k > BLINK_MAX_OPTIONS)
      return fail(BLINK_E_LIMIT, "question with %lld options; the limit is 1 to %d", (long long)k,
                  BLINK_MAX_OPTIONS);
  }
  const int32_t total = cand_off[n_questions];
  for (int32_t e = 0; e < total; ++e)
    if (cand_ids[e] < 0 || cand_ids[e] >= vocab)
      return fail(BLINK_E_INVALID, "option entry %d has token id %d outside [0, %lld)", e,
                  cand_ids[e], (long long)vocab);

  // Work arrays of this call (the library keeps nothing between calls): a bitmap of the
  // vocabulary and per-entry columns, tens of KB at a 151936-row vocabulary.
  const size_t words = size_t((vocab + 63) >> 6);
  std::vector<uint64_t> bits_v(words, 0);
  std::vector<int32_t> word_base_v(words), col_v(static_cast<size_t>(total));
  uint64_t *bits = bits_v.data();
  int32_t *word_base = word_base_v.data();
  int32_t *col = col_v.data();
  for (int32_t e = 0; e < total; ++e) {
    const uint32_t t = uint32_t(cand_ids[e]);
    bits[t >> 6] |= uint64_t(1) << (t & 63);
  }
  int32_t u = 0;
  for (size_t w = 0; w < words; ++w) {
    word_base[w] = u;
    for (uint64_t m = bits[w]; m; m &= m - 1)
      row_id[u++] = int32_t(w * 64 + size_t(__builtin_ctzll(m)));
  }
  std::vector<int32_t> cursor_v(size_t(u) + 1, 0);
  int32_t *cursor = cursor_v.data();
  for (int32_t e = 0; e < total; ++e) {
    const uint32_t t = uint32_t(cand_ids[e]);
    const uint64_t below = bits[t >> 6] & ((uint64_t(1) << (t & 63)) - 1);
    col[e] = word_base[t >> 6] + __builtin_popcountll(below);
    ++cursor[col[e] + 1];
  }
  for (int32_t j = 0; j < u; ++j) cursor[j + 1] += cursor[j];
  for (int32_t j = 0; j <= u; ++j) row_first[j] = cursor[j];
  for (int32_t e = 0; e < total; ++e) row_entry[cursor[col[e]]++] = e;
  *n_rows = u;
  return blink::ok();
}

// Shared-prefix plan of a request (blink.py page, "torch engine" section: _shared_prefix_len,
// _forward's switch to the shared path, _prefill_tokens). The shared length is found by
// walking token positions while every sequence agrees with the first one, and is cut so
// that every sequence keeps at least one token of its own.
extern "C" int blink_plan_prefix(const int32_t *tokens, const int64_t *seq_off, int32_t n_seqs,
                                 int32_t min_prefix_tokens, int32_t *shared_len,
                                 int32_t *prefix_len, int64_t *prefill_tokens) {
  using blink::fail;
  if (!tokens || !seq_off || !shared_len || !prefix_len || !prefill_tokens)
    return fail(BLINK_E_INVALID, "blink_plan_prefix: a pointer argument is NULL");
  if (n_seqs < 1 || n_seqs > BLINK_MAX_QUESTIONS)
    return fail(BLINK_E_LIMIT, "request of %d questions; the limit is 1 to %d", n_seqs, BLINK_MAX_QUESTIONS);
  if (min_prefix_tokens < 1)
    return fail(BLINK_E_INVALID, "the minimum shared prefix must be at least 1");
  if (seq_off[0] != 0) return fail(BLINK_E_INVALID, "sequence offsets must start at 0");
  int64_t shortest = INT64_MAX, total = 0;
  for (int i = 0; i < n_seqs; ++i) {
    const int64_t len = seq_off[i + 1] - seq_off[i];
    if (len < 1) return fail(BLINK_E_INVALID, "sequence %d needs at least one token", i);
    if (len > BLINK_MAX_INPUT_TOKENS)
      return fail(BLINK_E_LIMIT,
                  "question %d needs %lld tokens of context; the maximum context length is %d", i,
                  (long long)len, BLINK_MAX_INPUT_TOKENS);
    shortest = std::min(shortest, len);
    total += len;
  }
  int64_t p = 0;
  if (n_seqs >= 2) {
    const int32_t *first = tokens + seq_off[0];
    // Position by position; stop at the first mismatch or at the shortest sequence's last
    // token, which stays its own.
    for (bool same = true; same && p < shortest - 1; p += same) {
      const int32_t t = first[p];
      for (int i = 1; i < n_seqs && same; ++i) same = tokens[seq_off[i] + p] == t;
    }
  }
  *shared_len = int32_t(p);
  const bool use = p > 0 && p >= min_prefix_tokens;
  *prefix_len = use ? int32_t(p) : 0;
  *prefill_tokens = use ? total - int64_t(n_seqs - 1) * p : total;
  return blink::ok();
}

// Typed answers from one request's option probabilities (blink.py page, "answer assembly"
// section, answer_for): renormalise each question's probabilities (a zero sum divides by
// one), then a choice takes its first most probable option and the confidence
// (p_best - 1/K) / (1 - 1/K) (1 for a single option); a noul question (options yes, no)
// gives the probability of yes; a score question (levels 0..K-1, 2 <= K <= 10) gives the
// expected level, its first most probable level and the same confidence clipped to [0, 1].
extern "C" int blink_assemble_answers(const float *probs, const int32_t *cand_off,
                                      const int32_t *qtype, int32_t n_questions,
                                      int32_t *choice, double *confidence, double *value) {
  using blink::fail;
  if (!probs || !cand_off || !qtype || !choice || !confidence || !value)
    return fail(BLINK_E_INVALID, "blink_assemble_answers: a pointer argument is NULL");
  if (n_questions < 1 || n_questions > BLINK_MAX_QUESTIONS)
    return fail(BLINK_E_LIMIT, "request of %d questions; the limit is 1 to %d", n_questions, BLINK_MAX_QUESTIONS);
  if (cand_off[0] != 0) return fail(BLINK_E_INVALID, "candidate offsets must start at 0");
  for (int i = 0; i < n_questions; ++i) {
    const int64_t k = int64_t(cand_off[i + 1]) - cand_off[i];
    if (k < 1 || k > BLINK_MAX_OPTIONS)
      return fail(BLINK_E_LIMIT, "question with %lld options; the limit is 1 to %d", (long long)k,
                  BLINK_MAX_OPTIONS);
    if (qtype[i] == BLINK_ANSWER_NOUL && k != 2)
      return fail(BLINK_E_INVALID, "question %d: a noul question offers exactly yes and no", i);
    if (qtype[i] == BLINK_ANSWER_SCORE && (k < 2 || k > 10))
      return fail(BLINK_E_INVALID, "question %d: a score takes 2 to 10 levels", i);
    if (qtype[i] != BLINK_ANSWER_CHOICE && qtype[i] != BLINK_ANSWER_NOUL &&
        qtype[i] != BLINK_ANSWER_SCORE)
      return fail(BLINK_E_INVALID, "question %d: unknown question type %d", i, qtype[i]);
  }
  for (int i = 0; i < n_questions; ++i) {
    const float *p = probs + cand_off[i];
    const int k = cand_off[i + 1] - cand_off[i];
    double z = 0.0;
    for (int j = 0; j < k; ++j) z += double(p[j]);
    if (z == 0.0) z = 1.0;
    int best = 0;
    for (int j = 1; j < k; ++j)
      if (double(p[j]) / z > double(p[best]) / z) best = j;
    const double pb = double(p[best]) / z;
    const double conf = k > 1 ? (pb - 1.0 / k) / (1.0 - 1.0 / k) : 1.0;
    if (qtype[i] == BLINK_ANSWER_CHOICE) {
      choice[i] = best;
      confidence[i] = conf;
      value[i] = pb;
    } else if (qtype[i] == BLINK_ANSWER_NOUL) {
      choice[i] = -1;
      confidence[i] = NAN;
      value[i] = double(p[0]) / z;
    } else {
      double ev = 0.0;
      for (int j = 0; j < k; ++j) ev += j * (double(p[j]) / z);
      choice[i] = best;
      confidence[i] = std::min(1.0, std::max(0.0, conf));
      value[i] = ev;
    }
  }
  return blink::ok();
}

// Rotation averaging (ruling page, _score_plain): each pass's label logits become
// log-probabilities over the pass's own options (log-softmax, in double); a prior's
// log-probabilities for the same positions are subtracted when given; every option key's
// result is the mean over the passes that offered it (NaN if none did).
extern "C" int blink_combine_rotations(const float *pass_logits, const int32_t *pass_off,
                                       const int32_t *pass_question, const int32_t *pass_key,
                                       const float *prior, int32_t n_passes,
                                       const int32_t *key_off, int32_t n_questions,
                                       float *mean_logprob) {
  using blink::fail;
  if (!pass_logits || !pass_off || !pass_question || !pass_key || !key_off || !mean_logprob)
    return fail(BLINK_E_INVALID, "blink_combine_rotations: a pointer argument is NULL");
  if (n_passes < 1 || n_questions < 1 || n_questions > BLINK_MAX_QUESTIONS)
    return fail(BLINK_E_LIMIT, "%d passes over %d questions; need 1 or more passes and 1-%d "
                "questions", n_passes, n_questions, BLINK_MAX_QUESTIONS);
  if (pass_off[0] != 0 || key_off[0] != 0)
    return fail(BLINK_E_INVALID, "offsets must start at 0");
  for (int q = 0; q < n_questions; ++q)
    if (key_off[q + 1] - key_off[q] < 1 || key_off[q + 1] - key_off[q] > BLINK_MAX_OPTIONS)
      return fail(BLINK_E_LIMIT, "question with %d options; the limit is 1 to %d",
                  key_off[q + 1] - key_off[q], BLINK_MAX_OPTIONS);
  for (int p = 0; p < n_passes; ++p) {
    const int q = pass_question[p];
    const int k = pass_off[p + 1] - pass_off[p];
    if (q < 0 || q >= n_questions)
      return fail(BLINK_E_INVALID, "pass %d names question %d of %d", p, q, n_questions);
    if (k < 1 || k > key_off[q + 1] - key_off[q])
      return fail(BLINK_E_INVALID, "pass %d offers %d options; its question has %d", p, k,
                  key_off[q + 1] - key_off[q]);
    for (int i = pass_off[p]; i < pass_off[p + 1]; ++i)
      if (pass_key[i] < 0 || pass_key[i] >= key_off[q + 1] - key_off[q])
        return fail(BLINK_E_INVALID, "pass %d position %d names key %d", p, i - pass_off[p],
                    pass_key[i]);
  }
  const int total = key_off[n_questions];
  std::vector<double> sum(size_t(total), 0.0);
  std::vector<int32_t> count(size_t(total), 0);
  for (int p = 0; p < n_passes; ++p) {
    const int lo = pass_off[p], hi = pass_off[p + 1];
    double m = -INFINITY;
    for (int i = lo; i < hi; ++i) m = std::max(m, double(pass_logits[i]));
    double s = 0.0;
    for (int i = lo; i < hi; ++i) s += std::exp(double(pass_logits[i]) - m);
    const double lse = m + std::log(s);
    const int base = key_off[pass_question[p]];
    for (int i = lo; i < hi; ++i) {
      double v = double(pass_logits[i]) - lse;
      if (prior) v -= double(prior[i]);
      sum[size_t(base + pass_key[i])] += v;
      ++count[size_t(base + pass_key[i])];
    }
  }
  for (int j = 0; j < total; ++j)
    mean_logprob[j] = count[size_t(j)] ? float(sum[size_t(j)] / count[size_t(j)]) : NAN;
  return blink::ok();
}

// Two-stage choice (ruling page, TwoStageChoice): the options ranked by their stage-one score,
// highest first and earlier options first on ties, keep their first `keep` as finalists.
extern "C" int blink_two_stage_finalists(const float *stage_one, int32_t n_options,
                                         int32_t keep, int32_t *finalists,
                                         int32_t *n_finalists) {
  using blink::fail;
  if (!stage_one || !finalists || !n_finalists)
    return fail(BLINK_E_INVALID, "blink_two_stage_finalists: a pointer argument is NULL");
  if (n_options < 1 || n_options > BLINK_MAX_OPTIONS)
    return fail(BLINK_E_LIMIT, "question with %d options; the limit is 1 to %d", n_options,
                BLINK_MAX_OPTIONS);
  if (keep < 1) return fail(BLINK_E_INVALID, "keep must be at least 1");
  for (int i = 0; i < n_options; ++i)
    if (std::isnan(stage_one[i])) return fail(BLINK_E_INVALID, "stage-one score %d is NaN", i);
  std::vector<int32_t> order(static_cast<size_t>(n_options));
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b) { return stage_one[a] > stage_one[b]; });
  const int k = std::min(keep, n_options);
  for (int i = 0; i < k; ++i) finalists[i] = order[size_t(i)];
  *n_finalists = k;
  return blink::ok();
}
