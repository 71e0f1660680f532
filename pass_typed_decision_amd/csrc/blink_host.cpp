// Host half of the library: per-thread error text and the ragged right-padded packer.
//
// Packing rule (blink.py page, thegovind/blink-4b, "torch engine" section: _batches, _padded
// and the tail loop of _forward_shared): visit questions from the shortest tail to the
// longest (ties in question order); keep adding them to the open batch while the padded size
// of the batch with the newcomer, widest row times row count, stays within the budget and
// the optional row cap is not reached; otherwise open a new batch. Batch width is its
// longest row. Batches are laid end to end in one token-major buffer.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
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
    return fail(BLINK_E_LIMIT, "%d questions; supported 1-%d", n_questions, BLINK_MAX_QUESTIONS);
  if (prefix_len < 0) return fail(BLINK_E_INVALID, "prefix length must be non-negative");
  if (token_budget < 1) return fail(BLINK_E_INVALID, "token budget must be positive");
  if (max_rows < 0) return fail(BLINK_E_INVALID, "row cap must be non-negative");
  const int n = n_questions;
  for (int i = 0; i < n; ++i) {
    if (tail_len[i] < 1) return fail(BLINK_E_INVALID, "question %d has an empty tail", i);
    const int64_t total = int64_t(prefix_len) + tail_len[i];
    if (total > BLINK_MAX_INPUT_TOKENS)
      return fail(BLINK_E_LIMIT,
                  "question %d renders to %lld tokens, over the maximum context length of %d", i,
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
