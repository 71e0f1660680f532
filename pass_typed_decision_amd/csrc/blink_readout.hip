// Label readout on gfx950: gather each question's last real hidden row, score its offered
// labels against their unembedding rows in FP32, temperature softmax, first-index argmax.
//
// Method: blink.py page (thegovind/blink-4b), "torch engine" section, _read (per-question
// gather, FP32 upcast of the hidden row and of the label rows, FP32 matrix-vector product),
// and "answer assembly" section, softmax (divide by the temperature, subtract the maximum,
// exponentiate, normalise) and answer_for (most probable option, earlier option on ties).
//
// Design. Large option tables (bandwidth-bound) whose questions are too few, or too uneven,
// to balance the compute units one question per workgroup take two launches on the caller's
// stream:
//  * label_logits_flat_kernel streams the label rows: the options of all questions form one
//    flat list (the CSR order of cand_ids) and every wave scores one entry of it, so the work
//    is spread evenly whatever the mix of option counts (1..255 per question). A wave loads
//    its label row with 16-byte coalesced loads (a 2560-wide bf16 row is five 1 KiB wave
//    loads) while the workgroup stages the question offsets in LDS; a binary search there
//    names the question, whose hidden row (shared by many waves, so an L2 hit) then gives the
//    FP32 dot product (v_dot2: bf16 pairs, FP32 accumulate), reduced across the wave. Blocks
//    are mapped so that each XCD (dispatch is round-robin over the 8 XCDs) takes one
//    contiguous slice of the list. The kernel is bound by HBM bandwidth on the label rows.
//  * label_softmax_kernel: one wave per question over its (at most 255) logits: temperature,
//    max, exp, sum, normalise, and the first index of the largest logit.
// Small tables (launch-latency-bound) take one launch, label_readout_fused_kernel: one
// workgroup per question scores its rows and finishes it in the same kernel. Large tables of
// many questions take that kernel in its ranked form instead of the pair: workgroup b takes
// the question with the b-th most options (every workgroup derives the same order from the
// offsets), so the longest questions start first and the short ones fill in behind them, and
// each question's probabilities are written while other workgroups still stream rows.
// The batched form (blink_label_readout_batched, after _read_batched) replaces the first
// launch of the streaming path with label_logits_rows_kernel, which reads each distinct label
// row once however many questions offer it.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "blink_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxChunksPerLane = 16;  // d_model <= 16 * 64 * 8 = 8192
constexpr int kXcds = 8;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

constexpr int kFlatWaves = 16;

// Question owning flat entry r: the last i in [0, n) with off[i] <= r (off staged in LDS).
__device__ inline int owner_of(const int32_t *s_off, int n, int64_t r) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (int64_t(s_off[mid]) <= r)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

template <int NCH>
__global__ __launch_bounds__(64 * kFlatWaves) void label_logits_flat_kernel(
    const uint16_t *__restrict__ hidden, int64_t hidden_rows, int d_model,
    const int64_t *__restrict__ last_row, const uint16_t *__restrict__ w_u, int64_t vocab,
    const int32_t *__restrict__ cand_ids, const int32_t *__restrict__ cand_off, int n,
    int64_t total, int64_t n_blocks, float *__restrict__ logits) {
  __shared__ int32_t s_off[BLINK_MAX_QUESTIONS + 1];
  const int lane = threadIdx.x & 63;
  const int wave = uniform(int(threadIdx.x >> 6));
  const int64_t per = (n_blocks + kXcds - 1) / kXcds;
  const int64_t blk = int64_t(blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (blk >= n_blocks) return;
  const int64_t r = blk * kFlatWaves + wave;
  const bool live = r < total;
  const int32_t id = live ? cand_ids[r] : 0;  // scalar: uniform address
  for (int i = threadIdx.x; i <= n; i += 64 * kFlatWaves) s_off[i] = cand_off[i];
  const bool id_ok = id >= 0 && id < vocab;
  const uint16_t *wrow = w_u + int64_t(id_ok ? id : 0) * d_model;
  const int nchunks = d_model >> 3;
  u32x4 w[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ch = lane + 64 * c;
    w[c] = u32x4{0u, 0u, 0u, 0u};
    if (live && ch < nchunks) w[c] = *reinterpret_cast<const u32x4 *>(wrow + ch * 8);
  }
  __syncthreads();
  if (!live) return;
  const int q = uniform(owner_of(s_off, n, r));
  const int64_t row = last_row[q];
  const bool h_ok = row >= 0 && row < hidden_rows;
  const uint16_t *hrow = hidden + (h_ok ? row : 0) * int64_t(d_model);
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ch = lane + 64 * c;
    u32x4 h = u32x4{0u, 0u, 0u, 0u};
    if (ch < nchunks) h = *reinterpret_cast<const u32x4 *>(hrow + ch * 8);
#pragma unroll
    for (int m = 0; m < 4; ++m) acc = dot2(w[c][m], h[m], acc);
  }
  const float z = wave_sum(acc);
  if (lane == 0) logits[r] = (id_ok && h_ok) ? z : __builtin_nanf("");
}

// Batched form (blink.py page, "torch engine" section, _read_batched): every distinct label
// row of the request is fetched from HBM once and scored against the hidden row of each
// question that offers it. One wave per distinct row j: its unembedding row row_id[j] is
// loaded once (a streaming load: nothing reads it again), then for every flat option entry
// e in row_entry[row_first[j] .. row_first[j+1]) the owning question's hidden row (an L2 hit)
// gives logits[e]. Blocks map to XCDs as in label_logits_flat_kernel.
template <int NCH>
__global__ __launch_bounds__(64 * kFlatWaves) void label_logits_rows_kernel(
    const uint16_t *__restrict__ hidden, int64_t hidden_rows, int d_model,
    const int64_t *__restrict__ last_row, const uint16_t *__restrict__ w_u, int64_t vocab,
    const int32_t *__restrict__ cand_off, int n, int64_t total,
    const int32_t *__restrict__ row_id, const int32_t *__restrict__ row_first,
    const int32_t *__restrict__ row_entry, int64_t n_rows, int64_t n_blocks,
    float *__restrict__ logits) {
  __shared__ int32_t s_off[BLINK_MAX_QUESTIONS + 1];
  const int lane = threadIdx.x & 63;
  const int wave = uniform(int(threadIdx.x >> 6));
  const int64_t per = (n_blocks + kXcds - 1) / kXcds;
  const int64_t blk = int64_t(blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (blk >= n_blocks) return;
  const int64_t j = blk * kFlatWaves + wave;
  const bool live = j < n_rows;
  const int32_t id = live ? row_id[j] : 0;  // scalar: uniform address
  for (int i = threadIdx.x; i <= n; i += 64 * kFlatWaves) s_off[i] = cand_off[i];
  const bool id_ok = id >= 0 && id < vocab;
  const uint16_t *wrow = w_u + int64_t(id_ok ? id : 0) * d_model;
  const int nchunks = d_model >> 3;
  u32x4 w[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ch = lane + 64 * c;
    w[c] = u32x4{0u, 0u, 0u, 0u};
    if (live && ch < nchunks)
      w[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wrow + ch * 8));
  }
  int64_t lo = live ? row_first[j] : 0, hi = live ? row_first[j + 1] : 0;
  if (lo < 0 || hi > total || hi < lo) lo = hi = 0;  // malformed: the row's entries stay unwritten
  __syncthreads();
  for (int64_t k = lo; k < hi; ++k) {
    const int32_t e = row_entry[k];
    if (e < 0 || e >= total) continue;
    const int q = uniform(owner_of(s_off, n, e));
    const int64_t row = last_row[q];
    const bool h_ok = row >= 0 && row < hidden_rows;
    const uint16_t *hrow = hidden + (h_ok ? row : 0) * int64_t(d_model);
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = lane + 64 * c;
      u32x4 h = u32x4{0u, 0u, 0u, 0u};
      if (ch < nchunks) h = *reinterpret_cast<const u32x4 *>(hrow + ch * 8);
#pragma unroll
      for (int m = 0; m < 4; ++m) acc = dot2(w[c][m], h[m], acc);
    }
    const float z = wave_sum(acc);
    if (lane == 0) logits[e] = (id_ok && h_ok) ? z : __builtin_nanf("");
  }
}

// One wave finishes question i from its K logits (lane holds options lane + 64 j): softmax of
// the logits divided by the temperature and the first index of the largest logit. A NaN logit
// (an id or a hidden row out of range) makes the question's logits and probabilities NaN and
// its argmax -1. Logits are written only when `write_logits` (they may already be in place).
__device__ inline void finish_question(const float (&z)[4], int K, int lane, float temperature,
                                       int64_t lo, bool write_logits, float *__restrict__ logits,
                                       float *__restrict__ probs, int32_t *__restrict__ argmax_i) {
  float zt[4], best = -INFINITY, mt = -INFINITY;
  int best_k = K;
  bool bad = false;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int k = lane + 64 * j;
    zt[j] = -INFINITY;
    if (k < K) {
      bad |= isnan(z[j]);
      zt[j] = z[j] / temperature;
      mt = fmaxf(mt, zt[j]);
      if (z[j] > best) {  // strict: the earliest k of this lane wins ties
        best = z[j];
        best_k = k;
      }
    }
  }
  if (__builtin_amdgcn_ballot_w64(bad)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = lane + 64 * j;
      if (k < K) {
        logits[lo + k] = __builtin_nanf("");
        probs[lo + k] = __builtin_nanf("");
      }
    }
    if (lane == 0) *argmax_i = -1;
    return;
  }
  mt = wave_max(mt);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ob = __shfl_xor(best, o);
    const int ok = __shfl_xor(best_k, o);
    if (ob > best || (ob == best && ok < best_k)) {
      best = ob;
      best_k = ok;
    }
  }
  float e[4], part = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    e[j] = (lane + 64 * j < K) ? expf(zt[j] - mt) : 0.f;
    part += e[j];
  }
  const float sum = wave_sum(part);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int k = lane + 64 * j;
    if (k < K) {
      if (write_logits) logits[lo + k] = z[j];
      probs[lo + k] = e[j] / sum;
    }
  }
  if (lane == 0) *argmax_i = best_k;
}

__device__ inline bool offsets_usable(int64_t lo, int64_t hi, int64_t total, int max_options) {
  return lo >= 0 && hi <= total && hi - lo >= 1 && hi - lo <= max_options;
}

// Second launch of the streaming path: one wave per question over the logits just written.
// Unusable offsets: argmax -1 and nothing else written.
__global__ __launch_bounds__(kThreads) void label_softmax_kernel(
    const int32_t *__restrict__ cand_off, int n, int64_t total, int max_options,
    float temperature, float *__restrict__ logits, float *__restrict__ probs,
    int32_t *__restrict__ argmax) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * kWaves + uniform(int(threadIdx.x >> 6));
  if (i >= n) return;
  const int64_t lo = cand_off[i], hi = cand_off[i + 1];
  if (!offsets_usable(lo, hi, total, max_options)) {
    if (lane == 0) argmax[i] = -1;
    return;
  }
  const int K = int(hi - lo);
  float z[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) z[j] = (lane + 64 * j < K) ? logits[lo + lane + 64 * j] : 0.f;
  finish_question(z, K, lane, temperature, lo, false, logits, probs, argmax + i);
}

// The question of rank b (0-based) when questions are ordered by decreasing option count,
// ties by index (questions with unusable offsets count as 0 options and come last). Every
// workgroup of the grid computes the same permutation from cand_off, so with one workgroup per
// rank each question is taken exactly once. One pass over the n <= BLINK_MAX_QUESTIONS
// questions, one per thread: an LDS histogram of the option counts, a suffix scan of it by
// wave 0 that names the count K* holding rank b and b's place r among the questions with K*
// options, then a ballot prefix count over those questions in index order that finds the one
// at place r. The winning thread also hands over its offsets and hidden row, which saves the
// workgroup a dependent round trip to memory. Returns i = -1 if no question holds rank b,
// which only offsets rewritten during the launch can cause.
struct Ranked {
  int i;
  int64_t lo, hi, row;
};

template <int W>
__device__ inline Ranked ranked_question(const int32_t *__restrict__ cand_off,
                                         const int64_t *__restrict__ last_row, int n,
                                         int64_t total, int max_options, int b) {
  static_assert(64 * W >= BLINK_MAX_QUESTIONS, "one question per thread");
  constexpr int kBins = BLINK_MAX_OPTIONS + 1;
  static_assert(kBins == 256, "wave 0 scans four bins per lane");
  __shared__ int s_hist[kBins];
  __shared__ int s_wave[W];
  __shared__ int s_pick[2];
  __shared__ Ranked s_won;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  int key = -1;
  int64_t lo = 0, hi = 0, row = 0;
  if (t < n) {
    lo = cand_off[t];
    hi = cand_off[t + 1];
    row = last_row[t];
    key = offsets_usable(lo, hi, total, max_options) ? int(hi - lo) : 0;
  }
  for (int k = t; k < kBins; k += 64 * W) s_hist[k] = 0;
  if (t == 0) {  // stay "none" only if cand_off changed under the launch
    s_pick[0] = -1;
    s_won.i = -1;
  }
  __syncthreads();
  if (key >= 0) atomicAdd(&s_hist[key], 1);
  __syncthreads();
  if (wave == 0) {
    // Lane l holds bins 4l..4l+3; `above` counts the questions in bins of higher lanes.
    int h[4], sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) sum += h[j] = s_hist[4 * lane + j];
    int incl = sum;  // inclusive prefix over lanes 0..l
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    int above = __shfl(incl, 63) - incl;
#pragma unroll
    for (int j = 3; j >= 0; --j) {
      if (b >= above && b < above + h[j]) {
        s_pick[0] = 4 * lane + j;
        s_pick[1] = b - above;
      }
      above += h[j];
    }
  }
  __syncthreads();
  const int want = s_pick[0], place = s_pick[1];
  const bool mine = key >= 0 && key == want;
  const uint64_t mask = __builtin_amdgcn_ballot_w64(mine);
  const int below = __builtin_popcountll(mask & ((uint64_t(1) << lane) - 1));
  if (lane == 0) s_wave[wave] = __builtin_popcountll(mask);
  __syncthreads();
  int before = below;
  for (int w = 0; w < wave; ++w) before += s_wave[w];
  if (mine && before == place) s_won = Ranked{t, lo, hi, row};
  __syncthreads();
  return s_won;
}

// One workgroup of W waves per question: its waves take the question's label rows two at a
// time, wave 0 finishes. RANKED = false: workgroup b takes question b (small option tables,
// where launch latency, not bandwidth, bounds the readout). RANKED = true: workgroup b takes
// the question of rank b by decreasing option count, so the dispatcher hands out the longest
// questions first and the short ones fill in behind them (longest-processing-time-first
// scheduling), which balances the compute units without splitting a question; used for large
// tables whose questions outnumber the compute units. The probabilities' writes then overlap
// other workgroups' row streams instead of waiting for a second launch.
template <int NCH, int W, bool RANKED>
__global__ __launch_bounds__(64 * W) void label_readout_fused_kernel(
    const uint16_t *__restrict__ hidden, int64_t hidden_rows, int d_model,
    const int64_t *__restrict__ last_row, const uint16_t *__restrict__ w_u, int64_t vocab,
    const int32_t *__restrict__ cand_ids, const int32_t *__restrict__ cand_off, int n,
    int64_t total, int max_options, float temperature, float *__restrict__ logits,
    float *__restrict__ probs, int32_t *__restrict__ argmax) {
  __shared__ float s_z[BLINK_MAX_OPTIONS + 1];
  const int lane = threadIdx.x & 63;
  const int wave = uniform(int(threadIdx.x >> 6));
  int i;
  int64_t lo, hi, row;
  if constexpr (RANKED) {
    const Ranked r = ranked_question<W>(cand_off, last_row, n, total, max_options, blockIdx.x);
    if (r.i < 0) return;  // uniform: read from LDS
    i = r.i;
    lo = r.lo;
    hi = r.hi;
    row = r.row;
  } else {
    i = blockIdx.x;
    lo = cand_off[i];
    hi = cand_off[i + 1];
    row = last_row[i];
  }
  if (!offsets_usable(lo, hi, total, max_options)) {  // uniform across the workgroup
    if (threadIdx.x == 0) argmax[i] = -1;
    return;
  }
  const int K = int(hi - lo);
  const bool h_ok = row >= 0 && row < hidden_rows;
  const uint16_t *hrow = hidden + (h_ok ? row : 0) * int64_t(d_model);
  const int nchunks = d_model >> 3;
  u32x4 h[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ch = lane + 64 * c;
    h[c] = u32x4{0u, 0u, 0u, 0u};
    if (ch < nchunks) h[c] = *reinterpret_cast<const u32x4 *>(hrow + ch * 8);
  }
  for (int k = wave; k < K; k += 2 * W) {  // rows k and k + W
    const int k2 = k + W;
    const bool two = k2 < K;
    const int32_t id1 = cand_ids[lo + k];
    const int32_t id2 = two ? cand_ids[lo + k2] : 0;
    const bool ok1 = id1 >= 0 && id1 < vocab, ok2 = id2 >= 0 && id2 < vocab;
    const uint16_t *r1 = w_u + int64_t(ok1 ? id1 : 0) * d_model;
    const uint16_t *r2 = w_u + int64_t(ok2 ? id2 : 0) * d_model;
    u32x4 w1[NCH], w2[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = lane + 64 * c;
      w1[c] = u32x4{0u, 0u, 0u, 0u};
      w2[c] = u32x4{0u, 0u, 0u, 0u};
      if (ch < nchunks) {
        w1[c] = *reinterpret_cast<const u32x4 *>(r1 + ch * 8);
        if (two) w2[c] = *reinterpret_cast<const u32x4 *>(r2 + ch * 8);
      }
    }
    float acc1 = 0.f, acc2 = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        acc1 = dot2(w1[c][m], h[c][m], acc1);
        acc2 = dot2(w2[c][m], h[c][m], acc2);
      }
    const float z1 = wave_sum(acc1), z2 = wave_sum(acc2);
    if (lane == 0) {
      s_z[k] = (ok1 && h_ok) ? z1 : __builtin_nanf("");
      if (two) s_z[k2] = (ok2 && h_ok) ? z2 : __builtin_nanf("");
    }
  }
  __syncthreads();
  if (wave != 0) return;
  float z[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) z[j] = (lane + 64 * j < K) ? s_z[lane + 64 * j] : 0.f;
  finish_question(z, K, lane, temperature, lo, true, logits, probs, argmax + i);
}

struct ReadoutArgs {
  const uint16_t *hidden;
  int64_t hidden_rows;
  int d_model;
  const int64_t *last_row;
  const uint16_t *w_u;
  int64_t vocab;
  const int32_t *ids;
  const int32_t *off;
  int n;
  int64_t total;
  int max_options;
  float temperature;
  float *logits;
  float *probs;
  int32_t *argmax;
  // Distinct-row tables of the batched form (null for the per-option form).
  const int32_t *row_id;
  const int32_t *row_first;
  const int32_t *row_entry;
  int64_t n_rows;
};

// Below this many bytes of label rows the readout is bound by launch latency: one fused
// launch beats two (the streaming path pays off on large option tables, where questions with
// many options would otherwise serialise on one workgroup each).
constexpr int64_t kFusedMaxBytes = int64_t(32) << 20;

// Whether a large table takes the ranked one-launch form rather than the streaming pair:
// every compute unit gets at least two questions, so the longest-first order can pair long
// questions with short ones, and no question is longer than about one compute unit's share of
// the rows (max_options <= 9/8 of total / cus; the eighth stands for the second launch the
// ranked form saves). Both forms give bitwise the same results.
inline bool ranked_fits(const ReadoutArgs &a, int cus) {
  return int64_t(a.n) >= 2 * int64_t(cus) && int64_t(a.max_options) * cus * 8 <= a.total * 9;
}

template <int NCH>
hipError_t launch(const ReadoutArgs &a, int cus, hipStream_t stream) {
  if (a.row_id) {
    const int64_t n_blocks = (a.n_rows + kFlatWaves - 1) / kFlatWaves;
    const int64_t grid = (n_blocks + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL(label_logits_rows_kernel<NCH>, dim3(unsigned(grid)),
                       dim3(64 * kFlatWaves), 0, stream, a.hidden, a.hidden_rows, a.d_model,
                       a.last_row, a.w_u, a.vocab, a.off, a.n, a.total, a.row_id, a.row_first,
                       a.row_entry, a.n_rows, n_blocks, a.logits);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(label_softmax_kernel, dim3(unsigned((a.n + kWaves - 1) / kWaves)),
                       dim3(kThreads), 0, stream, a.off, a.n, a.total, a.max_options,
                       a.temperature, a.logits, a.probs, a.argmax);
    return hipGetLastError();
  }
  if (a.total * a.d_model * 2 <= kFusedMaxBytes) {
    hipLaunchKernelGGL((label_readout_fused_kernel<NCH, kWaves, false>), dim3(unsigned(a.n)),
                       dim3(kThreads), 0, stream, a.hidden, a.hidden_rows, a.d_model,
                       a.last_row, a.w_u, a.vocab, a.ids, a.off, a.n, a.total, a.max_options,
                       a.temperature, a.logits, a.probs, a.argmax);
    return hipGetLastError();
  }
  if (ranked_fits(a, cus)) {
    // 16 waves while a lane's hidden chunks and two label rows (12 NCH registers) leave room
    // under the 128 registers of a 1024-thread workgroup; 8 waves beyond.
    constexpr int W = NCH <= 8 ? 16 : 8;
    hipLaunchKernelGGL((label_readout_fused_kernel<NCH, W, true>), dim3(unsigned(a.n)),
                       dim3(64 * W), 0, stream, a.hidden, a.hidden_rows, a.d_model, a.last_row,
                       a.w_u, a.vocab, a.ids, a.off, a.n, a.total, a.max_options,
                       a.temperature, a.logits, a.probs, a.argmax);
    return hipGetLastError();
  }
  const int64_t n_blocks = (a.total + kFlatWaves - 1) / kFlatWaves;
  const int64_t grid = (n_blocks + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL(label_logits_flat_kernel<NCH>, dim3(unsigned(grid)), dim3(64 * kFlatWaves),
                     0, stream, a.hidden, a.hidden_rows, a.d_model, a.last_row, a.w_u, a.vocab,
                     a.ids, a.off, a.n, a.total, n_blocks, a.logits);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(label_softmax_kernel, dim3(unsigned((a.n + kWaves - 1) / kWaves)),
                     dim3(kThreads), 0, stream, a.off, a.n, a.total, a.max_options,
                     a.temperature, a.logits, a.probs, a.argmax);
  return hipGetLastError();
}

typedef hipError_t (*LaunchFn)(const ReadoutArgs &, int, hipStream_t);

}  // namespace

namespace {

// Checks shared by both readout entry points; returns BLINK_OK or the failing status.
int check_common(const void *hidden, int64_t hidden_rows, int32_t d_model,
                 const int64_t *d_last_row, const void *w_u, int64_t vocab,
                 const int32_t *d_cand_off, int32_t n_questions, int64_t total_candidates,
                 int32_t max_options, float temperature, const float *d_logits,
                 const float *d_probs, const int32_t *d_argmax) {
  using blink::fail;
  if (!(temperature > 0.f) || !isfinite(temperature))
    return fail(BLINK_E_INVALID, "temperature is not a positive finite number");
  if (n_questions < 1 || n_questions > BLINK_MAX_QUESTIONS)
    return fail(BLINK_E_LIMIT, "request of %d questions; the limit is 1 to %d", n_questions, BLINK_MAX_QUESTIONS);
  if (max_options < 1 || max_options > BLINK_MAX_OPTIONS)
    return fail(BLINK_E_LIMIT, "question with %d options; the limit is 1 to %d", max_options,
                BLINK_MAX_OPTIONS);
  if (!hidden || !d_last_row || !w_u || !d_cand_off || !d_logits || !d_probs || !d_argmax)
    return fail(BLINK_E_INVALID, "label readout: a pointer argument is NULL");
  if (d_model < 8 || d_model > 64 * 8 * kMaxChunksPerLane || d_model % 8)
    return fail(BLINK_E_INVALID, "d_model %d must be a multiple of 8 in 8..%d", d_model,
                64 * 8 * kMaxChunksPerLane);
  if (hidden_rows < 1 || vocab < 1)
    return fail(BLINK_E_INVALID, "hidden_rows and vocab must be positive");
  if (total_candidates < n_questions ||
      total_candidates > int64_t(n_questions) * int64_t(max_options))
    return fail(BLINK_E_INVALID, "total_candidates %lld does not fit %d questions of 1-%d options",
                (long long)total_candidates, n_questions, max_options);
  if (!blink::aligned16(hidden) || !blink::aligned16(w_u))
    return fail(BLINK_E_INVALID, "hidden and w_u must be 16-byte aligned");
  return BLINK_OK;
}

int run(const ReadoutArgs &a, void *stream) {
  int cus = 0;
  const int rc = blink::device_cus(cus, "label readout");
  if (rc != BLINK_OK) return rc;
  const int nch = (a.d_model / 8 + 63) / 64;  // 16-byte chunks per lane
  static constexpr LaunchFn fns[] = {launch<1>,  launch<2>,  launch<3>,  launch<4>,
                                     launch<5>,  launch<6>,  launch<7>,  launch<8>,
                                     launch<9>,  launch<10>, launch<11>, launch<12>,
                                     launch<13>, launch<14>, launch<15>, launch<16>};
  const hipError_t err = fns[nch - 1](a, cus, static_cast<hipStream_t>(stream));
  if (err != hipSuccess)
    return blink::fail(BLINK_E_DEVICE, "label readout launch: %s", hipGetErrorString(err));
  return blink::ok();
}

}  // namespace

extern "C" int blink_label_readout(const void *hidden, int64_t hidden_rows, int32_t d_model,
                                   const int64_t *d_last_row, const void *w_u, int64_t vocab,
                                   const int32_t *d_cand_ids, const int32_t *d_cand_off,
                                   int32_t n_questions, int64_t total_candidates,
                                   int32_t max_options, float temperature, float *d_logits,
                                   float *d_probs, int32_t *d_argmax, void *stream) {
  const int rc = check_common(hidden, hidden_rows, d_model, d_last_row, w_u, vocab, d_cand_off,
                              n_questions, total_candidates, max_options, temperature, d_logits,
                              d_probs, d_argmax);
  if (rc != BLINK_OK) return rc;
  if (!d_cand_ids)
    return blink::fail(BLINK_E_INVALID, "blink_label_readout: a pointer argument is NULL");
  const ReadoutArgs a{static_cast<const uint16_t *>(hidden), hidden_rows, d_model, d_last_row,
                      static_cast<const uint16_t *>(w_u), vocab, d_cand_ids, d_cand_off,
                      n_questions, total_candidates, max_options, temperature, d_logits,
                      d_probs, d_argmax, nullptr, nullptr, nullptr, 0};
  return run(a, stream);
}

extern "C" int blink_label_readout_batched(
    const void *hidden, int64_t hidden_rows, int32_t d_model, const int64_t *d_last_row,
    const void *w_u, int64_t vocab, const int32_t *d_cand_off, int32_t n_questions,
    int64_t total_candidates, int32_t max_options, const int32_t *d_row_id,
    const int32_t *d_row_first, const int32_t *d_row_entry, int32_t n_rows, float temperature,
    float *d_logits, float *d_probs, int32_t *d_argmax, void *stream) {
  const int rc = check_common(hidden, hidden_rows, d_model, d_last_row, w_u, vocab, d_cand_off,
                              n_questions, total_candidates, max_options, temperature, d_logits,
                              d_probs, d_argmax);
  if (rc != BLINK_OK) return rc;
  if (!d_row_id || !d_row_first || !d_row_entry)
    return blink::fail(BLINK_E_INVALID,
                       "blink_label_readout_batched: a pointer argument is NULL");
  if (n_rows < 1 || n_rows > total_candidates)
    return blink::fail(BLINK_E_INVALID, "n_rows %d outside 1..total_candidates (%lld)", n_rows,
                       (long long)total_candidates);
  const ReadoutArgs a{static_cast<const uint16_t *>(hidden), hidden_rows, d_model, d_last_row,
                      static_cast<const uint16_t *>(w_u), vocab, nullptr, d_cand_off,
                      n_questions, total_candidates, max_options, temperature, d_logits,
                      d_probs, d_argmax, d_row_id, d_row_first, d_row_entry, n_rows};
  return run(a, stream);
}
