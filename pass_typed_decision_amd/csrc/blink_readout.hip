// Label readout on gfx950: gather each question's last real hidden row, score its offered
// labels against their unembedding rows in FP32, temperature softmax, first-index argmax.
//
// Method: blink.py page (thegovind/blink-4b), "torch engine" section, _read (per-question
// gather, FP32 upcast of the hidden row and of the label rows, FP32 matrix-vector product),
// and "answer assembly" section, softmax (divide by the temperature, subtract the maximum,
// exponentiate, normalise) and answer_for (most probable option, earlier option on ties).
//
// Design: one workgroup (4 wave64) per question. The hidden row is widened once into
// registers, each lane owning 16-byte chunks lane, lane+64, ...; every wave streams whole
// label rows with 16-byte coalesced loads (a 2560-wide bf16 row is five 1 KiB wave loads),
// two rows at a time for memory-level parallelism, and reduces its partial sums across the
// wave. Logits go through LDS to wave 0, which does the softmax and argmax. The kernel is
// bound by HBM bandwidth on the label rows; nothing else is re-read.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "blink_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxChunksPerLane = 16;  // d_model <= 16 * 64 * 8 = 8192

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

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

template <int NCH>
__device__ inline float row_dot(const u32x4 (&w)[NCH], const float (&h)[NCH][8]) {
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      acc = fmaf(lo_bf16(w[c][m]), h[c][2 * m], acc);
      acc = fmaf(hi_bf16(w[c][m]), h[c][2 * m + 1], acc);
    }
  }
  return acc;
}

template <int NCH>
__global__ __launch_bounds__(kThreads) void label_readout_kernel(
    const uint16_t *__restrict__ hidden, int64_t hidden_rows, int d_model,
    const int64_t *__restrict__ last_row, const uint16_t *__restrict__ w_u, int64_t vocab,
    const int32_t *__restrict__ cand_ids, const int32_t *__restrict__ cand_off,
    int64_t total_cand, int max_options, float temperature, float *__restrict__ logits,
    float *__restrict__ probs, int32_t *__restrict__ argmax) {
  __shared__ float s_z[256];
  __shared__ int s_bad;
  const int i = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  const int64_t lo = cand_off[i], hi = cand_off[i + 1];
  if (!(lo >= 0 && hi <= total_cand && hi - lo >= 1 && hi - lo <= max_options)) {
    if (tid == 0) argmax[i] = -1;  // offsets unusable: nothing else can be written safely
    return;
  }
  const int K = int(hi - lo);
  const int64_t row = last_row[i];
  const bool row_ok = row >= 0 && row < hidden_rows;
  if (tid == 0) s_bad = row_ok ? 0 : 1;

  const int nchunks = d_model >> 3;
  float h[NCH][8];
  const uint16_t *hrow = hidden + (row_ok ? row : 0) * int64_t(d_model);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ch = lane + 64 * c;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (row_ok && ch < nchunks) w = *reinterpret_cast<const u32x4 *>(hrow + ch * 8);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      h[c][2 * m] = lo_bf16(w[m]);
      h[c][2 * m + 1] = hi_bf16(w[m]);
    }
  }
  __syncthreads();

  // Two label rows per wave per step: rows k and k + kWaves.
  for (int k = wave; k < K; k += 2 * kWaves) {
    const int k2 = k + kWaves;
    const int32_t id1 = cand_ids[lo + k];
    const int32_t id2 = k2 < K ? cand_ids[lo + k2] : 0;
    const bool ok1 = id1 >= 0 && id1 < vocab;
    const bool ok2 = k2 >= K || (id2 >= 0 && id2 < vocab);
    const uint16_t *r1 = w_u + int64_t(ok1 ? id1 : 0) * d_model;
    const uint16_t *r2 = w_u + int64_t(ok2 && k2 < K ? id2 : 0) * d_model;
    u32x4 w1[NCH], w2[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = lane + 64 * c;
      w1[c] = u32x4{0u, 0u, 0u, 0u};
      w2[c] = u32x4{0u, 0u, 0u, 0u};
      if (ch < nchunks) {
        w1[c] = *reinterpret_cast<const u32x4 *>(r1 + ch * 8);
        if (k2 < K) w2[c] = *reinterpret_cast<const u32x4 *>(r2 + ch * 8);
      }
    }
    const float z1 = wave_sum(row_dot<NCH>(w1, h));
    const float z2 = wave_sum(row_dot<NCH>(w2, h));
    if (lane == 0) {
      s_z[k] = z1;
      if (k2 < K) s_z[k2] = z2;
      if (!ok1 || !ok2) s_bad = 1;
    }
  }
  __syncthreads();
  if (wave != 0) return;

  if (s_bad) {
    for (int k = lane; k < K; k += 64) {
      logits[lo + k] = __builtin_nanf("");
      probs[lo + k] = __builtin_nanf("");
    }
    if (lane == 0) argmax[i] = -1;
    return;
  }

  // Softmax over the question's own options and first-index argmax (on the logits).
  float zt[4], best = -INFINITY, mt = -INFINITY;
  int best_k = K;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int k = lane + 64 * j;
    zt[j] = -INFINITY;
    if (k < K) {
      const float z = s_z[k];
      zt[j] = z / temperature;
      mt = fmaxf(mt, zt[j]);
      if (z > best) {  // strict: the earliest k of this lane wins ties
        best = z;
        best_k = k;
      }
    }
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
  const float total = wave_sum(part);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int k = lane + 64 * j;
    if (k < K) {
      logits[lo + k] = s_z[k];
      probs[lo + k] = e[j] / total;
    }
  }
  if (lane == 0) argmax[i] = best_k;
}

template <int NCH>
hipError_t launch(const void *hidden, int64_t hidden_rows, int d_model, const int64_t *last_row,
                  const void *w_u, int64_t vocab, const int32_t *ids, const int32_t *off,
                  int n, int64_t total, int max_options, float temperature, float *logits,
                  float *probs, int32_t *argmax, hipStream_t stream) {
  hipLaunchKernelGGL(label_readout_kernel<NCH>, dim3(n), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t *>(hidden), hidden_rows, d_model, last_row,
                     static_cast<const uint16_t *>(w_u), vocab, ids, off, total, max_options,
                     temperature, logits, probs, argmax);
  return hipGetLastError();
}

typedef hipError_t (*LaunchFn)(const void *, int64_t, int, const int64_t *, const void *, int64_t,
                               const int32_t *, const int32_t *, int, int64_t, int, float,
                               float *, float *, int32_t *, hipStream_t);

}  // namespace

extern "C" int blink_label_readout(const void *hidden, int64_t hidden_rows, int32_t d_model,
                                   const int64_t *d_last_row, const void *w_u, int64_t vocab,
                                   const int32_t *d_cand_ids, const int32_t *d_cand_off,
                                   int32_t n_questions, int64_t total_candidates,
                                   int32_t max_options, float temperature, float *d_logits,
                                   float *d_probs, int32_t *d_argmax, void *stream) {
  using blink::fail;
  if (!(temperature > 0.f) || !isfinite(temperature))
    return fail(BLINK_E_INVALID, "temperature must be positive");
  if (n_questions < 1 || n_questions > BLINK_MAX_QUESTIONS)
    return fail(BLINK_E_LIMIT, "%d questions; supported 1-%d", n_questions, BLINK_MAX_QUESTIONS);
  if (max_options < 1 || max_options > BLINK_MAX_OPTIONS)
    return fail(BLINK_E_LIMIT, "%d options per choice; supported 1-%d", max_options,
                BLINK_MAX_OPTIONS);
  if (!hidden || !d_last_row || !w_u || !d_cand_ids || !d_cand_off || !d_logits || !d_probs ||
      !d_argmax)
    return fail(BLINK_E_INVALID, "blink_label_readout: a pointer argument is NULL");
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

  const int nch = (d_model / 8 + 63) / 64;  // 16-byte chunks per lane
  static constexpr LaunchFn fns[] = {launch<1>,  launch<2>,  launch<3>,  launch<4>,
                                     launch<5>,  launch<6>,  launch<7>,  launch<8>,
                                     launch<9>,  launch<10>, launch<11>, launch<12>,
                                     launch<13>, launch<14>, launch<15>, launch<16>};
  const hipError_t err =
      fns[nch - 1](hidden, hidden_rows, d_model, d_last_row, w_u, vocab, d_cand_ids, d_cand_off,
                   n_questions, total_candidates, max_options, temperature, d_logits, d_probs,
                   d_argmax, static_cast<hipStream_t>(stream));
  if (err != hipSuccess)
    return fail(BLINK_E_DEVICE, "blink_label_readout launch: %s", hipGetErrorString(err));
  return blink::ok();
}
