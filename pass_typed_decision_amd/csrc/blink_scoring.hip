// Teacher-forced multi-token scoring on gfx950: the full-vocabulary log-softmax of selected
// hidden rows, read at each row's target token.
//
// Method: the simit MoT engine page, teacher-forced scoring (the job option score_len and the
// logits consumer): the rows at key positions n - score_len - 1 .. n - 2 of a sequence each
// predict the next token; each one's score is log_softmax(logits)[target] with the logits
// taken against every unembedding row. Here logits are FP32 sums of bf16 products.
//
// Design. The work is a contraction Z = H W^T of M scored rows (hidden d_model) with all V
// unembedding rows, M small (questions x score_len) and V = 151936, so W must be read from
// HBM exactly once while H (M x d_model, a few MB) is re-read from L2:
//  * score_partials_kernel: one workgroup per 128-row slice of the vocabulary and per block
//    of up to 256 scored rows (128 for calls of at most 128 rows). Both operands go through
//    LDS in chunks of 64 hidden elements (a 128 x 64 slice of W and a 256 x 64 slice of H,
//    rows padded by 16 bytes), and each wave computes Z^T for its 32 rows with
//    v_mfma_f32_32x32x16_bf16 (4 vocabulary tiles of 32). Computing Z^T puts one scored row
//    per lane (and its partner lane l ^ 32), so the slice's maximum and sum of exp are
//    lane-local but for one exchange. The slice writes (max, sum of exp(z - max)) per row to
//    the workspace, and the logit of the row's target if the target falls in the slice.
//  * score_finish_kernel: one wave per scored row merges its slices' (max, sum) pairs into the
//    log-sum-exp and subtracts it from the target's logit.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "blink_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kVocabPerBlock = 128;         // vocabulary rows per workgroup: 4 tiles of 32
constexpr int kChunk = 64;                  // hidden elements per LDS stage
constexpr int kStride = kChunk * 2 + 16;    // LDS row stride in bytes
constexpr int kMaxDModel = 16384;
constexpr int64_t kMaxRows = int64_t(1) << 20;

template <int ROWS>
struct Smem {
  alignas(16) char w[kVocabPerBlock * kStride];
  alignas(16) char h[ROWS * kStride];
};

__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ inline bool row_ok(int64_t idx, int64_t hidden_rows) {
  return idx >= 0 && idx < hidden_rows;
}

// WAVES waves of 32 scored rows each. With 8 waves (256 rows) the kernel keeps four waves per
// SIMD (at most 128 VGPRs), so two workgroups share a CU; with 4 waves (128 rows, for calls of
// at most 128 rows) it keeps three per SIMD, so three workgroups share a CU. Either way one
// workgroup's chunk loads overlap another's matrix work.
template <int WAVES, int MIN_WAVES_PER_SIMD>
__global__ __launch_bounds__(64 * WAVES, MIN_WAVES_PER_SIMD) void score_partials_kernel(
    const uint16_t *__restrict__ hidden, int64_t hidden_rows, int d_model,
    const int64_t *__restrict__ rows, const int32_t *__restrict__ targets, int n_rows,
    const uint16_t *__restrict__ w_u, int64_t vocab, float2 *__restrict__ part,
    float *__restrict__ target_z) {
  constexpr int kThreads = 64 * WAVES;
  constexpr int kRowsPerBlock = 32 * WAVES;
  constexpr int kWPieces = kVocabPerBlock * 8 / kThreads;  // W pieces per thread
  constexpr int kRowStep = kThreads / 8;                    // rows one pass of pieces covers
  __shared__ Smem<kRowsPerBlock> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int64_t v0 = int64_t(blockIdx.x) * kVocabPerBlock;
  const int m0 = int(blockIdx.y) * kRowsPerBlock;

  // Staging: 16-byte pieces, 8 per row of a chunk: 1024 W pieces (kWPieces per thread) and
  // 8 * kRowsPerBlock H pieces (4 per thread). A thread keeps the same rows for every chunk.
  const int piece_col = tid & 7;
  const uint16_t *wsrc[kWPieces];
  bool wvalid[kWPieces];
#pragma unroll
  for (int i = 0; i < kWPieces; ++i) {
    const int r = (tid >> 3) + kRowStep * i;
    wvalid[i] = v0 + r < vocab;
    wsrc[i] = w_u + (wvalid[i] ? (v0 + r) * int64_t(d_model) : 0) + piece_col * 8;
  }
  const uint16_t *hsrc[4];
  bool hvalid[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + kRowStep * i;
    const int m = m0 + r;
    const int64_t idx = m < n_rows ? rows[m] : -1;
    hvalid[i] = row_ok(idx, hidden_rows);
    hsrc[i] = hidden + (hvalid[i] ? idx * int64_t(d_model) : 0) + piece_col * 8;
  }

  f32x16 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x16{};
  const int col = lane & 31, half = lane >> 5;
  const char *afrag = sm.w + col * kStride + 16 * half;  // + tile * 32 rows, + ks * 32 bytes
  const char *bfrag = sm.h + (32 * wave + col) * kStride + 16 * half;

  // The next chunk's global loads are issued before the current chunk's matrix work, so
  // their latency overlaps it; they land in LDS after the second barrier.
  u32x4 wreg[kWPieces], hreg[4];
  auto fetch = [&](int kc) {
#pragma unroll
    for (int i = 0; i < kWPieces; ++i) {
      wreg[i] = u32x4{0u, 0u, 0u, 0u};
      if (wvalid[i])
        wreg[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wsrc[i] + kc));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hreg[i] = u32x4{0u, 0u, 0u, 0u};
      if (hvalid[i]) hreg[i] = *reinterpret_cast<const u32x4 *>(hsrc[i] + kc);
    }
  };
  fetch(0);
  for (int kc = 0; kc < d_model; kc += kChunk) {
#pragma unroll
    for (int i = 0; i < kWPieces; ++i)
      *reinterpret_cast<u32x4 *>(sm.w + ((tid >> 3) + kRowStep * i) * kStride + piece_col * 16) =
          wreg[i];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4 *>(sm.h + ((tid >> 3) + kRowStep * i) * kStride + piece_col * 16) =
          hreg[i];
    __syncthreads();
    if (kc + kChunk < d_model) fetch(kc + kChunk);
#pragma unroll
    for (int ks = 0; ks < kChunk / 16; ++ks) {
      const bf16x8 b = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4 *>(bfrag + ks * 32));
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4 *>(afrag + t * 32 * kStride + ks * 32));
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[t], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // Lane (col, half) holds scored row m0 + 32 wave + col and, in register r of tile t, the
  // vocabulary row v0 + 32 t + 8 (r / 4) + 4 half + r % 4.
  const int m = m0 + 32 * wave + col;
  if (m0 + 32 * wave >= n_rows) return;  // uniform: the wave has no scored row
  // Vocabulary rows of this lane relative to its first one, v0 + 4 half: 32 t + 8 (r/4) + r%4.
  const int64_t vlane = v0 + 4 * half;
  const int limit = int(min(int64_t(kVocabPerBlock), vocab - vlane));  // rows below vocab
  const int64_t tgt = m < n_rows ? int64_t(targets[m]) : -1;
  const int trel = (tgt >= vlane && tgt < vlane + kVocabPerBlock) ? int(tgt - vlane) : -1;
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rel = 32 * t + 8 * (r >> 2) + (r & 3);
      const float z = acc[t][r];
      if (rel < limit) mx = fmaxf(mx, z);
      if (rel == trel) target_z[m] = z;
    }
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  float s = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rel = 32 * t + 8 * (r >> 2) + (r & 3);
      if (rel < limit) s += __expf(acc[t][r] - mx);
    }
  s += __shfl_xor(s, 32);
  if (half == 0 && m < n_rows) part[int64_t(blockIdx.x) * n_rows + m] = make_float2(mx, s);
}

// One wave per scored row: log-sum-exp over the slices, then target logit minus it. A row
// whose index or target is out of range scores NaN.
__global__ __launch_bounds__(256) void score_finish_kernel(
    const int64_t *__restrict__ rows, int64_t hidden_rows, const int32_t *__restrict__ targets,
    int n_rows, int64_t vocab, int n_slices, const float2 *__restrict__ part,
    const float *__restrict__ target_z, float *__restrict__ logprob) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + uniform(int(threadIdx.x >> 6));
  if (m >= n_rows) return;
  float mx = -INFINITY, s = 0.f;
  for (int j = lane; j < n_slices; j += 64) {
    const float2 p = part[int64_t(j) * n_rows + m];
    if (p.x > mx) {
      s = s * __expf(mx - p.x) + p.y;
      mx = p.x;
    } else {
      s += p.y * __expf(p.x - mx);
    }
  }
  float gm = mx;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) gm = fmaxf(gm, __shfl_xor(gm, o));
  float gs = (mx == -INFINITY) ? 0.f : s * __expf(mx - gm);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) gs += __shfl_xor(gs, o);
  if (lane == 0) {
    const int32_t t = targets[m];
    const bool ok = row_ok(rows[m], hidden_rows) && t >= 0 && t < vocab;
    logprob[m] = ok ? target_z[m] - (gm + __logf(gs)) : __builtin_nanf("");
  }
}

inline int64_t n_slices_of(int64_t vocab) { return (vocab + kVocabPerBlock - 1) / kVocabPerBlock; }

inline size_t workspace_bytes_for(int64_t n_rows, int64_t vocab) {
  const size_t part = size_t(n_slices_of(vocab)) * size_t(n_rows) * sizeof(float2);
  return (part + 255) / 256 * 256 + (size_t(n_rows) * sizeof(float) + 255) / 256 * 256;
}

// Scratch of blink_score_targets_noalloc, for callers that cannot allocate device memory:
// one copy per GPU the library runs on, held until the process ends. In host code `scratch`
// names a host-side stand-in, not device memory: its device address on the current GPU comes
// from hipGetSymbolAddress, taken once per device and kept in scratch_ptr.
static __device__ __align__(256) unsigned char scratch[BLINK_SCORE_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, resolved on the first call per device.
int scratch_address(void **out) {
  using blink::fail;
  int device = -1;
  if (hipGetDevice(&device) != hipSuccess || device < 0 || device >= kMaxDevices)
    return fail(BLINK_E_DEVICE, "blink_score_targets_noalloc: no usable current device");
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[device]) {
    void *p = nullptr;
    const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || !p)
      return fail(BLINK_E_DEVICE, "blink_score_targets_noalloc: scratch address on device %d: %s",
                  device, hipGetErrorString(err));
    scratch_ptr[device] = p;
  }
  *out = scratch_ptr[device];
  return BLINK_OK;
}

// Argument checks shared by both entry points (no device call).
int check_args(const void *hidden, int64_t hidden_rows, int32_t d_model, const int64_t *d_rows,
               const int32_t *d_targets, int32_t n_rows, const void *w_u, int64_t vocab,
               const float *d_logprob) {
  using blink::fail;
  if (!hidden || !d_rows || !d_targets || !w_u || !d_logprob)
    return fail(BLINK_E_INVALID, "blink_score_targets: a pointer argument is NULL");
  if (n_rows < 1 || n_rows > kMaxRows)
    return fail(BLINK_E_LIMIT, "%d scored rows; the limit is 1 to %lld", n_rows,
                (long long)kMaxRows);
  if (d_model < kChunk || d_model > kMaxDModel || d_model % kChunk)
    return fail(BLINK_E_INVALID, "d_model %d must be a multiple of %d in %d..%d", d_model,
                kChunk, kChunk, kMaxDModel);
  if (hidden_rows < 1 || vocab < 1 || vocab > (int64_t(1) << 31))
    return fail(BLINK_E_INVALID, "hidden_rows must be positive and vocab in 1..2^31");
  if (!blink::aligned16(hidden) || !blink::aligned16(w_u))
    return fail(BLINK_E_INVALID, "hidden and w_u must be 16-byte aligned");
  if (n_slices_of(vocab) > 0x7fffffffLL) return fail(BLINK_E_LIMIT, "vocabulary too large");
  return BLINK_OK;
}

// Both kernels on `stream`, with the partials in `workspace` (checked large enough).
int launch_scoring(const void *hidden, int64_t hidden_rows, int32_t d_model,
                   const int64_t *d_rows, const int32_t *d_targets, int32_t n_rows,
                   const void *w_u, int64_t vocab, float *d_logprob, void *workspace,
                   void *stream) {
  const int64_t slices = n_slices_of(vocab);
  float2 *part = static_cast<float2 *>(workspace);
  const size_t part_bytes = (size_t(slices) * size_t(n_rows) * sizeof(float2) + 255) / 256 * 256;
  float *target_z = reinterpret_cast<float *>(static_cast<char *>(workspace) + part_bytes);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const uint16_t *h = static_cast<const uint16_t *>(hidden);
  const uint16_t *w = static_cast<const uint16_t *>(w_u);
  if (n_rows <= 128) {  // one block of 4 waves per slice: three workgroups per CU
    hipLaunchKernelGGL((score_partials_kernel<4, 3>), dim3(unsigned(slices)), dim3(256), 0, s, h,
                       hidden_rows, d_model, d_rows, d_targets, n_rows, w, vocab, part, target_z);
  } else {  // blocks of 256 rows: W is read once for every 256 scored rows
    const dim3 grid(unsigned(slices), unsigned((n_rows + 255) / 256));
    hipLaunchKernelGGL((score_partials_kernel<8, 4>), grid, dim3(512), 0, s, h, hidden_rows,
                       d_model, d_rows, d_targets, n_rows, w, vocab, part, target_z);
  }
  hipError_t err = hipGetLastError();
  if (err == hipSuccess) {
    hipLaunchKernelGGL(score_finish_kernel, dim3(unsigned((n_rows + 3) / 4)), dim3(256), 0, s,
                       d_rows, hidden_rows, d_targets, n_rows, vocab, int(slices), part,
                       target_z, d_logprob);
    err = hipGetLastError();
  }
  if (err != hipSuccess)
    return blink::fail(BLINK_E_DEVICE, "blink_score_targets launch: %s", hipGetErrorString(err));
  return blink::ok();
}

}  // namespace

extern "C" size_t blink_score_targets_workspace(int32_t n_rows, int64_t vocab) {
  if (n_rows < 1 || n_rows > kMaxRows || vocab < 1 || vocab > (int64_t(1) << 31)) return 0;
  return workspace_bytes_for(n_rows, vocab);
}

extern "C" int blink_score_targets(const void *hidden, int64_t hidden_rows, int32_t d_model,
                                   const int64_t *d_rows, const int32_t *d_targets,
                                   int32_t n_rows, const void *w_u, int64_t vocab,
                                   float *d_logprob, void *workspace, size_t workspace_bytes,
                                   void *stream) {
  using blink::fail;
  int rc = check_args(hidden, hidden_rows, d_model, d_rows, d_targets, n_rows, w_u, vocab,
                      d_logprob);
  if (rc != BLINK_OK) return rc;
  if (!workspace) return fail(BLINK_E_INVALID, "blink_score_targets: a pointer argument is NULL");
  if (!blink::aligned16(workspace))
    return fail(BLINK_E_INVALID, "hidden, w_u and workspace must be 16-byte aligned");
  const size_t need = workspace_bytes_for(n_rows, vocab);
  if (workspace_bytes < need)
    return fail(BLINK_E_INVALID, "workspace of %zu bytes; %zu needed", workspace_bytes, need);
  return launch_scoring(hidden, hidden_rows, d_model, d_rows, d_targets, n_rows, w_u, vocab,
                        d_logprob, workspace, stream);
}

extern "C" int blink_score_targets_noalloc(const void *hidden, int64_t hidden_rows,
                                           int32_t d_model, const int64_t *d_rows,
                                           const int32_t *d_targets, int32_t n_rows,
                                           const void *w_u, int64_t vocab, float *d_logprob,
                                           void *stream) {
  using blink::fail;
  int rc = check_args(hidden, hidden_rows, d_model, d_rows, d_targets, n_rows, w_u, vocab,
                      d_logprob);
  if (rc != BLINK_OK) return rc;
  const size_t need = workspace_bytes_for(n_rows, vocab);
  if (need > size_t(BLINK_SCORE_SCRATCH_BYTES))
    return fail(BLINK_E_LIMIT, "%d scored rows over a vocabulary of %lld need %zu bytes of "
                "scratch; the library's static scratch holds %zu", n_rows, (long long)vocab, need,
                size_t(BLINK_SCORE_SCRATCH_BYTES));
  void *ws = nullptr;
  if ((rc = scratch_address(&ws)) != BLINK_OK) return rc;
  return launch_scoring(hidden, hidden_rows, d_model, d_rows, d_targets, n_rows, w_u, vocab,
                        d_logprob, ws, stream);
}
