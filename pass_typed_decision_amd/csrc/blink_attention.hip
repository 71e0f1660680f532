// Shared-prefix tail-prefill attention on gfx950 (CDNA4).
//
// Method: blink.py page (thegovind/blink-4b), "torch engine" section, _forward_shared and
// _forward, and the PREFIX_CACHE comment in "constants the deployment sets": the shared
// prefix (system prompt plus evidence) is encoded once; every question's own tail then runs
// causally against that one cached prefix. Same tokens and positions as the plain path, so a
// tail row at position t sees every prefix key and the question's tail keys 0..t.
//
// Kernel design (one launch for every question of the request):
//  * Work unit = one KV head g and 256 consecutive "query rows" of that head's group, where
//    the rows are (real tail token, query head of the group) pairs, token-major, over all
//    questions in question order. Padding rows are never computed, and a unit may span
//    question boundaries, so a launch has no ragged-tile waste except at its very end.
//  * Workgroup = 4 wave64, one per SIMD; each wave owns 64 query rows (two 32-row blocks).
//    Every K/V tile (64 keys) is staged in LDS once and read by all four waves, i.e. one
//    prefix tile load serves 256 query rows of up to 256/G questions' tails.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: in the
//    accumulator layout a lane holds one query and 16 keys of each 32-key block, so the row
//    max and row sum are lane-local except for one exchange with the partner lane (l ^ 32).
//    The probabilities then feed O^T += V^T P^T directly from registers as the B operand;
//    V is written to LDS transposed, with the keys of each 16-key group permuted so that a
//    lane's eight keys are contiguous and come in with one 16-byte LDS read.
//  * Online softmax in FP32 (exp2 with scale*log2(e) folded into one FMA). The running max
//    is only raised when a tile's max exceeds it by more than 2^8, so the O rescale (a pass
//    over all accumulators) almost never runs; the decision is per row, so a row's result
//    does not depend on which other rows share its wave.
//  * Prefix tiles first (unmasked except the last partial tile), then the tail tiles of each
//    question the unit touches, masked per lane (same question and key <= position).
//  * blockIdx -> (KV head, unit) puts the KV head in the low bits, so with 8 KV heads each of
//    the 8 XCDs (dispatch is round-robin over XCDs) streams one head's prefix K/V through its
//    own L2.
//  * Double-buffered LDS: the next tile's global loads are issued before the current tile's
//    MFMAs and written to the other buffer afterwards; one barrier per tile.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "blink_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kTileKeys = 64;
constexpr int kMaxGroup = 16;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLazyRescale = 8.0f;  // log2 units: probabilities stay <= 256 between rescales

struct Args {
  const uint16_t *q;
  const uint16_t *k_tail;
  const uint16_t *v_tail;
  const uint16_t *k_pre;
  const uint16_t *v_pre;
  uint16_t *out;
  const int64_t *token_offset;
  const int32_t *valid_start;
  int n;
  int64_t total_valid;
  int64_t t_pad;
  int prefix_len;
  int hq;
  int hkv;
  int group;
  float scale_log2;
};

template <int D>
struct Smem {
  static constexpr int KS = D + 8;          // K row stride in bf16 (16-byte pad)
  static constexpr int VS = kTileKeys + 8;  // V^T row stride in bf16 (16-byte pad)
  uint16_t k[2][kTileKeys * KS];
  uint16_t v[2][D * VS];
  int32_t start[BLINK_MAX_QUESTIONS + 1];
};

// Largest q in [0, n) with start[q] <= c (start ascending). Terminates for any contents.
__device__ inline int find_question(const int32_t *start, int n, int64_t c) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (start[mid] <= c)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// Pair reduction over lanes l and l ^ 32 (they hold the same query, different keys).
__device__ inline float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Source of one 64-key tile: rows rowbase + kstart + [0, 64) of k/v, valid below klimit.
struct TileSrc {
  const uint16_t *k;
  const uint16_t *v;
  int64_t rowbase;
  int64_t rowcount;  // rows that exist in k/v (bounds check)
  int kstart;
  int klimit;
  int q;  // -1 for the prefix
  bool valid;
};

template <int D>
struct Stage {
  static constexpr int KCH = kTileKeys * D / 8 / kThreads;  // 16-byte K chunks per thread
  u32x4 k[KCH];
  u32x4 v[4];  // 4 keys x 8 dims (threads < 2 * D)
};

template <int D>
__device__ inline void load_tile(const Args &a, int g, const TileSrc &s, int tid, Stage<D> &st) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
#pragma unroll
  for (int i = 0; i < Stage<D>::KCH; ++i) {
    const int ci = tid + kThreads * i;
    const int key = ci / CPR, dch = ci % CPR;
    const int kk = s.kstart + key;
    const int64_t row = s.rowbase + kk;
    st.k[i] = u32x4{0u, 0u, 0u, 0u};
    if (kk < s.klimit && row >= 0 && row < s.rowcount)
      st.k[i] = *reinterpret_cast<const u32x4 *>(s.k + (row * a.hkv + g) * D + dch * 8);
  }
  if (tid < 2 * D) {
    const int kg = tid & 15, dc = tid >> 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kk = s.kstart + 4 * kg + r;
      const int64_t row = s.rowbase + kk;
      st.v[r] = u32x4{0u, 0u, 0u, 0u};
      if (kk < s.klimit && row >= 0 && row < s.rowcount)
        st.v[r] = *reinterpret_cast<const u32x4 *>(s.v + (row * a.hkv + g) * D + dc * 8);
    }
  }
}

template <int D>
__device__ inline void store_tile(Smem<D> &sm, int buf, int tid, const Stage<D> &st) {
  constexpr int CPR = D / 8;
#pragma unroll
  for (int i = 0; i < Stage<D>::KCH; ++i) {
    const int ci = tid + kThreads * i;
    const int key = ci / CPR, dch = ci % CPR;
    *reinterpret_cast<u32x4 *>(&sm.k[buf][key * Smem<D>::KS + dch * 8]) = st.k[i];
  }
  if (tid < 2 * D) {
    const int kg = tid & 15, dc = tid >> 4;
    // keys 4kg..4kg+3 land in slots (kg & ~3) * 4 + 4 * perm[kg & 3], perm = {0, 2, 1, 3}
    const int sub = kg & 3;
    const int slot = (kg >> 2) * 16 + 4 * ((sub == 1) ? 2 : (sub == 2) ? 1 : sub);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      // dims 8dc + 2m (low halves) and 8dc + 2m + 1 (high halves) of the four keys
      u32x2 even, odd;
      even[0] = __builtin_amdgcn_perm(st.v[1][m], st.v[0][m], 0x05040100u);
      even[1] = __builtin_amdgcn_perm(st.v[3][m], st.v[2][m], 0x05040100u);
      odd[0] = __builtin_amdgcn_perm(st.v[1][m], st.v[0][m], 0x07060302u);
      odd[1] = __builtin_amdgcn_perm(st.v[3][m], st.v[2][m], 0x07060302u);
      *reinterpret_cast<u32x2 *>(&sm.v[buf][(8 * dc + 2 * m) * Smem<D>::VS + slot]) = even;
      *reinterpret_cast<u32x2 *>(&sm.v[buf][(8 * dc + 2 * m + 1) * Smem<D>::VS + slot]) = odd;
    }
  }
}

struct RowState {
  float m;  // running max in scaled log2 units (-inf before any visible key)
  float l;  // this lane's partial sum of probabilities (the partner lane holds the rest)
};

// One 64-key tile for one wave, as two 32-key sub-tiles: S^T = K Q^T, online softmax,
// O^T += V^T P^T. lim[qb]: largest visible key index within the tile minus 4 * (lane >> 5);
// keys above it are masked (used only when MASKED).
template <int D, int QB, bool MASKED>
__device__ inline void compute_tile(const Smem<D> &sm, int buf, int lane, float scale_log2,
                                    const bf16x8 (&qf)[QB][D / 16], f32x16 (&o)[QB][D / 32],
                                    RowState (&rs)[QB], const int (&lim)[QB]) {
  const int col = lane & 31, half = lane >> 5;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    f32x16 s[QB];  // [query block]
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) s[qb] = f32x16{};
    const uint16_t *kbase = &sm.k[buf][(kb * 32 + col) * Smem<D>::KS + 8 * half];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8 kf = as_bf16x8(*reinterpret_cast<const u32x4 *>(kbase + ks * 16));
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][ks], s[qb], 0, 0, 0);
    }

    float factor[QB];
    bool rescale = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float x = s[qb][v];
        if (MASKED) {
          const int key = kb * 32 + 8 * (v >> 2) + (v & 3);
          x = (key <= lim[qb]) ? x : -INFINITY;
          s[qb][v] = x;
        }
        mx = fmaxf(mx, x);
      }
      const float mt = pair_max(mx) * scale_log2;
      const float m_old = rs[qb].m;
      const float m_new = (mt > m_old + kLazyRescale) ? mt : m_old;
      factor[qb] = (m_new == m_old) ? 1.0f : __builtin_amdgcn_exp2f(m_old - m_new);
      rescale |= factor[qb] != 1.0f;
      rs[qb].m = m_new;
      const float base = (m_new == -INFINITY) ? 0.0f : m_new;
      float sum = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[qb][v], scale_log2, -base));
        s[qb][v] = p;
        sum += p;
      }
      rs[qb].l = rs[qb].l * factor[qb] + sum;
    }
    if (__builtin_amdgcn_ballot_w64(rescale)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[qb][db] *= factor[qb];
    }

    const uint16_t *vbase = &sm.v[buf][col * Smem<D>::VS + 8 * half + 32 * kb];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      bf16x8 pb[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[qb][e] = (__bf16)s[qb][8 * c + e];
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x8 vf =
            as_bf16x8(*reinterpret_cast<const u32x4 *>(vbase + db * 32 * Smem<D>::VS + 16 * c));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[qb], o[qb][db], 0, 0, 0);
      }
    }
  }
}

struct Unit {
  int qa, qz, posz;  // questions touched by the workgroup; last row's position in qz
};

__device__ inline TileSrc tail_from(const Args &a, const int32_t *start, const Unit &u, int q,
                                    int g) {
  (void)g;
  TileSrc s{};
  s.valid = false;
  for (; q <= u.qz; ++q) {
    const int nq = start[q + 1] - start[q];
    const int limit = (q == u.qz) ? u.posz + 1 : nq;
    // A malformed table cannot make the loop run past the context length.
    if (limit > 0 && limit <= nq && nq <= BLINK_MAX_INPUT_TOKENS) {
      s.k = a.k_tail;
      s.v = a.v_tail;
      s.rowbase = a.token_offset[q];
      s.rowcount = a.t_pad;
      s.kstart = 0;
      s.klimit = limit;
      s.q = q;
      s.valid = true;
      return s;
    }
  }
  return s;
}

__device__ inline TileSrc first_tile(const Args &a, const int32_t *start, const Unit &u, int g) {
  if (a.prefix_len > 0) {
    TileSrc s{};
    s.k = a.k_pre;
    s.v = a.v_pre;
    s.rowbase = 0;
    s.rowcount = a.prefix_len;
    s.kstart = 0;
    s.klimit = a.prefix_len;
    s.q = -1;
    s.valid = true;
    return s;
  }
  return tail_from(a, start, u, u.qa, g);
}

__device__ inline TileSrc next_tile(const Args &a, const int32_t *start, const Unit &u,
                                    TileSrc s, int g) {
  s.kstart += kTileKeys;
  if (s.kstart < s.klimit) return s;
  return tail_from(a, start, u, s.q < 0 ? u.qa : s.q + 1, g);
}

template <int D, int QB>
__global__ __launch_bounds__(kThreads, 1) void prefix_tail_attention_kernel(Args a) {
  constexpr int kRowsPerWave = 32 * QB;
  constexpr int kRowsPerUnit = 4 * kRowsPerWave;
  __shared__ __attribute__((aligned(16))) Smem<D> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int G = a.group;
  const int g = int(blockIdx.x % unsigned(a.hkv));
  const int64_t unit = blockIdx.x / unsigned(a.hkv);

  for (int i = tid; i <= a.n; i += kThreads) sm.start[i] = a.valid_start[i];
  __syncthreads();
  const int64_t valid_total = min(int64_t(sm.start[a.n]), a.total_valid);
  const int64_t R = valid_total * G;
  const int64_t row0 = unit * kRowsPerUnit;
  if (row0 >= R) return;  // uniform across the workgroup

  // This lane's two query rows.
  bool rvalid[QB];
  int rq[QB], rpos[QB], rhead[QB];
  int64_t rtok[QB];
  bf16x8 qf[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int64_t r = row0 + wave * kRowsPerWave + qb * 32 + col;
    rvalid[qb] = r < R;
    const int64_t c = rvalid[qb] ? r / G : 0;
    const int hl = int(r % G);
    const int q = find_question(sm.start, a.n, c);
    const int nq = sm.start[q + 1] - sm.start[q];
    const int pos = int(c - sm.start[q]);
    rvalid[qb] = rvalid[qb] && pos >= 0 && pos < nq;
    const int64_t tok = a.token_offset[q] + pos;
    rvalid[qb] = rvalid[qb] && tok >= 0 && tok < a.t_pad;
    rq[qb] = rvalid[qb] ? q : -1;
    rpos[qb] = pos;
    rtok[qb] = tok;
    rhead[qb] = g * G + hl;
    const uint16_t *qrow = a.q + ((rvalid[qb] ? tok : 0) * a.hq + rhead[qb]) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (rvalid[qb]) v = *reinterpret_cast<const u32x4 *>(qrow + ks * 16);
      qf[qb][ks] = as_bf16x8(v);
    }
  }

  // Questions touched by the workgroup and by this wave.
  Unit u;
  {
    const int64_t c0 = row0 / G, cz = (min(row0 + kRowsPerUnit, R) - 1) / G;
    u.qa = find_question(sm.start, a.n, c0);
    u.qz = find_question(sm.start, a.n, cz);
    u.posz = int(cz - sm.start[u.qz]);
  }
  const int64_t wr0 = row0 + wave * kRowsPerWave;
  const bool wave_active = wr0 < R;
  int wqa = 0, wqz = -1, wposz = -1;
  if (wave_active) {
    const int64_t c0 = wr0 / G, cz = (min(wr0 + kRowsPerWave, R) - 1) / G;
    wqa = find_question(sm.start, a.n, c0);
    wqz = find_question(sm.start, a.n, cz);
    wposz = int(cz - sm.start[wqz]);
  }

  f32x16 o[QB][D / 32];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[qb][db] = f32x16{};
  RowState rs[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) rs[qb] = RowState{-INFINITY, 0.f};

  TileSrc cur = first_tile(a, sm.start, u, g);
  if (!cur.valid) return;  // uniform: nothing visible (cannot happen for a valid table)
  Stage<D> st;
  load_tile<D>(a, g, cur, tid, st);
  store_tile<D>(sm, 0, tid, st);
  __syncthreads();
  int buf = 0;
  while (true) {
    const TileSrc nxt = next_tile(a, sm.start, u, cur, g);
    if (nxt.valid) load_tile<D>(a, g, nxt, tid, st);

    bool active = wave_active;
    if (cur.q >= 0)
      active = active && cur.q >= wqa && cur.q <= wqz && !(cur.q == wqz && cur.kstart > wposz);
    if (active) {
      if (cur.q < 0 && cur.kstart + kTileKeys <= a.prefix_len) {
        int lim[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) lim[qb] = kTileKeys;
        compute_tile<D, QB, false>(sm, buf, lane, a.scale_log2, qf, o, rs, lim);
      } else {
        int lim[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          int last;  // last visible key of this row, relative to the tile start
          if (cur.q < 0)
            last = a.prefix_len - 1 - cur.kstart;
          else
            last = (rq[qb] == cur.q) ? rpos[qb] - cur.kstart : -1;
          last = min(last, kTileKeys - 1);
          lim[qb] = last - 4 * half;
        }
        compute_tile<D, QB, true>(sm, buf, lane, a.scale_log2, qf, o, rs, lim);
      }
    }

    if (nxt.valid) store_tile<D>(sm, buf ^ 1, tid, st);
    __syncthreads();
    if (!nxt.valid) break;
    cur = nxt;
    buf ^= 1;
  }

  // Normalise and store bf16 rows (four consecutive dims per 8-byte store).
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l = pair_sum(rs[qb].l);
    if (!rvalid[qb]) continue;
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    uint16_t *orow = a.out + (rtok[qb] * a.hq + rhead[qb]) * D + 4 * half;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        u32x2 packed;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const __bf16 x0 = (__bf16)(o[qb][db][4 * grp + 2 * j] * inv);
          const __bf16 x1 = (__bf16)(o[qb][db][4 * grp + 2 * j + 1] * inv);
          packed[j] = uint32_t(__builtin_bit_cast(uint16_t, x0)) |
                      (uint32_t(__builtin_bit_cast(uint16_t, x1)) << 16);
        }
        *reinterpret_cast<u32x2 *>(orow + db * 32 + 8 * grp) = packed;
      }
    }
  }
}

template <int D, int QB>
hipError_t launch(const Args &a, hipStream_t stream) {
  constexpr int kRowsPerUnit = 4 * 32 * QB;
  const int64_t rows = a.total_valid * a.group;
  const int64_t units = (rows + kRowsPerUnit - 1) / kRowsPerUnit;
  const int64_t blocks = units * a.hkv;
  hipLaunchKernelGGL((prefix_tail_attention_kernel<D, QB>), dim3(unsigned(blocks)), dim3(kThreads),
                     0, stream, a);
  return hipGetLastError();
}

}  // namespace

extern "C" int blink_prefix_tail_attention(const void *q, const void *k_tail, const void *v_tail,
                                           const void *k_prefix, const void *v_prefix, void *out,
                                           const int64_t *d_token_offset,
                                           const int32_t *d_valid_start, int32_t n_questions,
                                           int64_t total_valid_tokens,
                                           int64_t total_padded_tokens, int32_t prefix_len,
                                           int32_t n_heads_q, int32_t n_heads_kv,
                                           int32_t head_dim, float scale, void *stream) {
  using blink::fail;
  if (n_questions < 1 || n_questions > BLINK_MAX_QUESTIONS)
    return fail(BLINK_E_LIMIT, "%d questions; supported 1-%d", n_questions, BLINK_MAX_QUESTIONS);
  if (!q || !k_tail || !v_tail || !out || !d_token_offset || !d_valid_start)
    return fail(BLINK_E_INVALID, "blink_prefix_tail_attention: a pointer argument is NULL");
  if (prefix_len < 0 || prefix_len >= BLINK_MAX_INPUT_TOKENS)
    return fail(BLINK_E_LIMIT, "prefix of %d tokens leaves no room under the maximum context "
                "length of %d", prefix_len, BLINK_MAX_INPUT_TOKENS);
  if (prefix_len > 0 && (!k_prefix || !v_prefix))
    return fail(BLINK_E_INVALID, "prefix K/V pointers are NULL with prefix_len %d", prefix_len);
  if (head_dim != 64 && head_dim != 128)
    return fail(BLINK_E_INVALID, "head_dim %d is not supported (64 or 128)", head_dim);
  if (n_heads_kv < 1 || n_heads_q < n_heads_kv || n_heads_q % n_heads_kv ||
      n_heads_q / n_heads_kv > kMaxGroup)
    return fail(BLINK_E_INVALID, "head counts %d/%d: need H_q a multiple of H_kv, group <= %d",
                n_heads_q, n_heads_kv, kMaxGroup);
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(BLINK_E_INVALID, "scale must be finite and positive");
  if (total_valid_tokens < n_questions || total_padded_tokens < total_valid_tokens ||
      total_valid_tokens > int64_t(n_questions) * BLINK_MAX_INPUT_TOKENS)
    return fail(BLINK_E_INVALID, "token totals do not fit: %lld real of %lld padded for %d "
                "questions", (long long)total_valid_tokens, (long long)total_padded_tokens,
                n_questions);
  const int64_t blocks =
      (total_valid_tokens * (n_heads_q / n_heads_kv) + 127) / 128 * n_heads_kv;
  if (blocks > 0x7fffffffLL) return fail(BLINK_E_LIMIT, "launch too large");
  const void *ptrs[] = {q, k_tail, v_tail, out, prefix_len ? k_prefix : q, prefix_len ? v_prefix : q};
  for (const void *p : ptrs)
    if (!blink::aligned16(p)) return fail(BLINK_E_INVALID, "tensors must be 16-byte aligned");

  Args a;
  a.q = static_cast<const uint16_t *>(q);
  a.k_tail = static_cast<const uint16_t *>(k_tail);
  a.v_tail = static_cast<const uint16_t *>(v_tail);
  a.k_pre = static_cast<const uint16_t *>(k_prefix);
  a.v_pre = static_cast<const uint16_t *>(v_prefix);
  a.out = static_cast<uint16_t *>(out);
  a.token_offset = d_token_offset;
  a.valid_start = d_valid_start;
  a.n = n_questions;
  a.total_valid = total_valid_tokens;
  a.t_pad = total_padded_tokens;
  a.prefix_len = prefix_len;
  a.hq = n_heads_q;
  a.hkv = n_heads_kv;
  a.group = n_heads_q / n_heads_kv;
  a.scale_log2 = scale * kLog2e;

  (void)hipGetLastError();
  const hipError_t err = head_dim == 64 ? launch<64, 2>(a, static_cast<hipStream_t>(stream))
                                        : launch<128, 1>(a, static_cast<hipStream_t>(stream));
  if (err != hipSuccess)
    return fail(BLINK_E_DEVICE, "blink_prefix_tail_attention launch: %s", hipGetErrorString(err));
  return blink::ok();
}
