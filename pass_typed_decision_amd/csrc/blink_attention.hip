// Shared-prefix tail-prefill attention on gfx950 (CDNA4).
//
// Method: blink.py page (thegovind/blink-4b), "torch engine" section, _forward_shared and
// _forward, and the PREFIX_CACHE comment in "constants the deployment sets": the shared
// prefix (system prompt plus evidence) is encoded once; every question's own tail then runs
// causally against that one cached prefix. Same tokens and positions as the plain path, so a
// tail row at position t sees every prefix key and the question's tail keys 0..t.
//
// Kernel design (one launch for every question of the request):
//  * Work unit = one KV head g and 384 consecutive "query rows" of that head's group, where
//    the rows are (real tail token, query head of the group) pairs, token-major, over all
//    questions in question order. Padding rows are never computed, and a unit may span
//    question boundaries, so a launch has no ragged-tile waste except at its very end.
//  * Workgroup = 12 wave64, three per SIMD; each wave owns 32 query rows. Every K/V tile
//    brought from L2 feeds all 384 rows, which keeps the L2-to-CU traffic per FLOP low (at
//    256 rows per tile it alone cost a third of the run time), and three waves per SIMD let the
//    hardware overlap one wave's softmax (vector ALU) with the others' matrix work. Every
//    32x32x16 MFMA consumes 1 KiB of LDS fragment data, so the four SIMDs of a CU need
//    128 B/clk at the full MFMA rate, below the ~200 B/clk the LDS sustains for the
//    (bank-conflict-free) access patterns used here.
//  * K/V tiles of 64 keys go straight from global memory into LDS (buffer loads with the LDS
//    destination; no staging registers) in a 4-stage ring worked in pairs: while tiles t and
//    t + 1 are computed, tiles t + 2 and t + 3 load into the other two stages, and one wait
//    plus one workgroup barrier per pair (not per tile) publishes them; waves that run ahead
//    within a pair do not wait for the slowest one at every tile. The buffer descriptor's
//    record count covers exactly the keys that are visible for the tile, so the hardware
//    zero-fills everything past them.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: in the
//    accumulator layout a lane holds one query and 16 keys of each 32-key block, so row max and
//    row sum are lane-local except for one exchange with the partner lane (l ^ 32). The
//    probabilities then feed O^T += V^T P^T from registers as the B operand; the A operand
//    V^T comes from the row-major V tile through ds_read_b64_tr_b16 (LDS transpose reads).
//  * LDS rows are padded (K by 16 bytes, V by 64 bytes) so that the rows one LDS cycle serves
//    start in different banks: the K fragment reads and the V transpose reads are free of bank
//    conflicts, and every fragment address is one base register plus an immediate offset.
//    Each lane of a direct load computes which (row, 16-byte chunk) its fixed LDS slot holds;
//    pad slots load out of range and receive zeros.
//  * Softmax in FP32 on exp2. Q enters the score MFMAs as given; the FP32 score q . k is then
//    multiplied by scale * log2(e), so no rounding beyond the MFMA's own FP32 accumulation comes
//    before the exponential. (Rounding a pre-scaled Q to bf16 instead would move every score by
//    up to 2^-9 of |q| |k| relative, enough to shift the weights of keys with large norms by a
//    few percent.) The main pass gives every row the fixed reference 0: a probability is
//    exp2(c * q . k), so the score chains start from the MFMA's zero accumulator input, no row
//    maximum is taken and the O accumulators are never rescaled.
//    Softmax is invariant under the reference, and FP32 and bf16 keep full relative precision
//    while each row's sum of probabilities stays within 2^-64 .. 2^64; one check per row at the
//    end of the unit catches a row outside it (or an inf or NaN: scores beyond the range of
//    exp2, or all far below 0; extreme inputs only), and the workgroup recomputes exactly: one
//    pass for the exact row maxima, then the normal pass with m fixed at them. Row sums are
//    taken over the bf16-rounded probabilities that the PV product uses (v_dot2 with ones).
//    Nothing a row computes depends on which other rows share its wave.
//  * Prefix tiles first (unmasked except the last partial tile), then the tail tiles of each
//    question the unit touches, masked per lane (same question and key <= position).
//  * Two tile paths. Whole tiles of the main pass take a branch-free path: both 32-key score
//    blocks, then exp2, bf16, row sums and PV, with the next tiles' loads issued between the
//    score MFMAs, which run at raised wave priority so the matrix pipe is fed ahead of other
//    waves' softmax. A whole tile is a full prefix tile, or a tail tile of the wave's one
//    question whose 64 keys all lie at or before every row of the wave (in a long causal tail,
//    such as the prefix's own prefill, nearly all of them). Everything else (tiles that cut the
//    causal diagonal, the last partial prefix tile, every tile of the exact recomputation)
//    takes the general path, one 32-key block at a time.
//  * The request's row tables (valid_start, token_offset) are copied into LDS when the
//    workgroup starts, so every lookup on the way to the first tile is an LDS read.
//  * Output rows go through LDS (two idle stages of the ring, half a row at a time) so that
//    every global store writes 64 x 16 contiguous bytes of whole cache lines; from registers, a
//    store instruction would write 16 bytes into each of 32 rows.
//  * blockIdx -> (KV head, unit) puts the KV head in the low bits, so with 8 KV heads each of
//    the 8 XCDs (dispatch is round-robin over XCDs) streams one head's prefix K/V through its
//    own L2. The rows left for the last round of workgroups are re-cut into smaller units
//    (unit_split) so that that round covers every CU.
//  * Given a caller workspace, when the 384-row units left after the full rounds are few enough
//    that w >= 2 pieces of each fill one round (split_plan), each of them runs instead as w
//    pieces over disjoint runs of prefix tiles, only the last piece walking the tail. The
//    pieces write their FP32 partial sums (O, the row's reference, the row sum) to the
//    workspace, and a merge pass of the same kernel (one workgroup per split unit and head, no
//    matrix work) rescales them to their largest reference and adds them.
//  * Units are dispatched from the last row to the first. A causal row sees one more key than
//    the row before it, so later units carry more work; starting the heaviest first lets the
//    light ones fill in at the end (in a 65536-token causal prefill, 7-9% faster than row
//    order). The re-cut small units then run first, still one per CU.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "blink_internal.h"


namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kThreads = 768;
constexpr int kWaves = 12;
constexpr int kQB = 1;                               // 32-row query blocks per wave
constexpr int kRowsPerWave = 32 * kQB;
constexpr int kRowsPerUnit = kWaves * kRowsPerWave;  // 384
constexpr int kTileKeys = 64;
constexpr int kStages = 4;
constexpr int kMaxGroup = 16;
constexpr int kMaxRequests = BLINK_MAX_REQUESTS;  // prefixes in one grouped launch
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kHeadroom = 64.0f;              // log2 units a row sum may lie from 1
constexpr float kSumLimit = 0x1p64f;            // 2^kHeadroom: largest row sum a pass accepts
constexpr float kSumFloor = 0x1p-64f;           // 2^-kHeadroom: smallest row sum a pass accepts
static_assert(kSumLimit == 0x1p64f && kSumFloor == 0x1p-64f && kHeadroom == 64.0f,
              "the row-sum check is 2^-kHeadroom .. 2^kHeadroom");
constexpr uint32_t kBufferFlags = 0x00020000u;  // gfx9 buffer resource word 3 (32-bit data)

constexpr int kWaitFlags = 0xF70;               // s_waitcnt with expcnt/lgkmcnt at their max

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
  int64_t prefix_rows;  // rows of the prefix K/V buffers (every request's prefix)
  int hq;
  int hkv;
  int group;
  float scale_log2;
  int64_t full_units;  // per KV head: units [0, full_units) hold kRowsPerUnit rows each,
  int small_rows;      // later units small_rows each (see unit_split)
  int64_t n_units;     // per KV head
  // Requests of the launch: 1 for blink_prefix_tail_attention (units as above). A grouped
  // launch gives each request its own units (no unit spans two requests, so each unit has
  // exactly one prefix): request r holds questions [req_first[r], req_first[r+1]), units
  // [req_unit[r], req_unit[r+1]) and prefix rows [req_pstart[r], req_pstart[r] + req_plen[r]).
  // Its first req_full[r] units hold kRowsPerUnit rows each, the later ones req_small[r] rows
  // each (see grouped_split).
  // Key split of a single-request launch (split_ways >= 2): units [split_first, n_units) per
  // KV head are pieces. Piece p = unit - split_first works on the rows of base unit
  // b = p / split_ways (kRowsPerUnit rows from split_row0 + b * kRowsPerUnit) over prefix tiles
  // [(p % split_ways) * split_tiles, + split_tiles); only the last piece of a base unit walks
  // the tail keys. Pieces write their unnormalised sums to `part` (kPartFloats floats per lane
  // of each wave, per piece and KV head); the merge pass (merge = 1, one workgroup per base
  // unit and KV head) adds a base unit's pieces and stores its rows.
  int64_t split_first;
  int split_ways;
  int split_tiles;
  int64_t split_row0;
  float *part;
  int merge;
  int n_req;
  int req_first[kMaxRequests + 1];
  int64_t req_unit[kMaxRequests + 1];
  int64_t req_pstart[kMaxRequests];
  int req_plen[kMaxRequests];
  int req_full[kMaxRequests];
  int req_small[kMaxRequests];
};

template <int D>
struct Layout {
  static constexpr int KRS = D * 2 + 16;               // K row stride in LDS (bytes)
  static constexpr int VRS = D * 2 + 64;               // V row stride in LDS (bytes)
  static constexpr int KBYTES = kTileKeys * KRS;       // multiple of 1 KiB for D = 64, 128
  static constexpr int VBYTES = kTileKeys * VRS;
  static constexpr int KINST = KBYTES / 1024;          // 1 KiB direct-load instructions
  static constexpr int VINST = VBYTES / 1024;
  // Instruction i of a tile is issued by wave i % kWaves: every wave issues FULL loads, the
  // first EXTRA waves one more.
  static constexpr int TOTAL = KINST + VINST;
  static constexpr int FULL = TOTAL / kWaves;
  static constexpr int EXTRA = TOTAL % kWaves;
  static constexpr int PER_WAVE = FULL + (EXTRA > 0);
  static_assert(KBYTES % 1024 == 0 && VBYTES % 1024 == 0, "tile must be whole KiB");
};

// The request's row tables, copied into LDS when the workgroup starts: every later lookup
// (which question a row belongs to, where its tail starts) is then an LDS read, not a round
// trip to memory on the way to the first tile.
struct Tables {
  int32_t start[BLINK_MAX_QUESTIONS + 1];  // valid_start: first real-token index of each question
  int64_t toff[BLINK_MAX_QUESTIONS];       // token_offset: first packed row of each question
};

template <int D>
struct Smem {
  __attribute__((aligned(16))) char k[kStages][Layout<D>::KBYTES];
  __attribute__((aligned(16))) char v[kStages][Layout<D>::VBYTES];
  Tables tab;
  int overflow;  // some row of the workgroup ended with a sum of probabilities out of range
};

// Waits until this wave's tile loads have all landed. They are the only vector memory
// operations of the tile loop, so a zero vector-memory count means exactly that.
__device__ inline void wait_tile_loads() { __builtin_amdgcn_s_waitcnt(kWaitFlags); }

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

__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ inline int64_t uniform64(int64_t x) {
  const uint64_t u = uint64_t(x);
  return int64_t(uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(u))))) |
                 (uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(u >> 32))))) << 32));
}

// Workgroup barrier that orders LDS only: global stores issued before it are not waited for.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
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


// Source of one 64-key tile: keys [kstart, kstart + 64) of the prefix (q < 0) or of question
// q's tail (rows rowbase + key of k_tail / v_tail), visible below klimit.
struct TileSrc {
  int64_t rowbase;
  int kstart;
  int klimit;
  int q;  // -1 for the prefix
  bool valid;
};

// Global byte offset (from the tile's first row) of the 16 bytes that land in LDS byte `off`
// of a tile with row stride RS; pad slots get an offset past every buffer (hardware zeros).
template <int D, int RS>
__device__ inline int slot_source(int off, int64_t stride) {
  const int row = off / RS, chunk = (off % RS) / 16;
  return chunk < D / 8 ? int(row * stride * 2) + chunk * 16 : 0x7ffffff0;
}

// Per-lane source offsets of this wave's direct loads (identical for every tile): load i of
// wave w is instruction w + kWaves * i of the tile (K instructions first, then V).
template <int D>
struct LoadPlan {
  int voff[Layout<D>::PER_WAVE];
};

template <int D>
__device__ inline LoadPlan<D> make_load_plan(const Args &a, int wave, int lane) {
  using L = Layout<D>;
  const int64_t stride = int64_t(a.hkv) * D;
  LoadPlan<D> plan;
#pragma unroll
  for (int i = 0; i < L::PER_WAVE; ++i) {
    const int inst = wave + kWaves * i;
    const int koff = inst * 1024 + lane * 16;
    const int voff = (inst - L::KINST) * 1024 + lane * 16;
    plan.voff[i] = inst < L::KINST ? slot_source<D, L::KRS>(koff, stride)
                                   : slot_source<D, L::VRS>(voff, stride);
  }
  return plan;
}

// Buffer descriptors of one tile's K and V rows; their record counts end at the last visible
// key (and at the tensor's end), so every load past them reads zeros. An invalid tile gets
// empty descriptors: its loads write zeros into a free stage.
struct TileRsrc {
  __amdgpu_buffer_rsrc_t k, v;
};

template <int D>
__device__ inline TileRsrc tile_rsrc(const Args &a, int g, const TileSrc &s) {
  const bool pre = s.q < 0;
  const int64_t rowcount = pre ? a.prefix_rows : a.t_pad;  // rows that exist
  const int64_t row0 = s.rowbase + s.kstart;
  const int64_t stride = int64_t(a.hkv) * D;  // elements between consecutive rows
  int64_t nkeys = min(int64_t(kTileKeys), int64_t(s.klimit - s.kstart));
  nkeys = min(nkeys, rowcount - row0);
  const bool any = s.valid && nkeys > 0 && row0 >= 0;
  const int nbytes = any ? int(((nkeys - 1) * stride + D) * 2) : 0;
  const int64_t first = any ? row0 * stride + int64_t(g) * D : 0;
  const uint16_t *kb = !s.valid ? nullptr : pre ? a.k_pre : a.k_tail;
  const uint16_t *vb = !s.valid ? nullptr : pre ? a.v_pre : a.v_tail;
  return TileRsrc{
      __builtin_amdgcn_make_buffer_rsrc((void *)(kb + first), (short)0, nbytes, kBufferFlags),
      __builtin_amdgcn_make_buffer_rsrc((void *)(vb + first), (short)0, nbytes, kBufferFlags)};
}

// Issues load i (a plan entry; the caller keeps i < FULL, or i == FULL only for the first
// EXTRA waves) of one tile into the given stage.
template <int D>
__device__ inline void issue_load(const TileRsrc &r, char *lds_k, char *lds_v, int wave,
                                  const LoadPlan<D> &plan, int i) {
  using L = Layout<D>;
  const int inst = wave + kWaves * i;  // uniform
  const bool is_k = inst < L::KINST;
  char *dst = is_k ? lds_k + inst * 1024 : lds_v + (inst - L::KINST) * 1024;
  // The load is written in asm so that the compiler does not track it: tracked, it makes every
  // later LDS read of the wave (the V transpose reads of the tile being computed) wait for this
  // load, which only the next pair of tiles needs. The loads carry no output registers; the
  // explicit wait and barrier at the end of each pair (wait_tile_loads) publish them. The
  // s_nop keeps one wait state between the write of m0 and the load that reads it.
  const uint32_t lds = uint32_t(reinterpret_cast<uintptr_t>((lds_char *)dst));
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(plan.voff[i]), "s"(is_k ? r.k : r.v), "{m0}"(lds));
}

// All of this wave's loads of one tile.
template <int D>
__device__ inline void load_tile_async(const TileRsrc &r, char *lds_k, char *lds_v, int wave,
                                       const LoadPlan<D> &plan) {
  using L = Layout<D>;
#pragma unroll
  for (int i = 0; i < L::FULL; ++i) issue_load<D>(r, lds_k, lds_v, wave, plan, i);
  if (L::EXTRA > 0 && wave < L::EXTRA) issue_load<D>(r, lds_k, lds_v, wave, plan, L::FULL);
}

struct RowState {
  float m;  // running max in log2 units (-inf before any visible key)
  float l;  // this lane's partial sum of probabilities (the partner lane holds the rest)
};

// V^T fragment for one 16-key PV step starting at key0 and 32 dims of block db:
// lane (d = l % 32, half h) gets keys key0 + 4h + {0..3} and key0 + 8 + 4h + {0..3}.
// `vlane` is this lane's part of the address: row 4h + r, dims 16 * (grp & 1) + 4 * cc
// (grp = lane / 16, r = (lane % 16) / 4, cc = lane % 4).
template <int D>
__device__ inline int v_lane_offset(int lane) {
  const int grp = lane >> 4, i = lane & 15, r = i >> 2, cc = i & 3, h = lane >> 5;
  return (4 * h + r) * Layout<D>::VRS + (16 * (grp & 1) + 4 * cc) * 2;
}
template <int D>
__device__ inline bf16x8 read_v(const char *vt, int vlane, int key0, int db) {
  lds_char *base = (lds_char *)vt + vlane + key0 * Layout<D>::VRS + db * 64;
  const bf16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)base);
  const bf16x4 t1 =
      __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(base + 8 * Layout<D>::VRS));
  return bf16x8{t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
}

// Probabilities of one 16-value accumulator slice into bf16 B operands, with row-sum update.
// Probabilities of 16 raw scores (q . k, FP32): p = exp2(s * c - m), c = scale * log2(e) and m
// the row's reference in log2 units (0 for ZERO), rounded to bf16 for the PV product; their sum
// is added into l.
template <bool ZERO>
__device__ inline void probs_to_bf16(const f32x16 &s, float c, float m, bf16x8 (&pb)[2],
                                     float &l) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  auto arg = [&](float x) { return ZERO ? x * c : __builtin_fmaf(x, c, -m); };
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const bf16x2 p2 = {(__bf16)__builtin_amdgcn_exp2f(arg(s[8 * h + e])),
                         (__bf16)__builtin_amdgcn_exp2f(arg(s[8 * h + e + 1]))};
      pb[h][e] = p2[0];
      pb[h][e + 1] = p2[1];
      l = __builtin_amdgcn_fdot2_f32_bf16(p2, ones, l, false);
    }
  }
}

// O^T += V^T P^T over one 32-key sub-tile (two 16-key MFMA steps per 32-dim block).
template <int D>
__device__ inline void pv_product(const char *vt, int key0, const bf16x8 (&pb)[kQB][2],
                                  f32x16 (&o)[kQB][D / 32]) {
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const bf16x8 vf = read_v<D>(vt, 0, key0 + 16 * c, db);
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb)
        o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[qb][c], o[qb][db], 0, 0, 0);
    }
  }
}

// One 32-key sub-tile for one wave: S^T = K Q^T, softmax terms, O^T += V^T P^T.
// kt/vt point at the tile plus this lane's part of the fragment addresses; c = scale * log2(e).
// lim[qb]: largest visible key index within the sub-tile minus 4 * (lane >> 5); keys above it
// are masked (used only when `masked`).
// MAX_ONLY: only the row maxima are taken (scores times c, log2 units) for the exact pass.
// ZERO: every row's reference is 0 (the main pass); otherwise each row's reference is its m.
// The score chains start from the MFMA's zero accumulator input either way.
template <int D, bool MAX_ONLY, bool ZERO>
__device__ inline void compute_subtile(const char *kt, const char *vt, int key0,
                                       bf16x8 (&qf)[kQB][D / 16],
                                       f32x16 (&o)[kQB][D / 32], RowState (&rs)[kQB],
                                       bool masked, const int (&lim)[kQB], float c) {
  f32x16 s[kQB];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const bf16x8 kf = as_bf16x8(
        *reinterpret_cast<const u32x4 *>(kt + key0 * Layout<D>::KRS + ks * 32));
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
      s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          kf, qf[qb][ks], ks == 0 ? f32x16{} : s[qb], 0, 0, 0);
  }

  if (masked) {  // uniform: tail tiles and the last partial prefix tile
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = 8 * (v >> 2) + (v & 3);
        s[qb][v] = (key <= lim[qb]) ? s[qb][v] : -INFINITY;
      }
    }
  }
  if (MAX_ONLY) {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      float m = s[qb][0];
#pragma unroll
      for (int v = 1; v < 16; ++v) m = fmaxf(m, s[qb][v]);
      rs[qb].m = fmaxf(rs[qb].m, c * pair_max(m));  // c > 0
    }
    return;
  }
  // No row maxima: every row's reference is fixed for the pass (0, or its exact maximum in the
  // recomputation), and a row sum out of range is caught at the end of the unit.
  bf16x8 pb[kQB][2];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) probs_to_bf16<ZERO>(s[qb], c, rs[qb].m, pb[qb], rs[qb].l);
  pv_product<D>(vt, key0, pb, o);
}

// A full, unmasked 64-key tile in the main pass, where every row's reference is 0: the score
// chains start from the MFMA's zero accumulator input, so no vector instruction sets them up (on
// this chip the matrix pipe and the vector ALU share each SIMD's issue, so vector instructions
// taken out of the tile are time taken out of it). Both 32-key score blocks are computed first,
// all in one basic block, so one block's softmax (vector ALU) can be interleaved with the other
// block's matrix products.
// The next tile's FULL regular loads are issued between the score MFMAs, one per 4 MFMAs, so
// the waves of a CU do not all queue their loads at once after the barrier.
template <int D>
__device__ inline void compute_tile_fast(const char *kt, const char *vt,
                                         bf16x8 (&qf)[kQB][D / 16], f32x16 (&o)[kQB][D / 32],
                                         RowState (&rs)[kQB], const TileRsrc &load_src,
                                         char *next_k, char *next_v, int wave,
                                         const LoadPlan<D> &plan, float c) {
  constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100;
  constexpr int kSteps = 2 * (D / 16);  // score MFMA steps (each kQB MFMAs) in the tile
  // Raised wave priority for the score MFMAs: the SIMD issues this wave's matrix burst ahead
  // of the other waves' softmax vector work, so the matrix pipe stays fed (measured: +3 to +6%).
  __builtin_amdgcn_s_setprio(1);
  f32x16 s[2][kQB];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8 kf = as_bf16x8(
          *reinterpret_cast<const u32x4 *>(kt + 32 * sub * Layout<D>::KRS + ks * 32));
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb)
        s[sub][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            kf, qf[qb][ks], ks == 0 ? f32x16{} : s[sub][qb], 0, 0, 0);
      const int step = sub * (D / 16) + ks;
      if (step % 4 == 3 && step / 4 < Layout<D>::FULL)
        issue_load<D>(load_src, next_k, next_v, wave, plan, step / 4);
    }
  }
  __builtin_amdgcn_s_setprio(0);
  // Keep that order: K fragment read, its MFMAs, and a tile load after every fourth step.
#pragma unroll
  for (int step = 0; step < kSteps; ++step) {
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, kQB, 0);
    if (step % 4 == 3 && step / 4 < Layout<D>::FULL)
      __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
  }
  // No row maximum here: a row whose probabilities leave the representable range shows up in
  // its row sum, which the kernel checks once at the end of the unit.
  bf16x8 pb[2][kQB][2];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
      probs_to_bf16<true>(s[sub][qb], c, 0.0f, pb[sub][qb], rs[qb].l);
    pv_product<D>(vt, 32 * sub, pb[sub], o);
  }
}

struct Unit {
  int qa, qz, posz;  // questions touched by the workgroup; last row's position in qz
  int plen;          // the unit's prefix: rows [pstart, pstart + plen) of the prefix K/V
  int64_t pstart;
  int kbeg, kend;    // the prefix keys the unit walks: [kbeg, kend) (0, plen unless split)
  bool tail;         // the unit walks its questions' tail keys (all but non-last pieces)
};

__device__ inline TileSrc tail_from(const Args &a, const Tables &tab, const Unit &u, int q) {
  TileSrc s{};
  s.valid = false;
  for (; q <= u.qz; ++q) {
    const int nq = uniform(tab.start[q + 1] - tab.start[q]);
    const int limit = (q == u.qz) ? u.posz + 1 : nq;
    // A malformed table cannot make the loop run past the context length.
    if (limit > 0 && limit <= nq && nq <= BLINK_MAX_INPUT_TOKENS) {
      s.rowbase = uniform64(tab.toff[q]);
      s.kstart = 0;
      s.klimit = limit;
      s.q = q;
      s.valid = true;
      return s;
    }
  }
  return s;
}

__device__ inline TileSrc first_tile(const Args &a, const Tables &tab, const Unit &u) {
  if (u.kbeg < u.kend) {
    TileSrc s{};
    s.rowbase = u.pstart;
    s.kstart = u.kbeg;
    s.klimit = u.kend;
    s.q = -1;
    s.valid = true;
    return s;
  }
  if (!u.tail) {
    TileSrc s{};
    s.valid = false;
    return s;
  }
  return tail_from(a, tab, u, u.qa);
}

__device__ inline TileSrc next_tile(const Args &a, const Tables &tab, const Unit &u,
                                    TileSrc s) {
  if (!s.valid) return s;
  s.kstart += kTileKeys;
  if (s.kstart < s.klimit) return s;
  if (s.q < 0 && !u.tail) {
    s.valid = false;
    return s;
  }
  return tail_from(a, tab, u, s.q < 0 ? u.qa : s.q + 1);
}

struct RowTables {
  const int (&rq)[kQB];    // question of each of this lane's rows (-1 if not a real row)
  const int (&rpos)[kQB];  // tail position of each row
};
struct WaveSpan {
  bool active;     // the wave has at least one real row
  int qa, qz, posz;  // questions the wave's rows touch; last row's position in qz
  int posa;          // first row's position in qa
};

template <int D>
// Clears the accumulators; `m`: the rows' reference for the pass (0 for the main pass, -inf
// before the exact maxima are taken), or NaN to keep the references as they are.
__device__ inline void init_rows(f32x16 (&o)[kQB][D / 32], RowState (&rs)[kQB], float m) {
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[qb][db] = f32x16{};
    rs[qb].l = 0.f;
    if (!isnan(m)) rs[qb].m = m;
  }
}

// All tiles of the unit through the 4-stage LDS ring; max_only collects exact row maxima.
// Issues the ring's first pair of tiles (stages 0 and 1).
template <int D>
__device__ inline void start_tiles(const Args &a, Smem<D> &sm, const Unit &u, int g,
                                   const TileSrc &first, int wave, const LoadPlan<D> &plan) {
  __builtin_amdgcn_sched_barrier(0);
  load_tile_async<D>(tile_rsrc<D>(a, g, first), sm.k[0], sm.v[0], wave, plan);
  load_tile_async<D>(tile_rsrc<D>(a, g, next_tile(a, sm.tab, u, first)), sm.k[1], sm.v[1],
                     wave, plan);
  __builtin_amdgcn_sched_barrier(0);
}

// `started`: start_tiles has been called (its loads may still be in flight).
template <int D>
__device__ inline void run_tiles(const Args &a, Smem<D> &sm, const Unit &u, int g,
                                 const TileSrc &first, const RowTables &rt, const WaveSpan &ws,
                                 int klane, int vlane, int wave, int lane,
                                 const LoadPlan<D> &plan, bf16x8 (&qf)[kQB][D / 16],
                                 f32x16 (&o)[kQB][D / 32], RowState (&rs)[kQB], bool max_only,
                                 bool zero_ref, bool started) {
  const int half = lane >> 5;
  // Tiles go in pairs (2t, 2t + 1) -> stages (0, 1) or (2, 3). While a pair is computed, the
  // next pair is loaded into the other two stages; one wait for all loads plus one barrier at
  // the end of each pair makes the next pair visible and frees this one's stages.
  static_assert(kStages == 4, "pairs of tiles in a 4-stage ring");
  TileSrc cur = first;
  TileSrc nxt = next_tile(a, sm.tab, u, cur);  // tile t + 1
  if (!started) start_tiles<D>(a, sm, u, g, first, wave, plan);
  wait_tile_loads();
  __syncthreads();
  TileSrc nxt2 = next_tile(a, sm.tab, u, nxt);  // tile t + 2: the next pair's first
  int stage = 0;
  while (true) {
    // Tile t + 2 goes into the stage of tile t - 2 (the previous pair, done before the barrier).
    const TileSrc after = nxt2;
    const int stage2 = stage ^ 2;
    const TileRsrc ra = tile_rsrc<D>(a, g, after);
    __builtin_amdgcn_sched_barrier(0);
    if (Layout<D>::EXTRA > 0 && wave < Layout<D>::EXTRA)
      issue_load<D>(ra, sm.k[stage2], sm.v[stage2], wave, plan, Layout<D>::FULL);

    bool active = ws.active;
    if (cur.q >= 0)
      active = active && cur.q >= ws.qa && cur.q <= ws.qz &&
               !(cur.q == ws.qz && cur.kstart > ws.posz);
    // A whole tile: every key visible to every row of the wave (see the two tile paths).
    const bool whole = cur.q < 0 ? cur.kstart + kTileKeys <= cur.klimit
                                 : cur.q == ws.qa && ws.qa == ws.qz &&
                                       cur.kstart + kTileKeys <= ws.posa + 1;
    const bool fast = !max_only && zero_ref && whole;
    if (active && fast) {
      compute_tile_fast<D>(sm.k[stage] + klane, sm.v[stage] + vlane, qf, o, rs, ra,
                           sm.k[stage2], sm.v[stage2], wave, plan, a.scale_log2);
    } else {
#pragma unroll
      for (int i = 0; i < Layout<D>::FULL; ++i)
        issue_load<D>(ra, sm.k[stage2], sm.v[stage2], wave, plan, i);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (active && !fast) {
      const char *kt = sm.k[stage] + klane;
      const char *vt = sm.v[stage] + vlane;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int base = cur.kstart + 32 * sub;  // first key of the sub-tile
        const bool masked = !(cur.q < 0 && base + 32 <= cur.klimit);
        int lim[kQB];
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
          int last;  // last visible key of this row, relative to the sub-tile start
          if (cur.q < 0)
            last = cur.klimit - 1 - base;  // a prefix tile's klimit ends the unit's prefix keys
          else
            last = (rt.rq[qb] == cur.q) ? rt.rpos[qb] - base : -1;
          last = min(last, 31);
          lim[qb] = last - 4 * half;
        }
        if (max_only)
          compute_subtile<D, true, true>(kt, vt, 32 * sub, qf, o, rs, masked, lim, a.scale_log2);
        else if (zero_ref)
          compute_subtile<D, false, true>(kt, vt, 32 * sub, qf, o, rs, masked, lim, a.scale_log2);
        else
          compute_subtile<D, false, false>(kt, vt, 32 * sub, qf, o, rs, masked, lim,
                                           a.scale_log2);
      }
    }

    __builtin_amdgcn_sched_barrier(0);
    if (stage & 1) {  // end of a pair: the next pair has landed for every wave
      wait_tile_loads();
      __syncthreads();
    }
    if (!nxt.valid) break;
    cur = nxt;
    nxt = nxt2;
    nxt2 = next_tile(a, sm.tab, u, nxt2);
    stage = (stage + 1) & 3;
  }
  // The last loads (zeros for tiles past the end) must land before the stages are reused.
  wait_tile_loads();
  __syncthreads();
}

// A wave's output rows staged in LDS, half a row (D / 2 dims) at a time: bf16 half rows
// padded to RS bytes, then each row's destination (element offset into out, or -1 for a row
// that is not stored). The waves' areas fill two stages of the ring: the K halves of the pair
// first, then its V halves.
template <int D>
struct OutStage {
  static constexpr int RS = D + 16;
  static constexpr int BYTES = kRowsPerWave * RS + kRowsPerWave * 8;
  static constexpr int IN_K = 2 * Layout<D>::KBYTES / BYTES;  // areas in the pair's K stages
  static_assert(RS % 16 == 0 && BYTES % 16 == 0, "16-byte LDS reads");
  static_assert(IN_K + 2 * Layout<D>::VBYTES / BYTES >= kWaves,
                "every wave's half rows fit in two stages of the K/V ring");
};

// This wave's staging area in the stage pair (pair, pair + 1), pair = 0 or 2.
template <int D>
__device__ inline char *out_stage(Smem<D> &sm, int pair, int wave) {
  using S = OutStage<D>;
  return wave < S::IN_K ? &sm.k[pair][0] + wave * S::BYTES
                        : &sm.v[pair][0] + (wave - S::IN_K) * S::BYTES;
}

// Normalise the wave's rows to bf16 and store them. In the accumulator layout a lane holds
// 8-byte pieces of one row, so storing from registers makes every instruction write 16 bytes
// into each of 32 rows. The rows go through LDS instead (`stage`, this wave's area in two idle
// stages of the K/V ring), half a row at a time, so that each global store writes 64 x 16
// bytes of whole 128-byte lines: eight half rows of 128 bytes (D = 128).
template <int D>
__device__ inline void store_rows(const Args &a, char *stage, const f32x16 (&o)[kQB][D / 32],
                                  const RowState (&rs)[kQB], const bool (&rvalid)[kQB],
                                  const int64_t (&rtok)[kQB], const int (&rhead)[kQB],
                                  int lane) {
  using S = OutStage<D>;
  const int col = lane & 31, half = lane >> 5;
  int64_t *dst = reinterpret_cast<int64_t *>(stage + kRowsPerWave * S::RS);
  float inv[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const float l = pair_sum(rs[qb].l);
    inv[qb] = l > 0.f ? 1.0f / l : 0.f;
    if (half == 0)
      dst[32 * qb + col] = rvalid[qb] ? (rtok[qb] * a.hq + rhead[qb]) * D : int64_t(-1);
  }
  constexpr int kChunks = D / 16;  // 16-byte chunks per half row
#pragma unroll
  for (int part = 0; part < 2; ++part) {  // dims [part * D / 2, (part + 1) * D / 2)
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      char *lrow = stage + (32 * qb + col) * S::RS + 8 * half;  // dims 4 * half + 8 * grp + 32 * db
#pragma unroll
      for (int db = part * D / 64; db < (part + 1) * D / 64; ++db) {
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          u32x2 packed;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const __bf16 x0 = (__bf16)(o[qb][db][4 * grp + 2 * j] * inv[qb]);
            const __bf16 x1 = (__bf16)(o[qb][db][4 * grp + 2 * j + 1] * inv[qb]);
            packed[j] = uint32_t(__builtin_bit_cast(uint16_t, x0)) |
                        (uint32_t(__builtin_bit_cast(uint16_t, x1)) << 16);
          }
          *reinterpret_cast<u32x2 *>(lrow + ((db - part * D / 64) * 32 + 8 * grp) * 2) = packed;
        }
      }
    }
    // Lanes read what other lanes of the same wave wrote (and then overwrite what they read):
    // one wave's LDS operations complete in order, so only the compiler has to keep them so.
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
    for (int i = 0; i < kRowsPerWave * kChunks / 64; ++i) {
      const int k = lane + 64 * i, row = k / kChunks, chunk = k % kChunks;
      const int64_t d = dst[row];
      const u32x4 v = *reinterpret_cast<const u32x4 *>(stage + row * S::RS + chunk * 16);
      // Non-temporal: the kernel never reads its output back, and streaming it past the
      // caches leaves them clean for whatever runs next (the readout after a large request
      // otherwise starts by writing back hundreds of MB of dirty lines).
      if (d >= 0)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(a.out + d + part * D / 2 +
                                                                 chunk * 8));
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  }
}

// Floats one lane of a key-split piece leaves for the merge: its D/2 sums of O (the accumulator
// registers, in their MFMA layout), its row's reference m and its part l of the row sum.
__host__ __device__ constexpr int part_floats(int d) { return d / 2 + 2; }

// This wave's partial sums of a piece, register by register, lanes contiguous (each register is
// one 256-byte store of the wave): slot (piece, KV head g, wave) of `part`.
template <int D>
__device__ inline void write_partials(const Args &a, int64_t piece, int g, int wave, int lane,
                                      const f32x16 (&o)[kQB][D / 32], const RowState (&rs)[kQB]) {
  float *base =
      a.part + ((piece * a.hkv + g) * kWaves + wave) * int64_t(part_floats(D)) * 64 + lane;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) base[(db * 16 + v) * 64] = o[0][db][v];
  base[(D / 2) * 64] = rs[0].m;
  base[(D / 2 + 1) * 64] = rs[0].l;
}

// The merge pass for this wave's rows of base unit `bu`: the pieces' sums, each scaled by
// 2^(m_j - M) for the largest reference M (all 0 unless a piece recomputed exactly), added in
// piece order into o and rs (rs.l stays this lane's part of the row sum).
template <int D>
__device__ inline void merge_partials(const Args &a, int64_t bu, int g, int wave, int lane,
                                      f32x16 (&o)[kQB][D / 32], RowState (&rs)[kQB]) {
  const int ways = a.split_ways;
  const int64_t stride = int64_t(part_floats(D)) * 64;
  auto slot = [&](int j) {
    return a.part + (((bu * ways + j) * a.hkv + g) * kWaves + wave) * stride + lane;
  };
  float m = -INFINITY;
  for (int j = 0; j < ways; ++j) m = fmaxf(m, slot(j)[(D / 2) * 64]);
  init_rows<D>(o, rs, m);
  for (int j = 0; j < ways; ++j) {
    const float *p = slot(j);
    const float f = __builtin_amdgcn_exp2f(p[(D / 2) * 64] - m);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[0][db][v] += f * p[(db * 16 + v) * 64];
    rs[0].l += f * p[(D / 2 + 1) * 64];
  }
}

// One unit of work of KV head g (the row tables are in LDS and the overflow flag is clear).
// Every exit is uniform across the workgroup. (Kept as its own function: so compiled, the
// kernel measured 2% faster at the prefix workloads than with this body written inline.)
template <int D>
__device__ __forceinline__ void attention_unit(const Args &a, Smem<D> &sm, int64_t unit,
                                               int g) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);  // known to the compiler as wave-uniform (scalar)
  const int col = lane & 31, half = lane >> 5;
  const int G = a.group;
  (void)tid;
  const int64_t valid_total = min(int64_t(uniform(sm.tab.start[a.n])), a.total_valid);
  const int64_t R = valid_total * G;
  Unit u;
  int64_t row0, row_end;
  int64_t piece = -1;  // this workgroup's key-split piece, if it is one
  u.kbeg = 0;
  u.tail = true;
  if (a.merge) {  // `unit` is a split base unit; its pieces have run
    row0 = a.split_row0 + unit * kRowsPerUnit;
    row_end = row0 + kRowsPerUnit;
    u.plen = a.req_plen[0];
    u.pstart = a.req_pstart[0];
  } else if (a.n_req == 1) {
    if (unit >= a.split_first) {
      piece = unit - a.split_first;
      const int64_t bu = piece / a.split_ways;
      const int j = int(piece % a.split_ways);
      row0 = a.split_row0 + bu * kRowsPerUnit;
      row_end = row0 + kRowsPerUnit;
      u.kbeg = min(j * a.split_tiles * kTileKeys, a.req_plen[0]);
      u.tail = j == a.split_ways - 1;
    } else {
      row0 = unit < a.full_units
                 ? unit * kRowsPerUnit
                 : a.full_units * kRowsPerUnit + (unit - a.full_units) * a.small_rows;
      row_end = row0 + (unit < a.full_units ? int64_t(kRowsPerUnit) : int64_t(a.small_rows));
    }
    u.plen = a.req_plen[0];
    u.pstart = a.req_pstart[0];
  } else {
    int r = 0;  // the unit's request: the last r with req_unit[r] <= unit
    while (r + 1 < a.n_req && a.req_unit[r + 1] <= unit) ++r;
    const int64_t rows_end = int64_t(uniform(sm.tab.start[a.req_first[r + 1]])) * G;
    const int64_t k = unit - a.req_unit[r], full = a.req_full[r], small = a.req_small[r];
    row0 = int64_t(uniform(sm.tab.start[a.req_first[r]])) * G +
           (k < full ? k * kRowsPerUnit : full * kRowsPerUnit + (k - full) * small);
    row_end = min(rows_end, row0 + (k < full ? int64_t(kRowsPerUnit) : small));
    u.plen = a.req_plen[r];
    u.pstart = a.req_pstart[r];
  }
  u.kend = u.plen;
  if (piece >= 0)
    u.kend = min((int(piece % a.split_ways) + 1) * a.split_tiles * kTileKeys, u.plen);
  row_end = min(R, row_end);
  if (row0 < 0 || row0 >= row_end) return;  // uniform across the workgroup

  // Questions touched by the workgroup and by this wave.
  {
    const int64_t c0 = row0 / G, cz = (row_end - 1) / G;
    u.qa = uniform(find_question(sm.tab.start, a.n, c0));
    u.qz = uniform(find_question(sm.tab.start, a.n, cz));
    u.posz = uniform(int(cz - sm.tab.start[u.qz]));
  }
  const int64_t wr0 = row0 + wave * kRowsPerWave;
  const bool wave_active = wr0 < row_end;
  int wqa = 0, wqz = -1, wposz = -1, wposa = 0;
  if (wave_active) {
    const int64_t c0 = wr0 / G, cz = (min(wr0 + kRowsPerWave, row_end) - 1) / G;
    wqa = uniform(find_question(sm.tab.start, a.n, c0));
    wposa = uniform(int(c0 - sm.tab.start[wqa]));
    wqz = uniform(find_question(sm.tab.start, a.n, cz));
    wposz = uniform(int(cz - sm.tab.start[wqz]));
  }

  // The ring's first pair of K/V tiles goes out before the query rows are fetched, so the
  // two latencies overlap.
  const TileSrc first = first_tile(a, sm.tab, u);
  if (!first.valid && !a.merge) return;  // uniform: nothing visible (not for a valid table)
  const LoadPlan<D> plan = make_load_plan<D>(a, wave, lane);
  if (!a.merge) start_tiles<D>(a, sm, u, g, first, wave, plan);

  // This lane's query rows, as given (the scale is applied to the FP32 scores).
  bool rvalid[kQB];
  int rq[kQB], rpos[kQB], rhead[kQB];
  int64_t rtok[kQB];
  bf16x8 qf[kQB][D / 16];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int64_t r = row0 + wave * kRowsPerWave + qb * 32 + col;
    rvalid[qb] = r < row_end;
    const int64_t c = rvalid[qb] ? r / G : 0;
    const int hl = int(r % G);
    const int q = find_question(sm.tab.start, a.n, c);
    const int nq = sm.tab.start[q + 1] - sm.tab.start[q];
    const int pos = int(c - sm.tab.start[q]);
    rvalid[qb] = rvalid[qb] && pos >= 0 && pos < nq;
    const int64_t tok = sm.tab.toff[q] + pos;
    rvalid[qb] = rvalid[qb] && tok >= 0 && tok < a.t_pad;
    rq[qb] = rvalid[qb] ? q : -1;
    rpos[qb] = pos;
    rtok[qb] = tok;
    rhead[qb] = g * G + hl;
    const uint16_t *qrow = a.q + ((rvalid[qb] ? tok : 0) * a.hq + rhead[qb]) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (rvalid[qb] && !a.merge) v = *reinterpret_cast<const u32x4 *>(qrow + ks * 16);
      qf[qb][ks] = as_bf16x8(v);
    }
  }

  // Lane parts of the fragment addresses: K rows col (+ key0), chunk half (+ 2 ks).
  const int klane = col * Layout<D>::KRS + 16 * half;
  const int vlane = v_lane_offset<D>(lane);

  const RowTables rt{rq, rpos};
  // This wave's area in stages 0 and 1 for staging its output rows (used after the tiles).
  char *ostage = out_stage<D>(sm, 0, wave);
  const WaveSpan ws{wave_active, wqa, wqz, wposz, wposa};
  f32x16 o[kQB][D / 32];
  RowState rs[kQB];
  if (a.merge) {
    merge_partials<D>(a, unit, g, wave, lane, o, rs);
    store_rows<D>(a, ostage, o, rs, rvalid, rtok, rhead, lane);
    return;
  }
  init_rows<D>(o, rs, 0.0f);
  run_tiles<D>(a, sm, u, g, first, rt, ws, klane, vlane, wave, lane, plan, qf, o, rs, false,
               true, true);
  // A probability above 2^kHeadroom (or an inf or NaN) leaves its row sum above 2^kHeadroom; a
  // row whose scores all lie far below 0 leaves it below 2^-kHeadroom.
  bool over = false;
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const float l = pair_sum(rs[qb].l);
    over |= rvalid[qb] && !(l <= kSumLimit && l >= kSumFloor);
  }
  if (piece >= 0)
    write_partials<D>(a, piece, g, wave, lane, o, rs);
  else
    store_rows<D>(a, ostage, o, rs, rvalid, rtok, rhead, lane);
  // Did any wave of the workgroup overflow? (The flag was cleared before the first barrier.)
  // The barrier orders only the flag in LDS, so the workgroup does not wait for its stores to
  // complete: it ends, and the next one starts on this CU, while they drain.
  if (__builtin_amdgcn_ballot_w64(over)) sm.overflow = 1;
  lds_barrier();
  if (sm.overflow) {
    // Extreme inputs only: exact row maxima first, then the normal pass with those references;
    // its rows overwrite the ones just stored. (The accumulators are reused: the stored values
    // are dead, so nothing has to be merged.)
    init_rows<D>(o, rs, -INFINITY);
    run_tiles<D>(a, sm, u, g, first, rt, ws, klane, vlane, wave, lane, plan, qf, o, rs, true,
                 false, false);
    init_rows<D>(o, rs, __builtin_nanf(""));
    run_tiles<D>(a, sm, u, g, first, rt, ws, klane, vlane, wave, lane, plan, qf, o, rs, false,
                 false, false);
    if (piece >= 0)
      write_partials<D>(a, piece, g, wave, lane, o, rs);
    else
      store_rows<D>(a, ostage, o, rs, rvalid, rtok, rhead, lane);
  }
}

// The attention kernel: workgroup blockIdx takes KV head blockIdx % H_kv and unit
// n_units - 1 - blockIdx / H_kv of that head (heaviest first).
template <int D>
__global__ __launch_bounds__(kThreads, 1) void prefix_tail_attention_kernel(Args a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  __shared__ Smem<D> sm;
  const int tid = threadIdx.x;
  const int g = int(blockIdx.x % unsigned(a.hkv));
  const int64_t unit = a.n_units - 1 - int64_t(blockIdx.x / unsigned(a.hkv));
  if (unit < 0) return;  // uniform; the grid holds exactly n_units units per head

  for (int i = tid; i <= a.n; i += kThreads) {
    sm.tab.start[i] = a.valid_start[i];
    if (i < a.n) sm.tab.toff[i] = a.token_offset[i];
  }
  if (tid == 0) sm.overflow = 0;
  __syncthreads();
  attention_unit<D>(a, sm, unit, g);
#endif
}

// Work split per KV head (`rows` query rows each) over `cus` compute units, one workgroup per
// CU at a time. Uniform units of kRowsPerUnit rows leave the last round of workgroups partly
// empty, yet it lasts a full unit's time. Instead the rows left after the full rounds are
// spread over every CU of the last round, in units whose waves give each SIMD fewer waves
// (multiples of 4 waves), so that round ends sooner; a launch of less than one round is cut
// the same way from the start. Returns the units per head.
inline int64_t unit_split(int64_t rows, int hkv, int cus, int64_t &full_units, int &small_rows) {
  const int64_t units = (rows + kRowsPerUnit - 1) / kRowsPerUnit;
  full_units = units;
  small_rows = kRowsPerUnit;
  const int64_t per_round = cus / hkv;  // units of one head in one round
  const int64_t simd_rows = 4 * kRowsPerWave;  // one wave on each SIMD
  if (per_round < 1) return units;
  if (units * hkv <= cus) {
    // Less than one round: cut the rows into smaller units so that they cover every CU.
    const int64_t want = (rows + per_round - 1) / per_round;
    const int64_t up = max(simd_rows, (want + simd_rows - 1) / simd_rows * simd_rows);
    if (up >= kRowsPerUnit) return units;
    full_units = 0;
    small_rows = int(up);
    return (rows + up - 1) / up;
  }
  const int64_t full = units / per_round * per_round;
  const int64_t rem = rows - full * kRowsPerUnit;
  if (rem <= 0) return units;
  const int64_t small = (rem + per_round - 1) / per_round;
  const int64_t small_up = (small + simd_rows - 1) / simd_rows * simd_rows;
  if (small_up >= kRowsPerUnit) return units;
  full_units = full;
  small_rows = int(small_up);
  return full + (rem + small_up - 1) / small_up;
}

// Key split of the last round (a single request with a prefix, given workspace for the pieces'
// sums). When a head's rows need more than one round of 384-row units and the units left after
// the full rounds would leave CUs idle, each of those R units is cut by prefix keys into
// ways = cus / hkv / R pieces (each a run of whole 64-key tiles, the tail keys with the last
// piece), so the last round is R * ways pieces of full 384-row units, about one per CU, each a
// ways-th of a unit's keys, instead of smaller row units with fewer waves per SIMD; a merge pass
// then adds each unit's pieces. Fills the plan and returns true, or returns false (no split).
struct SplitPlan {
  int64_t full;   // 384-row units per head before the split ones
  int64_t split;  // split base units per head (R)
  int ways;       // pieces per split unit
  int tiles;      // prefix tiles per piece
};

inline bool split_plan(int64_t rows, int hkv, int cus, int prefix_len, SplitPlan &sp) {
  const int64_t units = (rows + kRowsPerUnit - 1) / kRowsPerUnit;
  const int64_t per_round = cus / hkv;
  if (per_round < 2 || units <= per_round) return false;
  const int64_t full = units / per_round * per_round;
  const int64_t left = units - full;
  if (left == 0) return false;
  const int64_t ways = per_round / left;
  const int64_t prefix_tiles = (prefix_len + kTileKeys - 1) / kTileKeys;
  if (ways < 2 || prefix_tiles < 2 * ways) return false;
  sp.full = full;
  sp.split = left;
  sp.tiles = int((prefix_tiles + ways - 1) / ways);
  // Recount the pieces for that piece size, so that none of them is left without a tile
  // (a piece with no keys would write no partial results); at least 2 remain.
  sp.ways = int((prefix_tiles + sp.tiles - 1) / sp.tiles);
  return true;
}

inline size_t split_workspace_bytes(const SplitPlan &sp, int hkv, int head_dim) {
  return size_t(sp.split) * size_t(sp.ways) * size_t(hkv) * size_t(kWaves) * 64 *
         size_t(part_floats(head_dim)) * sizeof(float);
}

// Work split of a grouped launch, with `rows[r]` query rows per KV head in request r: the
// same idea as unit_split, with no unit spanning two requests. Each request is cut into units
// of kRowsPerUnit rows. The units beyond the last full round of workgroups (the last ones in
// unit order, so they may span several requests) are re-cut, request by request, into units
// of the smallest multiple of 4 waves' rows that still fits them in one round; a launch of
// less than one round is cut the same way from the start. Fills full[r] (units of
// kRowsPerUnit rows) and small[r] (rows of each later unit) and returns the units per head.
inline int64_t grouped_split(const int64_t *rows, int n_req, int hkv, int cus, int *full,
                             int *small) {
  int64_t units = 0;
  for (int r = 0; r < n_req; ++r) {
    full[r] = int((rows[r] + kRowsPerUnit - 1) / kRowsPerUnit);
    small[r] = kRowsPerUnit;
    units += full[r];
  }
  const int64_t per_round = cus / hkv;  // units of one head in one round
  const int64_t simd_rows = 4 * kRowsPerWave;  // one wave on each SIMD
  if (per_round < 1) return units;
  const int64_t lead = units <= per_round ? 0 : units / per_round * per_round;  // kept whole
  if (lead == units) return units;
  int64_t keep[kMaxRequests];  // whole units a request keeps ahead of the re-cut ones
  int64_t seen = 0;
  for (int r = 0; r < n_req; ++r) {
    keep[r] = min(int64_t(full[r]), max(int64_t(0), lead - seen));
    seen += full[r];
  }
  for (int64_t s = simd_rows; s < kRowsPerUnit; s += simd_rows) {
    int64_t cut = 0;
    for (int r = 0; r < n_req; ++r)
      if (keep[r] < full[r]) cut += (rows[r] - keep[r] * kRowsPerUnit + s - 1) / s;
    if (cut > per_round) continue;
    for (int r = 0; r < n_req; ++r)
      if (keep[r] < full[r]) {
        full[r] = int(keep[r]);
        small[r] = int(s);
      }
    return lead + cut;
  }
  return units;
}

template <int D>
hipError_t launch(const Args &a, hipStream_t stream) {
  const int64_t blocks = a.n_units * a.hkv;  // exactly n_units units per KV head
  hipLaunchKernelGGL(prefix_tail_attention_kernel<D>, dim3(unsigned(blocks)), dim3(kThreads), 0,
                     stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.split_first >= a.n_units) return err;
  Args m = a;  // the merge pass: one workgroup per split base unit and KV head
  m.merge = 1;
  m.n_units = (a.n_units - a.split_first) / a.split_ways;
  hipLaunchKernelGGL(prefix_tail_attention_kernel<D>, dim3(unsigned(m.n_units * a.hkv)),
                     dim3(kThreads), 0, stream, m);
  return hipGetLastError();
}

}  // namespace

// The library builds this source twice. The main unit is compiled with an instruction scheduler
// that favours the matrix-bound launches (every launch with a prefix, and long causal
// prefills); a second unit, with BLINK_ATTENTION_PLAIN defined, holds only the kernel compiled
// with the compiler's default scheduler, which measured faster for prefix-free requests of
// short tails (bound by memory latency, not the matrix pipe). blink_attention_plain_launch runs
// that second instance for a filled argument block, passed as bytes so that neither unit
// depends on the other's internal types.
__attribute__((visibility("hidden"))) hipError_t blink_attention_plain_launch(
    const void *args, size_t args_bytes, int head_dim, hipStream_t stream);

#ifdef BLINK_ATTENTION_PLAIN

hipError_t blink_attention_plain_launch(const void *args, size_t args_bytes, int head_dim,
                                        hipStream_t stream) {
  Args a;
  if (args_bytes != sizeof(Args)) return hipErrorInvalidValue;
  memcpy(&a, args, sizeof(Args));
  return head_dim == 64 ? launch<64>(a, stream) : launch<128>(a, stream);
}

#else  // the main unit: host code and the library's entry points

namespace {

struct Shape {
  int32_t n_questions;
  int64_t total_valid_tokens, total_padded_tokens;
  int32_t n_heads_q, n_heads_kv, head_dim;
  float scale;
};

// Checks shared by both entry points; returns BLINK_OK or the failing status.
int check_shape(const void *q, const void *k_tail, const void *v_tail, const void *out,
                const int64_t *d_token_offset, const int32_t *d_valid_start, const Shape &sh) {
  using blink::fail;
  if (sh.n_questions < 1 || sh.n_questions > BLINK_MAX_QUESTIONS)
    return fail(BLINK_E_LIMIT, "request of %d questions; the limit is 1 to %d", sh.n_questions,
                BLINK_MAX_QUESTIONS);
  if (!q || !k_tail || !v_tail || !out || !d_token_offset || !d_valid_start)
    return fail(BLINK_E_INVALID, "prefix tail attention: a pointer argument is NULL");
  if (sh.head_dim != 64 && sh.head_dim != 128)
    return fail(BLINK_E_INVALID, "head_dim %d is not supported (64 or 128)", sh.head_dim);
  if (sh.n_heads_kv < 1 || sh.n_heads_q < sh.n_heads_kv || sh.n_heads_q % sh.n_heads_kv ||
      sh.n_heads_q / sh.n_heads_kv > kMaxGroup)
    return fail(BLINK_E_INVALID, "head counts %d/%d: need H_q a multiple of H_kv, group <= %d",
                sh.n_heads_q, sh.n_heads_kv, kMaxGroup);
  // A 64-key tile's byte span from its first row must fit a 32-bit buffer offset.
  if (int64_t(kTileKeys) * sh.n_heads_kv * sh.head_dim * 2 >= (int64_t(1) << 31))
    return fail(BLINK_E_LIMIT, "%d KV heads of %d dims are too wide for one tile", sh.n_heads_kv,
                sh.head_dim);
  if (!(sh.scale > 0.f) || !isfinite(sh.scale))
    return fail(BLINK_E_INVALID, "scale must be finite and positive");
  if (sh.total_valid_tokens < sh.n_questions ||
      sh.total_padded_tokens < sh.total_valid_tokens ||
      sh.total_valid_tokens > int64_t(sh.n_questions) * BLINK_MAX_INPUT_TOKENS)
    return fail(BLINK_E_INVALID, "token totals do not fit: %lld real of %lld padded for %d "
                "questions", (long long)sh.total_valid_tokens, (long long)sh.total_padded_tokens,
                sh.n_questions);
  return BLINK_OK;
}

// `plain`: launch the second build of the kernel (prefix-free requests of short tails).
int run(Args &a, const void *q, const void *k_tail, const void *v_tail, const void *k_prefix,
        const void *v_prefix, void *out, const int64_t *d_token_offset,
        const int32_t *d_valid_start, const Shape &sh, void *stream, bool plain = false) {
  using blink::fail;
  const void *ptrs[] = {q, k_tail, v_tail, out, a.prefix_rows ? k_prefix : q,
                        a.prefix_rows ? v_prefix : q};
  for (const void *p : ptrs)
    if (!blink::aligned16(p)) return fail(BLINK_E_INVALID, "tensors must be 16-byte aligned");
  a.q = static_cast<const uint16_t *>(q);
  a.k_tail = static_cast<const uint16_t *>(k_tail);
  a.v_tail = static_cast<const uint16_t *>(v_tail);
  a.k_pre = static_cast<const uint16_t *>(k_prefix);
  a.v_pre = static_cast<const uint16_t *>(v_prefix);
  a.out = static_cast<uint16_t *>(out);
  a.token_offset = d_token_offset;
  a.valid_start = d_valid_start;
  a.n = sh.n_questions;
  a.total_valid = sh.total_valid_tokens;
  a.t_pad = sh.total_padded_tokens;
  a.hq = sh.n_heads_q;
  a.hkv = sh.n_heads_kv;
  a.group = sh.n_heads_q / sh.n_heads_kv;
  a.scale_log2 = sh.scale * kLog2e;
  if (a.n_units * a.hkv > 0x7fffffffLL) return fail(BLINK_E_LIMIT, "launch too large");
  (void)hipGetLastError();
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t err = plain ? blink_attention_plain_launch(&a, sizeof(Args), sh.head_dim, s)
                         : sh.head_dim == 64 ? launch<64>(a, s)
                                             : launch<128>(a, s);
  if (err != hipSuccess)
    return fail(BLINK_E_DEVICE, "prefix tail attention launch: %s", hipGetErrorString(err));
  return blink::ok();
}

// The key-split plan of a single-request launch on the current device, if any; `cus` is set.
int single_plan(int64_t total_valid_tokens, int32_t n_heads_q, int32_t n_heads_kv,
                int32_t prefix_len, int &cus, SplitPlan &sp, bool &split) {
  int rc = blink::device_cus(cus, "prefix tail attention");
  if (rc != BLINK_OK) return rc;
  split = split_plan(total_valid_tokens * (n_heads_q / n_heads_kv), n_heads_kv, cus, prefix_len,
                     sp);
  return BLINK_OK;
}

}  // namespace

extern "C" size_t blink_prefix_tail_attention_workspace(int64_t total_valid_tokens,
                                                        int32_t n_heads_q, int32_t n_heads_kv,
                                                        int32_t head_dim, int32_t prefix_len) {
  if (total_valid_tokens < 1 || n_heads_kv < 1 || n_heads_q < n_heads_kv ||
      n_heads_q % n_heads_kv || (head_dim != 64 && head_dim != 128) || prefix_len < 0 ||
      total_valid_tokens > int64_t(BLINK_MAX_QUESTIONS) * BLINK_MAX_INPUT_TOKENS)
    return 0;
  int cus = 0;
  SplitPlan sp{};
  bool split = false;
  if (single_plan(total_valid_tokens, n_heads_q, n_heads_kv, prefix_len, cus, sp, split) !=
          BLINK_OK ||
      !split)
    return 0;
  return split_workspace_bytes(sp, n_heads_kv, head_dim);
}

extern "C" int blink_prefix_tail_attention(const void *q, const void *k_tail, const void *v_tail,
                                           const void *k_prefix, const void *v_prefix, void *out,
                                           const int64_t *d_token_offset,
                                           const int32_t *d_valid_start, int32_t n_questions,
                                           int64_t total_valid_tokens,
                                           int64_t total_padded_tokens, int32_t prefix_len,
                                           int32_t n_heads_q, int32_t n_heads_kv,
                                           int32_t head_dim, float scale, void *workspace,
                                           size_t workspace_bytes, void *stream) {
  using blink::fail;
  const Shape sh{n_questions, total_valid_tokens, total_padded_tokens, n_heads_q, n_heads_kv,
                 head_dim, scale};
  int rc = check_shape(q, k_tail, v_tail, out, d_token_offset, d_valid_start, sh);
  if (rc != BLINK_OK) return rc;
  if (prefix_len < 0 || prefix_len >= BLINK_MAX_INPUT_TOKENS)
    return fail(BLINK_E_LIMIT, "prefix of %d tokens leaves no room for a tail; the maximum "
                "context length is %d", prefix_len, BLINK_MAX_INPUT_TOKENS);
  if (prefix_len > 0 && (!k_prefix || !v_prefix))
    return fail(BLINK_E_INVALID, "prefix K/V pointers are NULL with prefix_len %d", prefix_len);
  if (workspace && !blink::aligned16(workspace))
    return fail(BLINK_E_INVALID, "the workspace must be 16-byte aligned");
  int cus = 0;
  SplitPlan sp{};
  bool split = false;
  if ((rc = single_plan(total_valid_tokens, n_heads_q, n_heads_kv, prefix_len, cus, sp, split)) !=
      BLINK_OK)
    return rc;
  Args a{};
  if (split && workspace && workspace_bytes >= split_workspace_bytes(sp, n_heads_kv, head_dim)) {
    a.full_units = sp.full;
    a.small_rows = kRowsPerUnit;
    a.split_first = sp.full;
    a.split_ways = sp.ways;
    a.split_tiles = sp.tiles;
    a.split_row0 = sp.full * kRowsPerUnit;
    a.part = static_cast<float *>(workspace);
    a.n_units = sp.full + sp.split * sp.ways;
  } else {
    a.n_units = unit_split(total_valid_tokens * (n_heads_q / n_heads_kv), n_heads_kv, cus,
                           a.full_units, a.small_rows);
    a.split_first = a.n_units;
  }
  a.prefix_rows = prefix_len;
  a.n_req = 1;
  a.req_first[0] = 0;
  a.req_first[1] = n_questions;
  a.req_unit[0] = 0;
  a.req_unit[1] = a.n_units;
  a.req_pstart[0] = 0;
  a.req_plen[0] = prefix_len;
  // Prefix-free requests of short tails (under 1024 tokens on average) go to the second build
  // of the kernel; a long causal prefill stays matrix-bound and stays here.
  const bool plain = prefix_len == 0 && a.split_first >= a.n_units &&
                     total_valid_tokens < int64_t(1024) * n_questions;
  return run(a, q, k_tail, v_tail, k_prefix, v_prefix, out, d_token_offset, d_valid_start, sh,
             stream, plain);
}

extern "C" int blink_prefix_tail_attention_grouped(
    const void *q, const void *k_tail, const void *v_tail, const void *k_prefix,
    const void *v_prefix, void *out, const int64_t *d_token_offset, const int32_t *d_valid_start,
    const int32_t *h_valid_start, int32_t n_questions, int64_t total_valid_tokens,
    int64_t total_padded_tokens, int32_t n_requests, const int32_t *h_request_first,
    const int64_t *h_prefix_start, const int32_t *h_prefix_len, int64_t total_prefix_rows,
    int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim, float scale, void *stream) {
  using blink::fail;
  const Shape sh{n_questions, total_valid_tokens, total_padded_tokens, n_heads_q, n_heads_kv,
                 head_dim, scale};
  int rc = check_shape(q, k_tail, v_tail, out, d_token_offset, d_valid_start, sh);
  if (rc != BLINK_OK) return rc;
  if (n_requests < 1 || n_requests > kMaxRequests)
    return fail(BLINK_E_LIMIT, "group of %d requests; the limit is 1 to %d", n_requests, kMaxRequests);
  if (!h_valid_start || !h_request_first || !h_prefix_start || !h_prefix_len)
    return fail(BLINK_E_INVALID, "prefix tail attention: a pointer argument is NULL");
  if (total_prefix_rows < 0 || (total_prefix_rows > 0 && (!k_prefix || !v_prefix)))
    return fail(BLINK_E_INVALID, "prefix K/V pointers are NULL with %lld prefix rows",
                (long long)total_prefix_rows);
  if (h_valid_start[0] != 0 || h_valid_start[n_questions] != total_valid_tokens)
    return fail(BLINK_E_INVALID, "valid_start must run from 0 to total_valid_tokens");
  for (int i = 0; i < n_questions; ++i)
    if (h_valid_start[i + 1] <= h_valid_start[i])
      return fail(BLINK_E_INVALID, "question %d has an empty tail", i);
  if (h_request_first[0] != 0 || h_request_first[n_requests] != n_questions)
    return fail(BLINK_E_INVALID, "request_first must run from 0 to n_questions");
  const int G = n_heads_q / n_heads_kv;
  Args a{};
  a.prefix_rows = total_prefix_rows;
  a.n_req = n_requests;
  a.full_units = 0;
  a.small_rows = kRowsPerUnit;
  int64_t rows[kMaxRequests];
  for (int r = 0; r < n_requests; ++r) {
    const int f = h_request_first[r], l = h_request_first[r + 1];
    if (l <= f) return fail(BLINK_E_INVALID, "request %d has no questions", r);
    const int64_t ps = h_prefix_start[r];
    const int pl = h_prefix_len[r];
    if (pl < 0 || ps < 0 || ps + pl > total_prefix_rows)
      return fail(BLINK_E_INVALID, "request %d: prefix rows [%lld, %lld) outside the %lld "
                  "prefix rows", r, (long long)ps, (long long)(ps + pl),
                  (long long)total_prefix_rows);
    for (int i = f; i < l; ++i) {
      const int64_t total = int64_t(pl) + (h_valid_start[i + 1] - h_valid_start[i]);
      if (total > BLINK_MAX_INPUT_TOKENS)
        return fail(BLINK_E_LIMIT, "question %d needs %lld tokens of context; the maximum "
                    "context length is %d", i, (long long)total, BLINK_MAX_INPUT_TOKENS);
    }
    a.req_first[r] = f;
    a.req_pstart[r] = ps;
    a.req_plen[r] = pl;
    rows[r] = int64_t(h_valid_start[l] - h_valid_start[f]) * G;
  }
  int cus = 0;
  if ((rc = blink::device_cus(cus, "prefix tail attention")) != BLINK_OK) return rc;
  grouped_split(rows, n_requests, n_heads_kv, cus, a.req_full, a.req_small);
  int64_t units = 0;  // the grid and the kernel's unit -> rows map follow the same counts
  for (int r = 0; r < n_requests; ++r) {
    a.req_unit[r] = units;
    units += a.req_full[r] + (rows[r] - int64_t(a.req_full[r]) * kRowsPerUnit +
                              a.req_small[r] - 1) / a.req_small[r];
  }
  a.req_first[n_requests] = n_questions;
  a.req_unit[n_requests] = units;
  a.n_units = units;
  a.full_units = units;
  a.split_first = units;  // no key split in a grouped launch
  return run(a, q, k_tail, v_tail, k_prefix, v_prefix, out, d_token_offset, d_valid_start, sh,
             stream);
}

#endif  // BLINK_ATTENTION_PLAIN
