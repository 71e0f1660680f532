// Host check of the attention launch's work split (built and run by test_unit_plan.py; no GPU
// call). It includes the kernel source to reach its planners, unit_split (one request) and
// grouped_split (several), and walks every unit through the same unit -> rows map the kernel
// applies, over many random layouts. Each must cover every query row of every request exactly
// once, in order, with no unit spanning two requests; re-cut units must be whole multiples of
// 4 waves' rows; and the launch must take as many rounds of workgroups as with whole
// 384-row units, so that the re-cut only shortens the last round.
#include "../pass_typed_decision_amd/csrc/blink_attention.hip"

#include <cstdio>
#include <random>
#include <vector>

namespace {

int64_t rounds_of(int64_t units, int64_t per_round) {
  return per_round < 1 ? units : (units + per_round - 1) / per_round;
}

bool check_single(int64_t rows, int hkv, int cus) {
  int64_t full = 0;
  int small = 0;
  const int64_t units = unit_split(rows, hkv, cus, full, small);
  const int64_t whole = (rows + kRowsPerUnit - 1) / kRowsPerUnit;
  int64_t covered = 0;
  for (int64_t unit = 0; unit < units; ++unit) {
    const int64_t row0 = unit < full ? unit * kRowsPerUnit
                                     : full * kRowsPerUnit + (unit - full) * small;
    const int64_t row_end =
        std::min(rows, row0 + (unit < full ? int64_t(kRowsPerUnit) : int64_t(small)));
    if (row0 != covered || row0 >= row_end) return false;
    covered = row_end;
  }
  if (covered != rows) return false;
  if (small < 4 * kRowsPerWave || small > kRowsPerUnit || small % (4 * kRowsPerWave)) return false;
  return rounds_of(units, cus / hkv) == rounds_of(whole, cus / hkv);
}

// The key split: full units then the split base units cover every row once; each base unit's
// pieces (key ranges computed as the kernel does) cover the prefix keys once, in order, each
// piece non-empty, only the last one walking the tail; the pieces fill at most one round.
bool check_split(int64_t rows, int hkv, int cus, int prefix) {
  SplitPlan sp{};
  if (!split_plan(rows, hkv, cus, prefix, sp)) return true;
  const int64_t units = (rows + kRowsPerUnit - 1) / kRowsPerUnit;
  if (sp.full + sp.split != units || sp.full % (cus / hkv) != 0) return false;
  if (sp.split * sp.ways > cus / hkv || sp.ways < 2 || sp.tiles < 1) return false;
  int covered = 0;
  for (int j = 0; j < sp.ways; ++j) {
    const int kbeg = std::min(j * sp.tiles * kTileKeys, prefix);
    const int kend = std::min((j + 1) * sp.tiles * kTileKeys, prefix);
    if (kbeg != covered || kbeg >= kend) return false;
    covered = kend;
  }
  return covered == prefix;
}

bool check_grouped(const std::vector<int64_t> &rows, int hkv, int cus) {
  const int n_req = int(rows.size());
  int full[kMaxRequests], small[kMaxRequests];
  const int64_t units = grouped_split(rows.data(), n_req, hkv, cus, full, small);
  // The entry point's request table, then the kernel's map for every unit.
  int64_t req_unit[kMaxRequests + 1], start[kMaxRequests + 1];
  int64_t u = 0, whole = 0;
  start[0] = 0;
  for (int r = 0; r < n_req; ++r) {
    req_unit[r] = u;
    u += full[r] + (rows[r] - int64_t(full[r]) * kRowsPerUnit + small[r] - 1) / small[r];
    start[r + 1] = start[r] + rows[r];
    whole += (rows[r] + kRowsPerUnit - 1) / kRowsPerUnit;
    if (small[r] < 4 * kRowsPerWave || small[r] > kRowsPerUnit ||
        small[r] % (4 * kRowsPerWave))
      return false;
  }
  req_unit[n_req] = u;
  if (u != units) return false;
  int64_t covered = 0;
  for (int64_t unit = 0; unit < units; ++unit) {
    int r = 0;
    while (r + 1 < n_req && req_unit[r + 1] <= unit) ++r;
    const int64_t k = unit - req_unit[r];
    const int64_t row0 = start[r] + (k < full[r] ? k * kRowsPerUnit
                                                 : full[r] * int64_t(kRowsPerUnit) +
                                                       (k - full[r]) * small[r]);
    const int64_t row_end =
        std::min(start[r + 1], row0 + (k < full[r] ? int64_t(kRowsPerUnit) : int64_t(small[r])));
    if (row0 != covered || row0 >= row_end) return false;
    covered = row_end;
  }
  if (covered != start[n_req]) return false;
  return rounds_of(units, cus / hkv) == rounds_of(whole, cus / hkv);
}

}  // namespace

int main(int argc, char **argv) {
  if (argc > 1) {  // "plan": "rows hkv cus prefix" per line -> "units full small" of the row
                   // split, then "full left ways tiles" of the key split (zeros if none)
    long long rows = 0;
    int hkv = 0, cus = 0, prefix = 0;
    while (scanf("%lld %d %d %d", &rows, &hkv, &cus, &prefix) == 4) {
      int64_t full = 0;
      int small = 0;
      const int64_t units = unit_split(rows, hkv, cus, full, small);
      SplitPlan sp{};
      if (!split_plan(rows, hkv, cus, prefix, sp)) sp = SplitPlan{0, 0, 0, 0};
      printf("%lld %lld %d %lld %lld %d %d\n", (long long)units, (long long)full, small,
             (long long)sp.full, (long long)sp.split, sp.ways, sp.tiles);
    }
    return 0;
  }
  std::mt19937_64 rng(20261202);
  long recut_single = 0, recut_grouped = 0, split_single = 0;
  for (int trial = 0; trial < 100000; ++trial) {
    const int hkv = 1 << (rng() % 4);
    const int cus = trial % 3 == 0 ? 256 : int(1 + rng() % 300);
    const int64_t lim[4] = {64, 2000, 30000, 400000};
    const int64_t rows = 1 + int64_t(rng() % lim[rng() % 4]);
    if (!check_single(rows, hkv, cus)) {
      printf("FAIL unit_split rows %lld hkv %d cus %d\n", (long long)rows, hkv, cus);
      return 1;
    }
    const int prefix = int(rng() % 70000);
    if (!check_split(rows, hkv, cus, prefix)) {
      printf("FAIL split_plan rows %lld hkv %d cus %d prefix %d\n", (long long)rows, hkv, cus,
             prefix);
      return 1;
    }
    SplitPlan sp{};
    split_single += split_plan(rows, hkv, cus, prefix, sp);
    int64_t full = 0;
    int small = 0;
    unit_split(rows, hkv, cus, full, small);
    recut_single += small != kRowsPerUnit;

    std::vector<int64_t> group(1 + rng() % kMaxRequests);
    const int64_t glim = lim[rng() % 4];
    for (auto &g : group) g = 1 + int64_t(rng() % glim);
    if (!check_grouped(group, hkv, cus)) {
      printf("FAIL grouped_split trial %d: %zu requests, hkv %d, cus %d\n", trial, group.size(),
             hkv, cus);
      return 1;
    }
    int fl[kMaxRequests], sm[kMaxRequests];
    grouped_split(group.data(), int(group.size()), hkv, cus, fl, sm);
    for (size_t r = 0; r < group.size(); ++r)
      if (sm[r] != kRowsPerUnit) {
        ++recut_grouped;
        break;
      }
  }
  // Two requests of 21352 rows per KV head (8 heads, 256 CUs): 56 whole units each, 3.5
  // rounds; the last 16 units are re-cut into 24 units of 256 rows.
  const int64_t two[2] = {21352, 21352};
  int fl[2], sm[2];
  const int64_t units = grouped_split(two, 2, 8, 256, fl, sm);
  printf("two requests: %lld units, full %d %d, small %d %d\n", (long long)units, fl[0], fl[1],
         sm[0], sm[1]);
  // The 27B-like request as drawn: 10864 tokens x 5 query heads per KV head, 8 KV heads, 256
  // CUs, a 65536-token prefix.
  SplitPlan c5{};
  split_plan(54320, 8, 256, 65536, c5);
  printf("27B-like split: full %lld, split %lld, ways %d, tiles %d\n", (long long)c5.full,
         (long long)c5.split, c5.ways, c5.tiles);
  printf("ok: 100000 layouts each, re-cut %ld single, %ld grouped, key-split %ld\n",
         recut_single, recut_grouped, split_single);
  return 0;
}
