// Host-side check of the summary init's split plan (csrc/common.hpp):
// init_plan, init_split_rows and the workspace bound init_split_bound, over
// many prefix lengths and grid shapes.  Built and run by
// tests/test_init_plan_host.py; prints one line per failure and exits 1.
//
// For every plan it checks that
//  * the splits cover the rows [0, L0) exactly once, each split non-empty;
//  * far splits hold only rows at least kInitNearRows before the newest one
//    (their faster slots are bounded on that distance), and only the plans
//    for bf16, d = 128, S in {64, 128} have far splits;
//  * near splits hold at most near_rows rows and far ones at most far_rows,
//    far_rows a multiple of the 128-row far tile;
//  * nsplit() stays within init_split_bound(d, M) for every M >= L0 (the
//    workspace sized for a longer prefix fits a shorter one).
#include <cstdio>
#include <vector>

#include "../fixed_cost_drafter_amd/csrc/common.hpp"

static int failures = 0;
#define CHECK(cond, ...)                       \
  do {                                         \
    if (!(cond)) {                             \
      if (failures < 50) {                     \
        std::printf("FAIL %s: ", #cond);       \
        std::printf(__VA_ARGS__);              \
        std::printf("\n");                     \
      }                                        \
      ++failures;                              \
    }                                          \
  } while (0)

static void check(const ls_dims& d, int L0, int bound_next) {
  const ls::InitPlan p = ls::init_plan(d, L0);
  const int n = p.nsplit();
  const char* tag = "C=%d Hkv=%d S=%d dtype=%d L0=%d";
#define ARGS d.C, d.Hkv, d.S, d.dtype, L0
  CHECK(p.n_near >= 1 && p.near_rows >= 1, tag, ARGS);
  CHECK(p.n_far == 0 || (ls::init_has_far(d) && p.far_rows % 128 == 0), tag, ARGS);
  CHECK(n <= ls::init_split_bound(d, L0), tag, ARGS);
  CHECK(ls::init_split_bound(d, L0) <= bound_next, tag, ARGS);
  std::vector<int> cover(size_t(L0), 0);
  for (int s = 0; s < n; ++s) {
    int rb = 0, re = 0;
    ls::init_split_rows(p, L0, s, &rb, &re);
    CHECK(0 <= rb && rb < re && re <= L0, "%s split %d [%d, %d)", "range", s, rb, re);
    if (!(0 <= rb && rb < re && re <= L0)) continue;
    const bool far = s >= p.n_near;
    CHECK(re - rb <= (far ? p.far_rows : p.near_rows), "split %d of L0=%d", s, L0);
    if (far) CHECK(int64_t(L0) - re >= ls::kInitNearRows, "far split %d of L0=%d ends at %d", s, L0, re);
    for (int r = rb; r < re; ++r) ++cover[size_t(r)];
  }
  for (int r = 0; r < L0; ++r)
    if (cover[size_t(r)] != 1) {
      CHECK(cover[size_t(r)] == 1, "row %d of L0=%d covered %d times", r, L0, cover[size_t(r)]);
      break;
    }
#undef ARGS
}

int main() {
  std::vector<ls_dims> dims;
  for (int dt : {LS_BF16, LS_F32})
    for (int S : {0, 4, 64, 128})
      for (int dd : {16, 128})
        for (int C : {1, 2, 16, 64})
          for (int Hkv : {1, 2, 8}) {
            ls_dims d{};
            d.C = C;
            d.Hq = 4 * Hkv;
            d.Hkv = Hkv;
            d.d = dd;
            d.W = 64;
            d.S = S;
            d.B = 4;
            d.V = 1000;
            d.dtype = dt;
            dims.push_back(d);
          }
  std::vector<int> lens;
  for (int L = 1; L <= 1000; ++L) lens.push_back(L);
  for (int L = 1000; L <= 140000; L += 997) lens.push_back(L);
  for (int base : {12288, 24576, 32768, 49152, 65536, 131072})
    for (int dl = -130; dl <= 130; ++dl) lens.push_back(base + dl);
  lens.push_back(262144);
  lens.push_back(1 << 20);
  int checked = 0;
  for (const ls_dims& d : dims)
    for (int L : lens) {
      // the bound at a longer prefix: the next length and a much longer one
      const int nxt = ls::init_split_bound(d, L + 1) < ls::init_split_bound(d, 4 * L)
                          ? ls::init_split_bound(d, L + 1)
                          : ls::init_split_bound(d, 4 * L);
      check(d, L, nxt);
      ++checked;
    }
  std::printf("%d plans checked, %d failures\n", checked, failures);
  return failures ? 1 : 0;
}
