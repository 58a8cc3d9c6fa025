// Prints the closed-form row and column intervals of masked_attention_amd/csrc/schedule.h
// for one (kind, source, L, S): "row i lo hi" and "col j lo hi" lines.  Built and run by
// tests/test_schedule_host.py on the host (no GPU).
#include <cstdio>
#include <cstdlib>

#include "schedule.h"

int main(int argc, char** argv) {
  if (argc != 5) return 2;
  const int kind = std::atoi(argv[1]), src = std::atoi(argv[2]);
  const int L = std::atoi(argv[3]), S = std::atoi(argv[4]);
  for (int i = 0; i < L; ++i) {
    const e2d2::Interval r = e2d2::row_interval(kind, src, i, S, L, 0);
    std::printf("row %d %d %d\n", i, r.lo, r.hi);
  }
  for (int j = 0; j < L; ++j) {
    const e2d2::Interval c = e2d2::col_interval(kind, src, j, S, L);
    std::printf("col %d %d %d\n", j, c.lo, c.hi);
  }
  for (int k0 = 0; k0 < L; k0 += 7) {
    const int k1 = k0 + 6 < L ? k0 + 6 : L - 1;
    const e2d2::Interval u = e2d2::col_union(kind, src, k0, k1, S, L);
    const e2d2::Interval c = e2d2::col_common(kind, src, k0, k1, S, L);
    std::printf("span %d %d %d %d %d %d\n", k0, k1, u.lo, u.hi, c.lo, c.hi);
  }
  return 0;
}
