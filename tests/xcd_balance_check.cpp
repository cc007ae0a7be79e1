// Prints, for every hardware workgroup x of a one-item-per-workgroup prefill
// launch, the XCD the dispatcher sends it to (x mod 8) and the (run, query
// tile) it works on, using the kernels' own item-order functions.  Built and
// run by tests/test_xcd_balance.py on the host.
// Usage: xcd_balance_check <n_groups> <n_qtiles> <local 0|1>
//        xcd_balance_check <n_groups> <n_qtiles> 1 <grid>: the local-layer
//        schedule with several items per workgroup (grid workgroups): one
//        line "xcd step item run qtile" per (workgroup, step).
#include <cstdio>
#include <cstdlib>

#include "g3_common.hpp"

int main(int argc, char** argv) {
  if (argc != 4 && argc != 5) return 2;
  const int n_groups = std::atoi(argv[1]), nq = std::atoi(argv[2]);
  const bool local = std::atoi(argv[3]) != 0;
  const int n = n_groups * nq;
  if (argc == 5) {
    const int grid = std::atoi(argv[4]);
    if (grid <= 0 || n % grid != 0 || nq % (n / grid) != 0) return 3;
    const int K = n / grid;
    for (int x = 0; x < grid; ++x)
      for (int kk = 0; kk < K; ++kk) {
        const int li = g3::prefill_spread_item(g3::xcd_remap(x, grid), kk, K, nq);
        int bg, qt;
        g3::prefill_item_coords(li, n_groups, nq, false, bg, qt);
        std::printf("%d %d %d %d %d\n", x % 8, kk, li, bg, qt);
      }
    return 0;
  }
  const bool rank_major = g3::prefill_rank_major(local, n_groups);
  for (int x = 0; x < n; ++x) {
    const int li = g3::prefill_item_of_workgroup(x, n, rank_major);
    int bg, qt;
    g3::prefill_item_coords(li, n_groups, nq, rank_major, bg, qt);
    std::printf("%d %d %d %d\n", x % 8, li, bg, qt);
  }
  return 0;
}
