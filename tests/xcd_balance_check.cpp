// Prints, for every hardware workgroup x of a one-item-per-workgroup prefill
// launch, the XCD the dispatcher sends it to (x mod 8) and the (run, query
// tile) it works on, using the kernels' own item-order functions.  Built and
// run by tests/test_xcd_balance.py on the host.
// Usage: xcd_balance_check <n_groups> <n_qtiles> <local 0|1>
#include <cstdio>
#include <cstdlib>

#include "g3_common.hpp"

int main(int argc, char** argv) {
  if (argc != 4) return 2;
  const int n_groups = std::atoi(argv[1]), nq = std::atoi(argv[2]);
  const bool local = std::atoi(argv[3]) != 0;
  const int n = n_groups * nq;
  const bool rank_major = g3::prefill_rank_major(local, n_groups);
  for (int x = 0; x < n; ++x) {
    const int li = g3::prefill_item_of_workgroup(x, n, rank_major);
    int bg, qt;
    g3::prefill_item_coords(li, n_groups, nq, rank_major, bg, qt);
    std::printf("%d %d %d %d\n", x % 8, li, bg, qt);
  }
  return 0;
}
