// Host-side check of the causal pairing of query tiles (paired_groups /
// paired_items in fa_schedule.h) used by the forward and dQ grids, including
// what a grid sized for a shorter max_seqlen leaves out.  Built with the host
// compiler and run by tests/test_schedule_host.py; no GPU is used.
#include <cstdio>
#include <vector>

#include "fa_schedule.h"

using namespace fa;

// Tiles visited when the grid deals paired_groups(n_grid) slots per head to a
// sequence of n tiles (slots past paired_groups(n) return early, as in the
// kernels).
static std::vector<int> visits(int n, int n_grid, int causal) {
  std::vector<int> seen(n, 0);
  const int slots = (int)paired_groups(n_grid, causal);
  for (int p = 0; p < slots; ++p) {
    if (p >= paired_groups(n, causal)) continue;
    uint32_t a, b;
    const int items = paired_items((uint32_t)p, (uint32_t)n, causal, &a, &b);
    if (a < (uint32_t)n) ++seen[a];
    if (items == 2 && b < (uint32_t)n) ++seen[b];
  }
  return seen;
}

int main() {
  int bad = 0;
  for (int causal = 0; causal < 2; ++causal)
    for (int n_grid = 1; n_grid <= 40; ++n_grid)
      for (int n = 1; n <= 48; ++n) {
        const std::vector<int> seen = visits(n, n_grid, causal);
        const int g = (int)paired_groups(n_grid, causal);
        for (int t = 0; t < n; ++t) {
          int want;
          if (n <= n_grid)
            want = 1;  // every tile exactly once
          else if (causal)
            want = (t < g || t > n - 1 - g) ? 1 : 0;  // both ends covered, interior left out
          else
            want = t < n_grid ? 1 : 0;  // the tail left out
          if (seen[t] != want) {
            if (bad < 10) printf("causal %d n_grid %d n %d tile %d: visited %d, expected %d\n", causal, n_grid, n, t, seen[t], want);
            ++bad;
          }
        }
      }
  if (bad == 0) printf("schedule check: ok\n");
  return bad != 0;
}
