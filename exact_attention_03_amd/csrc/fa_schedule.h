// fa_schedule.h - static schedule of the persistent dK/dV kernel.
//
// [FA-Ascend] (the page "把 FlashAttention 搬上昇腾：Triton-Ascend CV Pipeline
// 优化实战", BiumBiu) §五 runs as many programs as the chip has matrix cores
// and lets each program claim heads with a fixed stride, so that one program
// writes each gradient tile once and no atomics or cross-program reductions
// are needed.  Here the unit of work is (head, key tile) and the grid is the
// number of workgroups the GPU keeps resident.  Units are numbered so that, with
// the causal mask, cost never increases with the unit index (key tile j of
// every head comes before key tile j+1, and an earlier key tile sees more query
// tiles); they are then dealt to the P programs in snake order (round r hands
// units rP .. rP+P-1 to programs 0..P-1 on even rounds and P-1..0 on odd
// rounds), which balances the causal triangle.  Without the mask all units
// cost the same and the snake reduces to a fixed stride, as on the page.
//
// Pure integer code, usable on the host (tests, planning) and on the device.
#pragma once

#include <stdint.h>

#ifdef __HIPCC__
#define FA_SCHED_HD __host__ __device__ inline
#else
#define FA_SCHED_HD inline
#endif

namespace fa {

// Unit handed to program p in round r (may be >= the unit count: then the
// program has no unit in that round and every later round).
FA_SCHED_HD int64_t sched_unit(int64_t round, int64_t p, int64_t P) {
  return round * P + ((round & 1) ? (P - 1 - p) : p);
}

// Unit index -> (key tile, head).
FA_SCHED_HD void sched_decode(int64_t u, int64_t ZH, int64_t* key_tile, int64_t* head) {
  *key_tile = u / ZH;
  *head = u - (*key_tile) * ZH;
}

// Query tiles a unit visits: all of them, or with the causal mask those from
// the tile holding the unit's first key onwards.
FA_SCHED_HD int64_t sched_first_qtile(int64_t key_tile, int64_t keys_per_unit,
                                      int64_t queries_per_tile, int causal) {
  return causal ? (key_tile * keys_per_unit) / queries_per_tile : 0;
}

// Query-tile grids (forward and dQ passes) laid out so that the tiles of one
// head run on one XCD, back to back, and share its L2 copy of K and V.
// Workgroups are dealt to the XCDs round-robin by block index, so block b runs
// on XCD b % kXcds; the s-th block of XCD x (s = b / kXcds) takes head
// x + kXcds * (s / n_qtiles) and tile slot s % n_qtiles.  The grid is padded to
// kXcds * ceil(ZH / kXcds) * n_qtiles blocks; a block whose head is past the
// last one has no work.
constexpr int64_t kXcds = 8;
FA_SCHED_HD int64_t xcd_grid(int64_t ZH, int64_t n_qtiles) {
  return ((ZH + kXcds - 1) / kXcds) * kXcds * n_qtiles;
}
FA_SCHED_HD void xcd_tile(int64_t b, int64_t n_qtiles, int64_t* head, int64_t* slot) {
  const int64_t x = b % kXcds, s = b / kXcds;
  *head = x + kXcds * (s / n_qtiles);
  *slot = s % n_qtiles;
}

}  // namespace fa
