// fa_schedule.h - work layout of the kernels: the static schedule of the
// persistent dK/dV pass and the XCD-aware grid of the query-tile passes.
//
// [FA-Ascend] (the page "把 FlashAttention 搬上昇腾：Triton-Ascend CV Pipeline
// 优化实战", BiumBiu) §五 runs as many programs as the chip has matrix cores
// and lets each program claim heads with a fixed stride, so that one program
// writes each gradient tile once and no atomics or cross-program reductions
// are needed.  Here the unit of work is (head, key tile) and the grid is the
// number of workgroups the GPU keeps resident.
//
// XCD groups.  Workgroups are dealt to the 8 XCDs round-robin by block index,
// and each XCD has its own L2.  When the program count is a multiple of 8 (and
// there are at least 8 heads), program p belongs to group g = p % 8, which owns
// heads g, g+8, g+16, ...; otherwise there is one group owning every head.  A
// group lists its units head-major (all key tiles of a head, in order, then
// the next head), so the programs of one XCD work on a few heads at a time and
// share their Q and dO through L2.
//
// Dealing.  Round r hands the group's units rS .. rS+S-1 to its S programs,
// in order on even rounds and in reverse on odd rounds ("snake").  With the
// causal mask a unit's cost falls with its key tile; when S is a multiple of
// the key tiles per head, the snake pairs key tile j with key tile n-1-j and
// every program gets the same work.  Without the mask all units cost the
// same, and with one key tile per head the dealing is the page's fixed stride.
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

constexpr int64_t kXcds = 8;

// Number of XCD groups for P programs over ZH heads.
FA_SCHED_HD int64_t sched_groups(int64_t P, int64_t ZH) {
  return (P % kXcds == 0 && ZH >= kXcds) ? kXcds : 1;
}

// Unit of program p in round r: returns false when p has no unit in round r,
// and then none in any later round.
FA_SCHED_HD bool sched_unit(int64_t r, int64_t p, int64_t P, int64_t ZH, int64_t n_ktiles,
                            int64_t* head, int64_t* key_tile) {
  const int64_t G = sched_groups(P, ZH);
  const int64_t g = p % G, s = p / G, S = P / G;
  const int64_t heads_g = (ZH - g + G - 1) / G;  // heads g, g+G, ... below ZH
  const int64_t i = r * S + ((r & 1) ? (S - 1 - s) : s);
  if (i >= heads_g * n_ktiles) return false;
  *head = g + G * (i / n_ktiles);
  *key_tile = i % n_ktiles;
  return true;
}

// Query tiles a unit visits: all of them, or with the causal mask those from
// the tile holding the unit's first key onwards.
FA_SCHED_HD int64_t sched_first_qtile(int64_t key_tile, int64_t keys_per_unit,
                                      int64_t queries_per_tile, int causal) {
  return causal ? (key_tile * keys_per_unit) / queries_per_tile : 0;
}

// Causal pairing of query tiles (forward and dQ passes).  With the causal
// mask the cost of query tile i grows with i, so a workgroup takes tiles
// n-1-p and p of one head, one after the other: every workgroup has the same
// work (with an odd count the middle tile is alone), and the second tile's
// start overlaps the end of the first.  Without the mask a workgroup takes one
// tile.  paired_groups is the number of workgroups per head; paired_items
// returns how many tiles workgroup slot p takes and which.
FA_SCHED_HD int64_t paired_groups(int64_t n_qtiles, int causal) {
  return causal ? (n_qtiles + 1) / 2 : n_qtiles;
}
FA_SCHED_HD int paired_items(uint32_t p, uint32_t n_qtiles, int causal, uint32_t* first, uint32_t* second) {
  if (!causal) {
    *first = *second = p;
    return 1;
  }
  *first = n_qtiles - 1 - p;
  *second = p;
  return *first != *second ? 2 : 1;
}

// Query-tile grids (forward and dQ passes) laid out so that the tiles of one
// head run on one XCD, back to back, and share its L2 copy of K and V.
// Workgroups are dealt to the XCDs round-robin by block index, so block b runs
// on XCD b % kXcds; the s-th block of XCD x (s = b / kXcds) takes head
// x + kXcds * (s / n_qtiles) and tile slot s % n_qtiles.  The grid is padded to
// kXcds * ceil(ZH / kXcds) * n_qtiles blocks; a block whose head is past the
// last one has no work.  The decode runs in 32-bit arithmetic (a 64-bit
// division is a long instruction sequence on the GPU); callers keep the grid
// below 2^31 blocks.
FA_SCHED_HD int64_t xcd_grid(int64_t ZH, int64_t n_qtiles) {
  return ((ZH + kXcds - 1) / kXcds) * kXcds * n_qtiles;
}
FA_SCHED_HD void xcd_tile(uint32_t b, uint32_t n_qtiles, uint32_t* head, uint32_t* slot) {
  const uint32_t x = b % (uint32_t)kXcds, s = b / (uint32_t)kXcds;
  *head = x + (uint32_t)kXcds * (s / n_qtiles);
  *slot = s % n_qtiles;
}

// Grouped key/value heads (G query heads share one key/value head): the
// forward and dQ grids deal (key/value head, member, slot) so that the G
// query heads of a key/value head run on one XCD, back to back, and share its
// K and V through that XCD's L2.  Query head = kv_head * G + member.  With
// G = 1 this is xcd_tile over query heads.
FA_SCHED_HD int64_t xcd_grid_grouped(int64_t ZHkv, int64_t G, int64_t n_slots) {
  return xcd_grid(ZHkv, G * n_slots);
}
FA_SCHED_HD void xcd_tile_grouped(uint32_t b, uint32_t G, uint32_t n_slots, uint32_t* kv_head, uint32_t* head,
                                  uint32_t* slot) {
  uint32_t s;
  xcd_tile(b, G * n_slots, kv_head, &s);
  *head = *kv_head * G + s / n_slots;
  *slot = s % n_slots;
}

// Rows of one (sequence, query head) problem and of its key/value head.
// Dense batches are (Z, H, N, D): the problem of query head hq of batch z
// starts at row (z H + hq) N and has N rows.  Variable-length batches are
// packed head-major, (H, T, D) with sequence b at tokens cu[b] .. cu[b+1]-1:
// the problem starts at row hq T + cu[b] and has cu[b+1] - cu[b] rows.  The
// grids deal "batch key/value heads" bkv in [0, batch * Hkv) (bkv = z Hkv +
// hk) and members m in [0, G) of each (query head hk G + m).
struct HeadRows {
  int64_t q_row0;   // first row of the query head's problem (Q, O, dO, lse, ...)
  int64_t kv_row0;  // first row of the key/value head's problem (K, V, dK, dV)
  int64_t q_stride; // rows from one query head of the group to the next
  int n;            // rows of the problem (the sequence length)
};
FA_SCHED_HD HeadRows head_rows(uint32_t bkv, uint32_t member, uint32_t Hkv, uint32_t G, int N, const int* cu,
                               int64_t T) {
  HeadRows r;
  if (cu == nullptr) {
    r.q_row0 = ((int64_t)bkv * G + member) * N;
    r.kv_row0 = (int64_t)bkv * N;
    r.q_stride = N;
    r.n = N;
  } else {
    // Offsets are clamped into [0, T], so that no offsets array, however
    // wrong, makes a kernel touch rows outside the tensors.
    const uint32_t b = bkv / Hkv, hk = bkv % Hkv;
    const int64_t s0 = cu[b], s1 = cu[b + 1];
    const int64_t start = s0 < 0 ? 0 : (s0 > T ? T : s0);
    const int64_t end = s1 < start ? start : (s1 > T ? T : s1);
    r.n = (int)(end - start);
    r.q_row0 = ((int64_t)hk * G + member) * T + start;
    r.kv_row0 = (int64_t)hk * T + start;
    r.q_stride = T;
  }
  return r;
}

}  // namespace fa
