// Host-side check of the LDS tile layout used by every matrix kernel
// (CmTile, RowRead, TrRead in fa_device.h).  Built and run by
// tests/test_layout.py; no GPU is used.
//
// For each tile shape the kernels use it checks that
//  * global -> LDS copy slots map one-to-one onto (row, chunk) and agree with
//    CmTile::off;
//  * RowRead::at(t) addresses chunk 2t + h of the lane's row, and the 16 lanes
//    of a half (rows sigma(0..15) of a 16-row block) hit 16 distinct 16-byte
//    bank groups;
//  * TrRead's bases address exactly the elements the transposing operand read
//    documents (rows k0 + 8h + r and +4, columns 32 db + 16 (g % 2) +
//    4 swap01(c) .. +3) and 32 lanes hit 32 distinct 8-byte bank slots.
#include <cstdio>
#include <set>

#include "fa_device.h"

using namespace fa;

template <int R, int D>
static int check() {
  using T = CmTile<R>;
  int bad = 0;
  const int C = D / 8;
  std::set<int> seen;
  for (int s = 0; s < R * C; ++s) {
    const int r = T::slot_row(s), c = T::slot_chunk(s);
    if (r < 0 || r >= R || c < 0 || c >= C || T::off(r, c) != 16 * s) ++bad;
    seen.insert(r * C + c);
  }
  if ((int)seen.size() != R * C) ++bad;
  for (int blk = 0; blk < R / 32; ++blk)
    for (int h = 0; h < 2; ++h)
      for (int t = 0; t < D / 16; ++t) {
        std::set<int> groups;
        for (int l = 0; l < 32; ++l) {
          const int row = 32 * blk + sigma32(l);
          const int a = RowRead<R>(sigma32(l), h).at(t) + kRowBlockBytes * blk;
          if (a != T::off(row, 2 * t + h)) ++bad;
          if (l < 16) groups.insert((a / 16) % 16);
        }
        if (groups.size() != 16) ++bad;
      }
  for (int k0 = 0; k0 + 16 <= R; k0 += 16)
    for (int db = 0; db < D / 32; ++db)
      for (int h = 0; h < 2; ++h) {
        std::set<int> slots;
        for (int l = 32 * h; l < 32 * h + 32; ++l) {
          const TrRead<R> b(l);
          const int g = l >> 4, r = (l & 15) >> 2, c = l & 3;
          const int col = 32 * db + 16 * (g & 1) + 4 * swap01(c);
          const int o = k0 * 64 + db * T::GB;
          if (b.lo + o != T::off(k0 + 8 * h + r, col / 8) + 2 * (col % 8)) ++bad;
          if (b.hi + o != T::off(k0 + 8 * h + 4 + r, col / 8) + 2 * (col % 8)) ++bad;
          slots.insert(((b.lo + o) % 256) / 8);
        }
        if (slots.size() != 32) ++bad;
      }
  if (bad) std::printf("tile R=%d D=%d: %d failures\n", R, D, bad);
  return bad;
}

int main() {
  const int bad = check<32, 64>() + check<32, 128>() + check<32, 256>() + check<64, 64>() + check<64, 128>() +
                  check<128, 64>() + check<128, 128>() + check<128, 256>();
  std::printf("layout check: %s\n", bad ? "FAIL" : "ok");
  return bad ? 1 : 0;
}
