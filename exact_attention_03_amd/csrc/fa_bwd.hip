// fa_bwd.hip - exact attention backward for gfx950: Delta pass, dK/dV pass
// and dQ pass.
//
// [FA-Ascend] = the page "把 FlashAttention 搬上昇腾：Triton-Ascend CV Pipeline
// 优化实战" (BiumBiu).  §二 gives the backward:
//     Delta = rowsum(O * dO)
//     P     = recompute_softmax(Q K^T * scale)
//     dP    = dO V^T
//     dS    = scale * P * (dP - Delta)
//     dQ   += dS K ;  dK += dS^T Q ;  dV += P^T dO
// and the rules the page keeps: P is recomputed, never stored; each gradient
// tile has a single writer; scratch does not grow with N^2.  §二 also notes
// that dQ can be finished by the query tile itself while a dK/dV tile gathers
// contributions from every query tile; hence two passes with different owners:
// a persistent pass that owns key tiles (dK, dV) and a pass that owns query
// tiles (dQ).  The scale of dS is applied once to the finished dK and dQ
// accumulators, which is the same product.
//
// P is recomputed from the saved lse: P = exp2(S * scale * log2e - lse * log2e).
#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_schedule.h"

namespace fa {

// Straight-line sequence of N steps whose operands come from LDS:
// read(n) returns step n's operands and use(n, ops) issues its products.  The
// reads of step n + 1 are issued before the products of step n, so that one
// step's LDS latency overlaps the previous step's matrix instructions (without
// this the compiler, short of registers, waits for each read right before its
// product).  Costs one extra set of operand registers.
struct U4x2 {
  u32x4 a, b;
};
struct U4x3 {
  u32x4 a, b, c;
};
template <int N, typename Read, typename Use>
FA_DEV void read_ahead(Read read, Use use) {
  auto cur = read(0);
#pragma unroll
  for (int n = 0; n < N; ++n) {
    auto nxt = cur;
    if (n + 1 < N) nxt = read(n + 1);
    use(n, cur);
    cur = nxt;
  }
}

// ============================================================ Delta pass
// delta[row] = sum_d O[row, d] * dO[row, d] in fp32, and lse2[row] =
// lse[row] * log2(e), the row statistic in the exp2 units the gradient passes
// use (so they need no per-element conversion).  HBM-bound: each thread reads
// one 16-byte chunk of dO (8 elements) and the matching O elements; the D/8
// threads of a row combine their partial sums with lane shuffles.
template <int D, typename T, bool O32>
__global__ __launch_bounds__(256) void fa_bwd_pre_kernel(const void* __restrict__ o,
                                                         const uint16_t* __restrict__ dout,
                                                         const float* __restrict__ lse,
                                                         float* __restrict__ delta, float* __restrict__ lse2,
                                                         int64_t rows) {
  constexpr int TPR = D / 8;             // threads per row
  constexpr int RPB = 256 / TPR;         // rows per block
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / TPR;
  const int c = tid % TPR;
  float acc = 0.f;
  // The row's lse is loaded first, unconditionally (a clamped, in-bounds
  // index), so that its latency overlaps the O / dO loads.
  const float l = lse[row < rows ? row : rows - 1];
  if (row < rows) {
    const u32x4 g = *reinterpret_cast<const u32x4*>(dout + row * D + 8 * c);
    float ov[8];
    if constexpr (O32) {
      const f32x4* op = reinterpret_cast<const f32x4*>((const float*)o + row * D + 8 * c);
      const f32x4 a = op[0], b = op[1];
      ov[0] = a.x; ov[1] = a.y; ov[2] = a.z; ov[3] = a.w;
      ov[4] = b.x; ov[5] = b.y; ov[6] = b.z; ov[7] = b.w;
    } else {
      const u32x4 ow = *reinterpret_cast<const u32x4*>((const uint16_t*)o + row * D + 8 * c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ov[2 * i] = lo16_to_f32<T>(ow[i]);
        ov[2 * i + 1] = hi16_to_f32<T>(ow[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = __builtin_fmaf(ov[2 * i], lo16_to_f32<T>(g[i]), acc);
      acc = __builtin_fmaf(ov[2 * i + 1], hi16_to_f32<T>(g[i]), acc);
    }
  }
#pragma unroll
  for (int s = TPR / 2; s > 0; s >>= 1) acc += __shfl_xor(acc, s, 64);
  if (row < rows && c == 0) {
    delta[row] = acc;
    lse2[row] = l * kLog2e;
  }
}

// ============================================================ dK / dV pass
// A persistent workgroup of 4 waves owns a unit = (head, 128-key tile); wave w
// owns keys kw0 = k0 + 32w .. kw0+31, keeps their K rows in registers (and
// their V rows too at D = 64; at D >= 128 the unit's V rows stay in LDS, which
// frees the registers for two waves per SIMD at D = 128), and accumulates its
// dK and dV rows in fp32 registers.  Query tiles of 32 rows (Q, dO, lse2, Delta) stream through a
// two-stage LDS ring filled by direct global -> LDS copies.  Per query tile
// the wave computes
//     S  = Q K^T        (A = Q rows from LDS, B = K from registers)
//     dP = dO V^T       (A = dO rows from LDS, B = V)
//     P  = exp2(S c - lse2),  dS = P (dP - Delta)
//     dV^T += dO^T P    (A = dO^T by transposing LDS reads, B = P)
//     dK^T += Q^T dS    (A = Q^T by transposing LDS reads, B = dS)
// with queries as the MFMA rows and keys as the lanes, so that P and dS come
// out of the first two products already in the operand layout of the last two.
template <int D>
struct DkdvTile {
  static constexpr int NW = dkdv_waves(D);       // waves per workgroup
  static constexpr int BK = dkdv_keys(D);        // keys per unit (32 per wave)
  static constexpr int BQ = dkdv_queries(D);     // queries per staged tile
  static_assert(BQ == 32, "one 32-query MFMA block per stage");
  static constexpr bool V_LDS = D >= 128;        // V rows in LDS instead of registers
  static constexpr int QT_BYTES = BQ * D * 2;    // one Q (or dO) tile
  static constexpr int STAT_OFF = 2 * QT_BYTES;  // 64 lse2 values, then 64 Delta values
  static constexpr int STAGE_BYTES = 2 * QT_BYTES + 512;
  static constexpr int V_BYTES = V_LDS ? BK * D * 2 : 0;
  static constexpr int KSTEPS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int QCOPIES = QT_BYTES / 1024;     // 1 KiB copies per Q (or dO) tile
  static constexpr int VCOPIES = V_BYTES / 1024;      // 1 KiB copies per V tile
  static_assert(QCOPIES * 1024 == QT_BYTES && QCOPIES % NW == 0, "tile must split into 1 KiB copies per wave");
  static_assert(VCOPIES % NW == 0, "V tile must split into 1 KiB copies per wave");
  // Copy loops unrolled except at D = 256, where the unrolled form costs
  // registers the accumulators need.
  static constexpr int COPY_UNROLL = D == 256 ? 1 : 16;
  static_assert(BK == NW * 32, "one 32-key block per wave");
  // Waves per SIMD the registers are sized for.  At D = 64 (dK, dV, K and V
  // rows of a wave in 168 registers) three fit: 0.708 -> 0.643 ms on the
  // 128 x 8 x 1024 x 64 workload against two.
  static constexpr int OCC = D == 256 ? 1 : (D == 64 ? 3 : 2);
  // Query tiles handled in pairs with compile-time ring stages (see the LDS
  // declarations).  At D = 256 the doubled loop body costs more registers
  // than the stage-aliasing waits it removes.
  static constexpr bool PAIRS = D <= 128;
  // Causal: a wave whose keys all follow a query tile skips it.  At D = 256
  // the branch around the tile's products made the compiler keep the K rows
  // in scratch and reload them for every query tile: the causal pass of a
  // 128 x 8 x 1024 x 256 bf16 problem took 4.04 ms, more than the non-causal
  // one (2.66 ms).  There the wave runs the products on its masked tile
  // instead (P = 0, so dS = 0 and dK, dV do not change): 1.66 ms.
  // At D = 64 and 128 the skip measured faster (0.695 against 0.726 ms on
  // the causal D = 128 workload).
  static constexpr bool SKIP_IDLE = D <= 128;
};

template <int D, typename T, bool CAUSAL>
__global__ __launch_bounds__(DkdvTile<D>::NW * 64)
__attribute__((amdgpu_waves_per_eu(DkdvTile<D>::OCC, DkdvTile<D>::OCC)))
void fa_bwd_dkdv_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                        const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
                        const float* __restrict__ lse2, const float* __restrict__ delta, uint16_t* __restrict__ dk,
                        uint16_t* __restrict__ dv, int N_max, int ZHkv, int Hkv, int G, int n_ktiles_max,
                        float c2, float scale, int P, const int* __restrict__ cu, int64_t n_tokens) {
  using C = DkdvTile<D>;
  using QTile = CmTile<C::BQ>;
  using VTile = CmTile<C::BK>;
  // One LDS object per ring stage (Q tile, dO tile, lse2 and Delta) and one
  // for the unit's V rows, accessed with compile-time stages (query tiles in
  // pairs), so that the copy of the next query tile provably does not alias
  // the reads of the current one and does not hold them up.
  __shared__ __attribute__((aligned(1024))) char st0[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char st1[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vsm[C::V_LDS ? C::V_BYTES : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_id();
  const int h = lane >> 5;
  const int l32 = lane & 31;
  for (int64_t round = 0;; ++round) {
    int64_t kvh64, kt64;
    if (cu != nullptr) {
      // Packed variable-length batch: one unit per workgroup, key-tile major
      // (the first key tiles, which carry the most query tiles, go first), so
      // that the dispatcher balances units of very different sizes.
      if (round > 0) break;
      kvh64 = blockIdx.x % (uint32_t)ZHkv;
      kt64 = blockIdx.x / (uint32_t)ZHkv;
    } else if (!sched_unit(round, blockIdx.x, P, ZHkv, n_ktiles_max, &kvh64, &kt64)) {
      break;  // uniform
    }
    const int kt = (int)kt64;
    const int k0 = kt * C::BK;
    const int kw0 = k0 + 32 * w;  // first key of this wave
    // The unit's (batch) key/value head serves G query heads (G = 1 without
    // grouping), whose rows lie q_stride rows apart in Q, dO and the
    // statistics: one buffer resource spans the G heads' rows of this
    // problem and member m's rows start at m * q_stride.
    const HeadRows hr = head_rows((uint32_t)kvh64, 0, (uint32_t)Hkv, (uint32_t)G, N_max, cu, n_tokens);
    const int N = hr.n;  // this problem's sequence length
    if (k0 >= N) continue;  // key tile past this sequence (uniform)
    const int q_stride = (int)hr.q_stride;
    const uint32_t head_bytes = (uint32_t)N * D * 2;
    const uint32_t group_rows = (uint32_t)((G - 1) * q_stride + N);
    const size_t kvoff = (size_t)hr.kv_row0 * D;
    const size_t goff = (size_t)hr.q_row0 * D;
    const auto rq = make_rsrc(q + goff, group_rows * D * 2);
    const auto rk = make_rsrc(k + kvoff, head_bytes);
    const auto rv = make_rsrc(v + kvoff, head_bytes);
    const auto rdo = make_rsrc(dout + goff, group_rows * D * 2);
    const auto rl = make_rsrc(lse2 + hr.q_row0, group_rows * 4);
    const auto rd = make_rsrc(delta + hr.q_row0, group_rows * 4);
    const int n_qtiles = (N + C::BQ - 1) / C::BQ;
    const int i0 = (int)sched_first_qtile(kt, C::BK, C::BQ, CAUSAL);
    const int nq = n_qtiles - i0;
    const int n_items = nq * G;  // (member, query tile) pairs, member-major

    // Copy query tile i of member m (Q, dO, and the lse2 / Delta values from
    // its first query on) into ring stage st.
    auto issue_qtile = [&](int m, int i, char* base) {
      const int qq0 = m * q_stride + i * C::BQ;  // row in the group's rows
#pragma unroll(C::COPY_UNROLL)
      for (int x = 0; x < C::QCOPIES / C::NW; ++x) {
        const int blk = w * (C::QCOPIES / C::NW) + x;
        const int sl = blk * 64 + lane;
        const int row = QTile::slot_row(sl), chunk = QTile::slot_chunk(sl);
        const uint32_t off = (uint32_t)(((qq0 + row) * D + 8 * chunk) * 2);
        dma16(rq, base + blk * 1024, off);
        dma16(rdo, base + C::QT_BYTES + blk * 1024, off);
      }
      if (w == 0) dma4(rl, base + C::STAT_OFF, (uint32_t)(qq0 + lane) * 4);
      if (w == 1) dma4(rd, base + C::STAT_OFF + 256, (uint32_t)(qq0 + lane) * 4);
    };

    // Every wave is done with the previous unit's LDS before it is refilled.
    __syncthreads();
    if constexpr (C::V_LDS) {
#pragma unroll(C::COPY_UNROLL)
      for (int x = 0; x < C::VCOPIES / C::NW; ++x) {
        const int blk = w * (C::VCOPIES / C::NW) + x;
        const int sl = blk * 64 + lane;
        const int row = VTile::slot_row(sl), chunk = VTile::slot_chunk(sl);
        dma16(rv, vsm + blk * 1024, (uint32_t)(((k0 + row) * D + 8 * chunk) * 2));
      }
    }
    issue_qtile(0, n_qtiles - 1, st0);

    // K (and V) rows of this wave's keys, B-operand layout (lane = key, k = d).
    u32x4 kf[C::KSTEPS];
    u32x4 vf[C::V_LDS ? 1 : C::KSTEPS];
#pragma unroll
    for (int t = 0; t < C::KSTEPS; ++t) {
      const uint32_t off = (uint32_t)(((kw0 + l32) * D + 16 * t + 8 * h) * 2);
      kf[t] = gload16(rk, off);
      if constexpr (!C::V_LDS) vf[t] = gload16(rv, off);
    }
    f32x16 dka[C::DB], dva[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      dka[db] = f32x16{};
      dva[db] = f32x16{};
    }
    const int key = kw0 + l32;
    // Per-lane LDS read bases: Q / dO rows sigma(l32) as A operands, this
    // wave's V rows as the B operand, Q^T / dO^T through transposing reads.
    const RowRead<C::BQ> qrd(sigma32(l32), h);
    const RowRead<C::BK> vrd(l32, h);
    const char* vbase = vsm + kRowBlockBytes * w;
    const TrRead<C::BQ> trd(lane);

    // Item (member cm, query tile n_qtiles - 1 - cit), read from stage cs; the
    // copy of the next item goes to ns.  Query tiles are taken from the last
    // down: the units of one head (which run at the same time on one XCD)
    // then read the same query tiles at about the same time and share them
    // through L2 (with the causal mask they start on different first tiles
    // when walking up).  0.746 -> 0.728 ms on the causal D128 workload.
    int cm = 0, cit = 0;
    auto qtile = [&](const char* cs, char* ns) {
      // The item has landed for every wave; every wave is done with the last.
      wait_vmem();
      __syncthreads();
      const int it = cit;
      const bool wrap = cit + 1 == nq;
      const int nm = wrap ? cm + 1 : cm;
      cit = wrap ? 0 : cit + 1;
      if (nm < G) issue_qtile(nm, n_qtiles - 1 - cit, ns);
      cm = nm;
      const int qb0 = (n_qtiles - 1 - it) * C::BQ;  // first query of the tile
      // Causal: a tile whose last query precedes the wave's first key is empty.
      if (CAUSAL && C::SKIP_IDLE && qb0 + 31 < kw0) return;
      const char* qt = cs;
      const char* dot = qt + C::QT_BYTES;
      const float* stats = reinterpret_cast<const float*>(qt + C::STAT_OFF);
      f32x16 s = f32x16{}, dp = f32x16{};
      read_ahead<C::KSTEPS>(
          [&](int t) {
            u32x4 vb;
            if constexpr (C::V_LDS)
              vb = lds_read16(vbase, vrd.at(t));
            else
              vb = vf[t];
            return U4x3{lds_read16(qt, qrd.at(t)), lds_read16(dot, qrd.at(t)), vb};
          },
          [&](int t, const U4x3& x) {
            s = mfma32<T>(x.a, kf[t], s);
            dp = mfma32<T>(x.b, x.c, dp);
          });
      // Register jj holds query qb0 + 16(jj/8) + 8h + jj%8 for key kw0 + l32.
      // Each half (t2) of the registers is finished and fed to the dV / dK
      // products before the next, which keeps fewer values live.
      const bool need_mask = (CAUSAL && qb0 < kw0 + 31) || (qb0 + 32 > N);
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const int qi = 16 * t2 + 8 * h;
        const f32x4 la = *reinterpret_cast<const f32x4*>(stats + qi);
        const f32x4 lb = *reinterpret_cast<const f32x4*>(stats + qi + 4);
        const f32x4 da = *reinterpret_cast<const f32x4*>(stats + 64 + qi);
        const f32x4 dbv = *reinterpret_cast<const f32x4*>(stats + 64 + qi + 4);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int jj = 8 * t2 + i;
          const float l2 = i < 4 ? la[i & 3] : lb[i & 3];
          s[jj] = __builtin_fmaf(s[jj], c2, -l2);  // log2 of P
        }
        // Only the tile on the wave's diagonal and a ragged last tile are
        // masked; the (uniform) branch keeps the selects off every other tile.
        if (need_mask) {
          keep_branch();
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int query = qb0 + qi + i;
            if ((CAUSAL && key > query) || query >= N) s[8 * t2 + i] = -__builtin_inff();
          }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int jj = 8 * t2 + i;
          const float dl = i < 4 ? da[i & 3] : dbv[i & 3];
          const float p = fast_exp2(s[jj]);  // exp2(-inf) = 0
          s[jj] = p;
          dp[jj] = p * (dp[jj] - dl);
        }
        const u32x4 pf = pack8<T>(s, 8 * t2);
        const u32x4 dsf = pack8<T>(dp, 8 * t2);
        read_ahead<C::DB>(
            [&](int db) {
              return U4x2{lds_read_tr_operand<C::BQ>(dot, trd, 16 * t2, db),
                          lds_read_tr_operand<C::BQ>(qt, trd, 16 * t2, db)};
            },
            [&](int db, const U4x2& x) {
              dva[db] = mfma32<T>(x.a, pf, dva[db]);
              dka[db] = mfma32<T>(x.b, dsf, dka[db]);
            });
      }
    };
    if constexpr (C::PAIRS) {
      for (int f = 0; f < n_items; f += 2) {
        qtile(st0, st1);
        if (f + 1 < n_items) qtile(st1, st0);
      }
    } else {
      for (int f = 0; f < n_items; ++f) qtile((f & 1) ? st1 : st0, (f & 1) ? st0 : st1);
    }

    // Single write of this wave's dK and dV rows.  Register jj of block db
    // holds d = 32db + 16(jj/8) + 8h + jj%8 of key kw0 + l32.
    const auto rdk = make_rsrc(dk + kvoff, head_bytes);
    const auto rdv = make_rsrc(dv + kvoff, head_bytes);
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      // Element by element: the vector-times-scalar form kept a register per
      // element for the (uniform) scale.
      f32x16 ks;
#pragma unroll
      for (int i = 0; i < 16; ++i) ks[i] = dka[db][i] * scale;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const uint32_t off = (uint32_t)((key * D + 32 * db + 16 * half + 8 * h) * 2);
        gstore16(rdk, off, pack8<T>(ks, 8 * half));
        gstore16(rdv, off, pack8<T>(dva[db], 8 * half));
      }
    }
  }
}

// ============================================================ dQ pass
// A workgroup of 4 waves owns a query tile of 128 queries of one head (32 per
// wave, kept in registers together with their dO rows, lse2 and Delta); two
// (D = 128) or three (D = 64) workgroups share a compute unit.  With the
// causal mask a workgroup owns two tiles, a long and a short one, so every
// workgroup has the same work, and finishes them one after the other; the
// second tile's rows and first K/V tile are fetched while the first finishes.  K/V
// tiles stream through a two-stage LDS ring filled by direct global -> LDS
// copies.  Per key tile the wave computes, transposed so that each lane owns
// one query,
//     S^T  = K Q^T,  dP^T = V dO^T          (A = K/V rows from LDS)
//     P^T  = exp2(S^T c - lse2),  dS^T = P^T (dP^T - Delta)
//     dQ^T += K^T dS^T                      (A = K^T by transposing LDS reads)
// The workgroups of one head run back to back on one XCD.
template <int D>
struct DqTile {
  static constexpr int NW = 4;
  static constexpr int BM = NW * 32;
  static constexpr int BN = D == 64 ? 64 : 32;
  static constexpr int KB = BN / 32;
  static constexpr int TILE_BYTES = BN * D * 2;
  static constexpr int KSTEPS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int DMA = TILE_BYTES / (NW * 1024);
  static_assert(DMA * NW * 1024 == TILE_BYTES, "tile must split into 1 KiB copies per wave");
  static constexpr int OCC = D == 256 ? 1 : (D == 128 ? 2 : 3);  // waves per SIMD (registers)
  // The causal kernel at D = 64 needs 176-188 registers (masks, the second
  // tile of each pair): at three waves per SIMD (168) it spilled in the key
  // tile loop; two measured faster (dQ 0.357 -> 0.352 ms on the causal
  // 128 x 8 x 1024 x 64 workload).
  static constexpr int occ(bool causal) { return (D == 64 && causal) ? 2 : OCC; }
  // Causal: a wave whose queries all precede a key tile skips it, except at
  // D = 256, where the masked products run instead (P = 0, dQ unchanged):
  // the branch cost 50 registers there and the causal pass 1.49 -> 1.31 ms
  // on a 128 x 8 x 1024 x 256 bf16 problem without it; at D = 64 and 128 the
  // skip measured faster.
  static constexpr bool SKIP_IDLE = D <= 128;
  // Key tiles in pairs with compile-time ring stages (as in the dK/dV pass).
  static constexpr bool PAIRS = D <= 128;
};

// Where the dQ pass gets its row statistics: kStatsIn reads lse2 and Delta
// from the preprocess pass; kStatsO16 / kStatsO32 compute them itself from
// lse and the O rows (16-bit or fp32 O) and dO rows it loads anyway, and
// write them for the dK/dV pass, which then needs no preprocess pass.
enum DqStats { kStatsIn = 0, kStatsO16 = 1, kStatsO32 = 2 };

template <int D, typename T, bool CAUSAL, int STATS>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(DqTile<D>::occ(CAUSAL), DqTile<D>::occ(CAUSAL))))
void fa_bwd_dq_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                      const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
                      const float* __restrict__ lse2, const float* __restrict__ delta, uint16_t* __restrict__ dq,
                      int N_max, int64_t plane, int n_qtiles_max, float c2, float scale,
                      const void* __restrict__ o, const float* __restrict__ lse, float* __restrict__ stats_out,
                      int ZHkv, int Hkv, int G, const int* __restrict__ cu, int64_t n_tokens) {
  using C = DqTile<D>;
  using Tile = CmTile<C::BN>;
  // One LDS object per ring stage and operand, accessed with compile-time
  // stages (tiles in pairs), so that the copy of tile j+1 provably does not
  // alias the reads of tile j and does not hold them up.
  __shared__ __attribute__((aligned(1024))) char k0s[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v0s[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char k1s[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v1s[C::TILE_BYTES];
  // With 16-bit O and the statistics computed here, the O rows of a query
  // tile are copied into LDS ahead of use (see finish_rows).
  constexpr bool O_LDS = STATS == kStatsO16 && D <= 128;
  using OTile = CmTile<C::BM>;
  constexpr int O_BYTES = C::BM * D * 2;
  __shared__ __attribute__((aligned(1024))) char osm[O_LDS ? O_BYTES : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  // The same index as a scalar, for the LDS destinations of the tile copies
  // (kept separate from w: the divergent form gives better register use for
  // the rest of this kernel).
  const int ws = wave_id();
  const int h = lane >> 5;
  const int l32 = lane & 31;
  // Query tiles of this workgroup: one, or with the causal mask a long and a
  // short one of the same head.  The grid is dealt over (batch key/value
  // head, member, slot) for the longest sequence; blocks past their own
  // sequence's tiles have no work.
  uint32_t kvh_u, head_u, slot_u, qt_a_u, qt_b_u;
  xcd_tile_grouped(blockIdx.x, (uint32_t)G, (uint32_t)paired_groups(n_qtiles_max, CAUSAL), &kvh_u, &head_u, &slot_u);
  if (kvh_u >= (uint32_t)ZHkv) return;  // padding block
  const HeadRows hr = head_rows(kvh_u, head_u - kvh_u * (uint32_t)G, (uint32_t)Hkv, (uint32_t)G, N_max, cu, n_tokens);
  const int N = hr.n;  // this problem's sequence length
  const int n_qtiles = (N + C::BM - 1) / C::BM;
  if (slot_u >= (uint32_t)paired_groups(n_qtiles, CAUSAL)) return;  // past this sequence (uniform)
  const int n_items = paired_items(slot_u, n_qtiles, CAUSAL, &qt_a_u, &qt_b_u);
  const int qt_a = (int)qt_a_u, qt_b = (int)qt_b_u;
  const size_t hoff = (size_t)hr.q_row0 * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const size_t kvoff = (size_t)hr.kv_row0 * D;
  const auto rq = make_rsrc(q + hoff, head_bytes);
  const auto rk = make_rsrc(k + kvoff, head_bytes);
  const auto rv = make_rsrc(v + kvoff, head_bytes);
  const auto rdo = make_rsrc(dout + hoff, head_bytes);
  const auto rl = STATS == kStatsIn ? make_rsrc(lse2 + hr.q_row0, (uint32_t)N * 4)
                                    : make_rsrc(lse + hr.q_row0, (uint32_t)N * 4);
  const auto rdl = make_rsrc(delta + hr.q_row0, (uint32_t)N * 4);
  const auto rdq = make_rsrc(dq + hoff, head_bytes);
  auto n_tiles = [&](int qt) {
    const int kv_end = CAUSAL ? min(N, (qt + 1) * C::BM) : N;
    return (kv_end + C::BN - 1) / C::BN;
  };

  auto issue_tile = [&](int j, char* kdst, char* vdst) {
    const int kv0 = j * C::BN;
#pragma unroll
    for (int i = 0; i < C::DMA; ++i) {
      const int blk = ws * C::DMA + i;
      const int sl = blk * 64 + lane;
      const int row = Tile::slot_row(sl), chunk = Tile::slot_chunk(sl);
      const uint32_t off = (uint32_t)(((kv0 + row) * D + 8 * chunk) * 2);
      dma16(rk, kdst + blk * 1024, off);
      dma16(rv, vdst + blk * 1024, off);
    }
  };
  // The wave's query rows of tile qt: Q and dO in B-operand layout (lane =
  // query, k = d), lse2 and Delta.
  u32x4 qf[C::KSTEPS], dof[C::KSTEPS];
  float l2 = 0.f, dl = 0.f;
  auto load_rows = [&](int qt) {
    const int query = qt * C::BM + 32 * w + l32;
#pragma unroll
    for (int t = 0; t < C::KSTEPS; ++t) {
      const uint32_t off = (uint32_t)((query * D + 16 * t + 8 * h) * 2);
      qf[t] = gload16(rq, off);
      dof[t] = gload16(rdo, off);
    }
    if constexpr (STATS == kStatsIn) {
      l2 = gload_f32(rl, (uint32_t)query * 4);
      dl = gload_f32(rdl, (uint32_t)query * 4);
    } else {
      l2 = gload_f32(rl, (uint32_t)query * 4) * kLog2e;
    }
  };
  // Row statistics of tile qt computed here (STATS != kStatsIn), once its dO
  // rows are in registers: Delta = sum_d O * dO, in the exact order of the
  // preprocess pass (there D/8 threads each sum one 8-element chunk c of the
  // row with an fma chain and combine the chunks with an xor butterfly over c;
  // here lane half h holds the chunks c = 2t + h, so every butterfly level
  // but the last pairs chunks inside a lane and the last pairs the halves),
  // so that both paths give the same bits.  lse2 and Delta are then written
  // for the dK/dV pass.  16-bit O rows at D <= 128 come from LDS, copied there
  // one item ahead (issue_o), so their latency is hidden; fp32 O rows, and
  // the 64 KiB of a D = 256 tile, are loaded here.
  auto issue_o = [&](int qt) {
    if constexpr (O_LDS) {
      const auto ro = make_rsrc((const uint16_t*)o + hoff, head_bytes);
      const int q0 = qt * C::BM;
#pragma unroll
      for (int x = 0; x < O_BYTES / 1024 / C::NW; ++x) {
        const int blk = ws * (O_BYTES / 1024 / C::NW) + x;
        const int sl = blk * 64 + lane;
        const int row = OTile::slot_row(sl), chunk = OTile::slot_chunk(sl);
        dma16(ro, osm + blk * 1024, (uint32_t)(((q0 + row) * D + 8 * chunk) * 2));
      }
    }
  };
  auto finish_rows = [&](int qt) {
    if constexpr (STATS != kStatsIn) {
      const int query = qt * C::BM + 32 * w + l32;
      const RowRead<C::BM> ord(32 * w + l32, h);
      float part[C::KSTEPS];
#pragma unroll
      for (int t = 0; t < C::KSTEPS; ++t) {
        float ov[8];
        if constexpr (STATS == kStatsO32) {
          const auto ro = make_rsrc((const float*)o + hoff, (uint32_t)N * D * 4);
          const uint32_t off = (uint32_t)((query * D + 16 * t + 8 * h) * 4);
          const u32x4 a = gload16(ro, off), b = gload16(ro, off + 16);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ov[i] = __uint_as_float(a[i]);
            ov[4 + i] = __uint_as_float(b[i]);
          }
        } else {
          u32x4 a;
          if constexpr (O_LDS) {
            a = lds_read16(osm, ord.at(t));
          } else {
            const auto ro = make_rsrc((const uint16_t*)o + hoff, head_bytes);
            a = gload16(ro, (uint32_t)((query * D + 16 * t + 8 * h) * 2));
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ov[2 * i] = lo16_to_f32<T>(a[i]);
            ov[2 * i + 1] = hi16_to_f32<T>(a[i]);
          }
        }
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc = __builtin_fmaf(ov[2 * i], lo16_to_f32<T>(dof[t][i]), acc);
          acc = __builtin_fmaf(ov[2 * i + 1], hi16_to_f32<T>(dof[t][i]), acc);
        }
        part[t] = acc;
      }
#pragma unroll
      for (int sx = C::KSTEPS / 2; sx >= 1; sx >>= 1) {
        float nxt[C::KSTEPS];
#pragma unroll
        for (int t = 0; t < C::KSTEPS; ++t) nxt[t] = part[t] + part[t ^ sx];
#pragma unroll
        for (int t = 0; t < C::KSTEPS; ++t) part[t] = nxt[t];
      }
      dl = half_swap_sum(part[0]);
      if (h == 0) {
        gstore_f32(make_rsrc(stats_out + hr.q_row0, (uint32_t)N * 4), (uint32_t)query * 4, dl);
        gstore_f32(make_rsrc(stats_out + plane + hr.q_row0, (uint32_t)N * 4), (uint32_t)query * 4, l2);
      }
    }
  };

  // Per-lane LDS read bases: K / V rows 32 kb + sigma(l32) as A operands,
  // K^T through transposing reads.
  const RowRead<C::BN> krd(sigma32(l32), h);
  const TrRead<C::BN> trd(lane);

  issue_tile(0, k0s, v0s);
  issue_o(qt_a);
  load_rows(qt_a);
  bool first_tile_issued = true;
  bool o_issued = true;  // the current item's O rows are on their way to osm
  for (int it = 0; it < n_items; ++it) {
    const int qt = it == 0 ? qt_a : qt_b;
    const int q0 = qt * C::BM;
    const int wq0 = q0 + 32 * w;
    const int query = wq0 + l32;
    const int nt = n_tiles(qt);
    const bool more = it + 1 < n_items;
    // With an even tile count the next item's first tile follows in the
    // same ring (it lands in stage 0): copy it, and load the next rows,
    // during this item's last tile.
    const bool chain = more && (nt % 2 == 0);
    if (!first_tile_issued) issue_tile(0, k0s, v0s);
    if (!o_issued) issue_o(qt);  // (an item of one key tile came before)
    // fp32 O: the statistics right away; 16-bit O: in the first key step,
    // once the copy into osm has landed.
    if constexpr (!O_LDS) finish_rows(qt);

    f32x16 dqa[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) dqa[db] = f32x16{};

    // Key tile j, read from kt/vt; the copy of tile j+1 goes to kn/vn.
    auto tile = [&](int j, const char* kt, const char* vt, char* kn, char* vn) {
      wait_vmem();
      __syncthreads();
      if (j + 1 < nt)
        issue_tile(j + 1, kn, vn);
      else if (chain)
        issue_tile(0, kn, vn);
      if constexpr (O_LDS) {
        if (j == 0) finish_rows(qt);
        // Every wave has read osm (in step 0): copy the next item's O rows.
        if (j == 1 && more) issue_o(qt_b);
      }
      const int kv0 = j * C::BN;
      const bool active = !CAUSAL || !C::SKIP_IDLE || kv0 <= wq0 + 31;
      f32x16 s[C::KB], dp[C::KB];
      if (active) {
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
          s[kb] = f32x16{};
          dp[kb] = f32x16{};
        }
        read_ahead<C::KSTEPS * C::KB>(
            [&](int n) {
              const int off = krd.at(n / C::KB) + kRowBlockBytes * (n % C::KB);
              return U4x2{lds_read16(kt, off), lds_read16(vt, off)};
            },
            [&](int n, const U4x2& x) {
              const int t = n / C::KB, kb = n % C::KB;
              s[kb] = mfma32<T>(x.a, qf[t], s[kb]);
              dp[kb] = mfma32<T>(x.b, dof[t], dp[kb]);
            });
        // Keep that order: the reads of step n + 1, then the products of step n
        // (scheduling groups in sequence: mask 0x100 = LDS reads, 0x008 =
        // matrix instructions, two of each per step).
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int n = 0; n + 1 < C::KSTEPS * C::KB; ++n) {
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
      // This item's rows are not needed any more: load the next item's.
      const float l2c = l2, dlc = dl;
      if (j == nt - 1 && more) load_rows(qt_b);
      if (!active) return;
      const bool need_mask = (CAUSAL && kv0 + C::BN - 1 > wq0) || (kv0 + C::BN > N);
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) s[kb][jj] = __builtin_fmaf(s[kb][jj], c2, -l2c);  // log2 of P
        // Only tiles on the wave's diagonal and a ragged last tile are
        // masked; the (uniform) branch keeps the selects off every other tile.
        if (need_mask) {
          keep_branch();
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) {
            const int key = kv0 + 32 * kb + 16 * (jj >> 3) + 8 * h + (jj & 7);
            if ((CAUSAL && key > query) || key >= N) s[kb][jj] = -__builtin_inff();
          }
        }
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const float p = fast_exp2(s[kb][jj]);  // exp2(-inf) = 0
          dp[kb][jj] = p * (dp[kb][jj] - dlc);
        }
      }
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const u32x4 dsf = pack8<T>(dp[kb], 8 * t2);
#pragma unroll
          for (int db = 0; db < C::DB; ++db)
            dqa[db] = mfma32<T>(lds_read_tr_operand<C::BN>(kt, trd, 32 * kb + 16 * t2, db), dsf, dqa[db]);
        }
    };
    if constexpr (C::PAIRS) {
      for (int j = 0; j < nt; j += 2) {
        tile(j, k0s, v0s, k1s, v1s);
        if (j + 1 < nt) tile(j + 1, k1s, v1s, k0s, v0s);
      }
    } else {
      for (int j = 0; j < nt; ++j) {
        const bool odd = j & 1;
        tile(j, odd ? k1s : k0s, odd ? v1s : v0s, odd ? k0s : k1s, odd ? v0s : v1s);
      }
    }

#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      f32x16 y;
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = dqa[db][i] * scale;
#pragma unroll
      for (int half = 0; half < 2; ++half)
        gstore16(rdq, (uint32_t)((query * D + 32 * db + 16 * half + 8 * h) * 2), pack8<T>(y, 8 * half));
    }
    first_tile_issued = chain;
    o_issued = nt > 1;
    if (more && !chain) {
      // The ring restarts at stage 0 for the next item; every wave must be
      // done with this item's last tile before it is overwritten.
      __syncthreads();
    }
  }
}

// ============================================================ launchers
template <int D, typename T, bool O32>
static hipError_t launch_pre_t(const BwdArgs& a) {
  constexpr int RPB = 256 / (D / 8);
  const int64_t rows = a.rows();
  const dim3 grid((unsigned)((rows + RPB - 1) / RPB));
  hipLaunchKernelGGL((fa_bwd_pre_kernel<D, T, O32>), grid, dim3(256), 0, a.stream, a.o,
                     (const uint16_t*)a.dout, a.lse, a.stats, a.stats + rows, rows);
  return hipGetLastError();
}
template <int D, typename T>
static hipError_t launch_pre_d(const BwdArgs& a) {
  return a.o_dtype == F32::code ? launch_pre_t<D, T, true>(a) : launch_pre_t<D, T, false>(a);
}
template <typename T>
static hipError_t launch_pre_dt(const BwdArgs& a) {
  switch (a.D) {
    case 64: return launch_pre_d<64, T>(a);
    case 128: return launch_pre_d<128, T>(a);
    default: return launch_pre_d<256, T>(a);
  }
}
hipError_t launch_bwd_pre(const BwdArgs& a) {
  return a.dtype == BF16::code ? launch_pre_dt<BF16>(a) : launch_pre_dt<F16>(a);
}

template <int D, typename T, bool CAUSAL>
static hipError_t launch_dkdv_t(const BwdArgs& a) {
  using C = DkdvTile<D>;
  const int ZHkv = (int)(a.Z * a.Hkv);
  const int G = (int)(a.H / a.Hkv);
  const int n_kt = (int)((a.N + C::BK - 1) / C::BK);
  // Packed batches: one workgroup per (sequence key/value head, key tile) of
  // the longest sequence (units past a sequence's end exit at once).
  const int64_t grid = a.cu_seqlens ? (int64_t)ZHkv * n_kt : (int64_t)a.num_programs;
  hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, T, CAUSAL>), dim3((unsigned)grid), dim3(C::NW * 64), 0,
                     a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (const uint16_t*)a.dout, a.stats + a.rows(), a.stats, (uint16_t*)a.dk, (uint16_t*)a.dv,
                     (int)a.N, ZHkv, (int)a.Hkv, G, n_kt, a.scale * kLog2e, a.scale, a.num_programs, a.cu_seqlens,
                     a.T);
  return hipGetLastError();
}
template <int D, typename T>
static hipError_t launch_dkdv_d(const BwdArgs& a) {
  return a.causal ? launch_dkdv_t<D, T, true>(a) : launch_dkdv_t<D, T, false>(a);
}
template <typename T>
static hipError_t launch_dkdv_dt(const BwdArgs& a) {
  switch (a.D) {
    case 64: return launch_dkdv_d<64, T>(a);
    case 128: return launch_dkdv_d<128, T>(a);
    default: return launch_dkdv_d<256, T>(a);
  }
}
hipError_t launch_bwd_dkdv(const BwdArgs& a) {
  return a.dtype == BF16::code ? launch_dkdv_dt<BF16>(a) : launch_dkdv_dt<F16>(a);
}

template <int D, typename T>
static hipError_t occ_dkdv(int* out) {
  int n = 0;
  constexpr int threads = DkdvTile<D>::NW * 64;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fa_bwd_dkdv_kernel<D, T, true>, threads, 0);
  if (e != hipSuccess) return e;
  int n2 = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n2, fa_bwd_dkdv_kernel<D, T, false>, threads, 0);
  if (e != hipSuccess) return e;
  *out = n < n2 ? n : n2;
  if (*out < 1) *out = 1;
  return hipSuccess;
}
hipError_t dkdv_blocks_per_cu(int D, int dtype, int* out) {
  const bool bf = dtype == BF16::code;
  switch (D) {
    case 64: return bf ? occ_dkdv<64, BF16>(out) : occ_dkdv<64, F16>(out);
    case 128: return bf ? occ_dkdv<128, BF16>(out) : occ_dkdv<128, F16>(out);
    default: return bf ? occ_dkdv<256, BF16>(out) : occ_dkdv<256, F16>(out);
  }
}

template <int D, typename T, bool CAUSAL, int STATS>
static hipError_t launch_dq_t(const BwdArgs& a) {
  using C = DqTile<D>;
  const int ZHkv = (int)(a.Z * a.Hkv);
  const int G = (int)(a.H / a.Hkv);
  const int n_qt = (int)((a.N + C::BM - 1) / C::BM);
  hipLaunchKernelGGL((fa_bwd_dq_kernel<D, T, CAUSAL, STATS>),
                     dim3((unsigned)xcd_grid_grouped(ZHkv, G, paired_groups(n_qt, CAUSAL))), dim3(256), 0,
                     a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (const uint16_t*)a.dout, a.stats + a.rows(), a.stats, (uint16_t*)a.dq, (int)a.N, a.rows(), n_qt,
                     a.scale * kLog2e, a.scale, a.o, a.lse, a.stats, ZHkv, (int)a.Hkv, G, a.cu_seqlens, a.T);
  return hipGetLastError();
}
template <int D, typename T, int STATS>
static hipError_t launch_dq_s(const BwdArgs& a) {
  return a.causal ? launch_dq_t<D, T, true, STATS>(a) : launch_dq_t<D, T, false, STATS>(a);
}
template <int D, typename T>
static hipError_t launch_dq_d(const BwdArgs& a) {
  if (!a.dq_stats) return launch_dq_s<D, T, kStatsIn>(a);
  return a.o_dtype == F32::code ? launch_dq_s<D, T, kStatsO32>(a) : launch_dq_s<D, T, kStatsO16>(a);
}
template <typename T>
static hipError_t launch_dq_dt(const BwdArgs& a) {
  switch (a.D) {
    case 64: return launch_dq_d<64, T>(a);
    case 128: return launch_dq_d<128, T>(a);
    default: return launch_dq_d<256, T>(a);
  }
}
hipError_t launch_bwd_dq(const BwdArgs& a) {
  return a.dtype == BF16::code ? launch_dq_dt<BF16>(a) : launch_dq_dt<F16>(a);
}

}  // namespace fa
