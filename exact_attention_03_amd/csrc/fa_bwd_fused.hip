// fa_bwd_fused.hip - the backward as one pass per head: dQ, dK and dV of a
// whole head from one persistent workgroup.
//
// [FA-Ascend] = the page "把 FlashAttention 搬上昇腾：Triton-Ascend CV Pipeline
// 优化实战" (BiumBiu).  §五 runs a fixed number of persistent programs that
// claim heads with a fixed stride, each program computing everything of its
// heads; §二 gives the backward (P recomputed from the saved row statistic,
// dP = dO V^T, dS = scale P (dP - Delta), dQ = dS K, dK = dS^T Q,
// dV = P^T dO) and its rules: each gradient tile has a single writer and the
// scratch does not grow with N^2.
//
// Here a workgroup of NW waves is one program.  For each of its heads it walks
// the key tiles (32 keys per wave) in order; for a key tile it keeps the K
// tile in LDS, the wave's V rows in registers and its dK / dV rows in fp32
// registers, and streams the query tiles (32 queries: Q, dO, lse2, Delta)
// through a two-stage LDS ring.  Per query tile each wave computes, with keys
// on the lanes as in the dK/dV pass,
//     S = Q K^T,  dP = dO V^T,  P = exp2(S c - lse2),  dS = P (dP - Delta)
//     dV^T += dO^T P,  dK^T += Q^T dS
// and writes its dS^T block into LDS; then every wave takes its share of
//     dQ^T (of the query tile) += K^T dS^T   over the key tile's keys
// (16 x 16 x 32 products: A = K^T and B = dS^T both through transposing LDS
// reads) and adds it to the head's dQ partial, an fp32 copy of dQ in the
// caller's workspace (one per head, N x D, never N^2).  Because key tiles are
// taken in order, the key tile holding a query tile's last visible key (the
// last key tile without the causal mask) is the last contribution: that one
// writes the finished dQ rows (times scale, in the input type) instead of the
// partial, and the first (key tile 0) starts from zero instead of reading it.
// Every dQ, dK and dV element is written by one workgroup, once; no atomics.
// Against the two-pass form this runs the five products of §二 instead of
// seven (the dQ pass recomputes S and dP), at the price of the partial's
// traffic: one fp32 read and write of a query tile's dQ per (key tile, query
// tile) pair.
#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_schedule.h"

namespace fa {

template <int D>
struct FusedTile {
  // Waves per workgroup (32 keys each).  At D = 128 a key tile of 256 keys
  // (one workgroup per CU) halves the partial's traffic per key against 128
  // keys and leaves each wave one 16-wide dQ channel block.
  static constexpr int NW = D == 128 ? 8 : 4;
  static constexpr int BK = 32 * NW;               // keys per key tile
  static constexpr int BQ = 32;                    // queries per staged query tile
  static constexpr int KSTEPS = D / 16;            // k steps of the score products
  static constexpr int DB = D / 32;                // 32-wide channel blocks of dK, dV
  static constexpr int DQB = D / (16 * NW);        // 16-wide channel blocks of dQ per wave
  static constexpr int NB = 2 * DQB;               // 16 x 16 dQ blocks per wave (two 16-query blocks each)
  static_assert(DQB >= 1 && DQB * 16 * NW == D, "dQ channel blocks split evenly over the waves");
  static constexpr int QT_BYTES = BQ * D * 2;      // one Q (or dO) tile
  static constexpr int STAT_OFF = 2 * QT_BYTES;    // 64 lse2 values, then 64 Delta values
  static constexpr int STAGE_BYTES = 2 * QT_BYTES + 512;
  static constexpr int K_BYTES = BK * D * 2;
  static constexpr int DS_BYTES = BK * BQ * 2;     // dS^T of one query tile: rows = keys, 32 query columns
  static constexpr int QCOPIES = QT_BYTES / 1024;  // 1 KiB copies per Q (or dO) tile
  static constexpr int KCOPIES = K_BYTES / 1024;
  static_assert(QCOPIES % NW == 0 && KCOPIES % NW == 0, "copies split evenly over the waves");
  // Two dS^T buffers: query tile i's dQ product runs at the start of tile i+1
  // and shares its barrier.  (At D = 128, 4 waves of 128 keys with a single
  // buffer and a second barrier per tile fit two workgroups per CU, but
  // measured 1.43 against 1.21 ms on the causal workload: twice the partial's
  // traffic per key.)
  static constexpr int OCC = D == 64 ? 3 : (D == 128 ? 2 : 1);  // waves per SIMD the registers are sized for
  // The partial of tile i is loaded at the start of tile i (and used at the
  // start of tile i+1), except at D = 256, whose registers go to dK and dV.
  static constexpr bool PREFETCH = D != 256;
  static constexpr int COPY_UNROLL = D == 256 ? 1 : 16;
};

template <int D, typename T, bool CAUSAL>
__global__ __launch_bounds__(FusedTile<D>::NW * 64)
__attribute__((amdgpu_waves_per_eu(FusedTile<D>::OCC, FusedTile<D>::OCC)))
void fa_bwd_fused_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                         const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
                         const float* __restrict__ lse2, const float* __restrict__ delta,
                         uint16_t* __restrict__ dq, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
                         float* __restrict__ partial, int N, int ZH, float c2, float scale, int P) {
  using C = FusedTile<D>;
  using QTile = CmTile<C::BQ>;
  using KTile = CmTile<C::BK>;
  constexpr int NW = C::NW, BK = C::BK, BQ = C::BQ;
  __shared__ __attribute__((aligned(1024))) char st0[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char st1[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char ksm[C::K_BYTES];
  __shared__ __attribute__((aligned(1024))) char ds0[C::DS_BYTES];
  __shared__ __attribute__((aligned(1024))) char ds1[C::DS_BYTES];

  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int g16 = lane >> 4;
  const int n_kt = (N + BK - 1) / BK;
  const int n_qt = (N + BQ - 1) / BQ;
  const uint32_t head_bytes = (uint32_t)N * D * 2;

  // Per-lane LDS read bases: Q / dO rows sigma(l32) as A operands, this
  // wave's K rows as the B operand of S, Q^T / dO^T through transposing
  // reads, and the 16-row transposing reads of K^T and dS^T for dQ.
  const RowRead<BQ> qrd(sigma32(l32), h);
  const RowRead<BK> krd(l32, h);
  const TrRead<BQ> trd(lane);
  const TrRead16<BK> tr16(lane);
  const char* kbase = ksm + kRowBlockBytes * w;

  for (int head = blockIdx.x; head < ZH; head += P) {  // fixed stride over heads ([FA-Ascend] §五)
    const size_t hoff = (size_t)head * N * D;
    const auto rq = make_rsrc(q + hoff, head_bytes);
    const auto rk = make_rsrc(k + hoff, head_bytes);
    const auto rv = make_rsrc(v + hoff, head_bytes);
    const auto rdo = make_rsrc(dout + hoff, head_bytes);
    const auto rl = make_rsrc(lse2 + (size_t)head * N, (uint32_t)N * 4);
    const auto rd = make_rsrc(delta + (size_t)head * N, (uint32_t)N * 4);
    const auto rdq = make_rsrc(dq + hoff, head_bytes);
    // this head's dQ partial, laid out per (query tile, wave, block, lane) so
    // that every lane moves its own 16 bytes per block
    float* part = partial + (size_t)head * n_qt * BQ * D;

    // Copy query tile i (Q, dO, and lse2 / Delta from its first query on) into a ring stage.
    auto issue_item = [&](int i, char* base) {
      const int qq0 = i * BQ;
#pragma unroll C::COPY_UNROLL
      for (int x = 0; x < C::QCOPIES / NW; ++x) {
        const int blk = w * (C::QCOPIES / NW) + x;
        const int sl = blk * 64 + lane;
        const int row = QTile::slot_row(sl), chunk = QTile::slot_chunk(sl);
        const uint32_t off = (uint32_t)(((qq0 + row) * D + 8 * chunk) * 2);
        dma16(rq, base + blk * 1024, off);
        dma16(rdo, base + C::QT_BYTES + blk * 1024, off);
      }
      if (w == 0) dma4(rl, base + C::STAT_OFF, (uint32_t)(qq0 + lane) * 4);
      if (w == 1) dma4(rd, base + C::STAT_OFF + 256, (uint32_t)(qq0 + lane) * 4);
    };

    for (int kt = 0; kt < n_kt; ++kt) {
      const int k0 = kt * BK;
      const int kw0 = k0 + 32 * w;  // first key of this wave
      const int key = kw0 + l32;
      const int i0 = (int)sched_first_qtile(kt, BK, BQ, CAUSAL);
      const int nq = n_qt - i0;

      // Every wave is done with the previous key tile's LDS (K tile, ring, dS^T).
      __syncthreads();
#pragma unroll C::COPY_UNROLL
      for (int x = 0; x < C::KCOPIES / NW; ++x) {
        const int blk = w * (C::KCOPIES / NW) + x;
        const int sl = blk * 64 + lane;
        const int row = KTile::slot_row(sl), chunk = KTile::slot_chunk(sl);
        dma16(rk, ksm + blk * 1024, (uint32_t)(((k0 + row) * D + 8 * chunk) * 2));
      }
      issue_item(i0, st0);
      // V rows of this wave's keys, B-operand layout (lane = key, k = d).
      u32x4 vf[C::KSTEPS];
#pragma unroll
      for (int t = 0; t < C::KSTEPS; ++t) vf[t] = gload16(rv, (uint32_t)((key * D + 16 * t + 8 * h) * 2));
      f32x16 dka[C::DB], dva[C::DB];
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        dka[db] = f32x16{};
        dva[db] = f32x16{};
      }

      // dQ of query tile i from the dS^T of every wave of this key tile (in
      // dsr): this wave's channel blocks, added to the partial (loaded into
      // acc by dq_load one step ahead, so that its latency is hidden), or
      // written out on the tile's last contribution.
      f32x4 acc[C::NB];
      auto dq_load = [&](int i) {
        const float* pp = part + ((size_t)(i * NW + w) * C::NB * 64 + lane) * 4;
#pragma unroll
        for (int b = 0; b < C::NB; ++b)
          acc[b] = kt == 0 ? f32x4{} : *reinterpret_cast<const f32x4*>(pp + 256 * b);
      };
      auto dq_finish = [&](int i, const char* dsr) {
        const int qb0 = i * BQ;
        const int last_q = min(qb0 + BQ, N) - 1;
        const int j_last = CAUSAL ? min(last_q / BK, n_kt - 1) : n_kt - 1;
#pragma unroll
        for (int kb = 0; kb < NW; ++kb) {
          // key block kb: all masked when its first key follows the tile's
          // last query, or lies past the end
          if ((CAUSAL && k0 + 32 * kb > qb0 + BQ - 1) || k0 + 32 * kb >= N) continue;
          u32x4 bq[2];
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) bq[qb] = lds_read_tr16<BK>(dsr, tr16, 32 * kb, 16 * qb);
#pragma unroll
          for (int e = 0; e < C::DQB; ++e) {
            const u32x4 a = lds_read_tr16<BK>(ksm, tr16, 32 * kb, 16 * (w * C::DQB + e));
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) acc[2 * e + qb] = mfma16k32<T>(a, bq[qb], acc[2 * e + qb]);
          }
        }
        if (kt == j_last) {
          // register r of block (e, qb): channel 16 (w DQB + e) + 4 g16 + r of query qb0 + 16 qb + lane % 16
#pragma unroll
          for (int e = 0; e < C::DQB; ++e)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
              const f32x4 y = acc[2 * e + qb] * scale;
              const int query = qb0 + 16 * qb + (lane & 15);
              const int d = 16 * (w * C::DQB + e) + 4 * g16;
              gstore8(rdq, (uint32_t)((query * D + d) * 2), u32x2{pack2<T>(y[0], y[1]), pack2<T>(y[2], y[3])});
            }
        } else {
          float* pp = part + ((size_t)(i * NW + w) * C::NB * 64 + lane) * 4;
#pragma unroll
          for (int b = 0; b < C::NB; ++b) *reinterpret_cast<f32x4*>(pp + 256 * b) = acc[b];
        }
      };

      // This wave's products for the query tile in stage cs: S, dP, P, dS,
      // dV and dK, with its dS^T rows written to dsw.
      auto products = [&](const char* cs, char* dsw, int qb0) {
        const char* qt = cs;
        const char* dot = qt + C::QT_BYTES;
        const float* stats = reinterpret_cast<const float*>(qt + C::STAT_OFF);
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int t = 0; t < C::KSTEPS; ++t) {
          const int off = qrd.at(t);
          s = mfma32<T>(lds_read16(qt, off), lds_read16(kbase, krd.at(t)), s);
          dp = mfma32<T>(lds_read16(dot, off), vf[t], dp);
        }
        // Register jj holds query qb0 + 16(jj/8) + 8h + jj%8 for key kw0 + l32.
        const bool need_mask = (CAUSAL && qb0 < kw0 + 31) || (qb0 + 32 > N) || (kw0 + 32 > N);
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
          // Only tiles on the wave's diagonal and ragged ones are masked (keys
          // past N too: their dS feeds the dQ product).
          if (need_mask) {
            keep_branch();
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int query = qb0 + qi + i;
              if ((CAUSAL && key > query) || query >= N || key >= N) s[8 * t2 + i] = -__builtin_inff();
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
          // dS^T row key, queries 16 t2 + 8 h .. + 7 (chunk 2 t2 + h)
          *reinterpret_cast<u32x4*>(dsw + KTile::off(32 * w + l32, 2 * t2 + h)) = dsf;
#pragma unroll
          for (int db = 0; db < C::DB; ++db) {
            dva[db] = mfma32<T>(lds_read_tr_operand<BQ>(dot, trd, 16 * t2, db), pf, dva[db]);
            dka[db] = mfma32<T>(lds_read_tr_operand<BQ>(qt, trd, 16 * t2, db), dsf, dka[db]);
          }
        }
      };

      // Query tile i0 + f from stage cs (the copy of the next goes to ns); its
      // dS^T goes to dsw; the previous tile's dQ is taken from dsp.
      int cf = 0;
      auto item = [&](const char* cs, char* ns, char* dsw, const char* dsp) {
        // The tile has landed for every wave; every wave is done with the last
        // one, including its reads of the dS^T buffer written below, and has
        // written the previous tile's dS^T rows.
        wait_vmem();
        __syncthreads();
        const int f = cf++;
        if (f + 1 < nq) issue_item(i0 + f + 1, ns);
        // The previous tile's dQ, then this tile's partial on its way (its
        // latency hidden by this tile's products).  Putting the previous dQ
        // after the products on half of the waves (so that the two waves of a
        // SIMD start a tile in different phases) measured slower: 1.35 ->
        // 1.45 ms on the 128 x 8 x 1024 x 128 causal workload, as its partial
        // stores then sit just before the next barrier's wait.
        if (f > 0) {
          if constexpr (!C::PREFETCH) dq_load(i0 + f - 1);
          dq_finish(i0 + f - 1, dsp);
        }
        if constexpr (C::PREFETCH) dq_load(i0 + f);
        const int qb0 = (i0 + f) * BQ;
        // Causal: a tile whose last query precedes the wave's first key is
        // empty for this wave (its dS^T rows are never read: the dQ product
        // skips that key block).
        if (!(CAUSAL && qb0 + 31 < kw0)) products(cs, dsw, qb0);
      };
      for (int f = 0; f < nq; f += 2) {
        item(st0, st1, ds0, ds1);
        if (f + 1 < nq) item(st1, st0, ds1, ds0);
      }
      // The last tile's dQ, once every wave has written its dS^T rows.
      __syncthreads();
      if constexpr (!C::PREFETCH) dq_load(i0 + nq - 1);
      dq_finish(i0 + nq - 1, ((nq - 1) & 1) ? ds1 : ds0);

      // Single write of this wave's dK and dV rows.  Register jj of block db
      // holds d = 32db + 16(jj/8) + 8h + jj%8 of key kw0 + l32.
      const auto rdk = make_rsrc(dk + hoff, head_bytes);
      const auto rdv = make_rsrc(dv + hoff, head_bytes);
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const f32x16 ks = dka[db] * scale;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const uint32_t off = (uint32_t)((key * D + 32 * db + 16 * half + 8 * h) * 2);
          gstore16(rdk, off, pack8<T>(ks, 8 * half));
          gstore16(rdv, off, pack8<T>(dva[db], 8 * half));
        }
      }
    }
  }
}

template <int D, typename T, bool CAUSAL>
static hipError_t launch_fused_t(const BwdArgs& a) {
  using C = FusedTile<D>;
  const int ZH = (int)(a.Z * a.H);
  const int P = a.num_programs < ZH ? a.num_programs : ZH;
  hipLaunchKernelGGL((fa_bwd_fused_kernel<D, T, CAUSAL>), dim3((unsigned)P), dim3(C::NW * 64), 0, a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dout,
                     a.stats + a.rows(), a.stats, (uint16_t*)a.dq, (uint16_t*)a.dk, (uint16_t*)a.dv, a.partial,
                     (int)a.N, ZH, a.scale * kLog2e, a.scale, P);
  return hipGetLastError();
}
template <int D, typename T>
static hipError_t launch_fused_d(const BwdArgs& a) {
  return a.causal ? launch_fused_t<D, T, true>(a) : launch_fused_t<D, T, false>(a);
}
template <typename T>
static hipError_t launch_fused_dt(const BwdArgs& a) {
  switch (a.D) {
    case 64: return launch_fused_d<64, T>(a);
    case 128: return launch_fused_d<128, T>(a);
    default: return launch_fused_d<256, T>(a);
  }
}
hipError_t launch_bwd_fused(const BwdArgs& a) {
  return a.dtype == BF16::code ? launch_fused_dt<BF16>(a) : launch_fused_dt<F16>(a);
}

template <int D, typename T>
static hipError_t occ_fused(int* out) {
  int n = 0, n2 = 0;
  constexpr int threads = FusedTile<D>::NW * 64;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fa_bwd_fused_kernel<D, T, true>, threads, 0);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n2, fa_bwd_fused_kernel<D, T, false>, threads, 0);
  if (e != hipSuccess) return e;
  *out = n < n2 ? n : n2;
  if (*out < 1) *out = 1;
  return hipSuccess;
}
hipError_t fused_blocks_per_cu(int D, int dtype, int* out) {
  const bool bf = dtype == BF16::code;
  switch (D) {
    case 64: return bf ? occ_fused<64, BF16>(out) : occ_fused<64, F16>(out);
    case 128: return bf ? occ_fused<128, BF16>(out) : occ_fused<128, F16>(out);
    default: return bf ? occ_fused<256, BF16>(out) : occ_fused<256, F16>(out);
  }
}

}  // namespace fa
