// fa_fwd.hip - exact attention forward for gfx950.
//
// [FA-Ascend] = the page "把 FlashAttention 搬上昇腾：Triton-Ascend CV Pipeline
// 优化实战" (BiumBiu).  §一 of that page defines the pass: S = Q K^T * scale,
// P = softmax(S), O = P V, computed tile by tile with a Q tile kept on chip,
// K/V tiles streamed past it, an online softmax (running row max m, running
// denominator l, unnormalised accumulator), exp2 with log2(e) folded into the
// scale, fp32 statistics and accumulator, P cast to the 16-bit input type
// before the matrix unit, a shortened causal loop with masking only where a
// tile straddles the diagonal, and a single write of O.
//
// Work decomposition on gfx950
//   * one workgroup = 4 waves working on a Q tile of BM = 128 queries of one
//     head; wave w owns 32 consecutive queries and keeps them in registers as
//     the B operand of the score MFMA (at D = 256, 8 waves: two per 32
//     queries, each owning half of the output channels, see FwdTile).  With the causal mask a workgroup takes
//     two tiles of the head, a long and a short one, so every workgroup has
//     the same work; the second tile's Q rows and first K/V tile are fetched
//     during the first tile's last step;
//   * several workgroups share a compute unit (3 at D = 128, 4 at D = 64, with
//     registers and LDS sized for that), so one wave's softmax arithmetic and
//     memory waits overlap other waves' matrix instructions on the same SIMD;
//   * K/V tiles of BN keys are copied global -> LDS by the buffer unit itself
//     (no register staging) into a two-stage ring: the copy of tile j+1 is in
//     flight while tile j is consumed, with one barrier per tile;
//   * scores are computed transposed, S^T = K Q^T, so that each lane owns one
//     query (a column of the MFMA result) and its softmax statistics are
//     per-lane values; a row max needs one exchange between lane halves;
//   * the output is accumulated transposed as well, O^T = V^T P^T, with V^T
//     read straight from the V tile by transposing LDS reads;
//   * LDS tiles are chunk-major (see CmTile), so all LDS addresses in the loop
//     are per-lane bases plus compile-time offsets;
//   * the query tiles of one head are dispatched back to back on one XCD so
//     that the head's K and V are read from HBM about once.
// Refinement over the page's rescale-on-every-new-max (fp16 only): the running
// max used for the exponentials is only raised when some row's max grew by more
// than 8 in exp2 units, so most tiles skip rescaling the accumulator; the
// normalisation by the matching denominator makes the result the same.  P then
// reaches up to 2^8, harmless in fp16 (relative rounding 2^-11).  With bf16 P
// the row's largest weight must stay exactly 1: a weight of up to 2^8 rounded
// to bf16 is off by up to 2^-9 of itself, which in a near-one-hot row moves O by
// 2^-9 |v|.  So bf16 rescales whenever a row max grows, as on the page.
#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_schedule.h"

namespace fa {

template <int D>
struct FwdTile {
  // D = 256 is split into two D = 128 output halves ([FA-Ascend] §一, §七): a
  // pair of waves shares 32 queries and each wave owns 128 of the output
  // channels.  Both compute the full score tile (the same instructions on the
  // same data give the same bits, so both take the same softmax decisions).
  // That halves the output accumulator per wave, so two waves per SIMD fit
  // where one wave with all 256 channels did: 1.90 -> 1.75 ms on the
  // 128 x 8 x 1024 x 256 workload despite 1.5x the matrix instructions.
  // Splitting the score contraction as well and summing the two partial
  // tiles through LDS took 1.95 ms (one more barrier per tile).
  static constexpr int SPLIT = D == 256 ? 2 : 1;             // waves per 32 queries
  static constexpr int NW = 4 * SPLIT;                       // waves per workgroup
  static constexpr int BM = kFwdQueries;                     // queries per tile
  static constexpr int BN = fwd_keys(D);                     // keys per tile
  static constexpr int KB = BN / 32;                         // 32-key blocks per tile
  static_assert(BM == 4 * 32, "32 queries per wave (pair)");
  static constexpr int TILE_BYTES = BN * D * 2;
  static constexpr int DH = D / SPLIT;                       // channels per wave
  static constexpr int KSTEPS = D / 16;                      // k steps of the score MFMA
  static constexpr int DB = DH / 32;                         // this wave's 32-wide d blocks of O
  static constexpr int DMA = TILE_BYTES / (NW * 1024);       // 1 KiB copies per wave per tile
  static_assert(DMA * NW * 1024 == TILE_BYTES, "tile must split into 1 KiB copies per wave");
  // Waves per SIMD the register budget is sized for (measured best: more
  // resident waves hide the latency of each wave's chain of copy wait, LDS
  // reads, matrix products and softmax).
  static constexpr int OCC = D == 256 ? 2 : (D == 128 ? 3 : 4);
};

// Rescale threshold in exp2 units (see file comment).
template <typename T>
inline constexpr float kRescaleSlack = kIsBF16<T> ? 0.0f : 8.0f;

template <int D, typename T, bool CAUSAL, typename OT>
__global__ __launch_bounds__(FwdTile<D>::NW * 64)
__attribute__((amdgpu_waves_per_eu(FwdTile<D>::OCC, FwdTile<D>::OCC)))
void fa_fwd_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                   const uint16_t* __restrict__ v, void* __restrict__ o, float* __restrict__ lse, int N_max,
                   int ZHkv, int Hkv, int G, int n_qtiles_max, float c2, const int* __restrict__ cu, int64_t n_tokens) {
  using C = FwdTile<D>;
  using Tile = CmTile<C::BN>;
  // One LDS object per ring stage and operand.  With the stage of every
  // access known at compile time (the loop below handles tiles in pairs), the
  // compiler can tell that the copy of tile j+1 does not alias the reads of
  // tile j and need not make those reads wait for it.
  __shared__ __attribute__((aligned(1024))) char k0s[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v0s[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char k1s[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v1s[C::TILE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_id();
  const int qg = C::SPLIT == 1 ? w : w & 3;  // this wave's 32 queries of the tile
  const int hf = C::SPLIT == 1 ? 0 : w >> 2;  // this wave's channel half
  const int h = lane >> 5;
  const int l32 = lane & 31;

  // Query tiles of this workgroup: one, or with the causal mask a long and a
  // short one of the same head (the longest pairs go first).  The grid is
  // dealt over (batch key/value head, member, slot) for the longest
  // sequence; blocks past their own sequence's tiles have no work.
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
  const size_t kvoff = (size_t)hr.kv_row0 * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const auto rq = make_rsrc(q + hoff, head_bytes);
  const auto rk = make_rsrc(k + kvoff, head_bytes);
  const auto rv = make_rsrc(v + kvoff, head_bytes);

  // Copy K/V tile j into a ring stage (chunk-major layout, see CmTile).
  auto issue_tile = [&](int j, char* kdst, char* vdst) {
    const int kv0 = j * C::BN;
#pragma unroll
    for (int i = 0; i < C::DMA; ++i) {
      const int blk = w * C::DMA + i;
      const int sl = blk * 64 + lane;
      const int row = Tile::slot_row(sl), chunk = Tile::slot_chunk(sl);
      const uint32_t off = (uint32_t)(((kv0 + row) * D + 8 * chunk) * 2);
      dma16(rk, kdst + blk * 1024, off);
      dma16(rv, vdst + blk * 1024, off);
    }
  };
  // This wave's Q rows of tile qt -> registers, B-operand layout: lane owns
  // query qt BM + 32 qg + l32, k = d.
  u32x4 qf[C::KSTEPS];
  auto load_q = [&](int qt) {
#pragma unroll
    for (int t = 0; t < C::KSTEPS; ++t)
      qf[t] = gload16(rq, (uint32_t)(((qt * C::BM + 32 * qg + l32) * D + 16 * t + 8 * h) * 2));
  };

  // Per-lane LDS read bases: K rows 32 kb + sigma(l32) as the A operand of
  // the score product, V^T through transposing reads.
  const RowRead<C::BN> krd(sigma32(l32), h);
  const TrRead<C::BN> vrd(lane);

  issue_tile(0, k0s, v0s);
  load_q(qt_a);
  bool first_tile_issued = true;
  for (int it = 0; it < n_items; ++it) {
    const int qt = it == 0 ? qt_a : qt_b;
    const int q0 = qt * C::BM;
    const int wq0 = q0 + 32 * qg;  // first query of this wave
    const int kv_end = CAUSAL ? min(N, q0 + C::BM) : N;
    const int nt = (kv_end + C::BN - 1) / C::BN;
    const bool more = it + 1 < n_items;
    // With an even tile count the next item's first tile lands in stage 0 of
    // the ring: copy it during this item's last tile.
    const bool chain = more && (nt % 2 == 0);
    if (!first_tile_issued) issue_tile(0, k0s, v0s);

    float m_run = -1e30f;  // running max, exp2 units
    float l_run = 0.f;     // running denominator (this lane half's keys)
    bool fresh = true;     // no tile processed yet: acc and l_run are zero
    f32x16 acc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};

    // Tile j, read from kt/vt; the copy of tile j+1 goes to kn/vn.
    auto tile = [&](int j, const char* kt, const char* vt, char* kn, char* vn) {
      // Tile j has landed for every wave, and every wave is done with tile
      // j-1, whose stage the copy of tile j+1 now overwrites.
      wait_vmem();
      __syncthreads();
      if (j + 1 < nt)
        issue_tile(j + 1, kn, vn);
      else if (chain)
        issue_tile(0, kn, vn);
      const int kv0 = j * C::BN;
      // With the causal mask a wave whose last query precedes the tile skips it.
      const bool active = !CAUSAL || kv0 <= wq0 + 31;
      // ---- S^T = K Q^T : rows = keys (sigma order), columns = this wave's queries
      f32x16 s[C::KB];
      if (active) {
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) s[kb] = f32x16{};
#pragma unroll
        for (int t = 0; t < C::KSTEPS; ++t) {
#pragma unroll
          for (int kb = 0; kb < C::KB; ++kb) {
            const u32x4 a = lds_read16(kt, krd.at(t) + kRowBlockBytes * kb);
            s[kb] = mfma32<T>(a, qf[t], s[kb]);
          }
        }
      }
      // The Q rows are not needed any more: load the next item's.
      if (j == nt - 1 && more) load_q(qt_b);
      if (!active) return;
      // ---- masks: causal diagonal tile and ragged last tile only
      const bool need_mask = (CAUSAL && kv0 + C::BN - 1 > wq0) || (kv0 + C::BN > N);
      if (need_mask) {
        // Key kv0 + 8h + c (c = 32kb + 16(jj/8) + jj%8, a constant per
        // register) is dropped when it lies past the query (causal) or past
        // the sequence, i.e. when c exceeds one per-lane limit.
        const int last = CAUSAL ? min(wq0 + l32, N - 1) : N - 1;  // last key kept
        const int lim = last - kv0 - 8 * h;
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) {
            const int c = 32 * kb + 16 * (jj >> 3) + (jj & 7);
            s[kb][jj] = c > lim ? -INFINITY : s[kb][jj];
          }
      }
      // ---- online softmax, exp2 units
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) mx = fmaxf(mx, s[kb][jj]);
      mx = half_swap_max(mx);
      const float m_new = fmaxf(m_run, mx * c2);
      if (wave_any(m_new > m_run + kRescaleSlack<T>)) {
        // Before the first tile the accumulator and denominator are zero and
        // need no rescaling.
        if (!fresh) {
          const float alpha = fast_exp2(m_run - m_new);
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < C::DB; ++db) acc[db] *= alpha;
        }
        m_run = m_new;
      }
      fresh = false;
      // p = exp2(s c - m), packed to the 16-bit type for the PV product;
      // l_run sums the fp32 p.
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const float p = fast_exp2(__builtin_fmaf(s[kb][jj], c2, -m_run));
          s[kb][jj] = p;
          rs += p;
        }
      l_run += rs;
      // ---- O^T += V^T P^T : A = V^T from the V tile (transposing reads), B = P
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const u32x4 pk = pack8<T>(s[kb], 8 * t2);
#pragma unroll
          for (int db = 0; db < C::DB; ++db) {
            const u32x4 a = lds_read_tr_operand<C::BN>(vt, vrd, 32 * kb + 16 * t2, db + C::DB * hf);
            acc[db] = mfma32<T>(a, pk, acc[db]);
          }
        }
      }
    };
    for (int j = 0; j < nt; j += 2) {
      tile(j, k0s, v0s, k1s, v1s);
      if (j + 1 < nt) tile(j + 1, k1s, v1s, k0s, v0s);
    }

    // ---- epilogue: O = acc / l written once; lse = ln(sum exp(S)) per query
    const float lsum = half_swap_sum(l_run);
    const float inv = 1.0f / lsum;
    const int query = wq0 + l32;
    if constexpr (sizeof(OT) == 4) {
      const auto ro = make_rsrc((float*)o + hoff, (uint32_t)N * D * 4);
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int d = 32 * (db + C::DB * hf) + 16 * half + 8 * h;
          const int j0 = 8 * half;
          u32x4 lo, hi;
          lo.x = __float_as_uint(acc[db][j0 + 0] * inv);
          lo.y = __float_as_uint(acc[db][j0 + 1] * inv);
          lo.z = __float_as_uint(acc[db][j0 + 2] * inv);
          lo.w = __float_as_uint(acc[db][j0 + 3] * inv);
          hi.x = __float_as_uint(acc[db][j0 + 4] * inv);
          hi.y = __float_as_uint(acc[db][j0 + 5] * inv);
          hi.z = __float_as_uint(acc[db][j0 + 6] * inv);
          hi.w = __float_as_uint(acc[db][j0 + 7] * inv);
          const uint32_t off = (uint32_t)((query * D + d) * 4);
          gstore16(ro, off, lo);
          gstore16(ro, off + 16, hi);
        }
    } else {
      const auto ro = make_rsrc((uint16_t*)o + hoff, (uint32_t)N * D * 2);
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        f32x16 y = acc[db] * inv;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int d = 32 * (db + C::DB * hf) + 16 * half + 8 * h;
          gstore16(ro, (uint32_t)((query * D + d) * 2), pack8<T>(y, 8 * half));
        }
      }
    }
    if (h == 0 && hf == 0) {
      const auto rl = make_rsrc(lse + hr.q_row0, (uint32_t)N * 4);
      gstore_f32(rl, (uint32_t)query * 4, (m_run + __log2f(lsum)) * kLn2);
    }
    first_tile_issued = chain;
    if (more && !chain) {
      // The ring restarts at stage 0 for the next item; every wave must be
      // done with this item's last tile before it is overwritten.
      __syncthreads();
    }
  }
}

template <int D, typename T, bool CAUSAL, typename OT>
hipError_t launch_fwd_t(const FwdArgs& a) {
  using C = FwdTile<D>;
  const int n_qtiles = (int)((a.N + C::BM - 1) / C::BM);
  const int ZHkv = (int)(a.Z * a.Hkv);
  const int G = (int)(a.H / a.Hkv);
  const dim3 grid((unsigned)xcd_grid_grouped(ZHkv, G, paired_groups(n_qtiles, CAUSAL)));
  hipLaunchKernelGGL((fa_fwd_kernel<D, T, CAUSAL, OT>), grid, dim3(C::NW * 64), 0, a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.o, a.lse,
                     (int)a.N, ZHkv, (int)a.Hkv, G, n_qtiles, a.scale * kLog2e, a.cu_seqlens, a.T);
  return hipGetLastError();
}

template <int D, typename T>
hipError_t launch_fwd_d(const FwdArgs& a) {
  const bool of32 = a.o_dtype == F32::code;
  if (a.causal) return of32 ? launch_fwd_t<D, T, true, float>(a) : launch_fwd_t<D, T, true, uint16_t>(a);
  return of32 ? launch_fwd_t<D, T, false, float>(a) : launch_fwd_t<D, T, false, uint16_t>(a);
}

template <typename T>
hipError_t launch_fwd_dt(const FwdArgs& a) {
  switch (a.D) {
    case 64: return launch_fwd_d<64, T>(a);
    case 128: return launch_fwd_d<128, T>(a);
    default: return launch_fwd_d<256, T>(a);
  }
}

hipError_t launch_fwd(const FwdArgs& a) {
  return a.dtype == BF16::code ? launch_fwd_dt<BF16>(a) : launch_fwd_dt<F16>(a);
}

}  // namespace fa
