// fa_paged.hip - paged KV cache for gfx950: cache writes and decode attention.
//
// [Serving-Ascend] = the page "从算子到 Serving：昇腾推理评测链路实践" (BiumBiu).
// Its section "ReshapeAndCache" writes each new token's key and value to
// physical block slot // block_size at offset slot % block_size, skipping
// tokens whose slot is negative.  Its section "GQA Paged Attention" reads a
// sequence's pages through a block table, stops at the sequence's context
// length (masking the rest of the last block), lets G query heads share one
// key/value head, and keeps a running max, normaliser and output (online
// softmax) instead of the full score row.
//
// Cache layout (one page = one physical block of one key/value head):
//   k_cache (num_blocks, Hkv, D/8, block_size, 8): the page's keys in 16-byte
//     chunks of 8 channels, chunk-major (chunk c of every token, then chunk
//     c+1), the key layout vLLM uses for 16-bit caches;
//   v_cache (num_blocks, Hkv, D, block_size): the page's values transposed,
//     one row of block_size values per channel.
// Both layouts let the decode kernel load its matrix operands straight from
// memory in MFMA register layout with contiguous loads: one 16-byte key chunk
// per lane, 16 tokens x 4 chunks = 1 KiB per load; and 8-byte runs of four
// consecutive tokens of one value channel, 512 bytes per load.
//
// Decode.  A workgroup owns (sequence b, key/value head hk, a block of 16 of
// the query rows that use hk, split s) and a contiguous range of the
// context; its 4 waves take 16-token tiles in turn.  The query rows are the G
// query heads of hk (one query token per sequence), or the Tq x G (token,
// head) rows of several query tokens, each with its own count of visible
// tokens; blocks are padded to 16.  Per tile a wave computes
//     S^T (16 tokens x 16 rows) = K Q^T       4 or 8 or 16 x v_mfma 16x16x32
//     online softmax per row column (exp2 units)
//     O^T (D x 16 rows) += V^T P^T            D/16 x v_mfma 16x16x16
// where the score result is already the B operand of the output product.
// The waves' states are merged through LDS; with several splits per
// sequence the merged (O, lse) pairs go to a workspace and a second kernel
// combines them: O = sum_s exp(lse_s - lse) O_s, lse = ln sum_s exp(lse_s).
// The splits may come from two sources (two caches, or a whole context and
// a set of kept pages, [V4-A100] below), which the combine then normalises
// together.  HBM-bound: every cached key and value a block needs is read
// once.
//
// [V4-A100] = the page "在 4 张 A100 上部署 DeepSeek-V4-Flash-0731" (BiumBiu),
// section 7.5: one sparse attention kernel for one source or two sources
// under a single softmax denominator; prefill and decode share it because
// the causal constraint becomes per-row lengths.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

// ============================================================ cache writes
// One thread per 16-byte chunk of a (token, key/value head) row: the key chunk
// is stored as one 16-byte vector; the value chunk's 8 channels go to 8 rows
// of the transposed page.
template <int D>
__global__ __launch_bounds__(256) void fa_reshape_and_cache_kernel(
    const uint16_t* __restrict__ key, const uint16_t* __restrict__ value, const int64_t* __restrict__ slots,
    uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache, int64_t rows, int Hkv, int bs,
    int64_t num_blocks) {
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;  // token * Hkv + hk
  const int c = threadIdx.x % TPR;
  if (row >= rows) return;
  const int64_t tok = row / Hkv;
  const int64_t hk = row % Hkv;
  const int64_t slot = slots[tok];
  if (slot < 0 || slot >= num_blocks * bs) return;  // skipped (negative) or past the cache
  const int64_t blk = slot / bs;
  const int64_t off = slot % bs;
  const u32x4 kv = *reinterpret_cast<const u32x4*>(key + row * D + 8 * c);
  *reinterpret_cast<u32x4*>(k_cache + (((blk * Hkv + hk) * (D / 8) + c) * bs + off) * 8) = kv;
  const u32x4 vv = *reinterpret_cast<const u32x4*>(value + row * D + 8 * c);
  uint16_t* vdst = v_cache + ((blk * Hkv + hk) * D + 8 * c) * (int64_t)bs + off;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    vdst[(2 * i) * (int64_t)bs] = (uint16_t)(vv[i] & 0xffffu);
    vdst[(2 * i + 1) * (int64_t)bs] = (uint16_t)(vv[i] >> 16);
  }
}

// ============================================================ decode
template <int D>
struct DecodeTile {
  static constexpr int NW = 4;
  static constexpr int KSTEPS = D / 32;  // k = 32 steps of the score product
  static constexpr int DB = D / 16;      // 16-channel blocks of O^T
  static constexpr int OSTRIDE = D + 1;  // padded LDS row of a head's merged output
  // Waves per SIMD the registers are sized for.  Each wave holds two tiles of
  // operands (the current one and the next, in flight); at D = 128 three
  // waves per SIMD fit only if the compiler issues the next tile's loads
  // later, which measured slower than two waves.
  static constexpr int OCC = D == 64 ? 5 : (D == 128 ? 2 : 1);
};

// One KV source as the kernel sees it (see DecodeSource).
struct KvSrc {
  const uint16_t* k;
  const uint16_t* v;
  const int* tables;
  const int* lens;
  const int* sel;   // kept pages (B, Hkv, topk), or nullptr for the whole context
  const int* nsel;  // their count (B, Hkv)
  const int* rows;  // (B, Tq): tokens of this source each query row sees, or nullptr for all
  int64_t num_blocks;
  int64_t chunk;  // tokens per split
  int bs, max_blocks, topk, n_splits;
};

template <int D, typename T, typename OT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DecodeTile<D>::OCC, DecodeTile<D>::OCC)))
void fa_paged_decode_kernel(const uint16_t* __restrict__ q, KvSrc src0, KvSrc src1, void* __restrict__ o,
                            float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_lse, int H,
                            int Hkv, int G, int Tq, float c2) {
  using C = DecodeTile<D>;
  __shared__ float sm_m[C::NW][16];
  __shared__ float sm_l[C::NW][16];
  __shared__ float sm_o[C::NW][16 * C::OSTRIDE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_id();
  const int col = lane & 15;  // query-row column of the score / output tiles
  const int grp = lane >> 4;  // k group: tokens 4 grp .. 4 grp + 3 of a tile

  // Workgroup = (sequence b, key/value head hk, block hb of 16 of the
  // group's Tq * G query rows, split s_all); row r of the group is query
  // token r / G of head hk * G + r % G.  The splits of the first source come
  // first, then those of the second (src1.n_splits = 0 with one source).
  // Every split's partial result joins the same combine, so the tokens of
  // both sources share one softmax.
  const int R = Tq * G;  // query rows of one (sequence, key/value head)
  const int n_hb = (R + 15) / 16;
  const int n_splits = src0.n_splits + src1.n_splits;  // over all sources
  const int s_all = blockIdx.x % n_splits;
  const bool second = s_all >= src0.n_splits;
  const KvSrc src = second ? src1 : src0;
  const int s = second ? s_all - src0.n_splits : s_all;  // split within the source
  const int bs = src.bs;
  const int rest = blockIdx.x / n_splits;
  const int hb = rest % n_hb;
  const int bh = rest / n_hb;
  const int hk = bh % Hkv;
  const int b = bh / Hkv;
  const int g0 = 16 * hb;                          // first query row of the block (in the group)
  const int gn = R - g0 < 16 ? R - g0 : 16;        // query rows in the block
  const int64_t max_tokens = (int64_t)src.max_blocks * bs;
  const int ctx = src.lens[b];
  const int64_t n_real = ctx < 0 ? 0 : (ctx > max_tokens ? max_tokens : ctx);
  int64_t n_ctx = n_real;  // tokens this (sequence, head) attends to, in order
  // Sparse decode: the tokens of the kept pages, back to back (a virtual
  // context); the last kept page is cut at the context's end when it is the
  // context's last page.
  const int* selrow = nullptr;
  int ns = 0;
  if (src.sel != nullptr) {
    const int64_t row = (int64_t)b * Hkv + hk;
    const int cnt = src.nsel[row];
    ns = cnt < 0 ? 0 : (cnt > src.topk ? src.topk : cnt);
    selrow = src.sel + row * src.topk;
    const int64_t n_pages = (n_real + bs - 1) / bs;
    if (ns == 0) {
      n_ctx = 0;
    } else {
      const int64_t last = selrow[ns - 1];
      n_ctx = (int64_t)(ns - 1) * bs + (last == n_pages - 1 ? n_real - last * bs : bs);
    }
  }
  // This split's tokens: chunk tokens (a whole number of 64-token steps, one
  // 16-token tile per wave per step) from s * chunk on; the last split takes
  // the rest of a context longer than the split was sized for.
  const int64_t chunk = src.chunk;
  const int64_t t_begin = s * chunk < n_ctx ? s * chunk : n_ctx;
  int64_t t_end = (s + 1 < src.n_splits && (s + 1) * chunk < n_ctx) ? (s + 1) * chunk : n_ctx;

  // This lane's query row (column col of the block) and how many of the
  // source's tokens it sees (all n_ctx without row lengths).  The tile loop
  // stops at the block's largest count; tiles past the smallest are masked
  // per column.
  const int r_col = g0 + (col < gn ? col : 0);
  const int t_col = r_col / G;  // query token of the column
  const int n_ctx32 = (int)n_ctx;  // at most max_blocks * block_size < 2^31 (checked by the host)
  int lim = n_ctx32;
  if (src.rows != nullptr) {
    const int x = src.rows[(int64_t)b * Tq + t_col];
    lim = x < 0 ? 0 : (x < n_ctx32 ? x : n_ctx32);
  }
  if (col >= gn) lim = src.rows != nullptr ? 0 : n_ctx32;  // padding columns decide nothing
  int lim_hi = lim, lim_lo = col < gn ? lim : n_ctx32;
#pragma unroll
  for (int x = 1; x < 16; x <<= 1) {
    lim_hi = max(lim_hi, __shfl_xor(lim_hi, x, 64));
    lim_lo = min(lim_lo, __shfl_xor(lim_lo, x, 64));
  }
  lim_hi = __builtin_amdgcn_readfirstlane(lim_hi);  // the same in every 16-lane group
  lim_lo = __builtin_amdgcn_readfirstlane(lim_lo);
  if (t_end > lim_hi) t_end = lim_hi < t_begin ? t_begin : lim_hi;
  const int64_t t_mask = t_end < lim_lo ? t_end : lim_lo;  // tiles reaching past it need masks

  // Q^T as the B operand of the score product: lane supplies row col of the
  // block, channels 32 ks + 8 grp .. +7; columns past the block are zero.
  u32x4 qf[C::KSTEPS];
  {
    const int h = hk * G + r_col % G;
    const auto rq = make_rsrc(q + (((int64_t)b * Tq + t_col) * H + h) * D, D * 2);
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      const u32x4 x = gload16(rq, (uint32_t)((32 * ks + 8 * grp) * 2));
      qf[ks] = col < gn ? x : u32x4{0u, 0u, 0u, 0u};
    }
  }

  float m_run = -INFINITY;  // running max of this lane's head column (exp2 units)
  float l_run = 0.f;        // running normaliser over this lane's 4 tokens per tile
  f32x4 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Operands of one tile, loaded ahead of their use.
  struct Tile {
    u32x4 k[C::KSTEPS];
    u32x2 v[C::DB];
  };
  // Block-table entries of this wave's tiles, 64 tiles at a time: lane i
  // holds the physical block of tile j0 + i (read with one vector load, so
  // that the loop does not wait on a scalar load per tile).
  const int* table = src.tables + (int64_t)b * src.max_blocks;
  const int64_t w_first = t_begin + 16 * w;  // this wave's first token
  int vblk = -1;
  auto load_blocks = [&](int64_t j0) {
    int64_t page = (w_first + 64 * (j0 + lane)) / bs;  // position in the (virtual) context
    if (selrow != nullptr) page = page < ns ? selrow[page] : -1;  // kept page -> logical page
    // a logical page outside the context takes no part
    vblk = (page >= 0 && page < src.max_blocks && page * bs < n_real) ? table[page] : -1;
  };
  auto load_tile = [&](int64_t j, Tile& x) -> bool {
    const int64_t t0 = w_first + 64 * j;
    const int o0 = (int)(t0 % bs);
    const int blk = __builtin_amdgcn_readlane(vblk, (int)(j & 63));
    if (blk < 0 || blk >= src.num_blocks) return false;  // tokens of an invalid block take no part
    const int64_t pg = (int64_t)blk * Hkv + hk;
    const auto rk = make_rsrc(src.k + pg * bs * D, (uint32_t)(bs * D * 2));
    const auto rv = make_rsrc(src.v + pg * D * bs, (uint32_t)(D * bs * 2));
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks)  // chunk 4 ks + grp of token o0 + col: 1 KiB contiguous per load
      x.k[ks] = gload16(rk, (uint32_t)(((4 * ks + grp) * bs + o0 + col) * 16));
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
      x.v[db] = gload8(rv, (uint32_t)(((16 * db + col) * bs + o0 + 4 * grp) * 2));
    return true;
  };

  int64_t t0 = w_first;
  int64_t j = 0;  // this wave's tile index: tokens t0 = w_first + 64 j
  Tile cur;
  if (t0 < t_end) load_blocks(0);
  bool cur_ok = t0 < t_end ? load_tile(0, cur) : false;
  while (t0 < t_end) {
    const int64_t t1 = t0 + 16 * C::NW;
    Tile nxt;
    if (((j + 1) & 63) == 0 && t1 < t_end) load_blocks(j + 1);
    const bool nxt_ok = t1 < t_end ? load_tile(j + 1, nxt) : false;
    if (cur_ok) {
      f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks) sacc = mfma16k32<T>(cur.k[ks], qf[ks], sacc);
      float sc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[i] = sacc[i] * c2;
      if (t0 + 16 > t_mask) {  // the split's last tile, or a column's last visible token
        keep_branch();
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (t0 + 4 * grp + i >= t_end || t0 + 4 * grp + i >= lim) sc[i] = -INFINITY;
      }
      float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      // -inf while a column has seen no visible token: exponentiate against 0
      // then (every weight is 0) instead of forming -inf - (-inf)
      const float m_ref = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_ref);
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = fast_exp2(sc[i] - m_ref);
      l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
      if (wave_any(m_new > m_run)) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db) oacc[db] *= alpha;
      }
      m_run = m_new;
      const u32x2 pf = u32x2{pack2<T>(p[0], p[1]), pack2<T>(p[2], p[3])};
#pragma unroll
      for (int db = 0; db < C::DB; ++db) oacc[db] = mfma16k16<T>(cur.v[db], pf, oacc[db]);
    }
    cur = nxt;
    cur_ok = nxt_ok;
    t0 = t1;
    ++j;
  }

  // Merge the waves: each head column's normaliser over the 4 token groups,
  // then (m, l, unnormalised O) per wave into LDS.
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (grp == 0) {
    sm_m[w][col] = m_run;
    sm_l[w][col] = l_run;
  }
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm_o[w][col * C::OSTRIDE + 16 * db + 4 * grp + i] = oacc[db][i];
  __syncthreads();

  constexpr float kLn2 = 0.69314718055994531f;
  for (int e = tid; e < gn * D; e += 256) {
    const int c = e / D, d = e % D;
    float m = -INFINITY;
#pragma unroll
    for (int x = 0; x < C::NW; ++x) m = fmaxf(m, sm_m[x][c]);
    float l = 0.f, acc = 0.f;
    if (m != -INFINITY) {
#pragma unroll
      for (int x = 0; x < C::NW; ++x) {
        const float wgt = fast_exp2(sm_m[x][c] - m);  // 0 for a wave with no tokens
        l += wgt * sm_l[x][c];
        acc += wgt * sm_o[x][c * C::OSTRIDE + d];
      }
    }
    const float val = m != -INFINITY ? acc / l : 0.f;
    const float lse_n = m != -INFINITY ? (m + __log2f(l)) * kLn2 : -INFINITY;
    const int r = g0 + c;  // query row: token r / G of head hk * G + r % G
    const int64_t row = ((int64_t)b * Tq + r / G) * H + hk * G + r % G;
    if (n_splits == 1) {
      if constexpr (sizeof(OT) == 4) {
        reinterpret_cast<float*>(o)[row * D + d] = val;
      } else {
        reinterpret_cast<uint16_t*>(o)[row * D + d] = (uint16_t)(pack2<T>(val, 0.f) & 0xffffu);
      }
      if (d == 0 && lse != nullptr) lse[row] = lse_n;
    } else {
      part_o[(row * n_splits + s_all) * D + d] = val;
      if (d == 0) part_lse[row * n_splits + s_all] = lse_n;
    }
  }
}

// Split combine: one workgroup per (sequence, query head), one thread per
// channel.
template <int D, typename T, typename OT>
__global__ __launch_bounds__(D) void fa_paged_decode_combine_kernel(const float* __restrict__ part_o,
                                                                    const float* __restrict__ part_lse,
                                                                    void* __restrict__ o, float* __restrict__ lse,
                                                                    int n_splits) {
  const int64_t row = blockIdx.x;
  const int d = threadIdx.x;
  const float* pl = part_lse + row * n_splits;
  float m = -INFINITY;
  for (int x = 0; x < n_splits; ++x) m = fmaxf(m, pl[x]);
  float wsum = 0.f, acc = 0.f;
  if (m != -INFINITY) {
    for (int x = 0; x < n_splits; ++x) {
      if (pl[x] == -INFINITY) continue;  // a split with no tokens
      const float wgt = __expf(pl[x] - m);
      wsum += wgt;
      acc += wgt * part_o[(row * n_splits + x) * D + d];
    }
  }
  const float val = m != -INFINITY ? acc / wsum : 0.f;
  if constexpr (sizeof(OT) == 4) {
    reinterpret_cast<float*>(o)[row * D + d] = val;
  } else {
    reinterpret_cast<uint16_t*>(o)[row * D + d] = (uint16_t)(pack2<T>(val, 0.f) & 0xffffu);
  }
  if (d == 0 && lse != nullptr) lse[row] = m != -INFINITY ? m + __logf(wsum) : -INFINITY;
}

// ============================================================ launchers
template <int D>
static hipError_t launch_cache_d(const CacheArgs& a) {
  constexpr int RPB = 256 / (D / 8);
  const int64_t rows = a.num_tokens * a.Hkv;
  hipLaunchKernelGGL((fa_reshape_and_cache_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                     a.stream, (const uint16_t*)a.key, (const uint16_t*)a.value, a.slots, (uint16_t*)a.k_cache,
                     (uint16_t*)a.v_cache, rows, (int)a.Hkv, (int)a.block_size, a.num_blocks);
  return hipGetLastError();
}
hipError_t launch_reshape_and_cache(const CacheArgs& a) {
  switch (a.D) {
    case 64: return launch_cache_d<64>(a);
    case 128: return launch_cache_d<128>(a);
    default: return launch_cache_d<256>(a);
  }
}

static KvSrc kv_src(const DecodeSource& d) {
  KvSrc k{};
  k.k = (const uint16_t*)d.k_cache;
  k.v = (const uint16_t*)d.v_cache;
  k.tables = d.block_tables;
  k.lens = d.context_lens;
  k.sel = d.selected;
  k.nsel = d.n_selected;
  k.num_blocks = d.num_blocks;
  k.chunk = d.chunk;
  k.bs = (int)d.block_size;
  k.max_blocks = (int)d.max_blocks;
  k.topk = (int)d.topk;
  k.n_splits = d.n_splits;
  k.rows = d.row_lens;
  return k;
}

template <int D, typename T, typename OT>
static hipError_t launch_decode_t(const DecodeArgs& a) {
  const int G = (int)(a.H / a.Hkv);
  const KvSrc s0 = kv_src(a.src[0]);
  KvSrc s1 = a.n_sources > 1 ? kv_src(a.src[1]) : s0;
  if (a.n_sources < 2) s1.n_splits = 0;  // no workgroup takes the second source
  const int n_splits = s0.n_splits + s1.n_splits;
  const int64_t grid = a.B * a.Hkv * ((a.Tq * G + 15) / 16) * n_splits;
  float* part_o = a.workspace;
  float* part_lse = a.workspace + a.B * a.Tq * a.H * n_splits * a.D;
  hipLaunchKernelGGL((fa_paged_decode_kernel<D, T, OT>), dim3((unsigned)grid), dim3(256), 0, a.stream,
                     (const uint16_t*)a.q, s0, s1, a.o, a.lse, part_o, part_lse, (int)a.H, (int)a.Hkv, G, (int)a.Tq,
                     a.scale * kLog2e);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_splits == 1) return e;
  hipLaunchKernelGGL((fa_paged_decode_combine_kernel<D, T, OT>), dim3((unsigned)(a.B * a.Tq * a.H)), dim3(D), 0,
                     a.stream, part_o, part_lse, a.o, a.lse, n_splits);
  return hipGetLastError();
}
template <int D, typename T>
static hipError_t launch_decode_o(const DecodeArgs& a) {
  return a.o_dtype == F32::code ? launch_decode_t<D, T, float>(a) : launch_decode_t<D, T, uint16_t>(a);
}
template <typename T>
static hipError_t launch_decode_dt(const DecodeArgs& a) {
  switch (a.D) {
    case 64: return launch_decode_o<64, T>(a);
    case 128: return launch_decode_o<128, T>(a);
    default: return launch_decode_o<256, T>(a);
  }
}
hipError_t launch_paged_decode(const DecodeArgs& a) {
  return a.dtype == BF16::code ? launch_decode_dt<BF16>(a) : launch_decode_dt<F16>(a);
}

}  // namespace fa
