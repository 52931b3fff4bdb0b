// fa_quest.hip - query-aware page selection (Quest) over a paged KV cache.
//
// [Serving-Ascend] = the page "从算子到 Serving：昇腾推理评测链路实践" (BiumBiu),
// section "Quest Sparse Attention": score the logical blocks (pages) of a long
// context cheaply, keep the Top-K, and run exact attention over the tokens of
// the kept pages only (fa_paged_decode_sparse).  The page names the method,
// not its scoring rule; the rule here is the published Quest one: a page keeps
// the channel-wise minimum and maximum of its valid keys, and scores
// sum_d max(q_d * min_d, q_d * max_d), an upper bound of q . k over its keys.
// A key/value head keeps one set of pages for its G query heads, scored by
// the sum of their scores; ties go to the lower page index; the kept pages are
// listed in ascending order.
//
// Page metadata: kmeta (num_blocks, Hkv, 2, D) in the cache dtype (min then
// max; exact, min and max of 16-bit values).
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

// ============================================================ page min / max
// One thread per (sequence, logical page, key/value head, 8-channel chunk):
// the chunk of every valid token of the page (contiguous in the chunk-major
// key layout) is folded into 8 minima and 8 maxima.
template <int D, typename T>
__global__ __launch_bounds__(256) void fa_quest_minmax_kernel(const uint16_t* __restrict__ k_cache,
                                                              const int* __restrict__ block_tables,
                                                              const int* __restrict__ context_lens,
                                                              uint16_t* __restrict__ kmeta, int64_t n_items,
                                                              int Hkv, int bs, int64_t num_blocks, int max_blocks) {
  constexpr int NC = D / 8;
  const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (item >= n_items) return;
  const int c = (int)(item % NC);
  const int hk = (int)((item / NC) % Hkv);
  const int64_t bp = item / ((int64_t)NC * Hkv);
  const int p = (int)(bp % max_blocks);
  const int b = (int)(bp / max_blocks);
  int64_t n_ctx = context_lens[b];
  n_ctx = n_ctx < 0 ? 0 : (n_ctx > (int64_t)max_blocks * bs ? (int64_t)max_blocks * bs : n_ctx);
  const int64_t first = (int64_t)p * bs;
  if (first >= n_ctx) return;  // page past the context
  const int valid = (int)(n_ctx - first < bs ? n_ctx - first : bs);
  const int blk = block_tables[(int64_t)b * max_blocks + p];
  if (blk < 0 || blk >= num_blocks) return;
  const int64_t pg = (int64_t)blk * Hkv + hk;
  const u32x4* src = reinterpret_cast<const u32x4*>(k_cache + (pg * NC + c) * (int64_t)bs * 8);
  float mn[8], mx[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    mn[i] = INFINITY;
    mx[i] = -INFINITY;
  }
  for (int o = 0; o < valid; ++o) {
    const u32x4 x = src[o];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = lo16_to_f32<T>(x[i]), e = hi16_to_f32<T>(x[i]);
      mn[2 * i] = fminf(mn[2 * i], a);
      mx[2 * i] = fmaxf(mx[2 * i], a);
      mn[2 * i + 1] = fminf(mn[2 * i + 1], e);
      mx[2 * i + 1] = fmaxf(mx[2 * i + 1], e);
    }
  }
  u32x4 vmn, vmx;  // back to 16 bits: exact (the values are 16-bit values)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    vmn[i] = pack2<T>(mn[2 * i], mn[2 * i + 1]);
    vmx[i] = pack2<T>(mx[2 * i], mx[2 * i + 1]);
  }
  uint16_t* dst = kmeta + pg * 2 * D + 8 * c;
  *reinterpret_cast<u32x4*>(dst) = vmn;
  *reinterpret_cast<u32x4*>(dst + D) = vmx;
}

// ============================================================ scores + Top-K
// One workgroup per (sequence, key/value head): the page scores go to LDS, a
// radix select over their order-preserving integer form finds the topk-th
// best score (ties to the lower page), and a prefix count over the kept
// flags writes the kept pages in ascending page order.
// Threads per selection workgroup: 8 waves score the pages (one workgroup
// per (sequence, key/value head) has to finish them all); 0.050 -> 0.036 ms
// against 4 waves on the 64-sequence workload, 0.041 with 16.
constexpr int kSelThreads = 512;

template <int D, typename T>
__global__ __launch_bounds__(kSelThreads) void fa_quest_select_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kmeta, const int* __restrict__ block_tables,
    const int* __restrict__ context_lens, int* __restrict__ selected, int* __restrict__ n_selected, int H, int Hkv,
    int G, int bs, int64_t num_blocks, int max_blocks, int topk) {
  __shared__ float skey[kQuestMaxPages];
  __shared__ int sidx[kQuestMaxPages];
  __shared__ int scount[256];

  const int tid = threadIdx.x;
  const int hk = blockIdx.x % Hkv;
  const int b = blockIdx.x / Hkv;
  int64_t n_ctx = context_lens[b];
  n_ctx = n_ctx < 0 ? 0 : (n_ctx > (int64_t)max_blocks * bs ? (int64_t)max_blocks * bs : n_ctx);
  const int n_pages = (int)((n_ctx + bs - 1) / bs);
  const int keep = n_pages < topk ? n_pages : topk;

  // Scores.  For min <= max, max(a x, a y) = a (x + y) / 2 + |a| (y - x) / 2,
  // so the group's score sum_h sum_d max(q_hd min_d, q_hd max_d) equals
  // sum_d (A_d min_d + B_d max_d) with A = (Q1 - Q2) / 2, B = (Q1 + Q2) / 2,
  // Q1_d = sum_h q_hd and Q2_d = sum_h |q_hd|: one dot product per page for
  // any G.  Sixteen lanes score one page (lane holding channels E l .. E l +
  // E - 1 of the page's min and max rows), so a wave scores 4 pages per
  // instruction and sums over 16 lanes.
  __shared__ float sab[2 * D];
  constexpr int E = D / 16;
  const int lane = tid & 63;
  const int w = wave_id();
  const int sub = lane >> 4;  // which of the wave's 4 pages
  const int c0 = E * (lane & 15);
  for (int d = tid; d < D; d += kSelThreads) {
    float q1 = 0.f, q2 = 0.f;
    for (int h = 0; h < G; ++h) {
      const float x = lo16_to_f32<T>(q[((int64_t)b * H + hk * G + h) * D + d]);
      q1 += x;
      q2 += fabsf(x);
    }
    sab[d] = 0.5f * (q1 - q2);
    sab[D + d] = 0.5f * (q1 + q2);
  }
  int P2 = 1;
  while (P2 < n_pages) P2 <<= 1;
  __syncthreads();
  float va[E], vb[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    va[e] = sab[c0 + e];
    vb[e] = sab[D + c0 + e];
  }

  const int* table = block_tables + (int64_t)b * max_blocks;
  constexpr int U = 4;  // 4 pages per lane group per iteration: 16 pages per wave
  for (int base = 16 * w; base < P2; base += 16 * (kSelThreads / 64)) {
    constexpr int NV = E / 4;  // 8-byte pieces of the lane's channels
    u32x2 mn[U][NV], mx[U][NV];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = base + 4 * u + sub;
      const int blk = p < n_pages ? table[p] : -1;
      ok[u] = blk >= 0 && blk < num_blocks;
      if (ok[u]) {
        const uint16_t* m = kmeta + ((int64_t)blk * Hkv + hk) * 2 * D + c0;
#pragma unroll
        for (int x = 0; x < NV; ++x) {
          mn[u][x] = *reinterpret_cast<const u32x2*>(m + 4 * x);
          mx[u][x] = *reinterpret_cast<const u32x2*>(m + D + 4 * x);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = base + 4 * u + sub;
      float part = 0.f;
      if (ok[u]) {
#pragma unroll
        for (int x = 0; x < NV; ++x)
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int e = 4 * x + 2 * i;
            part = __builtin_fmaf(va[e], lo16_to_f32<T>(mn[u][x][i]), part);
            part = __builtin_fmaf(vb[e], lo16_to_f32<T>(mx[u][x][i]), part);
            part = __builtin_fmaf(va[e + 1], hi16_to_f32<T>(mn[u][x][i]), part);
            part = __builtin_fmaf(vb[e + 1], hi16_to_f32<T>(mx[u][x][i]), part);
          }
      }
#pragma unroll
      for (int x = 8; x >= 1; x >>= 1) part += __shfl_xor(part, x, 64);
      if ((lane & 15) == 0 && p < P2) {
        skey[p] = ok[u] ? part : -INFINITY;
        sidx[p] = p < n_pages ? p : 0x7fffffff;  // padding sorts last
      }
    }
  }
  __syncthreads();

  // Top-K by radix select: the key of the K-th best page is found 8 bits at a
  // time (most significant first) from LDS histograms of the order-preserving
  // integer form of the scores; every page above it is kept, and of the pages
  // equal to it the lowest ones, up to K in all.  Pages are then listed in
  // ascending order.  Thread t owns pages [t * per, (t + 1) * per).
  const int per = (n_pages + kSelThreads - 1) / kSelThreads;
  const int p0 = tid * per;
  const int p1 = p0 + per < n_pages ? p0 + per : n_pages;
  auto ukey = [&](int p) -> uint32_t {  // larger score -> larger key
    const uint32_t u = __float_as_uint(skey[p]);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  };
  uint32_t thr = 0;  // key of the K-th best page
  int need = keep;   // how many pages equal to thr are kept
  if (keep > 0 && keep < n_pages) {
    uint32_t mask = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) scount[tid] = 0;
      __syncthreads();
      for (int p = p0; p < p1; ++p) {
        const uint32_t u = ukey(p);
        if ((u & mask) == thr) atomicAdd(&scount[(u >> shift) & 255], 1);
      }
      __syncthreads();
      // wave 0 finds the digit: lane l holds bins 255 - 4l .. 252 - 4l
      if (tid < 64) {
        int c[4], tot = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          c[i] = scount[255 - 4 * tid - i];
          tot += c[i];
        }
        int incl = tot;  // inclusive prefix over lanes (bins in descending order)
#pragma unroll
        for (int x = 1; x < 64; x <<= 1) {
          const int y = __shfl_up(incl, x, 64);
          if (tid >= x) incl += y;
        }
        int above = incl - tot;  // pages in higher bins
        if (above < need && need <= incl) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (above < need && need <= above + c[i]) {
              sidx[0] = 255 - 4 * tid - i;  // the digit (sidx[0] is free scratch here)
              sidx[1] = need - above;
            }
            above += c[i];
          }
        }
      }
      __syncthreads();
      thr |= (uint32_t)sidx[0] << shift;
      need = sidx[1];
      mask |= 255u << shift;
      __syncthreads();
    }
  }
  // Block-wide exclusive prefix of one int per thread.
  auto block_scan = [&](int v) -> int {
    int incl = v;
#pragma unroll
    for (int x = 1; x < 64; x <<= 1) {
      const int y = __shfl_up(incl, x, 64);
      if ((tid & 63) >= x) incl += y;
    }
    __syncthreads();
    if ((tid & 63) == 63) scount[tid >> 6] = incl;
    __syncthreads();
    int off = 0;
    for (int x = 0; x < (tid >> 6); ++x) off += scount[x];
    return off + incl - v;
  };
  // Rank of each page equal to thr among those equal to it, in page order.
  int n_eq = 0;
  for (int p = p0; p < p1; ++p) n_eq += keep > 0 && keep < n_pages && ukey(p) == thr;
  int eq_rank = block_scan(n_eq);
  int n_kept = 0;
  bool kept_flags[kQuestMaxPages / kSelThreads];
#pragma unroll
  for (int i = 0; i < kQuestMaxPages / kSelThreads; ++i) {
    const int p = p0 + i;
    bool k = false;
    if (p < p1) {
      if (keep >= n_pages) {
        k = true;
      } else if (keep > 0) {
        const uint32_t u = ukey(p);
        k = u > thr || (u == thr && eq_rank++ < need);
      }
    }
    kept_flags[i] = k;
    n_kept += k;
  }
  int pos = block_scan(n_kept);
  int* out = selected + ((int64_t)b * Hkv + hk) * topk;
#pragma unroll
  for (int i = 0; i < kQuestMaxPages / kSelThreads; ++i)
    if (kept_flags[i]) out[pos++] = p0 + i;
  if (tid == 0) n_selected[(int64_t)b * Hkv + hk] = keep;
}

// ============================================================ launchers
template <int D, typename T>
static hipError_t launch_minmax_t(const QuestArgs& a) {
  const int64_t n_items = a.B * a.max_blocks * a.Hkv * (D / 8);
  hipLaunchKernelGGL((fa_quest_minmax_kernel<D, T>), dim3((unsigned)((n_items + 255) / 256)), dim3(256), 0, a.stream,
                     (const uint16_t*)a.k_cache, a.block_tables, a.context_lens, (uint16_t*)a.kmeta, n_items,
                     (int)a.Hkv, (int)a.block_size, a.num_blocks, (int)a.max_blocks);
  return hipGetLastError();
}
template <int D, typename T>
static hipError_t launch_select_t(const QuestArgs& a) {
  hipLaunchKernelGGL((fa_quest_select_kernel<D, T>), dim3((unsigned)(a.B * a.Hkv)), dim3(kSelThreads), 0, a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.kmeta, a.block_tables, a.context_lens, a.selected,
                     a.n_selected, (int)a.H, (int)a.Hkv, (int)(a.H / a.Hkv), (int)a.block_size, a.num_blocks,
                     (int)a.max_blocks, (int)a.topk);
  return hipGetLastError();
}
hipError_t launch_quest_minmax(const QuestArgs& a) {
  if (a.dtype == BF16::code)
    return a.D == 64 ? launch_minmax_t<64, BF16>(a)
                     : (a.D == 128 ? launch_minmax_t<128, BF16>(a) : launch_minmax_t<256, BF16>(a));
  return a.D == 64 ? launch_minmax_t<64, F16>(a)
                   : (a.D == 128 ? launch_minmax_t<128, F16>(a) : launch_minmax_t<256, F16>(a));
}
hipError_t launch_quest_select(const QuestArgs& a) {
  if (a.dtype == BF16::code)
    return a.D == 64 ? launch_select_t<64, BF16>(a)
                     : (a.D == 128 ? launch_select_t<128, BF16>(a) : launch_select_t<256, BF16>(a));
  return a.D == 64 ? launch_select_t<64, F16>(a)
                   : (a.D == 128 ? launch_select_t<128, F16>(a) : launch_select_t<256, F16>(a));
}

}  // namespace fa
