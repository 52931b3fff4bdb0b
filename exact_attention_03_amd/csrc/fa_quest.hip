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
// One workgroup per (sequence, key/value head): the page scores go to LDS,
// a bitonic sort orders (score, page) by score descending and page
// ascending, the first topk pages are flagged, and a prefix count over the
// flags writes them in ascending page order.
constexpr int kQuestMaxPages = 4096;

template <int D, typename T>
__global__ __launch_bounds__(256) void fa_quest_select_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kmeta, const int* __restrict__ block_tables,
    const int* __restrict__ context_lens, int* __restrict__ selected, int* __restrict__ n_selected, int H, int Hkv,
    int G, int bs, int64_t num_blocks, int max_blocks, int topk) {
  __shared__ float sq[16 * D];
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

  for (int e = tid; e < G * D; e += 256) {
    const int h = hk * G + e / D;
    const uint16_t x = q[((int64_t)b * H + h) * D + e % D];
    sq[e] = lo16_to_f32<T>(x);
  }
  int P2 = 1;
  while (P2 < n_pages) P2 <<= 1;
  __syncthreads();

  const int* table = block_tables + (int64_t)b * max_blocks;
  for (int p = tid; p < P2; p += 256) {
    float s = -INFINITY;
    int idx = 0x7fffffff;  // padding sorts last
    if (p < n_pages) {
      idx = p;
      const int blk = table[p];
      if (blk >= 0 && blk < num_blocks) {
        const uint16_t* m = kmeta + ((int64_t)blk * Hkv + hk) * 2 * D;
        s = 0.f;
        for (int d = 0; d < D; d += 8) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(m + d);
          const u32x4 z = *reinterpret_cast<const u32x4*>(m + D + d);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float mn = (i & 1) ? hi16_to_f32<T>(a[i / 2]) : lo16_to_f32<T>(a[i / 2]);
            const float mx = (i & 1) ? hi16_to_f32<T>(z[i / 2]) : lo16_to_f32<T>(z[i / 2]);
            for (int h = 0; h < G; ++h) {
              const float qd = sq[h * D + d + i];
              s += fmaxf(qd * mn, qd * mx);
            }
          }
        }
      }
    }
    skey[p] = s;
    sidx[p] = idx;
  }
  __syncthreads();

  // Bitonic sort of P2 entries: "before" = higher score, or equal score and
  // lower page.
  for (int k = 2; k <= P2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < P2; i += 256) {
        const int l = i ^ j;
        if (l > i) {
          const float si = skey[i], sl = skey[l];
          const int ii = sidx[i], il = sidx[l];
          const bool l_before_i = sl > si || (sl == si && il < ii);
          const bool i_before_l = si > sl || (si == sl && ii < il);
          const bool up = (i & k) == 0;  // this run sorts "before" first
          if (up ? l_before_i : i_before_l) {
            skey[i] = sl;
            skey[l] = si;
            sidx[i] = il;
            sidx[l] = ii;
          }
        }
      }
      __syncthreads();
    }
  }

  // Flag the kept pages (the first `keep` entries), then list them in order:
  // thread t owns pages [t * per, (t + 1) * per).
  const int kept0 = tid < keep ? sidx[tid] : -1;  // first 256 kept pages, read before reuse
  int kept_more[kQuestMaxPages / 256 - 1];
#pragma unroll
  for (int r = 1; r < kQuestMaxPages / 256; ++r) {
    const int e = r * 256 + tid;
    kept_more[r - 1] = e < keep ? sidx[e] : -1;
  }
  __syncthreads();
  for (int p = tid; p < n_pages; p += 256) sidx[p] = 0;
  __syncthreads();
  if (kept0 >= 0) sidx[kept0] = 1;
#pragma unroll
  for (int r = 0; r < kQuestMaxPages / 256 - 1; ++r)
    if (kept_more[r] >= 0) sidx[kept_more[r]] = 1;
  __syncthreads();
  const int per = (n_pages + 255) / 256;
  const int p0 = tid * per;
  int cnt = 0;
  for (int p = p0; p < p0 + per && p < n_pages; ++p) cnt += sidx[p];
  scount[tid] = cnt;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int t = 0; t < 256; ++t) {
      const int c = scount[t];
      scount[t] = run;
      run += c;
    }
  }
  __syncthreads();
  int* out = selected + ((int64_t)b * Hkv + hk) * topk;
  int pos = scount[tid];
  for (int p = p0; p < p0 + per && p < n_pages; ++p)
    if (sidx[p]) out[pos++] = p;
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
  hipLaunchKernelGGL((fa_quest_select_kernel<D, T>), dim3((unsigned)(a.B * a.Hkv)), dim3(256), 0, a.stream,
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
