// fa_kernels.h - internal launch interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
  int64_t Z, H, N, D;
  int64_t Hkv;  // key/value heads (H a whole multiple of it; H for plain attention)
  int dtype, o_dtype;
  const void *q, *k, *v;
  void* o;
  float* lse;
  float scale;
  int causal;
  hipStream_t stream;
  // Variable-length batches: Z sequences packed head-major, (H, T, D), with
  // sequence z at tokens cu_seqlens[z] .. cu_seqlens[z+1]-1 (device int32)
  // and N the longest sequence.  nullptr for dense (Z, H, N, D) batches.
  const int* cu_seqlens = nullptr;
  int64_t T = 0;
};

struct BwdArgs {
  int64_t Z, H, N, D;
  int64_t Hkv;  // key/value heads (H a whole multiple of it; H for plain attention)
  int dtype, o_dtype;
  const void *q, *k, *v, *o, *dout;
  const float* lse;  // preprocess input
  // (2, Z, H, N) float32 written by the preprocess and read by the gradient
  // passes: plane 0 = Delta, plane 1 = lse * log2(e).
  float* stats;
  void *dq, *dk, *dv;
  float scale;
  int causal;
  int num_programs;  // persistent dK/dV grid; resolved by the caller (> 0)
  // dQ pass: compute the row statistics from o and lse and write them to
  // stats (instead of reading them from the preprocess pass).
  bool dq_stats;
  hipStream_t stream;
  const int* cu_seqlens = nullptr;  // as in FwdArgs
  int64_t T = 0;
  // Fused per-head backward: the heads' fp32 dQ partials, Z*H*ceil(N/32)*32*D floats.
  float* partial = nullptr;
  // Query rows of every head and problem together: Z*H*N dense, H*T packed
  // (the offset of the second plane of stats).
  int64_t rows() const { return cu_seqlens ? H * T : Z * H * N; }
};

// Paged KV cache writes: token i's key / value rows (num_tokens, Hkv, D) go
// to block slots[i] / block_size, offset slots[i] % block_size.
struct CacheArgs {
  int64_t num_tokens, Hkv, D, block_size, num_blocks;
  const void *key, *value;
  const int64_t* slots;
  void *k_cache, *v_cache;
  hipStream_t stream;
};

// One paged KV source of a decode call: a cache with its block table and
// context lengths, attended whole or, with a selection, over its kept pages.
struct DecodeSource {
  const void *k_cache, *v_cache;
  const int* block_tables;
  const int* context_lens;
  int64_t block_size, num_blocks, max_blocks;
  // Sparse decode: the kept logical pages of each (sequence, key/value head),
  // (B, Hkv, topk) ascending, and their count (B, Hkv); nullptr for dense.
  const int* selected = nullptr;
  const int* n_selected = nullptr;
  int64_t topk = 0;
  const int* row_lens = nullptr;  // (B, Tq): tokens of this source each query row sees; nullptr = all
  int n_splits = 1;   // context splits of this source per (sequence, key/value head)
  int64_t chunk = 64;  // context tokens per split (a multiple of 64; the last split takes the rest)
};

// Decode attention (one query token per sequence) over one or two paged KV
// sources whose tokens share one softmax.
struct DecodeArgs {
  int64_t B, H, Hkv, D;
  int64_t Tq = 1;  // query tokens per sequence
  int dtype, o_dtype;
  const void* q;
  DecodeSource src[2];
  int n_sources;
  void* o;
  float* lse;  // may be nullptr
  float scale;
  // With more than one split over all sources: (B, Tq, H, S, D) partial
  // outputs, then (B, Tq, H, S) partial lse, S = the sources' splits together.
  float* workspace;
  hipStream_t stream;
};

// Query-aware page selection over a paged cache: page key min / max, then
// per (sequence, key/value head) the topk best pages.
struct QuestArgs {
  int64_t B, H, Hkv, D, block_size, num_blocks, max_blocks, topk;
  int dtype;
  const void* q;
  const void* k_cache;
  const int* block_tables;
  const int* context_lens;
  void* kmeta;     // (num_blocks, Hkv, 2, D) dtype
  int* selected;   // (B, Hkv, topk) int32
  int* n_selected; // (B, Hkv) int32
  hipStream_t stream;
};
hipError_t launch_quest_minmax(const QuestArgs& a);
hipError_t launch_quest_select(const QuestArgs& a);
constexpr int kQuestMaxPages = 4096;  // pages per context the selection handles (LDS sized for it)

hipError_t launch_reshape_and_cache(const CacheArgs& a);
hipError_t launch_paged_decode(const DecodeArgs& a);

// Context split of the decode kernel for B sequences over Hkv key/value heads
// and contexts up to max_context tokens.  Every split holds the same number
// of context tokens (chunk, a multiple of 64), so that workgroups of
// sequences of very different lengths carry equal work and the dispatcher
// balances them; chunk is sized for about 1024 (sequence, head, split)
// workgroups when every context has max_context tokens, at least 256 tokens
// (64 per wave) and at most 64 splits per sequence.  Shapes only, so that the
// workspace size is known without a device.
struct DecodeSplit {
  int64_t chunk;
  int n_splits;
};
inline DecodeSplit decode_split(int64_t B, int64_t Hkv, int64_t max_context) {
  const int64_t groups = B * Hkv;
  if (groups <= 0 || max_context <= 0) return {64, 1};
  const int64_t want = 1024;
  int64_t chunk = (groups * max_context + want - 1) / want;
  if (chunk < 256) chunk = 256;
  chunk = (chunk + 63) / 64 * 64;
  int64_t s = (max_context + chunk - 1) / chunk;
  if (s > 64) {
    s = 64;
    chunk = ((max_context + s - 1) / s + 63) / 64 * 64;
    s = (max_context + chunk - 1) / chunk;
  }
  return {chunk, (int)(s < 1 ? 1 : s)};
}

hipError_t launch_fwd(const FwdArgs& a);
hipError_t launch_bwd_pre(const BwdArgs& a);
hipError_t launch_bwd_dkdv(const BwdArgs& a);
hipError_t launch_bwd_dq(const BwdArgs& a);

// Resident dK/dV workgroups per CU for (D, dtype), from the occupancy API.
hipError_t dkdv_blocks_per_cu(int D, int dtype, int* out);

// The fused per-head backward (dQ, dK, dV in one pass, persistent programs
// over heads) and its resident workgroups per CU.
hipError_t launch_bwd_fused(const BwdArgs& a);
hipError_t fused_blocks_per_cu(int D, int dtype, int* out);

// Entry points of the C ABI layer for other translation units: record an
// error message (returns status), and fa_bwd itself (argument checks, both
// stages) with the caller's workspace.
int api_error(int status, const char* message);
int api_bwd(int64_t Z, int64_t H, int64_t N, int64_t D, int dtype, int o_dtype, const void* q, const void* k,
            const void* v, const void* o, const void* dout, const float* lse, void* dq, void* dk, void* dv,
            float scale, int causal, void* workspace, size_t workspace_bytes, hipStream_t stream);

// Queries per forward workgroup and keys per forward K/V tile.
constexpr int kFwdQueries = 128;
constexpr int fwd_keys(int D) { return D == 64 ? 64 : 32; }

// Keys per dK/dV work unit and queries per staged tile of the dK/dV kernel.
// Waves per dK/dV workgroup (32 keys each) and keys per dK/dV work unit.
constexpr int dkdv_waves(int /*D*/) { return 4; }
constexpr int dkdv_keys(int D) { return 32 * dkdv_waves(D); }
constexpr int dkdv_queries(int /*D*/) { return 32; }

}  // namespace fa
