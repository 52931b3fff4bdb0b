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
  // Query rows of every head and problem together: Z*H*N dense, H*T packed
  // (the offset of the second plane of stats).
  int64_t rows() const { return cu_seqlens ? H * T : Z * H * N; }
};

hipError_t launch_fwd(const FwdArgs& a);
hipError_t launch_bwd_pre(const BwdArgs& a);
hipError_t launch_bwd_dkdv(const BwdArgs& a);
hipError_t launch_bwd_dq(const BwdArgs& a);

// Resident dK/dV workgroups per CU for (D, dtype), from the occupancy API.
hipError_t dkdv_blocks_per_cu(int D, int dtype, int* out);

// Queries per forward workgroup and keys per forward K/V tile.
constexpr int kFwdQueries = 128;
constexpr int fwd_keys(int D) { return D == 64 ? 64 : 32; }

// Keys per dK/dV work unit and queries per staged tile of the dK/dV kernel.
// Waves per dK/dV workgroup (32 keys each) and keys per dK/dV work unit.
constexpr int dkdv_waves(int /*D*/) { return 4; }
constexpr int dkdv_keys(int D) { return 32 * dkdv_waves(D); }
constexpr int dkdv_queries(int /*D*/) { return 32; }

}  // namespace fa
