// fa_noalloc.hip - the backward without a caller workspace, for callers that
// cannot allocate device memory (code under graph capture, serving loops,
// harnesses that forbid allocation).
//
// fa_bwd keeps the per-row statistics (Delta and lse * log2 e, two float32 per
// query row) in a workspace between its two stages.  Here that workspace is a
// fixed array in the library's own device memory, `scratch`, which every GPU
// the library runs on holds from module load until the process ends.  Host
// code never passes the array's host-side name to a kernel: on the first call
// on each device (with that device current) hipGetSymbolAddress gives the
// device address of that GPU's copy, which is kept per device and used from
// then on.  Nothing here allocates or frees memory.
//
// Every call on one GPU shares that GPU's array and leaves the last call's
// statistics in it; nothing needs clearing, since the first stage writes every
// row the second reads.  Calls that overlap on one GPU (on different streams,
// or from different threads) race on the array.
#include "fa.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "fa_kernels.h"

namespace {

static_assert(FA_BWD_NOALLOC_MAX_ROWS == (int64_t)1 << 22, "scratch sized for the documented maximum");
constexpr int64_t kScratchFloats = 2 * (int64_t)FA_BWD_NOALLOC_MAX_ROWS;  // 32 MiB

static __device__ __align__(256) float scratch[kScratchFloats];

struct ScratchAddress {
  std::once_flag once;
  hipError_t err = hipSuccess;
  float* ptr = nullptr;
};
constexpr int kMaxDevices = 64;
ScratchAddress g_scratch[kMaxDevices];

}  // namespace

extern "C" int fa_bwd_noalloc(int64_t Z, int64_t H, int64_t N, int64_t D, int dtype, int o_dtype, const void* q,
                              const void* k, const void* v, const void* o, const void* dout, const float* lse,
                              void* dq, void* dk, void* dv, float scale, int causal, hipStream_t stream) {
  if (Z > 0 && H > 0 && N > 0 &&
      (Z > FA_BWD_NOALLOC_MAX_ROWS || H > FA_BWD_NOALLOC_MAX_ROWS || N > FA_BWD_NOALLOC_MAX_ROWS ||
       Z * H > FA_BWD_NOALLOC_MAX_ROWS || Z * H * N > FA_BWD_NOALLOC_MAX_ROWS))
    return fa::api_error(FA_ERR_UNSUPPORTED,
                         "fa_bwd_noalloc: Z*H*N exceeds FA_BWD_NOALLOC_MAX_ROWS (4194304 query rows); use fa_bwd "
                         "with a workspace");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fa::api_error(FA_ERR_HIP, "fa_bwd_noalloc: hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return fa::api_error(FA_ERR_HIP, "fa_bwd_noalloc: device index out of range");
  ScratchAddress& s = g_scratch[dev];
  std::call_once(s.once, [&s] {
    void* p = nullptr;
    s.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    s.ptr = static_cast<float*>(p);
  });
  if (s.err != hipSuccess || s.ptr == nullptr)
    return fa::api_error(FA_ERR_HIP, "fa_bwd_noalloc: hipGetSymbolAddress of the scratch array failed");
  return fa::api_bwd(Z, H, N, D, dtype, o_dtype, q, k, v, o, dout, lse, dq, dk, dv, scale, causal, s.ptr,
                     (size_t)kScratchFloats * sizeof(float), stream);
}
