// fa_api.cpp - the C ABI declared in include/fa.h.
//
// Argument validation (pure host code, no HIP call), dispatch to the kernel
// launchers, per-device launch facts cached once, and error reporting.
#include "fa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "fa_kernels.h"
#include "fa_schedule.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(FA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool debug_sync() {
  static const bool on = [] {
    const char* s = std::getenv("FA_DEBUG_SYNC");
    return s != nullptr && s[0] != '\0' && s[0] != '0';
  }();
  return on;
}

constexpr int64_t kMaxI32 = 2147483647;

struct Shape {
  int64_t Z, H, N, D;
  int64_t heads() const { return Z * H; }
  bool empty() const { return Z == 0 || H == 0 || N == 0; }
};

int check_shape(const Shape& s) {
  if (s.Z < 0 || s.H < 0 || s.N < 0 || s.D < 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "negative size (Z=%lld H=%lld N=%lld D=%lld)", (long long)s.Z,
                (long long)s.H, (long long)s.N, (long long)s.D);
  if (s.D != 64 && s.D != 128 && s.D != 256)
    return fail(FA_ERR_UNSUPPORTED, "head dim D=%lld not supported (64, 128 or 256)", (long long)s.D);
  if (s.empty()) return FA_OK;
  // Kernels index one head with 32-bit byte offsets (fp32 O included, plus a
  // tile of padding rows) and launch up to heads * tiles workgroups.
  if (s.Z > kMaxI32 || s.H > kMaxI32 || s.N > kMaxI32 || s.heads() > kMaxI32 ||
      (s.N + 256) * s.D * 4 > kMaxI32)
    return fail(FA_ERR_UNSUPPORTED, "problem too large (Z=%lld H=%lld N=%lld D=%lld)", (long long)s.Z,
                (long long)s.H, (long long)s.N, (long long)s.D);
  if (s.heads() * ((s.N + 63) / 64) > kMaxI32)
    return fail(FA_ERR_UNSUPPORTED, "grid too large (Z*H=%lld N=%lld)", (long long)s.heads(), (long long)s.N);
  return FA_OK;
}

// Grouped key/value heads: H query heads over Hkv key/value heads, H a whole
// multiple of Hkv.  The dK/dV pass indexes the G = H / Hkv query heads of a
// group with one 32-bit byte offset.
int check_groups(const Shape& s, int64_t Hkv) {
  if (Hkv < 0) return fail(FA_ERR_INVALID_ARGUMENT, "negative Hkv=%lld", (long long)Hkv);
  if (s.H == 0) return FA_OK;
  if (Hkv == 0 || s.H % Hkv != 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "H=%lld query heads must be a whole multiple of Hkv=%lld key/value heads",
                (long long)s.H, (long long)Hkv);
  const int64_t G = s.H / Hkv;
  if (!s.empty() && G * (s.N + 256) * s.D * 2 > kMaxI32)
    return fail(FA_ERR_UNSUPPORTED, "group too large (H/Hkv=%lld N=%lld D=%lld)", (long long)G, (long long)s.N,
                (long long)s.D);
  // Query-tile grids pad the key/value heads to a multiple of the XCD count.
  if (!s.empty() && (s.Z * Hkv + fa::kXcds) * G * ((s.N + 63) / 64) > kMaxI32)
    return fail(FA_ERR_UNSUPPORTED, "grid too large (Z*Hkv=%lld H/Hkv=%lld N=%lld)", (long long)(s.Z * Hkv),
                (long long)G, (long long)s.N);
  return FA_OK;
}

// Variable-length batches: Z sequences packed head-major, (H, T, D), at the
// token offsets cu (device int32, Z+1 entries), N = the longest sequence.
// Dense batches have cu == nullptr.
struct Packing {
  const int* cu = nullptr;
  int64_t T = 0;
  bool packed() const { return cu != nullptr; }
};

int check_packing(const Shape& s, int64_t Hkv, const Packing& pk) {
  if (!pk.packed()) return FA_OK;
  if (pk.T < 0) return fail(FA_ERR_INVALID_ARGUMENT, "negative token count T=%lld", (long long)pk.T);
  if (reinterpret_cast<uintptr_t>(pk.cu) % 4 != 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "cu_seqlens is not 4-byte aligned");
  if (s.empty() || pk.T == 0 || Hkv == 0) return FA_OK;
  // Row offsets of one group of query heads (G heads T rows apart) and of one
  // head's T rows stay 32-bit; the offsets array is read as int32.
  const int64_t G = s.H / Hkv;
  if (G * (pk.T + 256) * s.D * 2 > kMaxI32 || (pk.T + 256) * s.D * 4 > kMaxI32 || pk.T > kMaxI32)
    return fail(FA_ERR_UNSUPPORTED, "packed batch too large (T=%lld H/Hkv=%lld D=%lld)", (long long)pk.T,
                (long long)G, (long long)s.D);
  return FA_OK;
}

int check_dtypes(int dtype, int o_dtype, bool need_o) {
  if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16)
    return fail(FA_ERR_INVALID_ARGUMENT, "dtype %d must be FA_DTYPE_F16 or FA_DTYPE_BF16", dtype);
  if (need_o && o_dtype != dtype && o_dtype != FA_DTYPE_F32)
    return fail(FA_ERR_INVALID_ARGUMENT, "o_dtype %d must equal dtype (%d) or be FA_DTYPE_F32", o_dtype, dtype);
  return FA_OK;
}

int check_ptr(const void* p, const char* name) {
  if (p == nullptr) return fail(FA_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);
  return FA_OK;
}

int check_scale(float scale, int causal) {
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(FA_ERR_INVALID_ARGUMENT, "scale must be finite and > 0 (got %g)", (double)scale);
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1 (got %d)", causal);
  return FA_OK;
}

#define FA_TRY(x)            \
  do {                       \
    const int st_ = (x);     \
    if (st_ != FA_OK) return st_; \
  } while (0)

// Per-device launch facts, filled once per device.
struct DeviceFacts {
  std::once_flag once;
  hipError_t err = hipSuccess;
  int cus = 0;
  int dkdv_per_cu[3][2] = {};   // [D index][dtype]
  int fused_per_cu[3][2] = {};  // [D index][dtype]
};
constexpr int kMaxDevices = 64;
DeviceFacts g_facts[kMaxDevices];

int d_index(int64_t D) { return D == 64 ? 0 : (D == 128 ? 1 : 2); }

int device_facts(DeviceFacts** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(FA_ERR_HIP, "device index %d out of range", dev);
  DeviceFacts& f = g_facts[dev];
  std::call_once(f.once, [&f, dev] {
    int cus = 0;
    f.err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (f.err != hipSuccess) return;
    f.cus = cus;
    const int Ds[3] = {64, 128, 256};
    for (int di = 0; di < 3; ++di)
      for (int dt = 0; dt < 2; ++dt) {
        f.err = fa::dkdv_blocks_per_cu(Ds[di], dt, &f.dkdv_per_cu[di][dt]);
        if (f.err != hipSuccess) return;
        f.err = fa::fused_blocks_per_cu(Ds[di], dt, &f.fused_per_cu[di][dt]);
        if (f.err != hipSuccess) return;
      }
  });
  if (f.err != hipSuccess) return hip_fail(f.err, "querying device attributes");
  *out = &f;
  return FA_OK;
}

int finish(hipError_t launch_err, hipStream_t stream, const char* what) {
  if (launch_err != hipSuccess) return hip_fail(launch_err, what);
  if (debug_sync()) {
    hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, what);
  }
  return FA_OK;
}

int validate_bwd_common(const Shape& s, int dtype, const void* q, const void* k, const void* v,
                        const void* dout, const float* stats, float scale, int causal) {
  FA_TRY(check_shape(s));
  FA_TRY(check_dtypes(dtype, dtype, false));
  FA_TRY(check_scale(scale, causal));
  if (s.empty()) return FA_OK;
  FA_TRY(check_ptr(q, "q"));
  FA_TRY(check_ptr(k, "k"));
  FA_TRY(check_ptr(v, "v"));
  FA_TRY(check_ptr(dout, "dout"));
  FA_TRY(check_ptr(stats, "stats"));
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_version(void) { return 100; }

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARGUMENT: return "FA_ERR_INVALID_ARGUMENT";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    default: return "FA_UNKNOWN_STATUS";
  }
}

const char* fa_last_error(void) { return g_last_error.c_str(); }

size_t fa_bwd_workspace_bytes(int64_t Z, int64_t H, int64_t N, int64_t D) {
  (void)D;
  if (Z <= 0 || H <= 0 || N <= 0) return 0;
  return 2 * (size_t)(Z * H * N) * sizeof(float);
}

}  // extern "C"

namespace {

int fwd_impl(int64_t Z, int64_t H, int64_t Hkv, int64_t N, int64_t D, int dtype, int o_dtype, const void* q,
             const void* k, const void* v, void* o, float* lse, float scale, int causal, hipStream_t stream,
             const Packing& pk = Packing{}) {
  g_last_error.clear();
  const Shape s{Z, H, N, D};
  FA_TRY(check_shape(s));
  FA_TRY(check_groups(s, Hkv));
  FA_TRY(check_packing(s, Hkv, pk));
  FA_TRY(check_dtypes(dtype, o_dtype, true));
  FA_TRY(check_scale(scale, causal));
  if (s.empty() || (pk.packed() && pk.T == 0)) return FA_OK;
  FA_TRY(check_ptr(q, "q"));
  FA_TRY(check_ptr(k, "k"));
  FA_TRY(check_ptr(v, "v"));
  FA_TRY(check_ptr(o, "o"));
  FA_TRY(check_ptr(lse, "lse"));
  fa::FwdArgs a{Z, H, N, D, Hkv, dtype, o_dtype, q, k, v, o, lse, scale, causal, stream, pk.cu, pk.T};
  return finish(fa::launch_fwd(a), stream, "fa_fwd launch");
}

}  // namespace

extern "C" {

int fa_fwd(int64_t Z, int64_t H, int64_t N, int64_t D, int dtype, int o_dtype, const void* q, const void* k,
           const void* v, void* o, float* lse, float scale, int causal, hipStream_t stream) {
  return fwd_impl(Z, H, H, N, D, dtype, o_dtype, q, k, v, o, lse, scale, causal, stream);
}

int fa_fwd_gqa(int64_t Z, int64_t H, int64_t Hkv, int64_t N, int64_t D, int dtype, int o_dtype, const void* q,
               const void* k, const void* v, void* o, float* lse, float scale, int causal, hipStream_t stream) {
  return fwd_impl(Z, H, Hkv, N, D, dtype, o_dtype, q, k, v, o, lse, scale, causal, stream);
}

int fa_bwd_preprocess(int64_t Z, int64_t H, int64_t N, int64_t D, int dtype, int o_dtype, const void* o,
                      const void* dout, const float* lse, float* stats, hipStream_t stream) {
  g_last_error.clear();
  const Shape s{Z, H, N, D};
  FA_TRY(check_shape(s));
  FA_TRY(check_dtypes(dtype, o_dtype, true));
  if (s.empty()) return FA_OK;
  FA_TRY(check_ptr(o, "o"));
  FA_TRY(check_ptr(dout, "dout"));
  FA_TRY(check_ptr(lse, "lse"));
  FA_TRY(check_ptr(stats, "stats"));
  fa::BwdArgs a{};
  a.Z = Z; a.H = H; a.Hkv = H; a.N = N; a.D = D; a.dtype = dtype; a.o_dtype = o_dtype;
  a.o = o; a.dout = dout; a.lse = lse; a.stats = stats; a.stream = stream;
  return finish(fa::launch_bwd_pre(a), stream, "fa_bwd_preprocess launch");
}

}  // extern "C"

namespace {

int dkdv_impl(int64_t Z, int64_t H, int64_t Hkv, int64_t N, int64_t D, int dtype, const void* q, const void* k,
              const void* v, const void* dout, const float* stats, void* dk, void* dv, float scale, int causal,
              int num_programs, hipStream_t stream, const Packing& pk = Packing{}) {
  g_last_error.clear();
  const Shape s{Z, H, N, D};
  FA_TRY(validate_bwd_common(s, dtype, q, k, v, dout, stats, scale, causal));
  FA_TRY(check_groups(s, Hkv));
  FA_TRY(check_packing(s, Hkv, pk));
  if (num_programs < 0) return fail(FA_ERR_INVALID_ARGUMENT, "num_programs must be >= 0 (got %d)", num_programs);
  if (s.empty() || (pk.packed() && pk.T == 0)) return FA_OK;
  FA_TRY(check_ptr(dk, "dk"));
  FA_TRY(check_ptr(dv, "dv"));
  if (num_programs == 0) {
    DeviceFacts* f = nullptr;
    FA_TRY(device_facts(&f));
    num_programs = f->cus * f->dkdv_per_cu[d_index(D)][dtype];
  }
  fa::BwdArgs a{};
  a.Z = Z; a.H = H; a.Hkv = Hkv; a.N = N; a.D = D; a.dtype = dtype;
  a.q = q; a.k = k; a.v = v; a.dout = dout; a.stats = const_cast<float*>(stats);
  a.dk = dk; a.dv = dv; a.scale = scale; a.causal = causal; a.num_programs = num_programs; a.stream = stream;
  a.cu_seqlens = pk.cu; a.T = pk.T;
  return finish(fa::launch_bwd_dkdv(a), stream, "fa_bwd_dkdv launch");
}

}  // namespace

extern "C" {

int fa_bwd_dkdv(int64_t Z, int64_t H, int64_t N, int64_t D, int dtype, const void* q, const void* k,
                const void* v, const void* dout, const float* stats, void* dk, void* dv, float scale,
                int causal, int num_programs, hipStream_t stream) {
  return dkdv_impl(Z, H, H, N, D, dtype, q, k, v, dout, stats, dk, dv, scale, causal, num_programs, stream);
}

size_t fa_bwd_fused_workspace_bytes(int64_t Z, int64_t H, int64_t N, int64_t D) {
  if (Z <= 0 || H <= 0 || N <= 0 || D <= 0) return 0;
  return (size_t)(Z * H) * (size_t)((N + 31) / 32 * 32) * (size_t)D * sizeof(float);
}

int fa_bwd_fused(int64_t Z, int64_t H, int64_t N, int64_t D, int dtype, const void* q, const void* k,
                 const void* v, const void* dout, const float* stats, void* dq, void* dk, void* dv, float scale,
                 int causal, int num_programs, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_last_error.clear();
  const Shape s{Z, H, N, D};
  FA_TRY(validate_bwd_common(s, dtype, q, k, v, dout, stats, scale, causal));
  if (num_programs < 0) return fail(FA_ERR_INVALID_ARGUMENT, "num_programs must be >= 0 (got %d)", num_programs);
  if (s.empty()) return FA_OK;
  FA_TRY(check_ptr(dq, "dq"));
  FA_TRY(check_ptr(dk, "dk"));
  FA_TRY(check_ptr(dv, "dv"));
  FA_TRY(check_ptr(workspace, "workspace"));
  const size_t need = fa_bwd_fused_workspace_bytes(Z, H, N, D);
  if (workspace_bytes < need)
    return fail(FA_ERR_INVALID_ARGUMENT, "workspace of %zu bytes is smaller than the %zu bytes needed",
                workspace_bytes, need);
  if (num_programs == 0) {
    DeviceFacts* f = nullptr;
    FA_TRY(device_facts(&f));
    num_programs = f->cus * f->fused_per_cu[d_index(D)][dtype];
  }
  fa::BwdArgs a{};
  a.Z = Z; a.H = H; a.Hkv = H; a.N = N; a.D = D; a.dtype = dtype;
  a.q = q; a.k = k; a.v = v; a.dout = dout; a.stats = const_cast<float*>(stats);
  a.dq = dq; a.dk = dk; a.dv = dv; a.scale = scale; a.causal = causal; a.num_programs = num_programs;
  a.partial = static_cast<float*>(workspace); a.stream = stream;
  return finish(fa::launch_bwd_fused(a), stream, "fa_bwd_fused launch");
}

int fa_bwd_dq(int64_t Z, int64_t H, int64_t N, int64_t D, int dtype, const void* q, const void* k,
              const void* v, const void* dout, const float* stats, void* dq, float scale, int causal,
              hipStream_t stream) {
  g_last_error.clear();
  const Shape s{Z, H, N, D};
  FA_TRY(validate_bwd_common(s, dtype, q, k, v, dout, stats, scale, causal));
  if (s.empty()) return FA_OK;
  FA_TRY(check_ptr(dq, "dq"));
  fa::BwdArgs a{};
  a.Z = Z; a.H = H; a.Hkv = H; a.N = N; a.D = D; a.dtype = dtype;
  a.q = q; a.k = k; a.v = v; a.dout = dout; a.stats = const_cast<float*>(stats);
  a.dq = dq; a.scale = scale; a.causal = causal; a.stream = stream;
  return finish(fa::launch_bwd_dq(a), stream, "fa_bwd_dq launch");
}

}  // extern "C"

namespace {

int dq_and_stats_impl(int64_t Z, int64_t H, int64_t Hkv, int64_t N, int64_t D, int dtype, int o_dtype,
                      const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, float* stats, void* dq, float scale, int causal, hipStream_t stream,
                      const Packing& pk = Packing{}) {
  g_last_error.clear();
  const Shape s{Z, H, N, D};
  FA_TRY(check_shape(s));
  FA_TRY(check_groups(s, Hkv));
  FA_TRY(check_packing(s, Hkv, pk));
  FA_TRY(check_dtypes(dtype, o_dtype, true));
  FA_TRY(check_scale(scale, causal));
  if (s.empty() || (pk.packed() && pk.T == 0)) return FA_OK;
  FA_TRY(check_ptr(q, "q"));
  FA_TRY(check_ptr(k, "k"));
  FA_TRY(check_ptr(v, "v"));
  FA_TRY(check_ptr(o, "o"));
  FA_TRY(check_ptr(dout, "dout"));
  FA_TRY(check_ptr(lse, "lse"));
  FA_TRY(check_ptr(stats, "stats"));
  FA_TRY(check_ptr(dq, "dq"));
  fa::BwdArgs a{};
  a.Z = Z; a.H = H; a.Hkv = Hkv; a.N = N; a.D = D; a.dtype = dtype; a.o_dtype = o_dtype;
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse; a.stats = stats;
  a.dq = dq; a.scale = scale; a.causal = causal; a.dq_stats = true; a.stream = stream;
  a.cu_seqlens = pk.cu; a.T = pk.T;
  return finish(fa::launch_bwd_dq(a), stream, "fa_bwd_dq_and_stats launch");
}

// Both gradient passes: dQ with the row statistics into the workspace, then
// dK / dV from them.
int bwd_impl(int64_t Z, int64_t H, int64_t Hkv, int64_t N, int64_t D, int dtype, int o_dtype, const void* q,
             const void* k, const void* v, const void* o, const void* dout, const float* lse, void* dq, void* dk,
             void* dv, float scale, int causal, void* workspace, size_t workspace_bytes, hipStream_t stream,
             const Packing& pk = Packing{}) {
  g_last_error.clear();
  const Shape s{Z, H, N, D};
  FA_TRY(check_shape(s));
  FA_TRY(check_groups(s, Hkv));
  FA_TRY(check_packing(s, Hkv, pk));
  FA_TRY(check_dtypes(dtype, o_dtype, true));
  FA_TRY(check_scale(scale, causal));
  if (s.empty() || (pk.packed() && pk.T == 0)) return FA_OK;
  FA_TRY(check_ptr(q, "q"));
  FA_TRY(check_ptr(k, "k"));
  FA_TRY(check_ptr(v, "v"));
  FA_TRY(check_ptr(o, "o"));
  FA_TRY(check_ptr(dout, "dout"));
  FA_TRY(check_ptr(lse, "lse"));
  FA_TRY(check_ptr(dq, "dq"));
  FA_TRY(check_ptr(dk, "dk"));
  FA_TRY(check_ptr(dv, "dv"));
  FA_TRY(check_ptr(workspace, "workspace"));
  const size_t need = pk.packed() ? fa_bwd_workspace_bytes(1, H, pk.T, D) : fa_bwd_workspace_bytes(Z, H, N, D);
  if (workspace_bytes < need)
    return fail(FA_ERR_INVALID_ARGUMENT, "workspace of %zu bytes is smaller than the %zu bytes needed",
                workspace_bytes, need);
  float* stats = static_cast<float*>(workspace);
  FA_TRY(dq_and_stats_impl(Z, H, Hkv, N, D, dtype, o_dtype, q, k, v, o, dout, lse, stats, dq, scale, causal,
                           stream, pk));
  FA_TRY(dkdv_impl(Z, H, Hkv, N, D, dtype, q, k, v, dout, stats, dk, dv, scale, causal, 0, stream, pk));
  return FA_OK;
}

}  // namespace

namespace fa {

int api_error(int status, const char* message) { return fail(status, "%s", message); }

int api_bwd(int64_t Z, int64_t H, int64_t N, int64_t D, int dtype, int o_dtype, const void* q, const void* k,
            const void* v, const void* o, const void* dout, const float* lse, void* dq, void* dk, void* dv,
            float scale, int causal, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return bwd_impl(Z, H, H, N, D, dtype, o_dtype, q, k, v, o, dout, lse, dq, dk, dv, scale, causal, workspace,
                  workspace_bytes, stream);
}

}  // namespace fa

extern "C" {

int fa_bwd_dq_and_stats(int64_t Z, int64_t H, int64_t N, int64_t D, int dtype, int o_dtype, const void* q,
                        const void* k, const void* v, const void* o, const void* dout, const float* lse,
                        float* stats, void* dq, float scale, int causal, hipStream_t stream) {
  return dq_and_stats_impl(Z, H, H, N, D, dtype, o_dtype, q, k, v, o, dout, lse, stats, dq, scale, causal, stream);
}

int fa_bwd(int64_t Z, int64_t H, int64_t N, int64_t D, int dtype, int o_dtype, const void* q, const void* k,
           const void* v, const void* o, const void* dout, const float* lse, void* dq, void* dk, void* dv,
           float scale, int causal, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return bwd_impl(Z, H, H, N, D, dtype, o_dtype, q, k, v, o, dout, lse, dq, dk, dv, scale, causal, workspace,
                  workspace_bytes, stream);
}

int fa_bwd_gqa(int64_t Z, int64_t H, int64_t Hkv, int64_t N, int64_t D, int dtype, int o_dtype, const void* q,
               const void* k, const void* v, const void* o, const void* dout, const float* lse, void* dq, void* dk,
               void* dv, float scale, int causal, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return bwd_impl(Z, H, Hkv, N, D, dtype, o_dtype, q, k, v, o, dout, lse, dq, dk, dv, scale, causal, workspace,
                  workspace_bytes, stream);
}

int fa_bwd_dq_and_stats_gqa(int64_t Z, int64_t H, int64_t Hkv, int64_t N, int64_t D, int dtype, int o_dtype,
                            const void* q, const void* k, const void* v, const void* o, const void* dout,
                            const float* lse, float* stats, void* dq, float scale, int causal, hipStream_t stream) {
  return dq_and_stats_impl(Z, H, Hkv, N, D, dtype, o_dtype, q, k, v, o, dout, lse, stats, dq, scale, causal, stream);
}

int fa_bwd_dkdv_gqa(int64_t Z, int64_t H, int64_t Hkv, int64_t N, int64_t D, int dtype, const void* q,
                    const void* k, const void* v, const void* dout, const float* stats, void* dk, void* dv,
                    float scale, int causal, int num_programs, hipStream_t stream) {
  return dkdv_impl(Z, H, Hkv, N, D, dtype, q, k, v, dout, stats, dk, dv, scale, causal, num_programs, stream);
}

int fa_fwd_varlen(int64_t B, int64_t H, int64_t Hkv, int64_t T, int64_t max_seqlen, int64_t D, int dtype,
                  int o_dtype, const int32_t* cu_seqlens, const void* q, const void* k, const void* v, void* o,
                  float* lse, float scale, int causal, hipStream_t stream) {
  if (cu_seqlens == nullptr && B > 0 && H > 0 && max_seqlen > 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "cu_seqlens is NULL");
  return fwd_impl(B, H, Hkv, max_seqlen, D, dtype, o_dtype, q, k, v, o, lse, scale, causal, stream,
                  Packing{cu_seqlens, T});
}

int fa_bwd_varlen(int64_t B, int64_t H, int64_t Hkv, int64_t T, int64_t max_seqlen, int64_t D, int dtype,
                  int o_dtype, const int32_t* cu_seqlens, const void* q, const void* k, const void* v,
                  const void* o, const void* dout, const float* lse, void* dq, void* dk, void* dv, float scale,
                  int causal, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (cu_seqlens == nullptr && B > 0 && H > 0 && max_seqlen > 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "cu_seqlens is NULL");
  return bwd_impl(B, H, Hkv, max_seqlen, D, dtype, o_dtype, q, k, v, o, dout, lse, dq, dk, dv, scale, causal,
                  workspace, workspace_bytes, stream, Packing{cu_seqlens, T});
}

int fa_bwd_dq_and_stats_varlen(int64_t B, int64_t H, int64_t Hkv, int64_t T, int64_t max_seqlen, int64_t D,
                               int dtype, int o_dtype, const int32_t* cu_seqlens, const void* q, const void* k,
                               const void* v, const void* o, const void* dout, const float* lse, float* stats,
                               void* dq, float scale, int causal, hipStream_t stream) {
  if (cu_seqlens == nullptr && B > 0 && H > 0 && max_seqlen > 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "cu_seqlens is NULL");
  return dq_and_stats_impl(B, H, Hkv, max_seqlen, D, dtype, o_dtype, q, k, v, o, dout, lse, stats, dq, scale,
                           causal, stream, Packing{cu_seqlens, T});
}

int fa_bwd_dkdv_varlen(int64_t B, int64_t H, int64_t Hkv, int64_t T, int64_t max_seqlen, int64_t D, int dtype,
                       const int32_t* cu_seqlens, const void* q, const void* k, const void* v, const void* dout,
                       const float* stats, void* dk, void* dv, float scale, int causal, int num_programs,
                       hipStream_t stream) {
  if (cu_seqlens == nullptr && B > 0 && H > 0 && max_seqlen > 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "cu_seqlens is NULL");
  return dkdv_impl(B, H, Hkv, max_seqlen, D, dtype, q, k, v, dout, stats, dk, dv, scale, causal, num_programs,
                   stream, Packing{cu_seqlens, T});
}

int fa_reshape_and_cache(int64_t num_tokens, int64_t Hkv, int64_t D, int64_t block_size, int64_t num_blocks,
                         int dtype, const void* key, const void* value, const int64_t* slot_mapping, void* k_cache,
                         void* v_cache, hipStream_t stream) {
  g_last_error.clear();
  if (num_tokens < 0 || Hkv < 0 || num_blocks < 0 || block_size < 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "negative size (num_tokens=%lld Hkv=%lld num_blocks=%lld block_size=%lld)",
                (long long)num_tokens, (long long)Hkv, (long long)num_blocks, (long long)block_size);
  if (D != 64 && D != 128 && D != 256)
    return fail(FA_ERR_UNSUPPORTED, "head dim D=%lld not supported (64, 128 or 256)", (long long)D);
  if (block_size < 16 || block_size > 1024 || block_size % 16 != 0)
    return fail(FA_ERR_UNSUPPORTED, "block_size=%lld must be a multiple of 16 in [16, 1024]", (long long)block_size);
  FA_TRY(check_dtypes(dtype, dtype, false));
  if (num_tokens == 0 || Hkv == 0 || num_blocks == 0) return FA_OK;
  if (num_tokens * Hkv > kMaxI32 * 8) return fail(FA_ERR_UNSUPPORTED, "too many tokens");
  FA_TRY(check_ptr(key, "key"));
  FA_TRY(check_ptr(value, "value"));
  FA_TRY(check_ptr(k_cache, "k_cache"));
  FA_TRY(check_ptr(v_cache, "v_cache"));
  if (slot_mapping == nullptr || reinterpret_cast<uintptr_t>(slot_mapping) % 8 != 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "slot_mapping is NULL or not 8-byte aligned");
  fa::CacheArgs a{num_tokens, Hkv, D, block_size, num_blocks, key, value, slot_mapping, k_cache, v_cache, stream};
  return finish(fa::launch_reshape_and_cache(a), stream, "fa_reshape_and_cache launch");
}

size_t fa_paged_decode_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t D, int64_t max_context_len) {
  if (B <= 0 || H <= 0 || Hkv <= 0 || D <= 0) return 0;
  const int s = fa::decode_split(B, Hkv, max_context_len).n_splits;
  return s > 1 ? (size_t)(B * H * s * (D + 1)) * sizeof(float) : 0;
}

}  // extern "C"

namespace {

// The context split of one source: sized for its longest context (dense) or
// for topk pages (sparse).
fa::DecodeSplit source_split(const fa_kv_source& x, int64_t B, int64_t Hkv) {
  const int64_t longest = x.n_selected != nullptr ? x.topk * x.block_size : x.max_context_len;
  return fa::decode_split(B, Hkv, longest < 0 ? 0 : longest);
}

// Checks one KV source of a decode call and fills its kernel record (the
// split included).  A source with n_selected != NULL is sparse.
// With check_pointers false (an empty call) the pointers are not looked at.
int check_source(const fa_kv_source& x, int idx, int64_t B, int64_t Hkv, bool check_pointers,
                 fa::DecodeSource* out) {
  if (x.block_size < 0 || x.num_blocks < 0 || x.max_blocks_per_seq < 0 || x.max_context_len < 0 || x.topk < 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "source %d: negative size", idx);
  if (x.block_size < 16 || x.block_size > 1024 || x.block_size % 16 != 0)
    return fail(FA_ERR_UNSUPPORTED, "source %d: block_size=%lld must be a multiple of 16 in [16, 1024]", idx,
                (long long)x.block_size);
  if (x.max_blocks_per_seq > kMaxI32 || x.num_blocks > kMaxI32 || x.max_blocks_per_seq * x.block_size > kMaxI32 ||
      x.topk > kMaxI32 || B * Hkv * (x.topk > 0 ? x.topk : 1) > (int64_t)1 << 40)
    return fail(FA_ERR_UNSUPPORTED, "source %d: problem too large", idx);
  const bool sparse = x.n_selected != nullptr;
  if (!sparse && x.selected != nullptr)
    return fail(FA_ERR_INVALID_ARGUMENT, "source %d: selected given without n_selected", idx);
  if (!check_pointers) return FA_OK;
  if (reinterpret_cast<uintptr_t>(x.row_lens) % 4 != 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "source %d: row_lens not 4-byte aligned", idx);
  if (x.k_cache == nullptr || x.v_cache == nullptr || reinterpret_cast<uintptr_t>(x.k_cache) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(x.v_cache) % 16 != 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "source %d: k_cache / v_cache NULL or not 16-byte aligned", idx);
  if (x.block_tables == nullptr || x.context_lens == nullptr ||
      reinterpret_cast<uintptr_t>(x.block_tables) % 4 != 0 || reinterpret_cast<uintptr_t>(x.context_lens) % 4 != 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "source %d: block_tables / context_lens NULL or not 4-byte aligned", idx);
  if (sparse && ((x.selected == nullptr && x.topk > 0) || reinterpret_cast<uintptr_t>(x.selected) % 4 != 0 ||
                 reinterpret_cast<uintptr_t>(x.n_selected) % 4 != 0))
    return fail(FA_ERR_INVALID_ARGUMENT, "source %d: selected NULL with topk > 0, or not 4-byte aligned", idx);
  const fa::DecodeSplit split = source_split(x, B, Hkv);
  out->k_cache = x.k_cache;
  out->v_cache = x.v_cache;
  out->block_tables = x.block_tables;
  out->context_lens = x.context_lens;
  out->block_size = x.block_size;
  out->num_blocks = x.num_blocks;
  out->max_blocks = x.max_blocks_per_seq;
  // With topk == 0 no list entry is read (every count clamps to 0); the
  // kernel only needs a non-null list to take the sparse path.
  out->selected = sparse ? (x.selected != nullptr ? x.selected : x.n_selected) : nullptr;
  out->n_selected = sparse ? x.n_selected : nullptr;
  out->topk = sparse ? x.topk : 0;
  out->n_splits = split.n_splits;
  out->chunk = split.chunk;
  out->row_lens = x.row_lens;
  return FA_OK;
}

// Paged attention of Tq query tokens per sequence over one or two sources
// (Tq = 1: decode).
int paged_decode_impl(int64_t B, int64_t Tq, int64_t H, int64_t Hkv, int64_t D, int dtype, int o_dtype,
                      const void* q, int n_sources, const fa_kv_source* sources, void* o, float* lse, float scale,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_last_error.clear();
  if (B < 0 || Tq < 0 || H < 0 || Hkv < 0) return fail(FA_ERR_INVALID_ARGUMENT, "negative size");
  if (n_sources < 1 || n_sources > 2 || sources == nullptr)
    return fail(FA_ERR_INVALID_ARGUMENT, "n_sources=%d must be 1 or 2 with a sources array", n_sources);
  if (D != 64 && D != 128 && D != 256)
    return fail(FA_ERR_UNSUPPORTED, "head dim D=%lld not supported (64, 128 or 256)", (long long)D);
  FA_TRY(check_dtypes(dtype, o_dtype, true));
  FA_TRY(check_scale(scale, 0));
  if (H > 0 && (Hkv == 0 || H % Hkv != 0))
    return fail(FA_ERR_INVALID_ARGUMENT, "H=%lld query heads must be a whole multiple of Hkv=%lld", (long long)H,
                (long long)Hkv);
  fa::DecodeArgs a{};
  const bool empty = B == 0 || H == 0 || Tq == 0;
  for (int i = 0; i < n_sources; ++i) FA_TRY(check_source(sources[i], i, B, Hkv, !empty, &a.src[i]));
  if (empty) return FA_OK;
  const int64_t n_splits = a.src[0].n_splits + (n_sources > 1 ? a.src[1].n_splits : 0);
  if (Tq > kMaxI32 / H || B * Hkv * ((Tq * (H / Hkv) + 15) / 16) * n_splits > kMaxI32 ||
      B * Tq * H * n_splits * (D + 1) > ((int64_t)1 << 40))
    return fail(FA_ERR_UNSUPPORTED, "grid too large (B=%lld Tq=%lld Hkv=%lld H/Hkv=%lld)", (long long)B,
                (long long)Tq, (long long)Hkv, (long long)(H / Hkv));
  if (B * Tq * H > kMaxI32) return fail(FA_ERR_UNSUPPORTED, "problem too large");
  FA_TRY(check_ptr(q, "q"));
  FA_TRY(check_ptr(o, "o"));
  if (lse != nullptr && reinterpret_cast<uintptr_t>(lse) % 4 != 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "lse is not 4-byte aligned");
  const size_t need = n_splits > 1 ? (size_t)(B * Tq * H * n_splits * (D + 1)) * sizeof(float) : 0;
  if (need > 0) {
    if (workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
      return fail(FA_ERR_INVALID_ARGUMENT, "workspace is NULL or not 16-byte aligned");
    if (workspace_bytes < need)
      return fail(FA_ERR_INVALID_ARGUMENT, "workspace of %zu bytes is smaller than the %zu bytes needed",
                  workspace_bytes, need);
  }
  a.B = B; a.Tq = Tq; a.H = H; a.Hkv = Hkv; a.D = D; a.dtype = dtype; a.o_dtype = o_dtype; a.q = q;
  a.n_sources = n_sources; a.o = o; a.lse = lse; a.scale = scale; a.workspace = static_cast<float*>(workspace);
  a.stream = stream;
  return finish(fa::launch_paged_decode(a), stream, "fa_paged_decode launch");
}

// A single dense or sparse source from the arguments of the one-source calls.
fa_kv_source one_source(int64_t block_size, int64_t num_blocks, int64_t max_blocks_per_seq, int64_t max_context_len,
                        const void* k_cache, const void* v_cache, const int32_t* block_tables,
                        const int32_t* context_lens, const int32_t* selected, const int32_t* n_selected,
                        int64_t topk) {
  fa_kv_source x{};
  x.k_cache = k_cache;
  x.v_cache = v_cache;
  x.block_tables = block_tables;
  x.context_lens = context_lens;
  x.block_size = block_size;
  x.num_blocks = num_blocks;
  x.max_blocks_per_seq = max_blocks_per_seq;
  x.max_context_len = max_context_len;
  x.selected = selected;
  x.n_selected = n_selected;
  x.topk = topk;
  return x;
}

}  // namespace

extern "C" {

int fa_paged_decode(int64_t B, int64_t H, int64_t Hkv, int64_t D, int64_t block_size, int64_t num_blocks,
                    int64_t max_blocks_per_seq, int64_t max_context_len, int dtype, int o_dtype, const void* q,
                    const void* k_cache, const void* v_cache, const int32_t* block_tables,
                    const int32_t* context_lens, void* o, float* lse, float scale, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  const fa_kv_source x = one_source(block_size, num_blocks, max_blocks_per_seq, max_context_len, k_cache, v_cache,
                                    block_tables, context_lens, nullptr, nullptr, 0);
  return paged_decode_impl(B, 1, H, Hkv, D, dtype, o_dtype, q, 1, &x, o, lse, scale, workspace, workspace_bytes,
                           stream);
}

// The common checks of the page-selection calls.
static int check_quest(int64_t B, int64_t H, int64_t Hkv, int64_t D, int64_t block_size, int64_t num_blocks,
                       int64_t max_blocks_per_seq, int64_t topk, int dtype) {
  if (B < 0 || H < 0 || Hkv < 0 || num_blocks < 0 || block_size < 0 || max_blocks_per_seq < 0 || topk < 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "negative size");
  if (D != 64 && D != 128 && D != 256)
    return fail(FA_ERR_UNSUPPORTED, "head dim D=%lld not supported (64, 128 or 256)", (long long)D);
  if (block_size < 16 || block_size > 1024 || block_size % 16 != 0)
    return fail(FA_ERR_UNSUPPORTED, "block_size=%lld must be a multiple of 16 in [16, 1024]", (long long)block_size);
  FA_TRY(check_dtypes(dtype, dtype, false));
  if (H > 0 && (Hkv == 0 || H % Hkv != 0))
    return fail(FA_ERR_INVALID_ARGUMENT, "H=%lld query heads must be a whole multiple of Hkv=%lld", (long long)H,
                (long long)Hkv);
  if (max_blocks_per_seq > fa::kQuestMaxPages)
    return fail(FA_ERR_UNSUPPORTED, "at most %d pages per context (max_blocks_per_seq=%lld)", fa::kQuestMaxPages,
                (long long)max_blocks_per_seq);
  if (topk > kMaxI32) return fail(FA_ERR_UNSUPPORTED, "topk too large");
  if (B * Hkv > kMaxI32 || num_blocks > kMaxI32) return fail(FA_ERR_UNSUPPORTED, "problem too large");
  return FA_OK;
}

int fa_quest_page_minmax(int64_t B, int64_t Hkv, int64_t D, int64_t block_size, int64_t num_blocks,
                         int64_t max_blocks_per_seq, int dtype, const void* k_cache, const int32_t* block_tables,
                         const int32_t* context_lens, void* kmeta, hipStream_t stream) {
  g_last_error.clear();
  FA_TRY(check_quest(B, Hkv, Hkv, D, block_size, num_blocks, max_blocks_per_seq, 0, dtype));
  if (B == 0 || Hkv == 0 || max_blocks_per_seq == 0 || num_blocks == 0) return FA_OK;
  FA_TRY(check_ptr(k_cache, "k_cache"));
  FA_TRY(check_ptr(kmeta, "kmeta"));
  if (block_tables == nullptr || context_lens == nullptr ||
      reinterpret_cast<uintptr_t>(block_tables) % 4 != 0 || reinterpret_cast<uintptr_t>(context_lens) % 4 != 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "block_tables / context_lens NULL or not 4-byte aligned");
  fa::QuestArgs a{};
  a.B = B; a.Hkv = Hkv; a.H = Hkv; a.D = D; a.block_size = block_size; a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq; a.dtype = dtype; a.k_cache = k_cache; a.block_tables = block_tables;
  a.context_lens = context_lens; a.kmeta = kmeta; a.stream = stream;
  return finish(fa::launch_quest_minmax(a), stream, "fa_quest_page_minmax launch");
}

int fa_quest_select(int64_t B, int64_t H, int64_t Hkv, int64_t D, int64_t block_size, int64_t num_blocks,
                    int64_t max_blocks_per_seq, int64_t topk, int dtype, const void* q, const void* kmeta,
                    const int32_t* block_tables, const int32_t* context_lens, int32_t* selected,
                    int32_t* n_selected, hipStream_t stream) {
  g_last_error.clear();
  FA_TRY(check_quest(B, H, Hkv, D, block_size, num_blocks, max_blocks_per_seq, topk, dtype));
  if (B == 0 || H == 0) return FA_OK;
  FA_TRY(check_ptr(q, "q"));
  FA_TRY(check_ptr(kmeta, "kmeta"));
  if (block_tables == nullptr || context_lens == nullptr || (selected == nullptr && topk > 0) ||
      n_selected == nullptr || reinterpret_cast<uintptr_t>(block_tables) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(context_lens) % 4 != 0 || reinterpret_cast<uintptr_t>(selected) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(n_selected) % 4 != 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "an index array is NULL or not 4-byte aligned");
  fa::QuestArgs a{};
  a.B = B; a.H = H; a.Hkv = Hkv; a.D = D; a.block_size = block_size; a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq; a.topk = topk; a.dtype = dtype; a.q = q; a.block_tables = block_tables;
  a.context_lens = context_lens; a.kmeta = const_cast<void*>(kmeta); a.selected = selected;
  a.n_selected = n_selected; a.stream = stream;
  return finish(fa::launch_quest_select(a), stream, "fa_quest_select launch");
}

int fa_paged_decode_sparse(int64_t B, int64_t H, int64_t Hkv, int64_t D, int64_t block_size, int64_t num_blocks,
                           int64_t max_blocks_per_seq, int64_t topk, int dtype, int o_dtype, const void* q,
                           const void* k_cache, const void* v_cache, const int32_t* block_tables,
                           const int32_t* context_lens, const int32_t* selected, const int32_t* n_selected,
                           void* o, float* lse, float scale, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  g_last_error.clear();
  if (topk < 0) return fail(FA_ERR_INVALID_ARGUMENT, "negative topk");
  if (B > 0 && H > 0 && ((selected == nullptr && topk > 0) || n_selected == nullptr ||
                         reinterpret_cast<uintptr_t>(selected) % 4 != 0 ||
                         reinterpret_cast<uintptr_t>(n_selected) % 4 != 0))
    return fail(FA_ERR_INVALID_ARGUMENT, "selected / n_selected NULL or not 4-byte aligned");
  const fa_kv_source x = one_source(block_size, num_blocks, max_blocks_per_seq, 0, k_cache, v_cache, block_tables,
                                    context_lens, selected, n_selected, topk);
  return paged_decode_impl(B, 1, H, Hkv, D, dtype, o_dtype, q, 1, &x, o, lse, scale, workspace, workspace_bytes,
                           stream);
}

size_t fa_paged_attention_sources_workspace_bytes(int64_t B, int64_t Tq, int64_t H, int64_t Hkv, int64_t D,
                                                  int n_sources, const fa_kv_source* sources) {
  if (B <= 0 || Tq <= 0 || H <= 0 || Hkv <= 0 || D <= 0 || n_sources < 1 || n_sources > 2 || sources == nullptr)
    return 0;
  int64_t s = 0;
  for (int i = 0; i < n_sources; ++i) s += source_split(sources[i], B, Hkv).n_splits;
  return s > 1 ? (size_t)(B * Tq * H * s * (D + 1)) * sizeof(float) : 0;
}

int fa_paged_attention_sources(int64_t B, int64_t Tq, int64_t H, int64_t Hkv, int64_t D, int dtype, int o_dtype,
                               const void* q, int n_sources, const fa_kv_source* sources, void* o, float* lse,
                               float scale, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return paged_decode_impl(B, Tq, H, Hkv, D, dtype, o_dtype, q, n_sources, sources, o, lse, scale, workspace,
                           workspace_bytes, stream);
}

size_t fa_paged_decode_sources_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t D, int n_sources,
                                               const fa_kv_source* sources) {
  return fa_paged_attention_sources_workspace_bytes(B, 1, H, Hkv, D, n_sources, sources);
}

int fa_paged_decode_sources(int64_t B, int64_t H, int64_t Hkv, int64_t D, int dtype, int o_dtype, const void* q,
                            int n_sources, const fa_kv_source* sources, void* o, float* lse, float scale,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return paged_decode_impl(B, 1, H, Hkv, D, dtype, o_dtype, q, n_sources, sources, o, lse, scale, workspace,
                           workspace_bytes, stream);
}


int fa_device_info(int64_t D, int dtype, int* compute_units, int* dkdv_programs) {
  g_last_error.clear();
  FA_TRY(check_shape(Shape{1, 1, 1, D}));
  FA_TRY(check_dtypes(dtype, dtype, false));
  DeviceFacts* f = nullptr;
  FA_TRY(device_facts(&f));
  if (compute_units) *compute_units = f->cus;
  if (dkdv_programs) *dkdv_programs = f->cus * f->dkdv_per_cu[d_index(D)][dtype];
  return FA_OK;
}

int fa_dkdv_schedule(int64_t Z, int64_t H, int64_t N, int64_t D, int causal, int num_programs,
                     int64_t* units_per_program, int64_t* qtiles_per_program, int64_t* n_units) {
  g_last_error.clear();
  const Shape s{Z, H, N, D};
  FA_TRY(check_shape(s));
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1");
  if (num_programs <= 0) return fail(FA_ERR_INVALID_ARGUMENT, "num_programs must be > 0");
  const int64_t bk = fa::dkdv_keys((int)D), bq = fa::dkdv_queries((int)D);
  const int64_t ZH = s.heads();
  const int64_t n_kt = (N + bk - 1) / bk, n_qt = (N + bq - 1) / bq;
  const int64_t U = ZH * n_kt;
  if (n_units) *n_units = U;
  for (int64_t p = 0; p < num_programs; ++p) {
    int64_t units = 0, work = 0;
    int64_t head = 0, kt = 0;
    for (int64_t r = 0; fa::sched_unit(r, p, num_programs, ZH, n_kt, &head, &kt); ++r) {
      ++units;
      work += n_qt - fa::sched_first_qtile(kt, bk, bq, causal);
    }
    if (units_per_program) units_per_program[p] = units;
    if (qtiles_per_program) qtiles_per_program[p] = work;
  }
  return FA_OK;
}

int fa_fwd_tile_pairs(int64_t N, int64_t D, int causal, int64_t* visited, int64_t* total) {
  g_last_error.clear();
  FA_TRY(check_shape(Shape{1, 1, N, D}));
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1");
  const int64_t bm = fa::kFwdQueries, bn = fa::fwd_keys((int)D);
  const int64_t nq = (N + bm - 1) / bm, nk = (N + bn - 1) / bn;
  int64_t vis = 0;
  for (int64_t i = 0; i < nq; ++i) {
    const int64_t end = causal ? std::min(N, (i + 1) * bm) : N;
    vis += (end + bn - 1) / bn;
  }
  if (visited) *visited = vis;
  if (total) *total = nq * nk;
  return FA_OK;
}

}  // extern "C"
