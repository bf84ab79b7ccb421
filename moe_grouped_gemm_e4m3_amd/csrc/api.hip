// api.hip - the C ABI declared in include/dg.h: argument validation (before any HIP
// call), device check, schedule dispatch, status reporting.
#include <stdarg.h>
#include <stdlib.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "dg.h"
#include "dg_launch.h"

namespace {

thread_local char g_msg[512] = "";

dg_status_t fail(dg_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof g_msg, fmt, ap);
  va_end(ap);
  return st;
}

dg_status_t ok() {
  g_msg[0] = '\0';
  return DG_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kQ = 128;
constexpr int64_t kMaxDim = (int64_t)1 << 31;  // sizes stay below 2^31 per dimension

// Once per device: is it gfx950? Cached under a mutex (the only shared state).
dg_status_t check_device() {
  static std::mutex mu;
  static signed char cache[64];  // 0 unknown, 1 yes, -1 no
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(DG_ERR_UNSUPPORTED_DEVICE, "no HIP device is current");
  std::lock_guard<std::mutex> lock(mu);
  if (dev < 64 && cache[dev] != 0)
    return cache[dev] > 0 ? DG_OK : fail(DG_ERR_UNSUPPORTED_DEVICE, "device %d is not gfx950", dev);
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return fail(DG_ERR_UNSUPPORTED_DEVICE, "cannot query device %d", dev);
  const bool yes = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) cache[dev] = yes ? 1 : -1;
  return yes ? DG_OK : fail(DG_ERR_UNSUPPORTED_DEVICE, "device %d is %s, not gfx950", dev, prop.gcnArchName);
}

dg_status_t launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DG_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

dg_status_t check_nk(int64_t N, int64_t K) {
  if (N < 0 || K < 0) return fail(DG_ERR_INVALID_ARGUMENT, "negative size (N=%lld, K=%lld)", (long long)N, (long long)K);
  if (N % kQ != 0) return fail(DG_ERR_UNSUPPORTED_SHAPE, "N=%lld is not a multiple of 128", (long long)N);
  if (K % kQ != 0 || K == 0) return fail(DG_ERR_UNSUPPORTED_SHAPE, "K=%lld is not a positive multiple of 128", (long long)K);
  if (N >= kMaxDim || K >= kMaxDim) return fail(DG_ERR_UNSUPPORTED_SHAPE, "N or K >= 2^31");
  return DG_OK;
}

// Common part of the three GEMM entry points.
dg_status_t run_gemm(dg::Layout layout, int schedule, bool pow2, const uint8_t* a, const float* sfa, const uint8_t* b,
                     const float* sfb, const int32_t* meta, uint16_t* d, int64_t G, int64_t M, int64_t N,
                     int64_t K, int64_t expected_m, void* stream, const char* name) {
  if (M < 0 || G < 0) return fail(DG_ERR_INVALID_ARGUMENT, "%s: negative size", name);
  dg_status_t st = check_nk(N, K);
  if (st != DG_OK) return st;
  if (M >= kMaxDim || G >= kMaxDim) return fail(DG_ERR_UNSUPPORTED_SHAPE, "%s: M or G >= 2^31", name);
  if (layout == dg::Layout::Contiguous) {
    if (M % kQ != 0) return fail(DG_ERR_UNSUPPORTED_SHAPE, "%s: M_total=%lld is not a multiple of 128", name, (long long)M);
    if (G < 1) return fail(DG_ERR_INVALID_ARGUMENT, "%s: G must be >= 1", name);
  }
  if (schedule < 0 || schedule > 3) return fail(DG_ERR_INVALID_ARGUMENT, "%s: unknown schedule %d", name, schedule);
  if (M == 0 || N == 0 || G == 0) return ok();
  if (!a || !sfa || !b || !sfb || !d || (layout != dg::Layout::Dense && !meta))
    return fail(DG_ERR_INVALID_ARGUMENT, "%s: null pointer", name);
  if (!aligned16(a) || !aligned16(sfa) || !aligned16(b) || !aligned16(sfb) || !aligned16(d) ||
      (meta && !aligned16(meta)))
    return fail(DG_ERR_MISALIGNED, "%s: every pointer must be 16-byte aligned", name);
  st = check_device();
  if (st != DG_OK) return st;
  dg::GemmProblem p{};
  p.a = a; p.sfa = sfa; p.b = b; p.sfb = sfb; p.d = d;
  p.m_indices = layout == dg::Layout::Contiguous ? meta : nullptr;
  p.masked_m = layout == dg::Layout::Masked ? meta : nullptr;
  p.M = M; p.N = N; p.K = K; p.G = (int32_t)G; p.layout = layout; p.pow2 = pow2;
  const char* chosen = "";
  hipError_t e = dg::launch_gemm(p, static_cast<dg::Schedule>(schedule), expected_m,
                                 static_cast<hipStream_t>(stream), &chosen);
  if (dg::log_switch()) fprintf(stderr, "[dg] %s M=%lld N=%lld K=%lld G=%lld -> %s\n", name, (long long)M,
                                (long long)N, (long long)K, (long long)G, chosen);
  return launched(e, name);
}

dg_status_t run_cast(bool per_block, bool pow2, const void* x, dg_input_dtype_t dtype, int64_t groups, int64_t rows,
                     int64_t K, uint8_t* q, float* sf, void* stream, const int32_t* masked_m = nullptr,
                     const char* name = nullptr) {
  if (!name)
    name = per_block ? (pow2 ? "dg_cast_fp8_per_block_ue8m0" : "dg_cast_fp8_per_block")
                     : (pow2 ? "dg_cast_fp8_per_token_ue8m0" : "dg_cast_fp8_per_token");
  if (dtype != DG_INPUT_F32 && dtype != DG_INPUT_BF16) return fail(DG_ERR_INVALID_ARGUMENT, "%s: unknown dtype %d", name, (int)dtype);
  if (groups < 0 || rows < 0 || K < 0) return fail(DG_ERR_INVALID_ARGUMENT, "%s: negative size", name);
  if (K % kQ != 0) return fail(DG_ERR_UNSUPPORTED_SHAPE, "%s: K=%lld is not a multiple of 128", name, (long long)K);
  if (per_block && rows % kQ != 0) return fail(DG_ERR_UNSUPPORTED_SHAPE, "%s: N=%lld is not a multiple of 128", name, (long long)rows);
  if (groups >= kMaxDim || rows >= kMaxDim || K >= kMaxDim || (groups > 0 && rows >= kMaxDim / groups))
    return fail(DG_ERR_UNSUPPORTED_SHAPE, "%s: size >= 2^31", name);
  if (groups == 0 || rows == 0 || K == 0) return ok();
  if (!x || !q || !sf) return fail(DG_ERR_INVALID_ARGUMENT, "%s: null pointer", name);
  if (!aligned16(x) || !aligned16(q) || !aligned16(sf)) return fail(DG_ERR_MISALIGNED, "%s: every pointer must be 16-byte aligned", name);
  if (masked_m && !aligned16(masked_m)) return fail(DG_ERR_MISALIGNED, "%s: every pointer must be 16-byte aligned", name);
  dg_status_t st = check_device();
  if (st != DG_OK) return st;
  hipError_t e = per_block ? dg::launch_cast_per_block(x, dtype == DG_INPUT_BF16, pow2, rows, K, q, sf,
                                                       static_cast<hipStream_t>(stream))
                           : dg::launch_cast_per_token(x, dtype == DG_INPUT_BF16, pow2, groups, rows, K, masked_m, q, sf,
                                                       static_cast<hipStream_t>(stream));
  return launched(e, name);
}

// Common part of the SwiGLU GEMM and the expert FFN: every host-side argument check of the
// gate/up GEMM; then (unless validate_only) the device check and the launch.
dg_status_t run_swiglu(int32_t layout, int32_t scale_fmt, const uint8_t* a, const float* sfa, const uint8_t* b,
                       const float* sfb, const int32_t* meta, uint8_t* hq, float* sfh, int64_t G, int64_t M,
                       int64_t I, int64_t K, int64_t expected_m, void* stream, const char* name, bool validate_only) {
  if (layout < 0 || layout > 2) return fail(DG_ERR_INVALID_ARGUMENT, "%s: unknown layout %d", name, layout);
  if (scale_fmt != DG_SCALE_F32 && scale_fmt != DG_SCALE_UE8M0)
    return fail(DG_ERR_INVALID_ARGUMENT, "%s: unknown scale format %d", name, scale_fmt);
  const dg::Layout L = static_cast<dg::Layout>(layout);
  if (L == dg::Layout::Dense) G = 1;
  if (M < 0 || G < 0 || I < 0) return fail(DG_ERR_INVALID_ARGUMENT, "%s: negative size", name);
  dg_status_t st = check_nk(2 * I, K);
  if (st != DG_OK) return st;
  if (I % kQ != 0) return fail(DG_ERR_UNSUPPORTED_SHAPE, "%s: I=%lld is not a multiple of 128", name, (long long)I);
  if (M >= kMaxDim || G >= kMaxDim) return fail(DG_ERR_UNSUPPORTED_SHAPE, "%s: M or G >= 2^31", name);
  if (L == dg::Layout::Contiguous) {
    if (M % kQ != 0) return fail(DG_ERR_UNSUPPORTED_SHAPE, "%s: M_total=%lld is not a multiple of 128", name, (long long)M);
    if (G < 1) return fail(DG_ERR_INVALID_ARGUMENT, "%s: G must be >= 1", name);
  }
  // the fused kernel addresses one group's operands with 32-bit offsets and keeps a tile's
  // weight scales for every K block in LDS
  if (K / kQ > 256 || M * K >= ((int64_t)1 << 32) || 2 * I * K >= ((int64_t)1 << 32) ||
      M * (K / kQ) * 4 >= ((int64_t)1 << 32))
    return fail(DG_ERR_UNSUPPORTED_SHAPE, "%s: needs K <= 32768, M*K < 2^32 and 2*I*K < 2^32", name);
  if (M == 0 || I == 0 || G == 0) return ok();
  if (!a || !sfa || !b || !sfb || !hq || !sfh || (L != dg::Layout::Dense && !meta))
    return fail(DG_ERR_INVALID_ARGUMENT, "%s: null pointer", name);
  if (!aligned16(a) || !aligned16(sfa) || !aligned16(b) || !aligned16(sfb) || !aligned16(hq) || !aligned16(sfh) ||
      (L != dg::Layout::Dense && !aligned16(meta)))
    return fail(DG_ERR_MISALIGNED, "%s: every pointer must be 16-byte aligned", name);
  if (validate_only) return DG_OK;
  st = check_device();
  if (st != DG_OK) return st;
  dg::GemmProblem p{};
  p.a = a; p.sfa = sfa; p.b = b; p.sfb = sfb; p.d = nullptr;
  p.m_indices = L == dg::Layout::Contiguous ? meta : nullptr;
  p.masked_m = L == dg::Layout::Masked ? meta : nullptr;
  p.M = M; p.N = 2 * I; p.K = K; p.G = (int32_t)G; p.layout = L; p.pow2 = scale_fmt == DG_SCALE_UE8M0;
  const char* chosen = "";
  const hipError_t e = dg::launch_gemm_swiglu(p, hq, sfh, expected_m, static_cast<hipStream_t>(stream), &chosen);
  if (dg::log_switch()) fprintf(stderr, "[dg] %s M=%lld I=%lld K=%lld G=%lld -> %s\n", name, (long long)M,
                                (long long)I, (long long)K, (long long)G, chosen);
  if (e == hipErrorNotSupported) return fail(DG_ERR_UNSUPPORTED_SHAPE, "%s: shape out of the kernel's range", name);
  return launched(e, name);
}

// ---- static scratch for the entry point that allocates nothing ------------------------
// The FP8 activation between the FFN's two GEMMs (hq, then its scales sfh) lives in this
// file-scope device array for callers that cannot allocate. Each GPU the library runs on
// holds its own copy until the process ends. In host code `scratch` only names the array: its
// device address on the current GPU comes from hipGetSymbolAddress, once per device, and only
// that address is ever handed to a kernel.
constexpr int64_t kScratchBytes = (int64_t)32 << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of the current device's copy of `scratch` (looked up on the first call on
// that device, under a mutex, and kept); nullptr with the error in *err on failure.
uint8_t* scratch_address(hipError_t* err) {
  static std::mutex mu;
  static uint8_t* addr[64];
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= 64) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    addr[dev] = static_cast<uint8_t*>(p);
  }
  *err = hipSuccess;
  return addr[dev];
}

// Bytes of hq (rounded up to 256) and of sfh for an FFN call of `rows` rows.
int64_t ffn_hq_bytes(int64_t rows, int64_t I) { return (rows * I + 255) / 256 * 256; }
int64_t ffn_sfh_bytes(int64_t rows, int64_t I) { return 4 * rows * (I / kQ); }

}  // namespace

extern "C" {

dg_status_t dg_cast_fp8_per_token(const void* x, dg_input_dtype_t x_dtype, int64_t G, int64_t M, int64_t K,
                                  uint8_t* q, float* sf, void* stream) {
  return run_cast(false, false, x, x_dtype, G, M, K, q, sf, stream);
}

dg_status_t dg_cast_fp8_per_block(const void* w, dg_input_dtype_t w_dtype, int64_t N, int64_t K, uint8_t* q,
                                  float* sf, void* stream) {
  return run_cast(true, false, w, w_dtype, 1, N, K, q, sf, stream);
}

dg_status_t dg_cast_fp8_per_token_ue8m0(const void* x, dg_input_dtype_t x_dtype, int64_t G, int64_t M, int64_t K,
                                        uint8_t* q, float* sf, void* stream) {
  return run_cast(false, true, x, x_dtype, G, M, K, q, sf, stream);
}

dg_status_t dg_cast_fp8_per_block_ue8m0(const void* w, dg_input_dtype_t w_dtype, int64_t N, int64_t K, uint8_t* q,
                                        float* sf, void* stream) {
  return run_cast(true, true, w, w_dtype, 1, N, K, q, sf, stream);
}

dg_status_t dg_cast_fp8_per_token_masked(const void* x, dg_input_dtype_t x_dtype, int32_t scale_fmt, int32_t G,
                                         int64_t M_max, int64_t K, const int32_t* masked_m, uint8_t* q, float* sf,
                                         void* stream) {
  const char* name = "dg_cast_fp8_per_token_masked";
  if (scale_fmt != DG_SCALE_F32 && scale_fmt != DG_SCALE_UE8M0)
    return fail(DG_ERR_INVALID_ARGUMENT, "%s: unknown scale format %d", name, scale_fmt);
  if (G > 0 && M_max > 0 && K > 0 && !masked_m) return fail(DG_ERR_INVALID_ARGUMENT, "%s: null pointer", name);
  return run_cast(false, scale_fmt == DG_SCALE_UE8M0, x, x_dtype, G, M_max, K, q, sf, stream, masked_m, name);
}

dg_status_t dg_gemm_fp8_nt(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb, uint16_t* d,
                           int64_t M, int64_t N, int64_t K, void* stream) {
  return run_gemm(dg::Layout::Dense, 0, false, a, sfa, b, sfb, nullptr, d, 1, M, N, K, 0, stream, "dg_gemm_fp8_nt");
}

dg_status_t dg_grouped_gemm_contiguous(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                                       const int32_t* m_indices, uint16_t* d, int32_t G, int64_t M_total,
                                       int64_t N, int64_t K, void* stream) {
  return run_gemm(dg::Layout::Contiguous, 0, false, a, sfa, b, sfb, m_indices, d, G, M_total, N, K, 0, stream,
                  "dg_grouped_gemm_contiguous");
}

dg_status_t dg_grouped_gemm_masked(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                                   const int32_t* masked_m, uint16_t* d, int32_t G, int64_t M_max, int64_t N,
                                   int64_t K, int64_t expected_m, void* stream) {
  return run_gemm(dg::Layout::Masked, 0, false, a, sfa, b, sfb, masked_m, d, G, M_max, N, K, expected_m, stream,
                  "dg_grouped_gemm_masked");
}

dg_status_t dg_gemm_fp8_nt_ue8m0(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb, uint16_t* d,
                                 int64_t M, int64_t N, int64_t K, void* stream) {
  return run_gemm(dg::Layout::Dense, 0, true, a, sfa, b, sfb, nullptr, d, 1, M, N, K, 0, stream,
                  "dg_gemm_fp8_nt_ue8m0");
}

dg_status_t dg_grouped_gemm_contiguous_ue8m0(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                                             const int32_t* m_indices, uint16_t* d, int32_t G, int64_t M_total,
                                             int64_t N, int64_t K, void* stream) {
  return run_gemm(dg::Layout::Contiguous, 0, true, a, sfa, b, sfb, m_indices, d, G, M_total, N, K, 0, stream,
                  "dg_grouped_gemm_contiguous_ue8m0");
}

dg_status_t dg_grouped_gemm_masked_ue8m0(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                                         const int32_t* masked_m, uint16_t* d, int32_t G, int64_t M_max, int64_t N,
                                         int64_t K, int64_t expected_m, void* stream) {
  return run_gemm(dg::Layout::Masked, 0, true, a, sfa, b, sfb, masked_m, d, G, M_max, N, K, expected_m, stream,
                  "dg_grouped_gemm_masked_ue8m0");
}

dg_status_t dg_gemm_fp8_scheduled(int32_t layout, int32_t schedule, int32_t scale_fmt, const uint8_t* a,
                                  const float* sfa, const uint8_t* b, const float* sfb, const int32_t* meta,
                                  uint16_t* d, int32_t G, int64_t M, int64_t N, int64_t K, int64_t expected_m,
                                  void* stream) {
  if (layout < 0 || layout > 2) return fail(DG_ERR_INVALID_ARGUMENT, "dg_gemm_fp8_scheduled: unknown layout %d", layout);
  if (scale_fmt != DG_SCALE_F32 && scale_fmt != DG_SCALE_UE8M0)
    return fail(DG_ERR_INVALID_ARGUMENT, "dg_gemm_fp8_scheduled: unknown scale format %d", scale_fmt);
  const dg::Layout L = static_cast<dg::Layout>(layout);
  return run_gemm(L, schedule, scale_fmt == DG_SCALE_UE8M0, a, sfa, b, sfb, L == dg::Layout::Dense ? nullptr : meta, d,
                  L == dg::Layout::Dense ? 1 : G, M, N, K, expected_m, stream, "dg_gemm_fp8_scheduled");
}

dg_status_t dg_gemm_fp8_swiglu(int32_t layout, int32_t scale_fmt, const uint8_t* a, const float* sfa, const uint8_t* b,
                               const float* sfb, const int32_t* meta, uint8_t* hq, float* sfh, int32_t G, int64_t M,
                               int64_t I, int64_t K, int64_t expected_m, void* stream) {
  return run_swiglu(layout, scale_fmt, a, sfa, b, sfb, meta, hq, sfh, G, M, I, K, expected_m, stream,
                    "dg_gemm_fp8_swiglu", false);
}

dg_status_t dg_moe_ffn_fp8(int32_t layout, int32_t scale_fmt, const uint8_t* x, const float* sfx, const uint8_t* w1,
                           const float* sfw1, const uint8_t* w2, const float* sfw2, const int32_t* meta, uint8_t* hq,
                           float* sfh, uint16_t* y, int32_t G, int64_t M, int64_t H, int64_t I, int64_t expected_m,
                           void* stream) {
  const char* name = "dg_moe_ffn_fp8";
  // validate both GEMMs before launching either
  dg_status_t st = run_swiglu(layout, scale_fmt, x, sfx, w1, sfw1, meta, hq, sfh, G, M, I, H, expected_m, stream, name,
                              true);
  if (st != DG_OK) return st;
  if (M == 0 || I == 0 || (layout != 0 && G == 0)) return ok();
  if (!w2 || !sfw2 || !y) return fail(DG_ERR_INVALID_ARGUMENT, "%s: null pointer", name);
  if (!aligned16(w2) || !aligned16(sfw2) || !aligned16(y))
    return fail(DG_ERR_MISALIGNED, "%s: every pointer must be 16-byte aligned", name);
  st = run_swiglu(layout, scale_fmt, x, sfx, w1, sfw1, meta, hq, sfh, G, M, I, H, expected_m, stream, name, false);
  if (st != DG_OK) return st;
  const dg::Layout L = static_cast<dg::Layout>(layout);
  return run_gemm(L, 0, scale_fmt == DG_SCALE_UE8M0, hq, sfh, w2, sfw2, L == dg::Layout::Dense ? nullptr : meta, y,
                  L == dg::Layout::Dense ? 1 : G, M, H, I, expected_m, stream, name);
}

dg_status_t dg_convert_fp8_e4m3(const float* x, int64_t n, uint8_t* q, void* stream) {
  const char* name = "dg_convert_fp8_e4m3";
  if (n < 0) return fail(DG_ERR_INVALID_ARGUMENT, "%s: negative size", name);
  if (n % 4 != 0) return fail(DG_ERR_UNSUPPORTED_SHAPE, "%s: n=%lld is not a multiple of 4", name, (long long)n);
  if (n == 0) return ok();
  if (!x || !q) return fail(DG_ERR_INVALID_ARGUMENT, "%s: null pointer", name);
  if (!aligned16(x) || !aligned16(q)) return fail(DG_ERR_MISALIGNED, "%s: every pointer must be 16-byte aligned", name);
  const dg_status_t st = check_device();
  if (st != DG_OK) return st;
  return launched(dg::launch_convert_e4m3(x, q, n, static_cast<hipStream_t>(stream)), name);
}

dg_status_t dg_moe_ffn_fp8_noalloc(int32_t layout, int32_t scale_fmt, const uint8_t* x, const float* sfx,
                                   const uint8_t* w1, const float* sfw1, const uint8_t* w2, const float* sfw2,
                                   const int32_t* meta, uint16_t* y, int32_t G, int64_t M, int64_t H, int64_t I,
                                   int64_t expected_m, void* stream) {
  const char* name = "dg_moe_ffn_fp8_noalloc";
  // every host-side check of dg_moe_ffn_fp8 first, with stand-in (aligned, never used)
  // workspace pointers: the scratch size check and all argument errors need no device
  uint8_t* const hq_stub = reinterpret_cast<uint8_t*>(256);
  float* const sfh_stub = reinterpret_cast<float*>(512);
  dg_status_t st = run_swiglu(layout, scale_fmt, x, sfx, w1, sfw1, meta, hq_stub, sfh_stub, G, M, I, H, expected_m,
                              stream, name, true);
  if (st != DG_OK) return st;
  if (M == 0 || I == 0 || (layout != 0 && G == 0)) return ok();
  if (!w2 || !sfw2 || !y) return fail(DG_ERR_INVALID_ARGUMENT, "%s: null pointer", name);
  if (!aligned16(w2) || !aligned16(sfw2) || !aligned16(y))
    return fail(DG_ERR_MISALIGNED, "%s: every pointer must be 16-byte aligned", name);
  const int64_t rows = layout == 2 ? (int64_t)G * M : M;
  const int64_t need = ffn_hq_bytes(rows, I) + ffn_sfh_bytes(rows, I);
  if (need > kScratchBytes)
    return fail(DG_ERR_UNSUPPORTED_SHAPE, "%s: the FP8 activation needs %lld bytes, above the %lld-byte static scratch",
                name, (long long)need, (long long)kScratchBytes);
  st = check_device();
  if (st != DG_OK) return st;
  hipError_t e = hipSuccess;
  uint8_t* base = scratch_address(&e);
  if (base == nullptr) return fail(DG_ERR_LAUNCH, "%s: scratch address: %s", name, hipGetErrorString(e));
  uint8_t* hq = base;
  float* sfh = reinterpret_cast<float*>(base + ffn_hq_bytes(rows, I));
  st = run_swiglu(layout, scale_fmt, x, sfx, w1, sfw1, meta, hq, sfh, G, M, I, H, expected_m, stream, name, false);
  if (st != DG_OK) return st;
  const dg::Layout L = static_cast<dg::Layout>(layout);
  return run_gemm(L, 0, scale_fmt == DG_SCALE_UE8M0, hq, sfh, w2, sfw2, L == dg::Layout::Dense ? nullptr : meta, y,
                  L == dg::Layout::Dense ? 1 : G, M, H, I, expected_m, stream, name);
}

void dg_reload_tuning_switches(void) { dg::reload_tuning_switches(); }

const char* dg_status_string(dg_status_t status) {
  switch (status) {
    case DG_OK: return "DG_OK";
    case DG_ERR_INVALID_ARGUMENT: return "DG_ERR_INVALID_ARGUMENT";
    case DG_ERR_UNSUPPORTED_SHAPE: return "DG_ERR_UNSUPPORTED_SHAPE";
    case DG_ERR_MISALIGNED: return "DG_ERR_MISALIGNED";
    case DG_ERR_UNSUPPORTED_DEVICE: return "DG_ERR_UNSUPPORTED_DEVICE";
    case DG_ERR_LAUNCH: return "DG_ERR_LAUNCH";
  }
  return "DG_ERR_UNKNOWN";
}

const char* dg_last_error_message(void) { return g_msg; }

}  // extern "C"
