// dg_launch.h - internal interface between the C-ABI layer (api.hip) and the kernel
// translation units. Host-side only; no HIP types beyond hipStream_t / hipError_t.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

// Which operand layout a GEMM launch serves.
enum class Layout : int { Dense = 0, Contiguous = 1, Masked = 2 };

// One GEMM problem as the kernels see it. For Dense, G = 1. For Contiguous, rows of a/d
// are M_total = M and b/sfb are [G,N,K] / [G,N/128,K/128]. For Masked, a/sfa/d hold G
// groups of M rows each (M = M_max).
struct GemmProblem {
  const uint8_t* a;
  const float* sfa;
  const uint8_t* b;
  const float* sfb;
  uint16_t* d;
  const int32_t* m_indices;  // Contiguous only
  const int32_t* masked_m;   // Masked only
  int64_t M, N, K;
  int32_t G;
  Layout layout;
  bool pow2;  // every sfa / sfb value is a power of two (UE8M0 scales)
};

// Kernel schedules. Decode: 64-row M blocks, K split across the waves of a workgroup,
// operands streamed straight into registers. Tile: LDS-staged, double-buffered tiles.
// Tile64 (chosen internally for dense M <= 64, never passed in through the C ABI): 64x128
// direct-load tiles.
enum class Schedule : int { Auto = 0, Decode = 1, Tile128 = 2, Tile256 = 3, Tile64 = 4 };

hipError_t launch_gemm(const GemmProblem& p, Schedule s, int64_t expected_m, hipStream_t stream,
                       const char** chosen);

// Gate/up GEMM with the SwiGLU + per-token FP8 cast epilogue: p.b holds 2I = p.N rows per
// group (gate rows, then up rows); writes hq [rows, I] e4m3 and sh [I/128][rows] (per group
// for the masked layout). hipErrorNotSupported (before any launch) when the shape is out of
// the kernel's range.
hipError_t launch_gemm_swiglu(const GemmProblem& p, uint8_t* hq, float* sh, int64_t expected_m, hipStream_t stream,
                              const char** chosen);

// Per-token cast of G groups of M rows; masked_m (or nullptr): only rows r < masked_m[g] of
// group g are cast, the others left unwritten.
hipError_t launch_cast_per_token(const void* x, int bf16, int pow2, int64_t G, int64_t M, int64_t K,
                                 const int32_t* masked_m, uint8_t* q, float* sf, hipStream_t stream);
// x [n] fp32 -> q [n] e4m3 with the hardware conversion (n % 4 == 0, n > 0).
hipError_t launch_convert_e4m3(const float* x, uint8_t* q, int64_t n, hipStream_t stream);
hipError_t launch_cast_per_block(const void* w, int bf16, int pow2, int64_t N, int64_t K, uint8_t* q, float* sf,
                                 hipStream_t stream);

// The DG_* tuning switches (DG_TILE, DG_DECODE, DG_DECODE2, DG_DECODE3, DG_LOG) are read
// from the environment once per process; this reads them again.
void reload_tuning_switches();
// DG_LOG is set: every call names its chosen kernel on stderr.
bool log_switch();

}  // namespace dg
