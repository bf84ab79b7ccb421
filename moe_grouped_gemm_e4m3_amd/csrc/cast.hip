// cast.hip - FP8 e4m3 casts for gfx950: per-token (1x128) activation scales and
// 128x128 weight-block scales.
//
// Rule (DeepSeek-V3 repo review, "Innovations" 4: one scale per 128 elements;
// "Risks" 6: bound 448; DeepGEMM article, "FP8 and fine-grained scaling"):
//   s = amax / 448, q = e4m3(x / s), both divisions correctly rounded fp32; round to
//   nearest even with saturation; s == 0 gives signed zeros.
// Power-of-two (UE8M0) variant (DeepSeek-V3 repo review, "Innovations" item 4: V3.1 rounds
// the scales to powers of two so that scaling is a shift): s is the smallest power of two
// not below amax / 448, and at least 2^-126; x / s is then exact.
// Both kernels stream HBM: 4 B (fp32) or 2 B (bf16) read and ~1.03 B written per element.
#include "dg_device.h"
#include "dg_launch.h"

namespace dg {
namespace {

template <bool kBf16>
__device__ __forceinline__ void load4(const void* base, int64_t elem, float v[4]) {
  if constexpr (kBf16) {
    uint2 raw = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + elem);
    v[0] = bf16_to_f32(raw.x & 0xFFFFu);
    v[1] = bf16_to_f32(raw.x >> 16);
    v[2] = bf16_to_f32(raw.y & 0xFFFFu);
    v[3] = bf16_to_f32(raw.y >> 16);
  } else {
    float4 raw = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
    v[0] = raw.x; v[1] = raw.y; v[2] = raw.z; v[3] = raw.w;
  }
}

__device__ __forceinline__ uint32_t quant4(const float v[4], float s) {
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t code = (s == 0.0f) ? ((__float_as_uint(v[i]) >> 24) & 0x80u) : e4m3_encode(v[i] / s);
    packed |= code << (8 * i);
  }
  return packed;
}

// The codes of one chunk from its scale: q = e4m3(x / s) with the division correctly rounded
// and the hardware conversion, which equals the saturating encoder for every |x / s| <= 464
// (checked on every fp32 value). With s = fp32(amax / 448) >= amax / 448 * (1 - 2^-24), every
// quotient is at most 448.00003; power-of-two scales are >= amax / 448. s == 0 (an all-zero
// chunk, or amax / 448 underflowing) gives signed zeros.
__device__ __forceinline__ uint32_t quant4_hw(const float v[4], float s) {
  const uint32_t signs = ((__float_as_uint(v[0]) >> 31) << 7) | ((__float_as_uint(v[1]) >> 31) << 15) |
                         ((__float_as_uint(v[2]) >> 31) << 23) | ((__float_as_uint(v[3]) >> 31) << 31);
  const uint32_t codes = e4m3_hw_pack4(v[0] / s, v[1] / s, v[2] / s, v[3] / s);
  return s == 0.0f ? signs : codes;
}

// Masked layout helpers: the clamped counts min(max(masked_m[g], 0), M), 64 groups at a time
// (lane i holds group c + i), with an inclusive prefix sum over the wave. Wave-uniform results.
__device__ __forceinline__ int masked_count(const int32_t* __restrict__ masked_m, int G, int M, int g) {
  return g < G ? min(max(masked_m[g], 0), M) : 0;
}
__device__ __forceinline__ int wave_inclusive_sum(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  return v;
}
// Total valid rows over all groups.
__device__ __forceinline__ int64_t masked_valid_rows(const int32_t* __restrict__ masked_m, int G, int M) {
  const int lane = threadIdx.x & 63;
  int64_t total = 0;
  for (int c = 0; c < G; c += 64) total += __shfl(wave_inclusive_sum(masked_count(masked_m, G, M, c + lane)), 63, 64);
  return total;
}
// Group g and row r of valid row vr (0 <= vr < total): the groups' valid rows in order.
__device__ __forceinline__ void masked_valid_row(const int32_t* __restrict__ masked_m, int G, int M, int64_t vr,
                                                 int& g, int& r) {
  const int lane = threadIdx.x & 63;
  int64_t base = 0;  // valid rows of the groups before chunk c
  for (int c = 0; c < G; c += 64) {
    const int m = masked_count(masked_m, G, M, c + lane);
    const int incl = wave_inclusive_sum(m);
    const int chunk = __shfl(incl, 63, 64);
    if (vr < base + chunk) {
      // the groups whose inclusive prefix is <= vr lie wholly before vr's group
      const int k = __popcll(__ballot(base + incl <= vr));
      g = c + k;
      r = (int)(vr - base - (__shfl(incl, k, 64) - __shfl(m, k, 64)));
      return;
    }
    base += chunk;
  }
  g = G - 1;  // not reached for vr < total
  r = 0;
}

// One wave per unit: a row (over the G*M rows) and a run of up to 2*P of its K blocks. Lanes
// 0-31 take the even chunk of each pair, lanes 32-63 the odd one, 4 elements per lane, so a
// load instruction covers 1 KB of contiguous input (fp32) and a unit's P loads are all issued
// before its first reduction. The row's group, row and chunk offsets are computed once per
// unit (integer divisions cost tens of VALU instructions, and this kernel is VALU-bound
// otherwise). Units walk grid-stride; Idx is uint32_t when unit numbers stay below 2^32.
// masked_m (masked layout, else nullptr): only rows r < masked_m[g] (clamped to [0, M]) of
// group g are cast. Units then run over the valid rows alone, numbered group by group, so
// the waves stay evenly loaded whatever the counts; masked_valid_row maps a valid row back to
// its group and row.
template <bool kBf16, bool kPow2, typename Idx, int P>
__global__ __launch_bounds__(256) void cast_per_token_kernel(const void* __restrict__ x, Idx nunits, Idx nseg,
                                                             Idx M, Idx kblocks, const int32_t* __restrict__ masked_m,
                                                             int G, uint8_t* __restrict__ q, float* __restrict__ sf) {
  const int lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
  const Idx wave = (Idx)blockIdx.x * 4 + (Idx)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const Idx nwaves = (Idx)gridDim.x * 4;
  Idx total = nunits;
  if (masked_m != nullptr) total = (Idx)masked_valid_rows(masked_m, G, (int)M) * nseg;
  for (Idx u = wave; u < total; u += nwaves) {
    Idx gr, seg, g, r;
    if (masked_m != nullptr) {
      const Idx vr = u / nseg;
      seg = u - vr * nseg;
      int gg, rr;
      masked_valid_row(masked_m, G, (int)M, (int64_t)vr, gg, rr);
      g = (Idx)gg;
      r = (Idx)rr;
      gr = g * M + r;
    } else {
      gr = u / nseg;
      seg = u - gr * nseg;
      g = gr / M;
      r = gr - g * M;
    }
    const int kb0 = (int)(seg * (Idx)(2 * P));
    const int nk = min(2 * P, (int)kblocks - kb0);  // chunks of this unit
    const int64_t e0 = ((int64_t)gr * (int64_t)kblocks + kb0 + half) * kQ + l32 * 4;
    float v[P][4];
#pragma unroll
    for (int i = 0; i < P; ++i) {
      v[i][0] = v[i][1] = v[i][2] = v[i][3] = 0.0f;
      if (2 * i + half < nk) load4<kBf16>(x, e0 + (int64_t)(2 * i) * kQ, v[i]);
    }
    float* srow = sf + ((int64_t)g * (int64_t)kblocks + kb0 + half) * (int64_t)M + r;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      if (2 * i >= nk) break;  // wave-uniform
      float amax = fmaxf(fmaxf(fabsf(v[i][0]), fabsf(v[i][1])), fmaxf(fabsf(v[i][2]), fabsf(v[i][3])));
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 32));
      const float s = kPow2 ? pow2_ceil(amax / 448.0f) : amax / 448.0f;
      const uint32_t packed = quant4_hw(v[i], s);
      if (2 * i + half < nk) {
        *reinterpret_cast<uint32_t*>(q + e0 + (int64_t)(2 * i) * kQ) = packed;
        if (l32 == 0) srow[(int64_t)(2 * i) * (int64_t)M] = s;
      }
    }
  }
}

// One 256-thread block per 128x128 block. Thread t covers rows t/32 + 8*u (u = 0..15),
// columns 4*(t%32) .. +3, so every pass of 256 threads reads 8 full 512-byte rows.
template <bool kBf16, bool kPow2>
__global__ __launch_bounds__(256) void cast_per_block_kernel(const void* __restrict__ w,
                                                             int64_t K, int64_t kblocks,
                                                             uint8_t* __restrict__ q,
                                                             float* __restrict__ sf) {
  __shared__ float wave_max[4];
  const int64_t bn = blockIdx.x, bk = blockIdx.y;
  const int t = threadIdx.x;
  const int64_t col = bk * kQ + 4 * (t & 31);
  float v[16][4];
  float amax = 0.0f;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int64_t row = bn * kQ + (t >> 5) + 8 * u;
    load4<kBf16>(w, row * K + col, v[u]);
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[u][0]), fabsf(v[u][1])),
                             fmaxf(fabsf(v[u][2]), fabsf(v[u][3]))));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if ((t & 63) == 0) wave_max[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
  const float s = kPow2 ? pow2_ceil(amax / 448.0f) : amax / 448.0f;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int64_t row = bn * kQ + (t >> 5) + 8 * u;
    *reinterpret_cast<uint32_t*>(q + row * K + col) = quant4(v[u], s);
  }
  if (t == 0) sf[bn * kblocks + bk] = s;
}

// Plain conversion of fp32 values (already divided by their scale) with the hardware
// conversion of the fused SwiGLU epilogue: 4 values per thread, grid-stride.
__global__ __launch_bounds__(256) void convert_e4m3_kernel(const float4* __restrict__ x, uint32_t* __restrict__ q,
                                                           int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const float4 v = x[i];
    q[i] = e4m3_hw_pack4(v.x, v.y, v.z, v.w);
  }
}

template <bool kPow2, typename Idx, int P>
void launch_per_token(const void* x, int bf16, int64_t rows, int64_t M, int64_t kblocks, const int32_t* masked_m,
                      uint8_t* q, float* sf, hipStream_t stream) {
  const int64_t G = rows / M;
  // grid-stride beyond ~32 blocks per CU; the masked layout's valid rows at ~16 (measured on
  // 32 x 256 x 7168 with half the rows valid: 33 us at 4096 blocks, 35 us at 8192)
  const int64_t kMaxBlocks = masked_m ? 4096 : 8192;
  const int64_t nseg = (kblocks + 2 * P - 1) / (2 * P);
  const int64_t nunits = rows * nseg;
  int64_t blocks = (nunits + 3) / 4;
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  const dim3 grid((unsigned)blocks), block(256);
  if (bf16)
    cast_per_token_kernel<true, kPow2, Idx, P><<<grid, block, 0, stream>>>(x, (Idx)nunits, (Idx)nseg, (Idx)M,
                                                                            (Idx)kblocks, masked_m, (int)G, q, sf);
  else
    cast_per_token_kernel<false, kPow2, Idx, P><<<grid, block, 0, stream>>>(x, (Idx)nunits, (Idx)nseg, (Idx)M,
                                                                             (Idx)kblocks, masked_m, (int)G, q, sf);
}

template <bool kPow2>
hipError_t cast_per_token(const void* x, int bf16, int64_t G, int64_t M, int64_t K, const int32_t* masked_m,
                          uint8_t* q, float* sf, hipStream_t stream) {
  const int64_t kblocks = K / kQ;
  const int64_t rows = G * M;
  // runs of 8 K blocks per wave once that still gives every CU about 32 waves; pairs keep
  // small casts spread over more of the chip
  const bool wide = rows * ((kblocks + 7) / 8) >= 256 * 32;
  const bool small_idx = rows * kblocks < ((int64_t)1 << 32) - 4 * 8192 * 8;  // u + one stride < 2^32
  if (small_idx) {
    if (wide) launch_per_token<kPow2, uint32_t, 4>(x, bf16, rows, M, kblocks, masked_m, q, sf, stream);
    else launch_per_token<kPow2, uint32_t, 1>(x, bf16, rows, M, kblocks, masked_m, q, sf, stream);
  } else {
    launch_per_token<kPow2, int64_t, 4>(x, bf16, rows, M, kblocks, masked_m, q, sf, stream);
  }
  return hipGetLastError();
}

template <bool kPow2>
hipError_t cast_per_block(const void* w, int bf16, int64_t N, int64_t K, uint8_t* q, float* sf, hipStream_t stream) {
  const dim3 grid((unsigned)(N / kQ), (unsigned)(K / kQ));
  if (bf16)
    cast_per_block_kernel<true, kPow2><<<grid, dim3(256), 0, stream>>>(w, K, K / kQ, q, sf);
  else
    cast_per_block_kernel<false, kPow2><<<grid, dim3(256), 0, stream>>>(w, K, K / kQ, q, sf);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_cast_per_token(const void* x, int bf16, int pow2, int64_t G, int64_t M, int64_t K,
                                 const int32_t* masked_m, uint8_t* q, float* sf, hipStream_t stream) {
  return pow2 ? cast_per_token<true>(x, bf16, G, M, K, masked_m, q, sf, stream)
              : cast_per_token<false>(x, bf16, G, M, K, masked_m, q, sf, stream);
}

hipError_t launch_convert_e4m3(const float* x, uint8_t* q, int64_t n, hipStream_t stream) {
  const int64_t n4 = n / 4;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  convert_e4m3_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(reinterpret_cast<const float4*>(x),
                                                                         reinterpret_cast<uint32_t*>(q), n4);
  return hipGetLastError();
}

hipError_t launch_cast_per_block(const void* w, int bf16, int pow2, int64_t N, int64_t K, uint8_t* q,
                                 float* sf, hipStream_t stream) {
  return pow2 ? cast_per_block<true>(w, bf16, N, K, q, sf, stream) : cast_per_block<false>(w, bf16, N, K, q, sf, stream);
}

}  // namespace dg
