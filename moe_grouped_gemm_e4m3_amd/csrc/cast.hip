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

// 32 lanes per 128-element chunk, 4 elements per lane; a 256-thread block covers 8
// chunks per pass and walks the chunks grid-stride. Chunks are numbered in input order
// (K block fastest), so the 8 chunks of a pass are 4 KB (fp32) of contiguous input; each
// scale goes to its place in the K-block-major tensor [G][K/128][M]. Idx is uint32_t when
// the chunk count fits.
template <bool kBf16, bool kPow2, typename Idx>
__global__ __launch_bounds__(256) void cast_per_token_kernel(const void* __restrict__ x, Idx nchunks,
                                                             Idx M, Idx kblocks, uint8_t* __restrict__ q,
                                                             float* __restrict__ sf) {
  const int lane = threadIdx.x & 31;
  const int64_t K = (int64_t)kblocks * kQ;
  for (Idx c = (Idx)blockIdx.x * 8 + (Idx)(threadIdx.x >> 5); c < nchunks; c += (Idx)gridDim.x * 8) {
    // chunk c in input order: row-major over (group, row), K block fastest
    const Idx gr = c / kblocks, kb = c - gr * kblocks;
    const Idx g = gr / M, r = gr - g * M;
    const int64_t e0 = (int64_t)c * kQ + lane * 4;
    float v[4];
    load4<kBf16>(x, e0, v);
    float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 32));
    const float s = kPow2 ? pow2_ceil(amax / 448.0f) : amax / 448.0f;
    *reinterpret_cast<uint32_t*>(q + e0) = quant4(v, s);
    if (lane == 0) sf[((int64_t)g * kblocks + kb) * M + r] = s;
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

template <bool kPow2>
hipError_t cast_per_token(const void* x, int bf16, int64_t G, int64_t M, int64_t K, uint8_t* q, float* sf,
                          hipStream_t stream) {
  const int64_t kblocks = K / kQ;
  const int64_t nchunks = G * M * kblocks;
  int64_t blocks = (nchunks + 7) / 8;
  if (blocks > 8192) blocks = 8192;  // grid-stride beyond ~32 blocks per CU
  const dim3 grid((unsigned)blocks), block(256);
  if (nchunks < ((int64_t)1 << 32) - 8 * 8192) {  // c + one grid stride stays below 2^32
    const uint32_t n = (uint32_t)nchunks, m = (uint32_t)M, kbs = (uint32_t)kblocks;
    if (bf16) cast_per_token_kernel<true, kPow2, uint32_t><<<grid, block, 0, stream>>>(x, n, m, kbs, q, sf);
    else cast_per_token_kernel<false, kPow2, uint32_t><<<grid, block, 0, stream>>>(x, n, m, kbs, q, sf);
  } else {
    if (bf16) cast_per_token_kernel<true, kPow2, int64_t><<<grid, block, 0, stream>>>(x, nchunks, M, kblocks, q, sf);
    else cast_per_token_kernel<false, kPow2, int64_t><<<grid, block, 0, stream>>>(x, nchunks, M, kblocks, q, sf);
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

hipError_t launch_cast_per_token(const void* x, int bf16, int pow2, int64_t G, int64_t M, int64_t K, uint8_t* q,
                                 float* sf, hipStream_t stream) {
  return pow2 ? cast_per_token<true>(x, bf16, G, M, K, q, sf, stream)
              : cast_per_token<false>(x, bf16, G, M, K, q, sf, stream);
}

hipError_t launch_cast_per_block(const void* w, int bf16, int pow2, int64_t N, int64_t K, uint8_t* q,
                                 float* sf, hipStream_t stream) {
  return pow2 ? cast_per_block<true>(w, bf16, N, K, q, sf, stream) : cast_per_block<false>(w, bf16, N, K, q, sf, stream);
}

}  // namespace dg
