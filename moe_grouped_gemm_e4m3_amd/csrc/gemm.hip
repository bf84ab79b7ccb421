// gemm.hip - FP8 e4m3 block-scaled GEMM for gfx950 (dense, MoE contiguous, MoE masked).
//
// Method (DeepGEMM launch write-up, "Built for modern AI compute" and "Deployment
// guide"; DeepGEMM article, "FP8 and fine-grained scaling"): FP8 products are summed
// over one 128-wide K block on the matrix units, the partial is promoted to fp32,
// multiplied by scale_a[m,kb] * scale_b[n/128,kb] and accumulated; the result is written
// as bf16. On gfx950 one v_mfma_f32_16x16x128_f8f6f4 covers exactly one K block, so
// every MFMA starts from a zero accumulator and its result is folded into the fp32
// accumulators with one v_fma_f32 per element (the promotion runs on the VALU,
// overlapping the next MFMAs).
//
// Two schedules:
//  * decode (M <= 64 per block): HBM-bound on B. A workgroup owns 64 rows x BN columns;
//    its NW waves split the K blocks, stream A and B fragments straight from global
//    memory into registers (32 contiguous bytes per lane), and reduce their partial
//    tiles through LDS at the end.
//  * tile (large M, MFMA-bound): BM x BN workgroup tiles, A/B K-blocks staged through
//    double-buffered LDS (16-byte chunks XOR-swizzled by row to spread banks), 64x64
//    wave tiles of 4x4 MFMAs, a grouped raster of tiles and an XCD-aware workgroup remap
//    so neighbouring tiles share an L2.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "dg_device.h"
#include "dg_launch.h"


namespace dg {
namespace {

struct KParams {
  const uint8_t* a;
  const float* sfa;
  const uint8_t* b;
  const float* sfb;
  uint16_t* d;
  const int32_t* m_indices;
  const int32_t* masked_m;
  int64_t M;  // rows per group: dense M, contiguous M_total, masked M_max
  int64_t N, K;
  int nkb;    // K / 128
  int G;
  int tiles_m, tiles_n;
  int nwg;
  bool pow2;  // every scale is a power of two: the matrix unit applies them (where supported)
  // SwiGLU epilogue (gate/up GEMM of an expert FFN): b holds 2I rows per group, gate rows
  // [0, I) then up rows [I, 2I); the output is h = silu(gate) * up re-cast to FP8 per token
  uint8_t* hq;  // [rows, I] e4m3 (masked: [G, M_max, I])
  float* sh;    // [I/128][rows] fp32 scales (masked: [G][I/128][M_max])
  bool sort_groups;  // masked hybrid: groups taken in descending order of their valid rows
};

__device__ __forceinline__ int64_t clamp_rows(int64_t v, int64_t hi) { return v < 0 ? 0 : (v > hi ? hi : v); }

// Workgroup barrier that orders LDS only: outstanding global loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Direct global->LDS loads (global_load_lds_dwordx4 / _dword: lane i of a wave writes
// bytes [16i, 16i+16) (or [4i, 4i+4)) after the LDS base held in M0). They are issued from
// inline assembly: they write only LDS and have no output registers; an address is a
// wave-uniform 64-bit base plus a per-lane 32-bit offset. Waits for them are explicit.
// M0 is listed as clobbered (the compiler warns that it cannot preserve a reserved register
// across the statement): in these kernels nothing else uses M0, every M0 write in the
// generated code being one of these, so there is nothing to preserve.
// Wave-uniform values in scalar registers; a no-op for values already there. The operands
// below must be uniform, and the compiler cannot always prove that they are.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}
// kStream adds the non-temporal hint, for bytes that no other workgroup of the launch reads
// (the masked layout's expert weights: one tile streams each group's columns).
template <bool kStream = false>
__device__ __forceinline__ void lds_dma16(uint32_t voff, const void* sbase, uint32_t lds_base) {
  if constexpr (kStream)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(__builtin_amdgcn_readfirstlane(lds_base)),
                 "v"(voff), "s"(uniform_ptr(sbase))
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(__builtin_amdgcn_readfirstlane(lds_base)),
                 "v"(voff), "s"(uniform_ptr(sbase))
                 : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(uint32_t voff, const void* sbase, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" ::"s"(__builtin_amdgcn_readfirstlane(lds_base)),
               "v"(voff), "s"(uniform_ptr(sbase))
               : "memory", "m0");
}
// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Wait until at most n groups of P vector-memory loads are outstanding, for a runtime
// n (clamped to [0, MAXN]): s_waitcnt takes an immediate, so this unrolls to a chain.
template <int P, int MAXN>
__device__ __forceinline__ void wait_groups(int n) {
  if constexpr (MAXN <= 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= MAXN) wait_vmcnt<MAXN * P>();
    else wait_groups<P, MAXN - 1>(n);
  }
}

// K split of one 128-byte operand row over the four lane groups g = l >> 4 of an MFMA:
// group g holds bytes [16g, 16g+16) and [64+16g, 64+16g+16). A and B use the same split,
// so the products pair up; each 16-byte load instruction of a wave then covers whole
// 64-byte halves of 16 rows.
__device__ __forceinline__ v8i load_frag_global(const uint8_t* p) {
  const v4i lo = *reinterpret_cast<const v4i*>(p);
  const v4i hi = *reinterpret_cast<const v4i*>(p + 64);
  return cat8(lo, hi);
}
// the same with the non-temporal hint, for weights that no other workgroup reads
__device__ __forceinline__ v8i load_frag_stream(const uint8_t* p) {
  const v4i lo = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
  const v4i hi = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p + 64));
  return cat8(lo, hi);
}

// ---------------------------------------------------------------------------------
// decode schedule
// ---------------------------------------------------------------------------------
// Workgroup: 64 rows x BN columns, NW waves. Wave w owns K blocks kb = w + NW*(KPW*r + i),
// i < KPW, in rounds r. Within a round every load (A and B fragments, both scales) is
// issued before the first MFMA, so a wave keeps KPW K blocks of operands in flight; a
// K block past the end reloads the last block and is weighted by zero.
template <int BN, int NW, int KPW, Layout L>
__global__ __launch_bounds__(64 * NW) void gemm_decode_kernel(KParams p) {
  static_assert(L != Layout::Contiguous, "decode schedule serves dense and masked layouts");
  static_assert(BN % 16 == 0, "columns come in 16-wide MFMA strips");
  constexpr int TN = BN / 16;
  __shared__ __attribute__((aligned(16))) float red[NW][64 * BN];
  __shared__ __attribute__((aligned(16))) float sa_x[NW][KPW][64];

  const uint32_t wg = xcd_remap(blockIdx.x, (uint32_t)p.nwg);
  const int mb = (int)(wg % (uint32_t)p.tiles_m);
  const int nt = (int)((wg / (uint32_t)p.tiles_m) % (uint32_t)p.tiles_n);
  const int g = (int)(wg / (uint32_t)(p.tiles_m * p.tiles_n));
  const int64_t m0 = (int64_t)mb * 64;
  int64_t valid = p.M;
  if constexpr (L == Layout::Masked) valid = clamp_rows(p.masked_m[g], p.M);
  if (m0 >= valid) return;  // uniform over the workgroup
  const int64_t n0 = (int64_t)nt * BN;
  const int nkb = p.nkb;
  const int64_t K = p.K;

  const uint8_t* A = p.a + (int64_t)g * p.M * K;
  const float* SA = p.sfa + (int64_t)g * p.M * nkb;
  const uint8_t* B = p.b + (int64_t)g * p.N * K;
  // each 16-column strip lies inside one 128-column weight-scale block
  const float* SBg = p.sfb + (int64_t)g * (p.N / kQ) * nkb;
  const float* SBj[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) SBj[j] = SBg + ((n0 + 16 * j) / kQ) * nkb;
  uint16_t* D = p.d + (int64_t)g * p.M * p.N;

  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int kof = (l >> 4) * 16;
  const uint8_t* arow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) arow[i] = A + clamp_rows(m0 + 16 * i + (l & 15), valid - 1) * K + kof;
  const uint8_t* brow[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) brow[j] = B + (n0 + 16 * j + (l & 15)) * K + kof;
  const float* sacol = SA + clamp_rows(m0 + l, valid - 1);  // + kb * M: K-block-major scales

  v4f acc[4][TN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int base = w; base < nkb; base += NW * KPW) {
    v8i af[KPW][4], bf[KPW][TN];
    float sam[KPW], sbv[KPW][TN];
#pragma unroll
    for (int u = 0; u < KPW; ++u) {
      const int kb = base + NW * u;
      const int kc = kb < nkb ? kb : nkb - 1;
#pragma unroll
      for (int j = 0; j < TN; ++j) bf[u][j] = load_frag_global(brow[j] + (int64_t)kc * kQ);
#pragma unroll
      for (int i = 0; i < 4; ++i) af[u][i] = load_frag_global(arow[i] + (int64_t)kc * kQ);
      sam[u] = sacol[(int64_t)kc * p.M];
#pragma unroll
      for (int j = 0; j < TN; ++j) sbv[u][j] = SBj[j][kc] * (kb < nkb ? 1.0f : 0.0f);
    }
    // this lane's output rows of strip i are 16*i + 4*(l>>4) + r: route the activation
    // scales there through the wave's private LDS slots
#pragma unroll
    for (int u = 0; u < KPW; ++u) sa_x[w][u][l] = sam[u];
#pragma unroll
    for (int u = 0; u < KPW; ++u) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 s4 = *reinterpret_cast<const float4*>(&sa_x[w][u][16 * i + 4 * (l >> 4)]);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const float t0 = s4.x * sbv[u][j], t1 = s4.y * sbv[u][j], t2 = s4.z * sbv[u][j], t3 = s4.w * sbv[u][j];
          const v4f pp = mfma_f8_16x16x128(af[u][i], bf[u][j]);
          acc[i][j][0] = fmaf(pp[0], t0, acc[i][j][0]);
          acc[i][j][1] = fmaf(pp[1], t1, acc[i][j][1]);
          acc[i][j][2] = fmaf(pp[2], t2, acc[i][j][2]);
          acc[i][j][3] = fmaf(pp[3], t3, acc[i][j][3]);
        }
      }
    }
  }

  // cross-wave reduction of the split-K partial tiles
  float* myred = red[w];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) myred[(16 * i + 4 * (l >> 4) + r) * BN + 16 * j + (l & 15)] = acc[i][j][r];
  __syncthreads();
  constexpr int kGroups = 64 * BN / 4;  // 4 consecutive columns per thread-step
  for (int e = threadIdx.x; e < kGroups; e += 64 * NW) {
    const int row = e / (BN / 4);
    const int c4 = (e % (BN / 4)) * 4;
    float4 s = *reinterpret_cast<const float4*>(&red[0][row * BN + c4]);
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) {
      const float4 t = *reinterpret_cast<const float4*>(&red[ww][row * BN + c4]);
      s.x += t.x; s.y += t.y; s.z += t.z; s.w += t.w;
    }
    if (m0 + row < valid) {
      uint2 o;
      o.x = bf16_rne(s.x) | (bf16_rne(s.y) << 16);
      o.y = bf16_rne(s.z) | (bf16_rne(s.w) << 16);
      *reinterpret_cast<uint2*>(D + (m0 + row) * p.N + n0 + c4) = o;
    }
  }
}

// ---------------------------------------------------------------------------------
// decode schedule, activation block in LDS
// ---------------------------------------------------------------------------------
// Workgroup: 64 rows x BN columns over all of K, NW waves = KG K-groups x (NW/KG) column
// groups. Every weight byte is read once; the 64 x K activation block is read once per
// workgroup, straight into LDS with full-line direct loads, instead of once per wave.
//   1. Each wave issues its share of the activation block and its scales (direct loads
//      into LDS), then all its B fragment loads (K blocks kg, kg+KG, ... of its TN strips)
//      and weight scales; it waits for its share of A only and joins a barrier.
//   2. Per K block, as its B fragments arrive: A fragments from LDS (16-byte chunks
//      XOR-swizzled by row), 4 x TN MFMAs, promotion by sa * sb.
//   3. The K-groups' partial tiles are summed in a fixed order through LDS (the bytes that
//      held A) and written as bf16.
// LDS: A [nkb][64 rows][128 B] | sa [nkb][64] fp32; afterwards the partial tiles.
// The weight fragments and the bf16 results are touched by this workgroup alone and carry the
// non-temporal hint (measured: 7.4 against 7.7 us on 64x7168x2048).
template <int BN, int KG, int KPW, int NW, Layout L, bool kPow2>
__global__ __launch_bounds__(64 * NW) void gemm_decode2_kernel(KParams p) {
  static_assert(L != Layout::Contiguous, "decode schedule serves dense and masked layouts");
  constexpr int SG = NW / KG, TN = BN / 16 / SG;
  static_assert(SG * KG == NW && TN * 16 * SG == BN, "waves split evenly over K and columns");
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

  const uint32_t wg = xcd_remap(blockIdx.x, (uint32_t)p.nwg);
  const int nt = (int)(wg % (uint32_t)p.tiles_n);
  const int mb = (int)((wg / (uint32_t)p.tiles_n) % (uint32_t)p.tiles_m);
  const int g = (int)(wg / (uint32_t)(p.tiles_m * p.tiles_n));
  const int64_t m0 = (int64_t)mb * 64;
  int64_t valid = p.M;
  if constexpr (L == Layout::Masked) valid = clamp_rows(p.masked_m[g], p.M);
  if (m0 >= valid) return;  // uniform over the workgroup
  const int64_t n0 = (int64_t)nt * BN;
  const int nkb = p.nkb;
  const int64_t K = p.K;
  const uint8_t* A = p.a + ((L == Layout::Masked ? (int64_t)g * p.M : 0) + m0) * K;  // this row block
  const float* SA = p.sfa + (L == Layout::Masked ? (int64_t)g * p.M * nkb : 0) + m0;   // + kb * M
  const uint8_t* B = p.b + (int64_t)g * p.N * K;
  const float* SBg = p.sfb + (int64_t)g * (p.N / kQ) * nkb;
  uint16_t* D = p.d + (L == Layout::Masked ? (int64_t)g * p.M * p.N : 0);

  const int t = threadIdx.x, l = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int kg = w % KG, sg = w / KG;
  const int fr = l & 15, g4 = l >> 4;
  const int rows = (int)(valid - m0 < 64 ? valid - m0 : 64);  // rows >= this are clamped

  // 1. the weight scales of this wave's K blocks (a K block past the end reloads the last
  //    one, with weight 0); then the activation block and its scales, straight into LDS:
  //    instruction q covers rows 8*(q%8) .. +8 of K block q/8, and lane l fetches chunk
  //    (l&7) ^ (row&7) of its row, so LDS holds the swizzled layout; then the B fragments
  float sbv[KPW][TN];
#pragma unroll
  for (int u = 0; u < KPW; ++u) {
    const int kb = kg + KG * u;
    const int kc = kb < nkb ? kb : nkb - 1;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t col = n0 + 16 * (sg * TN + j);
      sbv[u][j] = kPow2 ? SBg[(col / kQ) * nkb + kc] : SBg[(col / kQ) * nkb + kc] * (kb < nkb ? 1.0f : 0.0f);
    }
  }
  const uint32_t sbase = (uint32_t)(uintptr_t)smem;
  {
    const int row = (l >> 3);  // + 8 * (q % 8)
    for (int q = w; q < 8 * nkb; q += NW) {
      const int kb = q >> 3, rb = q & 7;
      const int r = 8 * rb + row;
      const int rc = r < rows ? r : rows - 1;
      const uint32_t voff = (uint32_t)((int64_t)rc * K) + (uint32_t)(kb * kQ) + (uint32_t)((((l & 7) ^ (r & 7))) << 4);
      lds_dma16(voff, A, sbase + (uint32_t)(kb * 8192 + rb * 1024));
    }
    const uint32_t soff = (uint32_t)((l < rows ? l : rows - 1) * 4);
    for (int kb = w; kb < nkb; kb += NW)
      lds_dma4(soff, SA + (int64_t)kb * p.M, sbase + (uint32_t)(nkb * 8192 + kb * 256));
  }
  v8i bf[KPW][TN];
#pragma unroll
  for (int u = 0; u < KPW; ++u) {
    const int kb = kg + KG * u;
    const int kc = kb < nkb ? kb : nkb - 1;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t col = n0 + 16 * (sg * TN + j);
      bf[u][j] = load_frag_stream(B + (col + fr) * K + (int64_t)kc * kQ + g4 * 16);
    }
  }
  //    Loads complete in issue order, and the 2*KPW*TN B fragment loads were issued after
  //    the direct ones: at most that many outstanding means this wave's share of A is in
  //    LDS. The barrier then covers every wave's share; the B fragments keep
  //    arriving while the first K blocks are computed.
  wait_vmcnt<2 * KPW * TN>();
  lds_barrier();

  // 2. MFMAs per K block, promotion by sa * sb
  v4f acc[4][TN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  const uint32_t sw0 = (uint32_t)((g4 ^ (fr & 7)) << 4), sw1 = (uint32_t)(((g4 + 4) ^ (fr & 7)) << 4);
#pragma unroll
  for (int u = 0; u < KPW; ++u) {
    const int kb = kg + KG * u;
    const int kc = kb < nkb ? kb : nkb - 1;  // weight 0 past the end
    const uint8_t* ak = smem + kc * 8192 + fr * 128;
    const float* sk = reinterpret_cast<const float*>(smem + nkb * 8192 + kc * 256) + 4 * g4;
    if constexpr (kPow2) {
      // power-of-two scales, applied by the matrix unit (see the tile kernel); lane l gives
      // the E8M0 scale of row 16i + (l & 15) and of its strip's weight block
      if (kb < nkb) {
        const uint32_t* ek = reinterpret_cast<const uint32_t*>(smem + nkb * 8192 + kc * 256) + fr;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const v8i af = cat8(*reinterpret_cast<const v4i*>(ak + i * 2048 + sw0),
                              *reinterpret_cast<const v4i*>(ak + i * 2048 + sw1));
          const int ea = (int)(ek[16 * i] >> 23);
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = mfma_f8_16x16x128_scaled(af, bf[u][j], acc[i][j], ea, (int)(__float_as_uint(sbv[u][j]) >> 23));
        }
      }
      continue;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const v8i af = cat8(*reinterpret_cast<const v4i*>(ak + i * 2048 + sw0),
                          *reinterpret_cast<const v4i*>(ak + i * 2048 + sw1));
      const float4 s4 = *reinterpret_cast<const float4*>(sk + 16 * i);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const v4f pp = mfma_f8_16x16x128(af, bf[u][j]);
        acc[i][j][0] = fmaf(pp[0], s4.x * sbv[u][j], acc[i][j][0]);
        acc[i][j][1] = fmaf(pp[1], s4.y * sbv[u][j], acc[i][j][1]);
        acc[i][j][2] = fmaf(pp[2], s4.z * sbv[u][j], acc[i][j][2]);
        acc[i][j][3] = fmaf(pp[3], s4.w * sbv[u][j], acc[i][j][3]);
      }
    }
  }

  // 3. every wave stores its partial tile row-major in LDS (the bytes that held A); then
  //    each thread sums the KG partials of 4 consecutive columns in the fixed order kg = 0,
  //    1, ... and writes them as bf16
  __syncthreads();  // every wave is done with A in LDS
  float* part = reinterpret_cast<float*>(smem);  // [KG][64][BN]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        part[(kg * 64 + 16 * i + 4 * g4 + r) * BN + 16 * (sg * TN + j) + fr] = acc[i][j][r];
  __syncthreads();
  constexpr int kGroups = 64 * BN / 4;  // 4 consecutive columns per thread-step
  for (int e = t; e < kGroups; e += 64 * NW) {
    const int row = e / (BN / 4);
    const int c4 = (e % (BN / 4)) * 4;
    if (row < rows) {
      float4 v = *reinterpret_cast<const float4*>(&part[row * BN + c4]);
#pragma unroll
      for (int k2 = 1; k2 < KG; ++k2) {
        const float4 u4 = *reinterpret_cast<const float4*>(&part[(k2 * 64 + row) * BN + c4]);
        v.x += u4.x; v.y += u4.y; v.z += u4.z; v.w += u4.w;
      }
      uint2 o;
      o.x = bf16_rne(v.x) | (bf16_rne(v.y) << 16);
      o.y = bf16_rne(v.z) | (bf16_rne(v.w) << 16);
      __builtin_nontemporal_store(((uint64_t)o.y << 32) | o.x, reinterpret_cast<uint64_t*>(D + (m0 + row) * p.N + n0 + c4));
    }
  }
}

inline size_t decode2_need(int bn, int kg, int nkb) {  // bytes of dynamic LDS
  const size_t a = (size_t)nkb * 8192 + (size_t)nkb * 256;  // A block + its scales
  const size_t r = (size_t)kg * 64 * bn * 4;                 // the K-groups' partial tiles
  return a > r ? a : r;
}

// ---------------------------------------------------------------------------------
// decode schedule with the activation block resident in LDS and a weight ring
// ---------------------------------------------------------------------------------
// For 64-row blocks whose 64 x K activation bytes fit in LDS beside the ring. A workgroup
// owns 64 rows x BN = 16 * WN * TN columns; its WM x WN waves split them, wave (wm, wn)
// taking row strips wm*TM .. +TM (TM = 4 / WM) and column strips wn*TN .. +TN:
//   1. prologue: the activation block ([K block][64 rows][128 B], 16-byte chunks XOR-swizzled
//      by row), its scales and the weight scales of the (at most two) 128-column blocks the
//      tile touches go straight into LDS; then the first S-1 K blocks of the weight columns
//      ([BN rows][128 B], same swizzle) into the ring;
//   2. per K block: wait for its weights, one barrier, refill the slot the previous K block
//      freed, TM x TN MFMAs per wave promoted by sa * sb (or, with power-of-two scales, applied
//      by the matrix unit). Only weights move per K block: a CU keeps S-1 K blocks of them in
//      flight and reads the activation block once;
//   3. the bf16 tile goes through LDS and leaves as 16-byte row pieces.
// The K blocks are summed in order with the same fp32 operations and the same MFMA operand
// split as the tile kernels, so the results agree with theirs bit for bit. The weight ring's
// loads and the result stores carry the non-temporal hint, as in the kernel above (measured:
// 10.3 against 11.2 us on 64x24576x1536).
inline size_t decode3_need(int bn, int stages, int nkb) {  // bytes of dynamic LDS
  const size_t ring = (size_t)nkb * 8192 + (size_t)nkb * 256 + (size_t)((8 * nkb + 15) & ~15);
  const size_t need = ring + (size_t)stages * bn * 128;
  const size_t tile = (size_t)64 * (2 * bn + 16);  // the epilogue's bf16 tile
  return need > tile ? need : tile;
}

template <int WM, int WN, int TN, int S, Layout L, bool kPow2>
__global__ __launch_bounds__(64 * WM * WN) void gemm_decode3_kernel(KParams p) {
  static_assert(L != Layout::Contiguous, "decode schedule serves dense and masked layouts");
  constexpr int NW = WM * WN, TM = 4 / WM;  // wave (wm, wn): row strips wm*TM.., column strips wn*TN..
  constexpr int BN = 16 * WN * TN;
  static_assert(TM * WM == 4, "the wave rows split the 4 row strips");
  constexpr int PB = BN * 8 / (64 * NW);  // direct loads per wave per K block of weights
  constexpr int RING = BN * (int)kQ;      // bytes per ring slot
  constexpr int PITCH = 2 * BN + 16;      // epilogue tile row (the pad spreads LDS banks)
  static_assert(PB * 64 * NW == BN * 8 && BN <= (int)kQ, "weight ring split, at most two scale blocks");
  static_assert(S >= 2 && (S - 1) * PB < 64, "ring depth");
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

  const uint32_t wg = xcd_remap(blockIdx.x, (uint32_t)p.nwg);
  const int nt = (int)(wg % (uint32_t)p.tiles_n);
  const int mb = (int)((wg / (uint32_t)p.tiles_n) % (uint32_t)p.tiles_m);
  const int g = (int)(wg / (uint32_t)(p.tiles_m * p.tiles_n));
  const int64_t m0 = (int64_t)mb * 64;
  int64_t valid = p.M;
  if constexpr (L == Layout::Masked) valid = clamp_rows(p.masked_m[g], p.M);
  if (m0 >= valid) return;  // uniform over the workgroup
  const int64_t n0 = (int64_t)nt * BN;
  const int nkb = p.nkb;
  const int64_t K = p.K;
  const uint8_t* A = p.a + ((L == Layout::Masked ? (int64_t)g * p.M : 0) + m0) * K;  // this row block
  const float* SA = p.sfa + (L == Layout::Masked ? (int64_t)g * p.M * nkb : 0) + m0;   // + kb * M + row
  const uint8_t* B = p.b + ((int64_t)g * p.N + n0) * K;                                // the tile's rows
  const float* SBg = p.sfb + (int64_t)g * (p.N / kQ) * nkb;
  uint16_t* D = p.d + (L == Layout::Masked ? (int64_t)g * p.M * p.N : 0);

  const int t = threadIdx.x, l = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int rows = (int)(valid - m0 < 64 ? valid - m0 : 64);  // rows >= this are clamped
  const uint32_t base = (uint32_t)(uintptr_t)smem;
  const uint32_t offSA = (uint32_t)nkb * 8192, offSB = offSA + (uint32_t)nkb * 256;
  const uint32_t offR = offSB + (uint32_t)((8 * nkb + 15) & ~15);
  const int64_t b0 = n0 / kQ;  // the tile's first weight-scale block

  // 1. activation block, its scales and the weight scales, then the first weight K blocks;
  //    loads complete in issue order, so the wait for weight K block 0 covers all of these
  {
    const int row = l >> 3;
    for (int q = w; q < 8 * nkb; q += NW) {  // instruction q: K block q/8, rows 8*(q%8) .. +8
      const int kb = q >> 3, rb = q & 7;
      const int r = 8 * rb + row;
      const int rc = r < rows ? r : rows - 1;
      const uint32_t voff = (uint32_t)((int64_t)rc * K) + (uint32_t)(kb * kQ) + (uint32_t)((((l & 7) ^ (r & 7))) << 4);
      lds_dma16(voff, A, base + (uint32_t)(kb * 8192 + rb * 1024));
    }
    const uint32_t soff = (uint32_t)((l < rows ? l : rows - 1) * 4);
    for (int kb = w; kb < nkb; kb += NW) lds_dma4(soff, SA + (int64_t)kb * p.M, base + offSA + (uint32_t)(kb * 256));
    if (w == NW - 1) {
      const int64_t last = p.N / kQ - 1;
#pragma unroll
      for (int bi = 0; bi < 2; ++bi) {
        const float* src = SBg + (b0 + bi < last ? b0 + bi : last) * nkb;
        for (int q = 0; q < nkb; q += 64)
          if (q + l < nkb) lds_dma4((uint32_t)((q + l) * 4), src, base + offSB + (uint32_t)((bi * nkb + q) * 4));
      }
    }
  }
  uint32_t boff[PB];
#pragma unroll
  for (int u = 0; u < PB; ++u) {
    const int row = (u * NW + w) * 8 + (l >> 3);
    boff[u] = (uint32_t)(row * K) + (uint32_t)(((l & 7) ^ ((l >> 3) & 7)) << 4);
  }
  auto issue = [&](int kb) {
    const uint32_t sb = base + offR + (uint32_t)((kb % S) * RING);
    const uint8_t* bb = B + (int64_t)kb * kQ;
#pragma unroll
    for (int u = 0; u < PB; ++u) lds_dma16<true>(boff[u], bb, sb + (uint32_t)((u * NW + w) * 1024));
  };
#pragma unroll
  for (int q = 0; q < S - 1; ++q)
    if (q < nkb) issue(q);

  // 2. the K loop. The activation fragments and scales of K block kb+1 are read from LDS
  //    (resident, no wait needed) while K block kb's MFMAs run; every operand read of a K
  //    block is issued before its first MFMA.
  const int fr = l & 15, g4 = l >> 4;
  const uint32_t sw0 = (uint32_t)((g4 ^ (fr & 7)) << 4), sw1 = (uint32_t)(((g4 + 4) ^ (fr & 7)) << 4);
  const int wm = w % WM, wn = w / WM;
  int sbi[TN];  // weight-scale block of each strip, relative to b0
#pragma unroll
  for (int j = 0; j < TN; ++j) sbi[j] = (int)((n0 + 16 * (wn * TN + j)) / kQ - b0);
  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  // activation operands of one K block: fragments of the wave's TM row strips and, per lane,
  // the scales of its 4 output rows in each strip (fp32) or the E8M0 scale of its fragment row
  auto read_a = [&](v8i (&af)[TM], float4 (&s4)[TM], int kb) {
    const uint8_t* ak = smem + kb * 8192 + (wm * TM * 16 + fr) * 128;
#pragma unroll
    for (int i = 0; i < TM; ++i)
      af[i] = cat8(*reinterpret_cast<const v4i*>(ak + i * 2048 + sw0), *reinterpret_cast<const v4i*>(ak + i * 2048 + sw1));
    if constexpr (kPow2) {
      const float* ek = reinterpret_cast<const float*>(smem + offSA + kb * 256) + wm * TM * 16 + fr;
#pragma unroll
      for (int i = 0; i < TM; ++i) s4[i].x = ek[16 * i];
    } else {
      const float* sk = reinterpret_cast<const float*>(smem + offSA + kb * 256) + wm * TM * 16 + 4 * g4;
#pragma unroll
      for (int i = 0; i < TM; ++i) s4[i] = *reinterpret_cast<const float4*>(sk + 16 * i);
    }
  };
  // one K block: wait for its weights, refill the ring, read its weight fragments and the
  // next K block's activation operands (into the other buffer; past the end a harmless
  // re-read), then the MFMAs on this K block's activation operands
  auto step = [&](int kb, const v8i (&afc)[TM], const float4 (&s4c)[TM], v8i (&afn)[TM], float4 (&s4n)[TM]) {
    if (kb > 0) {
      wait_groups<PB, S - 2>(nkb - 1 - kb);  // K blocks kb .. min(kb+S-2, nkb-1) are in flight
      lds_barrier();
    }
    if (kb + S - 1 < nkb) issue(kb + S - 1);  // into the slot K block kb-1 used
    const uint8_t* ring = smem + offR + (kb % S) * RING;
    v8i bf[TN];
    float sb[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const uint8_t* bp = ring + (16 * (wn * TN + j) + fr) * (int)kQ;
      bf[j] = cat8(*reinterpret_cast<const v4i*>(bp + sw0), *reinterpret_cast<const v4i*>(bp + sw1));
      sb[j] = reinterpret_cast<const float*>(smem + offSB)[sbi[j] * nkb + kb];
    }
    read_a(afn, s4n, kb + 1 < nkb ? kb + 1 : kb);
    if constexpr (kPow2) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = mfma_f8_16x16x128_scaled(afc[i], bf[j], acc[i][j], (int)(__float_as_uint(s4c[i].x) >> 23),
                                               (int)(__float_as_uint(sb[j]) >> 23));
    } else {
      // every product of the K block in its own registers, so the MFMAs issue back to back
      // and the promotions of the first ones overlap the last ones (one shared result
      // register would serialise MFMA latency and promotion TM x TN times)
      v4f pp[TM][TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) pp[i][j] = mfma_f8_16x16x128(afc[i], bf[j]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          acc[i][j][0] = fmaf(pp[i][j][0], s4c[i].x * sb[j], acc[i][j][0]);
          acc[i][j][1] = fmaf(pp[i][j][1], s4c[i].y * sb[j], acc[i][j][1]);
          acc[i][j][2] = fmaf(pp[i][j][2], s4c[i].z * sb[j], acc[i][j][2]);
          acc[i][j][3] = fmaf(pp[i][j][3], s4c[i].w * sb[j], acc[i][j][3]);
        }
    }
  };
  v8i af0[TM], af1[TM];
  float4 s40[TM], s41[TM];
  if (nkb > 0) {
    wait_groups<PB, S - 2>(nkb - 1);  // K block 0's weights, and with them all of the prologue
    lds_barrier();
    read_a(af0, s40, 0);
  }
  for (int kb = 0; kb < nkb; kb += 2) {  // two K blocks per trip: the operand buffers alternate
    step(kb, af0, s40, af1, s41);
    if (kb + 1 < nkb) step(kb + 1, af1, s41, af0, s40);
  }

  // 3. epilogue: bf16 tile [64][PITCH] in LDS over the activation block, then 16-byte pieces
  //    of the valid rows
  wait_vmcnt<0>();
  __syncthreads();  // every wave is done with the ring and the activation block
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<uint16_t*>(smem + (16 * (wm * TM + i) + 4 * g4 + r) * PITCH + (16 * (wn * TN + j) + fr) * 2) =
            (uint16_t)bf16_rne(acc[i][j][r]);
  __syncthreads();
  constexpr int PPR = BN / 8;  // 16-byte pieces per row
  for (int e = t; e < 64 * PPR; e += 64 * NW) {
    const int row = e / PPR, c = e - row * PPR;
    if (row < rows)
      __builtin_nontemporal_store(*reinterpret_cast<const v4i*>(smem + row * PITCH + c * 16),
                                   reinterpret_cast<v4i*>(D + (m0 + row) * p.N + n0 + c * 8));
  }
}



template <int BN, int NW, int KPW, Layout L>
hipError_t run_decode(KParams kp, hipStream_t s) {
  if (kp.N % BN != 0) return hipErrorInvalidValue;
  kp.tiles_n = (int)(kp.N / BN);
  kp.tiles_m = (int)((kp.M + 63) / 64);
  const int64_t nwg = (int64_t)kp.G * kp.tiles_m * kp.tiles_n;
  if (nwg <= 0) return hipSuccess;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  kp.nwg = (int)nwg;
  gemm_decode_kernel<BN, NW, KPW, L><<<dim3((unsigned)nwg), dim3(64 * NW), 0, s>>>(kp);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// tile schedule, deep prefetch
// ---------------------------------------------------------------------------------
// BM x BN workgroup tile, (WM x WN) waves of (BM/WM) x (BN/WN). Global loads run two K
// blocks ahead of the MFMAs through two register staging sets; each K block is written
// to one of two LDS buffers and read back as MFMA fragments. Barriers order LDS only, so
// the loads for the next two K blocks stay in flight across them.
template <int BM, int BN, int WM, int WN, Layout L>
__global__ __launch_bounds__(64 * WM * WN) void gemm_tile2_kernel(KParams p) {
  constexpr int NT = 64 * WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 16, TN = WTN / 16;
  constexpr int ACH = BM * 8 / NT;  // 16-byte chunks of an A K-block per thread
  constexpr int BCH = BN * 8 / NT;
  static_assert(ACH * NT == BM * 8 && BCH * NT == BN * 8, "chunk split");
  // weight-scale column blocks per tile; each wave's columns lie inside one of them
  constexpr int NB = BN > (int)kQ ? BN / (int)kQ : 1;
  static_assert((BN % kQ == 0 || kQ % BN == 0) && kQ % WTN == 0, "tile vs weight-scale blocks");
  static_assert(L != Layout::Contiguous || BM == kQ, "contiguous layout: one expert per M tile");
  static_assert(BM <= NT, "one activation scale per thread");
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * kQ];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * kQ];
  __shared__ __attribute__((aligned(16))) float sSa[2][NB][BM];

  const uint32_t wg = xcd_remap(blockIdx.x, (uint32_t)p.nwg);
  int g = 0, tm, tn;
  if constexpr (L == Layout::Masked) {
    tm = (int)(wg % (uint32_t)p.tiles_m);
    tn = (int)((wg / (uint32_t)p.tiles_m) % (uint32_t)p.tiles_n);
    g = (int)(wg / (uint32_t)(p.tiles_m * p.tiles_n));
  } else {
    constexpr int GM = 8;
    const int per_band = GM * p.tiles_n;
    const int band = (int)wg / per_band;
    const int first = band * GM;
    const int gm = min(p.tiles_m - first, GM);
    const int in = (int)wg % per_band;
    tm = first + in % gm;
    tn = in / gm;
  }
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  int64_t valid = p.M;
  if constexpr (L == Layout::Masked) {
    valid = clamp_rows(p.masked_m[g], p.M);
    if (m0 >= valid) return;
  }
  if constexpr (L == Layout::Contiguous) {
    g = p.m_indices[m0];
    if (g < 0 || g >= p.G) return;
  }
  const int nkb = p.nkb;
  const int64_t K = p.K;
  const uint8_t* A = p.a + (L == Layout::Masked ? (int64_t)g * p.M * K : 0);
  const float* SA = p.sfa + (L == Layout::Masked ? (int64_t)g * p.M * nkb : 0);
  const uint8_t* B = p.b + (int64_t)g * p.N * K;
  const float* SB = p.sfb + ((int64_t)g * (p.N / kQ) + n0 / kQ) * nkb;
  uint16_t* D = p.d + (L == Layout::Masked ? (int64_t)g * p.M * p.N : 0);

  const int t = threadIdx.x, w = t >> 6, l = t & 63;
  const int wm = w % WM, wn = w / WM;

  // staging: chunk c = t + NT*u is row c/8, 16-byte column c%8 (rows read whole)
  const uint8_t* ga = A + clamp_rows(m0 + (t >> 3), valid - 1) * K + (t & 7) * 16;
  const uint8_t* gb = B + (n0 + (t >> 3)) * K + (t & 7) * 16;
  constexpr int RSTEP = NT / 8;  // rows advanced per staging step
  const uint32_t lst = (uint32_t)((t >> 3) * kQ + (((t & 7) ^ ((t >> 3) & 7)) << 4));
  // every thread loads and stores an activation scale (threads t and t+BM duplicate one
  // row): no divergent branch inside the pipelined loop
  const int srow = t % BM;
  const float* gsa = SA + clamp_rows(m0 + srow, valid - 1);  // + kb * M
  // byte offsets of the staged A rows from the first one (rows past the valid count are
  // clamped to the last valid row); B rows are always in range
  uint32_t aoff[ACH];
#pragma unroll
  for (int u = 0; u < ACH; ++u) {
    const int64_t r = m0 + (t >> 3) + RSTEP * u;
    aoff[u] = (uint32_t)((clamp_rows(r, valid - 1) - clamp_rows(m0 + (t >> 3), valid - 1)) * K);
  }
  const uint32_t bstep = (uint32_t)(RSTEP * K);

  v4i ra0[ACH], rb0[BCH], ra1[ACH], rb1[BCH];
  float rs0[NB], rs1[NB];
  // loads one K block; the activation scale is multiplied by the K block's weight scale
  // here, so LDS holds the full promotion factor sa[m,kb] * sb[n/128,kb]
  auto gload = [&](v4i (&ra)[ACH], v4i (&rb)[BCH], float (&rs)[NB], int kb) {
    const uint32_t ko = (uint32_t)kb * kQ;
#pragma unroll
    for (int u = 0; u < ACH; ++u) ra[u] = *reinterpret_cast<const v4i*>(ga + aoff[u] + ko);
#pragma unroll
    for (int u = 0; u < BCH; ++u) rb[u] = *reinterpret_cast<const v4i*>(gb + bstep * u + ko);
    const float sa = gsa[(int64_t)kb * p.M];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) rs[nb] = sa * SB[nb * nkb + kb];
  };
  auto lstore = [&](const v4i (&ra)[ACH], const v4i (&rb)[BCH], const float (&rs)[NB], int buf) {
#pragma unroll
    for (int u = 0; u < ACH; ++u) *reinterpret_cast<v4i*>(&sA[buf][lst + RSTEP * u * kQ]) = ra[u];
#pragma unroll
    for (int u = 0; u < BCH; ++u) *reinterpret_cast<v4i*>(&sB[buf][lst + RSTEP * u * kQ]) = rb[u];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) sSa[buf][nb][srow] = rs[nb];
  };

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int fr = l & 15, g4 = l >> 4;
  const uint32_t sw0 = (uint32_t)((g4 ^ (fr & 7)) << 4), sw1 = (uint32_t)(((g4 + 4) ^ (fr & 7)) << 4);
  const uint32_t a_lane = (uint32_t)((wm * WTM + fr) * kQ), b_lane = (uint32_t)((wn * WTN + fr) * kQ);
  const int sa_lane = wm * WTM + 4 * g4;

  // One K block: TM x TN MFMAs, each promoted with one FMA per output element. The
  // promotion of strip i-1 is interleaved with the MFMAs of strip i (software pipeline),
  // so the matrix pipe never waits on the FMAs that consume its previous results.
  // MFMA products and promotion factors of the two most recent strips. The promotion of
  // a strip runs under the MFMAs of the next one, also across K blocks: the last strip of
  // a K block is promoted under the first MFMAs of the next K block. The slots start at
  // zero, so the first promotion adds 0 * 0.
  static_assert(TM % 2 == 0, "strip parity must repeat every K block");
  v4f pp[2][TN];
  float4 tt[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    tt[q] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < TN; ++j) pp[q][j] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  auto promote = [&](int slot, int strip) {
    const float4 tp = tt[slot];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      acc[strip][j][0] = fmaf(pp[slot][j][0], tp.x, acc[strip][j][0]);
      acc[strip][j][1] = fmaf(pp[slot][j][1], tp.y, acc[strip][j][1]);
      acc[strip][j][2] = fmaf(pp[slot][j][2], tp.z, acc[strip][j][2]);
      acc[strip][j][3] = fmaf(pp[slot][j][3], tp.w, acc[strip][j][3]);
    }
  };
  auto compute = [&](int buf) {
    const uint8_t* a_s = sA[buf] + a_lane;
    const uint8_t* b_s = sB[buf] + b_lane;
    const float* t_s = &sSa[buf][(wn * WTN) / (int)kQ][sa_lane];
    v8i bfr[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j)
      bfr[j] = cat8(*reinterpret_cast<const v4i*>(b_s + j * 16 * kQ + sw0),
                    *reinterpret_cast<const v4i*>(b_s + j * 16 * kQ + sw1));
    v8i afr[2];
    float4 tn[2];
    afr[0] = cat8(*reinterpret_cast<const v4i*>(a_s + sw0), *reinterpret_cast<const v4i*>(a_s + sw1));
    tn[0] = *reinterpret_cast<const float4*>(t_s);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int cur = i & 1, prv = cur ^ 1;
      if (i + 1 < TM) {  // next strip's fragment and factors, one strip ahead
        afr[prv] = cat8(*reinterpret_cast<const v4i*>(a_s + (i + 1) * 16 * kQ + sw0),
                        *reinterpret_cast<const v4i*>(a_s + (i + 1) * 16 * kQ + sw1));
        tn[prv] = *reinterpret_cast<const float4*>(t_s + 16 * (i + 1));
      }
      // MFMAs of strip i into slot cur; promotion of the previous strip from slot prv
      v4f fresh[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) fresh[j] = mfma_f8_16x16x128(afr[cur], bfr[j]);
      promote(prv, i > 0 ? i - 1 : TM - 1);
#pragma unroll
      for (int j = 0; j < TN; ++j) pp[cur][j] = fresh[j];
      tt[cur] = tn[cur];
      // scheduling hint: alternate one MFMA with four promotion FMAs
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
    }
  };

  // prologue: K block 0 into LDS buffer 0, K block 1 in flight in set 1
  gload(ra0, rb0, rs0, 0);
  gload(ra1, rb1, rs1, min(1, nkb - 1));
  lstore(ra0, rb0, rs0, 0);
  lds_barrier();
  // steady state: two K blocks per trip, straight-line so that each LDS store waits only
  // for its own staging set while the other set's loads stay in flight
  int kb = 0;
  for (; kb + 3 < nkb; kb += 2) {
    gload(ra0, rb0, rs0, kb + 2);
    compute(0);
    lstore(ra1, rb1, rs1, 1);
    lds_barrier();
    gload(ra1, rb1, rs1, kb + 3);
    compute(1);
    lstore(ra0, rb0, rs0, 0);
    lds_barrier();
  }
  // tail: 1 to 3 K blocks left; buffer 0 holds kb, set 1 holds kb + 1
  if (kb + 2 < nkb) gload(ra0, rb0, rs0, kb + 2);
  compute(0);
  if (kb + 1 < nkb) {
    lstore(ra1, rb1, rs1, 1);
    lds_barrier();
    compute(1);
    if (kb + 2 < nkb) {
      lstore(ra0, rb0, rs0, 0);
      lds_barrier();
      compute(0);
    }
  }
  promote(1, TM - 1);  // the last strip (odd slot, TM even)
  __builtin_amdgcn_s_waitcnt(0);

  // epilogue: bf16 round-to-nearest-even, rows beyond the valid count are not written
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = m0 + wm * WTM + 16 * i + 4 * g4 + r;
      if (row < valid) {
        uint16_t* drow = D + row * p.N + n0 + wn * WTN + fr;
#pragma unroll
        for (int j = 0; j < TN; ++j) drow[16 * j] = (uint16_t)bf16_rne(acc[i][j][r]);
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// tile schedule, direct-to-LDS loads into a ring of LDS stages
// ---------------------------------------------------------------------------------
// A, B and the activation scales of a K block go straight from global memory into one of
// STAGES LDS stages (no staging registers). The loads for K block kb+STAGES are issued in
// the middle of K block kb, into the stage kb just released.
//
// Per K block a wave runs TM strips of 16 rows: strip i+1's A fragment is read while strip
// i's MFMAs run. After strip TM-2 nothing more is read from the current stage, so the wave
// waits for the next stage's loads, joins an LDS-only barrier, issues the loads that refill
// the stage just released, and reads the next K block's fragments while the last strip's
// MFMAs run. MFMA products and promotion factors rotate through two register slots, so
// every MFMA co-issues with the promotion FMAs of the previous strip.
//
// The loop issues no vector-memory loads besides the direct ones (the tile's weight scales
// are staged in LDS up front), so the explicit vmcnt values count exactly those.
//
// kSwiglu: the gate/up GEMM of an expert FFN with the activation and the FP8 re-cast in
// the epilogue (DeepGEMM article, "swapAB and Mega MoE": the FFN's two GEMMs and its
// SwiGLU activation fused). A 256-row B tile holds 128 gate rows and the 128 matching up
// rows, so a workgroup owns one 128-column block of h = silu(gate) * up for BM tokens:
// exactly the 1x128 chunks the per-token cast needs.
constexpr int kMaxKb3 = 256;  // K blocks the direct-load tile kernel supports (K <= 32768)

// silu(g) * u in fp32: exp and reciprocal on the transcendental unit (a few ulp each)
__device__ __forceinline__ float swiglu1(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.44269504088896341f);  // exp(-g)
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// Epilogue of the SwiGLU tile: h = silu(gate) * up from the fp32 accumulators, then the
// per-token cast of h (DeepSeek-V3 repo review, "Innovations" item 4: one scale per 128
// elements; "Risks" item 6: bound 448): per row of the tile's 128 h columns
// amax -> s = amax / 448 (or its power of two) -> q = e4m3(h / s), s == 0 giving signed
// zeros. Waves wn = 0, 1 hold gate columns, wn = 2, 3 the same columns of up (so the main
// loop is the plain one: one weight-scale block per wave). Partner waves wn and wn ^ 2 swap
// half of their strips through LDS: the gate wave forms h for the first TM/2 strips, the up
// wave for the last TM/2. Row maxima combine through LDS, the codes are staged in LDS and
// leave as 16-byte row segments. The LDS ring is free here.
//
// Both sides run the same code; a side's choices are selects of values read with
// compile-time indices (indexing the accumulators with a runtime strip, or branching per
// side, moves them to scratch memory).

// exchange slot of (direction, strip i of the half, fragment j) for this lane's pair
__device__ __forceinline__ int swg_slot(int pair, int dir, int i, int j, int TH, int TN, int l) {
  return ((pair * 2 + dir) * TH * TN + i * TN + j) * 64 + l;
}

// q = e4m3(h / s) for this wave's strips, staged in sQ ([rows][128] bytes; the 16-byte chunk
// c of row r sits at chunk c ^ (r & 7), which spreads LDS banks).
// The quotient is the correctly rounded fp32 h / s, from the row's reciprocal r = RN(1/s)
// and Markstein's correction step (q0 = RN(h r), e = h - s q0 exact by FMA,
// q = RN(q0 + e r)); that step is exact unless the residual underflows, so rows with
// s < 2^-80 divide. Power-of-two scales: h r is the exact quotient. s == 0: signed zeros.
// The hardware conversion (round to nearest even) is exact for |x| <= 448.0001, the range
// h / s stays in. A 4x4 byte transpose over each lane quad turns the four row codes of a
// lane into four column codes of one row.
template <int TH, int TN, int WM, Layout L, bool kPow2>
__device__ __forceinline__ void swg_quant(const v4f (&hv)[TH][TN], const float* sS, const float* sR, uint8_t* sQ,
                                          int strip0, int wm, int half, int l, int act) {
  const int fr = l & 15, g4 = l >> 4;
  const int k4 = fr & 3, c4 = fr >> 2;
  const uint32_t selA = (fr & 2) ? 0x03020706u : 0x05040100u;
  const uint32_t selB = (fr & 1) ? 0x03070105u : 0x06020400u;
#pragma unroll
  for (int i = 0; i < TH; ++i) {
    if (L == Layout::Masked && strip0 + i >= act) continue;
    const int rb = ((strip0 + i) * WM + wm) * 16 + 4 * g4;
    const float4 s4 = *reinterpret_cast<const float4*>(sS + rb);
    const float4 r4 = *reinterpret_cast<const float4*>(sR + rb);
    const float sv[4] = {s4.x, s4.y, s4.z, s4.w}, rv[4] = {r4.x, r4.y, r4.z, r4.w};
    constexpr float kTiny = 0x1p-80f;
    const bool fast = kPow2 || (s4.x >= kTiny && s4.y >= kTiny && s4.z >= kTiny && s4.w >= kTiny);
    const bool all_fast = __all(fast);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float h = hv[i][j][r];
        if (kPow2) {
          x[r] = h * rv[r];
        } else if (all_fast) {
          const float q0 = h * rv[r];
          x[r] = fmaf(fmaf(-q0, sv[r], h), rv[r], q0);
        } else {
          const float q0 = h * rv[r];
          x[r] = sv[r] == 0.0f ? h * 0.0f : (sv[r] >= kTiny ? fmaf(fmaf(-q0, sv[r], h), rv[r], q0) : h / sv[r]);
        }
      }
      uint32_t P = e4m3_hw_pack4(x[0], x[1], x[2], x[3]);  // |x| <= 448.0001 here
      uint32_t Q = (uint32_t)__builtin_amdgcn_mov_dpp((int)P, 0x4E, 0xF, 0xF, true);  // lane ^ 2
      P = __builtin_amdgcn_perm(Q, P, selA);
      Q = (uint32_t)__builtin_amdgcn_mov_dpp((int)P, 0xB1, 0xF, 0xF, true);           // lane ^ 1
      P = __builtin_amdgcn_perm(Q, P, selB);
      const int row = rb + k4, chunk = half * TN + j;
      *reinterpret_cast<uint32_t*>(sQ + row * (int)kQ + ((chunk ^ (row & 7)) << 4) + 4 * c4) = P;
    }
  }
}

template <int BM, int WM, int WN, int TM, int TN, Layout L, bool kPow2>
__device__ __forceinline__ void swiglu_epilogue(const KParams& p, v4f (&acc)[TM][TN], uint8_t* smem, int g, int tn,
                                                int64_t m0, int64_t valid, int act) {
  constexpr int NW = WM * WN, NT = 64 * NW;
  constexpr int TH = TM / 2;                 // strips each wave of a pair finishes
  constexpr int PART = 2 * 16;               // partial maxima per row: (column half, lane column)
  constexpr int PST = BM + 4;                // padded stride of a partial column (spreads LDS banks)
  constexpr int TPR = NT / BM;               // threads reducing one row
  static_assert(WN == 4 && TN * 16 * 2 == (int)kQ, "two column halves of 64 per operand");
  static_assert(TPR >= 1 && (TPR & (TPR - 1)) == 0 && PART % TPR == 0, "row reduction split");
  const int t = threadIdx.x, l = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = w % WM, wn = w / WM;
  const int fr = l & 15, g4 = l >> 4;
  const bool up_side = wn >= 2;
  const int half = wn & 1;                   // which 64 of the 128 h columns
  const int pair = wm * 2 + half;
  const int64_t I = p.N / 2;

  v4f* sX = reinterpret_cast<v4f*>(smem);   // [pairs][direction][TH][TN][64 lanes]
  const int strip0 = up_side ? TH : 0;       // the strips this wave finishes: strip0 .. +TH
  __syncthreads();  // every wave is past its last read of the LDS ring
  // the gate wave sends its gate values of strips TH.., the up wave its up values of strips 0..TH-1
#pragma unroll
  for (int i = 0; i < TH; ++i) {
    if (L == Layout::Masked && (TH - strip0) + i >= act) continue;
#pragma unroll
    for (int j = 0; j < TN; ++j) sX[swg_slot(pair, up_side, i, j, TH, TN, l)] = up_side ? acc[i][j] : acc[TH + i][j];
  }
  __syncthreads();
  // h for strips strip0.. from this wave's accumulators and the partner's
  v4f hv[TH][TN];
  float pm[TH][4];
#pragma unroll
  for (int i = 0; i < TH; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) pm[i][r] = 0.f;
#pragma unroll
    for (int j = 0; j < TN; ++j) hv[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    if (L == Layout::Masked && strip0 + i >= act) continue;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const v4f other = sX[swg_slot(pair, !up_side, i, j, TH, TN, l)];
      const v4f mine = up_side ? acc[TH + i][j] : acc[i][j];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float h = swiglu1(up_side ? other[r] : mine[r], up_side ? mine[r] : other[r]);
        hv[i][j][r] = h;
        pm[i][r] = fmaxf(pm[i][r], fabsf(h));
      }
    }
  }
  __syncthreads();  // the exchange area is reused below

  float* sAm = reinterpret_cast<float*>(smem);  // [PART][PST]
  float* sS = sAm + PART * PST;                 // [BM] row scales
  float* sR = sS + BM;                          // [BM] their reciprocals
  uint8_t* sQ = reinterpret_cast<uint8_t*>(sR + BM);  // [BM][128] codes
#pragma unroll
  for (int i = 0; i < TH; ++i) {
    const int si = strip0 + i;
    if (L == Layout::Masked && si >= act) continue;
    *reinterpret_cast<float4*>(sAm + (half * 16 + fr) * PST + (si * WM + wm) * 16 + 4 * g4) =
        make_float4(pm[i][0], pm[i][1], pm[i][2], pm[i][3]);
  }
  __syncthreads();
  {
    const int row = t / TPR, part = t % TPR;
    float am = 0.f;
#pragma unroll
    for (int k = 0; k < PART / TPR; ++k) am = fmaxf(am, sAm[(part * (PART / TPR) + k) * PST + row]);
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, TPR));
    const float s = kPow2 ? pow2_ceil(am / 448.0f) : am / 448.0f;
    if (part == 0) {
      sS[row] = s;
      sR[row] = 1.0f / s;
      if (m0 + row < valid) {
        float* SH = p.sh + (L == Layout::Masked ? (int64_t)g * (I / kQ) * p.M : 0);
        SH[(int64_t)tn * p.M + m0 + row] = s;
      }
    }
  }
  __syncthreads();
  swg_quant<TH, TN, WM, L, kPow2>(hv, sS, sR, sQ, strip0, wm, half, l, act);
  __syncthreads();
  uint8_t* HQ = p.hq + (L == Layout::Masked ? (int64_t)g * p.M * I : 0);
#pragma unroll
  for (int idx = t; idx < BM * 8; idx += NT) {
    const int row = idx >> 3, c16 = idx & 7;
    if (m0 + row < valid) {
      const v4i q = *reinterpret_cast<const v4i*>(sQ + row * (int)kQ + ((c16 ^ (row & 7)) << 4));
      v4i* dst = reinterpret_cast<v4i*>(HQ + (m0 + row) * I + (int64_t)tn * kQ + c16 * 16);
      if constexpr (L == Layout::Masked) __builtin_nontemporal_store(q, dst);  // as the bf16 stores
      else *dst = q;
    }
  }
}

// kSplit: a stage's weight rows are dead once every wave holds their fragments, at the start
// of the K block, while its activation rows are read strip by strip until the middle of it.
// The weights of K block kb+STAGES are then issued at the start of K block kb and its
// activations after the middle barrier, so that half a K block more of loads is in flight,
// for a second barrier per K block.
template <int BM, int BN, int WM, int WN, int STAGES, Layout L, bool kPow2, bool kSwiglu, bool kSplit>
__device__ __forceinline__ void tile3_main(const KParams& p, uint8_t* smem, float (*sSB)[kMaxKb3], int g, int tm,
                                           int tn) {
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 16, TN = WTN / 16;
  constexpr int NB = BN > (int)kQ ? BN / (int)kQ : 1;
  constexpr int ADMA = BM * 8 / (64 * NW);  // 1 KB direct loads per wave per K block (A)
  constexpr int BDMA = BN * 8 / (64 * NW);  // (B)
  constexpr int SROWS = BM / NW;            // activation-scale rows loaded per wave
  constexpr int PER_STAGE = ADMA + BDMA + 1;
  constexpr int STAGE_BYTES = (BM + BN) * (int)kQ + BM * 4;
  static_assert(ADMA * 64 * NW == BM * 8 && BDMA * 64 * NW == BN * 8, "direct-load split");
  static_assert(SROWS >= 1 && SROWS <= 64 && SROWS * NW == BM, "scale rows per wave");
  static_assert((BN % kQ == 0 || kQ % BN == 0) && kQ % WTN == 0, "tile vs weight-scale blocks");
  // contiguous layout: one expert per row tile; a 256-row tile is launched only over two
  // 128-row blocks of the same expert (gemm_contiguous_hybrid_kernel checks that)
  static_assert(L != Layout::Contiguous || BM == kQ || BM == 2 * kQ, "contiguous layout: one expert per M tile");
  static_assert(TM >= 2 && TM % 2 == 0, "strip slots alternate and repeat every K block");
  static_assert(STAGES >= 2 && STAGES <= 6 && (STAGES - 1) * PER_STAGE < 64, "LDS ring depth");
  static_assert(!kSplit || (STAGES - 2) * PER_STAGE + BDMA < 64, "split issue: loads in flight");
  static_assert(STAGES * STAGE_BYTES + NB * kMaxKb3 * 4 <= 160 * 1024, "LDS");
  static_assert(!kSwiglu || (BN == 2 * (int)kQ && TM % 2 == 0), "SwiGLU tile: 128 gate + 128 up rows");
  static_assert(!kSwiglu || (32 * (BM + 4) * 4 + BM * 8 + BM * (int)kQ <= STAGES * STAGE_BYTES &&
                             BM * BN * 2 <= STAGES * STAGE_BYTES),
                "SwiGLU epilogue fits in the LDS ring");
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  int64_t valid = p.M;
  if constexpr (L == Layout::Masked) {
    valid = clamp_rows(p.masked_m[g], p.M);
    if (m0 >= valid) return;
  }
  if constexpr (L == Layout::Contiguous) {
    g = p.m_indices[m0];
    if (g < 0 || g >= p.G) return;
  }
  const int nkb = p.nkb;
  const int64_t K = p.K;
  const uint8_t* A = p.a + (L == Layout::Masked ? (int64_t)g * p.M * K : 0);
  const float* SA = p.sfa + (L == Layout::Masked ? (int64_t)g * p.M * nkb : 0);
  const uint8_t* B = p.b + (int64_t)g * p.N * K;
  const float* SB = p.sfb + (int64_t)g * (p.N / kQ) * nkb;
  // B row of tile row r: plain tiles take rows n0.., SwiGLU tiles the gate block tn and
  // the up block I/128 + tn (I = N/2)
  auto b_row = [&](int r) -> int64_t {
    if constexpr (kSwiglu) return r < (int)kQ ? (int64_t)tn * kQ + r : p.N / 2 + (int64_t)tn * kQ + (r - (int)kQ);
    else return n0 + r;
  };
  uint16_t* D = p.d + (L == Layout::Masked ? (int64_t)g * p.M * p.N : 0);

  const int t = threadIdx.x, l = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform
  const int wm = w % WM, wn = w / WM;
  const uint32_t smem_base = (uint32_t)(uintptr_t)smem;

  // per-lane 32-bit source offsets of this wave's direct loads; LDS layout of a stage:
  // A [BM][128] | B [BN][128] | sa [BM] floats, 16-byte chunks XOR-swizzled by (row & 7)
  uint32_t aoff[ADMA], boff[BDMA];
#pragma unroll
  for (int u = 0; u < ADMA; ++u) {
    const int row = (u * NW + w) * 8 + (l >> 3);
    aoff[u] = (uint32_t)(clamp_rows(m0 + row, valid - 1) * K) + (uint32_t)(((l & 7) ^ ((l >> 3) & 7)) << 4);
  }
#pragma unroll
  for (int u = 0; u < BDMA; ++u) {
    const int row = (u * NW + w) * 8 + (l >> 3);
    boff[u] = (uint32_t)(b_row(row) * K) + (uint32_t)(((l & 7) ^ ((l >> 3) & 7)) << 4);
  }
  const uint32_t soff = (uint32_t)(clamp_rows(m0 + w * SROWS + (l < SROWS ? l : 0), valid - 1) * 4);
  // The masked layout streams each group's weight columns through exactly one tile and writes
  // results no kernel of this launch reads: its weight loads and its result stores (bf16, or
  // the fused FFN's codes) carry the non-temporal hint (6-7% faster there; on the dense and
  // contiguous layouts, whose weights other row tiles re-read from L2, the hint was slower).

  auto issue = [&](int kb, int stage) {
    const uint32_t sbase = smem_base + (uint32_t)(stage * STAGE_BYTES);
    const uint8_t* ab = A + (int64_t)kb * kQ;
    const uint8_t* bb = B + (int64_t)kb * kQ;
#pragma unroll
    for (int u = 0; u < ADMA; ++u) lds_dma16(aoff[u], ab, sbase + (uint32_t)((u * NW + w) * 1024));
#pragma unroll
    for (int u = 0; u < BDMA; ++u) lds_dma16<L == Layout::Masked>(boff[u], bb, sbase + (uint32_t)(BM * kQ + (u * NW + w) * 1024));
    if (l < SROWS) lds_dma4(soff, SA + (int64_t)kb * p.M, sbase + (uint32_t)((BM + BN) * kQ + w * SROWS * 4));
  };
  // the two halves of a stage, for the split issue: activation rows with their scales, and
  // weight rows
  auto issue_a = [&](int kb, int stage) {
    const uint32_t sbase = smem_base + (uint32_t)(stage * STAGE_BYTES);
    const uint8_t* ab = A + (int64_t)kb * kQ;
#pragma unroll
    for (int u = 0; u < ADMA; ++u) lds_dma16(aoff[u], ab, sbase + (uint32_t)((u * NW + w) * 1024));
    if (l < SROWS) lds_dma4(soff, SA + (int64_t)kb * p.M, sbase + (uint32_t)((BM + BN) * kQ + w * SROWS * 4));
  };
  auto issue_b = [&](int kb, int stage) {
    const uint32_t sbase = smem_base + (uint32_t)(stage * STAGE_BYTES);
    const uint8_t* bb = B + (int64_t)kb * kQ;
#pragma unroll
    for (int u = 0; u < BDMA; ++u) lds_dma16<L == Layout::Masked>(boff[u], bb, sbase + (uint32_t)(BM * kQ + (u * NW + w) * 1024));
  };
  // start of K block kb (split issue): every wave holds its weight fragments (read at the end
  // of the previous K block), so its stage's weight rows take those of K block kb+STAGES
  auto split_start = [&](int kb, int st) {
    if constexpr (kSplit) {
      lds_barrier();
      if (kb + STAGES < nkb) issue_b(kb + STAGES, st);
    }
  };
  // middle of K block kb: wait for K block kb+1, one barrier, refill stage st. Loads issued
  // after K block kb+1's may stay in flight: whole stages kb+2 .. kb+STAGES-1 and, with the
  // split issue, the weights of K block kb+STAGES
  auto refill = [&](int kb, int st) {
    if constexpr (kSplit) {
      if (kb + STAGES < nkb) wait_vmcnt<(STAGES - 2) * PER_STAGE + BDMA>();
      else wait_groups<PER_STAGE, STAGES - 2>(nkb - 2 - kb);
      lds_barrier();
      if (kb + STAGES < nkb) issue_a(kb + STAGES, st);
    } else {
      wait_groups<PER_STAGE, STAGES - 2>(nkb - 2 - kb);
      lds_barrier();
      if (kb + STAGES < nkb) issue(kb + STAGES, st);
    }
  };

  // the tile's weight scales for every K block, straight into LDS by wave 0 ahead of the
  // first stage (loads complete in issue order, so the first stage's wait covers them and
  // the barrier after it publishes them); the loop below issues no other vector-memory
  // loads (its vmcnt waits count the direct-to-LDS ones only)
  if (w == 0) {
    const uint32_t sb_lds = (uint32_t)(uintptr_t)&sSB[0][0];
#pragma unroll
    for (int bi = 0; bi < NB; ++bi) {
      const float* src = SB + (b_row(bi * (int)kQ) / kQ) * nkb;
      for (int q = 0; q < nkb; q += 64)
        if (q + l < nkb) lds_dma4((uint32_t)((q + l) * 4), src, sb_lds + (uint32_t)((bi * kMaxKb3 + q) * 4));
    }
  }

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int fr = l & 15, g4 = l >> 4;
  const uint32_t sw0 = (uint32_t)((g4 ^ (fr & 7)) << 4), sw1 = (uint32_t)(((g4 + 4) ^ (fr & 7)) << 4);
  // strip i of wave row wm holds rows (i * WM + wm) * 16 .. +16 of the tile: the wave rows
  // interleave by strips, so a partly valid tile (masked layout) leaves every wave a
  // similar number of active strips
  const uint32_t a_lane = (uint32_t)((wm * 16 + fr) * kQ);
  const uint32_t b_lane = (uint32_t)(BM * kQ + (wn * WTN + fr) * kQ);
  const uint32_t s_lane = (uint32_t)((BM + BN) * kQ + (wm * 16 + 4 * g4) * 4);
  const int wnb = (wn * WTN) / (int)kQ;  // this wave's weight-scale column block

  auto read_b = [&](v8i (&bf)[TN], int stage) {
    const uint8_t* b_s = smem + stage * STAGE_BYTES + b_lane;
#pragma unroll
    for (int j = 0; j < TN; ++j)
      bf[j] = cat8(*reinterpret_cast<const v4i*>(b_s + j * 16 * kQ + sw0),
                   *reinterpret_cast<const v4i*>(b_s + j * 16 * kQ + sw1));
  };
  auto read_a = [&](v8i& af, float4& s4, int stage, int i) {
    const uint8_t* st = smem + stage * STAGE_BYTES;
    af = cat8(*reinterpret_cast<const v4i*>(st + a_lane + i * 16 * WM * kQ + sw0),
              *reinterpret_cast<const v4i*>(st + a_lane + i * 16 * WM * kQ + sw1));
    s4 = *reinterpret_cast<const float4*>(st + s_lane + 64 * WM * i);
  };

  v4f pp[2][TN];
  float4 tt[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    tt[q] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < TN; ++j) pp[q][j] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  // masked layout: strips wholly beyond the valid rows skip their MFMAs and promotions
  // (their rows are never stored); act is wave-uniform
  int act = TM;
  if constexpr (L == Layout::Masked) {
    const int64_t left = valid - m0 - wm * 16;  // rows from this wave's first strip on
    act = left <= 0 ? 0 : (int)min((int64_t)TM, (left + 16 * WM - 1) / (16 * WM));
  }
  auto promote = [&](int slot, int strip) {
    if (L == Layout::Masked && strip >= act) return;
    const float4 tp = tt[slot];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      acc[strip][j][0] = fmaf(pp[slot][j][0], tp.x, acc[strip][j][0]);
      acc[strip][j][1] = fmaf(pp[slot][j][1], tp.y, acc[strip][j][1]);
      acc[strip][j][2] = fmaf(pp[slot][j][2], tp.z, acc[strip][j][2]);
      acc[strip][j][3] = fmaf(pp[slot][j][3], tp.w, acc[strip][j][3]);
    }
    // pin the FMAs here: left alone, the compiler sinks every promotion of a K block below
    // its last MFMA, which keeps all strips' products live and serialises MFMA and VALU work
#pragma unroll
    for (int j = 0; j < TN; ++j) asm volatile("" ::"v"(acc[strip][j]));
  };
  // MFMAs of one strip into `slot`, interleaved with the promotion of the other slot
  auto strip = [&](const v8i& af, const v8i (&bf)[TN], int slot, int cur_strip, int prev_strip) {
    if (!(L == Layout::Masked && cur_strip >= act)) {
#pragma unroll
      for (int j = 0; j < TN; ++j) pp[slot][j] = mfma_f8_16x16x128(af, bf[j]);
    }
    promote(slot ^ 1, prev_strip);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
  };
  auto factor = [](const float4& s4, float sb) {
    return make_float4(s4.x * sb, s4.y * sb, s4.z * sb, s4.w * sb);
  };

  // K block kb from stage `st` with B fragments `bf` and strip 0's A fragment `a0`; the
  // next K block's fragments (stage `sn`) replace them, B as the last strip's MFMAs
  // consume it
  auto kblock = [&](int kb, int st, int sn, v8i (&bf)[TN], v8i& a0, float4& s0) {
    split_start(kb, st);
    const float sb = sSB[wnb][kb];
    v8i af[2];
    float4 s4[2];
    af[0] = a0;
    s4[0] = s0;
#pragma unroll
    for (int i = 0; i < TM - 1; ++i) {
      const int c = i & 1;
      read_a(af[c ^ 1], s4[c ^ 1], st, i + 1);
      strip(af[c], bf, c, i, i == 0 ? TM - 1 : i - 1);  // strip 0 promotes the previous K block's last
      tt[c] = factor(s4[c], sb);
    }
    // every read of stage st is issued; wait for the next stage, then recycle stage st
    // (stages kb+1 .. min(kb+STAGES-1, nkb-1) are in flight; the last ones issue nothing)
    __builtin_amdgcn_sched_barrier(0);
    refill(kb, st);
    read_a(a0, s0, sn, 0);  // after the last K block: unused reads of a stale stage
    // last strip (odd slot): B fragment j is reloaded from stage sn right after the MFMA
    // that last reads it
#pragma unroll
    for (int j = 0; j < TN; ++j)
      if (!(L == Layout::Masked && TM - 1 >= act)) pp[1][j] = mfma_f8_16x16x128(af[1], bf[j]);
    promote(0, TM - 2);
    read_b(bf, sn);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
    tt[1] = factor(s4[1], sb);
  };

  // power-of-two scales: the matrix unit applies them. Lane l supplies the E8M0 scale of
  // row l & 15 of the A strip (every lane group the same, the scale being per 128-K block)
  // and of column l & 15 of the B strip; products accumulate straight into acc, with no
  // promotion on the vector ALUs. An E8M0 byte is the fp32 exponent field of the scale.
  const uint32_t e_lane = (uint32_t)((BM + BN) * kQ + (wm * 16 + fr) * 4);
  auto read_a2 = [&](v8i& af, int& ea, int stage, int i) {
    const uint8_t* st = smem + stage * STAGE_BYTES;
    af = cat8(*reinterpret_cast<const v4i*>(st + a_lane + i * 16 * WM * kQ + sw0),
              *reinterpret_cast<const v4i*>(st + a_lane + i * 16 * WM * kQ + sw1));
    ea = (int)(*reinterpret_cast<const uint32_t*>(st + e_lane + 64 * WM * i) >> 23);
  };
  auto kblock2 = [&](int kb, int st, int sn, v8i (&bf)[TN], v8i& a0, int& e0) {
    split_start(kb, st);
    const int eb = (int)(__float_as_uint(sSB[wnb][kb]) >> 23);
    v8i af[2];
    int ea[2];
    af[0] = a0;
    ea[0] = e0;
#pragma unroll
    for (int i = 0; i < TM - 1; ++i) {
      const int c = i & 1;
      read_a2(af[c ^ 1], ea[c ^ 1], st, i + 1);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        if (!(L == Layout::Masked && i >= act))
          acc[i][j] = mfma_f8_16x16x128_scaled(af[c], bf[j], acc[i][j], ea[c], eb);
    }
    __builtin_amdgcn_sched_barrier(0);
    refill(kb, st);
    read_a2(a0, e0, sn, 0);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      if (!(L == Layout::Masked && TM - 1 >= act))
        acc[TM - 1][j] = mfma_f8_16x16x128_scaled(af[1], bf[j], acc[TM - 1][j], ea[1], eb);
    read_b(bf, sn);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };

  // prologue: the first STAGES K blocks in flight; wait for K block 0
#pragma unroll
  for (int q = 0; q < STAGES; ++q)
    if (q < nkb) issue(q, q);
  wait_groups<PER_STAGE, STAGES - 1>((nkb < STAGES ? nkb : STAGES) - 1);
  lds_barrier();
  v8i bf[TN], a0;
  read_b(bf, 0);
  int st = 0;
  if constexpr (kPow2) {
    int e0;
    read_a2(a0, e0, 0, 0);
    for (int kb = 0; kb < nkb; ++kb) {
      const int sn = st == STAGES - 1 ? 0 : st + 1;
      kblock2(kb, st, sn, bf, a0, e0);
      st = sn;
    }
  } else {
    float4 s0;
    read_a(a0, s0, 0, 0);
    for (int kb = 0; kb < nkb; ++kb) {
      const int sn = st == STAGES - 1 ? 0 : st + 1;
      kblock(kb, st, sn, bf, a0, s0);
      st = sn;
    }
    promote(1, TM - 1);  // the last strip (odd slot)
  }
  wait_vmcnt<0>();     // nothing is in flight by now; kept as a guard before the epilogue

  if constexpr (kSwiglu) {
    swiglu_epilogue<BM, WM, WN, TM, TN, L, kPow2>(p, acc, smem, g, tn, m0, valid, act);
    return;
  }

  // epilogue: bf16 round-to-nearest-even, rows beyond the valid count are not written
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = m0 + (i * WM + wm) * 16 + 4 * g4 + r;
      if (row < valid) {
        uint16_t* drow = D + row * p.N + n0 + wn * WTN + fr;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const uint16_t v = (uint16_t)bf16_rne(acc[i][j][r]);
          if constexpr (L == Layout::Masked) __builtin_nontemporal_store(v, &drow[16 * j]);
          else drow[16 * j] = v;
        }
      }
    }
  }
}

// Logical workgroup -> tile. Masked: row tile fastest, then column tile, then group. Other
// layouts: bands of GM row tiles walked column by column, so neighbouring workgroups share
// weight columns (and, under the XCD remap, one L2).
__device__ __forceinline__ void tile_of(const KParams& p, uint32_t wg, bool masked, int& g, int& tm, int& tn,
                                        int GM = 8) {
  g = 0;
  if (masked) {
    tm = (int)(wg % (uint32_t)p.tiles_m);
    tn = (int)((wg / (uint32_t)p.tiles_m) % (uint32_t)p.tiles_n);
    g = (int)(wg / (uint32_t)(p.tiles_m * p.tiles_n));
  } else {
    const int per_band = GM * p.tiles_n;
    const int band = (int)wg / per_band;
    const int first = band * GM;
    const int gm = min(p.tiles_m - first, GM);
    const int in = (int)wg % per_band;
    tm = first + in % gm;
    tn = in / gm;
  }
}

template <int BM, int BN, int WM, int WN, int STAGES, Layout L, bool kPow2, bool kSwiglu = false, bool kSplit = false>
__global__ __launch_bounds__(64 * WM * WN) void gemm_tile3_kernel(KParams p) {
  constexpr int NB = BN > (int)kQ ? BN / (int)kQ : 1;
  constexpr int STAGE_BYTES = (BM + BN) * (int)kQ + BM * 4;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) float sSB[NB][kMaxKb3];  // this tile's weight scales
  int g, tm, tn;
  tile_of(p, xcd_remap(blockIdx.x, (uint32_t)p.nwg), L == Layout::Masked, g, tm, tn);
  tile3_main<BM, BN, WM, WN, STAGES, L, kPow2, kSwiglu, kSplit>(p, smem, sSB, g, tm, tn);
}

// The group of rank `pos` when the groups are ordered by descending valid-row count (ties by
// index); G <= 64: lane i ranks group i against every other, and the group whose rank is pos
// is the one lane that finds it. Every wave computes it alike (wave-uniform result).
__device__ __forceinline__ int group_by_rank(const KParams& p, int pos) {
  const int lane = threadIdx.x & 63;
  const int c = lane < p.G ? (int)clamp_rows(p.masked_m[lane], p.M) : -1;
  int rank = 0;
  for (int j = 0; j < p.G; ++j) {
    const int cj = __shfl(c, j, 64);
    rank += (cj > c || (cj == c && j < lane)) ? 1 : 0;
  }
  // the ranks of groups 0..G-1 are a permutation of 0..G-1, so exactly one lane matches
  return __ffsll((unsigned long long)__ballot(lane < p.G && rank == pos)) - 1;
}

// Masked layout, 256-row tiles: a tile with at most 128 valid rows (its group's count
// minus its first row) runs as a 128 x 256 tile with three LDS stages (two K blocks of
// weights in flight), a fuller one as a 256 x 256 tile with two stages and the split issue.
// Each tile streams its group's weight columns once either way; the smaller row tile only
// leaves LDS room for the third stage. Both bodies share one LDS allocation, and sum the K
// blocks with the same operations as every other tile kernel.
template <bool kPow2, bool kSwiglu>
__global__ __launch_bounds__(512) void gemm_masked_hybrid_kernel(KParams p) {
  constexpr int kSmallStage = (128 + 256) * (int)kQ + 128 * 4, kLargeStage = (256 + 256) * (int)kQ + 256 * 4;
  constexpr int kBytes = 3 * kSmallStage > 2 * kLargeStage ? 3 * kSmallStage : 2 * kLargeStage;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kBytes];
  __shared__ __attribute__((aligned(16))) float sSB[2][kMaxKb3];
  int g, tm, tn;
  if (p.sort_groups) {
    // at most two rounds: each XCD takes whole groups (a group's activation rows stay in one
    // L2), dealt by rank in a snake so that every XCD gets a like mix of large and small
    // groups, the largest first (slot k of XCD x: rank 8k + x, or 8k + 7 - x for odd k)
    tile_of(p, xcd_remap(blockIdx.x, (uint32_t)p.nwg), true, g, tm, tn);  // tm counts 256-row tiles
    int rank = g;
    if (p.G % 8 == 0) {
      const int per = p.G / 8, x = g / per, k = g % per;
      rank = k * 8 + ((k & 1) ? 7 - x : x);
    }
    g = group_by_rank(p, rank);
  } else {
    // more rounds: groups in order, without the XCD remap, so that a group's column tiles go to
    // all XCDs in turn (measured on 32 groups x 256 rows at N=7168, K=2048: 2-13% faster than
    // four whole groups per XCD, and 5-8% faster than any order by size)
    tile_of(p, blockIdx.x, true, g, tm, tn);
  }
  const int64_t left = clamp_rows(p.masked_m[g], p.M) - (int64_t)tm * 256;
  if (left <= 128)  // also the tiles with no valid row: the body returns at once
    tile3_main<128, 256, 2, 4, 3, Layout::Masked, kPow2, kSwiglu, false>(p, smem, sSB, g, 2 * tm, tn);
  else
    tile3_main<256, 256, 2, 4, 2, Layout::Masked, kPow2, kSwiglu, true>(p, smem, sSB, g, tm, tn);
}

// Contiguous layout, 256-row tiles over pairs of 128-row blocks: a pair whose two blocks
// belong to the same expert (the expert of each block's first row) runs as one 256 x 256
// tile (two LDS stages, 1.5x fewer operand bytes per MFMA than 128 x 256); any other pair
// runs as its two 128 x 256 blocks one after the other (three stages each; a block whose first
// row is -1 is skipped as always). Bands of 4 row tiles (about one expert's rows at 8 experts
// and 8192 tokens) walked column by column: the 32 workgroups an XCD takes in one round are
// 4 row tiles x 8 column tiles, so each weight column tile is read by 4 of them and each
// activation row tile by 8.
template <bool kPow2, bool kSwiglu>
__global__ __launch_bounds__(512) void gemm_contiguous_hybrid_kernel(KParams p) {
  constexpr int kSmallStage = (128 + 256) * (int)kQ + 128 * 4, kLargeStage = (256 + 256) * (int)kQ + 256 * 4;
  constexpr int kBytes = 3 * kSmallStage > 2 * kLargeStage ? 3 * kSmallStage : 2 * kLargeStage;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kBytes];
  __shared__ __attribute__((aligned(16))) float sSB[2][kMaxKb3];
  int g, tm, tn;
  tile_of(p, xcd_remap(blockIdx.x, (uint32_t)p.nwg), false, g, tm, tn, 4);  // tm counts 256-row tiles
  const int64_t r0 = (int64_t)tm * 256;
  const int e0 = p.m_indices[r0];
  const int e1 = r0 + 128 < p.M ? p.m_indices[r0 + 128] : -1;
  if (e0 >= 0 && e0 < p.G && e1 == e0) {
    tile3_main<256, 256, 2, 4, 2, Layout::Contiguous, kPow2, kSwiglu, false>(p, smem, sSB, 0, tm, tn);
    return;
  }
  tile3_main<128, 256, 2, 4, 3, Layout::Contiguous, kPow2, kSwiglu, false>(p, smem, sSB, 0, 2 * tm, tn);
  if (r0 + 128 >= p.M) return;
  __syncthreads();  // every wave is done with the first block's LDS stages
  tile3_main<128, 256, 2, 4, 3, Layout::Contiguous, kPow2, kSwiglu, false>(p, smem, sSB, 0, 2 * tm + 1, tn);
}

template <int BM, int BN, int WM, int WN, Layout L>
hipError_t run_tile2(KParams kp, hipStream_t s) {
  kp.tiles_n = (int)(kp.N / BN);
  kp.tiles_m = (int)((kp.M + BM - 1) / BM);
  const int64_t nwg = (int64_t)(L == Layout::Masked ? kp.G : 1) * kp.tiles_m * kp.tiles_n;
  if (nwg <= 0) return hipSuccess;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  kp.nwg = (int)nwg;
  gemm_tile2_kernel<BM, BN, WM, WN, L><<<dim3((unsigned)nwg), dim3(64 * WM * WN), 0, s>>>(kp);
  return hipGetLastError();
}

// direct-to-LDS tile schedule; hipErrorNotSupported when the problem exceeds what its
// 32-bit per-lane offsets or its LDS table of weight scales can address
template <int BM, int BN, int WM, int WN, int STAGES, Layout L, bool kSwiglu = false, bool kSplit = false>
hipError_t run_tile3(KParams kp, hipStream_t s) {
  if (kp.N % BN != 0 || kp.nkb > kMaxKb3 || kp.M * kp.K >= ((int64_t)1 << 32) ||
      kp.N * kp.K >= ((int64_t)1 << 32) || kp.M * kp.nkb * 4 >= ((int64_t)1 << 32))
    return hipErrorNotSupported;
  kp.tiles_n = (int)(kp.N / BN);
  kp.tiles_m = (int)((kp.M + BM - 1) / BM);
  const int64_t nwg = (int64_t)(L == Layout::Masked ? kp.G : 1) * kp.tiles_m * kp.tiles_n;
  if (nwg <= 0) return hipSuccess;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  kp.nwg = (int)nwg;
  if (kp.pow2)
    gemm_tile3_kernel<BM, BN, WM, WN, STAGES, L, true, kSwiglu, kSplit><<<dim3((unsigned)nwg), dim3(64 * WM * WN), 0, s>>>(kp);
  else
    gemm_tile3_kernel<BM, BN, WM, WN, STAGES, L, false, kSwiglu, kSplit><<<dim3((unsigned)nwg), dim3(64 * WM * WN), 0, s>>>(kp);
  return hipGetLastError();
}

// Tuning switches, read from the environment once per process (at the first GEMM call) and
// again only on request (reload_tuning_switches):
//   DG_TILE=<name>    forces one of the tile kernels where it applies (names in launch_gemm);
//   DG_DECODE=v1      the register-fed decode schedule; any DG_DECODE value keeps dense M <= 64
//                     on the decode schedules;
//   DG_DECODE2=bn,kg,kpw,waves   one LDS decode configuration (set at all: not decode3);
//   DG_DECODE3=wm,wn,strips,slots one activation-resident decode configuration;
//   DG_LOG            names the chosen kernel of every call on stderr.
struct Tuning {
  char tile[32] = "";
  bool decode_set = false, decode_v1 = false;
  bool decode2_set = false, decode2_ok = false;
  int decode2[4] = {0, 0, 0, 0};
  bool decode3_ok = false;
  int decode3[4] = {0, 0, 0, 0};
  bool log = false;
};

Tuning read_tuning() {
  Tuning t;
  if (const char* v = getenv("DG_TILE")) snprintf(t.tile, sizeof t.tile, "%s", v);
  if (const char* v = getenv("DG_DECODE")) {
    t.decode_set = true;
    t.decode_v1 = strcmp(v, "v1") == 0;
  }
  if (const char* v = getenv("DG_DECODE2")) {
    t.decode2_set = true;
    int* c = t.decode2;
    t.decode2_ok = sscanf(v, "%d,%d,%d,%d", &c[0], &c[1], &c[2], &c[3]) == 4;
  }
  if (const char* v = getenv("DG_DECODE3")) {
    int* c = t.decode3;
    t.decode3_ok = sscanf(v, "%d,%d,%d,%d", &c[0], &c[1], &c[2], &c[3]) == 4;
  }
  t.log = getenv("DG_LOG") != nullptr;
  return t;
}

std::mutex g_tuning_mu;
std::atomic<const Tuning*> g_tuning{nullptr};

// The current record. A reload publishes a new one and keeps the old one alive, since a launch
// on another thread may still be reading it (a few dozen bytes per reload).
const Tuning& tuning() {
  const Tuning* t = g_tuning.load(std::memory_order_acquire);
  if (t) return *t;
  std::lock_guard<std::mutex> lock(g_tuning_mu);
  t = g_tuning.load(std::memory_order_relaxed);
  if (!t) {
    t = new Tuning(read_tuning());
    g_tuning.store(t, std::memory_order_release);
  }
  return *t;
}

// Compute units of the current device (cached per device; 256 on MI355X).
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// the masked hybrid of 128- and 256-row tiles; hipErrorNotSupported where run_tile3 would
// refuse either body
template <bool kSwiglu>
hipError_t run_masked_hybrid(KParams kp, hipStream_t s) {
  if (kp.N % 256 != 0 || kp.nkb > kMaxKb3 || kp.M * kp.K >= ((int64_t)1 << 32) ||
      kp.N * kp.K >= ((int64_t)1 << 32) || kp.M * kp.nkb * 4 >= ((int64_t)1 << 32))
    return hipErrorNotSupported;
  kp.tiles_n = (int)(kp.N / 256);
  kp.tiles_m = (int)((kp.M + 255) / 256);
  const int64_t nwg = (int64_t)kp.G * kp.tiles_m * kp.tiles_n;
  if (nwg <= 0) return hipSuccess;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  kp.nwg = (int)nwg;
  // groups by descending valid rows when the grid is at most two rounds of workgroups: the
  // largest tiles start first and the smallest fill the end (measured on 32 groups x 256 rows,
  // valid ~U{0..256}, N=4096, K=7168, 512 workgroups: 4-7% faster than in order with the XCD
  // remap); with more rounds the groups in order (sorted: 5-8% slower at N=7168, K=2048)
  kp.sort_groups = kp.G <= 64 && nwg <= 2 * (int64_t)cu_count();
  if (kp.pow2)
    gemm_masked_hybrid_kernel<true, kSwiglu><<<dim3((unsigned)nwg), dim3(512), 0, s>>>(kp);
  else
    gemm_masked_hybrid_kernel<false, kSwiglu><<<dim3((unsigned)nwg), dim3(512), 0, s>>>(kp);
  return hipGetLastError();
}

// The contiguous hybrid pays off when its rounds of 256-row tiles, each worth two 128-row
// tiles, take no longer than the rounds of 128-row tiles: measured on 8 experts x 8192
// tokens, 160 against 169 us at N = 7168, K = 2048 (8 rounds either way), but 340 against
// 305 us at N = 4096, K = 7168 (544 tiles: 3 rounds of double tiles against 4.25 rounds).
bool contiguous_hybrid_pays(const KParams& kp) {
  const int64_t cus = cu_count();
  const int64_t tn = kp.N / 256;
  const int64_t t256 = ((kp.M + 255) / 256) * tn, t128 = (kp.M / 128) * tn;
  return 2 * ((t256 + cus - 1) / cus) <= (t128 + cus - 1) / cus;
}

template <bool kSwiglu>
hipError_t run_contiguous_hybrid(KParams kp, hipStream_t s) {
  if (kp.N % 256 != 0 || kp.M % 128 != 0 || kp.nkb > kMaxKb3 || kp.M * kp.K >= ((int64_t)1 << 32) ||
      kp.N * kp.K >= ((int64_t)1 << 32) || kp.M * kp.nkb * 4 >= ((int64_t)1 << 32))
    return hipErrorNotSupported;
  kp.tiles_n = (int)(kp.N / 256);
  kp.tiles_m = (int)((kp.M + 255) / 256);
  const int64_t nwg = (int64_t)kp.tiles_m * kp.tiles_n;
  if (nwg <= 0) return hipSuccess;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  kp.nwg = (int)nwg;
  if (kp.pow2)
    gemm_contiguous_hybrid_kernel<true, kSwiglu><<<dim3((unsigned)nwg), dim3(512), 0, s>>>(kp);
  else
    gemm_contiguous_hybrid_kernel<false, kSwiglu><<<dim3((unsigned)nwg), dim3(512), 0, s>>>(kp);
  return hipGetLastError();
}

constexpr size_t kLdsBytes = 163840;  // gfx950 LDS per workgroup

// Lets kernel Fn use the whole LDS as dynamic shared memory. The attribute belongs to the
// current device, so it is set once per kernel and device (devices 0..63; others every call).
template <auto Fn>
hipError_t allow_full_lds() {
  static std::atomic<bool> done[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return hipErrorInvalidDevice;
  if (dev < 64 && done[dev].load(std::memory_order_acquire)) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(Fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)kLdsBytes);
  if (e == hipSuccess && dev < 64) done[dev].store(true, std::memory_order_release);
  return e;
}

// Instantiated configurations of the register-fed decode schedule, the ones its automatic
// choice takes: (columns per workgroup, waves, K blocks per wave per round).
#define DG_DECODE_CONFIGS(X) \
  X(48, 4, 3) X(32, 4, 3) X(32, 8, 2) X(32, 4, 4) X(16, 8, 2) X(16, 4, 3) X(16, 4, 4)

template <Layout L>
hipError_t run_decode_cfg(int bn, int nw, int kpw, const KParams& kp, hipStream_t s, bool* found) {
  *found = true;
#define DG_X(a, b, c) \
  if (bn == a && nw == b && kpw == c) return run_decode<a, b, c, L>(kp, s);
  DG_DECODE_CONFIGS(DG_X)
#undef DG_X
  *found = false;
  return hipSuccess;
}

template <int BN, int KG, int KPW, int NW, Layout L, bool kPow2>
hipError_t run_decode2(KParams kp, hipStream_t s) {
  const size_t lds = decode2_need(BN, KG, kp.nkb);
  if (kp.N % BN != 0 || (int64_t)KG * KPW < kp.nkb || lds > kLdsBytes || 64 * kp.K >= ((int64_t)1 << 32))
    return hipErrorNotSupported;
  kp.tiles_n = (int)(kp.N / BN);
  kp.tiles_m = (int)((kp.M + 63) / 64);
  const int64_t nwg = (int64_t)kp.G * kp.tiles_m * kp.tiles_n;
  if (nwg <= 0) return hipSuccess;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  kp.nwg = (int)nwg;
  const hipError_t attr = allow_full_lds<&gemm_decode2_kernel<BN, KG, KPW, NW, L, kPow2>>();
  if (attr != hipSuccess) return attr;
  gemm_decode2_kernel<BN, KG, KPW, NW, L, kPow2><<<dim3((unsigned)nwg), dim3(64 * NW), lds, s>>>(kp);
  return hipGetLastError();
}

template <int WM, int WN, int TN, int S, Layout L>
hipError_t run_decode3(KParams kp, hipStream_t s) {
  constexpr int BN = 16 * WN * TN, NW = WM * WN;
  const size_t lds = decode3_need(BN, S, kp.nkb);
  if (kp.N % BN != 0 || lds > kLdsBytes || 64 * kp.K >= ((int64_t)1 << 31) || kp.N * 64 >= ((int64_t)1 << 31))
    return hipErrorNotSupported;
  kp.tiles_n = (int)(kp.N / BN);
  kp.tiles_m = (int)((kp.M + 63) / 64);
  const int64_t nwg = (int64_t)kp.G * kp.tiles_m * kp.tiles_n;
  if (nwg <= 0) return hipSuccess;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  kp.nwg = (int)nwg;
  if (kp.pow2) {
    const hipError_t attr = allow_full_lds<&gemm_decode3_kernel<WM, WN, TN, S, L, true>>();
    if (attr != hipSuccess) return attr;
    gemm_decode3_kernel<WM, WN, TN, S, L, true><<<dim3((unsigned)nwg), dim3(64 * NW), lds, s>>>(kp);
  } else {
    const hipError_t attr = allow_full_lds<&gemm_decode3_kernel<WM, WN, TN, S, L, false>>();
    if (attr != hipSuccess) return attr;
    gemm_decode3_kernel<WM, WN, TN, S, L, false><<<dim3((unsigned)nwg), dim3(64 * NW), lds, s>>>(kp);
  }
  return hipGetLastError();
}

// Instantiated configurations of the activation-resident decode schedule: (wave rows, wave
// columns, column strips per wave, ring slots). DG_DECODE3="wm,wn,strips,slots" forces one
// (tuning, tests).
#define DG_DECODE3_CONFIGS(X) \
  X(2, 2, 3, 4) X(2, 2, 3, 5) X(1, 6, 1, 4) X(1, 6, 1, 5) X(2, 3, 2, 4) X(4, 1, 6, 4) X(1, 8, 1, 3) X(2, 4, 1, 3)

template <Layout L>
hipError_t run_decode3_cfg(int wm, int wn, int tn, int st, const KParams& kp, hipStream_t s) {
#define DG_X(a, b, c, d) \
  if (wm == a && wn == b && tn == c && st == d) return run_decode3<a, b, c, d, L>(kp, s);
  DG_DECODE3_CONFIGS(DG_X)
#undef DG_X
  return hipErrorNotSupported;
}

// The activation-resident decode schedule when it applies: the configuration from
// DG_DECODE3, else 96-column tiles (2 x 3 waves of 2 x 2 MFMA tiles, 4 ring slots: measured
// fastest of the instantiated ones on 64x24576x1536, 5% ahead of the 64x128 tile kernel) when
// N splits into enough of them to give every CU a workgroup. false leaves the choice to the
// caller.
template <Layout L>
bool try_decode3(const KParams& kp, hipStream_t s, const char** chosen, hipError_t* err) {
  static thread_local char name[48];
  int wm = 2, wn = 3, tn = 2, st = 4;
  const Tuning& t = tuning();
  if (t.decode3_ok) {
    wm = t.decode3[0]; wn = t.decode3[1]; tn = t.decode3[2]; st = t.decode3[3];
  } else {
    const int64_t rowblocks = (int64_t)kp.G * ((kp.M + 63) / 64);
    if (kp.N % 96 != 0 || rowblocks * (kp.N / 96) < 240) return false;
  }
  const hipError_t e = run_decode3_cfg<L>(wm, wn, tn, st, kp, s);
  if (e == hipErrorNotSupported) return false;
  *err = e;
  snprintf(name, sizeof name, "decode3_%dx%d_tn%d_s%d", wm, wn, tn, st);
  if (chosen) *chosen = name;
  return true;
}

// Instantiated configurations of the LDS decode schedule, in order of preference:
// (columns per workgroup, K-groups, K blocks per wave, waves). Wider workgroups read the
// activation block fewer times; the first one that covers K, divides N, fits LDS and
// leaves enough workgroups to cover the CUs is taken.
#define DG_DECODE2_CONFIGS(X) \
  X(128, 4, 3, 8) X(96, 4, 3, 8) X(96, 1, 12, 6) X(96, 2, 6, 6) X(64, 8, 2, 8) X(64, 8, 3, 8) X(32, 8, 2, 8) \
  X(32, 8, 3, 8) X(32, 2, 8, 4) X(32, 4, 4, 4) X(32, 1, 16, 2) X(16, 8, 2, 8) X(16, 8, 3, 8)

template <Layout L>
hipError_t run_decode2_cfg(int bn, int kg, int kpw, int nw, const KParams& kp, hipStream_t s) {
#define DG_X(a, b, c, d)                                                                     \
  if (bn == a && kg == b && kpw == c && nw == d)                                           \
    return kp.pow2 ? run_decode2<a, b, c, d, L, true>(kp, s) : run_decode2<a, b, c, d, L, false>(kp, s);
  DG_DECODE2_CONFIGS(DG_X)
#undef DG_X
  return hipErrorNotSupported;
}

// LDS decode schedule if some configuration applies; false leaves the choice to the caller.
template <Layout L>
bool try_decode2(const KParams& kp, hipStream_t s, const char** chosen, hipError_t* err) {
  static thread_local char name[48];
  struct C { int bn, kg, kpw, nw; };
  static const C cfgs[] = {
#define DG_X(a, b, c, d) {a, b, c, d},
      DG_DECODE2_CONFIGS(DG_X)
#undef DG_X
  };
  const int64_t rowblocks = (int64_t)kp.G * ((kp.M + 63) / 64);
  C c{0, 0, 0, 0};
  const Tuning& t = tuning();
  if (t.decode2_ok) {
    c = C{t.decode2[0], t.decode2[1], t.decode2[2], t.decode2[3]};
  } else {
    int64_t best = 0;
    for (const C& q : cfgs) {
      if ((int64_t)q.kg * q.kpw < kp.nkb || kp.N % q.bn != 0) continue;
      if (decode2_need(q.bn, q.kg, kp.nkb) > kLdsBytes) continue;
      const int64_t wgs = rowblocks * (kp.N / q.bn);
      if (wgs >= 200) { c = q; best = -1; break; }
      if (wgs > best) { best = wgs; c = q; }  // otherwise the most workgroups
    }
    if (c.bn == 0) return false;
  }
  const hipError_t e = run_decode2_cfg<L>(c.bn, c.kg, c.kpw, c.nw, kp, s);
  if (e == hipErrorNotSupported) return false;
  *err = e;
  snprintf(name, sizeof name, "decode2_bn%d_kg%d_kpw%d_w%d", c.bn, c.kg, c.kpw, c.nw);
  if (chosen) *chosen = name;
  return true;
}

template <Layout L>
hipError_t run_decode_auto(const KParams& kp, hipStream_t s, const char** chosen) {
  static thread_local char name[64];
  const Tuning& t = tuning();
  if (!t.decode_v1) {
    hipError_t e = hipSuccess;
    if (!t.decode2_set && try_decode3<L>(kp, s, chosen, &e)) return e;
    if (try_decode2<L>(kp, s, chosen, &e)) return e;
  }
  // register-fed schedule: one round per wave (all K blocks of a wave in flight at once);
  // among those, the first configuration (measured order: nkb 12 -> (48,4,3) or (32,4,3),
  // nkb 16 -> (32,8,2)) whose workgroup count covers the CUs
  struct C { int bn, nw, kpw; };
  static const C prefs[] = {{48, 4, 3}, {32, 4, 3}, {32, 8, 2}, {32, 4, 4}, {16, 8, 2}, {16, 4, 3}, {16, 4, 4}};
  const int64_t rowblocks = (int64_t)kp.G * ((kp.M + 63) / 64);
  C c{0, 0, 0};
  for (const C& q : prefs) {
    if (q.nw * q.kpw < kp.nkb || kp.N % q.bn != 0) continue;
    if (rowblocks * (kp.N / q.bn) < 200) continue;
    c = q;
    break;
  }
  if (c.bn == 0) c = rowblocks * (kp.N / 32) >= 200 ? C{32, 8, 2} : C{16, 8, 2};
  bool found = false;
  const hipError_t e = run_decode_cfg<L>(c.bn, c.nw, c.kpw, kp, s, &found);
  if (!found) return hipErrorInvalidValue;  // every entry of prefs is instantiated
  snprintf(name, sizeof name, "decode_bn%d_w%d_k%d", c.bn, c.nw, c.kpw);
  if (chosen) *chosen = name;
  return e;
}

}  // namespace

hipError_t launch_gemm(const GemmProblem& p, Schedule sched, int64_t expected_m, hipStream_t stream,
                       const char** chosen) {
  KParams kp{};
  kp.a = p.a; kp.sfa = p.sfa; kp.b = p.b; kp.sfb = p.sfb; kp.d = p.d;
  kp.m_indices = p.m_indices; kp.masked_m = p.masked_m;
  kp.M = p.M; kp.N = p.N; kp.K = p.K; kp.nkb = (int)(p.K / kQ); kp.G = p.G; kp.pow2 = p.pow2;

  if (sched == Schedule::Auto) {
    // dense M <= 64: the decode schedules, which take the activation-resident one (96-column
    // tiles) when N gives every CU a tile; otherwise 64x128 direct-load tiles when they make
    // enough workgroups to cover the chip (measured 5% faster than the LDS decode schedule on
    // 64x24576x1536), else the LDS decode schedule
    if (p.layout == Layout::Dense) {
      const bool d3 = p.N % 96 == 0 && p.N / 96 >= 240 && decode3_need(96, 4, kp.nkb) <= kLdsBytes;
      const Tuning& t = tuning();
      sched = p.M <= 64 ? (!d3 && p.N % 128 == 0 && p.N / 128 >= 160 && !t.decode_set && !t.decode2_set
                               ? Schedule::Tile64
                               : Schedule::Decode)
                        : (p.M >= 512 ? Schedule::Tile256 : Schedule::Tile128);
    }
    else if (p.layout == Layout::Masked)
      // the direct-load tiles at every count: at decode-sized counts they stream the weights
      // at 5-6.4 TB/s where the decode schedule (one 64-row block per workgroup, weights
      // re-streamed per block) reached 1.2-3.9 TB/s
      sched = Schedule::Tile256;
    else
      sched = Schedule::Tile128;
  }
  if (p.layout == Layout::Contiguous && sched != Schedule::Tile128) sched = Schedule::Tile128;

  // DG_TILE=<name> forces one of the tile kernels below where it applies (for tuning and
  // for tests that compare them)
  const char* force = tuning().tile[0] ? tuning().tile : nullptr;
  auto is = [&](const char* name) { return force && strcmp(force, name) == 0; };
  auto pick = [&](const char* name) { if (chosen) *chosen = name; };
  switch (p.layout) {
    case Layout::Dense:
      if (sched == Schedule::Decode) return run_decode_auto<Layout::Dense>(kp, stream, chosen);
      if (is("t2_256x128")) {
        pick("tile2_256x128");
        return run_tile2<256, 128, 4, 2, Layout::Dense>(kp, stream);
      }
      if (is("t2_128x128")) {
        pick("tile2_128x128");
        return run_tile2<128, 128, 2, 4, Layout::Dense>(kp, stream);
      }
      if (is("t3_256x128")) {
        pick("tile3_256x128");
        const hipError_t e = run_tile3<256, 128, 4, 2, 3, Layout::Dense>(kp, stream);
        if (e != hipErrorNotSupported) return e;
      }
      if (is("t3_128x256")) {
        pick("tile3_128x256");
        const hipError_t e = run_tile3<128, 256, 2, 4, 3, Layout::Dense>(kp, stream);
        if (e != hipErrorNotSupported) return e;
      }
      if (is("d3_96")) {  // the activation-resident decode kernel, where it fits
        pick("decode3_2x3_tn2_s4");
        const hipError_t e = run_decode3<2, 3, 2, 4, Layout::Dense>(kp, stream);
        if (e != hipErrorNotSupported) return e;
      }
      if (sched == Schedule::Tile64 || is("t3_64x128")) {
        pick("tile3_64x128");
        const hipError_t e = run_tile3<64, 128, 2, 4, 3, Layout::Dense>(kp, stream);
        if (e != hipErrorNotSupported) return e;
        if (sched == Schedule::Tile64) return run_decode_auto<Layout::Dense>(kp, stream, chosen);
      }
      if (sched == Schedule::Tile256 && is("t3_256x256b")) {  // the split issue (same sums; not faster here)
        pick("tile3_256x256_split");
        const hipError_t e = run_tile3<256, 256, 2, 4, 2, Layout::Dense, false, true>(kp, stream);
        if (e != hipErrorNotSupported) return e;
      }
      if (sched == Schedule::Tile256) {
        pick("tile3_256x256");
        const hipError_t e = run_tile3<256, 256, 2, 4, 2, Layout::Dense>(kp, stream);
        if (e != hipErrorNotSupported) return e;
        pick("tile2_256x128");
        return run_tile2<256, 128, 4, 2, Layout::Dense>(kp, stream);
      }
      if (!force && p.M > 64 && p.M < 512) {
        // skinny M: the largest direct-load tile that still gives about 3/4 of the CUs a
        // workgroup, else the one with the most workgroups (64 x 128). Measured on the decode
        // layers' shapes at M = 128 and 256: 1.5-1.7x faster than 128 x 128 register-staged
        // tiles where N / 128 is small (56 workgroups), equal where N is wide
        const int64_t tn128 = p.N / 128, tn256 = p.N % 256 == 0 ? p.N / 256 : 0;
        hipError_t e = hipErrorNotSupported;
        if (((p.M + 255) / 256) * tn128 >= 192) {
          pick("tile3_256x128");
          e = run_tile3<256, 128, 4, 2, 3, Layout::Dense>(kp, stream);
        } else if (((p.M + 127) / 128) * tn256 >= 192) {
          pick("tile3_128x256");
          e = run_tile3<128, 256, 2, 4, 3, Layout::Dense>(kp, stream);
        } else {
          pick("tile3_64x128");
          e = run_tile3<64, 128, 2, 4, 3, Layout::Dense>(kp, stream);
        }
        if (e != hipErrorNotSupported) return e;
      }
      pick("tile2_128x128");
      return run_tile2<128, 128, 2, 4, Layout::Dense>(kp, stream);
    case Layout::Masked:
      if (sched == Schedule::Decode) return run_decode_auto<Layout::Masked>(kp, stream, chosen);
      if (sched == Schedule::Tile256) {
        if (is("t2_256x128")) {
          pick("tile2_256x128");
          return run_tile2<256, 128, 4, 2, Layout::Masked>(kp, stream);
        }
        // 128-row tiles when most groups fit in one (each group's weights are then streamed
        // once, with two LDS stages of them in flight); 256-row tiles otherwise
        const bool small = p.M <= 128 || (expected_m > 0 && expected_m <= 64);
        if (is("t3_128x256b")) {
          pick("tile3_128x256_split");
          const hipError_t e = run_tile3<128, 256, 2, 4, 3, Layout::Masked, false, true>(kp, stream);
          if (e != hipErrorNotSupported) return e;
        }
        if (is("t3_128x256") || (!force && small)) {
          pick("tile3_128x256");
          const hipError_t e = run_tile3<128, 256, 2, 4, 3, Layout::Masked>(kp, stream);
          if (e != hipErrorNotSupported) return e;
        }
        if (is("t3_256x128")) {
          pick("tile3_256x128");
          const hipError_t e = run_tile3<256, 128, 4, 2, 3, Layout::Masked>(kp, stream);
          if (e != hipErrorNotSupported) return e;
        }
        // weights of K block kb+2 issued at the start of K block kb (split issue): measured 5%
        // faster than whole-stage refills on the HBM-bound masked shapes
        if (is("t3_256x256b")) {
          pick("tile3_256x256_split");
          const hipError_t e = run_tile3<256, 256, 2, 4, 2, Layout::Masked, false, true>(kp, stream);
          if (e != hipErrorNotSupported) return e;
        }
        {
          pick("masked_hybrid_128_256");
          const hipError_t e = run_masked_hybrid<false>(kp, stream);
          if (e != hipErrorNotSupported) return e;
        }
        pick("tile3_256x256_split");
        const hipError_t e = run_tile3<256, 256, 2, 4, 2, Layout::Masked, false, true>(kp, stream);
        if (e != hipErrorNotSupported) return e;
        pick("tile2_256x128");
        return run_tile2<256, 128, 4, 2, Layout::Masked>(kp, stream);
      }
      pick("tile2_128x128");
      return run_tile2<128, 128, 2, 4, Layout::Masked>(kp, stream);
    case Layout::Contiguous:
      // 256-row tiles over blocks of one expert, 128-row ones elsewhere, where the rounds of
      // workgroups allow it
      if ((!force && kp.N % 256 == 0 && contiguous_hybrid_pays(kp)) || is("hybrid")) {
        pick("contiguous_hybrid_128_256");
        const hipError_t e = run_contiguous_hybrid<false>(kp, stream);
        if (e != hipErrorNotSupported) return e;
      }
      // the three-stage direct-load ring pays off once K is long enough to fill it (measured:
      // 8% faster than the register-staged kernel at K = 2048)
      if (is("t3_128x256b")) {
        pick("tile3_128x256_split");
        const hipError_t e = run_tile3<128, 256, 2, 4, 3, Layout::Contiguous, false, true>(kp, stream);
        if (e != hipErrorNotSupported) return e;
      }
      if (is("t3_128x256") || (!force && kp.nkb >= 16)) {
        pick("tile3_128x256");
        const hipError_t e = run_tile3<128, 256, 2, 4, 3, Layout::Contiguous>(kp, stream);
        if (e != hipErrorNotSupported) return e;
      }
      if (kp.N % 256 == 0 && !is("t2_128x128")) {
        pick("tile2_128x256");
        return run_tile2<128, 256, 2, 4, Layout::Contiguous>(kp, stream);
      }
      pick("tile2_128x128");
      return run_tile2<128, 128, 2, 4, Layout::Contiguous>(kp, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_swiglu(const GemmProblem& p, uint8_t* hq, float* sh, int64_t expected_m, hipStream_t stream,
                              const char** chosen) {
  KParams kp{};
  kp.a = p.a; kp.sfa = p.sfa; kp.b = p.b; kp.sfb = p.sfb; kp.d = nullptr;
  kp.m_indices = p.m_indices; kp.masked_m = p.masked_m;
  kp.M = p.M; kp.N = p.N; kp.K = p.K; kp.nkb = (int)(p.K / kQ); kp.G = p.G; kp.pow2 = p.pow2;
  kp.hq = hq; kp.sh = sh;
  const char* force = tuning().tile[0] ? tuning().tile : nullptr;
  auto is = [&](const char* name) { return force && strcmp(force, name) == 0; };
  auto pick = [&](const char* name) { if (chosen) *chosen = name; };
  switch (p.layout) {
    case Layout::Contiguous:
      if (is("t3_128x256b")) {
        pick("tile3_swiglu_128x256_split");
        return run_tile3<128, 256, 2, 4, 3, Layout::Contiguous, true, true>(kp, stream);
      }
      if (is("hybrid") || (!force && contiguous_hybrid_pays(kp))) {
        pick("contiguous_hybrid_swiglu_128_256");
        return run_contiguous_hybrid<true>(kp, stream);
      }
      pick("tile3_swiglu_128x256");
      return run_tile3<128, 256, 2, 4, 3, Layout::Contiguous, true>(kp, stream);
    case Layout::Masked:
      if (is("t3_128x256b")) {
        pick("tile3_swiglu_128x256_split");
        return run_tile3<128, 256, 2, 4, 3, Layout::Masked, true, true>(kp, stream);
      }
      if (is("t3_128x256") || (!force && (p.M <= 128 || (expected_m > 0 && expected_m <= 64)))) {
        pick("tile3_swiglu_128x256");
        return run_tile3<128, 256, 2, 4, 3, Layout::Masked, true>(kp, stream);
      }
      if (is("t3_256x256b")) {
        pick("tile3_swiglu_256x256_split");
        return run_tile3<256, 256, 2, 4, 2, Layout::Masked, true, true>(kp, stream);
      }
      pick("masked_hybrid_swiglu_128_256");
      return run_masked_hybrid<true>(kp, stream);
    case Layout::Dense:
      (void)is;
      pick("tile3_swiglu_128x256");
      return run_tile3<128, 256, 2, 4, 3, Layout::Dense, true>(kp, stream);
  }
  return hipErrorInvalidValue;
}

void reload_tuning_switches() {
  std::lock_guard<std::mutex> lock(g_tuning_mu);
  g_tuning.store(new Tuning(read_tuning()), std::memory_order_release);
}

bool log_switch() { return tuning().log; }

}  // namespace dg
