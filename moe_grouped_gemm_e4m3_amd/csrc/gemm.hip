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
};

__device__ __forceinline__ int64_t clamp_rows(int64_t v, int64_t hi) { return v < 0 ? 0 : (v > hi ? hi : v); }

// 32 bytes of one operand row for MFMA lane group (l >> 4): two 16-byte global loads.
__device__ __forceinline__ v8i load_frag_global(const uint8_t* p) {
  const v4i lo = *reinterpret_cast<const v4i*>(p);
  const v4i hi = *reinterpret_cast<const v4i*>(p + 16);
  return cat8(lo, hi);
}

// ---------------------------------------------------------------------------------
// decode schedule
// ---------------------------------------------------------------------------------
template <int BN, int NW, Layout L>
__global__ __launch_bounds__(64 * NW) void gemm_decode_kernel(KParams p) {
  static_assert(L != Layout::Contiguous, "decode schedule serves dense and masked layouts");
  static_assert(BN % 16 == 0 && kQ % BN == 0, "tile must sit inside one weight-scale block");
  constexpr int TN = BN / 16;
  __shared__ __attribute__((aligned(16))) float red[NW][64 * BN];
  __shared__ __attribute__((aligned(16))) float sa_x[NW][64];

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
  const float* SB = p.sfb + ((int64_t)g * (p.N / kQ) + n0 / kQ) * nkb;
  uint16_t* D = p.d + (int64_t)g * p.M * p.N;

  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int kof = (l >> 4) * 32;
  const uint8_t* arow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) arow[i] = A + clamp_rows(m0 + 16 * i + (l & 15), valid - 1) * K + kof;
  const uint8_t* brow[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) brow[j] = B + (n0 + 16 * j + (l & 15)) * K + kof;
  const float* sarow = SA + clamp_rows(m0 + l, valid - 1) * nkb;
  float* my_sa = sa_x[w];

  v4f acc[4][TN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  v8i af[4], bf[TN];
  float sam = 0.f, sbv = 0.f;
  int kb = w;
  if (kb < nkb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = load_frag_global(arow[i] + (int64_t)kb * kQ);
#pragma unroll
    for (int j = 0; j < TN; ++j) bf[j] = load_frag_global(brow[j] + (int64_t)kb * kQ);
    sam = sarow[kb];
    sbv = SB[kb];
  }
  while (kb < nkb) {
    const int kn = kb + NW;
    v8i af2[4], bf2[TN];
    float sam2 = 0.f, sbv2 = 0.f;
    if (kn < nkb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) af2[i] = load_frag_global(arow[i] + (int64_t)kn * kQ);
#pragma unroll
      for (int j = 0; j < TN; ++j) bf2[j] = load_frag_global(brow[j] + (int64_t)kn * kQ);
      sam2 = sarow[kn];
      sbv2 = SB[kn];
    }
    // this lane's 4 output rows of strip i are 16*i + 4*(l>>4) + r: fetch their
    // activation scales through the wave's private LDS slot
    my_sa[l] = sam;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 s4 = *reinterpret_cast<const float4*>(&my_sa[16 * i + 4 * (l >> 4)]);
      const float t0 = s4.x * sbv, t1 = s4.y * sbv, t2 = s4.z * sbv, t3 = s4.w * sbv;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const v4f pp = mfma_f8_16x16x128(af[i], bf[j]);
        acc[i][j][0] = fmaf(pp[0], t0, acc[i][j][0]);
        acc[i][j][1] = fmaf(pp[1], t1, acc[i][j][1]);
        acc[i][j][2] = fmaf(pp[2], t2, acc[i][j][2]);
        acc[i][j][3] = fmaf(pp[3], t3, acc[i][j][3]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = af2[i];
#pragma unroll
    for (int j = 0; j < TN; ++j) bf[j] = bf2[j];
    sam = sam2;
    sbv = sbv2;
    kb = kn;
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
// tile schedule
// ---------------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, Layout L>
__global__ __launch_bounds__(64 * WM * WN) void gemm_tile_kernel(KParams p) {
  constexpr int NT = 64 * WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 16, TN = WTN / 16;
  constexpr int ACH = BM * 8 / NT;  // 16-byte chunks of an A K-block per thread
  constexpr int BCH = BN * 8 / NT;
  static_assert(ACH * NT == BM * 8 && BCH * NT == BN * 8, "chunk split");
  static_assert(kQ % BN == 0, "tile must sit inside one weight-scale block column");
  static_assert(L != Layout::Contiguous || BM == kQ, "contiguous layout: one expert per M tile");
  static_assert(BM <= NT, "one activation scale per thread");
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * kQ];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * kQ];
  __shared__ __attribute__((aligned(16))) float sSa[2][BM];

  const uint32_t wg = xcd_remap(blockIdx.x, (uint32_t)p.nwg);
  int g = 0, tm, tn;
  if constexpr (L == Layout::Masked) {
    // m-tiles of one (group, n-tile) are adjacent, so they meet the same B tile in L2
    tm = (int)(wg % (uint32_t)p.tiles_m);
    tn = (int)((wg / (uint32_t)p.tiles_m) % (uint32_t)p.tiles_n);
    g = (int)(wg / (uint32_t)(p.tiles_m * p.tiles_n));
  } else {
    // raster in bands of 8 m-tiles: n advances after each band column
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
    if (m0 >= valid) return;  // uniform over the workgroup
  }
  if constexpr (L == Layout::Contiguous) {
    g = p.m_indices[m0];
    if (g < 0 || g >= p.G) return;  // padding block (or an id outside the groups)
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

  // global -> LDS staging assignment: chunk c = t + NT*u is row c/8, 16-byte column c%8
  const uint8_t* ga[ACH];
  uint32_t la[ACH];
#pragma unroll
  for (int u = 0; u < ACH; ++u) {
    const int c = t + NT * u, row = c >> 3, ch = c & 7;
    ga[u] = A + clamp_rows(m0 + row, valid - 1) * K + ch * 16;
    la[u] = row * kQ + ((ch ^ (row & 7)) << 4);
  }
  const uint8_t* gb[BCH];
  uint32_t lb[BCH];
#pragma unroll
  for (int u = 0; u < BCH; ++u) {
    const int c = t + NT * u, row = c >> 3, ch = c & 7;
    gb[u] = B + (n0 + row) * K + ch * 16;
    lb[u] = row * kQ + ((ch ^ (row & 7)) << 4);
  }
  const float* gsa = SA + clamp_rows(m0 + (t < BM ? t : 0), valid - 1) * nkb;

  v4i ra[ACH], rb[BCH];
  float rsa = 0.f;
  auto gload = [&](int kb) {
#pragma unroll
    for (int u = 0; u < ACH; ++u) ra[u] = *reinterpret_cast<const v4i*>(ga[u] + (int64_t)kb * kQ);
#pragma unroll
    for (int u = 0; u < BCH; ++u) rb[u] = *reinterpret_cast<const v4i*>(gb[u] + (int64_t)kb * kQ);
    if (t < BM) rsa = gsa[kb];
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < ACH; ++u) *reinterpret_cast<v4i*>(&sA[buf][la[u]]) = ra[u];
#pragma unroll
    for (int u = 0; u < BCH; ++u) *reinterpret_cast<v4i*>(&sB[buf][lb[u]]) = rb[u];
    if (t < BM) sSa[buf][t] = rsa;
  };

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // fragment read offsets (swizzled 16-byte columns 2*(l>>4) and 2*(l>>4)+1)
  const int fr = l & 15;
  const int c0 = 2 * (l >> 4), c1 = c0 + 1;

  gload(0);
  lstore(0);
  __syncthreads();
  float sb = SB[0];
  for (int kb = 0; kb < nkb; ++kb) {
    const int cur = kb & 1;
    float sb_next = 0.f;
    if (kb + 1 < nkb) {
      gload(kb + 1);
      sb_next = SB[kb + 1];
    }
    const uint8_t* a_s = sA[cur];
    const uint8_t* b_s = sB[cur];
    v8i bfr[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int row = wn * WTN + 16 * j + fr;
      const uint8_t* base = b_s + row * kQ;
      bfr[j] = cat8(*reinterpret_cast<const v4i*>(base + ((c0 ^ (row & 7)) << 4)),
                    *reinterpret_cast<const v4i*>(base + ((c1 ^ (row & 7)) << 4)));
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = wm * WTM + 16 * i + fr;
      const uint8_t* base = a_s + row * kQ;
      const v8i afr = cat8(*reinterpret_cast<const v4i*>(base + ((c0 ^ (row & 7)) << 4)),
                           *reinterpret_cast<const v4i*>(base + ((c1 ^ (row & 7)) << 4)));
      const float4 s4 = *reinterpret_cast<const float4*>(&sSa[cur][wm * WTM + 16 * i + 4 * (l >> 4)]);
      const float t0 = s4.x * sb, t1 = s4.y * sb, t2 = s4.z * sb, t3 = s4.w * sb;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const v4f pp = mfma_f8_16x16x128(afr, bfr[j]);
        acc[i][j][0] = fmaf(pp[0], t0, acc[i][j][0]);
        acc[i][j][1] = fmaf(pp[1], t1, acc[i][j][1]);
        acc[i][j][2] = fmaf(pp[2], t2, acc[i][j][2]);
        acc[i][j][3] = fmaf(pp[3], t3, acc[i][j][3]);
      }
    }
    if (kb + 1 < nkb) lstore(cur ^ 1);
    sb = sb_next;
    __syncthreads();
  }

  // epilogue: bf16 round-to-nearest-even, rows beyond the valid count are not written
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = m0 + wm * WTM + 16 * i + 4 * (l >> 4) + r;
      if (row < valid) {
        uint16_t* drow = D + row * p.N + n0 + wn * WTN + fr;
#pragma unroll
        for (int j = 0; j < TN; ++j) drow[16 * j] = (uint16_t)bf16_rne(acc[i][j][r]);
      }
    }
  }
}

template <int BN, int NW, Layout L>
hipError_t run_decode(KParams kp, hipStream_t s) {
  kp.tiles_n = (int)(kp.N / BN);
  kp.tiles_m = (int)((kp.M + 63) / 64);
  const int64_t nwg = (int64_t)kp.G * kp.tiles_m * kp.tiles_n;
  if (nwg <= 0) return hipSuccess;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  kp.nwg = (int)nwg;
  gemm_decode_kernel<BN, NW, L><<<dim3((unsigned)nwg), dim3(64 * NW), 0, s>>>(kp);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, Layout L>
hipError_t run_tile(KParams kp, hipStream_t s) {
  kp.tiles_n = (int)(kp.N / BN);
  kp.tiles_m = (int)((kp.M + BM - 1) / BM);
  const int64_t nwg = (int64_t)(L == Layout::Masked ? kp.G : 1) * kp.tiles_m * kp.tiles_n;
  if (nwg <= 0) return hipSuccess;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  kp.nwg = (int)nwg;
  gemm_tile_kernel<BM, BN, WM, WN, L><<<dim3((unsigned)nwg), dim3(64 * WM * WN), 0, s>>>(kp);
  return hipGetLastError();
}

template <Layout L>
hipError_t run_decode_auto(const KParams& kp, hipStream_t s, const char** chosen) {
  // Enough workgroups to cover the 256 CUs twice: prefer the widest column tile that
  // still yields >= 512 workgroups; split K over 8 waves when there are >= 16 K blocks.
  const int64_t rowblocks = (int64_t)kp.G * ((kp.M + 63) / 64);
  const bool eight = kp.nkb >= 16;
  if (rowblocks * (kp.N / 64) >= 512) {
    if (chosen) *chosen = eight ? "decode_bn64_w8" : "decode_bn64_w4";
    return eight ? run_decode<64, 8, L>(kp, s) : run_decode<64, 4, L>(kp, s);
  }
  if (rowblocks * (kp.N / 32) >= 512) {
    if (chosen) *chosen = eight ? "decode_bn32_w8" : "decode_bn32_w4";
    return eight ? run_decode<32, 8, L>(kp, s) : run_decode<32, 4, L>(kp, s);
  }
  if (chosen) *chosen = eight ? "decode_bn16_w8" : "decode_bn16_w4";
  return eight ? run_decode<16, 8, L>(kp, s) : run_decode<16, 4, L>(kp, s);
}

}  // namespace

hipError_t launch_gemm(const GemmProblem& p, Schedule sched, int64_t expected_m, hipStream_t stream,
                       const char** chosen) {
  KParams kp{};
  kp.a = p.a; kp.sfa = p.sfa; kp.b = p.b; kp.sfb = p.sfb; kp.d = p.d;
  kp.m_indices = p.m_indices; kp.masked_m = p.masked_m;
  kp.M = p.M; kp.N = p.N; kp.K = p.K; kp.nkb = (int)(p.K / kQ); kp.G = p.G;

  if (sched == Schedule::Auto) {
    if (p.layout == Layout::Dense)
      sched = p.M <= 64 ? Schedule::Decode : Schedule::Tile128;
    else if (p.layout == Layout::Masked)
      sched = (expected_m > 0 && expected_m <= 64) ? Schedule::Decode : Schedule::Tile128;
    else
      sched = Schedule::Tile128;
  }
  if (p.layout == Layout::Contiguous && sched != Schedule::Tile128) sched = Schedule::Tile128;

  switch (p.layout) {
    case Layout::Dense:
      if (sched == Schedule::Decode) return run_decode_auto<Layout::Dense>(kp, stream, chosen);
      if (sched == Schedule::Tile256) {
        if (chosen) *chosen = "tile_256x128";
        return run_tile<256, 128, 4, 2, Layout::Dense>(kp, stream);
      }
      if (chosen) *chosen = "tile_128x128";
      return run_tile<128, 128, 2, 2, Layout::Dense>(kp, stream);
    case Layout::Masked:
      if (sched == Schedule::Decode) return run_decode_auto<Layout::Masked>(kp, stream, chosen);
      if (sched == Schedule::Tile256) {
        if (chosen) *chosen = "tile_256x128";
        return run_tile<256, 128, 4, 2, Layout::Masked>(kp, stream);
      }
      if (chosen) *chosen = "tile_128x128";
      return run_tile<128, 128, 2, 2, Layout::Masked>(kp, stream);
    case Layout::Contiguous:
      if (chosen) *chosen = "tile_128x128";
      return run_tile<128, 128, 2, 2, Layout::Contiguous>(kp, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace dg
