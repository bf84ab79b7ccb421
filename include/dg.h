/*
 * dg.h - C ABI of the FP8 (e4m3) block-scaled GEMM library for MI355X (gfx950).
 *
 * The method (DeepGEMM-style fine-grained FP8 scaling):
 *   - activations: FP8 e4m3 with one fp32 scale per token per 128 consecutive K
 *     elements ("1x128"); weights: FP8 e4m3 with one fp32 scale per 128x128 block.
 *     DeepGEMM article, section "FP8 and fine-grained scaling" (activations scaled per
 *     slice, weights per matrix block, accumulation kept in higher precision);
 *     DeepSeek-V3 repo review, "Innovations" item 4 (one scale per 128 elements) and
 *     "Solution philosophy" (128x128 block scaling).
 *   - the GEMM multiplies within each 128-wide K block on FP8 matrix hardware, then
 *     promotes the partial sum to fp32, multiplies it by scale_a * scale_b and
 *     accumulates: DeepGEMM launch write-up, "Built for modern AI compute" (two-level
 *     accumulation) and "Deployment guide" (promotion outside the matrix units).
 *   - normal (dense) GEMM plus MoE grouped GEMM in a contiguous layout (groups stacked
 *     along M) and a masked layout (per-group valid-row count, the format a
 *     communication library hands over): DeepGEMM article, section "~300-line JIT
 *     core"; DeepGEMM launch write-up, "Performance" (the three table headings).
 *   - quantisation bound 448 (OCP E4M3FN max finite): DeepSeek-V3 repo review,
 *     "Risks and shortcomings" item 6.
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is DEVICE memory owned by the caller, contiguous, row-major,
 *     and 16-byte aligned. The library never allocates, frees or keeps a pointer.
 *   - Activation scales (sfa) are stored K-block-major: [K/128][M], i.e. for each
 *     128-wide K block the scales of all M rows are contiguous (with a leading [G] for
 *     the masked layout). This is NOT the row-major [M][K/128] layout a reader might
 *     assume: both have M*K/128 elements, so a caller that passes row-major scales gets
 *     wrong results with no error (the library cannot tell them apart). The pages leave
 *     the layout open. K-block-major lets a GEMM tile fetch the scales of its rows for one
 *     K block as one contiguous run of cache lines; stored row-major, the 32 scales one
 *     wave needs per K block lay in 32 different lines, which cost about a third of the
 *     prefill kernel's load time. The per-token cast writes this layout directly (its G
 *     argument gives the masked layout's [G][K/128][M_max]). Weight scales (sfb) are
 *     [N/128][K/128].
 *   - FP8 tensors are raw OCP E4M3FN bytes (uint8_t); bf16 tensors are raw uint16_t bits.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Calls only
 *     enqueue work on it and return without synchronising; inputs must stay alive
 *     until the stream has run the work.
 *   - "NT": A is [M,K] and B is [N,K], both K-major, and D = A * B^T.
 *   - K and N must be multiples of 128. M may be any value >= 0.
 *   - Arguments the host can see are validated before anything is enqueued. On an error
 *     nothing is launched, outputs are untouched, and the status says why;
 *     dg_last_error_message() gives a thread-local detail string.
 *   - Empty problems (M = 0, G = 0) enqueue nothing and return DG_OK.
 *   - Device-resident metadata (m_indices, masked_m) is not validated on the host; see
 *     each entry point.
 *   - Calls are thread-safe; the only shared state is a once-initialised record of the
 *     current device's architecture.
 */
#ifndef DG_H
#define DG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DG_OK = 0,
  DG_ERR_INVALID_ARGUMENT = 1,  /* null pointer, negative size, unknown dtype */
  DG_ERR_UNSUPPORTED_SHAPE = 2, /* K or N not a multiple of 128, M_total not a multiple of 128 */
  DG_ERR_MISALIGNED = 3,        /* a pointer not 16-byte aligned */
  DG_ERR_UNSUPPORTED_DEVICE = 4, /* current device is not gfx950, or no device */
  DG_ERR_LAUNCH = 5             /* the kernel launch failed */
} dg_status_t;

typedef enum { DG_INPUT_F32 = 0, DG_INPUT_BF16 = 1 } dg_input_dtype_t;

/* Scale format of a GEMM call: any fp32 values, or powers of two (UE8M0, see below). */
typedef enum { DG_SCALE_F32 = 0, DG_SCALE_UE8M0 = 1 } dg_scale_format_t;

/*
 * Per-token FP8 cast of activations (DeepSeek-V3 repo review, "Innovations" item 4:
 * one scale per 128 elements; "Risks" item 6: bound 448).
 *   x  [G,M,K]  fp32 or bf16 (x_dtype), finite values; G = 1 for a plain [M,K] tensor.
 *   q  [G,M,K]  e4m3 bytes (output).
 *   sf [G,K/128,M] fp32 scales (output), K-block-major: sf[g][j][m] is the scale of
 *      row m, chunk j of group g. G = 1 gives the sfa of the dense and contiguous GEMMs,
 *      G groups of M_max rows the sfa of the masked GEMM.
 * For each row m and chunk j = columns [128j, 128j+128):
 *   amax = max |x|; s = amax / 448 (correctly rounded fp32 division);
 *   q = e4m3(x / s) with correctly rounded division, round-to-nearest-even, saturation
 *   to +-448, the sign of zero kept; if s == 0 the chunk gets s = 0 and signed zeros.
 * Requires K % 128 == 0, G >= 0, G*M < 2^31.
 */
dg_status_t dg_cast_fp8_per_token(const void* x, dg_input_dtype_t x_dtype, int64_t G, int64_t M,
                                  int64_t K, uint8_t* q, float* sf, void* stream);

/*
 * The per-token cast of the masked layout's activations, valid rows only: x, q, sf as above
 * with G groups of M_max rows; of group g only rows m < masked_m[g] (clamped to [0, M_max])
 * are cast, the others' codes and scales are not written. Those are exactly the rows the
 * masked grouped GEMM reads (it never reads an activation row at or beyond masked_m[g]), so
 * in a masked layer this cast does the same job with the padding rows skipped.
 *   scale_fmt: DG_SCALE_F32 (the rule above) or DG_SCALE_UE8M0 (dg_cast_fp8_per_token_ue8m0).
 *   masked_m: [G] int32, device, 16-byte aligned (read on the device).
 * Same requirements and errors as dg_cast_fp8_per_token.
 */
dg_status_t dg_cast_fp8_per_token_masked(const void* x, dg_input_dtype_t x_dtype, int32_t scale_fmt, int32_t G,
                                         int64_t M_max, int64_t K, const int32_t* masked_m, uint8_t* q, float* sf,
                                         void* stream);

/*
 * Per-block FP8 cast of weights: the same rule as above with the amax taken over each
 * 128x128 block (DeepSeek-V3 repo review, "Solution philosophy": 128x128 block scaling).
 *   w  [N,K] fp32 or bf16; q [N,K] e4m3 (output); sf [N/128, K/128] fp32 (output).
 * Requires N % 128 == 0 and K % 128 == 0. For a grouped weight tensor [G,N,K] pass
 * N' = G*N (blocks never straddle groups because N % 128 == 0).
 */
dg_status_t dg_cast_fp8_per_block(const void* w, dg_input_dtype_t w_dtype, int64_t N, int64_t K,
                                  uint8_t* q, float* sf, void* stream);

/*
 * Dense FP8 GEMM with fine-grained scaling (DeepGEMM article, "~300-line JIT core";
 * launch write-up, "Performance": normal GEMM for dense models).
 *   a   [M,K] e4m3,      sfa [K/128, M] fp32 (per-token scales, K-block-major)
 *   b   [N,K] e4m3,      sfb [N/128, K/128] fp32 (block scales)
 *   d   [M,N] bf16 (output):
 *   d[m,n] = bf16_rne( sum_kb  P_kb[m,n] * sfa[kb,m] * sfb[n/128,kb] ),
 *   P_kb = the FP8 product sum over K block kb, promoted to fp32 once per block.
 * Requires N % 128 == 0, K % 128 == 0.
 */
dg_status_t dg_gemm_fp8_nt(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                           uint16_t* d, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * MoE grouped GEMM, contiguous layout (DeepGEMM article, "~300-line JIT core": groups
 * formed dynamically along M; launch write-up, "Performance": contiguous layout).
 *   a [M_total,K] e4m3, sfa [K/128,M_total]; b [G,N,K] e4m3, sfb [G,N/128,K/128];
 *   m_indices [M_total] int32 (device): expert id of each row, or -1 for padding;
 *   d [M_total,N] bf16 (output).
 * Each aligned 128-row block belongs to one expert: the expert of the block's first row.
 * A block whose first row is -1 is skipped (its rows of d are left untouched). Rows
 * marked -1 inside a computed block get unspecified values. Values outside [-1, G) and
 * blocks mixing experts are undefined behaviour (not checked on the device).
 * Requires M_total % 128 == 0, N % 128 == 0, K % 128 == 0, G >= 1.
 */
dg_status_t dg_grouped_gemm_contiguous(const uint8_t* a, const float* sfa, const uint8_t* b,
                                       const float* sfb, const int32_t* m_indices, uint16_t* d,
                                       int32_t G, int64_t M_total, int64_t N, int64_t K,
                                       void* stream);

/*
 * MoE grouped GEMM, masked layout (DeepGEMM article, "~300-line JIT core": the masked
 * layout interfaces with the communication library; launch write-up, "Performance").
 *   a [G,M_max,K] e4m3, sfa [G,K/128,M_max]; b [G,N,K] e4m3, sfb [G,N/128,K/128];
 *   masked_m [G] int32 (device): valid rows of each group, clamped to [0, M_max];
 *   d [G,M_max,N] bf16 (output).
 * Rows r < masked_m[g] of group g are computed; rows r >= masked_m[g] are not written.
 * expected_m is a host-side hint of the typical masked_m (0 = unknown) that only selects
 * the kernel schedule; results do not depend on it.
 * Requires N % 128 == 0, K % 128 == 0, G >= 0, M_max >= 0.
 */
dg_status_t dg_grouped_gemm_masked(const uint8_t* a, const float* sfa, const uint8_t* b,
                                   const float* sfb, const int32_t* masked_m, uint16_t* d,
                                   int32_t G, int64_t M_max, int64_t N, int64_t K,
                                   int64_t expected_m, void* stream);

/*
 * Power-of-two (UE8M0) scales (DeepSeek-V3 repo review, "Innovations" item 4: V3.1's UE8M0
 * format rounds every scale to a power of two, so that applying it is a shift).
 *   The _ue8m0 casts are the casts above with s = the smallest power of two not below
 *   fp32(amax / 448), and at least 2^-126; x / s is then exact. Same arguments, layouts
 *   and errors; the scales are stored as fp32 (exact powers of two).
 *   The _ue8m0 GEMMs compute the same D as the GEMMs above, with the same arguments,
 *   layouts and errors, under the precondition that every sfa and sfb value is a power of
 *   two in [2^-126, 2^127] (what the _ue8m0 casts produce). Where the shape allows, gfx950's
 *   block-scaled MFMA then applies the scales itself and the products accumulate in its
 *   fp32 accumulator, with no promotion on the vector ALUs. A scale that is not a power of
 *   two gives unspecified output (not checked on the device).
 */
dg_status_t dg_cast_fp8_per_token_ue8m0(const void* x, dg_input_dtype_t x_dtype, int64_t G, int64_t M,
                                        int64_t K, uint8_t* q, float* sf, void* stream);
dg_status_t dg_cast_fp8_per_block_ue8m0(const void* w, dg_input_dtype_t w_dtype, int64_t N, int64_t K,
                                        uint8_t* q, float* sf, void* stream);
dg_status_t dg_gemm_fp8_nt_ue8m0(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                                 uint16_t* d, int64_t M, int64_t N, int64_t K, void* stream);
dg_status_t dg_grouped_gemm_contiguous_ue8m0(const uint8_t* a, const float* sfa, const uint8_t* b,
                                             const float* sfb, const int32_t* m_indices, uint16_t* d,
                                             int32_t G, int64_t M_total, int64_t N, int64_t K, void* stream);
dg_status_t dg_grouped_gemm_masked_ue8m0(const uint8_t* a, const float* sfa, const uint8_t* b,
                                         const float* sfb, const int32_t* masked_m, uint16_t* d, int32_t G,
                                         int64_t M_max, int64_t N, int64_t K, int64_t expected_m,
                                         void* stream);

/*
 * The GEMMs above with the kernel schedule chosen by the caller (for tuning and for tests
 * that must cover every schedule on the same problem). Same math, same arguments and same
 * validation as the named entry points.
 *   layout:   0 = dense (meta ignored, G ignored), 1 = contiguous (meta = m_indices),
 *             2 = masked (meta = masked_m).
 *   scale_fmt: DG_SCALE_F32, or DG_SCALE_UE8M0 with the precondition of the _ue8m0 GEMMs.
 *   schedule: 0 = automatic (what the named entry points use), 1 = decode (64-row
 *             blocks, K split over the waves of a workgroup; dense and masked only),
 *             2 = 128x128 LDS-staged tiles, 3 = 256x128 LDS-staged tiles (dense and
 *             masked only). A schedule a layout does not support falls back to 2.
 */
dg_status_t dg_gemm_fp8_scheduled(int32_t layout, int32_t schedule, int32_t scale_fmt, const uint8_t* a,
                                  const float* sfa, const uint8_t* b, const float* sfb, const int32_t* meta,
                                  uint16_t* d, int32_t G, int64_t M, int64_t N, int64_t K,
                                  int64_t expected_m, void* stream);

/*
 * Gate/up GEMM of an MoE expert FFN with the SwiGLU activation and the per-token FP8
 * re-cast fused into its epilogue (DeepGEMM article, section "swapAB and Mega MoE": the
 * expert FFN's two GEMMs and its SwiGLU activation in one fused kernel; this is the
 * single-GPU part, without the network transfer).
 *   layout:    0 = dense (meta ignored, G ignored), 1 = contiguous (meta = m_indices),
 *              2 = masked (meta = masked_m), with the row rules of the GEMMs above.
 *   scale_fmt: DG_SCALE_F32, or DG_SCALE_UE8M0 (every sfa / sfb a power of two; the h
 *              scales are then powers of two as well, as in the _ue8m0 casts).
 *   a   [rows,K] e4m3 with sfa [K/128,rows] (masked: [G,M_max,K], [G,K/128,M_max]);
 *   b   [G,2I,K] e4m3 with sfb [G,2I/128,K/128]: rows [0,I) of each group are the gate
 *       projection, rows [I,2I) the up projection;
 *   hq  [rows,I] e4m3 (output; masked [G,M_max,I]);
 *   sfh [I/128,rows] fp32 (output, K-block-major like every activation scale; masked
 *       [G,I/128,M_max]): hq and sfh are exactly the operands the down GEMM takes.
 * With gate/up = the fp32 GEMM result of the two halves of b (computed as in the GEMMs
 * above, without the bf16 rounding):
 *   h = silu(gate) * up, silu(x) = x / (1 + exp(-x)), evaluated in fp32;
 *   per row and per 128-column block of h: s = amax|h| / 448 (UE8M0: its power of two),
 *   q = e4m3(h / s), the rule of dg_cast_fp8_per_token.
 * Rows that are not computed (masked rows >= masked_m, contiguous blocks that start with
 * -1) are not written. Requires I % 128 == 0, K % 128 == 0, K <= 32768, rows*K < 2^32 and
 * 2*I*K < 2^32 (per group), M_total % 128 == 0 for the contiguous layout.
 */
dg_status_t dg_gemm_fp8_swiglu(int32_t layout, int32_t scale_fmt, const uint8_t* a, const float* sfa,
                               const uint8_t* b, const float* sfb, const int32_t* meta, uint8_t* hq,
                               float* sfh, int32_t G, int64_t M, int64_t I, int64_t K, int64_t expected_m,
                               void* stream);

/*
 * MoE expert FFN (DeepGEMM article, section "swapAB and Mega MoE"):
 *   y = down( SwiGLU( gate/up(x) ) ), the two grouped GEMMs with the activation and the
 *   FP8 re-cast between them fused into the first one (dg_gemm_fp8_swiglu), then the
 *   grouped GEMM of the same layout on (hq, sfh) with w2.
 *   x [rows,H] e4m3 with sfx [H/128,rows] (masked: [G,M_max,H], [G,H/128,M_max]);
 *   w1 [G,2I,H] with sfw1 [G,2I/128,H/128] (gate rows, then up rows);
 *   w2 [G,H,I] with sfw2 [G,H/128,I/128];
 *   hq, sfh: caller-provided workspace for the FP8 activation between the GEMMs, shaped
 *       as the outputs of dg_gemm_fp8_swiglu (they hold it when the stream has run);
 *   y [rows,H] bf16 (output; masked [G,M_max,H]).
 * Both launches go to `stream` in order. Every argument of both GEMMs is validated before
 * either is launched; the requirements are those of dg_gemm_fp8_swiglu plus H % 128 == 0.
 */
dg_status_t dg_moe_ffn_fp8(int32_t layout, int32_t scale_fmt, const uint8_t* x, const float* sfx,
                           const uint8_t* w1, const float* sfw1, const uint8_t* w2, const float* sfw2,
                           const int32_t* meta, uint8_t* hq, float* sfh, uint16_t* y, int32_t G, int64_t M,
                           int64_t H, int64_t I, int64_t expected_m, void* stream);

/*
 * dg_moe_ffn_fp8 for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same two launches,
 * the same arguments minus hq and sfh, and the same results. The FP8 activation between the
 * GEMMs lives in a static device array of the library instead of a caller workspace.
 *   - The array holds 32 MiB (33554432 bytes) on every GPU the library runs on, from the
 *     first call on that GPU until the process ends. A call needs rows*I bytes (rounded up to
 *     256) plus 4*rows*I/128 bytes of scales, rows = M (masked: G*M_max); larger calls return
 *     DG_ERR_UNSUPPORTED_SHAPE before anything is enqueued (e.g. I = 2048 allows 15887 rows).
 *   - No memory is allocated or freed, by the library or any routine it calls. The first call
 *     on a GPU looks up the array's device address (hipGetSymbolAddress) and keeps it.
 *   - Every call on one GPU uses the same array and leaves its contents there. Nothing in it
 *     needs to start at zero (each call writes every value its down GEMM's stored results
 *     read). Calls that overlap on one GPU (several streams, or host threads) race on it:
 *     order them, e.g. on one stream.
 */
dg_status_t dg_moe_ffn_fp8_noalloc(int32_t layout, int32_t scale_fmt, const uint8_t* x, const float* sfx,
                                   const uint8_t* w1, const float* sfw1, const uint8_t* w2, const float* sfw2,
                                   const int32_t* meta, uint16_t* y, int32_t G, int64_t M, int64_t H, int64_t I,
                                   int64_t expected_m, void* stream);

/*
 * Plain fp32 -> e4m3 conversion with gfx950's hardware instruction, the conversion the fused
 * SwiGLU epilogue of dg_gemm_fp8_swiglu applies to h / s (its quotients never exceed
 * 448.0001). OCP E4M3FN codes (DeepSeek-V3 repo review, "Risks" item 6: bound 448), round to
 * nearest even, sign of zero kept. It exists so that this conversion can be checked against
 * the per-token cast's rule on every input of interest.
 *   x [n] fp32 (device), q [n] e4m3 bytes (device, output); n % 4 == 0.
 * Precondition: |x| <= 464 and finite. Within it the result equals the saturating encoder of
 * dg_cast_fp8_per_token (values in (448, 464] round to 448); beyond it the hardware does not
 * saturate and the codes are unspecified (never a fault).
 */
dg_status_t dg_convert_fp8_e4m3(const float* x, int64_t n, uint8_t* q, void* stream);

/*
 * Re-reads the tuning switches from the environment. The library reads them once, at its first
 * GEMM call; they only force a kernel schedule, never change what is computed, and are meant
 * for tuning sessions and tests that compare schedules within one process:
 *   DG_TILE=<name> (a tile kernel), DG_DECODE=v1 (the register-fed decode schedule),
 *   DG_DECODE2="bn,kg,kpw,waves", DG_DECODE3="wave rows,wave columns,strips,slots" (one
 *   decode configuration), DG_LOG (print each call's chosen kernel on stderr).
 * Safe to call at any time; calls already enqueued are not affected.
 */
void dg_reload_tuning_switches(void);

/* Human-readable name of a status code (static string). */
const char* dg_status_string(dg_status_t status);

/* Detail of the last failed call on this thread (static per-thread buffer; "" if none). */
const char* dg_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* DG_H */
