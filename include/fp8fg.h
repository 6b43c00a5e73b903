/*
 * fp8fg.h -- fine-grained FP8 quantization and block-scaled FP8 GEMM on
 * AMD Instinct MI355X (gfx950).  C ABI of libfp8fg.so.
 *
 * What is computed follows the DeepSeek-V3 FP8 training text as it appears
 * on these pages (no section numbers; passages are named by subject):
 *   [why-be]   why-be.why-be.co.kr (untitled): online max-abs per 1x128
 *              activation tile / 128x128 weight block; E4M3 on all tensors;
 *              1x128 -> 128x1 tiles in the backward pass; integral
 *              power-of-two scaling factors.
 *   [thedaegu] thedaegu.com, "OMG! The most effective Deepseek Ever!":
 *              max-abs mapped onto the largest FP8 value; promotion of
 *              partial sums to FP32 with per-group scaling along K
 *              (Figure 7(b) passage); Fprop / Dgrad / Wgrad in FP8
 *              (Figure 6 passage).
 *   [hearaon]  hearaon.co.kr (untitled): limited accumulation width of
 *              FP8 MMA; activations quantized before the MoE up-projection.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees, copies to the host or synchronizes:
 *     it validates the host-visible arguments, enqueues its kernels on
 *     `stream` (a hipStream_t passed as void*; NULL = the default stream)
 *     on the current HIP device, and returns.
 *   - Sizes and strides are in ELEMENTS of the pointed-to type.
 *   - FP8 is OCP E4M3 (bias 7, largest finite 448, no infinity); bytes are
 *     produced with round-to-nearest-even and saturation.
 *   - Return value: FP8FG_OK (0) or an error code.  On any error other than
 *     FP8FG_ELAUNCH nothing was enqueued.  FP8FG_ELAUNCH reports a HIP
 *     launch failure after enqueue (the stream state is then undefined).
 *   - Inputs must be finite; results for NaN/Inf inputs are unspecified.
 *   - Outputs must not alias inputs.
 *   - Calls are thread-safe; the only global state is a per-device cache of
 *     the compute-unit count, filled once.
 */
#ifndef FP8FG_H
#define FP8FG_H

#include <stdint.h>

#if defined(FP8FG_BUILDING_LIBRARY)
#define FP8FG_API __attribute__((visibility("default")))
#else
#define FP8FG_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum fp8fg_status {
  FP8FG_OK = 0,
  FP8FG_EINVAL = 1,       /* null pointer, negative size, bad enum value     */
  FP8FG_ESHAPE = 2,       /* size not a required multiple; stride too small  */
  FP8FG_EALIGN = 3,       /* pointer or row pitch misaligned                  */
  FP8FG_EUNSUPPORTED = 4, /* valid combination that is not implemented        */
  FP8FG_ELAUNCH = 5       /* HIP reported an error at launch                  */
};

/* element types */
enum { FP8FG_BF16 = 0, FP8FG_F32 = 1, FP8FG_E4M3 = 2 };
/* tile orientation of fp8_quantize_rowtile */
enum { FP8FG_TILE_1x128 = 0, FP8FG_TILE_128x1 = 1 };
/* scale rules */
enum { FP8FG_SCALE_AMAX = 0, FP8FG_SCALE_POW2 = 1 };
/* how the B operand of the GEMM is scaled along N */
enum { FP8FG_BSCALE_BLOCK128 = 0, FP8FG_BSCALE_COL = 1 };
/* GEMM flags (bit set) */
enum {
  FP8FG_GEMM_DEFAULT = 0,
  /* sum the whole K inside the FP8 matrix-core datapath and scale once at the
     end (the naive per-tensor baseline; implies FP8FG_GEMM_FP8_MFMA) */
  FP8FG_GEMM_NO_PROMOTION = 1,
  /* form each 128-wide K group's partial sum with the FP8 MFMA instead of the
     default exact path (faster, but gfx950's FP8 MFMA keeps only ~14 bits
     below the largest of every 8 consecutive products) */
  FP8FG_GEMM_FP8_MFMA = 2,
  /* the FP8 matrix instruction dequantizes, with the scales' powers of two
     as its E8M0 operand scales (the microscaling form; implies
     FP8FG_GEMM_FP8_MFMA and its precision; fastest with power-of-two
     scales) */
  FP8FG_GEMM_E8M0_SCALES = 4,
  /* default path with BLOCK128 scales only: fix the tile shape instead of
     choosing it from the sizes -- WIDE the 256-row tiles, NARROW the 64x128
     weight-streaming tiles.  Every choice gives the same result bit for bit
     (for N >= 256); for tests and tuning.  Setting both, or either together
     with an FP8 flag or COL scales, is FP8FG_EINVAL. */
  FP8FG_GEMM_TILES_WIDE = 8,
  FP8FG_GEMM_TILES_NARROW = 16
};

/*
 * fp8_quantize_rowtile -- online max-abs per tile, scale, E4M3 quantization.
 * [why-be] fine-grained quantization and backward-pass paragraphs;
 * [thedaegu] dynamic-range paragraph.
 *
 *   x      : input [rows][cols], row pitch ldx (elements of x_type).
 *            x_type BF16 or F32: the values themselves.
 *            x_type E4M3 (requantization, tile == 128x1 only): bytes of a
 *            1x128-quantized tensor whose scales are
 *            x_scale[r * xs_rs + (c / 128) * xs_ts]; the source value is
 *            RN32(dec(x[r][c]) * scale).  x_scale is ignored otherwise.
 *   tile == FP8FG_TILE_1x128: a tile is 128 consecutive columns of one row.
 *            Requires cols % 128 == 0.  Output q[r * ldq + c] (u8, same
 *            orientation), scale s[r * s_rs + (c / 128) * s_ts].
 *   tile == FP8FG_TILE_128x1: a tile is 128 consecutive rows of one column.
 *            Requires rows % 128 == 0 and cols % 128 == 0.  Output is
 *            TRANSPOSED: q[c * ldq + r], scale s[c * s_rs + (r / 128) * s_ts]
 *            (i.e. the 1x128 tiling of the transpose).
 *   scale_rule AMAX: s = max(RN32(amax / 448), 2^-126);
 *              POW2: s = max(2^ceil(log2(amax / 448)), 2^-126).
 *   q = E4M3_RNE(RN32(x / s)) with correctly rounded fp32 division.
 *
 *   Alignment: x, q 16-byte aligned; ldx * sizeof(x_type) and ldq multiples
 *   of 16 bytes; s and x_scale 4-byte aligned.  rows == 0 or cols == 0 is a
 *   valid no-op.
 *   Limits (FP8FG_EUNSUPPORTED beyond them): 1x128, at most 2^31 tiles
 *   (rows * cols / 128); 128x1, rows / 128 <= 65535 and
 *   cols / 128 <= (2^32 - 1) / 256.
 */
FP8FG_API int fp8_quantize_rowtile(const void* x, int x_type, int64_t rows, int64_t cols,
                         int64_t ldx, const float* x_scale, int64_t xs_rs,
                         int64_t xs_ts, int tile, int scale_rule, uint8_t* q,
                         int64_t ldq, float* s, int64_t s_rs, int64_t s_ts,
                         void* stream);

/*
 * fp8_quantize_block -- 128x128 weight blocks.  [why-be] / [thedaegu]
 * paragraphs on computing the max-abs online per 128x128 weight block.
 *
 *   w      : input [rows][cols] (BF16 or F32), row pitch ldw; rows and cols
 *            multiples of 128.  One scale per block:
 *            s[(r / 128) * s_rs + (c / 128) * s_cs], same rules as above.
 *   transpose_out == 0: q[r * ldq + c];  == 1: q[c * ldq + r] (cols x rows,
 *            rows contiguous -- the K-contiguous operand layout the GEMM
 *            reads when w is a K x N weight).
 *   Alignment as for fp8_quantize_rowtile.
 *   Limits: rows / 128 <= 65535, cols / 128 <= (2^32 - 1) / 256
 *   (FP8FG_EUNSUPPORTED beyond).
 */
FP8FG_API int fp8_quantize_block(const void* w, int w_type, int64_t rows, int64_t cols,
                       int64_t ldw, int scale_rule, int transpose_out,
                       uint8_t* q, int64_t ldq, float* s, int64_t s_rs,
                       int64_t s_cs, void* stream);

/*
 * fp8_gemm_blockscaled -- C = A . B^T with per-group dequantization scales
 * and FP32 accumulation promoted every 128 elements of K.  [thedaegu]
 * Figure 7(b) passage (promotion; per-group scaling along K) and Figure 6
 * passage (Fprop / Dgrad / Wgrad in FP8); [hearaon] accumulation-precision
 * paragraph.
 *
 *   C[m][n] = sum_kb  sa(m, kb) * sb(kb, n) * P_kb[m][n],
 *   P_kb[m][n] = sum_{k = 128 kb}^{128 kb + 127} dec(a[m * lda + k]) * dec(b[n * ldb + k])
 *
 *   Default path: the products of each P_kb are exact (the FP8 operands are
 *   converted exactly to BF16 in registers and multiplied on the BF16 matrix
 *   cores) and added in FP32; the group's two scales are applied to the FP32
 *   accumulator once per output element and K group (with 128x128 B block
 *   scales the accumulator is kept in units of the current group's scale and
 *   rescaled at each group; a group whose scale lies more than 2^64 below
 *   the largest taken so far for that element is added in units of 2^-64 of
 *   it).  Kernels, tiles and launch counts are chosen from the arguments;
 *   with block scales and N >= 256 every choice gives the same result bit
 *   for bit (so a row's result does not depend on M or on the expert
 *   counts); N = 128 and per-column scales use a kernel that promotes
 *   separate group sums, whose rounding differs within the same accuracy.
 *   Small grids (few 256x256 tiles for the compute units, as with a small
 *   M x N and a long K) run on 64x128 tiles; the flags
 *   FP8FG_GEMM_TILES_WIDE / FP8FG_GEMM_TILES_NARROW fix that choice.  The
 *   library reads no environment variables.
 *
 *   a : E4M3 [M][K] (K contiguous), sa(m, kb) = sa[m * sa_ms + kb * sa_ks].
 *   b : E4M3 [N][K] (K contiguous -- the transposed weight),
 *       b_scale_mode BLOCK128: sb(kb, n) = sb[(n / 128) * sb_ns + kb * sb_ks]
 *       b_scale_mode COL     : sb(kb, n) = sb[n * sb_ns + kb * sb_ks]
 *   c : [M][N] of c_type BF16 (round-to-nearest-even of the FP32 result)
 *       or F32, row pitch ldc.
 *   Requires K % 128 == 0 and N % 128 == 0; any M >= 0.  Scale strides may
 *   be 0 (broadcast).
 *   flags: a bit set of FP8FG_GEMM_NO_PROMOTION, FP8FG_GEMM_FP8_MFMA,
 *       FP8FG_GEMM_E8M0_SCALES and one of FP8FG_GEMM_TILES_WIDE /
 *       FP8FG_GEMM_TILES_NARROW.
 *       NO_PROMOTION: the whole K is summed in the FP8 matrix-core
 *       accumulator and scaled once by sa(m, 0) * sb(0, n); only meaningful
 *       for per-tensor scales, so sa_ks and sb_ks must then be 0.
 *       FP8_MFMA: P_kb comes from the FP8 MFMA (limited internal precision,
 *       see above); promotion and scaling as in the default path.
 *       E8M0_SCALES ([why-be] power-of-two scaling factors; [thedaegu]
 *       passage on exponents shared within small groups): the FP8 MFMA
 *       dequantizes: each scale's power of two 2^(E - 127), E its exponent
 *       field, is the instruction's E8M0 operand scale, and the rest
 *       f = s * 2^(127 - E) -- exactly 1 when s is a power of two, as
 *       FP8FG_SCALE_POW2 produces -- is applied in FP32.  With block scales
 *       and N a multiple of 256 the kernel runs on 256x256 tiles and adds
 *       the products into the accumulator inside the instruction; the
 *       accumulator is kept in units of the current group's f per row and
 *       rescaled by one multiply where f changes (never for power-of-two
 *       scales), as the default path does with whole scales.  Its rounding
 *       then differs from FP8_MFMA's within the same bound.  Otherwise (N
 *       not a multiple of 256, per-column scales) each group's partial sum
 *       is multiplied by f as it is added, and power-of-two scales give
 *       FP8_MFMA's result bit for bit.  Scales must be finite and positive
 *       (an E8M0 scale has no zero; the quantizers' scales are at least
 *       2^-126).  Not combinable with NO_PROMOTION (FP8FG_EINVAL).
 *   Alignment: a, b 16-byte aligned, lda and ldb multiples of 16; c aligned
 *   to its element; scales 4-byte aligned.  (c 16-byte aligned with ldc a
 *   multiple of 4 lets the kernel store 4 outputs per instruction.)
 *   Limits (FP8FG_EUNSUPPORTED beyond them; the kernels address a tile with
 *   32-bit offsets): lda < 2^23, ldb < 2^24, K < 2^31; when promoting,
 *   sa_ms < 2^21 (and sb_ns < 2^21 in the COL mode) and
 *   sa_ks * K/128, sb_ks * K/128 < 2^29; every launch of the chosen kernel
 *   within HIP's 2^32 - 1 work-items per grid dimension (the workgroup
 *   count is computed for the tile shape that will run).
 */
FP8FG_API int fp8_gemm_blockscaled(int64_t M, int64_t N, int64_t K, const uint8_t* a,
                         int64_t lda, const float* sa, int64_t sa_ms,
                         int64_t sa_ks, const uint8_t* b, int64_t ldb,
                         const float* sb, int64_t sb_ns, int64_t sb_ks,
                         int b_scale_mode, void* c, int c_type, int64_t ldc,
                         int flags, void* stream);

/*
 * fp8_grouped_gemm_blockscaled -- the same GEMM for G experts sharing one
 * activation matrix sorted by expert (MoE up/down projections on FP8
 * activations quantized before dispatch: [hearaon] and [thedaegu]
 * paragraphs on FP8 Fprop in MoE up-projections).
 *
 *   offsets : DEVICE int32 [G + 1]; expert e owns rows [offsets[e],
 *             offsets[e+1]) of a and c.  Caller contract (not checked --
 *             that would need a synchronization): offsets[0] == 0,
 *             nondecreasing, offsets[G] == M_total.  Empty experts are legal.
 *   b_e  = b + e * b_gs   ([N][K], K contiguous, pitch ldb)
 *   sb_e = sb + e * sb_gs (128x128 block scales, indexed as BLOCK128 above)
 *   Other arguments as for fp8_gemm_blockscaled (B scaling is BLOCK128).
 *   Requires G >= 1 (G == 0 with M_total == 0 is a no-op), K % 128 == 0,
 *   N % 128 == 0; b_gs a multiple of 16.  M_total and G at most 2^31 - 1
 *   (the offsets are int32), plus the limits of fp8_gemm_blockscaled
 *   (FP8FG_EUNSUPPORTED beyond them).
 */
FP8FG_API int fp8_grouped_gemm_blockscaled(int64_t G, const int32_t* offsets,
                                 int64_t M_total, int64_t N, int64_t K,
                                 const uint8_t* a, int64_t lda,
                                 const float* sa, int64_t sa_ms, int64_t sa_ks,
                                 const uint8_t* b, int64_t ldb, int64_t b_gs,
                                 const float* sb, int64_t sb_ns, int64_t sb_ks,
                                 int64_t sb_gs, void* c, int c_type,
                                 int64_t ldc, int flags, void* stream);

/* Static, thread-safe description of a status code. */
FP8FG_API const char* fp8fg_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FP8FG_H */
