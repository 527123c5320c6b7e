/*
 * bsg.h -- C ABI of the block-scaled GEMM library for AMD Instinct MI355X (gfx950).
 *
 * The library computes D = A * B^T on one GPU:
 *   - BF16 x BF16,
 *   - FP8 e4m3 x e4m3 with UE8M0 block scales,
 *   - FP4 e2m1 x e2m1 with UE8M0 block scales,
 *   - M-grouped variants (FP8, BF16, FP4, and a masked FP8 layout) for
 *     mixture-of-experts layers,
 * always accumulating in fp32 and writing bf16 (round to nearest even).  It also
 * packs and unpacks UE8M0 scales into the int16, MN-major layout the scaled GEMMs
 * read, quantises bf16 rows into that format (the producer side), runs the MoE
 * FFN core on one GPU's share (grouped up-projection with SwiGLU and FP8
 * requantisation fused into its epilogue, grouped down-projection), and computes
 * the MQA logits of a lightning-indexer step in FP8 and FP4.
 *
 * The pages this follows list BF16, FP8 and FP4 dense GEMM plus grouped (MoE)
 * GEMM as the library's coverage ("DeepGEMM-Ascend cobre quantas operacoes no
 * Ascend 950?", section "Cobertura de operacoes e a lacuna declarada no
 * repositorio"; "DeepSeek lanza kernels de DeepGEMM para Huawei Ascend 950",
 * section "Que incluye el lanzamiento"), and describe the scale layout: UE8M0
 * scale factors packed in pairs along K into 16-bit integers, stored MN-major,
 * reused as they are when already in that layout and converted otherwise (first
 * page, section "Fatores de escala FP8 e o formato UE8M0 no Ascend").  Formulas,
 * layouts and bit formats are not on the pages; the readings below are this
 * library's.
 *
 * Common conventions
 *  - Layout (NT): A is [M][K] and B is [N][K], K contiguous; D is [M][N], N
 *    contiguous.  Leading dimensions (lda, ldb, ldd, ld_sf*) count storage
 *    elements: bf16 elements for BF16 operands and D, bytes for FP8 and FP4
 *    operands (an FP4 byte holds two values, the even K index in the low nibble).
 *  - Formats: FP8 is OCP e4m3fn (bias 7, max 448, no infinities); FP4 is OCP
 *    e2m1 ({0, .5, 1, 1.5, 2, 3, 4, 6} with sign); a UE8M0 byte b is 2^(b-127).
 *  - Packed scales: int16 P[ceil(Kb/2)][ld_sf] where Kb is the number of K-blocks;
 *    element (kp, mn) sits at kp*ld_sf + mn, its low byte is K-block 2kp and its
 *    high byte K-block 2kp+1 (0x7F when Kb is odd).  "Scale rows" (mn) are the
 *    rows of A, the 128-row blocks of B (FP8; its rows with sfb_gran_mn = 1) or
 *    the rows of B (FP4).
 *  - Every pointer is a device pointer owned by the caller; the library allocates
 *    nothing, keeps no state between calls (apart from the fixed device array of
 *    moe_ffn_fp8_noalloc) and never synchronises.  Work is
 *    enqueued on `stream` (a hipStream_t; NULL is the default stream) and is
 *    complete when the stream says so.  The one exception is the scale
 *    pack/unpack pair: there NULL means host pointers and a synchronous call.
 *  - Every call validates its arguments on the host before touching the GPU and
 *    returns a status code; nothing is launched when the status is not BSG_OK.
 *    A launch failure reported by the runtime returns BSG_ERR_HIP.
 *  - M == 0 or N == 0 is a no-op.  K == 0 writes zeros to D and reads neither
 *    A, B nor the scales (their pointers may then be NULL).
 *  - A wrongly laid out scale array cannot be detected: it gives wrong numbers,
 *    not an error (the pages warn of exactly this failure mode).
 *  - Sizes: every leading dimension times 256 must stay below 2^31 bytes.  A
 *    packed scale array of the GEMMs, kp packed rows of ld_sf int16, must keep
 *    2 (kp + 1) ld_sf below 2^31 bytes (the kernels address one packed row past
 *    the last on a K tail).  Larger shapes return BSG_ERR_UNSUPPORTED_SHAPE.
 */
#ifndef BSG_H
#define BSG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum bsg_status {
  BSG_OK = 0,
  BSG_ERR_INVALID_ARG = 1,       /* null pointer, negative size, leading dimension too small */
  BSG_ERR_UNSUPPORTED_SHAPE = 2, /* K not a multiple of the format's K granularity, too large */
  BSG_ERR_MISALIGNED = 3,        /* base pointer or row stride not 16-byte aligned */
  BSG_ERR_HIP = 4,               /* the HIP runtime reported an error at launch */
};

/* Scale rules of the per-token quantisers (below). */
enum bsg_scale_rule {
  BSG_SCALE_CEIL = 0,   /* smallest power of two that holds the block's amax: nothing clips */
  BSG_SCALE_OCP_MX = 1, /* OCP Microscaling: 2^(floor(log2 amax) - emax), larger values saturate */
};

/* Human-readable name of a status code (static storage). */
const char* bsg_status_string(int status);

/* BF16 GEMM: D[m][n] = bf16( sum_k A[m][k] * B[n][k] ), fp32 accumulation.
 *   A: bf16 [M][lda], B: bf16 [N][ldb], D: bf16 [M][ldd] (device pointers).
 *   Requires K % 8 == 0, lda >= K, ldb >= K, ldd >= N; A and B 16-byte aligned,
 *   lda and ldb multiples of 8; D 2-byte aligned (rows that are 8-byte aligned
 *   are written with wider stores). */
int gemm_bf16(const void* A, int64_t lda, const void* B, int64_t ldb, void* D, int64_t ldd,
              int64_t M, int64_t N, int64_t K, void* stream);

/* FP8 block-scaled GEMM:
 *   D[m][n] = bf16( sum_k a[m][k] * 2^(sa[m][k/128]-127) * b[n][k] * 2^(sb[n/gb][k/128]-127) )
 *   A: e4m3 [M][lda] bytes; sfa: packed int16 [K/256 rounded up][ld_sfa], scale rows = M
 *   (one scale per row of A per 128-wide K-block: sfa_gran_mn must be 1).
 *   B: e4m3 [N][ldb] bytes; sfb: packed int16 [..][ld_sfb] with gb = sfb_gran_mn:
 *   128, one scale per 128x128 block of B (scale rows = ceil(N/128)), or 1, one
 *   per row of B per 128-wide K-block (scale rows = N).
 *   D: bf16 [M][ldd].
 *   Requires K % 128 == 0, ld_sfa >= M, ld_sfb >= the scale rows of B, lda, ldb >= K,
 *   ldd >= N; A and B 16-byte aligned, lda and ldb multiples of 16; D, sfa and
 *   sfb 2-byte aligned.  Other granularities: BSG_ERR_UNSUPPORTED_SHAPE. */
int gemm_fp8_blockscaled(const void* A, int64_t lda, const int16_t* sfa, int64_t ld_sfa,
                         int32_t sfa_gran_mn, const void* B, int64_t ldb, const int16_t* sfb,
                         int64_t ld_sfb, int32_t sfb_gran_mn, void* D, int64_t ldd, int64_t M,
                         int64_t N, int64_t K, void* stream);

/* FP4 block-scaled GEMM:
 *   D[m][n] = bf16( sum_k a[m][k] * 2^(sa[m][k/32]-127) * b[n][k] * 2^(sb[n][k/32]-127) )
 *   A: e2m1 [M][lda] bytes (two values per byte), B: e2m1 [N][ldb] bytes;
 *   sfa: packed int16 [K/64 rounded up][ld_sfa], scale rows = M;
 *   sfb: packed int16 [..][ld_sfb], scale rows = N (one scale per row per 32-wide
 *   K-block on both operands).  D: bf16 [M][ldd].
 *   Requires K % 32 == 0, lda, ldb >= K/2 (bytes), ld_sfa >= M, ld_sfb >= N,
 *   ldd >= N; A and B 16-byte aligned, lda and ldb multiples of 16; D, sfa and
 *   sfb 2-byte aligned. */
int gemm_fp4_blockscaled(const void* A, int64_t lda, const int16_t* sfa, int64_t ld_sfa,
                         const void* B, int64_t ldb, const int16_t* sfb, int64_t ld_sfb,
                         void* D, int64_t ldd, int64_t M, int64_t N, int64_t K, void* stream);

/* M-grouped FP8 GEMM for mixture-of-experts layers (the pages name M-grouped GEMM
 * among the released kernels: "aireiter.com -- DeepSeek Ascend infrastructure
 * components", table "Mapa de componentes").
 *   Rows [off[g], off[g+1]) of A and D belong to expert g (0 <= g < G) and use
 *   expert g's weights B_g = B + g*stride_b (e4m3 [N][ldb] bytes) and scales
 *   sfb_g = sfb + g*stride_sfb (packed int16, scale rows = ceil(N/128)):
 *     D[m][n] = bf16( sum_k a[m][k] * 2^(sa[m][k/128]-127) * b_g[n][k] * 2^(sb_g[n/128][k/128]-127) )
 *   A: e4m3 [M_total][lda]; sfa packed, scale rows = M_total; D: bf16 [M_total][ldd].
 *   group_offsets: DEVICE int32 [G+1].  Precondition (not checked by the host, the
 *   offsets live on the device): 0 <= off[0] <= off[1] <= ... <= off[G] <= M_total.
 *   The kernel clamps each expert's range into [0, M_total] (lo = clamp(off[g]),
 *   hi = clamp(off[g+1]) >= lo), so offsets that break it give wrong rows (experts
 *   whose ranges overlap race on the shared rows) but never an access outside A,
 *   D or their scales.  Rows outside [off[0], off[G]) are not written.  Empty
 *   groups are allowed.
 *   Offsets need no alignment; 128-row aligned groups waste no tile rows.
 *   G == 0 is a no-op.  Requires G <= 1024, K % 128 == 0, stride_b >= (N-1)*ldb + K,
 *   stride_sfb >= ceil(K/256)*ld_sfb, plus the dense FP8 requirements. */
int m_grouped_gemm_fp8(const void* A, int64_t lda, const int16_t* sfa, int64_t ld_sfa,
                       const void* B, int64_t ldb, int64_t stride_b,
                       const int16_t* sfb, int64_t ld_sfb, int64_t stride_sfb,
                       void* D, int64_t ldd, const int32_t* group_offsets, int32_t G,
                       int64_t M_total, int64_t N, int64_t K, void* stream);

/* M-grouped BF16 GEMM: as m_grouped_gemm_fp8 without scales (the pages list BF16
 * among the formats and grouped MoE GEMM among the kernels: same passages).
 *   A: bf16 [M_total][lda]; B_g = B + g*stride_b: bf16 [N][ldb] (strides in bf16
 *   elements); D: bf16 [M_total][ldd]; group_offsets: DEVICE int32 [G+1] with the
 *   same precondition and row rules as m_grouped_gemm_fp8.
 *   Requires K % 8 == 0, G <= 1024, stride_b >= (N-1)*ldb + K, stride_b*2 % 16 == 0,
 *   plus the gemm_bf16 requirements. */
int m_grouped_gemm_bf16(const void* A, int64_t lda, const void* B, int64_t ldb, int64_t stride_b,
                        void* D, int64_t ldd, const int32_t* group_offsets, int32_t G,
                        int64_t M_total, int64_t N, int64_t K, void* stream);

/* M-grouped FP4 GEMM: as m_grouped_gemm_fp8 with the FP4 operand and scale rules
 * of gemm_fp4_blockscaled (1x32 UE8M0 scales on both operands; expert g's B scales
 * sfb + g*stride_sfb, scale rows = N).
 *   Requires K % 32 == 0, G <= 1024, stride_b >= (N-1)*ldb + K/2 (bytes),
 *   stride_sfb >= ceil(K/64)*ld_sfb, plus the gemm_fp4_blockscaled requirements. */
int m_grouped_gemm_fp4(const void* A, int64_t lda, const int16_t* sfa, int64_t ld_sfa,
                       const void* B, int64_t ldb, int64_t stride_b,
                       const int16_t* sfb, int64_t ld_sfb, int64_t stride_sfb,
                       void* D, int64_t ldd, const int32_t* group_offsets, int32_t G,
                       int64_t M_total, int64_t N, int64_t K, void* stream);

/* Masked M-grouped FP8 GEMM: every expert owns a fixed capacity of max_m rows and
 * a device-side count of valid rows (the pages list masked grouped GEMM among
 * the interfaces the reference repository declares but leaves unimplemented:
 * first page, "Cobertura de operacoes e a lacuna declarada no repositorio").
 * The layout reading: A is [G][max_m][K] viewed as [G*max_m][lda] rows, D is
 * [G][max_m][N] viewed as [G*max_m][ldd]; sfa packs the scales of all G*max_m
 * rows (ld_sfa >= G*max_m), exactly what quantize_fp8_per_token writes for that
 * view.  For expert g and r < m_g = min(max(masked_m[g], 0), max_m):
 *     D[g*max_m + r][n] = bf16( sum_k a[g*max_m + r][k] * 2^(sa-127) * b_g[n][k] * 2^(sb_g-127) )
 * with B_g, sfb_g as in m_grouped_gemm_fp8.  Rows r >= m_g are not written.
 *   masked_m: DEVICE int32 [G] (read by the kernel; no host synchronisation).
 *   G == 0 or max_m == 0 is a no-op.  Requires G * max_m < 2^31 plus the
 *   requirements of m_grouped_gemm_fp8 with M_total = G * max_m. */
int m_grouped_gemm_fp8_masked(const void* A, int64_t lda, const int16_t* sfa, int64_t ld_sfa,
                              const void* B, int64_t ldb, int64_t stride_b,
                              const int16_t* sfb, int64_t ld_sfb, int64_t stride_sfb,
                              void* D, int64_t ldd, const int32_t* masked_m, int32_t G,
                              int64_t max_m, int64_t N, int64_t K, void* stream);

/* Pack UE8M0 scales: the conversion half of the pages' reuse-or-convert scale
 * helper, which passes scales through when they already have the packed layout
 * and converts them otherwise (first page, "DeepGEMM-Ascend cobre quantas
 * operacoes no Ascend 950?", section "Fatores de escala FP8 e o formato UE8M0
 * no Ascend"):
 *   sf: uint8 [mn][ld_sf], K-blocks contiguous (kb of them per scale row)
 *   -> packed: int16 [ceil(kb/2)][ld_packed], MN-major, as described above
 *      (columns mn .. ld_packed-1 are not written).
 *   stream == NULL: sf and packed are HOST pointers; the work is done on the
 *     calling thread before the call returns (no HIP call is made, so this also
 *     works on a machine without a GPU).
 *   stream != NULL: sf and packed are DEVICE pointers; a kernel is enqueued on
 *     that hipStream_t.  To use the legacy default stream pass hipStreamLegacy
 *     ((void*)1), since NULL selects the host path.
 *   Requires ld_sf >= kb, ld_packed >= mn, packed 2-byte aligned; mn == 0 or
 *   kb == 0 is a no-op.  Errors: BSG_ERR_INVALID_ARG (null pointer, negative size,
 *   leading dimension too small), BSG_ERR_MISALIGNED, BSG_ERR_HIP (launch). */
int pack_ue8m0_scales(const uint8_t* sf, int64_t mn, int64_t kb, int64_t ld_sf,
                      int16_t* packed, int64_t ld_packed, void* stream);

/* Pack fp32 scale factors: the conversion half of the same reuse-or-convert helper
 * for scales that arrive as fp32 tensors holding powers of two (the form in which
 * block-scaled operands often carry their factors; the pages' helper converts
 * whatever layout it is given into the packed one: first page, section "Fatores de
 * escala FP8 e o formato UE8M0 no Ascend").
 *   sf: fp32 [mn][ld_sf], K-blocks contiguous -> packed as in pack_ue8m0_scales.
 *   A value 2^e with -127 <= e <= 127 becomes the byte e + 127 exactly (2^-127 is
 *   the fp32 subnormal 0x00400000).  Any other value (not a power of two, zero or
 *   negative, inf, NaN, below 2^-127) has no UE8M0 code: its byte is unspecified
 *   and it is counted into *inexact (a DEVICE int32 with stream != NULL, added to
 *   atomically, so the caller zeroes it first; a HOST int32 with stream == NULL;
 *   NULL: not counted).
 *   Stream rule, requirements and errors as pack_ue8m0_scales; sf 4-byte aligned. */
int pack_ue8m0_scales_f32(const float* sf, int64_t mn, int64_t kb, int64_t ld_sf,
                          int16_t* packed, int64_t ld_packed, int32_t* inexact, void* stream);

/* Inverse of pack_ue8m0_scales, with the same stream rule (NULL: host pointers,
 * synchronous; otherwise device pointers and a kernel on `stream`): packed int16
 * [ceil(kb/2)][ld_packed] -> sf uint8 [mn][ld_sf]; the 0x7F filler byte of an odd
 * kb is not written back.  Columns kb .. ld_sf-1 of sf are not written. */
int unpack_ue8m0_scales(const int16_t* packed, int64_t mn, int64_t kb, int64_t ld_packed,
                        uint8_t* sf, int64_t ld_sf, void* stream);

/* Per-token quantisation of bf16 rows into the operand formats above, with the
 * scales written straight into the packed int16, MN-major layout (device kernel
 * on `stream`).  The pages say operands carry UE8M0 scales that the accelerator
 * wants packed in pairs along K, MN-major, and that converting them on each call
 * costs time ("DeepGEMM-Ascend cobre quantas operacoes no Ascend 950?", section
 * "Fatores de escala FP8 e o formato UE8M0 no Ascend"); producing that layout
 * here leaves no conversion for the GEMM call.  The scale rule and the rounding
 * are readings (the pages do not give them):
 *   per block of GK elements of a row (GK = 128 for FP8, 32 for FP4), with amax
 *   its largest magnitude and qmax the format's largest finite value (448, 6):
 *     rule BSG_SCALE_CEIL  : e = smallest integer with amax <= qmax * 2^e;
 *     rule BSG_SCALE_OCP_MX: e = floor(log2 amax) - emax (emax 8 for e4m3, 2 for
 *                            e2m1); magnitudes above qmax * 2^e saturate;
 *     scale byte = clamp(e + 127, 0, 254); an all-zero block gets byte 0;
 *     code = x / 2^e rounded to the nearest grid value, ties to the even code,
 *            saturating at qmax, with x's sign bit (so -0 gives the -0 code).
 *   X: bf16 [M][ldx], finite values (NaN or infinity give unspecified codes).
 *   Q: FP8: e4m3 [M][ldq] bytes, ldq >= K;  FP4: e2m1 [M][ldq] bytes, ldq >= K/2,
 *      two values per byte, the even K index in the low nibble.
 *   sf: packed int16 [ceil(Kb/2)][ld_sf], ld_sf >= M, Kb = K/GK; element (kp, m)
 *       holds the bytes of blocks 2kp (low) and 2kp+1 (high, 0x7F when Kb is
 *       odd).  This is exactly the sfa operand of gemm_fp8_blockscaled /
 *       gemm_fp4_blockscaled (and of m_grouped_gemm_fp8 for FP8).
 *   Requires K % GK == 0, K / 512 < 65536; X 16-byte aligned with ldx % 8 == 0;
 *   Q 8-byte (FP8) or 4-byte (FP4) aligned with ldq a multiple of that; sf 2-byte
 *   aligned.  M == 0 or K == 0 is a no-op.  Columns of Q beyond K and of sf beyond
 *   M are not written. */
int quantize_fp8_per_token(const void* X, int64_t ldx, void* Q, int64_t ldq, int16_t* sf,
                           int64_t ld_sf, int64_t M, int64_t K, int32_t rule, void* stream);

int quantize_fp4_per_token(const void* X, int64_t ldx, void* Q, int64_t ldq, int16_t* sf,
                           int64_t ld_sf, int64_t M, int64_t K, int32_t rule, void* stream);

/* SwiGLU followed by FP8 1x128 quantisation (device kernel on `stream`), the step
 * between the two grouped GEMMs of an MoE FFN (the pages list SwiGLU between the
 * two grouped GEMMs of the fused MoE benchmark: third page, "Kernels de computacao:
 * DeepGEMM-Ascend versus DeepGEMM", section "Execucao de MoE: MegaMoE e
 * distribuicao de especialistas"; the function itself is not defined there, the
 * textbook SwiGLU is the reading):
 *   y[m][i] = silu(H[m][i]) * H[m][I + i],  silu(g) = g / (1 + e^-g),  0 <= i < I,
 * formed in fp32, then quantised per 128-wide block of each row exactly as
 * quantize_fp8_per_token does (same rules, codes and packed scales).
 *   H: bf16 [M][ldh], ldh >= 2I (gate in columns [0, I), up in [I, 2I)).
 *   Q: e4m3 [M][ldq] bytes, ldq >= I; sf: packed int16 [ceil(I/256)][ld_sf >= M].
 *   Requires I % 128 == 0 plus the alignment rules of quantize_fp8_per_token (H
 *   takes X's).  Because y is an fp32 result (a few ulps from the exact value), a
 *   code whose exact value sits within that distance of a rounding boundary may
 *   round either way. */
int swiglu_quantize_fp8(const void* H, int64_t ldh, void* Q, int64_t ldq, int16_t* sf,
                        int64_t ld_sf, int64_t M, int64_t I, int32_t rule, void* stream);

/* MoE FFN core on one GPU (the expert computation of the fused MoE step named on
 * the pages, without the dispatch / combine communication):
 *   H = m_grouped_gemm_fp8(A, W13)          bf16 [M_total][2*inter]
 *   (Y, sfy) = swiglu_quantize_fp8(H)       e4m3 [M_total][inter] + packed 1x128 scales
 *   D = m_grouped_gemm_fp8(Y, W2)           bf16 [M_total][hidden]
 * as two launches on `stream`, with the same expert row ranges (group_offsets,
 * device int32 [G+1]) in both GEMMs: the up-projection applies SwiGLU and the
 * requantisation to each tile in its epilogue, with the same bits as the first two
 * calls above, so H is never formed.  H may be NULL (then ldh is ignored); a
 * non-NULL H is checked as that output would be but is not written.
 *   A: e4m3 [M_total][lda] tokens, hidden wide; sfa packed [ceil(hidden/256)][ld_sfa].
 *   W13: e4m3 [G][2*inter][ldw13] (expert g at W13 + g*stride_w13 bytes; gate
 *        rows [0, inter), up rows [inter, 2*inter)); sfw13 packed int16
 *        [G][ceil(hidden/256)][ld_sfw13 >= ceil(2*inter/128)], expert stride
 *        stride_sfw13 elements.
 *   W2: e4m3 [G][hidden][ldw2] (K = inter); sfw2 packed [G][ceil(inter/256)][ld_sfw2].
 *   Y, sfy: caller-owned workspace (the library allocates nothing), with
 *        ldy >= inter, ld_sfy >= M_total (H: see above, ldh >= 2*inter).
 *   D: bf16 [M_total][ldd].  Rows outside [off[0], off[G]) of H, Y and D are not
 *   meaningful.  Every argument of all three steps is checked before the first
 *   launch; the requirements are those of the three calls above (hidden and inter
 *   multiples of 128), and (inter + 128) * ldw13 < 2^31 (the up-projection reads a
 *   tile's gate rows and the matching up rows through one record of 32-bit byte
 *   offsets); larger shapes return BSG_ERR_UNSUPPORTED_SHAPE. */
int moe_ffn_fp8(const void* A, int64_t lda, const int16_t* sfa, int64_t ld_sfa,
                const void* W13, int64_t ldw13, int64_t stride_w13, const int16_t* sfw13,
                int64_t ld_sfw13, int64_t stride_sfw13,
                const void* W2, int64_t ldw2, int64_t stride_w2, const int16_t* sfw2,
                int64_t ld_sfw2, int64_t stride_sfw2,
                const int32_t* group_offsets, int32_t G, int64_t M_total, int64_t hidden,
                int64_t inter, void* H, int64_t ldh, void* Y, int64_t ldy, int16_t* sfy,
                int64_t ld_sfy, void* D, int64_t ldd, int32_t rule, void* stream);

/* MQA logits, FP8 and FP4 (the pages list "MQA logits" among the library's
 * kernels: attention scores of multi-query attention on the DeepSeek Lightning
 * Indexer path, with FP8 and FP4 prefill and decode cases; first page,
 * "DeepGEMM-Ascend cobre quantas operacoes no Ascend 950?", section "Cobertura de
 * operacoes e a lacuna declarada no repositorio"; third page, section "Kernels
 * especificos de modelo: logits de MQA e prenorm mHC").  The pages do not define
 * the computation; the reading is the indexer's score, with the head dimension
 * fixed at 128:
 *   L[t][s] = sum_{h<H} w[t][h] * max(0, q[t][h] . k[g(t)][s])   ks[t] <= s < ke[t]
 *   L[t][s] = -inf                                               other s < S
 * where q and k are dequantised with their UE8M0 block scales and accumulated in
 * fp32, g(t) = t / q_per_group is the query's key group (a sequence: prefill has
 * one group of all T queries, decode one group per request), and key s of group g
 * is row g*group_rows + s of K.
 *   Q: codes [T*H][ldq] (row t*H + h): mqa_logits_fp8 e4m3, 128 bytes a row, one
 *      scale per row (sfq packed int16 [1][ld_sfq >= T*H], the low byte);
 *      mqa_logits_fp4 e2m1, two per byte (even index in the low nibble), 64 bytes
 *      a row, one scale per 32 elements (sfq packed [2][ld_sfq]).
 *   K: codes [k_rows][ldk] with k_rows = (ceil(T/q_per_group) - 1)*group_rows + S,
 *      same formats; sfk packed over K's rows (ld_sfk >= k_rows).
 *   W: fp32 [T][ldw >= H].  ks, ke: DEVICE int32 [T]; windows are clamped to
 *      [0, S], and ks >= ke gives a row of -inf.
 *   L: fp32 [T][ldl >= S]; columns S .. ldl-1 are not written.
 *   Requires H a multiple of 32, at most 128; Q, K 16-byte aligned with ldq, ldk
 *   multiples of 16 bytes; sfq, sfk 2-byte aligned; W, L 4-byte aligned;
 *   q_per_group >= 1, group_rows >= 0.  T == 0 or S == 0 is a no-op.  Errors:
 *   BSG_ERR_INVALID_ARG, BSG_ERR_UNSUPPORTED_SHAPE (H, or offsets past 2^31 bytes),
 *   BSG_ERR_MISALIGNED, BSG_ERR_HIP (launch). */
int mqa_logits_fp8(const void* Q, int64_t ldq, const int16_t* sfq, int64_t ld_sfq,
                   const void* K, int64_t ldk, const int16_t* sfk, int64_t ld_sfk,
                   const float* W, int64_t ldw, const int32_t* ks, const int32_t* ke,
                   float* L, int64_t ldl, int64_t T, int64_t S, int32_t H,
                   int64_t q_per_group, int64_t group_rows, void* stream);

int mqa_logits_fp4(const void* Q, int64_t ldq, const int16_t* sfq, int64_t ld_sfq,
                   const void* K, int64_t ldk, const int16_t* sfk, int64_t ld_sfk,
                   const float* W, int64_t ldw, const int32_t* ks, const int32_t* ke,
                   float* L, int64_t ldl, int64_t T, int64_t S, int32_t H,
                   int64_t q_per_group, int64_t group_rows, void* stream);

/* MoE FFN core that allocates nothing and takes no workspace: for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It computes exactly what moe_ffn_fp8 computes,
 * with the same kernels and the same bits, but keeps the requantised intermediate
 * Y (e4m3 [M_total][inter]) and its packed scales in a fixed device array inside
 * the library (64 MiB on every GPU the library runs on, held until the process
 * ends) instead of in caller buffers.
 *   Arguments: as moe_ffn_fp8 without H, Y and sfy.
 *   Limit: M_total * inter (rounded up to 256) + ceil(inter/256) * 2 * M_total
 *   (M_total rounded up to 4) bytes must fit 64 MiB, else BSG_ERR_UNSUPPORTED_SHAPE
 *   before anything runs (the one-GPU share of the 384-expert MoE step, 28 672
 *   rows at inter 2048, takes 59 MB).
 *   All calls on one GPU share that GPU's array, which keeps the last call's
 *   contents: calls that overlap on one GPU (two streams, or two threads) race on
 *   it and give wrong results; serialise them.  Nothing in the array needs to start
 *   at any value (every byte read is written earlier in the same call).
 *   The first call on a device looks the array up (hipGetSymbolAddress, no
 *   allocation); a failure there returns BSG_ERR_HIP. */
int moe_ffn_fp8_noalloc(const void* A, int64_t lda, const int16_t* sfa, int64_t ld_sfa,
                        const void* W13, int64_t ldw13, int64_t stride_w13, const int16_t* sfw13,
                        int64_t ld_sfw13, int64_t stride_sfw13,
                        const void* W2, int64_t ldw2, int64_t stride_w2, const int16_t* sfw2,
                        int64_t ld_sfw2, int64_t stride_sfw2,
                        const int32_t* group_offsets, int32_t G, int64_t M_total, int64_t hidden,
                        int64_t inter, void* D, int64_t ldd, int32_t rule, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BSG_H */
