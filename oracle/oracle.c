/*
 * oracle.c -- plain, slow, obviously correct CPU reference for the block-scaled
 * GEMM D = A * B^T in BF16, FP8 (e4m3) and FP4 (e2m1) with UE8M0 block scales.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code, table
 * or header with the GPU library, and the GPU library never calls it.
 *
 * What it computes (the plain definition; every step is exact up to the single
 * fp64 rounding of each running sum):
 *
 *   D[i][j] = sum_k  dec(A[i][k]) * 2^(sa(i, k) - 127) * dec(B[j][k]) * 2^(sb(j, k) - 127)
 *
 * Sources:
 *  - The pages list BF16, FP8 and FP4 dense GEMM and an M-grouped (MoE) GEMM as
 *    the library's coverage ("DeepGEMM-Ascend cobre quantas operacoes no Ascend
 *    950?", section "Cobertura de operacoes e a lacuna declarada no
 *    repositorio"; "DeepSeek lanza kernels de DeepGEMM para Huawei Ascend 950",
 *    section "Que incluye el lanzamiento").
 *  - Low-precision operands carry scale factors in the UE8M0 format; pairs of
 *    them along K share one 16-bit integer and the packed array is MN-major
 *    (first page, section "Fatores de escala FP8 e o formato UE8M0 no Ascend";
 *    fourth page, section "Que incluye el lanzamiento").
 *  - The pages do not write the formula, the layouts, the scale granularities or
 *    the bit-level formats down.  The readings taken here:
 *      * D = A * B^T, A [M][K] and B [N][K] both K-contiguous (NT layout).
 *      * UE8M0 byte b means 2^(b-127); b = 255 is NaN (OCP MX E8M0).
 *      * FP8 is OCP e4m3fn: bias 7, subnormals m/8 * 2^-6, max 448,
 *        S.1111.111 is NaN, no infinities.
 *      * FP4 is OCP e2m1: bias 1, values {0, .5, 1, 1.5, 2, 3, 4, 6} with sign;
 *        two values per byte along K, the even K index in the low nibble.
 *      * FP8 scales: one per row of A per 128-wide K-block, one per 128x128
 *        (N x K) block of B.  FP4 scales: one per row per 32-wide K-block on both
 *        operands.
 *      * Packed scales: int16 array P[ceil(Kb/2)][ld], element (kp, mn) at
 *        kp*ld + mn; its low byte is K-block 2kp, its high byte K-block 2kp+1;
 *        a missing high byte (odd Kb) is filled with 0x7F (the value 1.0).
 *      * M-grouped: rows [off[g], off[g+1]) of A use expert g's B and scales.
 *
 * Arithmetic: every operand element is decoded to fp64 exactly, multiplied by
 * its scale exactly (ldexp of a power of two), and each output is one fp64 dot
 * product accumulated in plain k order.  OpenMP only splits the independent
 * output rows between threads; it does not change any sum.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ----------------------------------------------------------------------------
 * Format decoders (bit-field definitions, exact in fp64)
 * ------------------------------------------------------------------------- */

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 mantissa bits. */
double orc_bf16_to_f64(uint16_t h) {
  int s = (h >> 15) & 1;
  int e = (h >> 7) & 0xFF;
  int m = h & 0x7F;
  double v;
  if (e == 0xFF)
    v = m ? NAN : INFINITY;
  else if (e == 0)
    v = ldexp((double)m, -126 - 7); /* subnormal: m * 2^-133 */
  else
    v = ldexp((double)(128 + m), e - 127 - 7);
  return s ? -v : v;
}

/* OCP FP8 e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities,
 * exponent and mantissa all ones is NaN. */
double orc_e4m3_to_f64(uint8_t b) {
  int s = (b >> 7) & 1;
  int e = (b >> 3) & 0xF;
  int m = b & 0x7;
  double v;
  if (e == 0xF && m == 0x7)
    return NAN;
  if (e == 0)
    v = ldexp((double)m, -6 - 3); /* subnormal: m/8 * 2^-6 */
  else
    v = ldexp((double)(8 + m), e - 7 - 3);
  return s ? -v : v;
}

/* OCP FP4 e2m1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; every code is a
 * finite number. */
double orc_e2m1_to_f64(uint8_t nibble) {
  int s = (nibble >> 3) & 1;
  int e = (nibble >> 1) & 0x3;
  int m = nibble & 0x1;
  double v;
  if (e == 0)
    v = 0.5 * (double)m; /* subnormal: m/2 * 2^0 */
  else
    v = ldexp((double)(2 + m), e - 1 - 1);
  return s ? -v : v;
}

/* UE8M0: an unsigned 8-bit exponent with bias 127 and no mantissa; 0xFF is NaN. */
double orc_ue8m0_to_f64(uint8_t b) {
  if (b == 0xFF)
    return NAN;
  return ldexp(1.0, (int)b - 127);
}

/* fp64 -> bfloat16 bits, round to nearest, ties to even, straight from fp64
 * (one rounding).  Overflow goes to infinity as IEEE round-to-nearest does. */
uint16_t orc_f64_to_bf16_rne(double x) {
  if (isnan(x))
    return 0x7FC0;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a == 0.0)
    return sign;
  if (isinf(a))
    return sign | 0x7F80;
  int e;
  frexp(a, &e); /* a = f * 2^e, 0.5 <= f < 1, so 2^(e-1) <= a < 2^e */
  int q = e - 1 - 7;           /* quantum of an 8-significant-bit number */
  if (q < -133)
    q = -133;                  /* below the normal range the quantum is fixed */
  double r = nearbyint(ldexp(a, -q)); /* default rounding mode: ties to even */
  double v = ldexp(r, q);
  if (v >= ldexp(1.0, 128))
    return sign | 0x7F80;
  /* v is exactly representable in bf16 and therefore in binary32. */
  float f = (float)v;
  uint32_t bits;
  memcpy(&bits, &f, sizeof(bits));
  return sign | (uint16_t)(bits >> 16);
}

/* Array form of orc_f64_to_bf16_rne. */
void orc_f64_to_bf16_rne_array(const double* x, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    out[i] = orc_f64_to_bf16_rne(x[i]);
}

/* ----------------------------------------------------------------------------
 * Packed UE8M0 scales: the oracle's own pack and unpack
 * ------------------------------------------------------------------------- */

/* Byte of K-block kb for scale row mn, read from the packed MN-major array. */
uint8_t orc_scale_byte(const int16_t* packed, int64_t ld_packed, int64_t mn, int64_t kb) {
  uint16_t word = (uint16_t)packed[(kb / 2) * ld_packed + mn];
  return (uint8_t)((word >> (8 * (kb % 2))) & 0xFF);
}

/* sf: uint8 [mn][ld_sf] (K-blocks contiguous) -> packed int16 [ceil(kb/2)][ld_packed]. */
void orc_pack_scales(const uint8_t* sf, int64_t mn, int64_t kb, int64_t ld_sf,
                     int16_t* packed, int64_t ld_packed) {
  int64_t kp_n = (kb + 1) / 2;
  for (int64_t kp = 0; kp < kp_n; ++kp)
    for (int64_t r = 0; r < mn; ++r) {
      uint16_t lo = sf[r * ld_sf + 2 * kp];
      uint16_t hi = (2 * kp + 1 < kb) ? sf[r * ld_sf + 2 * kp + 1] : 0x7F;
      packed[kp * ld_packed + r] = (int16_t)(lo | (hi << 8));
    }
}

/* packed int16 [ceil(kb/2)][ld_packed] -> sf uint8 [mn][ld_sf]. */
void orc_unpack_scales(const int16_t* packed, int64_t mn, int64_t kb, int64_t ld_packed,
                       uint8_t* sf, int64_t ld_sf) {
  for (int64_t r = 0; r < mn; ++r)
    for (int64_t k = 0; k < kb; ++k)
      sf[r * ld_sf + k] = orc_scale_byte(packed, ld_packed, r, k);
}

/* ----------------------------------------------------------------------------
 * Dequantised rows
 * ------------------------------------------------------------------------- */

enum { ORC_BF16 = 0, ORC_E4M3 = 1, ORC_E2M1 = 2 };

/* One operand: element storage, its leading dimension in storage units (bf16
 * elements, or bytes for e4m3 and e2m1), and, for the scaled formats, the packed
 * scales with their granularity (gran_mn rows share a scale row; gran_k
 * consecutive K elements share a scale). */
typedef struct {
  int fmt;
  const void* data;
  int64_t ld;
  const int16_t* sf;
  int64_t ld_sf;
  int64_t gran_mn;
  int64_t gran_k;
} orc_operand;

/* Dequantised value of element (row, k). */
static double orc_element(const orc_operand* op, int64_t row, int64_t k) {
  double v;
  if (op->fmt == ORC_BF16) {
    const uint16_t* p = (const uint16_t*)op->data;
    return orc_bf16_to_f64(p[row * op->ld + k]);
  } else if (op->fmt == ORC_E4M3) {
    const uint8_t* p = (const uint8_t*)op->data;
    v = orc_e4m3_to_f64(p[row * op->ld + k]);
  } else {
    const uint8_t* p = (const uint8_t*)op->data;
    uint8_t byte = p[row * op->ld + k / 2];
    uint8_t nib = (k % 2 == 0) ? (byte & 0xF) : (byte >> 4);
    v = orc_e2m1_to_f64(nib);
  }
  uint8_t s = orc_scale_byte(op->sf, op->ld_sf, row / op->gran_mn, k / op->gran_k);
  return v * orc_ue8m0_to_f64(s);
}

static void orc_decode_row(const orc_operand* op, int64_t row, int64_t K, double* out) {
  for (int64_t k = 0; k < K; ++k)
    out[k] = orc_element(op, row, k);
}

/* ----------------------------------------------------------------------------
 * GEMM:  out[r][c] = D[rows[r]][cols[c]]   (fp64)
 * ------------------------------------------------------------------------- */

static double orc_dot(const double* a, const double* b, int64_t K) {
  double s = 0.0;
  for (int64_t k = 0; k < K; ++k)
    s += a[k] * b[k];
  return s;
}

/* Returns 0 on success, -1 if memory could not be allocated. */
static int orc_gemm(const orc_operand* a, const orc_operand* b, int64_t K,
                    const int64_t* rows, int64_t nrows, const int64_t* cols, int64_t ncols,
                    double* out) {
  double* bd = (double*)malloc(sizeof(double) * (size_t)(ncols > 0 ? ncols : 1) * (size_t)K);
  if (!bd)
    return -1;
  int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t c = 0; c < ncols; ++c)
    orc_decode_row(b, cols[c], K, bd + c * K);
#pragma omp parallel
  {
    double* ad = (double*)malloc(sizeof(double) * (size_t)K);
    if (!ad) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
      if (!ad)
        continue;
      orc_decode_row(a, rows[r], K, ad);
      for (int64_t c = 0; c < ncols; ++c)
        out[r * ncols + c] = orc_dot(ad, bd + c * K, K);
    }
    free(ad);
  }
  free(bd);
  return failed ? -1 : 0;
}

/* BF16 x BF16: A uint16 [M][lda], B uint16 [N][ldb]. */
int orc_gemm_bf16(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int64_t K,
                  const int64_t* rows, int64_t nrows, const int64_t* cols, int64_t ncols,
                  double* out) {
  orc_operand a = {ORC_BF16, A, lda, NULL, 0, 1, 1};
  orc_operand b = {ORC_BF16, B, ldb, NULL, 0, 1, 1};
  return orc_gemm(&a, &b, K, rows, nrows, cols, ncols, out);
}

/* FP8 e4m3: A [M][lda] with packed per-row, per-128-K scales (sfa, scale rows =
 * M); B [N][ldb] with packed per-128-K scales shared by sfb_gran_mn consecutive
 * rows: 128 (128x128 blocks, scale rows = ceil(N/128)) or 1 (one per row, scale
 * rows = N). */
int orc_gemm_fp8(const uint8_t* A, int64_t lda, const int16_t* sfa, int64_t ld_sfa,
                 const uint8_t* B, int64_t ldb, const int16_t* sfb, int64_t ld_sfb,
                 int64_t sfb_gran_mn, int64_t K,
                 const int64_t* rows, int64_t nrows, const int64_t* cols, int64_t ncols,
                 double* out) {
  orc_operand a = {ORC_E4M3, A, lda, sfa, ld_sfa, 1, 128};
  orc_operand b = {ORC_E4M3, B, ldb, sfb, ld_sfb, sfb_gran_mn, 128};
  return orc_gemm(&a, &b, K, rows, nrows, cols, ncols, out);
}

/* FP4 e2m1: A uint8 [M][lda bytes] and B uint8 [N][ldb bytes], two values per
 * byte along K; packed per-row, per-32-K scales on both. */
int orc_gemm_fp4(const uint8_t* A, int64_t lda, const int16_t* sfa, int64_t ld_sfa,
                 const uint8_t* B, int64_t ldb, const int16_t* sfb, int64_t ld_sfb, int64_t K,
                 const int64_t* rows, int64_t nrows, const int64_t* cols, int64_t ncols,
                 double* out) {
  orc_operand a = {ORC_E2M1, A, lda, sfa, ld_sfa, 1, 32};
  orc_operand b = {ORC_E2M1, B, ldb, sfb, ld_sfb, 1, 32};
  return orc_gemm(&a, &b, K, rows, nrows, cols, ncols, out);
}

/* M-grouped FP8: rows [off[g], off[g+1]) of A use expert g, whose B starts at
 * B + g*stride_b and whose packed scales start at sfb + g*stride_sfb.  A row at
 * or beyond off[G] belongs to no expert: its outputs are set to NaN ("not
 * written").  Rows are looked up one by one; experts are decoded one at a time so
 * the fp64 copy of B never exceeds one expert. */
int orc_grouped_fp8(const uint8_t* A, int64_t lda, const int16_t* sfa, int64_t ld_sfa,
                    const uint8_t* B, int64_t ldb, int64_t stride_b,
                    const int16_t* sfb, int64_t ld_sfb, int64_t stride_sfb,
                    const int32_t* off, int32_t G, int64_t K,
                    const int64_t* rows, int64_t nrows, const int64_t* cols, int64_t ncols,
                    double* out) {
  int64_t* grp = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nrows > 0 ? nrows : 1));
  int64_t* sel = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nrows > 0 ? nrows : 1));
  double* tmp = (double*)malloc(sizeof(double) * (size_t)(nrows > 0 ? nrows : 1) *
                                (size_t)(ncols > 0 ? ncols : 1));
  if (!grp || !sel || !tmp) {
    free(grp);
    free(sel);
    free(tmp);
    return -1;
  }
  for (int64_t r = 0; r < nrows; ++r) {
    grp[r] = -1;
    for (int32_t g = 0; g < G; ++g)
      if (rows[r] >= off[g] && rows[r] < off[g + 1]) {
        grp[r] = g;
        break;
      }
    if (grp[r] < 0)
      for (int64_t c = 0; c < ncols; ++c)
        out[r * ncols + c] = NAN;
  }
  int rc = 0;
  for (int32_t g = 0; g < G && rc == 0; ++g) {
    int64_t n = 0;
    for (int64_t r = 0; r < nrows; ++r)
      if (grp[r] == g)
        sel[n++] = rows[r];
    if (n == 0)
      continue;
    orc_operand a = {ORC_E4M3, A, lda, sfa, ld_sfa, 1, 128};
    orc_operand b = {ORC_E4M3, B + (size_t)g * (size_t)stride_b, ldb,
                     sfb + (size_t)g * (size_t)stride_sfb, ld_sfb, 128, 128};
    rc = orc_gemm(&a, &b, K, sel, n, cols, ncols, tmp);
    int64_t i = 0;
    for (int64_t r = 0; r < nrows; ++r)
      if (grp[r] == g) {
        memcpy(out + r * ncols, tmp + i * ncols, sizeof(double) * (size_t)ncols);
        ++i;
      }
  }
  free(grp);
  free(sel);
  free(tmp);
  return rc;
}

/* Euclidean norms of dequantised rows (the denominators of the error metric). */
static int orc_row_norms(const orc_operand* op, int64_t K, const int64_t* rows, int64_t nrows,
                         double* out) {
  int failed = 0;
#pragma omp parallel
  {
    double* d = (double*)malloc(sizeof(double) * (size_t)K);
    if (!d) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
      if (!d)
        continue;
      orc_decode_row(op, rows[r], K, d);
      out[r] = sqrt(orc_dot(d, d, K));
    }
    free(d);
  }
  return failed ? -1 : 0;
}

/* fmt: 0 bf16, 1 e4m3, 2 e2m1.  For e4m3 and e2m1, gran_mn / gran_k give the scale
 * granularity of this operand (1/128 and 128/128 for FP8 A and B, 1/32 for FP4). */
int orc_norms(int fmt, const void* data, int64_t ld, const int16_t* sf, int64_t ld_sf,
              int64_t gran_mn, int64_t gran_k, int64_t K, const int64_t* rows, int64_t nrows,
              double* out) {
  orc_operand op = {fmt, data, ld, sf, ld_sf, gran_mn > 0 ? gran_mn : 1,
                    gran_k > 0 ? gran_k : 1};
  return orc_row_norms(&op, K, rows, nrows, out);
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
