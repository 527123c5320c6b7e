// quant.hip -- per-token block quantisation of bf16 rows into FP8 e4m3 (1x128
// blocks) or FP4 e2m1 (1x32 blocks) with UE8M0 scales, written straight into the
// packed int16, MN-major scale layout the scaled GEMMs read.
//
// The pages describe the scale side of this step: low-precision operands carry
// UE8M0 scale factors that the accelerator expects packed in pairs along K into
// 16-bit integers, MN-major, and converting them on every call costs time
// ("DeepGEMM-Ascend cobre quantas operacoes no Ascend 950?", section "Fatores de
// escala FP8 e o formato UE8M0 no Ascend").  Producing the packed layout in the
// quantiser itself removes that conversion.  How a block's scale is chosen and
// how elements round is not on the pages; the readings (identical to the CPU
// oracle's) are:
//   rule CEIL   : e = smallest integer with amax <= qmax * 2^e (448 e4m3, 6 e2m1);
//   rule OCP_MX : e = floor(log2 amax) - emax (8 e4m3, 2 e2m1), larger values saturate;
//   byte = clamp(e + 127, 0, 254) (all-zero block: 0);
//   code = x / 2^e rounded to the nearest grid value, ties to the even code,
//          saturating at qmax, sign bit copied from x.
//
// The step is HBM-bound (2 bytes read per element, 1 or 1/2 written), so the
// kernel is built for streaming: one workgroup of 4 waves owns 64 rows x 512
// elements; each lane reads 16 bytes (8 elements) of a row, a wave covers the
// 512 elements of one row at a time and keeps its 16 rows' loads in flight
// together.  A block's amax is a max over the 16 (e4m3) or 4 (e2m1) lanes that
// hold it.  The rounding is done in integer and fp32 ALU code, which is free next
// to the memory traffic and exact by construction.  Scale words are gathered in
// LDS as [pair][row] and leave as whole 128-byte rows of the MN-major array.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bsg.h"

namespace bsg_quant {

constexpr int kRows = 64;        // rows per workgroup
constexpr int kCols = 512;       // elements per workgroup row
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = kRows / kWaves;

enum { FMT_E4M3 = 0, FMT_E2M1 = 1 };

template <int FMT>
struct Fmt;
template <>
struct Fmt<FMT_E4M3> {
  static constexpr int GK = 128;        // elements per block
  static constexpr int LANES = GK / 8;  // lanes per block
  static constexpr int QX = 9;          // 448 = 0.875 * 2^9
  static constexpr int QT = 224;        // 0.875 * 256
  static constexpr int EMAX = 8;
};
template <>
struct Fmt<FMT_E2M1> {
  static constexpr int GK = 32;
  static constexpr int LANES = GK / 8;
  static constexpr int QX = 3;          // 6 = 0.75 * 2^3
  static constexpr int QT = 192;        // 0.75 * 256
  static constexpr int EMAX = 2;
};

// Scale byte of a block from its largest bf16 magnitude h (sign bit clear).
// A bf16 magnitude is sig * 2^ex with sig the 8-bit significand (hidden bit
// included) or, below the normal range, the 7-bit fraction at ex = -133.
// Normalising sig to sn in [128, 256) gives floor(log2) p, and amax = sn/256 *
// 2^(p+1), so with qmax = qt/256 * 2^qx the smallest e with amax <= qmax * 2^e
// is p + 1 - qx, plus one when sn > qt.
template <int FMT, int RULE>
__device__ __forceinline__ int scale_byte(uint32_t h) {
  using F = Fmt<FMT>;
  if (h == 0) return 0;
  const uint32_t E = h >> 7;
  const uint32_t sig = E ? (0x80u | (h & 0x7Fu)) : (h & 0x7Fu);
  const int ex = E ? (int)E - 134 : -133;
  const int lz = __clz(sig) - 24;
  const uint32_t sn = sig << lz;
  const int p = 7 - lz + ex;
  const int e = RULE == BSG_SCALE_CEIL ? p + 1 - F::QX + (sn > (uint32_t)F::QT ? 1 : 0)
                                       : p - F::EMAX;
  const int b = e + 127;
  return b < 0 ? 0 : (b > 254 ? 254 : b);
}

// e4m3 code of v, |v| <= 448 after the clamp (round to nearest even).
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t bits = __float_as_uint(v);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = fminf(__uint_as_float(bits & 0x7FFFFFFFu), 448.0f);
  uint32_t mag;
  if (a < 0x1p-6f) {
    // subnormal range: multiples of 2^-9, v_rndne rounds half to even;
    // 8 * 2^-9 = 2^-6 lands on code 8, the smallest normal, as it should
    mag = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    // keep 3 fraction bits, round half to even, re-bias the exponent 127 -> 7
    const uint32_t u = __float_as_uint(a);
    const uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20;
    mag = r - (120u << 3);
  }
  return sign | mag;
}

// e2m1 code of v (round to nearest, ties to the even code, saturating at 6).
// The grid is 0, .5, 1, 1.5, 2, 3, 4, 6 for codes 0..7; each decision point is
// a midpoint, included in the upper code when that code is even.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 28) & 0x8u;
  const float a = fabsf(v);
  uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
               (a >= 3.5f) + (a > 5.0f);
  return sign | c;
}

template <int FMT, int RULE>
__global__ __launch_bounds__(kThreads) void quant_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, uint8_t* __restrict__ Q, int64_t ldq,
    int16_t* __restrict__ sf, int64_t ld_sf, int M, int K) {
  using F = Fmt<FMT>;
  constexpr int KPT = kCols / F::GK / 2;  // packed scale words per row per workgroup
  __shared__ uint16_t words[KPT][kRows];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m0 = blockIdx.x * kRows;
  const int k0 = blockIdx.y * kCols;
  const int k = k0 + lane * 8;
  const bool kin = k < K;
  const int kb_total = K / F::GK;

  // All loads of the wave's rows first, so that they are in flight together.
  uint4 raw[kRowsPerWave];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int r = m0 + wave + i * kWaves;
    raw[i] = make_uint4(0, 0, 0, 0);
    if (kin && r < M) raw[i] = *(const uint4*)(X + (int64_t)r * ldx + k);
  }

#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int rl = wave + i * kWaves;
    const int r = m0 + rl;
    const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
    // largest magnitude of the lane's 8 values, then of the block's lanes
    // (finite bf16 magnitudes order like their bit patterns)
    uint32_t h = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h = max(h, w[j] & 0x7FFFu);
      h = max(h, (w[j] >> 16) & 0x7FFFu);
    }
#pragma unroll
    for (int d = 1; d < F::LANES; d <<= 1) h = max(h, (uint32_t)__shfl_xor((int)h, d));
    const int byte = scale_byte<FMT, RULE>(h);
    const int sh = 127 - byte;  // x / 2^e = ldexp(x, 127 - byte), exact
    if (FMT == FMT_E4M3) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x0 = __uint_as_float(w[j] << 16);
        const float x1 = __uint_as_float(w[j] & 0xFFFF0000u);
        const uint32_t c = e4m3_code(ldexpf(x0, sh)) | (e4m3_code(ldexpf(x1, sh)) << 8);
        if (j < 2) lo |= c << (16 * j);
        else hi |= c << (16 * (j - 2));
      }
      if (kin && r < M) *(uint2*)(Q + (int64_t)r * ldq + k) = make_uint2(lo, hi);
    } else {
      uint32_t q = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x0 = __uint_as_float(w[j] << 16);
        const float x1 = __uint_as_float(w[j] & 0xFFFF0000u);
        q |= (e2m1_code(ldexpf(x0, sh)) | (e2m1_code(ldexpf(x1, sh)) << 4)) << (8 * j);
      }
      if (kin && r < M) *(uint32_t*)(Q + (int64_t)r * ldq + k / 2) = q;
    }
    // pack the block pair's bytes: the even block's lanes hold the low byte
    const int hb = __shfl_down(byte, F::LANES);
    if ((lane % (2 * F::LANES)) == 0) {
      const int blk = (k0 / F::GK) + lane / F::LANES;  // even block of the pair
      const uint32_t hi = (blk + 1 < kb_total) ? (uint32_t)hb : 0x7Fu;
      words[lane / (2 * F::LANES)][rl] = (uint16_t)(byte | (hi << 8));
    }
  }
  __syncthreads();
  const int kp0 = k0 / (2 * F::GK);
  const int kp_total = (kb_total + 1) / 2;
  for (int t = threadIdx.x; t < KPT * kRows; t += kThreads) {
    const int kp = t / kRows, rl = t % kRows;
    if (kp0 + kp < kp_total && m0 + rl < M)
      sf[(int64_t)(kp0 + kp) * ld_sf + m0 + rl] = (int16_t)words[kp][rl];
  }
}

template <int FMT>
static int launch(const void* X, int64_t ldx, void* Q, int64_t ldq, int16_t* sf, int64_t ld_sf,
                  int64_t M, int64_t K, int32_t rule, hipStream_t stream) {
  const dim3 grid((unsigned)((M + kRows - 1) / kRows), (unsigned)((K + kCols - 1) / kCols));
  (void)hipGetLastError();
  if (rule == BSG_SCALE_CEIL)
    hipLaunchKernelGGL((quant_kernel<FMT, BSG_SCALE_CEIL>), grid, dim3(kThreads), 0, stream,
                       (const uint16_t*)X, ldx, (uint8_t*)Q, ldq, sf, ld_sf, (int)M, (int)K);
  else
    hipLaunchKernelGGL((quant_kernel<FMT, BSG_SCALE_OCP_MX>), grid, dim3(kThreads), 0, stream,
                       (const uint16_t*)X, ldx, (uint8_t*)Q, ldq, sf, ld_sf, (int)M, (int)K);
  return hipGetLastError() == hipSuccess ? BSG_OK : BSG_ERR_HIP;
}

// Shared argument checks.  q_row_bytes: bytes of Q per row; q_align: store width.
static int check(const void* X, int64_t ldx, const void* Q, int64_t ldq, const int16_t* sf,
                 int64_t ld_sf, int64_t M, int64_t K, int32_t rule, int64_t gk, int64_t q_row_bytes,
                 int64_t q_align) {
  if (M < 0 || K < 0) return BSG_ERR_INVALID_ARG;
  if (rule != BSG_SCALE_CEIL && rule != BSG_SCALE_OCP_MX) return BSG_ERR_INVALID_ARG;
  if (K % gk) return BSG_ERR_UNSUPPORTED_SHAPE;
  if (M == 0 || K == 0) return BSG_OK;
  if (M > INT32_MAX || K > INT32_MAX) return BSG_ERR_UNSUPPORTED_SHAPE;
  if ((M + kRows - 1) / kRows > INT32_MAX || (K + kCols - 1) / kCols > 65535)
    return BSG_ERR_UNSUPPORTED_SHAPE;
  if (!X || !Q || !sf) return BSG_ERR_INVALID_ARG;
  if (ldx < K || ldq < q_row_bytes || ld_sf < M) return BSG_ERR_INVALID_ARG;
  if (((uintptr_t)X & 15) || (ldx % 8)) return BSG_ERR_MISALIGNED;
  if (((uintptr_t)Q & (q_align - 1)) || (ldq % q_align)) return BSG_ERR_MISALIGNED;
  if ((uintptr_t)sf & 1) return BSG_ERR_MISALIGNED;
  return BSG_OK;
}

}  // namespace bsg_quant

using namespace bsg_quant;

extern "C" {

int quantize_fp8_per_token(const void* X, int64_t ldx, void* Q, int64_t ldq, int16_t* sf,
                           int64_t ld_sf, int64_t M, int64_t K, int32_t rule, void* stream) {
  const int st = check(X, ldx, Q, ldq, sf, ld_sf, M, K, rule, 128, K, 8);
  if (st != BSG_OK || M == 0 || K == 0) return st;
  return launch<FMT_E4M3>(X, ldx, Q, ldq, sf, ld_sf, M, K, rule, (hipStream_t)stream);
}

int quantize_fp4_per_token(const void* X, int64_t ldx, void* Q, int64_t ldq, int16_t* sf,
                           int64_t ld_sf, int64_t M, int64_t K, int32_t rule, void* stream) {
  const int st = check(X, ldx, Q, ldq, sf, ld_sf, M, K, rule, 32, K / 2, 4);
  if (st != BSG_OK || M == 0 || K == 0) return st;
  return launch<FMT_E2M1>(X, ldx, Q, ldq, sf, ld_sf, M, K, rule, (hipStream_t)stream);
}

}  // extern "C"
