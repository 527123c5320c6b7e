// quant_math.h -- the per-block arithmetic of the FP8 / FP4 quantisers (scale
// byte from a block's amax, block max across lanes, SwiGLU), shared by the
// quantiser kernels and by the GEMM epilogue that applies SwiGLU and FP8
// requantisation to an up-projection tile, so both produce the same bits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bsg.h"

namespace bsg_qm {

typedef __attribute__((ext_vector_type(2))) short qm_short2_t;
typedef __attribute__((ext_vector_type(2))) uint32_t qm_u32x2_t;
typedef __attribute__((ext_vector_type(4))) uint32_t qm_u32x4_t;

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

// Scale byte of a block from its largest magnitude, given as fp32 bits a (sign
// bit clear; a bf16 magnitude h is a = h << 16).  The magnitude is sig * 2^ex
// with sig the 24-bit significand (hidden bit included) or, below the normal
// range, the 23-bit fraction at ex = -149.  Normalising sig to sn in [2^23,
// 2^24) gives floor(log2) p, and amax = sn/2^24 * 2^(p+1); with qmax = qt/256 *
// 2^qx the smallest e with amax <= qmax * 2^e is p + 1 - qx, plus one when
// sn > qt * 2^16.  a == 0 needs no branch: clz gives 32, p = -150 and the byte
// clamps to 0.
template <int FMT, int RULE>
__device__ __forceinline__ int scale_byte(uint32_t a) {
  using F = Fmt<FMT>;
  const uint32_t E = a >> 23;
  const uint32_t sig = E ? (0x800000u | (a & 0x7FFFFFu)) : (a & 0x7FFFFFu);
  const int ex = E ? (int)E - 150 : -149;
  const int lz = __clz(sig) - 8;
  const uint32_t sn = sig << lz;
  const int p = 23 - lz + ex;
  const int e = RULE == BSG_SCALE_CEIL
                    ? p + 1 - F::QX + (sn > ((uint32_t)F::QT << 16) ? 1 : 0)
                    : p - F::EMAX;
  const int b = e + 127;
  return b < 0 ? 0 : (b > 254 ? 254 : b);
}

// 2^(byte-127) as an fp32 (byte 0 is the subnormal 2^-127).
__device__ __forceinline__ float scale_f32(int byte) {
  return __uint_as_float(byte ? ((uint32_t)byte << 23) : 0x00400000u);
}

// Max over the lanes of one block: 16 lanes (e4m3) or 4 (e2m1), all DPP moves.
// quad_perm [1,0,3,2] and [2,3,0,1] make a quad uniform; row_ror 4 and 8 then
// combine the four quads of a 16-lane row.
template <int LANES>
__device__ __forceinline__ uint32_t block_max(uint32_t h) {
  h = max(h, (uint32_t)__builtin_amdgcn_mov_dpp((int)h, 0xB1, 0xF, 0xF, false));
  h = max(h, (uint32_t)__builtin_amdgcn_mov_dpp((int)h, 0x4E, 0xF, 0xF, false));
  if (LANES == 16) {
    h = max(h, (uint32_t)__builtin_amdgcn_mov_dpp((int)h, 0x124, 0xF, 0xF, false));
    h = max(h, (uint32_t)__builtin_amdgcn_mov_dpp((int)h, 0x128, 0xF, 0xF, false));
  }
  return h;
}

__device__ __forceinline__ float silu_f32(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + expf(-g));
}

// SwiGLU of eight consecutive elements of one 128-wide block and their FP8 e4m3
// codes: g and u hold eight bf16 values each (two per word, the lower element in
// the low half); y = silu(g) * u in fp32, the block's scale byte from the amax over
// the 16 lanes that hold the block (rule RULE), codes = y / 2^(byte-127) by the
// gfx950 scaled conversion (OCP_MX: saturated at 448 first).
template <int RULE>
__device__ __forceinline__ void swiglu_fp8x8(const qm_u32x4_t& gr, const qm_u32x4_t& ur, qm_u32x2_t& v,
                                             int& byte) {
  using F = Fmt<FMT_E4M3>;
  float y[8];
  uint32_t a = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t g = gr[j], u = ur[j];
    y[2 * j] = silu_f32(__uint_as_float(g << 16)) * __uint_as_float(u << 16);
    y[2 * j + 1] = silu_f32(__uint_as_float(g & 0xFFFF0000u)) * __uint_as_float(u & 0xFFFF0000u);
    a = max(a, __float_as_uint(y[2 * j]) & 0x7FFFFFFFu);
    a = max(a, __float_as_uint(y[2 * j + 1]) & 0x7FFFFFFFu);
  }
  a = block_max<F::LANES>(a);
  byte = scale_byte<FMT_E4M3, RULE>(a);
  const float sc = scale_f32(byte);
  if (RULE == BSG_SCALE_OCP_MX) {
    // saturate at 448 * sc before the conversion (which would give NaN)
    const float lim = 448.0f * sc;
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = __builtin_copysignf(fminf(fabsf(y[j]), lim), y[j]);
  }
  qm_short2_t lo = {0, 0}, hi = {0, 0};
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, y[0], y[1], sc, false);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, y[2], y[3], sc, true);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, y[4], y[5], sc, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, y[6], y[7], sc, true);
  v = (qm_u32x2_t){__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

}  // namespace bsg_qm
