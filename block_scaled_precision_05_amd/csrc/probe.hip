// probe.hip -- the sustained matrix-core rate of one gfx950 GPU, for comparison with
// the GEMM kernels (libbsg_probe.so, declared in bsg_probe.h).
//
// Every wave holds the GEMM kernels' register tile: 4 x 2 accumulators of 32 x 32
// fp32 (a 128 x 64 block), and two sets of operand fragments (4 A, 2 B, and their
// scale words), filled once.  It then issues only MFMAs: per round one k-step of
// 8 MFMAs on each fragment set, the accumulators carried from round to round, in
// the order a GEMM k-step issues them (A fragment outer, B fragment inner).  The
// two sets alternate, so the matrix cores' operand inputs change at every MFMA
// much as they do in a GEMM's k-loop.  No memory is touched until the sums are
// written at the end.  Eight waves a workgroup and 160 KiB of LDS reserved make a
// CU run one workgroup, two waves per SIMD: the GEMM kernels' occupancy.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "bsg_probe.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 pb_bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float pb_f32x16_t;
typedef __attribute__((ext_vector_type(8))) int pb_i32x8_t;
typedef __attribute__((ext_vector_type(4))) int pb_i32x4_t;

constexpr int kFM = 4, kFN = 2, kSets = 2, kThreads = 512;
constexpr int kLdsBytes = 160 * 1024;
constexpr int kMaxIters = 1 << 24;

// A 32-bit integer mixing function (the finaliser of MurmurHash3, public domain):
// every output bit depends on every input bit.
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x85ebca6bu;
  x ^= x >> 13;
  x *= 0xc2b2ae35u;
  x ^= x >> 16;
  return x;
}

// Operand word `idx` of this thread: four FP8 codes, eight FP4 codes or two bf16
// values, all 1.0 when seed == 0.
template <int KIND>
__device__ __forceinline__ uint32_t operand_word(uint32_t seed, uint32_t tid, uint32_t idx) {
  if (seed == 0) return KIND == 0 ? 0x3F803F80u : (KIND == 1 ? 0x38383838u : 0x22222222u);
  const uint32_t h = mix32(mix32(seed ^ (tid * 0x9E3779B9u)) + idx * 0x7F4A7C15u);
  if constexpr (KIND == 0) {
    // sign and 7 mantissa bits at random, exponent 124 .. 130: |x| in [2^-3, 2^4)
    auto one = [](uint32_t r) { return (r & 0x807Fu) | ((124u + ((r >> 7) & 0xFFu) % 7u) << 7); };
    return one(h & 0xFFFFu) | (one(h >> 16) << 16);
  } else if constexpr (KIND == 1) {
    // any e4m3 code but the two NaNs (S.1111.111), which become the largest finite
    uint32_t w = h;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if (((w >> (8 * b)) & 0x7Fu) == 0x7Fu) w ^= 1u << (8 * b);
    return w;
  } else {
    return h;   // every e2m1 code is a finite value
  }
}

// A scale word: UE8M0 byte 127 (2^0) when seed == 0, else 119 .. 131 (2^-8 .. 2^4)
// in each byte.
__device__ __forceinline__ uint32_t scale_word(uint32_t seed, uint32_t tid, uint32_t idx) {
  if (seed == 0) return 0x7F7F7F7Fu;
  const uint32_t h = mix32(mix32(seed ^ (tid * 0x85EBCA77u)) + idx * 0xC2B2AE3Du);
  uint32_t w = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) w |= (119u + ((h >> (8 * b)) & 0xFFu) % 13u) << (8 * b);
  return w;
}

template <int KIND>
__global__ __launch_bounds__(kThreads) void mfma_probe_kernel(uint32_t seed, int iters, float* out) {
  // reserved so that a CU holds one workgroup, as the GEMM kernels' ring does
  __shared__ uint8_t lds[kLdsBytes];
  const uint32_t tid = blockIdx.x * kThreads + threadIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) lds[wave * (kLdsBytes / 8)] = 0;

  using frag_t = typename std::conditional<KIND == 0, pb_bf16x8_t, pb_i32x8_t>::type;
  // BF16 fragments are 4 words (8 values), FP8 8 words (32 codes), FP4 4 words (32
  // codes; the MFMA reads the low half of its 8-word operand)
  constexpr int WORDS = KIND == 1 ? 8 : 4;
  frag_t fa[kSets][kFM], fb[kSets][kFN];
  uint32_t sa[kSets][kFM], sb[kSets][kFN];
  uint32_t idx = 0;
#pragma unroll
  for (int s = 0; s < kSets; ++s) {
#pragma unroll
    for (int f = 0; f < kFM + kFN; ++f) {
      pb_i32x8_t w = {};
#pragma unroll
      for (int i = 0; i < WORDS; ++i) w[i] = (int)operand_word<KIND>(seed, tid, idx++);
      frag_t v;
      if constexpr (KIND == 0)
        v = __builtin_bit_cast(pb_bf16x8_t, (pb_i32x4_t){w[0], w[1], w[2], w[3]});
      else
        v = w;
      if (f < kFM) {
        fa[s][f] = v;
        sa[s][f] = scale_word(seed, tid, (uint32_t)(s * 8 + f));
      } else {
        fb[s][f - kFM] = v;
        sb[s][f - kFM] = scale_word(seed, tid, (uint32_t)(s * 8 + f));
      }
    }
  }

  pb_f32x16_t acc[kFM][kFN];
#pragma unroll
  for (int a = 0; a < kFM; ++a)
#pragma unroll
    for (int b = 0; b < kFN; ++b) acc[a][b] = (pb_f32x16_t){};

  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < kSets; ++s)
#pragma unroll
      for (int a = 0; a < kFM; ++a)
#pragma unroll
        for (int b = 0; b < kFN; ++b) {
          if constexpr (KIND == 0)
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[s][b], fa[s][a], acc[a][b], 0, 0, 0);
          else
            acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fb[s][b], fa[s][a], acc[a][b], KIND == 1 ? 0 : 4, KIND == 1 ? 0 : 4, 0, (int)sb[s][b], 0,
                (int)sa[s][a]);
        }
  }

  float sum = 0.0f;
#pragma unroll
  for (int a = 0; a < kFM; ++a)
#pragma unroll
    for (int b = 0; b < kFN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) sum += acc[a][b][r];
  // another wave's byte (zero), read back so that the LDS reservation stays
  __syncthreads();
  sum += (float)lds[((wave + 1) & 7) * (kLdsBytes / 8)];
  out[tid] = sum;
}

}  // namespace

extern "C" int bsg_probe_mfma(int kind, uint32_t seed, int workgroups, int iters, float* out,
                              void* stream) {
  if (kind < 0 || kind > 2 || workgroups < 1 || workgroups > 65535 || iters < 0 || iters > kMaxIters ||
      out == nullptr || ((uintptr_t)out & 3) != 0)
    return BSG_ERR_INVALID_ARG;
  (void)hipGetLastError();
  const dim3 grid((unsigned)workgroups), block(kThreads);
  hipStream_t s = (hipStream_t)stream;
  if (kind == 0)
    hipLaunchKernelGGL(mfma_probe_kernel<0>, grid, block, 0, s, seed, iters, out);
  else if (kind == 1)
    hipLaunchKernelGGL(mfma_probe_kernel<1>, grid, block, 0, s, seed, iters, out);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<2>, grid, block, 0, s, seed, iters, out);
  return hipGetLastError() == hipSuccess ? BSG_OK : BSG_ERR_HIP;
}
