// mqa.hip -- MQA logits of a lightning-indexer step, FP8 e4m3 and FP4 e2m1 operands
// with UE8M0 block scales, on gfx950.
//
// The pages list "MQA logits" among the library's kernels: attention scores of
// multi-query attention on the DeepSeek Lightning Indexer path, benchmarked for
// prefill and decode in FP8 and FP4 (first page, "DeepGEMM-Ascend cobre quantas
// operacoes no Ascend 950?", section "Cobertura de operacoes e a lacuna declarada
// no repositorio"; third page, section "Kernels especificos de modelo: logits de
// MQA e prenorm mHC").  They do not define the computation; the reading is the
// indexer's published score: query token t has H heads q[t][h] of dimension 128 and
// weights w[t][h], all heads share the key k[s], and
//     L[t][s] = sum_h w[t][h] * max(0, q[t][h] . k[s])   for ks[t] <= s < ke[t],
//     L[t][s] = -inf                                        for the other s < S.
//
// Mapping onto the matrix cores.  One wave owns one query: its H heads are the
// rows of the scaled MFMA (32 heads per fragment), 32 keys its columns, and the
// two 64-wide k-steps cover the head dimension.  In the 32x32 accumulator a lane
// holds one key (lane % 32) and 16 heads, so the weighted sum over heads is 16
// fused multiply-adds per fragment in the lane plus one add across the wave's
// halves; no LDS and no barriers.  The four waves of a workgroup take four
// consecutive queries over the same keys: queries of one sequence read the same
// key rows, which the CU's caches then serve.  The query fragments and the
// weights stay in registers for the wave's whole key range; key fragments are
// read straight from memory into registers (16-byte buffer loads), the next
// fragment's loads issued before the current fragment's MFMAs.  Block scales
// enter as the MFMA's per-lane scale operands, exact powers of two.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/bsg.h"

namespace bsg_mqa {

typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;

constexpr int kD = 128;            // head dimension
constexpr int kWaves = 4;          // queries per workgroup
constexpr int kKeysPerWg = 512;    // keys per workgroup (16 fragments of 32)
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(lo | (hi << 32)), (short)0,
                                           __builtin_amdgcn_readfirstlane((int)bytes), kRsrcWord3);
}

struct MqaArgs {
  const uint8_t* Q;       // [T*H][ldq] codes
  const int16_t* sfq;     // packed [kp][ld_sfq] over the T*H rows
  const uint8_t* K;       // [k_rows][ldk] codes
  const int16_t* sfk;     // packed [kp][ld_sfk] over K's rows
  const float* W;         // [T][ldw]
  const int32_t* ks;      // [T]
  const int32_t* ke;      // [T]
  float* L;               // [T][ldl]
  int64_t ldq, ld_sfq, ldk, ld_sfk, ldw, ldl;
  int64_t group_rows;     // key rows between consecutive groups
  int32_t T, S, H;
  int32_t q_per_group;
  int32_t k_rows;         // rows of K the calls may read
};

// FMT 0: e4m3, 32 bytes of a row per lane per k-step, one scale per row (the
// head dimension is one 128-wide block).  FMT 4: e2m1, 16 bytes per lane per
// k-step, one scale per 32 elements: lane half lg of k-step j holds block 2j + lg,
// which is byte lg of packed row j.
template <int FMT, int HF>
__global__ __launch_bounds__(64 * kWaves) void mqa_logits_kernel(const MqaArgs a) {
  constexpr bool FP4 = FMT == 4;
  constexpr int ROW_BYTES = FP4 ? kD / 2 : kD;     // bytes of one head or key row
  constexpr int KS = 2;                             // k-steps of 64 elements
  constexpr int STEP_BYTES = ROW_BYTES / KS;        // bytes of a row per k-step
  constexpr int LANE_BYTES = STEP_BYTES / 2;        // bytes per lane per k-step
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, lg = lane >> 5;
  const int t = blockIdx.y * kWaves + wave;
  if (t >= a.T) return;
  const int s0 = blockIdx.x * kKeysPerWg;
  const int s_end = s0 + kKeysPerWg < a.S ? s0 + kKeysPerWg : a.S;
  // The query's window inside this workgroup's keys (clamped to [0, S]).
  int lo = __builtin_amdgcn_readfirstlane(a.ks[t]);
  int hi = __builtin_amdgcn_readfirstlane(a.ke[t]);
  lo = lo < s0 ? s0 : (lo > s_end ? s_end : lo);
  hi = hi > s_end ? s_end : (hi < lo ? lo : hi);
  float* const out = a.L + (int64_t)t * a.ldl;
  const float ninf = -__builtin_inff();
  // keys of this range outside the window: -inf
  for (int s = s0 + lane; s < s_end; s += 64)
    if (s < lo || s >= hi) out[s] = ninf;
  if (lo >= hi) return;

  // Query fragments and their scales: head row hf*32 + l32, bytes of k-step j.
  const int64_t qrow0 = (int64_t)t * a.H;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.Q + qrow0 * a.ldq, (uint32_t)(a.H * a.ldq));
  i32x4_t qf[HF][KS][FP4 ? 1 : 2];
  uint32_t qs[HF][KS];
#pragma unroll
  for (int hf = 0; hf < HF; ++hf) {
    const uint32_t rowoff = (uint32_t)((hf * 32 + l32) * a.ldq);
#pragma unroll
    for (int j = 0; j < KS; ++j) {
#pragma unroll
      for (int c = 0; c < (FP4 ? 1 : 2); ++c)
        qf[hf][j][c] = __builtin_amdgcn_raw_buffer_load_b128(
            rq, rowoff + j * STEP_BYTES + lg * LANE_BYTES + 16 * c, 0, 0);
      const int64_t row = qrow0 + hf * 32 + l32;
      const uint32_t word = (uint16_t)a.sfq[(FP4 ? j : 0) * a.ld_sfq + row];
      qs[hf][j] = FP4 ? (word >> (8 * lg)) : word;
    }
  }
  // Weights of the heads this lane's accumulator registers hold: register r of
  // fragment hf is head hf*32 + 8*(r/4) + 4*lg + r%4.
  float wv[HF][16];
  const float* wrow = a.W + (int64_t)t * a.ldw;
#pragma unroll
  for (int hf = 0; hf < HF; ++hf)
#pragma unroll
    for (int r = 0; r < 16; ++r) wv[hf][r] = wrow[hf * 32 + 8 * (r / 4) + 4 * lg + r % 4];

  // Keys of the query's group: rows g*group_rows + s for s < S (rows past S read 0).
  const int64_t krow0 = (int64_t)(t / a.q_per_group) * a.group_rows;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.K + krow0 * a.ldk, (uint32_t)(a.S * a.ldk));
  const __amdgpu_buffer_rsrc_t rsk =
      make_rsrc(a.sfk, (uint32_t)(2 * ((int64_t)(FP4 ? 1 : 0) * a.ld_sfk + a.k_rows)));

  i32x4_t kf[2][KS][FP4 ? 1 : 2];
  uint32_t ksw[2][KS];
  auto load_keys = [&](int buf, int f0) {
    const int key = f0 + l32;
    const uint32_t rowoff = (uint32_t)(key * a.ldk);
#pragma unroll
    for (int j = 0; j < KS; ++j) {
#pragma unroll
      for (int c = 0; c < (FP4 ? 1 : 2); ++c)
        kf[buf][j][c] = __builtin_amdgcn_raw_buffer_load_b128(
            rk, rowoff + j * STEP_BYTES + lg * LANE_BYTES + 16 * c, 0, 0);
      const uint32_t soff = (uint32_t)(2 * ((FP4 ? j : 0) * a.ld_sfk + krow0 + key));
      const uint32_t word = __builtin_amdgcn_raw_buffer_load_b16(rsk, soff, 0, 0);
      ksw[buf][j] = FP4 ? (word >> (8 * lg)) : word;
    }
  };

  const int f_begin = lo & ~31, f_end = hi;
  load_keys(0, f_begin);
  int buf = 0;
#pragma unroll 1
  for (int f0 = f_begin; f0 < f_end; f0 += 32) {
    if (f0 + 32 < f_end) load_keys(buf ^ 1, f0 + 32);
    f32x16_t acc[HF];
#pragma unroll
    for (int hf = 0; hf < HF; ++hf) {
      acc[hf] = (f32x16_t){};
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        i32x8_t qa, kb;
        if constexpr (FP4) {
          qa = (i32x8_t){qf[hf][j][0][0], qf[hf][j][0][1], qf[hf][j][0][2], qf[hf][j][0][3], 0, 0, 0, 0};
          kb = (i32x8_t){kf[buf][j][0][0], kf[buf][j][0][1], kf[buf][j][0][2], kf[buf][j][0][3], 0, 0, 0, 0};
        } else {
          qa = (i32x8_t){qf[hf][j][0][0], qf[hf][j][0][1], qf[hf][j][0][2], qf[hf][j][0][3],
                         qf[hf][j][1][0], qf[hf][j][1][1], qf[hf][j][1][2], qf[hf][j][1][3]};
          kb = (i32x8_t){kf[buf][j][0][0], kf[buf][j][0][1], kf[buf][j][0][2], kf[buf][j][0][3],
                         kf[buf][j][1][0], kf[buf][j][1][1], kf[buf][j][1][2], kf[buf][j][1][3]};
        }
        // rows of the product: heads (operand A), columns: keys (operand B)
        acc[hf] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa, kb, acc[hf], FMT, FMT, 0,
                                                                  (int)qs[hf][j], 0, (int)ksw[buf][j]);
      }
    }
    // sum over heads of w * max(0, score): 16 heads per register set in this lane,
    // the other 16 of each fragment in lane l ^ 32
    float v = 0.0f;
#pragma unroll
    for (int hf = 0; hf < HF; ++hf)
#pragma unroll
      for (int r = 0; r < 16; ++r) v = __builtin_fmaf(wv[hf][r], __builtin_fmaxf(acc[hf][r], 0.0f), v);
    v += __shfl_xor(v, 32, 64);
    const int s = f0 + l32;
    if (lg == 0 && s >= lo && s < hi) out[s] = v;
    buf ^= 1;
  }
}

// Host side: argument checks and the launch.
static int check(int fmt, const void* Q, int64_t ldq, const int16_t* sfq, int64_t ld_sfq,
                 const void* K, int64_t ldk, const int16_t* sfk, int64_t ld_sfk, const float* W,
                 int64_t ldw, const int32_t* ks, const int32_t* ke, const float* L, int64_t ldl,
                 int64_t T, int64_t S, int32_t H, int64_t q_per_group, int64_t group_rows,
                 int64_t* k_rows) {
  if (T < 0 || S < 0 || H < 0 || q_per_group < 1 || group_rows < 0) return BSG_ERR_INVALID_ARG;
  if (T == 0 || S == 0) return BSG_OK;
  if (H == 0 || H % 32 || H > 128) return BSG_ERR_UNSUPPORTED_SHAPE;
  const int64_t row_bytes = fmt == 4 ? kD / 2 : kD;
  const int64_t groups = (T + q_per_group - 1) / q_per_group;
  *k_rows = (groups - 1) * group_rows + S;
  if (T * H > INT32_MAX || S > INT32_MAX || *k_rows > INT32_MAX) return BSG_ERR_UNSUPPORTED_SHAPE;
  if (!Q || !sfq || !K || !sfk || !W || !ks || !ke || !L) return BSG_ERR_INVALID_ARG;
  if (ldq < row_bytes || ldk < row_bytes || ldw < H || ldl < S) return BSG_ERR_INVALID_ARG;
  if (ld_sfq < T * H || ld_sfk < *k_rows) return BSG_ERR_INVALID_ARG;
  // byte offsets inside one query's rows, one group's keys and the scale arrays stay
  // below 2^31
  if (H * ldq >= (int64_t(1) << 31) || S * ldk >= (int64_t(1) << 31) ||
      2 * (ld_sfk + *k_rows) >= (int64_t(1) << 31))
    return BSG_ERR_UNSUPPORTED_SHAPE;
  if (((uintptr_t)Q & 15) || ((uintptr_t)K & 15) || (ldq % 16) || (ldk % 16))
    return BSG_ERR_MISALIGNED;
  if (((uintptr_t)sfq & 1) || ((uintptr_t)sfk & 1) || ((uintptr_t)W & 3) || ((uintptr_t)L & 3))
    return BSG_ERR_MISALIGNED;
  return BSG_OK;
}

template <int FMT>
static int launch(const void* Q, int64_t ldq, const int16_t* sfq, int64_t ld_sfq, const void* K,
                  int64_t ldk, const int16_t* sfk, int64_t ld_sfk, const float* W, int64_t ldw,
                  const int32_t* ks, const int32_t* ke, float* L, int64_t ldl, int64_t T, int64_t S,
                  int32_t H, int64_t q_per_group, int64_t group_rows, void* stream) {
  int64_t k_rows = 0;
  const int st = check(FMT, Q, ldq, sfq, ld_sfq, K, ldk, sfk, ld_sfk, W, ldw, ks, ke, L, ldl, T, S,
                       H, q_per_group, group_rows, &k_rows);
  if (st != BSG_OK || T == 0 || S == 0) return st;
  MqaArgs a = {};
  a.Q = (const uint8_t*)Q;
  a.sfq = sfq;
  a.K = (const uint8_t*)K;
  a.sfk = sfk;
  a.W = W;
  a.ks = ks;
  a.ke = ke;
  a.L = L;
  a.ldq = ldq;
  a.ld_sfq = ld_sfq;
  a.ldk = ldk;
  a.ld_sfk = ld_sfk;
  a.ldw = ldw;
  a.ldl = ldl;
  a.group_rows = group_rows;
  a.T = (int32_t)T;
  a.S = (int32_t)S;
  a.H = H;
  a.q_per_group = (int32_t)(q_per_group < T ? q_per_group : T);
  a.k_rows = (int32_t)k_rows;
  const dim3 grid((unsigned)((S + kKeysPerWg - 1) / kKeysPerWg), (unsigned)((T + kWaves - 1) / kWaves));
  if (grid.y > 65535) return BSG_ERR_UNSUPPORTED_SHAPE;
  (void)hipGetLastError();
  switch (H / 32) {
    case 1: hipLaunchKernelGGL((mqa_logits_kernel<FMT, 1>), grid, dim3(64 * kWaves), 0, (hipStream_t)stream, a); break;
    case 2: hipLaunchKernelGGL((mqa_logits_kernel<FMT, 2>), grid, dim3(64 * kWaves), 0, (hipStream_t)stream, a); break;
    case 3: hipLaunchKernelGGL((mqa_logits_kernel<FMT, 3>), grid, dim3(64 * kWaves), 0, (hipStream_t)stream, a); break;
    default: hipLaunchKernelGGL((mqa_logits_kernel<FMT, 4>), grid, dim3(64 * kWaves), 0, (hipStream_t)stream, a); break;
  }
  return hipGetLastError() == hipSuccess ? BSG_OK : BSG_ERR_HIP;
}

}  // namespace bsg_mqa

extern "C" {

int mqa_logits_fp8(const void* Q, int64_t ldq, const int16_t* sfq, int64_t ld_sfq, const void* K,
                   int64_t ldk, const int16_t* sfk, int64_t ld_sfk, const float* W, int64_t ldw,
                   const int32_t* ks, const int32_t* ke, float* L, int64_t ldl, int64_t T, int64_t S,
                   int32_t H, int64_t q_per_group, int64_t group_rows, void* stream) {
  return bsg_mqa::launch<0>(Q, ldq, sfq, ld_sfq, K, ldk, sfk, ld_sfk, W, ldw, ks, ke, L, ldl, T, S, H,
                            q_per_group, group_rows, stream);
}

int mqa_logits_fp4(const void* Q, int64_t ldq, const int16_t* sfq, int64_t ld_sfq, const void* K,
                   int64_t ldk, const int16_t* sfk, int64_t ld_sfk, const float* W, int64_t ldw,
                   const int32_t* ks, const int32_t* ke, float* L, int64_t ldl, int64_t T, int64_t S,
                   int32_t H, int64_t q_per_group, int64_t group_rows, void* stream) {
  return bsg_mqa::launch<4>(Q, ldq, sfq, ld_sfq, K, ldk, sfk, ld_sfk, W, ldw, ks, ke, L, ldl, T, S, H,
                            q_per_group, group_rows, stream);
}

}  // extern "C"
