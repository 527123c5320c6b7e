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
// halves.  The query fragments and the weights stay in registers for the wave's
// whole key range; keys stream through an LDS ring (below), shared by the four
// waves of a workgroup when their queries read the same keys.  Block scales enter
// as the MFMA's per-lane scale operands, exact powers of two.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "../../include/bsg.h"

namespace bsg_mqa {

typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kD = 128;            // head dimension
constexpr int kWaves = 4;          // queries per workgroup
// Keys per workgroup: a multiple of every chunk (32 FP8 or 64 FP4 keys) and of 64
// (the -inf fill's stride); the launcher picks it (below).
constexpr int kKeysPerWgMin = 1024;
constexpr int kKeysPerWgMax = 4096;
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(lo | (hi << 32)), (short)0,
                                           __builtin_amdgcn_readfirstlane((int)bytes), kRsrcWord3);
}

__device__ __forceinline__ float relu(float x) {
  const int b = __builtin_bit_cast(int, x);
  return __builtin_bit_cast(float, b > 0 ? b : 0);
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
  int32_t keys_per_wg;    // keys of one workgroup's range
};

// FMT 0: e4m3 rows of 128 bytes, one scale per row (the head dimension is one
// 128-wide block), 32 bytes per lane per k-step.  FMT 4: e2m1 rows of 64 bytes, one
// scale per 32 elements, 16 bytes per lane per k-step: lane half lg of k-step j
// holds block 2j + lg, which is byte lg of packed row j.
//
// Keys go through an LDS ring of NB chunks of 4 KiB (32 FP8 or 64 FP4 key rows).
// A chunk is filled by 1 KiB direct-to-LDS copies of whole rows (16 bytes a lane,
// 8 or 16 rows a copy), so one copy instruction touches 8 or 16 cache lines; read
// straight in the MFMA operand layout, every load would touch 32 rows.  Each row's
// 16-byte chunks are XOR-swizzled by (row / RPS) % NC so that the 16 lanes of one
// ds_read_b128 phase hit all 64 banks once.  SHARED (the four queries of the
// workgroup read the same keys, as in prefill): each wave copies a quarter of every
// chunk and a workgroup barrier per chunk hands it to all four; otherwise (decode:
// every query its own keys) each wave streams its own keys through its own ring.
template <int FMT, int HF, bool SHARED>
__global__ __launch_bounds__(64 * kWaves) void mqa_logits_kernel(const MqaArgs a) {
  constexpr bool FP4 = FMT == 4;
  constexpr int ROW_BYTES = FP4 ? kD / 2 : kD;     // bytes of one head or key row
  constexpr int KS = 2;                             // k-steps of 64 elements
  constexpr int STEP_BYTES = ROW_BYTES / KS;        // bytes of a row per k-step
  constexpr int NC = ROW_BYTES / 16;                // 16-byte chunks per row
  constexpr int RPS = 16 / NC;                      // rows sharing one swizzle value
  constexpr int CHUNK_BYTES = 4096;
  constexpr int CK = CHUNK_BYTES / ROW_BYTES;       // keys per chunk
  constexpr int NF = CK / 32;                       // MFMA key fragments per chunk
  constexpr int ROWS_PER_COPY = 1024 / ROW_BYTES;
  constexpr int COPIES = SHARED ? 1 : 4;            // 1 KiB copies per wave per chunk
  // chunks in the ring: NB - 1 in flight while one is read; a wave streaming its
  // own keys keeps 16 KiB in flight (two workgroups per CU, 128 KiB per CU)
  constexpr int NB = SHARED ? 4 : 5;
  constexpr int RING_BYTES = NB * CHUNK_BYTES;
  constexpr int SCALES = NF * (FP4 ? KS : 1);       // scale-word loads per wave per chunk
  constexpr int VM = SCALES + COPIES;               // vector memory ops per wave per chunk
  static_assert((NB - 2) * VM <= 63, "the loads in flight fit the vmcnt field");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[(SHARED ? 1 : kWaves) * RING_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, lg = lane >> 5;
  // Query blocks in reverse order: under causal windows the last queries have the
  // most keys, so the longest workgroups start first and the short ones fill the
  // tail (3% faster on the 4096-token prefill).
  const int t0 = (gridDim.y - 1 - blockIdx.y) * kWaves;
  const int t = t0 + wave;
  const bool valid = t < a.T;
  if (!SHARED && !valid) return;
  const int s0 = blockIdx.x * a.keys_per_wg;
  const int s_end = s0 + a.keys_per_wg < a.S ? s0 + a.keys_per_wg : a.S;
  auto window = [&](int q, int& lo, int& hi) {
    lo = __builtin_amdgcn_readfirstlane(a.ks[q]);
    hi = __builtin_amdgcn_readfirstlane(a.ke[q]);
    lo = lo < s0 ? s0 : (lo > s_end ? s_end : lo);
    hi = hi > s_end ? s_end : (hi < lo ? lo : hi);
  };
  // This query's window inside the workgroup's keys (clamped to [0, S]); the
  // keys of the range outside it are -inf.
  int lo = s0, hi = s0;
  if (valid) {
    window(t, lo, hi);
    float* const row = a.L + (int64_t)t * a.ldl;
    for (int s = s0 + lane; s < s_end; s += 64)
      if (s < lo || s >= hi) row[s] = -__builtin_inff();
  }
  // The chunks to stream: the union of the workgroup's windows when the waves
  // share keys (every wave then runs the same chunks and barriers), else its own.
  int ulo = lo, uhi = hi;
  if constexpr (SHARED) {
    ulo = s_end;
    uhi = s0;
    for (int w = 0; w < kWaves && t0 + w < a.T; ++w) {
      int l2, h2;
      window(t0 + w, l2, h2);
      if (l2 < h2) {
        ulo = l2 < ulo ? l2 : ulo;
        uhi = h2 > uhi ? h2 : uhi;
      }
    }
  }
  if (ulo >= uhi) return;   // uniform over the workgroup when SHARED

  // Query fragments and their scales (head row hf*32 + l32, bytes of k-step j) and
  // the weights of the heads this lane's accumulator registers hold: register r of
  // fragment hf is head hf*32 + 8*(r/4) + 4*lg + r%4.  Issued before any key copy,
  // so the loop's explicit waits never count them.
  i32x4_t qf[HF][KS][FP4 ? 1 : 2];
  uint32_t qs[HF][KS];
  float wv[HF][16];
  if (valid) {
    const int64_t qrow0 = (int64_t)t * a.H;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.Q + qrow0 * a.ldq, (uint32_t)(a.H * a.ldq));
#pragma unroll
    for (int hf = 0; hf < HF; ++hf) {
      const uint32_t rowoff = (uint32_t)((hf * 32 + l32) * a.ldq);
#pragma unroll
      for (int j = 0; j < KS; ++j) {
#pragma unroll
        for (int c = 0; c < (FP4 ? 1 : 2); ++c)
          qf[hf][j][c] = __builtin_amdgcn_raw_buffer_load_b128(
              rq, rowoff + j * STEP_BYTES + lg * (STEP_BYTES / 2) + 16 * c, 0, 0);
        const uint32_t word = (uint16_t)a.sfq[(FP4 ? j : 0) * a.ld_sfq + qrow0 + hf * 32 + l32];
        qs[hf][j] = FP4 ? (word >> (8 * lg)) : word;
      }
    }
    // registers 4i .. 4i+3 hold four consecutive heads: one 16-byte load each
    // (W rows are 16-byte aligned when ldw is a multiple of 4, else 4-byte loads)
    const float* wrow = a.W + (int64_t)t * a.ldw;
    const bool w16 = (((uintptr_t)wrow) & 15) == 0;
#pragma unroll
    for (int hf = 0; hf < HF; ++hf)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float* p = wrow + hf * 32 + 8 * i + 4 * lg;
        if (w16) {
          const f32x4_t v = *(const f32x4_t*)p;
#pragma unroll
          for (int e = 0; e < 4; ++e) wv[hf][4 * i + e] = v[e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) wv[hf][4 * i + e] = p[e];
        }
      }
  }

  // Keys of the query's group: rows g*group_rows + s for s < S (rows past S read
  // zero).  Shared waves all read the workgroup's group.
  const int64_t krow0 = (int64_t)((SHARED ? t0 : t) / a.q_per_group) * a.group_rows;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.K + krow0 * a.ldk, (uint32_t)(a.S * a.ldk));
  const __amdgpu_buffer_rsrc_t rsk =
      make_rsrc(a.sfk, (uint32_t)(2 * ((int64_t)(FP4 ? 1 : 0) * a.ld_sfk + a.k_rows)));
  uint8_t* const ring = smem + (SHARED ? 0 : wave * RING_BYTES);
  const int c_begin = ulo / CK * CK;
  const int nch = (uhi - c_begin + CK - 1) / CK;
  // Copy lanes: lane l of copy ci writes 16 bytes at 16*l of its 1 KiB: chunk row
  // ci*ROWS_PER_COPY + l / NC, physical chunk l % NC, which holds the logical chunk
  // (l % NC) ^ swizzle(row).
  const int cp_row = lane / NC;

  uint32_t ksw[NB][NF][KS];
  // Chunk c into ring slot sl: the scale words of its keys first, then the copies
  // (the loop's waits count on that order).
  auto issue = [&](auto slot, int c) {
    constexpr int sl = decltype(slot)::value;
    const int key0 = c_begin + c * CK;
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        if (FP4 || j == 0) {
          const uint32_t soff = (uint32_t)(2 * ((FP4 ? j : 0) * a.ld_sfk + krow0 + key0 + f * 32 + l32));
          const uint32_t word = __builtin_amdgcn_raw_buffer_load_b16(rsk, soff, 0, 0);
          ksw[sl][f][j] = FP4 ? (word >> (8 * lg)) : word;
        } else {
          ksw[sl][f][j] = ksw[sl][f][0];
        }
      }
#pragma unroll
    for (int q = 0; q < COPIES; ++q) {
      const int ci = SHARED ? wave : q;                   // copy index within the chunk
      const int row = ci * ROWS_PER_COPY + cp_row;
      const int lc = (lane % NC) ^ ((row / RPS) % NC);
      const uint32_t off = (uint32_t)(key0 + row) * (uint32_t)a.ldk + 16u * (uint32_t)lc;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rk, (__attribute__((address_space(3))) void*)(ring + sl * CHUNK_BYTES + ci * 1024), 16, off,
          0, 0, 0);
    }
  };
  // LDS offset of logical 16-byte chunk lc of key row r of a chunk.
  auto lds_at = [&](int r, int lc) { return r * ROW_BYTES + 16 * (lc ^ ((r / RPS) % NC)); };

  // One chunk: for each of its fragments, the scores (heads x 32 keys), the
  // weighted max-sum over heads, the store.
  float* const orow = a.L + (int64_t)t * a.ldl;
  auto compute = [&](auto slot, int c) {
    constexpr int sl = decltype(slot)::value;
    const uint8_t* base = ring + sl * CHUNK_BYTES;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int r = f * 32 + l32;
      i32x8_t kb[KS];
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        if constexpr (FP4) {
          const i32x4_t v = *(const i32x4_t*)(base + lds_at(r, 2 * j + lg));
          kb[j] = (i32x8_t){v[0], v[1], v[2], v[3], 0, 0, 0, 0};
        } else {
          const i32x4_t v0 = *(const i32x4_t*)(base + lds_at(r, 4 * j + 2 * lg));
          const i32x4_t v1 = *(const i32x4_t*)(base + lds_at(r, 4 * j + 2 * lg + 1));
          kb[j] = (i32x8_t){v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        }
      }
      f32x16_t acc[HF];
#pragma unroll
      for (int hf = 0; hf < HF; ++hf) {
        acc[hf] = (f32x16_t){};
#pragma unroll
        for (int j = 0; j < KS; ++j) {
          i32x8_t qa;
          if constexpr (FP4)
            qa = (i32x8_t){qf[hf][j][0][0], qf[hf][j][0][1], qf[hf][j][0][2], qf[hf][j][0][3], 0, 0, 0, 0};
          else
            qa = (i32x8_t){qf[hf][j][0][0], qf[hf][j][0][1], qf[hf][j][0][2], qf[hf][j][0][3],
                           qf[hf][j][1][0], qf[hf][j][1][1], qf[hf][j][1][2], qf[hf][j][1][3]};
          // rows of the product: heads (operand A), columns: keys (operand B)
          acc[hf] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa, kb[j], acc[hf], FMT, FMT, 0,
                                                                    (int)qs[hf][j], 0, (int)ksw[sl][f][j]);
        }
      }
      // sum over heads of w * max(0, score): 16 heads per fragment in this lane, the
      // other 16 of each fragment in lane l ^ 32.  max(0, x) is taken on the bit
      // pattern as a signed integer (negative values and -0 have the sign bit set),
      // one instruction where a float max would also canonicalise x.
      float v = 0.0f;
#pragma unroll
      for (int hf = 0; hf < HF; ++hf)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) v = __builtin_fmaf(wv[hf][rr], relu(acc[hf][rr]), v);
      v += __shfl_xor(v, 32, 64);
      const int s = c_begin + c * CK + f * 32 + l32;
      if (lg == 0 && s >= lo && s < hi) orow[s] = v;
    }
  };

  // Prologue: chunks 0 .. NB-2 in flight.  Each loop step waits for its chunk's
  // copies (the later chunks' operations may stay in flight) and for this
  // wave's LDS reads of the chunk before (its slot is refilled right after), meets
  // the other waves when they share the ring, refills that slot NB-1 chunks ahead
  // (unconditionally, so the counts hold on every path: copies past the keys read
  // zeros), then computes.
  [&]<int... ps>(std::integer_sequence<int, ps...>) {
    (issue(std::integral_constant<int, ps>{}, ps), ...);
  }(std::make_integer_sequence<int, NB - 1>{});
  // after chunk c's copies, chunks c+1 .. c+NB-2 (VM operations each) were issued
  constexpr int AFTER = (NB - 2) * VM;
  constexpr int WAIT = (AFTER & 15) | (7 << 4) | (0 << 8) | ((AFTER >> 4) << 14);   // vmcnt, lgkmcnt(0)
#pragma unroll 1
  for (int i0 = 0; i0 < nch; i0 += NB) {
    [&]<int... bs>(std::integer_sequence<int, bs...>) {
      ((__builtin_amdgcn_s_waitcnt(WAIT),
        SHARED ? (__atomic_signal_fence(__ATOMIC_SEQ_CST), __builtin_amdgcn_s_barrier(),
                  __atomic_signal_fence(__ATOMIC_SEQ_CST))
               : void(),
        issue(std::integral_constant<int, (bs + NB - 1) % NB>{}, i0 + bs + NB - 1),
        i0 + bs < nch && valid ? compute(std::integral_constant<int, bs>{}, i0 + bs) : void()),
       ...);
    }(std::make_integer_sequence<int, NB>{});
  }
  // the last copies are never read: let them land before the wave ends
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
}

// Host side: argument checks and the launch.
static int num_cus() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

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
  // The four queries of a workgroup share their keys when they lie in one group:
  // groups of a multiple of four queries, or a single group.
  const bool shared = a.q_per_group % kWaves == 0 || a.q_per_group >= T;
  // Key range per workgroup.  Shared keys: the longest range (up to 4096 keys) that
  // still leaves at least two workgroups per CU, since every workgroup loads its four
  // queries' fragments and weights once (4096 against 1024 keys: 25% faster on the
  // 4096-token prefill).  Keys of their own (decode): 1024, where longer ranges
  // measured 4-6% slower.
  const int64_t qblocks = (T + kWaves - 1) / kWaves;
  int kpw = kKeysPerWgMin;
  if (shared)
    for (int c = kKeysPerWgMax; c > kKeysPerWgMin; c /= 2)
      if (qblocks * ((S + c - 1) / c) >= 2 * (int64_t)num_cus()) {
        kpw = c;
        break;
      }
  a.keys_per_wg = kpw;
  const dim3 grid((unsigned)((S + kpw - 1) / kpw), (unsigned)qblocks);
  if (qblocks > 65535) return BSG_ERR_UNSUPPORTED_SHAPE;
  (void)hipGetLastError();
  auto go = [&](auto hf_c, auto sh_c) {
    constexpr int HFv = decltype(hf_c)::value;
    constexpr bool SH = decltype(sh_c)::value;
    hipLaunchKernelGGL((mqa_logits_kernel<FMT, HFv, SH>), grid, dim3(64 * kWaves), 0,
                       (hipStream_t)stream, a);
  };
  auto by_h = [&](auto sh_c) {
    switch (H / 32) {
      case 1: go(std::integral_constant<int, 1>{}, sh_c); break;
      case 2: go(std::integral_constant<int, 2>{}, sh_c); break;
      case 3: go(std::integral_constant<int, 3>{}, sh_c); break;
      default: go(std::integral_constant<int, 4>{}, sh_c); break;
    }
  };
  if (shared)
    by_h(std::true_type{});
  else
    by_h(std::false_type{});
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
