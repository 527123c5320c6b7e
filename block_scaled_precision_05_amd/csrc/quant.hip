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
// kernel is built for streaming: one workgroup of 4 waves owns 32 rows x 512
// elements; each lane reads 16 bytes (8 elements) of a row, a wave covers the
// 512 elements of one row at a time and keeps its 8 rows' loads in flight
// together.  A block's amax is a max over the 16 (e4m3) or 4 (e2m1) lanes that
// hold it (packed 16-bit max, then DPP moves).  The division by the scale, the
// rounding and the packing of two codes are one gfx950 scaled-conversion
// instruction per two elements; a stream of ~20 plain ALU instructions per
// element would bound the kernel below the HBM rate.  Scale words are gathered in
// LDS as [pair][row] and leave as 64-byte row segments of the MN-major array.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/bsg.h"
#include "internal.h"
#include "quant_math.h"

namespace bsg_quant {

using namespace bsg_qm;

constexpr int kRows = 32;        // rows per workgroup
constexpr int kCols = 512;       // elements per workgroup row
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
// Operand loads carry the non-temporal hint: each byte of X is read once, and
// not allocating it in the last-level cache avoids evicting (and writing back)
// other lines.  Measured on 4096x16384: 40 us warm / 46 us after a 512 MiB
// cache scrub, against 37 / 65 us without the hint and 42 / 77 us with 64-row
// workgroups.
constexpr int kLoadAux = 2;



typedef __attribute__((ext_vector_type(2))) short short2_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

// Raw byte-addressed buffer resource (gfx9 word 3): reads past `bytes` return
// zero and writes past it are dropped.
constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kOOB = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) unsigned short ushort2_t;


__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(ushort2_t, a),
                                                                __builtin_bit_cast(ushort2_t, b)));
}

__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(ushort2_t, a),
                                                                __builtin_bit_cast(ushort2_t, b)));
}


// ROWS: rows per workgroup (at most 64); LAUX / SAUX: cache-policy bits of
// the operand loads and the code stores.
template <int FMT, int RULE, int ROWS = kRows, int LAUX = kLoadAux, int SAUX = 0>
__global__ __launch_bounds__(kThreads) void quant_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, uint8_t* __restrict__ Q, int64_t ldq,
    int16_t* __restrict__ sf, int64_t ld_sf, int M, int K) {
  using F = Fmt<FMT>;
  static_assert(ROWS % kWaves == 0 && ROWS <= 64, "rows per workgroup");
  constexpr int kRowsPerWave = ROWS / kWaves;
  constexpr int KPT = kCols / F::GK / 2;  // packed scale words per row per workgroup
  __shared__ uint16_t words[KPT][ROWS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m0 = blockIdx.x * ROWS;
  const int rows = min(ROWS, M - m0);
  const int k0 = blockIdx.y * kCols;
  const int k = k0 + lane * 8;
  const bool kin = k < K;
  const int kb_total = K / F::GK;
  const int64_t qcols = FMT == FMT_E4M3 ? K : K / 2;

  // The workgroup's rows as buffers: rows past M read zero and their stores are
  // dropped; lanes past K get an offset past every record.  Row offsets are
  // wave-uniform (scalar); the host keeps 63 * row stride + 2^31 below 2^32.
  const __amdgpu_buffer_rsrc_t xr =
      make_rsrc(X + (int64_t)m0 * ldx, (uint32_t)(((int64_t)(rows - 1) * ldx + K) * 2));
  const __amdgpu_buffer_rsrc_t qr =
      make_rsrc(Q + (int64_t)m0 * ldq, (uint32_t)((int64_t)(rows - 1) * ldq + qcols));
  const uint32_t xoff = kin ? (uint32_t)k * 2 : kOOB;
  const uint32_t qoff = kin ? (uint32_t)(FMT == FMT_E4M3 ? k : k / 2) : kOOB;

  // All loads of the wave's rows first, so that they are in flight together.
  u32x4_t raw[kRowsPerWave];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i)
    raw[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, xoff, (wave + i * kWaves) * (int)ldx * 2, LAUX);

#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int rl = wave + i * kWaves;
    uint32_t w[4] = {raw[i][0], raw[i][1], raw[i][2], raw[i][3]};
    // largest magnitude of the lane's 8 values, then of the block's lanes
    // (finite bf16 magnitudes order like their bit patterns)
    const uint32_t m01 = pk_max_u16(w[0] & 0x7FFF7FFFu, w[1] & 0x7FFF7FFFu);
    const uint32_t m23 = pk_max_u16(w[2] & 0x7FFF7FFFu, w[3] & 0x7FFF7FFFu);
    const uint32_t m = pk_max_u16(m01, m23);
    const uint32_t h = block_max<F::LANES>(max(m & 0xFFFFu, m >> 16));
    const int byte = scale_byte<FMT, RULE>(h << 16);
    const float sc = scale_f32(byte);
    // The gfx950 scaled conversions compute x / sc, round to nearest even and
    // saturate e2m1 at 6; e4m3 beyond 448 would turn into NaN, which only the
    // OCP MX rule can reach: there the bf16 magnitudes are first clamped to
    // 448 * sc (exactly representable), the value saturating rounding gives.
    if (FMT == FMT_E4M3 && RULE == BSG_SCALE_OCP_MX) {
      const uint32_t lim = 0x43E0u + (uint32_t)((byte - 127) << 7);
      const uint32_t lim2 = lim | (lim << 16);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = pk_min_u16(w[j] & 0x7FFF7FFFu, lim2) | (w[j] & 0x80008000u);
    }
    if (FMT == FMT_E4M3) {
      short2_t lo = {0, 0}, hi = {0, 0};
      lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(lo, __builtin_bit_cast(bf16x2_t, w[0]), sc, false);
      lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(lo, __builtin_bit_cast(bf16x2_t, w[1]), sc, true);
      hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hi, __builtin_bit_cast(bf16x2_t, w[2]), sc, false);
      hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hi, __builtin_bit_cast(bf16x2_t, w[3]), sc, true);
      const u32x2_t v = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
      __builtin_amdgcn_raw_buffer_store_b64(v, qr, qoff, rl * (int)ldq, SAUX);
    } else {
      uint32_t q = 0;
      q = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(q, __builtin_bit_cast(bf16x2_t, w[0]), sc, 0);
      q = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(q, __builtin_bit_cast(bf16x2_t, w[1]), sc, 1);
      q = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(q, __builtin_bit_cast(bf16x2_t, w[2]), sc, 2);
      q = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(q, __builtin_bit_cast(bf16x2_t, w[3]), sc, 3);
      __builtin_amdgcn_raw_buffer_store_b32(q, qr, qoff, rl * (int)ldq, SAUX);
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
  for (int t = threadIdx.x; t < KPT * ROWS; t += kThreads) {
    const int kp = t / ROWS, rl = t % ROWS;
    if (kp0 + kp < kp_total && m0 + rl < M)
      sf[(int64_t)(kp0 + kp) * ld_sf + m0 + rl] = (int16_t)words[kp][rl];
  }
}

// SiLU in fp32: g / (1 + e^-g) with the accurate expf and a reciprocal (about 3
// ulp in all).  For g below about -88 e^-g is +inf, the reciprocal 0 and the
// result a zero with g's sign, the limit.

// SwiGLU of an up-projection output followed by FP8 1x128 quantisation.  H is
// bf16 [M][ldh] with the gate in columns [0, I) and the up projection in
// [I, 2I); y = silu(gate) * up is formed in fp32 and quantised exactly as
// quant_kernel quantises its input (same tile, scale rules and scale layout),
// with the gfx950 fp32 scaled conversion.  The pages place SwiGLU between the
// two grouped GEMMs of the fused MoE step ("DeepGEMM-Ascend cobre quantas
// operacoes no Ascend 950?" third page, "Kernels de computacao: DeepGEMM-Ascend
// versus DeepGEMM", section "Execucao de MoE: MegaMoE e distribuicao de
// especialistas").
template <int RULE, int ROWS = kRows, int LAUX = kLoadAux>
__global__ __launch_bounds__(kThreads) void swiglu_quant_kernel(
    const uint16_t* __restrict__ H, int64_t ldh, uint8_t* __restrict__ Q, int64_t ldq,
    int16_t* __restrict__ sf, int64_t ld_sf, int M, int I) {
  using F = Fmt<FMT_E4M3>;
  constexpr int kRowsPerWave = ROWS / kWaves;
  constexpr int KPT = kCols / F::GK / 2;
  __shared__ uint16_t words[KPT][ROWS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m0 = blockIdx.x * ROWS;
  const int rows = min(ROWS, M - m0);
  const int k0 = blockIdx.y * kCols;
  const int k = k0 + lane * 8;
  const bool kin = k < I;
  const int kb_total = I / F::GK;

  const __amdgpu_buffer_rsrc_t hr =
      make_rsrc(H + (int64_t)m0 * ldh, (uint32_t)(((int64_t)(rows - 1) * ldh + 2 * (int64_t)I) * 2));
  const __amdgpu_buffer_rsrc_t qr =
      make_rsrc(Q + (int64_t)m0 * ldq, (uint32_t)((int64_t)(rows - 1) * ldq + I));
  const uint32_t goff = kin ? (uint32_t)k * 2 : kOOB;
  const uint32_t uoff = kin ? (uint32_t)(I + k) * 2 : kOOB;
  const uint32_t qoff = kin ? (uint32_t)k : kOOB;

  u32x4_t gr[kRowsPerWave], ur[kRowsPerWave];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int so = (wave + i * kWaves) * (int)ldh * 2;
    gr[i] = __builtin_amdgcn_raw_buffer_load_b128(hr, goff, so, LAUX);
    ur[i] = __builtin_amdgcn_raw_buffer_load_b128(hr, uoff, so, LAUX);
  }

#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int rl = wave + i * kWaves;
    u32x2_t v;
    int byte;
    swiglu_fp8x8<RULE>(gr[i], ur[i], v, byte);
    __builtin_amdgcn_raw_buffer_store_b64(v, qr, qoff, rl * (int)ldq, 0);
    const int hb = __shfl_down(byte, F::LANES);
    if ((lane % (2 * F::LANES)) == 0) {
      const int blk = (k0 / F::GK) + lane / F::LANES;
      const uint32_t hbyte = (blk + 1 < kb_total) ? (uint32_t)hb : 0x7Fu;
      words[lane / (2 * F::LANES)][rl] = (uint16_t)(byte | (hbyte << 8));
    }
  }
  __syncthreads();
  const int kp0 = k0 / (2 * F::GK);
  const int kp_total = (kb_total + 1) / 2;
  for (int t = threadIdx.x; t < KPT * ROWS; t += kThreads) {
    const int kp = t / ROWS, rl = t % ROWS;
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
  // 63 row strides plus the out-of-range lane offset 2^31 must stay below 2^32.
  if (ldx >= (int64_t(1) << 24) || ldq >= (int64_t(1) << 25)) return BSG_ERR_UNSUPPORTED_SHAPE;
  if (((uintptr_t)X & 15) || (ldx % 8)) return BSG_ERR_MISALIGNED;
  if (((uintptr_t)Q & (q_align - 1)) || (ldq % q_align)) return BSG_ERR_MISALIGNED;
  if ((uintptr_t)sf & 1) return BSG_ERR_MISALIGNED;
  return BSG_OK;
}

static int swiglu_check(const void* H, int64_t ldh, const void* Q, int64_t ldq, const int16_t* sf,
                        int64_t ld_sf, int64_t M, int64_t I, int32_t rule) {
  // H rows are read as 2I elements; the checks of an FP8 quantiser of width I
  // cover Q and sf, and ldh must hold both halves.
  if (I < 0) return BSG_ERR_INVALID_ARG;
  const int st = check(H, ldh, Q, ldq, sf, ld_sf, M, I, rule, 128, I, 8);
  if (st != BSG_OK || M == 0 || I == 0) return st;
  if (ldh < 2 * I) return BSG_ERR_INVALID_ARG;
  return BSG_OK;
}

static int swiglu_launch(const void* H, int64_t ldh, void* Q, int64_t ldq, int16_t* sf,
                         int64_t ld_sf, int64_t M, int64_t I, int32_t rule, hipStream_t stream) {
  const dim3 grid((unsigned)((M + kRows - 1) / kRows), (unsigned)((I + kCols - 1) / kCols));
  (void)hipGetLastError();
  if (rule == BSG_SCALE_CEIL)
    hipLaunchKernelGGL((swiglu_quant_kernel<BSG_SCALE_CEIL>), grid, dim3(kThreads), 0, stream,
                       (const uint16_t*)H, ldh, (uint8_t*)Q, ldq, sf, ld_sf, (int)M, (int)I);
  else
    hipLaunchKernelGGL((swiglu_quant_kernel<BSG_SCALE_OCP_MX>), grid, dim3(kThreads), 0, stream,
                       (const uint16_t*)H, ldh, (uint8_t*)Q, ldq, sf, ld_sf, (int)M, (int)I);
  return hipGetLastError() == hipSuccess ? BSG_OK : BSG_ERR_HIP;
}

// ---------------------------------------------------------------------------
// MoE FFN core: argument checks and the two launches, shared by moe_ffn_fp8
// (caller's workspace) and moe_ffn_fp8_noalloc (the library's scratch array).
// ---------------------------------------------------------------------------
static int ffn_check(const void* A, int64_t lda, const int16_t* sfa, int64_t ld_sfa,
                     const void* W13, int64_t ldw13, int64_t stride_w13, const int16_t* sfw13,
                     int64_t ld_sfw13, int64_t stride_sfw13, const void* W2, int64_t ldw2,
                     int64_t stride_w2, const int16_t* sfw2, int64_t ld_sfw2, int64_t stride_sfw2,
                     const int32_t* group_offsets, int32_t G, int64_t M_total, int64_t hidden,
                     int64_t inter, const void* H, int64_t ldh, const void* Y, int64_t ldy,
                     const int16_t* sfy, int64_t ld_sfy, const void* D, int64_t ldd, int32_t rule) {
  if (inter < 0 || hidden < 0) return BSG_ERR_INVALID_ARG;
  // H is never written (the up-projection's epilogue forms Y directly), so it may be
  // NULL; when given it is checked as the up-projection's output would be.  The
  // checks below take a stand-in that is never dereferenced: a 16-byte aligned
  // non-null address with the smallest valid leading dimension.
  const void* Hc = H ? H : (const void*)(uintptr_t)256;
  const int64_t ldhc = H ? ldh : 2 * inter;
  int st = bsg::grouped_fp8_check(A, lda, sfa, ld_sfa, W13, ldw13, stride_w13, sfw13, ld_sfw13,
                                  stride_sfw13, Hc, ldhc, group_offsets, G, M_total, 2 * inter,
                                  hidden);
  if (st != BSG_OK) return st;
  st = swiglu_check(Hc, ldhc, Y, ldy, sfy, ld_sfy, M_total, inter, rule);
  if (st != BSG_OK) return st;
  // The up-projection tile reads gate rows n0 .. n0+127 and the matching up rows
  // inter + n0 .. of W13 through one buffer record of 32-bit byte offsets, so
  // inter + 128 rows of W13 must stay below 2^31 bytes.
  if ((inter + 128) * ldw13 >= (int64_t(1) << 31)) return BSG_ERR_UNSUPPORTED_SHAPE;
  return bsg::grouped_fp8_check(Y, ldy, sfy, ld_sfy, W2, ldw2, stride_w2, sfw2, ld_sfw2,
                                stride_sfw2, D, ldd, group_offsets, G, M_total, hidden, inter);
}

// Arguments checked; M_total, G, hidden and inter all positive.
static int ffn_launch(const void* A, int64_t lda, const int16_t* sfa, int64_t ld_sfa,
                      const void* W13, int64_t ldw13, int64_t stride_w13, const int16_t* sfw13,
                      int64_t ld_sfw13, int64_t stride_sfw13, const void* W2, int64_t ldw2,
                      int64_t stride_w2, const int16_t* sfw2, int64_t ld_sfw2, int64_t stride_sfw2,
                      const int32_t* group_offsets, int32_t G, int64_t M_total, int64_t hidden,
                      int64_t inter, void* Y, int64_t ldy, int16_t* sfy, int64_t ld_sfy, void* D,
                      int64_t ldd, int32_t rule, void* stream) {
  // The up-projection applies SwiGLU and the requantisation in its epilogue (the
  // checks guarantee what that needs: inter a multiple of 128, Y 8-byte aligned
  // with ldy a multiple of 8); H is not formed.
  int st = bsg::grouped_fp8_swiglu(A, lda, sfa, ld_sfa, W13, ldw13, stride_w13, sfw13, ld_sfw13,
                                   stride_sfw13, group_offsets, G, M_total, hidden, inter, Y, ldy,
                                   sfy, ld_sfy, rule, stream);
  if (st != BSG_OK) return st;
  return m_grouped_gemm_fp8(Y, ldy, sfy, ld_sfy, W2, ldw2, stride_w2, sfw2, ld_sfw2, stride_sfw2,
                            D, ldd, group_offsets, G, M_total, hidden, inter, stream);
}

// Scratch memory of moe_ffn_fp8_noalloc: the requantised intermediate Y and its
// packed scales live here instead of in caller-provided buffers.  Every GPU the
// library runs on holds its own copy for the life of the process.  Host code never
// uses the array's name as an address: each device's copy is located once, with
// that device current, and the address kept per device.
constexpr size_t kFfnScratchBytes = size_t(64) << 20;
__device__ __align__(256) uint8_t scratch[kFfnScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64];

static int ffn_scratch(uint8_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return BSG_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BSG_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = (uint8_t*)g_scratch_ptr[dev];
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

int swiglu_quantize_fp8(const void* H, int64_t ldh, void* Q, int64_t ldq, int16_t* sf,
                        int64_t ld_sf, int64_t M, int64_t I, int32_t rule, void* stream) {
  const int st = swiglu_check(H, ldh, Q, ldq, sf, ld_sf, M, I, rule);
  if (st != BSG_OK || M == 0 || I == 0) return st;
  return swiglu_launch(H, ldh, Q, ldq, sf, ld_sf, M, I, rule, (hipStream_t)stream);
}

int moe_ffn_fp8(const void* A, int64_t lda, const int16_t* sfa, int64_t ld_sfa,
                const void* W13, int64_t ldw13, int64_t stride_w13, const int16_t* sfw13,
                int64_t ld_sfw13, int64_t stride_sfw13,
                const void* W2, int64_t ldw2, int64_t stride_w2, const int16_t* sfw2,
                int64_t ld_sfw2, int64_t stride_sfw2,
                const int32_t* group_offsets, int32_t G, int64_t M_total, int64_t hidden,
                int64_t inter, void* H, int64_t ldh, void* Y, int64_t ldy, int16_t* sfy,
                int64_t ld_sfy, void* D, int64_t ldd, int32_t rule, void* stream) {
  // every check before the first launch, so a bad argument launches nothing
  const int st = ffn_check(A, lda, sfa, ld_sfa, W13, ldw13, stride_w13, sfw13, ld_sfw13,
                           stride_sfw13, W2, ldw2, stride_w2, sfw2, ld_sfw2, stride_sfw2,
                           group_offsets, G, M_total, hidden, inter, H, ldh, Y, ldy, sfy, ld_sfy,
                           D, ldd, rule);
  if (st != BSG_OK || M_total == 0 || G == 0 || hidden == 0 || inter == 0) return st;
  return ffn_launch(A, lda, sfa, ld_sfa, W13, ldw13, stride_w13, sfw13, ld_sfw13, stride_sfw13,
                    W2, ldw2, stride_w2, sfw2, ld_sfw2, stride_sfw2, group_offsets, G, M_total,
                    hidden, inter, Y, ldy, sfy, ld_sfy, D, ldd, rule, stream);
}

int moe_ffn_fp8_noalloc(const void* A, int64_t lda, const int16_t* sfa, int64_t ld_sfa,
                        const void* W13, int64_t ldw13, int64_t stride_w13, const int16_t* sfw13,
                        int64_t ld_sfw13, int64_t stride_sfw13,
                        const void* W2, int64_t ldw2, int64_t stride_w2, const int16_t* sfw2,
                        int64_t ld_sfw2, int64_t stride_sfw2,
                        const int32_t* group_offsets, int32_t G, int64_t M_total, int64_t hidden,
                        int64_t inter, void* D, int64_t ldd, int32_t rule, void* stream) {
  if (M_total < 0 || inter < 0 || hidden < 0) return BSG_ERR_INVALID_ARG;
  // Y [M_total][inter] at the start of the scratch array, its packed scales
  // [ceil(inter/256)][ld_sfy] at the next 256-byte boundary; ld_sfy a multiple of
  // 4 so the down-projection takes the 8-byte scale loads.
  const int64_t ldy = inter, ld_sfy = (M_total + 3) / 4 * 4;
  const int64_t y_bytes = (M_total * inter + 255) / 256 * 256;
  const int64_t s_bytes = (inter / 128 + 1) / 2 * ld_sfy * 2;
  if (M_total > INT32_MAX || inter > INT32_MAX || y_bytes + s_bytes > (int64_t)kFfnScratchBytes)
    return BSG_ERR_UNSUPPORTED_SHAPE;
  // The checks see stand-in workspace addresses with the scratch array's alignment;
  // nothing is dereferenced before the real address is known.
  uint8_t* const y_dummy = (uint8_t*)(uintptr_t)256;
  int st = ffn_check(A, lda, sfa, ld_sfa, W13, ldw13, stride_w13, sfw13, ld_sfw13, stride_sfw13,
                     W2, ldw2, stride_w2, sfw2, ld_sfw2, stride_sfw2, group_offsets, G, M_total,
                     hidden, inter, nullptr, 0, y_dummy, ldy, (int16_t*)(y_dummy + y_bytes),
                     ld_sfy, D, ldd, rule);
  if (st != BSG_OK || M_total == 0 || G == 0 || hidden == 0 || inter == 0) return st;
  uint8_t* base = nullptr;
  st = ffn_scratch(&base);
  if (st != BSG_OK) return st;
  return ffn_launch(A, lda, sfa, ld_sfa, W13, ldw13, stride_w13, sfw13, ld_sfw13, stride_sfw13,
                    W2, ldw2, stride_w2, sfw2, ld_sfw2, stride_sfw2, group_offsets, G, M_total,
                    hidden, inter, base, ldy, (int16_t*)(base + y_bytes), ld_sfy, D, ldd, rule,
                    stream);
}

}  // extern "C"
