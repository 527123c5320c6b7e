// api.hip -- C ABI entry points of the block-scaled GEMM library (see include/bsg.h).
//
// Every entry point validates its arguments on the host before any HIP call and
// returns a status code; kernels are launched asynchronously on the caller's
// stream; nothing is allocated and nothing is synchronised.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bsg.h"
#include "configs.h"
#include "gemm_kernel.h"
#include "internal.h"

namespace bsg {

// ---------------------------------------------------------------------------
// Scale pack / unpack kernels: one thread per packed int16.
// The pages describe the packed layout (pairs of UE8M0 factors along K in one
// 16-bit integer, MN-major) and the reuse-or-convert step that produces it
// ("DeepGEMM-Ascend cobre quantas operacoes no Ascend 950?", section "Fatores de
// escala FP8 e o formato UE8M0 no Ascend").  Reading adopted: the even K-block
// is the low byte; an odd K-block count pads the last high byte with 0x7F.
// Consecutive threads walk the MN index, so the packed stores are coalesced.
// ---------------------------------------------------------------------------
__global__ void pack_kernel(const uint8_t* __restrict__ sf, int64_t mn, int64_t kb, int64_t ld_sf,
                            int16_t* __restrict__ packed, int64_t ld_packed) {
  const int64_t kp_n = (kb + 1) / 2;
  const int64_t total = kp_n * mn;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t kp = idx / mn, r = idx - kp * mn;
    const uint32_t lo = sf[r * ld_sf + 2 * kp];
    const uint32_t hi = (2 * kp + 1 < kb) ? sf[r * ld_sf + 2 * kp + 1] : 0x7Fu;
    packed[kp * ld_packed + r] = (int16_t)(uint16_t)(lo | (hi << 8));
  }
}

// fp32 scale factors (exact powers of two, as fp32 scale tensors of block-scaled
// operands hold them) -> UE8M0 byte: the exponent field of a positive normal with
// zero mantissa is the byte itself; 2^-127 is the fp32 subnormal 0x00400000 and
// gives byte 0.  Anything else (not a power of two, <= 0, inf, NaN, below 2^-127)
// has no UE8M0 code: it is counted as inexact and gets its exponent field.
__host__ __device__ inline uint32_t ue8m0_of_f32(uint32_t bits, bool& exact) {
  const uint32_t e = (bits >> 23) & 0xFF;
  if (bits == 0x00400000u) {
    exact = true;
    return 0;
  }
  exact = (bits & 0x807FFFFFu) == 0 && e >= 1 && e <= 254;
  return e;
}

__global__ void pack_f32_kernel(const float* __restrict__ sf, int64_t mn, int64_t kb, int64_t ld_sf,
                                int16_t* __restrict__ packed, int64_t ld_packed,
                                int32_t* __restrict__ inexact) {
  const int64_t kp_n = (kb + 1) / 2;
  const int64_t total = kp_n * mn;
  int bad = 0;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t kp = idx / mn, r = idx - kp * mn;
    bool ex_lo = true, ex_hi = true;
    const uint32_t lo = ue8m0_of_f32(__float_as_uint(sf[r * ld_sf + 2 * kp]), ex_lo);
    const uint32_t hi =
        (2 * kp + 1 < kb) ? ue8m0_of_f32(__float_as_uint(sf[r * ld_sf + 2 * kp + 1]), ex_hi) : 0x7Fu;
    bad += !ex_lo + !ex_hi;
    packed[kp * ld_packed + r] = (int16_t)(uint16_t)(lo | (hi << 8));
  }
  if (inexact && bad) atomicAdd(inexact, bad);
}

__global__ void unpack_kernel(const int16_t* __restrict__ packed, int64_t mn, int64_t kb,
                              int64_t ld_packed, uint8_t* __restrict__ sf, int64_t ld_sf) {
  const int64_t kp_n = (kb + 1) / 2;
  const int64_t total = kp_n * mn;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t kp = idx / mn, r = idx - kp * mn;
    const uint32_t w = (uint16_t)packed[kp * ld_packed + r];
    sf[r * ld_sf + 2 * kp] = (uint8_t)(w & 0xFF);
    if (2 * kp + 1 < kb) sf[r * ld_sf + 2 * kp + 1] = (uint8_t)((w >> 8) & 0xFF);
  }
}

static int g_num_cus[64];

static int num_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (g_num_cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    g_num_cus[dev] = n;
  }
  return g_num_cus[dev];
}

template <int KIND, int BM, int BN, int WM, int WN, int SB, int NS, int PR, bool GROUPED, int SV = 0,
          int EPI = 0>
static int launch(GemmArgs a, hipStream_t stream) {
  using T = GemmTile<KIND, BM, BN, WM, WN, SB, NS, PR, SV, GROUPED>;
  a.d_vec = (((uintptr_t)a.D & 15) == 0 && (a.ldd % 8) == 0) ? 2
            : (((uintptr_t)a.D & 7) == 0 && (a.ldd % 4) == 0) ? 1 : 0;
  a.tiles_m = (a.M + BM - 1) / BM;
  a.tiles_n = (a.N + BN - 1) / BN;
  a.nk = (a.k_bytes + SB - 1) / SB;
  int grid;
  if (GROUPED) {
    grid = num_cus();
  } else {
    // As many tiles per workgroup as the CUs require, then as few workgroups as give
    // every one that many: 448 tiles run as 224 workgroups of two rather than 256 of
    // one or two.  The idle CUs leave power to the busy ones (1-1.4% faster at
    // 4096x7168x16384 in an alternating A/B).  A multiple of 8, so a workgroup's later
    // tiles stay on its XCD (tile i runs on XCD i % 8; see xcd_remap).
    const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
    const int64_t cus = num_cus();
    const int64_t per = (tiles + cus - 1) / cus;
    int64_t g = (tiles + per - 1) / per;
    if (per > 1) g = (g + 7) / 8 * 8;
    grid = (int)(g < cus ? g : cus);
  }
  // Leading dead stages of the first round: nk padded up to whole rounds of U
  // stages, the padding rounded down to an even count (paired stages).  BF16 and FP4
  // peel it at any size (at K = 16384, 8 of 520 and 2 of 130 stages: 0.7% and 0.4%
  // faster than the same padding at the end, in an alternating A/B).  FP8 keeps a
  // padding under 2% of the loop at the end, where it multiplies zeros: its 8-register
  // fragments leave the peeled round no registers to spare (the dense kernel spills
  // there, 2% slower at K = 16384).
  constexpr int U = T::U;
  int koff = a.nk % U ? (U - a.nk % U) & ~1 : 0;
  if (KIND == KIND_FP8 && koff * 50 <= a.nk + koff) koff = 0;
  (void)hipGetLastError();
  int st = BSG_OK;
  auto go = [&](auto kc) {
    constexpr int KO = decltype(kc)::value;
    if constexpr (KO < U)
      hipLaunchKernelGGL((gemm_kernel<KIND, BM, BN, WM, WN, SB, NS, PR, GROUPED, SV, KO, EPI>), dim3(grid),
                         dim3(T::NT), 0, stream, a);
    else
      st = BSG_ERR_UNSUPPORTED_SHAPE;   // not reached: koff < U by construction
  };
  static_assert(U <= 16, "leading dead stages are instantiated up to 14");
  switch (koff) {
    case 0: go(std::integral_constant<int, 0>{}); break;
    case 2: go(std::integral_constant<int, 2>{}); break;
    case 4: go(std::integral_constant<int, 4>{}); break;
    case 6: go(std::integral_constant<int, 6>{}); break;
    case 8: go(std::integral_constant<int, 8>{}); break;
    case 10: go(std::integral_constant<int, 10>{}); break;
    case 12: go(std::integral_constant<int, 12>{}); break;
    case 14: go(std::integral_constant<int, 14>{}); break;
    default: return BSG_ERR_UNSUPPORTED_SHAPE;
  }
  if (st != BSG_OK) return st;
  return hipGetLastError() == hipSuccess ? BSG_OK : BSG_ERR_HIP;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// A packed scale array whose rows of four int16 can be fetched as one 8-byte word.
static bool sv_ok(const int16_t* sf, int64_t ld) { return ((uintptr_t)sf % 8 == 0) && (ld % 4 == 0); }

// Byte strides must keep 256 rows of offsets inside 31 bits.
static const int64_t kMaxRowBytes = (int64_t(1) << 31) / 256 - 1;
static const int64_t kMaxDim = (int64_t(1) << 31) - 1;

// Shared checks of the dense entry points.  elem: bytes per stored element of A/B
// (2 for bf16, 1 for e4m3, 1/2 for e2m1 expressed as k_bytes = K/2).
static int check_dense(const void* A, int64_t lda, const void* B, int64_t ldb, const void* D,
                       int64_t ldd, int64_t M, int64_t N, int64_t K, int64_t kgran, int64_t k_bytes,
                       int64_t elem_bytes) {
  if (M < 0 || N < 0 || K < 0) return BSG_ERR_INVALID_ARG;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return BSG_ERR_UNSUPPORTED_SHAPE;
  if (K % kgran) return BSG_ERR_UNSUPPORTED_SHAPE;
  if (M == 0 || N == 0) return BSG_OK;
  if (!D || ldd < N) return BSG_ERR_INVALID_ARG;
  if ((uintptr_t)D & 1) return BSG_ERR_MISALIGNED;
  if (ldd > kMaxDim) return BSG_ERR_UNSUPPORTED_SHAPE;
  if (K == 0) return BSG_OK;  // A and B are not read
  if (!A || !B) return BSG_ERR_INVALID_ARG;
  if (lda * elem_bytes < k_bytes || ldb * elem_bytes < k_bytes) return BSG_ERR_INVALID_ARG;
  if (lda * elem_bytes > kMaxRowBytes || ldb * elem_bytes > kMaxRowBytes)
    return BSG_ERR_UNSUPPORTED_SHAPE;
  if (!aligned16(A) || !aligned16(B)) return BSG_ERR_MISALIGNED;
  if ((lda * elem_bytes) % 16 || (ldb * elem_bytes) % 16) return BSG_ERR_MISALIGNED;
  return BSG_OK;
}

// Packed scale arrays of kp = ceil(K / kgran / 2) rows.  The kernels address them
// with 32-bit byte offsets, up to one packed row past the last (FP4 lane groups on a
// K tail), so 2 (kp + 1) ld bytes must stay inside 31 bits.
static int check_scales(const int16_t* sfa, int64_t ld_sfa, int64_t rows_a, const int16_t* sfb,
                        int64_t ld_sfb, int64_t rows_b, int64_t K, int64_t kgran) {
  if (K == 0) return BSG_OK;
  if (!sfa || !sfb) return BSG_ERR_INVALID_ARG;
  if (ld_sfa < rows_a || ld_sfb < rows_b) return BSG_ERR_INVALID_ARG;
  if (((uintptr_t)sfa & 1) || ((uintptr_t)sfb & 1)) return BSG_ERR_MISALIGNED;
  const int64_t kp = (K / kgran + 1) / 2;
  if (ld_sfa > kMaxDim || ld_sfb > kMaxDim || 2 * (kp + 1) * ld_sfa > kMaxDim ||
      2 * (kp + 1) * ld_sfb > kMaxDim)
    return BSG_ERR_UNSUPPORTED_SHAPE;
  return BSG_OK;
}

// Argument checks of the M-grouped GEMMs.  kind: KIND_BF16, KIND_FP8, KIND_FP4.
int grouped_check(int kind, const void* A, int64_t lda, const int16_t* sfa, int64_t ld_sfa,
                  const void* B, int64_t ldb, int64_t stride_b, const int16_t* sfb,
                  int64_t ld_sfb, int64_t stride_sfb, const void* D, int64_t ldd,
                  const int32_t* group_offsets, int32_t G, int64_t M_total, int64_t N, int64_t K) {
  if (G < 0 || G > 1024) return G < 0 ? BSG_ERR_INVALID_ARG : BSG_ERR_UNSUPPORTED_SHAPE;
  const int64_t gran = kind == KIND_BF16 ? 8 : (kind == KIND_FP8 ? 128 : 32);
  const int64_t k_bytes = kind == KIND_BF16 ? 2 * K : (kind == KIND_FP8 ? K : K / 2);
  const int64_t elem = kind == KIND_BF16 ? 2 : 1;
  int st = check_dense(A, lda, B, ldb, D, ldd, M_total, N, K, gran, k_bytes, elem);
  if (st != BSG_OK || M_total == 0 || N == 0 || G == 0) return st;
  if (!group_offsets) return BSG_ERR_INVALID_ARG;
  int64_t kp = 0;
  if (kind != KIND_BF16) {
    const int64_t b_rows = kind == KIND_FP8 ? (N + 127) / 128 : N;
    st = check_scales(sfa, ld_sfa, M_total, sfb, ld_sfb, b_rows, K, gran);
    if (st != BSG_OK) return st;
    kp = (K / gran + 1) / 2;
  }
  if (G > 1 && (stride_b < (N - 1) * ldb + k_bytes / elem || (K > 0 && stride_sfb < kp * ld_sfb)))
    return BSG_ERR_INVALID_ARG;
  if (stride_b < 0 || stride_sfb < 0) return BSG_ERR_INVALID_ARG;
  if ((stride_b * elem) % 16) return BSG_ERR_MISALIGNED;
  return BSG_OK;
}

int grouped_fp8_check(const void* A, int64_t lda, const int16_t* sfa, int64_t ld_sfa,
                      const void* B, int64_t ldb, int64_t stride_b, const int16_t* sfb,
                      int64_t ld_sfb, int64_t stride_sfb, const void* D, int64_t ldd,
                      const int32_t* group_offsets, int32_t G, int64_t M_total, int64_t N,
                      int64_t K) {
  return grouped_check(KIND_FP8, A, lda, sfa, ld_sfa, B, ldb, stride_b, sfb, ld_sfb, stride_sfb, D,
                       ldd, group_offsets, G, M_total, N, K);
}

}  // namespace bsg

using namespace bsg;

extern "C" {

const char* bsg_status_string(int status) {
  switch (status) {
    case BSG_OK: return "BSG_OK";
    case BSG_ERR_INVALID_ARG: return "BSG_ERR_INVALID_ARG";
    case BSG_ERR_UNSUPPORTED_SHAPE: return "BSG_ERR_UNSUPPORTED_SHAPE";
    case BSG_ERR_MISALIGNED: return "BSG_ERR_MISALIGNED";
    case BSG_ERR_HIP: return "BSG_ERR_HIP";
    default: return "BSG_ERR_UNKNOWN";
  }
}

int gemm_bf16(const void* A, int64_t lda, const void* B, int64_t ldb, void* D, int64_t ldd,
              int64_t M, int64_t N, int64_t K, void* stream) {
  int st = check_dense(A, lda, B, ldb, D, ldd, M, N, K, 8, 2 * K, 2);
  if (st != BSG_OK || M == 0 || N == 0) return st;
  GemmArgs a = {};
  a.A = (const uint8_t*)A;
  a.B = (const uint8_t*)B;
  a.D = (uint16_t*)D;
  a.lda = lda * 2;
  a.ldb = ldb * 2;
  a.ldd = ldd;
  a.M = (int32_t)M;
  a.N = (int32_t)N;
  a.K = (int32_t)K;
  a.k_bytes = (int32_t)(2 * K);
  return launch<KIND_BF16, BSG_BF16_CFG, false>(a, (hipStream_t)stream);
}

int gemm_fp8_blockscaled(const void* A, int64_t lda, const int16_t* sfa, int64_t ld_sfa,
                         int32_t sfa_gran_mn, const void* B, int64_t ldb, const int16_t* sfb,
                         int64_t ld_sfb, int32_t sfb_gran_mn, void* D, int64_t ldd, int64_t M,
                         int64_t N, int64_t K, void* stream) {
  if (sfa_gran_mn != 1 || (sfb_gran_mn != 128 && sfb_gran_mn != 1)) return BSG_ERR_UNSUPPORTED_SHAPE;
  int st = check_dense(A, lda, B, ldb, D, ldd, M, N, K, 128, K, 1);
  if (st != BSG_OK || M == 0 || N == 0) return st;
  const int64_t sfb_rows = (N + sfb_gran_mn - 1) / sfb_gran_mn;
  st = check_scales(sfa, ld_sfa, M, sfb, ld_sfb, sfb_rows, K, 128);
  if (st != BSG_OK) return st;
  GemmArgs a = {};
  a.A = (const uint8_t*)A;
  a.B = (const uint8_t*)B;
  a.D = (uint16_t*)D;
  a.sfa = sfa;
  a.sfb = sfb;
  a.lda = lda;
  a.ldb = ldb;
  a.ldd = ldd;
  a.ld_sfa = ld_sfa;
  a.ld_sfb = ld_sfb;
  a.M = (int32_t)M;
  a.N = (int32_t)N;
  a.K = (int32_t)K;
  a.k_bytes = (int32_t)K;
  a.kp_count = (int32_t)((K / 128 + 1) / 2);
  a.sfb_rows = (int32_t)sfb_rows;
  // one 8-byte load for a lane's four A scale words when sfa allows it; per-row B
  // scales (one word per B fragment, the lane's own row) are the kernel's flag 2
  const bool wide = sv_ok(sfa, ld_sfa);
  if (sfb_gran_mn == 1)
    return wide ? launch<KIND_FP8, BSG_FP8_CFG, false, 3>(a, (hipStream_t)stream)
                : launch<KIND_FP8, BSG_FP8_CFG, false, 2>(a, (hipStream_t)stream);
  return wide ? launch<KIND_FP8, BSG_FP8_CFG, false, 1>(a, (hipStream_t)stream)
              : launch<KIND_FP8, BSG_FP8_CFG, false, 0>(a, (hipStream_t)stream);
}

int gemm_fp4_blockscaled(const void* A, int64_t lda, const int16_t* sfa, int64_t ld_sfa,
                         const void* B, int64_t ldb, const int16_t* sfb, int64_t ld_sfb,
                         void* D, int64_t ldd, int64_t M, int64_t N, int64_t K, void* stream) {
  int st = check_dense(A, lda, B, ldb, D, ldd, M, N, K, 32, K / 2, 1);
  if (st != BSG_OK || M == 0 || N == 0) return st;
  st = check_scales(sfa, ld_sfa, M, sfb, ld_sfb, N, K, 32);
  if (st != BSG_OK) return st;
  GemmArgs a = {};
  a.A = (const uint8_t*)A;
  a.B = (const uint8_t*)B;
  a.D = (uint16_t*)D;
  a.sfa = sfa;
  a.sfb = sfb;
  a.lda = lda;
  a.ldb = ldb;
  a.ldd = ldd;
  a.ld_sfa = ld_sfa;
  a.ld_sfb = ld_sfb;
  a.M = (int32_t)M;
  a.N = (int32_t)N;
  a.K = (int32_t)K;
  a.k_bytes = (int32_t)(K / 2);
  a.kp_count = (int32_t)((K / 32 + 1) / 2);
  a.sfb_rows = (int32_t)N;
  // 8-byte scale loads when both packed arrays allow them (8-byte aligned, leading
  // dimensions multiples of 4 int16), 2-byte loads otherwise.
  if (sv_ok(sfa, ld_sfa) && sv_ok(sfb, ld_sfb)) return launch<KIND_FP4, BSG_FP4_CFG, false, 1>(a, (hipStream_t)stream);
  return launch<KIND_FP4, BSG_FP4_CFG, false, 0>(a, (hipStream_t)stream);
}

int m_grouped_gemm_fp8(const void* A, int64_t lda, const int16_t* sfa, int64_t ld_sfa,
                       const void* B, int64_t ldb, int64_t stride_b,
                       const int16_t* sfb, int64_t ld_sfb, int64_t stride_sfb,
                       void* D, int64_t ldd, const int32_t* group_offsets, int32_t G,
                       int64_t M_total, int64_t N, int64_t K, void* stream) {
  const int st = grouped_fp8_check(A, lda, sfa, ld_sfa, B, ldb, stride_b, sfb, ld_sfb, stride_sfb, D,
                                   ldd, group_offsets, G, M_total, N, K);
  if (st != BSG_OK || M_total == 0 || N == 0 || G == 0) return st;
  const int64_t kp = (K / 128 + 1) / 2;
  GemmArgs a = {};
  a.A = (const uint8_t*)A;
  a.B = (const uint8_t*)B;
  a.D = (uint16_t*)D;
  a.sfa = sfa;
  a.sfb = sfb;
  a.offsets = group_offsets;
  a.lda = lda;
  a.ldb = ldb;
  a.ldd = ldd;
  a.ld_sfa = ld_sfa;
  a.ld_sfb = ld_sfb;
  a.stride_b = stride_b;
  a.stride_sfb = stride_sfb;
  a.M = (int32_t)M_total;
  a.N = (int32_t)N;
  a.K = (int32_t)K;
  a.k_bytes = (int32_t)K;
  a.kp_count = (int32_t)kp;
  a.sfb_rows = (int32_t)((N + 127) / 128);
  a.G = G;
  if (sv_ok(sfa, ld_sfa)) return launch<KIND_FP8, BSG_GROUPED_CFG, true, 1>(a, (hipStream_t)stream);
  return launch<KIND_FP8, BSG_GROUPED_CFG, true, 0>(a, (hipStream_t)stream);
}

}  // extern "C"

namespace bsg {

// The FFN core's up-projection with the SwiGLU epilogue: Y = fp8(silu(gate) * up)
// and its packed 1x128 scales straight from the grouped FP8 GEMM over W13 = [gate;
// up] (2*inter rows per expert); H is never formed.  Arguments were checked by the
// caller; inter is a multiple of 128, Y 8-byte aligned with ldy a multiple of 8.
int grouped_fp8_swiglu(const void* A, int64_t lda, const int16_t* sfa, int64_t ld_sfa, const void* W13,
                       int64_t ldw, int64_t stride_w, const int16_t* sfw, int64_t ld_sfw,
                       int64_t stride_sfw, const int32_t* group_offsets, int32_t G, int64_t M_total,
                       int64_t hidden, int64_t inter, void* Y, int64_t ldy, int16_t* sfy, int64_t ld_sfy,
                       int32_t rule, void* stream) {
  const int64_t K = hidden, N = 2 * inter;
  GemmArgs a = {};
  a.A = (const uint8_t*)A;
  a.B = (const uint8_t*)W13;
  a.sfa = sfa;
  a.sfb = sfw;
  a.offsets = group_offsets;
  a.lda = lda;
  a.ldb = ldw;
  a.ld_sfa = ld_sfa;
  a.ld_sfb = ld_sfw;
  a.stride_b = stride_w;
  a.stride_sfb = stride_sfw;
  a.M = (int32_t)M_total;
  a.N = (int32_t)N;
  a.K = (int32_t)K;
  a.k_bytes = (int32_t)K;
  a.kp_count = (int32_t)((K / 128 + 1) / 2);
  a.sfb_rows = (int32_t)((N + 127) / 128);
  a.G = G;
  a.Y = (uint8_t*)Y;
  a.sfy = sfy;
  a.ldy = ldy;
  a.ld_sfy = ld_sfy;
  a.inter = (int32_t)inter;
  const bool sv = sv_ok(sfa, ld_sfa);
  if (rule == BSG_SCALE_CEIL)
    return sv ? launch<KIND_FP8, BSG_GROUPED_CFG, true, 1, 1>(a, (hipStream_t)stream)
              : launch<KIND_FP8, BSG_GROUPED_CFG, true, 0, 1>(a, (hipStream_t)stream);
  return sv ? launch<KIND_FP8, BSG_GROUPED_CFG, true, 1, 2>(a, (hipStream_t)stream)
            : launch<KIND_FP8, BSG_GROUPED_CFG, true, 0, 2>(a, (hipStream_t)stream);
}

}  // namespace bsg

extern "C" {

int m_grouped_gemm_fp8_masked(const void* A, int64_t lda, const int16_t* sfa, int64_t ld_sfa,
                              const void* B, int64_t ldb, int64_t stride_b,
                              const int16_t* sfb, int64_t ld_sfb, int64_t stride_sfb,
                              void* D, int64_t ldd, const int32_t* masked_m, int32_t G,
                              int64_t max_m, int64_t N, int64_t K, void* stream) {
  if (max_m < 0) return BSG_ERR_INVALID_ARG;
  if (G > 0 && max_m > kMaxDim / G) return BSG_ERR_UNSUPPORTED_SHAPE;
  const int64_t M_total = (int64_t)(G > 0 ? G : 0) * max_m;
  const int st = grouped_fp8_check(A, lda, sfa, ld_sfa, B, ldb, stride_b, sfb, ld_sfb, stride_sfb, D,
                                   ldd, masked_m, G, M_total, N, K);
  if (st != BSG_OK || M_total == 0 || N == 0 || G == 0) return st;
  const int64_t kp = (K / 128 + 1) / 2;
  GemmArgs a = {};
  a.A = (const uint8_t*)A;
  a.B = (const uint8_t*)B;
  a.D = (uint16_t*)D;
  a.sfa = sfa;
  a.sfb = sfb;
  a.offsets = masked_m;
  a.cap = (int32_t)max_m;
  a.lda = lda;
  a.ldb = ldb;
  a.ldd = ldd;
  a.ld_sfa = ld_sfa;
  a.ld_sfb = ld_sfb;
  a.stride_b = stride_b;
  a.stride_sfb = stride_sfb;
  a.M = (int32_t)M_total;
  a.N = (int32_t)N;
  a.K = (int32_t)K;
  a.k_bytes = (int32_t)K;
  a.kp_count = (int32_t)kp;
  a.sfb_rows = (int32_t)((N + 127) / 128);
  a.G = G;
  if (sv_ok(sfa, ld_sfa)) return launch<KIND_FP8, BSG_MASKED_CFG, true, 1>(a, (hipStream_t)stream);
  return launch<KIND_FP8, BSG_MASKED_CFG, true, 0>(a, (hipStream_t)stream);
}

int m_grouped_gemm_bf16(const void* A, int64_t lda, const void* B, int64_t ldb, int64_t stride_b,
                        void* D, int64_t ldd, const int32_t* group_offsets, int32_t G,
                        int64_t M_total, int64_t N, int64_t K, void* stream) {
  const int st = grouped_check(KIND_BF16, A, lda, nullptr, 0, B, ldb, stride_b, nullptr, 0, 0, D,
                               ldd, group_offsets, G, M_total, N, K);
  if (st != BSG_OK || M_total == 0 || N == 0 || G == 0) return st;
  GemmArgs a = {};
  a.A = (const uint8_t*)A;
  a.B = (const uint8_t*)B;
  a.D = (uint16_t*)D;
  a.offsets = group_offsets;
  a.lda = lda * 2;
  a.ldb = ldb * 2;
  a.ldd = ldd;
  a.stride_b = stride_b * 2;
  a.M = (int32_t)M_total;
  a.N = (int32_t)N;
  a.K = (int32_t)K;
  a.k_bytes = (int32_t)(2 * K);
  a.G = G;
  return launch<KIND_BF16, BSG_GROUPED_BF16_CFG, true>(a, (hipStream_t)stream);
}

int m_grouped_gemm_fp4(const void* A, int64_t lda, const int16_t* sfa, int64_t ld_sfa,
                       const void* B, int64_t ldb, int64_t stride_b,
                       const int16_t* sfb, int64_t ld_sfb, int64_t stride_sfb,
                       void* D, int64_t ldd, const int32_t* group_offsets, int32_t G,
                       int64_t M_total, int64_t N, int64_t K, void* stream) {
  const int st = grouped_check(KIND_FP4, A, lda, sfa, ld_sfa, B, ldb, stride_b, sfb, ld_sfb,
                               stride_sfb, D, ldd, group_offsets, G, M_total, N, K);
  if (st != BSG_OK || M_total == 0 || N == 0 || G == 0) return st;
  GemmArgs a = {};
  a.A = (const uint8_t*)A;
  a.B = (const uint8_t*)B;
  a.D = (uint16_t*)D;
  a.sfa = sfa;
  a.sfb = sfb;
  a.offsets = group_offsets;
  a.lda = lda;
  a.ldb = ldb;
  a.ldd = ldd;
  a.ld_sfa = ld_sfa;
  a.ld_sfb = ld_sfb;
  a.stride_b = stride_b;
  a.stride_sfb = stride_sfb;
  a.M = (int32_t)M_total;
  a.N = (int32_t)N;
  a.K = (int32_t)K;
  a.k_bytes = (int32_t)(K / 2);
  a.kp_count = (int32_t)((K / 32 + 1) / 2);
  a.sfb_rows = (int32_t)N;
  a.G = G;
  // the per-expert scale arrays must all allow 8-byte loads: base and stride
  const bool sv = sv_ok(sfa, ld_sfa) && sv_ok(sfb, ld_sfb) && (stride_sfb % 4 == 0);
  if (sv) return launch<KIND_FP4, BSG_GROUPED_FP4_CFG, true, 1>(a, (hipStream_t)stream);
  return launch<KIND_FP4, BSG_GROUPED_FP4_CFG, true, 0>(a, (hipStream_t)stream);
}

static int launch_pack(bool unpack, const void* src, int64_t mn, int64_t kb, int64_t ld_src,
                       void* dst, int64_t ld_dst, void* stream) {
  const int64_t total = (kb + 1) / 2 * mn;
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  (void)hipGetLastError();
  if (unpack)
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)blocks), dim3(threads), 0, (hipStream_t)stream,
                       (const int16_t*)src, mn, kb, ld_src, (uint8_t*)dst, ld_dst);
  else
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(threads), 0, (hipStream_t)stream,
                       (const uint8_t*)src, mn, kb, ld_src, (int16_t*)dst, ld_dst);
  return hipGetLastError() == hipSuccess ? BSG_OK : BSG_ERR_HIP;
}

// Host forms of the two kernels (stream == NULL: the caller's pointers are host
// memory and the call returns when the work is done).  No HIP call is made, so
// they also run where no GPU is present.  Same layout rule as the kernels.
static void pack_host(const uint8_t* sf, int64_t mn, int64_t kb, int64_t ld_sf, int16_t* packed,
                      int64_t ld_packed) {
  for (int64_t kp = 0; kp < (kb + 1) / 2; ++kp)
    for (int64_t r = 0; r < mn; ++r) {
      const uint32_t lo = sf[r * ld_sf + 2 * kp];
      const uint32_t hi = 2 * kp + 1 < kb ? sf[r * ld_sf + 2 * kp + 1] : 0x7Fu;
      packed[kp * ld_packed + r] = (int16_t)(uint16_t)(lo | (hi << 8));
    }
}

static void unpack_host(const int16_t* packed, int64_t mn, int64_t kb, int64_t ld_packed,
                        uint8_t* sf, int64_t ld_sf) {
  for (int64_t kp = 0; kp < (kb + 1) / 2; ++kp)
    for (int64_t r = 0; r < mn; ++r) {
      const uint32_t w = (uint16_t)packed[kp * ld_packed + r];
      sf[r * ld_sf + 2 * kp] = (uint8_t)(w & 0xFF);
      if (2 * kp + 1 < kb) sf[r * ld_sf + 2 * kp + 1] = (uint8_t)(w >> 8);
    }
}

int pack_ue8m0_scales(const uint8_t* sf, int64_t mn, int64_t kb, int64_t ld_sf, int16_t* packed,
                      int64_t ld_packed, void* stream) {
  if (mn < 0 || kb < 0) return BSG_ERR_INVALID_ARG;
  if (mn == 0 || kb == 0) return BSG_OK;
  if (!sf || !packed || ld_sf < kb || ld_packed < mn) return BSG_ERR_INVALID_ARG;
  if ((uintptr_t)packed & 1) return BSG_ERR_MISALIGNED;
  if (!stream) {
    pack_host(sf, mn, kb, ld_sf, packed, ld_packed);
    return BSG_OK;
  }
  return launch_pack(false, sf, mn, kb, ld_sf, packed, ld_packed, stream);
}

int pack_ue8m0_scales_f32(const float* sf, int64_t mn, int64_t kb, int64_t ld_sf, int16_t* packed,
                          int64_t ld_packed, int32_t* inexact, void* stream) {
  if (mn < 0 || kb < 0) return BSG_ERR_INVALID_ARG;
  if (mn == 0 || kb == 0) return BSG_OK;
  if (!sf || !packed || ld_sf < kb || ld_packed < mn) return BSG_ERR_INVALID_ARG;
  if (((uintptr_t)packed & 1) || ((uintptr_t)sf & 3) || ((uintptr_t)inexact & 3))
    return BSG_ERR_MISALIGNED;
  if (!stream) {
    int32_t bad = 0;
    for (int64_t kp = 0; kp < (kb + 1) / 2; ++kp)
      for (int64_t r = 0; r < mn; ++r) {
        bool ex_lo = true, ex_hi = true;
        uint32_t b;
        const float* p = sf + r * ld_sf + 2 * kp;
        __builtin_memcpy(&b, p, 4);
        const uint32_t lo = bsg::ue8m0_of_f32(b, ex_lo);
        uint32_t hi = 0x7Fu;
        if (2 * kp + 1 < kb) {
          __builtin_memcpy(&b, p + 1, 4);
          hi = bsg::ue8m0_of_f32(b, ex_hi);
        }
        bad += !ex_lo + !ex_hi;
        packed[kp * ld_packed + r] = (int16_t)(uint16_t)(lo | (hi << 8));
      }
    if (inexact) *inexact += bad;
    return BSG_OK;
  }
  const int64_t total = (kb + 1) / 2 * mn;
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  (void)hipGetLastError();
  hipLaunchKernelGGL(bsg::pack_f32_kernel, dim3((unsigned)blocks), dim3(threads), 0,
                     (hipStream_t)stream, sf, mn, kb, ld_sf, packed, ld_packed, inexact);
  return hipGetLastError() == hipSuccess ? BSG_OK : BSG_ERR_HIP;
}

int unpack_ue8m0_scales(const int16_t* packed, int64_t mn, int64_t kb, int64_t ld_packed,
                        uint8_t* sf, int64_t ld_sf, void* stream) {
  if (mn < 0 || kb < 0) return BSG_ERR_INVALID_ARG;
  if (mn == 0 || kb == 0) return BSG_OK;
  if (!sf || !packed || ld_sf < kb || ld_packed < mn) return BSG_ERR_INVALID_ARG;
  if ((uintptr_t)packed & 1) return BSG_ERR_MISALIGNED;
  if (!stream) {
    unpack_host(packed, mn, kb, ld_packed, sf, ld_sf);
    return BSG_OK;
  }
  return launch_pack(true, packed, mn, kb, ld_packed, sf, ld_sf, stream);
}

}  // extern "C"
