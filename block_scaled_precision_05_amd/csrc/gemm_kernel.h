// gemm_kernel.h -- gfx950 GEMM kernel template for D = A * B^T (NT layout), BF16,
// FP8 e4m3 and FP4 e2m1 operands, fp32 accumulation on MFMA, bf16 output.
//
// Data path of one workgroup (WM x WN waves, one wave per SIMD):
//   HBM/L2 --buffer_load ... lds (16 B per lane, no VGPR round trip)--> LDS
//   LDS (two stages of 128 bytes of K per tile row, XOR-swizzled) --ds_read_b128--> VGPRs
//   VGPRs --v_mfma_f32_32x32x16_bf16 / v_mfma_scale_f32_32x32x64_f8f6f4--> fp32 accumulators
//   accumulators --v_cvt to bf16 (round to nearest even)--> D
// The global loads of stage k+1 are in flight while stage k is multiplied.  This
// is the MI355X counterpart of the staged, double-buffered operand pipeline the
// pages describe for the other accelerator ("DeepGEMM-Ascend cobre quantas
// operacoes no Ascend 950?", sections "O que muda de fato entre CUDA e o Huawei
// Ascend?" and "Reuso de operandos e pipelining na pratica").
//
// Scale handling (FP8 and FP4): the UE8M0 bytes go straight into the scaled
// MFMA's per-lane scale operand, so promotion by 2^(e-127) happens inside the
// matrix core and is exact.  FP8 uses one byte per (row, 128-K block): the stage
// is exactly one K-block, so every MFMA of a stage sees a row-uniform scale.
// FP4 uses one byte per (row, 32-K block): each lane's 16-byte operand is
// exactly one K-block and carries that block's byte.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsg {

enum Kind { KIND_BF16 = 0, KIND_FP8 = 1, KIND_FP4 = 2 };

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(2))) int i32x2_t;

// Kernel arguments (by value).  Leading dimensions are in bytes here.
struct GemmArgs {
  const uint8_t* A;
  const uint8_t* B;
  uint16_t* D;
  const int16_t* sfa;
  const int16_t* sfb;
  const int32_t* offsets;   // grouped only: device [G+1]
  int64_t lda;              // bytes
  int64_t ldb;              // bytes
  int64_t ldd;              // bf16 elements
  int64_t ld_sfa;           // int16 elements
  int64_t ld_sfb;           // int16 elements
  int64_t stride_b;         // grouped: bytes between experts' B
  int64_t stride_sfb;       // grouped: int16 elements between experts' scales
  int32_t M;                // rows of A (M_total for grouped)
  int32_t N;
  int32_t K;                // logical K (elements)
  int32_t k_bytes;          // bytes of K per row
  int32_t nk;               // K stages (128 bytes of K each)
  int32_t kp_count;         // rows of the packed scale arrays, ceil(Kb/2)
  int32_t sfb_rows;         // scale rows of B (ceil(N/128) for FP8, N for FP4)
  int32_t tiles_m;          // dense: M tiles
  int32_t tiles_n;
  int32_t G;                // grouped: number of experts
  int32_t d_vec;            // 1 when D rows allow 8-byte stores (D and ldd*2 8-aligned)
};

// Buffer resource word 3 for raw (unswizzled, stride 0) byte-addressed buffers on
// gfx9-family GPUs; out-of-range loads return zero.
constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kOOB = 0x80000000u;  // a byte offset past any valid record count

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}

// LDS position of 16-byte chunk c (0..7) of tile row r: rows are 128 bytes; the
// chunk is XOR-swizzled with (r/2)%8 so that 16 lanes reading one logical chunk
// of 16 consecutive rows hit 16 distinct (bank-half, chunk) pairs of the 64-bank
// LDS (conflict-free ds_read_b128).
__device__ __forceinline__ uint32_t lds_off(int r, int c) {
  return (uint32_t)(r * 128 + ((c ^ ((r >> 1) & 7)) << 4));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo;   // v_cvt_pk_bf16_f32: round to nearest even
  __bf16 b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// FP4 scaled MFMA whose scale byte (K-block s of the lane's scale word) is picked
// by the instruction's op_sel immediate.
__device__ __forceinline__ f32x16_t mfma_fp4_sel(int s, i32x8_t b, i32x8_t a, f32x16_t c,
                                                 uint32_t sb, uint32_t sa) {
  switch (s) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, 4, 4, 0, (int)sb, 0, (int)sa);
    case 1: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, 4, 4, 1, (int)sb, 1, (int)sa);
    case 2: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, 4, 4, 2, (int)sb, 2, (int)sa);
    default: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, 4, 4, 3, (int)sb, 3, (int)sa);
  }
}

template <int KIND, int BM, int BN, int WM, int WN, bool GROUPED>
struct GemmTile {
  static constexpr int NW = WM * WN;
  static constexpr int NT = NW * 64;
  static constexpr int TM = BM / WM;     // rows of A per wave
  static constexpr int TN = BN / WN;     // rows of B per wave
  static constexpr int FM = TM / 32;     // 32x32 fragments per wave along M
  static constexpr int FN = TN / 32;
  static constexpr int STAGE_BYTES = (BM + BN) * 128;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
  static constexpr int A_LOADS = BM / 8 / NW;   // buffer_load_lds x4 per wave per stage
  static constexpr int B_LOADS = BN / 8 / NW;
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be made of 32x32 fragments");
  static_assert((BM / 8) % NW == 0 && (BN / 8) % NW == 0, "rows must split evenly over waves");
  static_assert(LDS_BYTES <= 163840, "two stages must fit in LDS");
};

// Wave-wide inclusive prefix sum of one int per lane.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  return v;
}

// Grouped scheduler state: experts are scanned 64 at a time; `g0` is the first
// expert of the current window and `before` counts the row tiles of all experts
// ahead of it.  Row tiles are asked for in increasing order by each workgroup,
// so the window only moves forward.
struct GroupCursor {
  int g0;
  int before;
};

template <int BM>
__device__ __forceinline__ int group_tiles(const int32_t* off, int g, int G) {
  if (g >= G) return 0;
  int lo = off[g], hi = off[g + 1];
  return hi > lo ? (hi - lo + BM - 1) / BM : 0;
}

// Total row tiles over all experts.
template <int BM>
__device__ int grouped_total_row_tiles(const int32_t* off, int G) {
  int total = 0;
  for (int g0 = 0; g0 < G; g0 += 64) {
    int t = group_tiles<BM>(off, g0 + (threadIdx.x & 63), G);
    int s = wave_incl_scan(t);
    total += __shfl(s, 63, 64);
  }
  return total;
}

// Finds the expert owning row tile `rt`; returns false when rt is past the end.
template <int BM>
__device__ bool grouped_find(const int32_t* off, int G, int rt, GroupCursor& cur, int& g,
                             int& row_lo, int& row_hi) {
  const int lane = threadIdx.x & 63;
  while (cur.g0 < G) {
    int t = group_tiles<BM>(off, cur.g0 + lane, G);
    int incl = wave_incl_scan(t) + cur.before;
    uint64_t hit = __ballot(incl > rt);
    if (hit) {
      int j = __builtin_ctzll(hit);
      int incl_j = __shfl(incl, j, 64);
      int t_j = __shfl(t, j, 64);
      g = cur.g0 + j;
      int tile_in_g = rt - (incl_j - t_j);
      int base = off[g];
      row_lo = base + tile_in_g * BM;
      int end = off[g + 1];
      row_hi = row_lo + BM < end ? row_lo + BM : end;
      return true;
    }
    cur.before = __shfl(incl, 63, 64);
    cur.g0 += 64;
  }
  return false;
}

// Maps a workgroup's i-th tile to a position in the rasterised tile order so that
// the tiles one XCD works on at the same time form a compact block: workgroups are
// dispatched round-robin over the 8 XCDs, so XCD x owns a contiguous chunk of the
// order and walks it in steps of one tile per workgroup.
__device__ __forceinline__ int xcd_remap(int i, int T) {
  const int x = i & 7, j = i >> 3;
  const int q = T >> 3, rem = T & 7;
  return x * q + (x < rem ? x : rem) + j;
}

// Rasterisation: super-rows of GM M-tiles, N-major inside a super-row.
__device__ __forceinline__ void raster(int p, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int GM = 4;
  const int per_group = GM * tiles_n;
  const int grp = p / per_group;
  const int first_m = grp * GM;
  const int gm = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
  const int r = p - grp * per_group;
  tm = first_m + r % gm;
  tn = r / gm;
}

template <int KIND, int BM, int BN, int WM, int WN, bool GROUPED>
__global__ __launch_bounds__(WM* WN * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_kernel(const GemmArgs args) {
  using T = GemmTile<KIND, BM, BN, WM, WN, GROUPED>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, lg = lane >> 5;

  int total_tiles;
  GroupCursor cur{0, 0};
  if constexpr (GROUPED) {
    total_tiles = grouped_total_row_tiles<BM>(args.offsets, args.G) * args.tiles_n;
  } else {
    total_tiles = args.tiles_m * args.tiles_n;
  }

  for (int i = blockIdx.x; i < total_tiles; i += gridDim.x) {
    const int p = xcd_remap(i, total_tiles);
    int m0, m_end, n0;
    const uint8_t* Bbase = args.B;
    const int16_t* sfb = args.sfb;
    if constexpr (GROUPED) {
      const int rt = p / args.tiles_n;
      n0 = (p - rt * args.tiles_n) * BN;
      int g;
      if (!grouped_find<BM>(args.offsets, args.G, rt, cur, g, m0, m_end)) break;
      Bbase += (int64_t)g * args.stride_b;
      sfb += (int64_t)g * args.stride_sfb;
    } else {
      int tm, tn;
      raster(p, args.tiles_m, args.tiles_n, tm, tn);
      m0 = tm * BM;
      m_end = m0 + BM < args.M ? m0 + BM : args.M;
      n0 = tn * BN;
    }
    const int n_end = n0 + BN < args.N ? n0 + BN : args.N;
    const int rows_a = m_end - m0, rows_b = n_end - n0;

    // Buffer resources cover exactly the bytes of this tile's rows: rows past the
    // end of the matrix (or of the expert) read as zero.
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc(args.A + (int64_t)m0 * args.lda, (uint32_t)((rows_a - 1) * args.lda + args.k_bytes));
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(Bbase + (int64_t)n0 * args.ldb, (uint32_t)((rows_b - 1) * args.ldb + args.k_bytes));

    // Per-lane load offsets for the global->LDS copies: lane t of a wave-load
    // covering rows r0..r0+7 writes LDS bytes r0*128 + 16t, i.e. row r0 + t/8,
    // physical chunk t%8, which holds logical chunk (t%8) ^ ((row/2)%8).
    uint32_t a_voff[T::A_LOADS], b_voff[T::B_LOADS];
    int a_chunk[T::A_LOADS], b_chunk[T::B_LOADS];
#pragma unroll
    for (int q = 0; q < T::A_LOADS; ++q) {
      const int r = 8 * (q * T::NW + wave) + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      a_chunk[q] = c;
      a_voff[q] = (uint32_t)(r * args.lda) + (uint32_t)(c * 16);
    }
#pragma unroll
    for (int q = 0; q < T::B_LOADS; ++q) {
      const int r = 8 * (q * T::NW + wave) + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      b_chunk[q] = c;
      b_voff[q] = (uint32_t)(r * args.ldb) + (uint32_t)(c * 16);
    }

    auto issue_stage = [&](int kt, int buf) {
      uint8_t* sA = smem + buf * T::STAGE_BYTES;
      uint8_t* sB = sA + BM * 128;
      const int kb = kt * 128;
#pragma unroll
      for (int q = 0; q < T::A_LOADS; ++q) {
        const uint32_t off = (kb + a_chunk[q] * 16 < args.k_bytes) ? a_voff[q] + kb : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, (__attribute__((address_space(3))) void*)(sA + 8 * (q * T::NW + wave) * 128), 16, off,
            0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < T::B_LOADS; ++q) {
        const uint32_t off = (kb + b_chunk[q] * 16 < args.k_bytes) ? b_voff[q] + kb : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb, (__attribute__((address_space(3))) void*)(sB + 8 * (q * T::NW + wave) * 128), 16, off,
            0, 0, 0);
      }
    };

    // Scale rows this lane feeds to the MFMAs (clamped into the arrays; rows past
    // the end only meet zero operands).
    int sa_row[T::FM], sb_row[T::FN];
#pragma unroll
    for (int f = 0; f < T::FM; ++f) {
      int m = m0 + wm * T::TM + 32 * f + l32;
      sa_row[f] = m < args.M ? m : args.M - 1;
    }
#pragma unroll
    for (int f = 0; f < T::FN; ++f) {
      int n = n0 + wn * T::TN + 32 * f + l32;
      n = n < args.N ? n : args.N - 1;
      sb_row[f] = KIND == KIND_FP8 ? n / 128 : n;
    }
    // FP8: one byte per stage (K-block kt).  FP4: four bytes per stage for lane
    // group lg (K-blocks 8kt + 4lg + s, s = 0..3), assembled from two packed words.
    auto load_scales = [&](int kt, uint32_t* va, uint32_t* vb) {
      if constexpr (KIND == KIND_FP8) {
        const int64_t kp = kt >> 1;
        const int sh = (kt & 1) * 8;
#pragma unroll
        for (int f = 0; f < T::FM; ++f)
          va[f] = ((uint32_t)(uint16_t)args.sfa[kp * args.ld_sfa + sa_row[f]] >> sh) & 0xFF;
#pragma unroll
        for (int f = 0; f < T::FN; ++f)
          vb[f] = ((uint32_t)(uint16_t)sfb[kp * args.ld_sfb + sb_row[f]] >> sh) & 0xFF;
      } else if constexpr (KIND == KIND_FP4) {
        int kp0 = 4 * kt + 2 * lg, kp1 = kp0 + 1;
        kp0 = kp0 < args.kp_count ? kp0 : args.kp_count - 1;
        kp1 = kp1 < args.kp_count ? kp1 : args.kp_count - 1;
#pragma unroll
        for (int f = 0; f < T::FM; ++f)
          va[f] = (uint32_t)(uint16_t)args.sfa[(int64_t)kp0 * args.ld_sfa + sa_row[f]] |
                  ((uint32_t)(uint16_t)args.sfa[(int64_t)kp1 * args.ld_sfa + sa_row[f]] << 16);
#pragma unroll
        for (int f = 0; f < T::FN; ++f)
          vb[f] = (uint32_t)(uint16_t)sfb[(int64_t)kp0 * args.ld_sfb + sb_row[f]] |
                  ((uint32_t)(uint16_t)sfb[(int64_t)kp1 * args.ld_sfb + sb_row[f]] << 16);
      }
    };

    f32x16_t acc[T::FM][T::FN];
#pragma unroll
    for (int a = 0; a < T::FM; ++a)
#pragma unroll
      for (int b = 0; b < T::FN; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    uint32_t sa_cur[T::FM], sb_cur[T::FN], sa_nxt[T::FM], sb_nxt[T::FN];
    if (args.nk > 0) {
      issue_stage(0, 0);
      load_scales(0, sa_cur, sb_cur);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    const int a_row0 = wm * T::TM + l32;   // first tile row of this lane's A fragments
    const int b_row0 = wn * T::TN + l32;

    for (int kt = 0; kt < args.nk; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < args.nk) {
        issue_stage(kt + 1, buf ^ 1);
        load_scales(kt + 1, sa_nxt, sb_nxt);
      }
      const uint8_t* sA = smem + buf * T::STAGE_BYTES;
      const uint8_t* sB = sA + BM * 128;

      if constexpr (KIND == KIND_BF16) {
        // 4 k-steps of 16; lane group lg takes chunk 2s + lg.
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          bf16x8_t fa[T::FM], fb[T::FN];
#pragma unroll
          for (int f = 0; f < T::FM; ++f)
            fa[f] = *(const bf16x8_t*)(sA + lds_off(a_row0 + 32 * f, 2 * s + lg));
#pragma unroll
          for (int f = 0; f < T::FN; ++f)
            fb[f] = *(const bf16x8_t*)(sB + lds_off(b_row0 + 32 * f, 2 * s + lg));
#pragma unroll
          for (int a = 0; a < T::FM; ++a)
#pragma unroll
            for (int b = 0; b < T::FN; ++b)
              acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[b], fa[a], acc[a][b], 0, 0, 0);
        }
      } else if constexpr (KIND == KIND_FP8) {
        // 2 k-steps of 64; lane group lg takes chunks 4s + 2lg and 4s + 2lg + 1.
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          i32x8_t fa[T::FM], fb[T::FN];
#pragma unroll
          for (int f = 0; f < T::FM; ++f) {
            const i32x4_t lo = *(const i32x4_t*)(sA + lds_off(a_row0 + 32 * f, 4 * s + 2 * lg));
            const i32x4_t hi = *(const i32x4_t*)(sA + lds_off(a_row0 + 32 * f, 4 * s + 2 * lg + 1));
            fa[f] = (i32x8_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
#pragma unroll
          for (int f = 0; f < T::FN; ++f) {
            const i32x4_t lo = *(const i32x4_t*)(sB + lds_off(b_row0 + 32 * f, 4 * s + 2 * lg));
            const i32x4_t hi = *(const i32x4_t*)(sB + lds_off(b_row0 + 32 * f, 4 * s + 2 * lg + 1));
            fb[f] = (i32x8_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
#pragma unroll
          for (int a = 0; a < T::FM; ++a)
#pragma unroll
            for (int b = 0; b < T::FN; ++b)
              acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  fb[b], fa[a], acc[a][b], 0, 0, 0, (int)sb_cur[b], 0, (int)sa_cur[a]);
        }
      } else {
        // FP4: 4 k-steps of 64; lane group lg takes chunk 4lg + s = K-block 8kt + 4lg + s,
        // whose scale is byte s of the lane's assembled scale word.
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          i32x8_t fa[T::FM], fb[T::FN];
#pragma unroll
          for (int f = 0; f < T::FM; ++f) {
            const i32x4_t v = *(const i32x4_t*)(sA + lds_off(a_row0 + 32 * f, 4 * lg + s));
            fa[f] = (i32x8_t){v[0], v[1], v[2], v[3], 0, 0, 0, 0};
          }
#pragma unroll
          for (int f = 0; f < T::FN; ++f) {
            const i32x4_t v = *(const i32x4_t*)(sB + lds_off(b_row0 + 32 * f, 4 * lg + s));
            fb[f] = (i32x8_t){v[0], v[1], v[2], v[3], 0, 0, 0, 0};
          }
#pragma unroll
          for (int a = 0; a < T::FM; ++a)
#pragma unroll
            for (int b = 0; b < T::FN; ++b)
              acc[a][b] = mfma_fp4_sel(s, fb[b], fa[a], acc[a][b], sb_cur[b], sa_cur[a]);
        }
      }

      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if constexpr (KIND != KIND_BF16) {
#pragma unroll
        for (int f = 0; f < T::FM; ++f) sa_cur[f] = sa_nxt[f];
#pragma unroll
        for (int f = 0; f < T::FN; ++f) sb_cur[f] = sb_nxt[f];
      }
    }

    // Epilogue.  MFMA operands were (B fragment, A fragment), so accumulator
    // register r of lane l holds D[m][n] with m = l%32 and
    // n = 8*(r/4) + 4*(l/32) + r%4: four consecutive columns per register quad.
#pragma unroll
    for (int a = 0; a < T::FM; ++a) {
      const int m = m0 + wm * T::TM + 32 * a + l32;
      if (m >= m_end) continue;
      uint16_t* drow = args.D + (int64_t)m * args.ldd;
#pragma unroll
      for (int b = 0; b < T::FN; ++b) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + wn * T::TN + 32 * b + 8 * q + 4 * lg;
          const float v0 = acc[a][b][4 * q + 0], v1 = acc[a][b][4 * q + 1];
          const float v2 = acc[a][b][4 * q + 2], v3 = acc[a][b][4 * q + 3];
          if (args.d_vec && n + 3 < n_end) {
            i32x2_t w = {(int)pack_bf16x2(v0, v1), (int)pack_bf16x2(v2, v3)};
            *(i32x2_t*)(drow + n) = w;
          } else {
            const float vv[4] = {v0, v1, v2, v3};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < n_end) drow[n + e] = (uint16_t)(pack_bf16x2(vv[e], 0.0f) & 0xFFFF);
          }
        }
      }
    }
  }
}

}  // namespace bsg
