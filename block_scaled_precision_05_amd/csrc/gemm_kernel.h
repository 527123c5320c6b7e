// gemm_kernel.h -- gfx950 GEMM kernel template for D = A * B^T (NT layout), BF16,
// FP8 e4m3 and FP4 e2m1 operands, fp32 accumulation on MFMA, bf16 output.
//
// Data path of one workgroup (WM x WN waves; four waves: one per SIMD, eight: two):
//   HBM/L2 --buffer_load ... lds (16 B per lane, no VGPR round trip)--> LDS
//   LDS (a ring of NS stages of SB bytes of K per tile row, XOR-swizzled) --ds_read_b128--> VGPRs
//   VGPRs --v_mfma_f32_32x32x16_bf16 / v_mfma_scale_f32_32x32x64_f8f6f4--> fp32 accumulators
//   accumulators --v_cvt to bf16 (round to nearest even)--> D
//
// Software pipeline.  A stage is SB bytes of K for every row of the tile, split
// into J k-steps of one MFMA per (A fragment, B fragment) pair; the LDS holds a
// ring of NS stages.  Fragments are double-buffered in registers: the LDS reads
// of k-step j+1 are interleaved with the MFMAs of k-step j.  The single
// workgroup barrier of a stage sits before its last k-step, whose fragments are
// already in registers, so the matrix cores keep working while the waves meet;
// it waits (explicit vmcnt) only for the copies of the next stage, never for the
// whole ring.  Copies into the buffers that barrier released start right after
// it and trickle out between the MFMAs of the following k-steps, so NS-1 or
// NS-2 stages of MFMA time cover each copy.  With 64-byte stages the copies go
// in pairs of stages, so the two halves of each 128-byte line are requested back
// to back.  This is the MI355X counterpart of the staged, multi-buffered operand
// pipeline with ready signals that the pages describe for the other accelerator
// ("DeepGEMM-Ascend cobre quantas operacoes no Ascend 950?", sections "O que
// muda de fato entre CUDA e o Huawei Ascend?" and "Reuso de operandos e
// pipelining na pratica").
//
// Scale handling (FP8 and FP4): the UE8M0 bytes go straight into the scaled
// MFMA's per-lane scale operand, so promotion by 2^(e-127) happens inside the
// matrix core and is exact; the instruction's per-operand byte select picks one
// of the four bytes of the 32-bit scale register.  FP8 uses one byte per (row,
// 128-K block): the two 64-byte stages of a pair lie in one K-block and share
// its scale word.  FP4 uses one byte per (row, 32-K block): each lane's 16-byte
// operand is exactly one K-block and carries that block's byte.  Operands with a
// scale per row permute the rows of each wave block (GemmTile::PERM_A, PERM_B)
// so that a lane's fragment rows (four, or two for a 64-column B block), and
// their packed scale words, are adjacent: one 8-byte (4-byte) load fetches them.  Scale words are loaded together
// with the tile copy of their stage and only decoded after the barrier that
// waits for that copy, so they never add a wait.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "quant_math.h"
#include <utility>

namespace bsg {

enum Kind { KIND_BF16 = 0, KIND_FP8 = 1, KIND_FP4 = 2 };

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(2))) int i32x2_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

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
  int32_t nk;               // K stages (SB bytes of K each)
  int32_t kp_count;         // rows of the packed scale arrays, ceil(Kb/2)
  int32_t sfb_rows;         // scale rows of B (ceil(N/128) for FP8, N for FP4)
  int32_t tiles_m;          // dense: M tiles
  int32_t tiles_n;
  int32_t G;                // grouped: number of experts
  int32_t d_vec;            // widest D store: 2 = 16 bytes (D and ldd*2 16-aligned), 1 = 8, 0 = 2
  int32_t cap;              // grouped: 0 = contiguous experts, rows [offsets[g], offsets[g+1]);
                            // > 0 = masked layout, rows [g*cap, g*cap + min(offsets[g], cap))
  // SwiGLU epilogue (up-projection of an FFN, EPI > 0): B holds [gate; up] rows of
  // each expert, gate in rows [0, inter), up in [inter, 2*inter); a tile of BN B
  // rows takes BN/2 gate and the matching BN/2 up rows; instead of D the tile writes
  // Y = fp8(silu(gate) * up) [M][ldy bytes] and its 1x128 UE8M0 scales, packed int16
  // MN-major sfy [ceil(inter/256)][ld_sfy].
  uint8_t* Y;
  int16_t* sfy;
  int64_t ldy;
  int64_t ld_sfy;
  int32_t inter;
};

// Buffer resource word 3 for raw (unswizzled, stride 0) byte-addressed buffers on
// gfx9-family GPUs; out-of-range loads return zero.
constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kOOB = 0x80000000u;  // a byte offset past any valid record count

// Every caller passes a wave-uniform base and size; reading them from the first
// lane states that to the compiler, which otherwise may keep a descriptor in
// VGPRs and wrap each buffer access in a loop over lanes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(lo | (hi << 32)), (short)0,
                                           __builtin_amdgcn_readfirstlane((int)bytes), kRsrcWord3);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo;   // v_cvt_pk_bf16_f32: round to nearest even
  __bf16 b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Scaled MFMA (32x32x64, fp32 accumulate).  FMT 0 = e4m3, 4 = e2m1; the scale byte
// used is byte SEL of each lane's scale word (the instruction's op_sel immediate).
template <int FMT, int SEL>
__device__ __forceinline__ f32x16_t mfma_scaled(i32x8_t b, i32x8_t a, f32x16_t c, uint32_t sb,
                                                uint32_t sa) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, FMT, FMT, SEL, (int)sb, SEL,
                                                         (int)sa);
}

// Scaled MFMA with separate byte selects for the B and A scale words.
template <int FMT, int SELB, int SELA>
__device__ __forceinline__ f32x16_t mfma_scaled2(i32x8_t b, i32x8_t a, f32x16_t c, uint32_t sb,
                                                 uint32_t sa) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, FMT, FMT, SELB, (int)sb, SELA,
                                                         (int)sa);
}

// Compile-time shape of one kernel instance.
//   BM x BN   workgroup tile, WM x WN waves (one per SIMD), each wave TM x TN made
//             of 32x32 MFMA fragments (FM x FN of them);
//   SB        bytes of K per tile row per stage (64 or 128): 16-byte chunks NC;
//   NS        LDS stages in the ring;
//   PR        0: the copy of stage s+NS is issued at the barrier of stage s, into
//             the buffer stage s just released (NS-1 stages ahead);
//             1 (64-byte stages only): stages are copied in pairs, the two 64-byte
//             halves of every 128-byte line back to back, so each line costs the
//             memory system one request.  A pair (t, t+1) starts at the barrier of
//             stage t-NS+1, which frees the buffers of stages t-NS and t-NS+1, and
//             its copies are spread over the next 2J k-steps (one chunk per
//             k-step): a copy instruction waits in the address unit, and in-order
//             issue makes the MFMAs behind it wait too, so copies must trickle.
template <int KIND, int BM, int BN, int WM, int WN, int SB, int NS, int PR, int SV = 0, bool GR = false>
struct GemmTile {
  static constexpr int NW = WM * WN;
  static constexpr int NT = NW * 64;
  static constexpr int TM = BM / WM;     // rows of A per wave
  static constexpr int TN = BN / WN;     // rows of B per wave
  static constexpr int FM = TM / 32;     // 32x32 fragments per wave along M
  static constexpr int FN = TN / 32;
  static constexpr int NC = SB / 16;     // 16-byte chunks per row per stage
  static constexpr int RPS = 16 / NC;    // consecutive rows sharing one swizzle value
  // k-steps per stage and 16-byte LDS reads per fragment per k-step:
  //   BF16 32x32x16 (16 bytes per lane), FP8 32x32x64 (32 bytes), FP4 32x32x64 (16 bytes)
  static constexpr int J = KIND == KIND_FP8 ? NC / 4 : NC / 2;
  static constexpr int RPF = KIND == KIND_FP8 ? 2 : 1;
  static constexpr int STAGE_BYTES = (BM + BN) * SB;
  static constexpr int ROWS_PER_COPY = 1024 / SB;          // rows of one 1 KiB wave copy
  static constexpr int A_COPIES = BM / ROWS_PER_COPY;      // 1 KiB copies per stage
  static constexpr int B_COPIES = BN / ROWS_PER_COPY;
  // Waves that issue the copies.  A copy instruction holds its wave's in-order issue
  // while the CU's address unit takes it; with eight waves the upper row (waves 0 ..
  // NW/2-1, one on each SIMD: waves w and w + NW/2 share one) issues every copy and
  // the lower row none, so on each SIMD one wave's MFMAs are never held behind a copy
  // (alternating A/B at the benchmark shapes: BF16 -3.2%, FP4 -1.2%, grouped FP8 MoE
  // -1.9%, grouped FP4 -2.2%; dense FP8, whose k-step is one stage long, +0.4%, so
  // there every wave keeps its share).  GR: the grouped kernels.
  static constexpr int NWC = NW > 4 && (KIND != KIND_FP8 || GR) ? NW / 2 : NW;
  static_assert(NWC == NW || NWC == WN, "the copying waves are the upper row of waves");
  static constexpr int A_LOADS = (A_COPIES + NWC - 1) / NWC; // copies per copying wave per stage
  static constexpr int B_LOADS = (B_COPIES + NWC - 1) / NWC;
  static constexpr int N_DMA = A_LOADS + B_LOADS;
  // When the copies do not split evenly over the copying waves, the short waves issue
  // an out-of-range copy into a spare 1 KiB of LDS instead, so every copying wave
  // issues the same number of copies and the vmcnt arithmetic holds for all of them.
  static constexpr bool DUMMY = A_LOADS * NWC != A_COPIES || B_LOADS * NWC != B_COPIES;
  static constexpr int LDS_BYTES = NS * STAGE_BYTES + (DUMMY ? 1024 : 0);
  // Epilogue staging: each wave's TM x TN bf16 block, row-major (EPI_ROW bytes a
  // row) in the ring's LDS; 16-byte chunk c of row r sits at chunk c ^ epi_swz(r),
  // which walks the chunks along the rows that one lane-row group writes at once
  // (consecutive rows, or every fourth row when the rows are permuted).
  static constexpr int EPI_ROW = 2 * TN;
  static constexpr int EPI_WAVE_BYTES = TM * EPI_ROW;
  static constexpr int EPI_CHUNKS = EPI_ROW / 16;
  static_assert(TN % 8 == 0 && 64 % (TN / 8) == 0 && TM % (64 / (TN / 8)) == 0,
                "staged rows must split evenly over the lanes");
  static_assert(NW * EPI_WAVE_BYTES <= NS * STAGE_BYTES, "the epilogue staging must fit the ring");
  static_assert((EPI_CHUNKS & (EPI_CHUNKS - 1)) == 0, "the chunk swizzle is a mask");
  // SV is a set of flags.  Bit 0 (WIDE): a lane's packed scale words of its
  // fragment rows come in one wide load (below).  Bit 1 (B_ROW, FP8 only): B has
  // one scale per row and 128-wide K-block instead of one per 128x128 block.
  static constexpr bool WIDE = (SV & 1) != 0;
  static constexpr bool B_ROW = KIND == KIND_FP8 && (SV & 2) != 0;
  static_assert((SV & ~3) == 0 && (KIND == KIND_FP8 || (SV & 2) == 0), "unknown scale-form flags");
  // FP8 B scales in 128x128 blocks: one block per wave when the wave's TN rows
  // stay inside one, else one word per 32-row fragment.  Per-row B scales: one
  // word per fragment, the lane's own row.
  static constexpr bool ONE_B_SCALE = !B_ROW && TN <= 128 && 128 % TN == 0 && BN % 128 == 0;
  // A fragments double-buffered in registers (the next k-step's read beside the
  // current MFMAs) unless two waves share a SIMD on the halved register budget and
  // the fragments do not fit it (FP8: 8 registers each): then the MFMAs come first
  // and the other wave covers the read's latency.
  static constexpr bool DBA = NW <= 4 || KIND == KIND_BF16 || KIND == KIND_FP4;
  static constexpr int NSB = KIND == KIND_FP8 ? (ONE_B_SCALE ? 1 : FN) : FN;
  // packed scale words per lane per fragment per stage: FP8 one (the K-block's
  // pair), FP4 NC/4 (lane group lg takes NC/2 K-blocks of 32)
  static constexpr int SW = KIND == KIND_BF16 ? 0 : (KIND == KIND_FP8 ? 1 : NC / 4);
  // Operands with one scale per row (A for FP8 and FP4, B for FP4) permute the
  // rows of every wave block of n fragments (n = 4 for A; n = FN, 4 or 2, for
  // B): LDS slot 32f + i (fragment f, lane row i) holds block row n*i + f.  A
  // lane's n fragment rows are then adjacent in memory, and so are their packed
  // scale words: WIDE fetches them with one 8-byte (n = 4) or 4-byte (n = 2)
  // load per operand (the packed arrays must be 8-byte aligned, with leading
  // dimensions that are multiples of 4), otherwise n 2-byte loads.
  static constexpr bool PERM_A = KIND != KIND_BF16;
  static constexpr bool PERM_B = KIND == KIND_FP4;
  static constexpr bool PERM = PERM_B;   // FP4: both operands
  static_assert(!PERM_A || (FM == 4 && SW == 1),
                "the row permutation needs 128-row wave blocks and one scale word per stage");
  static_assert(!PERM_B || FN == 4 || FN == 2, "the B row permutation needs 128- or 64-row wave blocks");
  // slot x -> row within blocks of 32n rows (n a power of two; n = 1: identity)
  static constexpr int perm_rows(int n, int x) {
    return n > 1 ? ((x & ~(32 * n - 1)) | ((x & 31) * n) | ((x >> 5) & (n - 1))) : x;
  }
  static constexpr int perm_a(int x) { return perm_rows(PERM_A ? 4 : 1, x); }
  static constexpr int epi_swz(int row) {
    return (PERM_A ? (row >> 2) : row) & (EPI_CHUNKS - 1);
  }
  static constexpr int perm_b(int x) { return perm_rows(PERM_B ? FN : 1, x); }
  static constexpr int NSC = WIDE ? (1 + (PERM_B ? 1 : NSB)) * SW : (FM + NSB) * SW;
  static constexpr int VMEM_PER_STAGE = N_DMA + NSC;
  static_assert(SB == 64 || SB == 128, "a stage is 64 or 128 bytes of K per row");
  static_assert(NS >= 2 && NS <= 8, "ring of 2..8 stages");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be made of 32x32 fragments");
  static_assert(BM % ROWS_PER_COPY == 0 && BN % ROWS_PER_COPY == 0,
                "tile rows must be whole copies");
  static_assert(LDS_BYTES <= 163840, "the ring must fit in LDS");
  static_assert((NS - 1) * N_DMA <= 63, "outstanding copies must fit the vmcnt counter");
  static_assert(PR == 0 || SB == 64, "paired copies fetch the two halves of 128-byte lines");
  static_assert(PR == 0 || NS >= 3, "a pair needs two free buffers besides the one in use");
  // stages per unrolled round: buffer index and pair phase are compile-time
  static constexpr int U = PR ? (NS % 2 ? 2 * NS : NS) : NS;
  static_assert((U * J) % 2 == 0, "a round of the ring must hold an even number of k-steps");
  static constexpr int pmod(int x, int m) { return ((x % m) + m) % m; }
  // Paired issue: chunks per pair, copies of each of the two stages per chunk,
  // and the parity of the stages whose barrier starts a pair.
  static constexpr int CH = 2 * J;
  static constexpr int QPC = N_DMA / CH;
  static_assert(PR == 0 || N_DMA % CH == 0, "a pair's copies must split into whole chunks");
  static constexpr int P0 = (NS - 1) % 2;
  // chunk due at (global) k-step g, and the stage whose barrier started its pair
  static constexpr int chunk_at(int g) { return pmod(g - (P0 * J + J - 1), 2 * J); }
  static constexpr int pair_start(int g) { return (g - chunk_at(g) - (J - 1)) / J; }
  // FP8 with paired 64-byte stages: both stages of a pair lie in one 128-wide
  // K-block, so the pair loads its scale words once (chunk 0) and both stages
  // decode them from the first stage's register set.
  static constexpr bool SHARED_SCALES = PR && KIND == KIND_FP8;
  static constexpr int chunk_vmem(int g) {
    return 2 * QPC + (chunk_at(g) == 0 || (chunk_at(g) == 1 && !SHARED_SCALES) ? NSC : 0);
  }
  // Vector memory loads of one wave issued after the last copy of stage st,
  // counted at the moment the barrier of stage s waits (s = -1: the prologue's
  // wait for stage 0).  Replays the kernel's issue order: every chunk due at a
  // k-step g < 0 is issued by the prologue, the rest at their k-steps, the barrier
  // k-step's chunk after its wait; a chunk that loads scale words issues them
  // before its copies.  Non-paired: stage s+NS (its scale words, then its copies)
  // is issued whole at the barrier of s.  The scale loads count like the copies:
  // vmcnt counts every load, so leaving them out would make each barrier wait for
  // as many copies of later stages as there are scale loads after stage st (FP4
  // four, FP8 two: most of a stage, the ring one stage shallower; counting them
  // took 3 to 6% off the FP4 and grouped FP8 GEMMs).  A chunk's loads stay in
  // its k-step (a scheduling barrier closes each), and inside the chunk holding
  // stage st's last copy the compiler may only move scale loads after it, which
  // makes the wait stricter, never looser.  kd: pairs at ring positions below kd
  // (the first round's dead stages) issue nothing.
  static constexpr int copies_after(int s, int st, bool sc = true, int kd = 0) {
    const int nsc = sc ? NSC : 0;
    int issued = 0, last = -1;
    if (!PR) {
      for (int t = 0; t < NS; ++t) {
        issued += nsc;
        for (int q = 0; q < N_DMA; ++q) { if (t == st) last = issued; ++issued; }
      }
      for (int b = 0; b <= s; ++b) {
        if (b == s) return issued - 1 - last;
        issued += nsc;
        for (int q = 0; q < N_DMA; ++q) { if (b + NS == st) last = issued; ++issued; }
      }
      return issued - 1 - last;
    }
    auto chunk = [&](int g) {
      const int c = chunk_at(g), t = pair_start(g) + NS - 1;
      if (t < 0 || t < kd) return;
      if (c == 0 || (c == 1 && !SHARED_SCALES)) issued += nsc;
      for (int q = c * QPC; q < (c + 1) * QPC; ++q) {
        if (t == st) last = issued;
        ++issued;
        if (t + 1 == st) last = issued;
        ++issued;
      }
    };
    for (int g = -(NS + 2) * J; g < 0; ++g) chunk(g);
    if (s < 0) return issued - 1 - last;
    for (int g = 0;; ++g) {
      if (g % J == J - 1 && g / J == s) return issued - 1 - last;
      chunk(g);
    }
  }
  // vmcnt for the barrier of stage s (position si in the round): safe for every
  // round (the first round may differ from the steady state).  sc: the wave
  // loads scale words (a wave with no MFMAs on its tile loads none).
  static constexpr int wait_at(int si, bool sc) {
    const int a = copies_after(si, si + 1, sc), b = copies_after(si + U, si + U + 1, sc),
              c = copies_after(si + 2 * U, si + 2 * U + 1, sc);
    const int m = a < b ? a : b;
    return m < c ? m : c;
  }
  // With kd leading dead positions (KOFF > 0, paired copies) the first round is
  // peeled and its dead pairs issue nothing: the peeled round waits with its own
  // counts (none before a dead stage), the loop's rounds with theirs.
  static constexpr int wait_first(int si, bool sc, int kd) {
    return si + 1 < kd ? 63 : copies_after(si, si + 1, sc, kd);
  }
  static constexpr int wait_steady(int si, bool sc, int kd) {
    const int b = copies_after(si + U, si + U + 1, sc, kd), c = copies_after(si + 2 * U, si + 2 * U + 1, sc, kd);
    return b < c ? b : c;
  }
  static constexpr bool steady(int si) {
    return copies_after(si + U, si + U + 1, true) == copies_after(si + 2 * U, si + 2 * U + 1, true) &&
           copies_after(si + U, si + U + 1, false) == copies_after(si + 2 * U, si + 2 * U + 1, false);
  }
  static constexpr int wait_prologue(bool sc) { return copies_after(-1, 0, sc); }
  static_assert(wait_at(0, true) >= 0 && wait_at(0, true) <= 63 && wait_at(1, true) >= 0 &&
                    wait_at(1, true) <= 63 && wait_prologue(true) >= 0 && wait_prologue(true) <= 63 &&
                    wait_at(0, false) >= 0 && wait_at(1, false) >= 0 && wait_prologue(false) >= 0,
                "vmcnt is 6 bits");
  // LDS position of 16-byte chunk c of tile row r: the chunk is XOR-swizzled with
  // (r / RPS) % NC so that the 16 lanes of one ds_read_b128 phase, reading one
  // logical chunk of 16 consecutive rows, cover all 64 banks exactly once.
  static __device__ __forceinline__ uint32_t lds_off(int r, int c) {
    return (uint32_t)(r * SB + ((c ^ ((r / RPS) % NC)) << 4));
  }
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

// Rows of expert g: [off[g], off[g+1]) in the contiguous layout, or, in the masked
// layout (cap > 0, off = per-expert valid counts), the first min(off[g], cap) of
// its cap rows.
// Rows of expert g.  The offsets live on the device and are not checked by the
// host; clamped here into [0, M] (contiguous layout: lo <= hi <= M; masked: the
// count into [0, cap]), offsets that break the precondition give wrong rows but
// never an access outside A, D or their scales.
__device__ __forceinline__ void group_range(const int32_t* off, int g, int cap, int M, int& lo,
                                            int& hi) {
  if (cap > 0) {
    const int m = off[g];
    lo = g * cap;
    hi = lo + (m < 0 ? 0 : (m > cap ? cap : m));
  } else {
    const int a = off[g], b = off[g + 1];
    lo = a < 0 ? 0 : (a > M ? M : a);
    hi = b < lo ? lo : (b > M ? M : b);
  }
}

template <int BM>
__device__ __forceinline__ int group_tiles(const int32_t* off, int g, int G, int cap, int M) {
  if (g >= G) return 0;
  int lo, hi;
  group_range(off, g, cap, M, lo, hi);
  return hi > lo ? (hi - lo + BM - 1) / BM : 0;
}

// Total row tiles over all experts.
template <int BM>
__device__ int grouped_total_row_tiles(const int32_t* off, int G, int cap, int M) {
  int total = 0;
  for (int g0 = 0; g0 < G; g0 += 64) {
    int t = group_tiles<BM>(off, g0 + (threadIdx.x & 63), G, cap, M);
    int s = wave_incl_scan(t);
    total += __shfl(s, 63, 64);
  }
  return total;
}

// Finds the expert owning row tile `rt` (row tiles numbered over all experts in
// order); returns false when rt is past the end.  Outputs the expert g, the index
// of its first row tile, its number of row tiles and its row range.
template <int BM>
__device__ bool grouped_find(const int32_t* off, int G, int cap, int M, int rt, GroupCursor& cur,
                             int& g, int& tile0, int& ntiles, int& row_lo, int& row_hi) {
  const int lane = threadIdx.x & 63;
  while (cur.g0 < G) {
    int t = group_tiles<BM>(off, cur.g0 + lane, G, cap, M);
    int incl = wave_incl_scan(t) + cur.before;
    uint64_t hit = __ballot(incl > rt);
    if (hit) {
      int j = __builtin_ctzll(hit);
      int incl_j = __shfl(incl, j, 64);
      ntiles = __shfl(t, j, 64);
      g = cur.g0 + j;
      tile0 = incl_j - ntiles;
      group_range(off, g, cap, M, row_lo, row_hi);
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
template <int GM>
__device__ __forceinline__ void raster(int p, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int per_group = GM * tiles_n;
  const int grp = p / per_group;
  const int first_m = grp * GM;
  const int gm = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
  const int r = p - grp * per_group;
  tm = first_m + r % gm;
  tn = r / gm;
}

// Interleaves, inside one scheduling region, each MFMA with the next LDS read and
// the next global load, front-loading the loads so their latency hides behind the
// remaining MFMAs.
template <int NMFMA, int NDS, int NVMEM, int I>
__device__ __forceinline__ void interleave_one() {
  constexpr int ds_per = (NDS + NMFMA - 1) / NMFMA;
  constexpr int ds_n = I * ds_per < NDS ? ((NDS - I * ds_per) < ds_per ? NDS - I * ds_per : ds_per) : 0;
  // global loads spread evenly over the MFMAs (front-loaded LDS reads)
  constexpr int vm_n = (I + 1) * NVMEM / NMFMA - I * NVMEM / NMFMA;
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                        // MFMA
  if constexpr (ds_n > 0) __builtin_amdgcn_sched_group_barrier(0x100, ds_n, 0);  // DS read
  if constexpr (vm_n > 0) __builtin_amdgcn_sched_group_barrier(0x020, vm_n, 0);  // VMEM read
}

template <int NMFMA, int NDS, int NVMEM>
__device__ __forceinline__ void interleave() {
  [&]<int... is>(std::integer_sequence<int, is...>) {
    (interleave_one<NMFMA, NDS, NVMEM, is>(), ...);
  }(std::make_integer_sequence<int, NMFMA>{});
}

// s_waitcnt immediate (gfx9 encoding) that waits until at most `vm` vector memory
// loads are outstanding and every LDS access has completed.
template <int VM>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(VM >= 0 && VM <= 63, "vmcnt is 6 bits");
  constexpr int imm = (VM & 15) | (7 << 4) | (0 << 8) | ((VM >> 4) << 14);
  __builtin_amdgcn_s_waitcnt(imm);
}

// The same without the LDS part: waits for the vector memory loads only.
template <int VM>
__device__ __forceinline__ void wait_vm() {
  static_assert(VM >= 0 && VM <= 63, "vmcnt is 6 bits");
  constexpr int imm = (VM & 15) | (7 << 4) | (15 << 8) | ((VM >> 4) << 14);
  __builtin_amdgcn_s_waitcnt(imm);
}

// Workgroup barrier of the LDS ring.  The caller waits for exactly the copies and
// LDS reads it needs first (wait_vm_lds); a __syncthreads() would also wait for
// every copy still in flight, which would empty the ring at each stage.  The
// signal fences keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void ring_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int KIND, int BM, int BN, int WM, int WN, int SB, int NS, int PR, bool GROUPED, int SV = 0,
          int KOFF = 0, int EPI = 0>
__global__ __launch_bounds__(WM* WN * 64)
__attribute__((amdgpu_waves_per_eu((WM * WN + 3) / 4, (WM * WN + 3) / 4)))
void gemm_kernel(const GemmArgs args) {
  using T = GemmTile<KIND, BM, BN, WM, WN, SB, NS, PR, SV, GROUPED>;
  constexpr int FM = T::FM, FN = T::FN, J = T::J, RPF = T::RPF, NC = T::NC, SW = T::SW;
  // EPI: 0 = bf16 D; 1 + rule = SwiGLU and FP8 1x128 requantisation (rule CEIL / OCP_MX)
  static_assert(EPI == 0 || (KIND == KIND_FP8 && GROUPED && !T::PERM_B && T::ONE_B_SCALE &&
                             (BN / 2) % (T::NWC * T::ROWS_PER_COPY) == 0 && BN / 2 == 128 && T::TN <= 64),
                "the SwiGLU epilogue: FP8 grouped tiles whose B copies and scale blocks stay in one half");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, lg = lane >> 5;
  const int nk = args.nk;
  // The stage loop runs whole rounds of U stages (buffer indices and register sets
  // are compile-time), so nk is padded up to whole rounds.  The padding either sits
  // at the end, where those stages multiply zeros, or (KOFF > 0) at the start of the
  // first round: KOFF stages that hold no data, an even count so that paired stages
  // stay the two halves of one 128-byte line.  The first round, peeled off the loop,
  // issues no copies or scale loads for them (each load instruction, even one that
  // reads nothing, holds the CU's address unit for 16 cycles) and leaves out their
  // MFMAs; its barriers wait with counts of their own.  The launcher picks KOFF =
  // U - nk % U rounded down to even (one stage stays at the end when nk is odd; FP8
  // keeps a padding under 2% at the end).  Ring position p holds K stage p - KOFF.
  static_assert(KOFF >= 0 && KOFF < T::U && KOFF % 2 == 0, "leading dead stages: even, under a round");
  constexpr int koff = KOFF;
  const int nk_pad = (nk + koff + T::U - 1) / T::U * T::U;

  int total_tiles;
  GroupCursor cur{0, 0};
  if constexpr (GROUPED) {
    total_tiles = grouped_total_row_tiles<BM>(args.offsets, args.G, args.cap, args.M) * args.tiles_n;
  } else {
    total_tiles = args.tiles_m * args.tiles_n;
  }

  // Per-lane LDS byte offsets of this lane's fragment reads for k-step j (fragment
  // f adds 32*f rows; the swizzle depends only on l32 since 32 rows is a whole
  // number of swizzle periods).
  //   BF16: lane group lg reads chunk 2j + lg (8 bf16 = K 16j + 8lg .. +7).
  //   FP8:  chunks 4j + 2lg and 4j + 2lg + 1 (32 e4m3 values).
  //   FP4:  chunk (NC/2)*lg + j (32 e2m1 values = one 32-wide K-block).
  const int a_row0 = wm * T::TM + l32;
  const int b_row0 = wn * T::TN + l32;
  uint32_t a_rd[J][RPF], b_rd[J][RPF];
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int h = 0; h < RPF; ++h) {
      const int c = KIND == KIND_BF16 ? 2 * j + lg
                                      : (KIND == KIND_FP8 ? 4 * j + 2 * lg + h : (NC / 2) * lg + j);
      a_rd[j][h] = T::lds_off(a_row0, c);
      b_rd[j][h] = (uint32_t)(BM * SB) + T::lds_off(b_row0, c);
    }

  // Copy lanes: lane t of a wave copy covering rows r0 .. r0 + 1024/SB - 1 writes
  // LDS bytes r0*SB + 16t, i.e. row r0 + t/NC, physical chunk t%NC, which holds
  // logical chunk (t%NC) ^ swizzle(row).  Copy q of copying wave w starts at row
  // r0 = (q*NWC + w) * 1024/SB, and r0 / RPS = 4*(q*NWC + w), so the swizzle of a
  // copy row is (4w + (t/NC)/RPS) % NC whatever q is.
  static_assert((4 * T::NWC) % NC == 0, "copy swizzle must not depend on the copy index");
  const int cp_row = lane / NC;
  const int cp_c16 = 16 * ((lane % NC) ^ ((4 * wave + cp_row / T::RPS) % NC));

  for (int i = blockIdx.x; i < total_tiles; i += gridDim.x) {
    const int p = xcd_remap(i, total_tiles);
    int m0, m_end, n0;
    const uint8_t* Bbase = args.B;
    const int16_t* sfb = args.sfb;
    if constexpr (GROUPED) {
      // An expert's tiles form a contiguous range of the order; inside it they
      // are rasterised like a dense matrix (super-rows of two row tiles, N-major),
      // so the tiles an XCD runs together share expert weights as well as rows.
      // (Two-row super-rows measured 1% faster than four on the MoE shapes.)
      int g, tile0, ntl, row_lo, row_hi;
      if (!grouped_find<BM>(args.offsets, args.G, args.cap, args.M, p / args.tiles_n, cur, g, tile0, ntl,
                            row_lo, row_hi))
        break;
      int tm, tn;
      raster<2>(p - tile0 * args.tiles_n, ntl, args.tiles_n, tm, tn);
      m0 = row_lo + tm * BM;
      m_end = m0 + BM < row_hi ? m0 + BM : row_hi;
      n0 = tn * (EPI ? BN / 2 : BN);
      Bbase += (int64_t)g * args.stride_b;
      sfb += (int64_t)g * args.stride_sfb;
    } else {
      int tm, tn;
      raster<4>(p, args.tiles_m, args.tiles_n, tm, tn);
      m0 = tm * BM;
      m_end = m0 + BM < args.M ? m0 + BM : args.M;
      n0 = tn * BN;
    }
    m0 = __builtin_amdgcn_readfirstlane(m0);
    m_end = __builtin_amdgcn_readfirstlane(m_end);
    n0 = __builtin_amdgcn_readfirstlane(n0);

    // Waves whose rows all lie past the edge (the lower row of waves on an
    // expert's last row tile when it holds at most BM/2 rows) run the tile without
    // MFMAs, fragment reads, scale loads or stores, and meet every barrier; the SIMD
    // they share with a computing wave is left to it.  When every wave copies (NWC ==
    // NW) they still issue their share of the copies, and their barriers wait with
    // counts for a wave without scale loads.
    auto tile_body = [&](auto mm_c, auto iss_c) __attribute__((always_inline)) {
      constexpr bool MM = decltype(mm_c)::value;
      constexpr bool ISS = decltype(iss_c)::value;   // the wave issues copies
      const int n_end = n0 + BN < args.N ? n0 + BN : args.N;
      const int rows_a = m_end - m0, rows_b = n_end - n0;

      // Buffer resources cover exactly the bytes of this tile's rows: rows past the
      // end of the matrix (or of the expert) read as zero.
      const __amdgpu_buffer_rsrc_t ra =
          make_rsrc(args.A + (int64_t)m0 * args.lda, (uint32_t)((rows_a - 1) * args.lda + args.k_bytes));
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(
          Bbase + (int64_t)n0 * args.ldb,
          (uint32_t)(((EPI ? args.inter + BN / 2 : rows_b) - 1) * args.ldb + args.k_bytes));
      // Copy q of a copying wave fills LDS rows (slots) (q*NWC + wave) * ROWS_PER_COPY + cp_row
      // from tile row perm(slot); the lane part and the q part of the slot occupy
      // disjoint bits, so perm splits into a per-lane row and a per-q row.
      uint32_t a_vbase = (uint32_t)(T::perm_a(T::ROWS_PER_COPY * wave + cp_row) * args.lda) + cp_c16;
      uint32_t b_vbase = (uint32_t)(T::perm_b(T::ROWS_PER_COPY * wave + cp_row) * args.ldb) + cp_c16;
      // Opaque per tile: otherwise the compiler hoists every copy offset of the
      // prologue out of the tile loop and spills them all.
      asm volatile("" : "+v"(a_vbase), "+v"(b_vbase));

      // Copy q of K stage kt into LDS buffer `buf` (A copies first, then B); a stage
      // before the start or past the end copies nothing (every lane's offset is out
      // of range, so no memory is read, and the LDS receives zeros).
      auto copy_one = [&](int kt, int buf, int q) {
        uint8_t* sA = smem + buf * T::STAGE_BYTES;
        uint8_t* sB = sA + BM * SB;
        const int kb = kt * SB;
        // outside the K extent the offset gets bit 31, which no record count reaches
        const uint32_t oob = (uint32_t)kt < (uint32_t)nk && kb + cp_c16 < args.k_bytes ? 0u : kOOB;
        uint8_t* const spare = smem + NS * T::STAGE_BYTES;
        if (q < T::A_LOADS) {
          const int ci = q * T::NWC + wave;
          const bool dummy = T::DUMMY && ci >= T::A_COPIES;
          const uint32_t qrow = (uint32_t)T::perm_a(q * T::NWC * T::ROWS_PER_COPY);
          // The row and K parts stay below 2^31 (256 rows of at most 2^31/256
          // bytes), so OR-ing or adding the out-of-range bit give the same offset;
          // the dense kernels run 1.7% faster (FP8) with the sum, the grouped ones
          // 1% slower (the compiler allocates the registers differently).
          const uint32_t off = GROUPED ? (a_vbase + qrow * (uint32_t)args.lda + kb) | oob | (dummy ? kOOB : 0u)
                                       : a_vbase + qrow * (uint32_t)args.lda + (uint32_t)kb + (oob | (dummy ? kOOB : 0u));
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              ra, (__attribute__((address_space(3))) void*)(dummy ? spare : sA + T::ROWS_PER_COPY * ci * SB),
              16, off, 0, 0, 0);
        } else {
          const int qb = q - T::A_LOADS;
          const int ci = qb * T::NWC + wave;
          const bool dummy = T::DUMMY && ci >= T::B_COPIES;
          const uint32_t qrow0 = (uint32_t)T::perm_b(qb * T::NWC * T::ROWS_PER_COPY);
          // (SwiGLU epilogue: tile rows past BN/2 are up rows, inter rows further on)
          const uint32_t qrow = EPI && qrow0 >= (uint32_t)(BN / 2) ? qrow0 - BN / 2 + (uint32_t)args.inter : qrow0;
          const uint32_t off = GROUPED ? (b_vbase + qrow * (uint32_t)args.ldb + kb) | oob | (dummy ? kOOB : 0u)
                                       : b_vbase + qrow * (uint32_t)args.ldb + (uint32_t)kb + (oob | (dummy ? kOOB : 0u));
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rb, (__attribute__((address_space(3))) void*)(dummy ? spare : sB + T::ROWS_PER_COPY * ci * SB),
              16, off, 0, 0, 0);
        }
      };
      auto issue_stage = [&](int kt, int buf) {
        if constexpr (ISS) {
#pragma unroll
          for (int q = 0; q < T::N_DMA; ++q) copy_one(kt, buf, q);
        }
      };
      // Chunk c of pair (kt, kt+1): copies c*QPC .. (c+1)*QPC-1 of both stages, the
      // two halves of every line back to back.
      auto issue_chunk = [&](int kt, int buf0, int buf1, int c) {
        if constexpr (ISS) {
#pragma unroll
          for (int q = 0; q < T::QPC; ++q) {
            copy_one(kt, buf0, c * T::QPC + q);
            copy_one(kt + 1, buf1, c * T::QPC + q);
          }
        }
      };

      // Scale loads.  Each lane reads the packed words of the rows it feeds to the
      // MFMAs: A row m0 + wm*TM + 32f + l32 (f < FM), whose word sits 64f bytes after
      // fragment 0's; for FP4 B row n likewise; for FP8 the 128-row block of B that
      // holds the wave's rows (one block) or fragment f's 32 rows.  Rows past M or N
      // read some other finite word or zero (out of range): they only meet zero
      // operands and their outputs are never stored.
      constexpr int NSB = T::NSB;   // B scale words per lane per packed row
      const int nrow0 = n0 + wn * T::TN;   // first B row of this wave (uniform)
      // The records end after the last packed row's scale rows; with the wide scale
      // loads (SV) they extend to the next multiple of four rows, which a wide load
      // of the last row group reads whole (the launcher takes SV only when the
      // leading dimension is a multiple of 4, so those words lie inside the array):
      // a record ending at row M would drop the valid words of a dword that
      // straddles it.
      constexpr bool SV_B = T::WIDE && T::PERM_B;
      const int a_rows = T::WIDE ? (args.M + 3) & ~3 : args.M;
      const int b_rows = SV_B ? (args.sfb_rows + 3) & ~3 : args.sfb_rows;
      const __amdgpu_buffer_rsrc_t rsa = make_rsrc(
          args.sfa, (uint32_t)(2 * ((int64_t)(args.kp_count - 1) * args.ld_sfa + a_rows)));
      const __amdgpu_buffer_rsrc_t rsb = make_rsrc(
          sfb, (uint32_t)(2 * ((int64_t)(args.kp_count - 1) * args.ld_sfb + b_rows)));
      // (FP4: the lane's fragment rows are 4*l32 .. 4*l32 + 3 of the wave block)
      // (FP4: lane group lg reads packed rows (NC/4)*lg further on)
      const uint32_t ld_a = (uint32_t)args.ld_sfa, ld_b = (uint32_t)args.ld_sfb;
      constexpr uint32_t lg_rows = KIND == KIND_FP4 ? NC / 4 : 0;
      uint32_t sa_voff = 2u * (uint32_t)(m0 + wm * T::TM + (T::PERM_A ? 4 * l32 : l32)) +
                         2u * lg_rows * (uint32_t)lg * ld_a;
      asm volatile("" : "+v"(sa_voff));
      const int brow0 = EPI && wn * T::TN >= BN / 2 ? args.inter + n0 + wn * T::TN - BN / 2 : n0 + wn * T::TN;
      uint32_t sb_voff = KIND == KIND_FP8 && !T::B_ROW
                             ? 2u * (uint32_t)(brow0 / 128)
                             : 2u * (uint32_t)(n0 + wn * T::TN + (T::PERM_B ? FN * l32 : l32)) +
                                   2u * lg_rows * (uint32_t)lg * ld_b;
      asm volatile("" : "+v"(sb_voff));
      // Raw scale words of stage kt (packed int16, not decoded yet).
      //   FP8: K-block kt*SB/128, held in packed row kb/2, byte kb%2.
      //   FP4: lane group lg needs K-blocks kt*NC + (NC/2)*lg + j (j < NC/2), the
      //        packed rows kt*NC/2 + (NC/4)*lg + w for w < NC/4.
      // Raw scale words, one register set per ring slot (the slot is a compile-time
      // value at every call).  FP4 with SV: the two dwords of each operand's 8-byte
      // load, fragments 2i and 2i+1 in the low and high halves of dword i.
      uint16_t rs_a[NS][FM][SW > 0 ? SW : 1] = {}, rs_b[NS][NSB][SW > 0 ? SW : 1] = {};
      uint32_t rv_a[T::WIDE ? NS : 1][2] = {}, rv_b[T::WIDE ? NS : 1][2] = {};
      // The barrier waits count these loads (a wave that runs the tile without MFMAs
      // issues none), so every call must issue exactly its loads: each address is
      // made opaque, so that no two calls merge (the clamped stages of the first
      // round read the same words), and decode_scales keeps every result alive.
      auto load_scales = [&](int kt, auto slot) {
        constexpr int sl = decltype(slot)::value;
        if constexpr (MM && KIND != KIND_BF16) {
#pragma unroll
          for (int w = 0; w < SW; ++w) {
            // Wave-uniform packed row (the lane group's part is in sa_voff / sb_voff).
            // FP8 clamps it to the last packed row; FP4 lane group 1 may read one row
            // past the end on a K tail, which the record count turns into zero
            // words: those scales only meet zero operands.
            int kp = KIND == KIND_FP8 ? (kt * SB / 128) >> 1 : kt * (NC / 2) + w;
            if constexpr (KIND == KIND_FP8) kp = kp < args.kp_count ? kp : args.kp_count - 1;
            kp = __builtin_amdgcn_readfirstlane(kp);
            uint32_t va = sa_voff + 2u * (uint32_t)kp * ld_a;
            uint32_t vb = sb_voff + 2u * (uint32_t)kp * ld_b;
            uint32_t kq = 2u * (uint32_t)kp * ld_b;
            asm volatile("" : "+v"(va), "+v"(vb), "+s"(kq));
            // fragment f's word: 2 bytes further on (permuted rows: adjacent) or
            // 64 bytes (32 rows) further on
            constexpr uint32_t fstep_a = T::PERM_A ? 2 : 64, fstep_b = T::PERM_B ? 2 : 64;
            if constexpr (T::WIDE) {
              const u32x2_t da = __builtin_amdgcn_raw_buffer_load_b64(rsa, va, 0, 0);
              rv_a[sl][0] = da[0];
              rv_a[sl][1] = da[1];
            } else {
#pragma unroll
              for (int f = 0; f < FM; ++f)
                rs_a[sl][f][w] = __builtin_amdgcn_raw_buffer_load_b16(rsa, va + fstep_a * f, 0, 0);
            }
            if constexpr (T::WIDE && T::PERM_B && FN == 4) {
              const u32x2_t db = __builtin_amdgcn_raw_buffer_load_b64(rsb, vb, 0, 0);
              rv_b[sl][0] = db[0];
              rv_b[sl][1] = db[1];
            } else if constexpr (T::WIDE && T::PERM_B) {
              rv_b[sl][0] = __builtin_amdgcn_raw_buffer_load_b32(rsb, vb, 0, 0);
            } else {
#pragma unroll
              for (int f = 0; f < NSB; ++f) {
                if constexpr (KIND == KIND_FP8 && !T::ONE_B_SCALE && !T::B_ROW) {
                  // (fragments in one 128-row block read the same word: opaque, so
                  // that the loads stay apart)
                  uint32_t o = 2u * (uint32_t)((nrow0 + 32 * f) >> 7) + kq;
                  asm volatile("" : "+v"(o));
                  rs_b[sl][f][w] = __builtin_amdgcn_raw_buffer_load_b16(rsb, o, 0, 0);
                } else
                  rs_b[sl][f][w] = __builtin_amdgcn_raw_buffer_load_b16(rsb, vb + fstep_b * f, 0, 0);
              }
            }
          }
        }
      };
      // Decoded per-lane scale operand of stage kt.  FP8: the K-block's byte in
      // bits 0..7.  FP4 (permuted rows): dword i holds fragment 2i's word in its low
      // half and fragment 2i+1's in its high half; k-step j of fragment f uses byte
      // 2*(f%2) + j of dword f/2, picked by the MFMA's byte select.  (The raw words
      // stay untouched until here, so nothing uses a load's result before the
      // barrier that waits for it.)
      auto decode_scales = [&](int kt, auto slot, uint32_t (&sa)[FM], uint32_t (&sb)[FN]) {
        if constexpr (!MM) return;
        constexpr int sl = decltype(slot)::value;
        if constexpr (KIND == KIND_FP8) {
          const int sh = ((kt * SB / 128) & 1) * 8;
          if constexpr (T::WIDE) {
            // the K-block's byte of fragments 2i and 2i+1 moves to bytes 0 and 2
            sa[0] = rv_a[sl][0] >> sh;
            sa[1] = rv_a[sl][1] >> sh;
          } else {
#pragma unroll
            for (int f = 0; f < FM; ++f) sa[f] = ((uint32_t)rs_a[sl][f][0] >> sh) & 0xFF;
          }
#pragma unroll
          for (int f = 0; f < FN; ++f) sb[f] = ((uint32_t)rs_b[sl][T::ONE_B_SCALE ? 0 : f][0] >> sh) & 0xFF;
          // (kept alive: a stage without MFMAs would otherwise drop its loads)
#pragma unroll
          for (int f = 0; f < (T::WIDE ? 2 : FM); ++f) asm volatile("" ::"v"(sa[f]));
#pragma unroll
          for (int f = 0; f < FN; ++f) asm volatile("" ::"v"(sb[f]));
        } else if constexpr (KIND == KIND_FP4) {
          if constexpr (T::WIDE) {
            sa[0] = rv_a[sl][0];
            sa[1] = rv_a[sl][1];
            sb[0] = rv_b[sl][0];
            if constexpr (FN > 2) sb[1] = rv_b[sl][1];
          } else {
#pragma unroll
            for (int i = 0; i < 2; ++i)
              sa[i] = (uint32_t)rs_a[sl][2 * i][0] | ((uint32_t)rs_a[sl][2 * i + 1][0] << 16);
#pragma unroll
            for (int i = 0; i < FN / 2; ++i) {
              sb[i] = (uint32_t)rs_b[sl][2 * i][0] | ((uint32_t)rs_b[sl][2 * i + 1][0] << 16);
            }
          }
#pragma unroll
          for (int i = 0; i < 2; ++i) asm volatile("" ::"v"(sa[i]));
#pragma unroll
          for (int i = 0; i < FN / 2; ++i) asm volatile("" ::"v"(sb[i]));
        }
      };

      // Fragment registers, double-buffered across k-steps.
      typedef typename std::conditional<KIND == KIND_BF16, bf16x8_t, i32x8_t>::type frag_t;
      frag_t fa[T::DBA ? 2 : 1][FM], fb[2][FN];
      auto read_frags = [&](int buf, int j, frag_t (&xa)[FM], frag_t (&xb)[FN]) {
        if constexpr (!MM) return;
        const uint8_t* base = smem + buf * T::STAGE_BYTES;
#pragma unroll
        for (int f = 0; f < FM; ++f) {
          const uint8_t* p0 = base + a_rd[j][0] + 32 * SB * f;
          if constexpr (KIND == KIND_BF16) {
            xa[f] = *(const bf16x8_t*)p0;
          } else if constexpr (KIND == KIND_FP8) {
            const i32x4_t lo = *(const i32x4_t*)p0;
            const i32x4_t hi = *(const i32x4_t*)(base + a_rd[j][RPF - 1] + 32 * SB * f);
            xa[f] = (i32x8_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          } else {
            const i32x4_t v = *(const i32x4_t*)p0;
            xa[f] = (i32x8_t){v[0], v[1], v[2], v[3], 0, 0, 0, 0};
          }
        }
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          const uint8_t* p0 = base + b_rd[j][0] + 32 * SB * f;
          if constexpr (KIND == KIND_BF16) {
            xb[f] = *(const bf16x8_t*)p0;
          } else if constexpr (KIND == KIND_FP8) {
            const i32x4_t lo = *(const i32x4_t*)p0;
            const i32x4_t hi = *(const i32x4_t*)(base + b_rd[j][RPF - 1] + 32 * SB * f);
            xb[f] = (i32x8_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          } else {
            const i32x4_t v = *(const i32x4_t*)p0;
            xb[f] = (i32x8_t){v[0], v[1], v[2], v[3], 0, 0, 0, 0};
          }
        }
      };

      f32x16_t acc[FM][FN];
#pragma unroll
      for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

      // One k-step's MFMAs: acc += A_frag x B_frag for every fragment pair.
      auto mfmas = [&](auto jc, const frag_t (&xa)[FM], const frag_t (&xb)[FN], const uint32_t (&sa)[FM],
                       const uint32_t (&sb)[FN]) {
        constexpr int j = decltype(jc)::value;
        if constexpr (!MM) return;
        if constexpr (KIND == KIND_FP8 && T::WIDE) {
          // A fragment f's scale: byte 2*(f%2) of dword f/2 (decoded per K-block)
          [&]<int... ab>(std::integer_sequence<int, ab...>) {
            ((acc[ab / FN][ab % FN] = mfma_scaled2<0, 0, 2 * ((ab / FN) % 2)>(
                  xb[ab % FN], xa[ab / FN], acc[ab / FN][ab % FN], sb[ab % FN], sa[(ab / FN) / 2])),
             ...);
          }(std::make_integer_sequence<int, FM * FN>{});
        } else if constexpr (T::PERM) {
          // a-outer, b-inner as below; fragment f's scale is byte 2*(f%2) + j of
          // dword f/2
          [&]<int... ab>(std::integer_sequence<int, ab...>) {
            ((acc[ab / FN][ab % FN] = mfma_scaled2<4, 2 * ((ab % FN) % 2) + j, 2 * ((ab / FN) % 2) + j>(
                  xb[ab % FN], xa[ab / FN], acc[ab / FN][ab % FN], sb[(ab % FN) / 2], sa[(ab / FN) / 2])),
             ...);
          }(std::make_integer_sequence<int, FM * FN>{});
        } else {
#pragma unroll
          for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b) {
              if constexpr (KIND == KIND_BF16)
                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xb[b], xa[a], acc[a][b], 0, 0, 0);
              else if constexpr (KIND == KIND_FP8)
                acc[a][b] = mfma_scaled<0, 0>(xb[b], xa[a], acc[a][b], sb[b], sa[a]);
              else
                acc[a][b] = mfma_scaled<4, j>(xb[b], xa[a], acc[a][b], sb[b], sa[a]);
            }
        }
      };

      uint32_t sa_cur[FM] = {}, sb_cur[FN] = {};

      // Prologue: the previous tile's LDS reads are over once every wave has
      // drained its own and met the others here; then stages 0 .. T0-1 are put in
      // flight and stage 0 is waited for.  The previous tile's D stores are not
      // waited for (a __syncthreads would wait for every outstanding memory
      // operation): their latency overlaps this tile's first copies, and since
      // loads complete in order, the prologue's vmcnt wait below still covers
      // stage 0 whatever the stores do.
      wait_vm_lds<63>();
      ring_barrier();
      // Paired copies due at a k-step g: chunk chunk_at(g) of the pair started at
      // the barrier of stage pair_start(g); chunk 0 also loads the first stage's
      // scale words, chunk 1 the second's.
      auto pair_chunk = [&](auto gc, int round) {
        constexpr int g = decltype(gc)::value;
        constexpr int c = T::chunk_at(g), tl = T::pair_start(g) + NS - 1;
        constexpr int b0 = T::pmod(tl, NS), b1 = T::pmod(tl + 1, NS);
        const int t = round + tl - koff;   // K stage of the pair's first position
        if constexpr (c == 0) load_scales(t >= 0 && t < nk ? t : 0, std::integral_constant<int, b0>{});
        if constexpr (c == 1 && !T::SHARED_SCALES)
          load_scales(t + 1 >= 0 && t + 1 < nk ? t + 1 : 0, std::integral_constant<int, b1>{});
        issue_chunk(t, b0, b1, c);
      };
      if constexpr (PR) {
        // every chunk due before k-step 0 (pairs with a first stage t >= 0)
        [&]<int... gs>(std::integer_sequence<int, gs...>) {
          ((T::pair_start(gs - (NS + 2) * J) + NS - 1 >= koff
                ? pair_chunk(std::integral_constant<int, gs - (NS + 2) * J>{}, 0)
                : void()),
           ...);
        }(std::make_integer_sequence<int, (NS + 2) * J>{});
      } else {
        [&]<int... bs>(std::integer_sequence<int, bs...>) {
          ((load_scales(bs - koff >= 0 && bs - koff < nk ? bs - koff : 0, std::integral_constant<int, bs>{}),
            issue_stage(bs - koff, bs)),
           ...);
        }(std::make_integer_sequence<int, NS>{});
      }
      wait_vm_lds<(!ISS || (PR && koff > 0)) ? 63 : T::wait_prologue(MM)>();
      ring_barrier();
      decode_scales(-koff, std::integral_constant<int, 0>{}, sa_cur, sb_cur);
      read_frags(0, 0, fa[0], fb[0]);

      // One stage at ring position s.  Every stage of the steady loop runs the same
      // code, free of branches around the MFMAs.  A DEAD stage (the first round's
      // leading positions, which hold no data) keeps the barrier and the fragment
      // reads (of buffers no copy fills) and leaves out the MFMAs; the pairs of dead
      // positions issue neither copies nor scale loads, and the first round's
      // barriers wait for the live loads it did issue (wait_first).
      auto stage = [&](auto ic, auto deadc, auto firstc, int s) {
        constexpr int si = decltype(ic)::value;   // position of the stage in the round
        constexpr bool DEAD = decltype(deadc)::value;
        constexpr bool FIRST = decltype(firstc)::value;   // the peeled first round
        // (a wave that issues no copies has none to wait for: the copying waves'
        // waits and the barrier cover the stage, and the compiler waits for its scale
        // words where it decodes them)
        constexpr int WAIT_SI = !ISS ? 63
                                : (!PR || koff == 0 ? T::wait_at(si, MM)
                                   : (FIRST ? T::wait_first(si, MM, koff) : T::wait_steady(si, MM, koff)));
        constexpr int buf = si % NS;
        constexpr int nbuf = (buf + 1) % NS;
        static_assert(!PR || T::steady(si), "the copy schedule must repeat every round");
        const int round = s - si;
        // dead pairs of the first round issue nothing (their copies would read
        // nothing and their scale words are never used)
        auto chunk_at_g = [&](auto gc) __attribute__((always_inline)) {
          constexpr int gg = decltype(gc)::value;
          if constexpr (!(FIRST && T::pair_start(gg) + NS - 1 < koff)) pair_chunk(gc, round);
        };
        auto body = [&](auto jc) {
          constexpr int j = decltype(jc)::value;
          constexpr int g = si * J + j;             // k-step index within the round
          constexpr int nvm = PR ? T::chunk_vmem(g) - (ISS ? 0 : 2 * T::QPC)
                                 : (j + 1 < J ? 0 : (ISS ? T::VMEM_PER_STAGE : T::NSC));
          // fragment register set of this k-step: k-steps alternate sets across
          // stage boundaries too (a round has an even number of them)
          constexpr int cu = (si * J + j) & 1, nx = cu ^ 1;
          constexpr int ca = T::DBA ? cu : 0, na = T::DBA ? nx : 0;
          if constexpr (j + 1 < J) {
            if constexpr (T::DBA) {
              read_frags(buf, j + 1, fa[na], fb[nx]);
              if constexpr (PR) chunk_at_g(std::integral_constant<int, g>{});
              if constexpr (!DEAD) mfmas(jc, fa[ca], fb[cu], sa_cur, sb_cur);
            } else {
              if constexpr (PR) chunk_at_g(std::integral_constant<int, g>{});
              if constexpr (!DEAD) mfmas(jc, fa[ca], fb[cu], sa_cur, sb_cur);
              read_frags(buf, j + 1, fa[na], fb[nx]);
            }
            if constexpr (MM && !DEAD) interleave<FM * FN, (FM + FN) * RPF, nvm>();
            __builtin_amdgcn_sched_barrier(0);
          } else {
            // Stage s+1 has landed once no more than wait_at() of this wave's copies
            // are outstanding and every wave has passed the barrier.  A barrier that
            // starts a pair of copies also hands that pair the buffers read before
            // it, so there every wave first waits for its own LDS reads; at the other
            // barriers no copy targets a buffer just read, the reads stay in flight
            // across the barrier, and the compiler waits for each one just before
            // the first MFMA that uses its registers.
            if constexpr (PR && T::chunk_at(g) != 0)
              wait_vm<WAIT_SI>();
            else
              wait_vm_lds<WAIT_SI>();
            ring_barrier();
            if constexpr (PR) {
              chunk_at_g(std::integral_constant<int, g>{});
            } else {
              const int kt = s + NS - koff;
              load_scales(kt >= 0 && kt < nk ? kt : 0, std::integral_constant<int, buf>{});
              issue_stage(kt, buf);
            }
            if constexpr (T::DBA) {
              read_frags(nbuf, 0, fa[na], fb[nx]);
              if constexpr (!DEAD) mfmas(jc, fa[ca], fb[cu], sa_cur, sb_cur);
            } else {
              if constexpr (!DEAD) mfmas(jc, fa[ca], fb[cu], sa_cur, sb_cur);
              read_frags(nbuf, 0, fa[na], fb[nx]);
            }
            if constexpr (MM && !DEAD) interleave<FM * FN, (FM + FN) * RPF, nvm>();
            __builtin_amdgcn_sched_barrier(0);
            // (shared scales: stage s+1 reads the set of its pair's first stage)
            constexpr int sbuf = T::SHARED_SCALES ? T::pmod(((si + 1) & ~1), NS) : nbuf;
            decode_scales(s + 1 - koff, std::integral_constant<int, sbuf>{}, sa_cur, sb_cur);
          }
        };
        [&]<int... js>(std::integer_sequence<int, js...>) {
          (body(std::integral_constant<int, js>{}), ...);
        }(std::make_integer_sequence<int, J>{});
      };
      // With leading dead stages the first round is peeled off the loop.  (Its
      // start is made opaque: known to be 0, it would let the compiler hoist that
      // round's copy offsets out of the tile loop and spill them.)
      if constexpr (koff > 0) {
        if (nk_pad > 0) {
          int s0 = 0;
          asm volatile("" : "+s"(s0));
          [&]<int... is>(std::integer_sequence<int, is...>) {
            (stage(std::integral_constant<int, is>{}, std::integral_constant<bool, (is < koff)>{},
                   std::true_type{}, s0 + is),
             ...);
          }(std::make_integer_sequence<int, T::U>{});
        }
      }
      for (int s = koff > 0 ? T::U : 0; s < nk_pad; s += T::U) {
        [&]<int... is>(std::integer_sequence<int, is...>) {
          (stage(std::integral_constant<int, is>{}, std::false_type{}, std::false_type{}, s + is), ...);
        }(std::make_integer_sequence<int, T::U>{});
      }

      // Epilogue.  MFMA operands were (B fragment, A fragment), so accumulator
      // register r of lane l holds D[m][n] with m = l%32 and
      // n = 8*(r/4) + 4*(l/32) + r%4: four consecutive columns per register quad.
      // Permuted rows: fragment a's row l32 is tile row 4*l32 + a; with B permuted
      // too (FP4), fragment b's column i is tile column FN*i + b, so the FN
      // fragments b hold FN consecutive columns in the same register.
      //
      // Stored straight from those registers, every store instruction would put 16
      // bytes into each of 32 rows, one L2 request per 16 bytes.  Instead each wave
      // converts its TM x TN block to bf16 into its own part of the idle LDS ring,
      // row-major, then stores it row by row with 16 bytes per lane, so an
      // instruction writes whole 2*TN-byte row segments.  The 16-byte chunks of a
      // staged row are XOR-swizzled by the row (epi_swz) so that the 32 rows one
      // write instruction touches spread over the banks.
      //
      // The ring is idle once no copy is in flight (the dead stages' out-of-range
      // copies still write zeros into it) and every wave has passed the barrier.
      wait_vm_lds<0>();
      ring_barrier();
      // rows of this wave's block that exist (an expert's last row tile, the
      // matrix edge): a wave with none skips its part
      const int rows_w = m_end - (m0 + wm * T::TM) < T::TM ? m_end - (m0 + wm * T::TM) : T::TM;
      // (the SwiGLU epilogue has every wave meet one more barrier: no early exit)
      if (EPI == 0 && rows_w <= 0) return;
      uint8_t* const stg = smem + wave * T::EPI_WAVE_BYTES;
      // The lane index, made opaque here: every staging address derives from it,
      // and the compiler would otherwise hoist all of them out of the tile loop and
      // spill them.
      int el = lane;
      asm volatile("" : "+v"(el));
      const int el32 = el & 31, elg = el >> 5;
      auto stage_quad = [&](int row, int col, float v0, float v1, float v2, float v3) {
        // four consecutive columns col .. col+3 (col a multiple of 4) of `row`
        const int chunk = (col >> 3) ^ T::epi_swz(row);
        const i32x2_t w = {(int)pack_bf16x2(v0, v1), (int)pack_bf16x2(v2, v3)};
        *(i32x2_t*)(stg + row * T::EPI_ROW + 16 * chunk + 2 * (col & 7)) = w;
      };
#pragma unroll
      for (int a = 0; a < FM; ++a) {
        const int row = T::PERM_A ? 4 * el32 + a : 32 * a + el32;
        if constexpr (T::PERM && FN == 4) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            stage_quad(row, 4 * (8 * (r / 4) + 4 * elg + r % 4), acc[a][0][r], acc[a][1][r], acc[a][2][r],
                       acc[a][3][r]);
        } else if constexpr (T::PERM) {
          // two B fragments: the same register of both holds two consecutive columns,
          // so a register quad holds one whole 16-byte chunk (8 columns), written with
          // one 16-byte store instead of four 4-byte ones (grouped FP4 MoE shape -0.7%)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int chunk = (2 * q + elg) ^ T::epi_swz(row);
            const i32x4_t w = {(int)pack_bf16x2(acc[a][0][4 * q], acc[a][1][4 * q]),
                               (int)pack_bf16x2(acc[a][0][4 * q + 1], acc[a][1][4 * q + 1]),
                               (int)pack_bf16x2(acc[a][0][4 * q + 2], acc[a][1][4 * q + 2]),
                               (int)pack_bf16x2(acc[a][0][4 * q + 3], acc[a][1][4 * q + 3])};
            *(i32x4_t*)(stg + row * T::EPI_ROW + 16 * chunk) = w;
          }
        } else {
#pragma unroll
          for (int b = 0; b < FN; ++b)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              stage_quad(row, 32 * b + 8 * q + 4 * elg, acc[a][b][4 * q], acc[a][b][4 * q + 1],
                         acc[a][b][4 * q + 2], acc[a][b][4 * q + 3]);
        }
        // one fragment row at a time: the compiler would otherwise move every
        // accumulator into VGPRs first and spill
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (EPI > 0) {
        // SwiGLU and FP8 1x128 requantisation.  Tile row r's gate values (tile columns
        // 0 .. BN/2-1) and up values (BN/2 .. BN-1) lie in the staged blocks of other
        // waves, so every wave's block must be in place first.  Wave w then takes
        // rows 32w .. 32w+31, four rows a pass, 16 lanes a row, 8 outputs a lane:
        // exactly the arithmetic of the SwiGLU quantiser, on the same bf16 values.
        wait_vm_lds<63>();
        ring_barrier();
        constexpr int RULE = EPI - 1;
        const int seg = el & 15, rsub = el >> 4;
        const int blk = n0 / 128, kb_total = args.inter / 128;
        const int gcol = 8 * seg, ucol = BN / 2 + 8 * seg;
#pragma unroll 1
        for (int it = 0; it < 8; ++it) {
          const int row = 32 * wave + 4 * it + rsub;
          const int wmr = row / T::TM, r_in = row - wmr * T::TM;
          const int sw = T::epi_swz(r_in);
          const uint8_t* gp = smem + (wmr * WN + gcol / T::TN) * T::EPI_WAVE_BYTES + r_in * T::EPI_ROW +
                              16 * (((gcol % T::TN) / 8) ^ sw);
          const uint8_t* upp = smem + (wmr * WN + ucol / T::TN) * T::EPI_WAVE_BYTES + r_in * T::EPI_ROW +
                               16 * (((ucol % T::TN) / 8) ^ sw);
          const bsg_qm::qm_u32x4_t g = *(const bsg_qm::qm_u32x4_t*)gp;
          const bsg_qm::qm_u32x4_t u = *(const bsg_qm::qm_u32x4_t*)upp;
          bsg_qm::qm_u32x2_t codes;
          int byte;
          bsg_qm::swiglu_fp8x8<RULE>(g, u, codes, byte);
          if (m0 + row < m_end) {
            *(bsg_qm::qm_u32x2_t*)(args.Y + (int64_t)(m0 + row) * args.ldy + n0 + 8 * seg) = codes;
            if (seg == 0) {
              uint8_t* sp = (uint8_t*)args.sfy + 2 * ((int64_t)(blk >> 1) * args.ld_sfy + m0 + row);
              sp[blk & 1] = (uint8_t)byte;
              // an odd number of 128-blocks: the last pair's high byte is the neutral 1.0
              if ((blk & 1) == 0 && blk + 1 == kb_total) sp[1] = 0x7F;
            }
          }
        }
        return;
      }
      // (a wave reads back only what it wrote; its LDS accesses execute in order)
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      constexpr int LPR = T::TN / 8;   // lanes per staged row, 16 bytes each
      constexpr int RPI = 64 / LPR;    // rows per store instruction
      const int rr = el / LPR, seg = el % LPR;
      const int n = n0 + wn * T::TN + 8 * seg;
      const int vec = n + 7 < n_end ? args.d_vec : 0;
      // The stores carry the non-temporal hint: D is written once and never read
      // here, and a tile-wave of workgroups writes about 4 MB per XCD at once, as much
      // as its L2, which would otherwise evict the operand lines the next tiles read
      // (alternating A/B: 0.3-1.9% faster on every shape).
      const uint8_t* src = stg + rr * T::EPI_ROW;
      uint16_t* d = args.D + (int64_t)(m0 + wm * T::TM + rr) * args.ldd + n;
      const int64_t dstep = (int64_t)RPI * args.ldd;
      // Whole blocks with 16-byte stores on every lane (the common case): every row
      // read back first, then every store, so the LDS reads overlap (grouped FP4 MoE
      // shape -2.5%, others 0 to -0.5%, alternating A/B).  Otherwise the rows are
      // walked with running pointers, one read and store at a time.
      if (rows_w == T::TM && __ballot(vec == 2) == ~0ull) {
        constexpr int NR = T::TM / RPI;
        i32x4_t v[NR];
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          const int row = i * RPI + rr;
          v[i] = *(const i32x4_t*)(src + i * RPI * T::EPI_ROW + 16 * (seg ^ T::epi_swz(row)));
        }
#pragma unroll
        for (int i = 0; i < NR; ++i) __builtin_nontemporal_store(v[i], (i32x4_t*)(d + i * dstep));
        return;
      }
#pragma unroll 1
      for (int row0 = 0; row0 < rows_w; row0 += RPI) {
        const int row = row0 + rr;
        const i32x4_t v = *(const i32x4_t*)(src + 16 * (seg ^ T::epi_swz(row)));
        if (row < rows_w) {
          if (vec == 2) {
            __builtin_nontemporal_store(v, (i32x4_t*)d);
          } else if (vec == 1) {
            __builtin_nontemporal_store((i32x2_t){v[0], v[1]}, (i32x2_t*)d);
            __builtin_nontemporal_store((i32x2_t){v[2], v[3]}, (i32x2_t*)(d + 4));
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (n + e < n_end) d[e] = (uint16_t)(((uint32_t)v[e / 2] >> (16 * (e % 2))) & 0xFFFF);
          }
        }
        src += RPI * T::EPI_ROW;
        d += dstep;
      }
    };
    // The copying waves (ISS) run one variant of the tile body, the others another;
    // on an expert's last row tile the lower row of waves may hold no rows (MM false).
    // The copying waves are the upper row, which always holds rows of the tile.
    if constexpr (T::NWC == T::NW) {
      if constexpr (GROUPED && WM > 1 && T::NW > 4) {
        if (m0 + wm * T::TM < m_end)
          tile_body(std::true_type{}, std::true_type{});
        else
          tile_body(std::false_type{}, std::true_type{});
      } else {
        tile_body(std::true_type{}, std::true_type{});
      }
    } else if (wave < T::NWC) {
      tile_body(std::true_type{}, std::true_type{});
    } else if constexpr (GROUPED && WM > 1) {
      if (m0 + wm * T::TM < m_end)
        tile_body(std::true_type{}, std::false_type{});
      else
        tile_body(std::false_type{}, std::false_type{});
    } else {
      tile_body(std::true_type{}, std::false_type{});
    }
  }
}

}  // namespace bsg
