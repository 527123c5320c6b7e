// configs.h -- tile configurations of the GEMM kernels (template arguments of
// gemm_kernel: BM, BN, WM, WN, SB, NS, PR).
#pragma once

// Dense FP8 / FP4: 256x256 workgroup tile, 2x2 waves of 128x128 (16 fragments of 32x32 per
// wave, 256 fp32 accumulators per lane), a ring of five 64-byte stages (32 KiB
// each) copied in pairs.  The copies are limited by the requests a CU keeps in
// flight and by the issue cost of the copy instructions (spread over the MFMAs);
// the MFMAs by the chip's power limit.  256x224 tiles (exactly two per CU at
// 4096x7168) measured no faster: with the chip power-bound, the CUs left idle in
// the last wave of 256x256 tiles let the others clock higher.
#define BSG_FP8_CFG 256, 256, 2, 2, 64, 5, 1
#define BSG_FP4_CFG 256, 256, 2, 2, 64, 5, 1
// BF16: the same tile over eight waves (2x4 of 128x64, two per SIMD): while one
// wave of a SIMD waits on a copy or an LDS read, the other issues MFMAs.  Its
// fragments fit the halved register budget (213 registers, no spills); FP8's do
// not (they spill), and FP4's row permutation needs 128x128 wave blocks.  On
// 4096x7168x16384 8 waves ran 717-719 us against 734-741 us, on the grouped MoE
// shape 3430 us against 3471 us.
#define BSG_BF16_CFG 256, 256, 2, 4, 64, 5, 1
// Grouped: the dense tile.  128x512 tiles (1x4 waves) waste no rows on
// 128-aligned experts, but move 25% more bytes from L2 to LDS per flop; on the
// MoE workload (256 experts, N=2048, K=7168) 256x256 measured 1914 us against
// 2100 us, although a quarter of its row tiles are half empty.
#define BSG_GROUPED_CFG 256, 256, 2, 2, 64, 5, 1
// Grouped BF16 and FP4: the dense tiles of their kind.
#define BSG_GROUPED_BF16_CFG 256, 256, 2, 4, 64, 5, 1
#define BSG_GROUPED_FP4_CFG 256, 256, 2, 2, 64, 5, 1
// Masked (decode-sized experts, tens of rows each): 128-row tiles, 1x4 waves of
// 128x128 over 512 columns, four 40 KiB stages; 256-row tiles would multiply
// mostly empty rows (measured 419 us against 340 us on the decode case).
#define BSG_MASKED_CFG 128, 512, 1, 4, 64, 4, 1
