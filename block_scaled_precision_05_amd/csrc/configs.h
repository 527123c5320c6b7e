// configs.h -- tile configurations of the GEMM kernels (template arguments of
// gemm_kernel: BM, BN, WM, WN, SB, NS, PR).
#pragma once

// Dense: 256x256 workgroup tile over eight waves, 2x4 of 128x64 (8 fragments of
// 32x32 per wave, 128 fp32 accumulators per lane), two waves per SIMD: while one
// wave of a SIMD waits on a copy or an LDS read, the other issues MFMAs.  A ring
// of five 64-byte stages (32 KiB each) copied in pairs.  The fragments fit the
// halved register budget (FP8 and FP4 with their A fragments single-buffered; FP4
// permutes B rows in 64-row blocks).  Alternating A/B, 8 against 4 waves of
// 128x128: BF16 4096x7168x16384 717-719 against 734-741 us, FP8 385 against
// 403 us, FP4 219-222 against 222-226 us; grouped BF16 MoE shape 3430 against
// 3471 us, grouped FP8 1932 against 1957 us, FFN down-projection 919 against
// 1007 us.  The copies are limited by the requests a CU keeps in flight and by
// the issue cost of the copy instructions (spread over the MFMAs); the MFMAs by
// the chip's power limit.  256x224 tiles (exactly two per CU at 4096x7168)
// measured no faster: with the chip power-bound, the CUs left idle in the last
// wave of 256x256 tiles let the others clock higher.
#define BSG_FP4_CFG 256, 256, 2, 4, 64, 5, 1
#define BSG_BF16_CFG 256, 256, 2, 4, 64, 5, 1
#define BSG_FP8_CFG 256, 256, 2, 4, 64, 5, 1
// Grouped: the dense FP8 tile and waves.  128x512 tiles (1x4 waves) waste no rows on
// 128-aligned experts, but move 25% more bytes from L2 to LDS per flop; on the
// MoE workload (256 experts, N=2048, K=7168) 256x256 measured 1914 us against
// 2100 us, although a quarter of its row tiles are half empty.
#define BSG_GROUPED_CFG 256, 256, 2, 4, 64, 5, 1
// Grouped BF16 and FP4: the dense tiles of their kind.
#define BSG_GROUPED_BF16_CFG 256, 256, 2, 4, 64, 5, 1
#define BSG_GROUPED_FP4_CFG 256, 256, 2, 4, 64, 5, 1
// Masked (decode-sized experts, tens of rows each): a stream of expert weights,
// bound by HBM.  128-row tiles, 1x4 waves of 128x64 over 256 columns, a ring of six
// 24 KiB stages (120 KiB of copies in flight per CU); on the decode case (48 experts,
// N=4096, K=7168) 309 us against 318 us for 128x512 tiles with four 40 KiB stages
// (the same bytes in flight, but 1.5 waves of workgroup tiles on 256 CUs), and 378 us
// for 128x256 with four stages (72 KiB in flight).  256-row tiles would multiply
// mostly empty rows (419 against 340 us).
#define BSG_MASKED_CFG 128, 256, 1, 4, 64, 6, 1
