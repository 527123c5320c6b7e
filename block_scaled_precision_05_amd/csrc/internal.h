// internal.h -- host-side helpers shared between the library's translation units
// (not part of the C ABI).
#pragma once

#include <stdint.h>

namespace bsg {

// Argument checks of the M-grouped GEMMs without the launch (kind 0 BF16, 1 FP8,
// 2 FP4): BSG_OK or the status the entry point would return.
int grouped_check(int kind, const void* A, int64_t lda, const int16_t* sfa, int64_t ld_sfa,
                  const void* B, int64_t ldb, int64_t stride_b, const int16_t* sfb,
                  int64_t ld_sfb, int64_t stride_sfb, const void* D, int64_t ldd,
                  const int32_t* group_offsets, int32_t G, int64_t M_total, int64_t N, int64_t K);

// Argument checks of m_grouped_gemm_fp8 without the launch: BSG_OK or the status
// the entry point would return.
int grouped_fp8_check(const void* A, int64_t lda, const int16_t* sfa, int64_t ld_sfa,
                      const void* B, int64_t ldb, int64_t stride_b, const int16_t* sfb,
                      int64_t ld_sfb, int64_t stride_sfb, const void* D, int64_t ldd,
                      const int32_t* group_offsets, int32_t G, int64_t M_total, int64_t N,
                      int64_t K);

}  // namespace bsg
