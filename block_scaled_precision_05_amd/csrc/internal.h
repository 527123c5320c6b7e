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

// The FFN core's up-projection with the SwiGLU epilogue (Y codes and packed 1x128
// scales instead of H); arguments already checked.
int grouped_fp8_swiglu(const void* A, int64_t lda, const int16_t* sfa, int64_t ld_sfa, const void* W13,
                       int64_t ldw, int64_t stride_w, const int16_t* sfw, int64_t ld_sfw,
                       int64_t stride_sfw, const int32_t* group_offsets, int32_t G, int64_t M_total,
                       int64_t hidden, int64_t inter, void* Y, int64_t ldy, int16_t* sfy, int64_t ld_sfy,
                       int32_t rule, void* stream);

}  // namespace bsg
