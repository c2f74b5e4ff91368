// nvfp4_fused.h -- fused single-launch per-token cast for large aligned shapes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

bool fused_per_token_supported(int64_t M, int64_t K, bool row, bool col);
hipError_t fused_per_token(const uint16_t* x, int64_t M, int64_t K,
                           uint8_t* row_q, uint8_t* row_sf, float* row_amax,
                           uint8_t* col_q, uint8_t* col_sf, float* col_amax, hipStream_t st);

}  // namespace nvfp4
