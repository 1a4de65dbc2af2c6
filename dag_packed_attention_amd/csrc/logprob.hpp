// Launchers of the log-probability kernels (defined in logprob.hip, called by abi.cpp).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace dagattn {

// lse[c] and lambda[s] for every row with at least one position (HARTS Sec. 3.5 Eq. 17).
// T: uint16_t (bf16 bits) or float.
template <typename T>
void launch_lp_fwd(const T* z, int64_t C, int V, const int32_t* row_first, const int32_t* row_pos,
                   const int32_t* pos_target, int64_t n_pos, float* lse, float* lam, hipStream_t st);

// dz for every row (HARTS Sec. 3.5 Eq. 19-20); TG: uint16_t (bf16 bits) or float.
template <typename T, typename TG>
void launch_lp_bwd(const T* z, const float* lse, int64_t C, int V, const int32_t* row_first, const int32_t* row_pos,
                   const int32_t* pos_target, const float* g, int64_t n_pos, TG* dz, hipStream_t st);

}  // namespace dagattn
