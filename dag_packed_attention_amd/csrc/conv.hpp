// Launchers of the short-convolution kernels (defined in conv.hip, called by abi.cpp).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.hpp"

namespace dagattn {

// Blocks of the backward launch: the rows of its dW partial buffer ([blocks][Ch][4] fp32).
int conv_bwd_blocks(int64_t pages);

// y = act(conv(x)) for every page's rows (HARTS Sec. 4.2); x, y bf16 [pages * 64][Ch].
void launch_conv_fwd(const uint16_t* x, const float* W, int Ch, int w, int act, const int32_t* page_nrows,
                     const int32_t* prev, int64_t pages, uint16_t* y, hipStream_t st);

// dx (TG = uint16_t bf16 bits or float) and dW [Ch][w]; part: conv_bwd_blocks(pages) * Ch * 4 floats.
template <typename TG>
void launch_conv_bwd(const uint16_t* x, const uint16_t* dy, const float* W, int Ch, int w, int act,
                     const int32_t* page_nrows, const int32_t* prev, const int64_t* ext_off, const ConvExt* ext,
                     int64_t pages, TG* dx, float* dW, float* part, hipStream_t st);

}  // namespace dagattn
