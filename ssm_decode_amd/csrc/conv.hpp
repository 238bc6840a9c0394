// Internal declarations of the convolution input ring (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rs {

constexpr int kConvMaxW = 4;  // widths 1..4 have kernels

struct ConvArgs {
  float* ring;        // [B][Cc][D], Cc = W - 1 + T_max
  int32_t* start;     // [B] slot of the oldest input of the committed window
  int32_t* pend;      // [B] pending drafts
  int32_t* arrive;    // [B] arrival counters of the step kernel's channel blocks
  int32_t* err;
  const float* x;     // [B][T][D]
  const float* w;     // [D][W]
  const float* bias;  // [D] or NULL
  float* y;           // [B][T][D]
  int B, D, W, T, T_max, silu;
  int commit;  // step: commit the T inputs at once (start += T) instead of leaving them pending
};

hipError_t launch_conv_init(const ConvArgs& a, hipStream_t s);
hipError_t launch_conv_step(const ConvArgs& a, hipStream_t s);
hipError_t launch_conv_accept(const ConvArgs& a, const int32_t* accepted, hipStream_t s);

}  // namespace rs
