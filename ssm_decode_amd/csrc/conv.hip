// The short causal convolution on the input side of a Mamba-2 layer, kept the
// ReplaySSM way: its state is nothing but its last W - 1 inputs, so those stay
// in a ring per sequence, drafts are appended after them as pending inputs,
// every draft's output is computed from the window that ends at it, and
// accepting a prefix only moves the ring's start ("ReplaySSM: Cache SSM Inputs,
// Not State", How it works: cache the inputs, and Speculative decoding:
// acceptance advances a pointer, rejected entries are overwritten later).
//
// Per channel c and token t:
//     y_t[c] = act(bias[c] + sum_{j<W} w[c][j] x_{t-W+1+j}[c]),  x_s = 0 for s < 0,
// act = SiLU (z / (1 + e^-z)) or the identity.
#include "conv.hpp"
#include "device.hpp"

namespace rs {

__global__ void __launch_bounds__(256) conv_init_kernel(const ConvArgs a, int64_t n4) {
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
    st4(a.ring + 4 * i, f32x4{0.f, 0.f, 0.f, 0.f});
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b < a.B) {
    a.start[b] = 0;
    a.pend[b] = 0;
    a.arrive[b] = 0;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) a.err[0] = 0;
}

// Grid (channel groups, sequence groups): a thread owns four channels of kConvSeqs
// sequences, so each workgroup reads its channels' weights once for all of them.
// The window and the drafts sit in registers (indices fixed by unrolling over W
// and TMAX); the drafts' inputs are written to their ring slots; for each
// sequence the last workgroup to finish publishes pend = T (or commits).
constexpr int kConvSeqs = 8;

template <int W, int TMAX>
__global__ void __launch_bounds__(256) conv_step_kernel(const ConvArgs a) {
  const int D = a.D, T = a.T;
  const int Cc = W - 1 + a.T_max;
  const int c4 = blockIdx.x * 256 + threadIdx.x;
  const bool lane_ok = 4 * c4 < D;
  float wc[4][W];
  f32x4 bias = f32x4{0.f, 0.f, 0.f, 0.f};
  if (lane_ok) {
    if constexpr (W == 4) {
      // a channel's four taps are one 16-byte row of w
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f32x4 t = ld4(a.w + (int64_t)(4 * c4 + e) * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) wc[e][j] = t[j];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int j = 0; j < W; ++j) wc[e][j] = a.w[(int64_t)(4 * c4 + e) * W + j];
    }
    if (a.bias) bias = ld4(a.bias + 4 * c4);
  }
  for (int sb = 0; sb < kConvSeqs; ++sb) {
    const int b = blockIdx.y * kConvSeqs + sb;
    if (b >= a.B) break;  // (uniform over the workgroup)
    const int start = a.start[b], pend = a.pend[b];
    const bool corrupt = start < 0 || start >= Cc || pend < 0;
    const bool bad = corrupt || pend != 0;
    if (!bad && lane_ok) {
      const int64_t row = (int64_t)b * Cc;
      f32x4 seq[W - 1 + TMAX];
#pragma unroll
      for (int j = 0; j < W - 1; ++j) {
        int slot = start + j;
        if (slot >= Cc) slot -= Cc;
        seq[j] = ld4(a.ring + (row + slot) * D + 4 * c4);
      }
#pragma unroll
      for (int i = 0; i < TMAX; ++i) {
        seq[W - 1 + i] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (i < T) {
          const f32x4 x = ld4_stream(a.x + ((int64_t)b * T + i) * D + 4 * c4);
          seq[W - 1 + i] = x;
          int slot = start + W - 1 + i;
          while (slot >= Cc) slot -= Cc;
          st4(a.ring + (row + slot) * D + 4 * c4, x);
        }
      }
#pragma unroll
      for (int i = 0; i < TMAX; ++i) {
        if (i < T) {
          f32x4 acc = bias;
#pragma unroll
          for (int j = 0; j < W; ++j) {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(wc[e][j], seq[i + j][e], acc[e]);
          }
          if (a.silu) {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = acc[e] / (1.f + expf(-acc[e]));
          }
          st4_stream(a.y + ((int64_t)b * T + i) * D + 4 * c4, acc);
        }
      }
    }
    __syncthreads();
    if (threadIdx.x == 0 && arrive_last(a.arrive, b, gridDim.x)) {
      if (bad) {
        atomicOr(a.err, corrupt ? REPLAYSSM_DEVERR_CORRUPT : REPLAYSSM_DEVERR_PENDING);
      } else if (a.commit) {
        int s = start + T;  // standard decoding: the token joins the window at once
        if (s >= Cc) s -= Cc;
        a.start[b] = s;
      } else {
        a.pend[b] = T;
      }
    }
  }
}

// Accept: the first a drafts join the window, which therefore starts a slots
// later; the rest are overwritten by the next step. a outside 0..pend is
// clamped and flagged.
__global__ void __launch_bounds__(256) conv_accept_kernel(const ConvArgs a, const int32_t* acc) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= a.B) return;
  const int Cc = a.W - 1 + a.T_max;
  const int start = a.start[b], pend = a.pend[b];
  if (start < 0 || start >= Cc || pend < 0 || pend > a.T_max) {
    atomicOr(a.err, REPLAYSSM_DEVERR_CORRUPT);
    return;
  }
  int n = acc[b];
  if (n < 0 || n > pend) {
    atomicOr(a.err, REPLAYSSM_DEVERR_ACCEPT);
    n = n < 0 ? 0 : pend;
  }
  int s = start + n;
  if (s >= Cc) s -= Cc;
  a.start[b] = s;
  a.pend[b] = 0;
}

hipError_t launch_conv_init(const ConvArgs& a, hipStream_t s) {
  const int64_t n4 = (int64_t)a.B * (a.W - 1 + a.T_max) * a.D / 4;
  int64_t blocks = (n4 + 255) / 256;
  const int64_t need = (a.B + 255) / 256;
  if (blocks < need) blocks = need;
  if (blocks > 65536) blocks = 65536 > need ? 65536 : need;
  hipLaunchKernelGGL(conv_init_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a, n4);
  return hipGetLastError();
}

template <int W>
static hipError_t launch_w(const ConvArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.D / 4 + 255) / 256), (unsigned)((a.B + kConvSeqs - 1) / kConvSeqs));
  if (a.T <= 1)
    hipLaunchKernelGGL((conv_step_kernel<W, 1>), grid, dim3(256), 0, s, a);
  else if (a.T <= 4)
    hipLaunchKernelGGL((conv_step_kernel<W, 4>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((conv_step_kernel<W, 8>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_conv_step(const ConvArgs& a, hipStream_t s) {
  switch (a.W) {
    case 1: return launch_w<1>(a, s);
    case 2: return launch_w<2>(a, s);
    case 3: return launch_w<3>(a, s);
    case 4: return launch_w<4>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_conv_accept(const ConvArgs& a, const int32_t* accepted, hipStream_t s) {
  hipLaunchKernelGGL(conv_accept_kernel, dim3((unsigned)((a.B + 255) / 256)), dim3(256), 0, s, a, accepted);
  return hipGetLastError();
}

}  // namespace rs
