// Device helpers shared by the kernels of libreplayssm.
#pragma once

#include "internal.hpp"

namespace rs {

// fp32 -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_bits_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return bf16_bits_rne(lo) | (bf16_bits_rne(hi) << 16);
}

// Two bf16 packed in a 32-bit word -> the two exact fp32 values.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 16-byte chunk of the bf16 layout -> the lane's float4 of two tiles.
__device__ __forceinline__ void unpack_lp_chunk(const uint4 x, f32x4& a, f32x4& b) {
  a = f32x4{bf16_lo(x.x), bf16_hi(x.x), bf16_lo(x.y), bf16_hi(x.y)};
  b = f32x4{bf16_lo(x.z), bf16_hi(x.z), bf16_lo(x.w), bf16_hi(x.w)};
}

__device__ __forceinline__ uint4 pack_lp_chunk(const f32x4& a, const f32x4& b) {
  return uint4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
               pack_bf16x2(b[2], b[3])};
}

__device__ __forceinline__ float dot4(const f32x4& a, const f32x4& b) {
  return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
}

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4(float* p, const f32x4& v) { *reinterpret_cast<f32x4*>(p) = v; }

// Sum over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the four 16-lane groups).
__device__ __forceinline__ float sum_groups(float x) {
  x += __shfl_xor(x, 16, kWave);
  x += __shfl_xor(x, 32, kWave);
  return x;
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
template <int WIDTH>
__device__ __forceinline__ float sum_width(float x) {
#pragma unroll
  for (int off = WIDTH / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

// Counts the workgroups of sequence b that have finished; returns true in the
// single thread of the last one, which may then update b's pointers: every
// other workgroup of b read them before arriving, so nothing reads them after.
// The caller must have synchronised its workgroup before calling. The counter
// is reset to zero for the next launch.
//
// No fence is needed, and none is issued: nothing is published through the
// counter. A workgroup's pointer reads have returned before its relaxed
// agent-scope atomic is issued (every address and branch of the workgroup
// depends on them), and the last workgroup writes the pointers only after its
// own atomic has returned, i.e. after every other arrival. The new pointer
// values become visible to the next kernel at the kernel boundary. (An
// agent-scope fence here would write back and invalidate the XCD's L2 once
// per workgroup, which costs more than the whole decode.)
__device__ __forceinline__ bool arrive_last(int32_t* arrive, int b, int expected) {
  const int prev = atomicAdd(arrive + b, 1);
  if (prev != expected - 1) return false;
  atomicExch(arrive + b, 0);
  return true;
}

}  // namespace rs
