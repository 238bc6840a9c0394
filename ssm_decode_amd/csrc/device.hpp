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

// Checkpoints are streamed: every byte is read once per call and never again
// before the next call, so their loads and stores are non-temporal (they do not
// displace the ring records, which the next kernel reads again, from the caches).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 ld4_stream(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ void st4_stream(float* p, const f32x4& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}

// A head's fp32 checkpoint (private tile layout) into the registers of one
// wavefront: tile (wave, nt) is the lane's float4 S[nt].
template <int NT>
__device__ __forceinline__ void load_hp(const float* head_base, int wave, int lane, f32x4 (&S)[NT]) {
  const float* src = head_base + (wave * NT) * 256 + lane * 4;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) S[nt] = ld4_stream(src + nt * 256);
}

template <int NT>
__device__ __forceinline__ void store_hp(float* head_base, int wave, int lane, const f32x4 (&S)[NT]) {
  float* dst = head_base + (wave * NT) * 256 + lane * 4;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) st4_stream(dst + nt * 256, S[nt]);
}

// The same from the bf16 copy (pairs of tiles per 16-byte chunk), widened exactly.
template <int NT>
__device__ __forceinline__ void load_lp(const uint16_t* head_base, int wave, int lane, f32x4 (&S)[NT]) {
  static_assert(NT % 2 == 0, "the bf16 layout pairs tiles");
  const u32x4* src = reinterpret_cast<const u32x4*>(head_base) + (wave * NT / 2) * 64 + lane;
#pragma unroll
  for (int m = 0; m < NT / 2; ++m) {
    const u32x4 w = __builtin_nontemporal_load(src + m * 64);
    unpack_lp_chunk(uint4{w[0], w[1], w[2], w[3]}, S[2 * m], S[2 * m + 1]);
  }
}

// The raw 16-byte chunks of the bf16 copy land in S[0 .. NT/2) as loaded;
// widen_lp turns them into the lane's fp32 tiles in place. Keeping the loaded
// bits untouched until the values are needed lets the load stay in flight.
template <int NT>
__device__ __forceinline__ void widen_lp(f32x4 (&S)[NT]) {
  static_assert(NT % 2 == 0, "the bf16 layout pairs tiles");
  // highest chunk first: chunk m fills tiles 2m and 2m + 1, which hold no chunk still to be read
#pragma unroll
  for (int m = NT / 2 - 1; m >= 0; --m) {
    const u32x4 w = __builtin_bit_cast(u32x4, S[m]);
    unpack_lp_chunk(uint4{w[0], w[1], w[2], w[3]}, S[2 * m], S[2 * m + 1]);
  }
}

// fp32 registers -> bf16 copy (round to nearest even); returns the rounded values in S when asked.
template <int NT>
__device__ __forceinline__ void store_lp(uint16_t* head_base, int wave, int lane, f32x4 (&S)[NT],
                                         bool keep_rounded) {
  static_assert(NT % 2 == 0, "the bf16 layout pairs tiles");
  u32x4* dst = reinterpret_cast<u32x4*>(head_base) + (wave * NT / 2) * 64 + lane;
#pragma unroll
  for (int m = 0; m < NT / 2; ++m) {
    const uint4 x = pack_lp_chunk(S[2 * m], S[2 * m + 1]);
    __builtin_nontemporal_store(u32x4{x.x, x.y, x.z, x.w}, dst + m * 64);
    if (keep_rounded) unpack_lp_chunk(x, S[2 * m], S[2 * m + 1]);
  }
}

__device__ __forceinline__ float dot4(const f32x4& a, const f32x4& b) {
  return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
}

// acc + a . b as a chain of four fused multiply-adds (one instruction per
// product: no separate add of a dot4 result)
__device__ __forceinline__ float fma4(const f32x4& a, const f32x4& b, float acc) {
  acc = __builtin_fmaf(a[0], b[0], acc);
  acc = __builtin_fmaf(a[1], b[1], acc);
  acc = __builtin_fmaf(a[2], b[2], acc);
  return __builtin_fmaf(a[3], b[3], acc);
}

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4(float* p, const f32x4& v) { *reinterpret_cast<f32x4*>(p) = v; }

// Cross-lane sums without the LDS crossbar. Every step adds a lane's value to
// its partner's, and both partners form the same sum (a + b and b + a are the
// same float), so every lane of a group ends with bit-identical totals.
//  - within a 16-lane row: DPP moves (quad_perm for partners 1 and 2 apart,
//    row_half_mirror and row_mirror once the value is uniform over 4 and 8 lanes);
//  - across rows: gfx950's v_permlane16_swap (row 0 <-> 1, 2 <-> 3) and
//    v_permlane32_swap (lanes l <-> l + 32); with both operands the same value
//    the two results are a lane's own value and its partner's.
namespace dpp {
constexpr int kQuadXor1 = 0xB1;     // quad_perm [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2, 3, 0, 1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;
}  // namespace dpp

template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float swap_add16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float swap_add32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// DPP move whose lanes without a source lane (past the row end) get `fill`.
template <int CTRL>
__device__ __forceinline__ float dpp_move_fill(float x, float fill) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Product of x over lanes l .. 63, in every lane l. Within a 16-lane row a
// doubling scan on row_shl (lane l reads lane l + d of its row; past the row
// end it reads 1); then each row takes the totals of the rows after it, which
// sit in their first lanes.
__device__ __forceinline__ float suffix_product64(float x, int lane) {
  x *= dpp_move_fill<0x101>(x, 1.f);  // row_shl:1
  x *= dpp_move_fill<0x102>(x, 1.f);  // row_shl:2
  x *= dpp_move_fill<0x104>(x, 1.f);  // row_shl:4
  x *= dpp_move_fill<0x108>(x, 1.f);  // row_shl:8
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  const int row = lane >> 4;
  const float tail = row == 0 ? r1 * (r2 * r3) : row == 1 ? r2 * r3 : row == 2 ? r3 : 1.f;
  return x * tail;
}

// Sum over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the four 16-lane groups).
__device__ __forceinline__ float sum_groups(float x) { return swap_add32(swap_add16(x)); }

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
template <int WIDTH>
__device__ __forceinline__ float sum_width(float x) {
  static_assert(WIDTH >= 1 && WIDTH <= 64 && (WIDTH & (WIDTH - 1)) == 0, "power of two up to 64");
  if constexpr (WIDTH >= 2) x += dpp_move<dpp::kQuadXor1>(x);
  if constexpr (WIDTH >= 4) x += dpp_move<dpp::kQuadXor2>(x);
  if constexpr (WIDTH >= 8) x += dpp_move<dpp::kRowHalfMirror>(x);
  if constexpr (WIDTH >= 16) x += dpp_move<dpp::kRowMirror>(x);
  if constexpr (WIDTH >= 32) x = swap_add16(x);
  if constexpr (WIDTH >= 64) x = swap_add32(x);
  return x;
}

// Arrival counting for the pointer update ("last arriver"). Counts the
// workgroups that have read the pointers guarded by counter b; returns true in
// the single thread of the last one, which may then update them: every other
// workgroup read them before arriving, so nothing reads them after.
// The caller must have synchronised its workgroup after its pointer reads. The
// counter is reset to zero for the next launch.
//
// No fence is needed, and none is issued: nothing is published through the
// counter. A workgroup's pointer reads have returned before its relaxed
// agent-scope atomic is issued (every address and branch of the workgroup
// depends on them), and the last workgroup writes the pointers only after its
// own atomic has returned, i.e. after every other arrival. The new pointer
// values become visible to the next kernel at the kernel boundary. (An
// agent-scope fence here would write back and invalidate the XCD's L2 once
// per workgroup, which costs more than the whole decode.) The replay kernel
// uses it once per workgroup, after the workgroup's last item.
__device__ __forceinline__ bool arrive_last(int32_t* arrive, int b, int expected) {
  const int prev = atomicAdd(arrive + b, 1);
  if (prev != expected - 1) return false;
  atomicExch(arrive + b, 0);
  return true;
}

}  // namespace rs
