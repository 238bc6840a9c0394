// Host-side driver of the C ABI for sanitizer builds: the library's host code
// (api.cpp) is linked against stand-ins for its kernel launchers that only
// count calls, so every entry point runs its complete validation and argument
// packing with valid and invalid arguments, and no device memory is touched
// (the pointers are aligned addresses that nothing dereferences).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "conv.hpp"
#include "internal.hpp"
#include "replayssm.h"

namespace rs {
static int g_launches = 0;
static hipError_t count() {
  ++g_launches;
  return hipSuccess;
}
hipError_t persistent_grid(const void*, int, size_t, int, int* grid) { *grid = 1; return count(); }
hipError_t launch_replay(int, int, int, const ReplayArgs&, hipStream_t) { return count(); }
hipError_t launch_append(int, const AppendArgs&, hipStream_t) { return count(); }
hipError_t device_max_lds(int* bytes) { *bytes = kArchMaxLdsBytes; return hipSuccess; }
hipError_t launch_append_static(int, const AppendArgs& a, hipStream_t) { return a.arrive ? hipErrorInvalidValue : count(); }
hipError_t launch_accept(int32_t*, int32_t*, int32_t*, const int32_t*, int, int, hipStream_t) { return count(); }
hipError_t launch_init(int32_t*, int32_t*, int32_t*, int64_t*, int32_t*, int32_t*, int, hipStream_t) { return count(); }
hipError_t launch_pack(const float*, float*, uint16_t*, int64_t, int, int, hipStream_t) { return count(); }
hipError_t launch_unpack(const float*, const uint16_t*, float*, int64_t, int, int, hipStream_t) { return count(); }
hipError_t launch_snapshot(const float*, const uint16_t*, const int32_t*, int32_t*, const int32_t*, int, float*, int,
                           int, int, int, hipStream_t) { return count(); }
hipError_t launch_restore(float*, uint16_t*, int32_t*, int32_t*, int32_t*, int64_t*, int32_t*, const int32_t*, int,
                          const float*, int, int, int, int, hipStream_t) { return count(); }
hipError_t launch_eager(int, int, const EagerArgs&, hipStream_t) { return count(); }
hipError_t launch_eager_accept(int32_t*, const int32_t*, int, int, hipStream_t) { return count(); }
hipError_t launch_probe_read(const void*, int64_t, float*, hipStream_t) { return count(); }
static int tiling = REPLAYSSM_TILES_AUTO;
void set_tiling(int policy) { tiling = policy; }
int get_tiling() { return tiling; }
hipError_t device_cus(int* cus) { *cus = 256; return count(); }
hipError_t launch_conv_init(const ConvArgs&, hipStream_t) { return count(); }
hipError_t launch_conv_step(const ConvArgs&, hipStream_t) { return count(); }
hipError_t launch_conv_accept(const ConvArgs&, const int32_t*, hipStream_t) { return count(); }
}  // namespace rs

static int g_fail = 0;
#define EXPECT(expr, want)                                                                       \
  do {                                                                                           \
    const int got_ = (expr);                                                                     \
    if (got_ != (want)) {                                                                        \
      std::printf("line %d: %s returned %d, expected %d (%s)\n", __LINE__, #expr, got_, (want),  \
                  replayssm_last_error());                                                       \
      ++g_fail;                                                                                  \
    }                                                                                            \
  } while (0)

static float* F(uintptr_t i) { return reinterpret_cast<float*>((i + 1) << 20); }
static int32_t* I(uintptr_t i) { return reinterpret_cast<int32_t*>((i + 1) << 20); }

static replayssm_state state_for(const replayssm_config& c) {
  replayssm_sizes sz{};
  replayssm_get_sizes(&c, &sz);
  replayssm_state s{};
  s.hp = sz.hp_bytes ? F(1) : nullptr;
  s.lp = sz.lp_bytes ? reinterpret_cast<uint16_t*>(F(2)) : nullptr;
  s.ring_alpha = F(3);
  s.ring_beta = sz.ring_beta_bytes ? F(4) : nullptr;
  s.ring_k = F(5);
  s.ring_v = F(6);
  s.head = I(7);
  s.h = I(8);
  s.p = I(9);
  s.folded = reinterpret_cast<int64_t*>(F(10));
  s.arrive = I(11);
  s.err = I(12);
  s.ring_vraw = sz.ring_vraw_bytes ? F(13) : nullptr;
  return s;
}

static void every_call(const replayssm_config& c) {
  const replayssm_state s = state_for(c);
  const float* beta = c.kind == REPLAYSSM_MAMBA2 ? nullptr : F(20);
  EXPECT(replayssm_init(&c, &s, nullptr), REPLAYSSM_OK);
  for (int T = 1; T <= c.T_max; ++T) {
    EXPECT(replayssm_append(&c, &s, T, F(21), F(22), F(23), beta, nullptr), REPLAYSSM_OK);
    EXPECT(replayssm_verify(&c, &s, T, F(24), F(25), nullptr), REPLAYSSM_OK);
    EXPECT(replayssm_verify_step(&c, &s, T, F(21), F(22), F(23), beta, F(24), F(25), nullptr), REPLAYSSM_OK);
    if (c.precision == REPLAYSSM_FP32)
      EXPECT(replayssm_eager_verify(&c, F(26), I(27), T, F(21), F(22), F(23), beta, F(24), F(25), nullptr),
             REPLAYSSM_OK);
  }
  EXPECT(replayssm_append(&c, &s, c.T_max + 1, F(21), F(22), F(23), beta, nullptr), REPLAYSSM_EINVAL);
  {
    // the variant without the caller's scratch: arrive may be NULL, B is capped
    replayssm_state s0 = s;
    s0.arrive = nullptr;
    EXPECT(replayssm_append_static(&c, &s0, 1, F(21), F(22), F(23), beta, nullptr),
           c.B <= REPLAYSSM_STATIC_SCRATCH_SEQS ? REPLAYSSM_OK : REPLAYSSM_EINVAL);
    EXPECT(replayssm_append_static(&c, &s0, c.T_max + 1, F(21), F(22), F(23), beta, nullptr), REPLAYSSM_EINVAL);
    EXPECT(replayssm_append(&c, &s0, 1, F(21), F(22), F(23), beta, nullptr), REPLAYSSM_EINVAL);
  }
  EXPECT(replayssm_append_dt(&c, &s, 1, F(28), F(29), nullptr, F(22), F(23), beta, nullptr),
         c.kind == REPLAYSSM_KDA ? REPLAYSSM_ENOTSUP : REPLAYSSM_OK);
  EXPECT(replayssm_decode(&c, &s, F(24), F(25), nullptr), REPLAYSSM_OK);
  EXPECT(replayssm_decode(&c, &s, F(24) + 1, F(25), nullptr), REPLAYSSM_EINVAL);
  EXPECT(replayssm_decode_step(&c, &s, F(21), F(22), F(23), beta, F(24), F(25), nullptr), REPLAYSSM_OK);
  EXPECT(replayssm_accept(&c, &s, I(30), nullptr), REPLAYSSM_OK);
  EXPECT(replayssm_flush(&c, &s, nullptr), REPLAYSSM_OK);
  EXPECT(replayssm_flush_selected(&c, &s, I(31), nullptr), REPLAYSSM_OK);
  EXPECT(replayssm_snapshot(&c, &s, 2, I(32), F(33), nullptr), REPLAYSSM_OK);
  EXPECT(replayssm_restore(&c, &s, 2, I(32), F(33), nullptr), REPLAYSSM_OK);
  EXPECT(replayssm_pack_state(&c, F(34), s.hp, s.lp, nullptr), REPLAYSSM_OK);
  EXPECT(replayssm_unpack_state(&c, s.hp, s.hp ? nullptr : s.lp, F(35), nullptr), REPLAYSSM_OK);
  if (c.precision == REPLAYSSM_FP32) {
    EXPECT(replayssm_eager_step(&c, F(26), F(21), F(22), F(23), beta, F(24), F(25), nullptr), REPLAYSSM_OK);
    EXPECT(replayssm_eager_accept(&c, I(27), I(30), c.T_max, nullptr), REPLAYSSM_OK);
  }
  replayssm_state bad = s;
  bad.ring_k = nullptr;
  EXPECT(replayssm_decode(&c, &bad, F(24), F(25), nullptr), REPLAYSSM_EINVAL);
}

int main() {
  replayssm_sizes sz{};
  // configurations at and beyond every limit
  const int kinds[3] = {REPLAYSSM_MAMBA2, REPLAYSSM_GDN, REPLAYSSM_KDA};
  const int dims[][2] = {{16, 16}, {64, 128}, {256, 128}, {48, 64}, {256, 32}};
  for (int kind : kinds)
    for (int prec = 0; prec < 3; ++prec)
      for (const auto& d : dims)
        for (int L : {1, 4, 16, 64})
          for (int T : {1, 4, 8}) {
            const replayssm_config c{kind, prec, 3, 5, d[0], d[1], L, T};
            if (replayssm_get_sizes(&c, &sz) == REPLAYSSM_OK) every_call(c);
          }
  // the static-scratch append at and just past its sequence limit
  for (int B : {REPLAYSSM_STATIC_SCRATCH_SEQS, REPLAYSSM_STATIC_SCRATCH_SEQS + 1}) {
    const replayssm_config c{REPLAYSSM_MAMBA2, REPLAYSSM_FP32, B, 2, 64, 128, 16, 4};
    every_call(c);
  }
  const replayssm_config huge{REPLAYSSM_MAMBA2, REPLAYSSM_FP32, 65535, 16385, 64, 128, 16, 1};
  EXPECT(replayssm_get_sizes(&huge, &sz), REPLAYSSM_EINVAL);
  const replayssm_config wide{REPLAYSSM_MAMBA2, REPLAYSSM_FP32, 1, 1 << 21, 64, 128, 16, 1};
  EXPECT(replayssm_get_sizes(&wide, &sz), REPLAYSSM_EINVAL);
  const replayssm_config big{REPLAYSSM_GDN, REPLAYSSM_FP32, 65535, 16384, 256, 128, 16, 8};
  EXPECT(replayssm_get_sizes(&big, &sz), REPLAYSSM_OK);
  EXPECT(replayssm_get_sizes(nullptr, &sz), REPLAYSSM_EINVAL);
  EXPECT(replayssm_probe_read(F(40), 1 << 20, F(41), nullptr), REPLAYSSM_OK);
  EXPECT(replayssm_probe_read(F(40), 1000, F(41), nullptr), REPLAYSSM_EINVAL);
  EXPECT(replayssm_set_tiling(REPLAYSSM_TILES_TWO), REPLAYSSM_OK);
  EXPECT(replayssm_get_tiling(), REPLAYSSM_TILES_TWO);
  EXPECT(replayssm_set_tiling(3), REPLAYSSM_EINVAL);
  EXPECT(replayssm_set_tiling(-1), REPLAYSSM_EINVAL);
  EXPECT(replayssm_get_tiling(), REPLAYSSM_TILES_TWO);
  EXPECT(replayssm_set_tiling(REPLAYSSM_TILES_AUTO), REPLAYSSM_OK);

  // the convolution ring
  for (int W = 0; W <= 5; ++W)
    for (int T = 1; T <= 8; ++T) {
      const replayssm_conv_config cc{4, 40960, W, T};
      int64_t ring = 0, ptr = 0;
      const int st = replayssm_conv_sizes(&cc, &ring, &ptr);
      EXPECT(st, (W >= 1 && W <= 4) ? REPLAYSSM_OK : REPLAYSSM_EINVAL);
      if (st != REPLAYSSM_OK) continue;
      const replayssm_conv_state cs{F(50), I(51), I(52), I(53), I(54)};
      EXPECT(replayssm_conv_init(&cc, &cs, nullptr), REPLAYSSM_OK);
      EXPECT(replayssm_conv_step(&cc, &cs, T, F(55), F(56), F(57), 1, 0, F(58), nullptr), REPLAYSSM_OK);
      EXPECT(replayssm_conv_step(&cc, &cs, T + 1, F(55), F(56), nullptr, 1, 0, F(58), nullptr), REPLAYSSM_EINVAL);
      EXPECT(replayssm_conv_step(&cc, &cs, T, F(55), F(56), nullptr, 0, 1, F(58), nullptr), REPLAYSSM_OK);
      EXPECT(replayssm_conv_accept(&cc, &cs, I(59), nullptr), REPLAYSSM_OK);
    }
  const replayssm_conv_config odd{4, 6, 4, 1};
  EXPECT(replayssm_conv_sizes(&odd, nullptr, nullptr), REPLAYSSM_EINVAL);
  const replayssm_conv_config vast{65535, 256 * 65535 * 4, 4, 8};
  int64_t ring = 0;
  EXPECT(replayssm_conv_sizes(&vast, &ring, nullptr), REPLAYSSM_OK);
  for (int code : {0, -1, -2, -3, -99}) std::printf("%s;", replayssm_status_string(code));
  std::printf("\nlaunches=%d failures=%d\n", rs::g_launches, g_fail);
  return g_fail == 0 && rs::g_launches > 1000 ? 0 : 1;
}
