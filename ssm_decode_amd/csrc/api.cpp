// C ABI of libreplayssm: host-side validation, sizing and kernel dispatch.
// Every entry point validates its arguments completely before it enqueues
// anything, never allocates, and never synchronises (replayssm_read_error
// excepted, which exists for tests and debugging).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "conv.hpp"
#include "internal.hpp"
#include "replayssm.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_result(hipError_t e, const char* what) {
  if (e == hipSuccess) return REPLAYSSM_OK;
  return fail(REPLAYSSM_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool exact_u(const replayssm_config* c);

// Launches the replay kernel after checking its LDS carve against what the current device
// gives one workgroup (ENOTSUP beyond it).
int replay(const replayssm_config* cfg, int tmax, const rs::ReplayArgs& a, hipStream_t s, const char* what) {
  // (the launcher may pick padded rows where they fit more workgroups; the unpadded carve is the least LDS)
  const rs::ReplayLds lds(cfg->L + cfg->T_max, cfg->dk, cfg->dv, tmax, exact_u(cfg) ? rs::kKindGdnExact : cfg->kind,
                          true);
  int max_lds = 0;
  if (int r = hip_result(rs::device_max_lds(&max_lds), what)) return r;
  if (lds.total * 4 > max_lds)
    return fail(REPLAYSSM_ENOTSUP, "%s: L + T_max and dims need %d bytes of LDS; the device gives a workgroup %d",
                what, lds.total * 4, max_lds);
  return hip_result(rs::launch_replay(cfg->kind, cfg->dk, tmax, a, s), what);
}

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Pointer must be non-NULL and 16-byte aligned.
#define NEED(ptr)                                                                   \
  do {                                                                              \
    if ((ptr) == nullptr) return fail(REPLAYSSM_EINVAL, "%s is NULL", #ptr);        \
    if (!aligned(ptr)) return fail(REPLAYSSM_EINVAL, "%s is not 16-byte aligned", #ptr); \
  } while (0)

int tmax_bucket(int T) { return T <= 1 ? 1 : (T <= 4 ? 4 : 8); }

// GDN with the two-precision checkpoint keeps the raw v of every record: its folds
// recompute the folded records' corrections from the fp32 checkpoint.
bool exact_u(const replayssm_config* c) {
  return c->kind == REPLAYSSM_GDN && c->precision == REPLAYSSM_FP32_HP_BF16_LP;
}

int check_config(const replayssm_config* c) {
  if (c == nullptr) return fail(REPLAYSSM_EINVAL, "cfg is NULL");
  if (c->kind != REPLAYSSM_MAMBA2 && c->kind != REPLAYSSM_GDN && c->kind != REPLAYSSM_KDA)
    return fail(REPLAYSSM_EINVAL, "kind %d unknown", c->kind);
  if (c->precision < REPLAYSSM_FP32 || c->precision > REPLAYSSM_BF16_SHARED)
    return fail(REPLAYSSM_EINVAL, "precision %d unknown", c->precision);
  if (c->B < 1 || c->B > 65535) return fail(REPLAYSSM_EINVAL, "B=%d outside 1..65535", c->B);
  if (c->H < 1) return fail(REPLAYSSM_EINVAL, "H=%d < 1", c->H);
  // (item indices plus the grid stride stay below 2^31)
  if ((int64_t)c->B * c->H > (int64_t)1 << 30) return fail(REPLAYSSM_EINVAL, "B*H above 2^30");
  if (c->dv < 16 || c->dv > rs::kMaxDv || c->dv % 16 != 0)
    return fail(REPLAYSSM_EINVAL, "dv=%d must be a multiple of 16 in 16..256", c->dv);
  if (c->dk != 16 && c->dk != 32 && c->dk != 64 && c->dk != 128)
    return fail(REPLAYSSM_EINVAL, "dk=%d must be 16, 32, 64 or 128", c->dk);
  if (c->L < 1 || c->L > rs::kMaxL) return fail(REPLAYSSM_EINVAL, "L=%d outside 1..64", c->L);
  // one sequence's appended rows are counted in 32-bit float4 units
  if ((int64_t)c->H * 8 * (2 * c->dk + c->dv) / 4 > (int64_t)1 << 30)
    return fail(REPLAYSSM_EINVAL, "H=%d too large for one sequence's records", c->H);
  if (c->T_max < 1 || c->T_max > rs::kMaxDrafts || c->T_max > c->L)
    return fail(REPLAYSSM_EINVAL, "T_max=%d outside 1..min(8, L)", c->T_max);
  if (c->precision != REPLAYSSM_FP32 && c->dk % 32 != 0)
    return fail(REPLAYSSM_ENOTSUP, "a bf16 checkpoint needs dk %% 32 == 0 (dk=%d)", c->dk);
  if (c->kind == REPLAYSSM_KDA && c->precision != REPLAYSSM_FP32)
    return fail(REPLAYSSM_ENOTSUP, "KDA layers keep an fp32 checkpoint only (precision FP32)");
  if (c->precision == REPLAYSSM_BF16_SHARED && c->kind == REPLAYSSM_GDN)
    return fail(REPLAYSSM_ENOTSUP,
                "the shared bf16 checkpoint is built for Mamba-2 only (GDN takes FP32 or "
                "FP32_HP_BF16_LP)");
  const rs::ReplayLds lds(c->L + c->T_max, c->dk, c->dv, tmax_bucket(c->T_max),
                          exact_u(c) ? rs::kKindGdnExact : c->kind, true);
  if (lds.total * 4 > rs::kArchMaxLdsBytes)
    return fail(REPLAYSSM_ENOTSUP, "L + T_max and dims need %d bytes of LDS (> %d on gfx950)", lds.total * 4,
                rs::kArchMaxLdsBytes);
  return REPLAYSSM_OK;
}

int check_state(const replayssm_config* c, const replayssm_state* s, bool need_arrive = true) {
  if (s == nullptr) return fail(REPLAYSSM_EINVAL, "state is NULL");
  if (c->precision != REPLAYSSM_BF16_SHARED) NEED(s->hp);
  if (c->precision != REPLAYSSM_FP32) NEED(s->lp);
  NEED(s->ring_alpha);
  NEED(s->ring_k);
  NEED(s->ring_v);
  if (c->kind != REPLAYSSM_MAMBA2) NEED(s->ring_beta);
  if (exact_u(c)) NEED(s->ring_vraw);
  NEED(s->head);
  NEED(s->h);
  NEED(s->p);
  NEED(s->folded);
  if (need_arrive) NEED(s->arrive);
  NEED(s->err);
  return REPLAYSSM_OK;
}

rs::ReplayArgs replay_args(const replayssm_config* c, const replayssm_state* s, int T, int mode,
                           const float* q, float* out) {
  rs::ReplayArgs a{};
  a.hp = s->hp;
  a.lp = s->lp;
  a.ring_alpha = s->ring_alpha;
  a.ring_beta = s->ring_beta;
  a.ring_k = s->ring_k;
  a.ring_v = s->ring_v;
  a.ring_vraw = exact_u(c) ? s->ring_vraw : nullptr;
  a.head = s->head;
  a.h = s->h;
  a.p = s->p;
  a.folded = s->folded;
  a.arrive = s->arrive;
  a.err = s->err;
  a.q = q;
  a.out = out;
  a.in_alpha = nullptr;
  a.in_beta = nullptr;
  a.in_k = nullptr;
  a.in_v = nullptr;
  a.fused = 0;
  a.B = c->B;
  a.H = c->H;
  a.dv = c->dv;
  a.L = c->L;
  a.C = c->L + c->T_max;
  a.T = T;
  a.precision = c->precision;
  a.mode = mode;
  return a;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

const char* replayssm_status_string(int status) {
  switch (status) {
    case REPLAYSSM_OK: return "ok";
    case REPLAYSSM_EINVAL: return "invalid argument";
    case REPLAYSSM_ENOTSUP: return "not supported";
    case REPLAYSSM_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* replayssm_last_error(void) { return g_last_error.c_str(); }

int replayssm_get_sizes(const replayssm_config* cfg, replayssm_sizes* out) {
  if (int r = check_config(cfg)) return r;
  if (out == nullptr) return fail(REPLAYSSM_EINVAL, "out is NULL");
  const int64_t BH = (int64_t)cfg->B * cfg->H;
  const int C = cfg->L + cfg->T_max;
  const int64_t state = BH * cfg->dv * cfg->dk;
  out->C = C;
  out->alignment = 256;
  out->hp_bytes = cfg->precision == REPLAYSSM_BF16_SHARED ? 0 : state * 4;
  out->lp_bytes = cfg->precision == REPLAYSSM_FP32 ? 0 : state * 2;
  out->ring_alpha_bytes = BH * C * 4 * (cfg->kind == REPLAYSSM_KDA ? cfg->dk : 1);
  out->ring_beta_bytes = cfg->kind != REPLAYSSM_MAMBA2 ? BH * C * 4 : 0;
  out->ring_k_bytes = BH * C * cfg->dk * 4;
  out->ring_v_bytes = BH * C * cfg->dv * 4;
  out->ptr_bytes = (int64_t)cfg->B * 4;
  out->folded_bytes = (int64_t)cfg->B * 8;
  out->err_bytes = 4;
  out->ring_vraw_bytes = exact_u(cfg) ? BH * C * cfg->dv * 4 : 0;
  return REPLAYSSM_OK;
}

int replayssm_init(const replayssm_config* cfg, const replayssm_state* st, void* stream) {
  if (int r = check_config(cfg)) return r;
  if (int r = check_state(cfg, st)) return r;
  return hip_result(rs::launch_init(st->head, st->h, st->p, st->folded, st->arrive, st->err, cfg->B,
                                    as_stream(stream)),
                    "init");
}

int replayssm_pack_state(const replayssm_config* cfg, const float* src, float* hp_dst,
                         uint16_t* lp_dst, void* stream) {
  if (int r = check_config(cfg)) return r;
  NEED(src);
  if (hp_dst == nullptr && lp_dst == nullptr)
    return fail(REPLAYSSM_EINVAL, "both destinations are NULL");
  if (hp_dst && !aligned(hp_dst)) return fail(REPLAYSSM_EINVAL, "hp_dst is not 16-byte aligned");
  if (lp_dst) {
    if (!aligned(lp_dst)) return fail(REPLAYSSM_EINVAL, "lp_dst is not 16-byte aligned");
    if (cfg->dk % 32 != 0) return fail(REPLAYSSM_ENOTSUP, "a bf16 checkpoint needs dk %% 32 == 0");
  }
  return hip_result(rs::launch_pack(src, hp_dst, lp_dst, (int64_t)cfg->B * cfg->H, cfg->dv,
                                    cfg->dk, as_stream(stream)),
                    "pack_state");
}

int replayssm_unpack_state(const replayssm_config* cfg, const float* hp_src, const uint16_t* lp_src,
                           float* dst, void* stream) {
  if (int r = check_config(cfg)) return r;
  NEED(dst);
  if (hp_src == nullptr && lp_src == nullptr) return fail(REPLAYSSM_EINVAL, "both sources are NULL");
  if (hp_src && !aligned(hp_src)) return fail(REPLAYSSM_EINVAL, "hp_src is not 16-byte aligned");
  if (!hp_src) {
    if (!aligned(lp_src)) return fail(REPLAYSSM_EINVAL, "lp_src is not 16-byte aligned");
    if (cfg->dk % 32 != 0) return fail(REPLAYSSM_ENOTSUP, "a bf16 checkpoint needs dk %% 32 == 0");
  }
  return hip_result(rs::launch_unpack(hp_src, hp_src ? nullptr : lp_src, dst,
                                      (int64_t)cfg->B * cfg->H, cfg->dv, cfg->dk, as_stream(stream)),
                    "unpack_state");
}

int replayssm_read_error(const replayssm_state* st, int32_t* err_out, void* stream) {
  if (st == nullptr || err_out == nullptr) return fail(REPLAYSSM_EINVAL, "NULL argument");
  NEED(st->err);
  hipError_t e = hipMemcpyAsync(err_out, st->err, sizeof(int32_t), hipMemcpyDeviceToHost,
                                as_stream(stream));
  if (e == hipSuccess) e = hipStreamSynchronize(as_stream(stream));
  return hip_result(e, "read_error");
}

static int append_common(const replayssm_config* cfg, const replayssm_state* st, int T, const float* alpha,
                         const float* dt, const float* A, const float* dt_bias, const float* k, const float* v,
                         const float* beta, void* stream, bool static_scratch = false) {
  NEED(k);
  NEED(v);
  if (cfg->kind != REPLAYSSM_MAMBA2) NEED(beta);
  rs::AppendArgs a{};
  a.dt = dt;
  a.A = A;
  a.dt_bias = dt_bias;
  a.ring_alpha = st->ring_alpha;
  a.ring_beta = st->ring_beta;
  a.ring_k = st->ring_k;
  a.ring_v = st->ring_v;
  a.ring_vraw = exact_u(cfg) ? st->ring_vraw : nullptr;
  a.head = st->head;
  a.h = st->h;
  a.p = st->p;
  a.arrive = st->arrive;
  a.err = st->err;
  a.alpha = alpha;
  a.beta = cfg->kind != REPLAYSSM_MAMBA2 ? beta : nullptr;
  a.k = k;
  a.v = v;
  a.B = cfg->B;
  a.H = cfg->H;
  a.dv = cfg->dv;
  a.dk = cfg->dk;
  a.C = cfg->L + cfg->T_max;
  a.T = T;
  a.T_max = cfg->T_max;
  // float4 units per sequence: k rows, KDA gate rows, v rows
  a.units_per_seq = T * cfg->H * ((cfg->kind == REPLAYSSM_KDA ? 2 : 1) * cfg->dk + cfg->dv) / 4;
  if (static_scratch) {
    a.arrive = nullptr;
    return hip_result(rs::launch_append_static(cfg->kind, a, as_stream(stream)), "append_static");
  }
  return hip_result(rs::launch_append(cfg->kind, a, as_stream(stream)), dt ? "append_dt" : "append");
}

int replayssm_append_static(const replayssm_config* cfg, const replayssm_state* st, int T,
                            const float* alpha, const float* k, const float* v, const float* beta,
                            void* stream) {
  if (int r = check_config(cfg)) return r;
  if (int r = check_state(cfg, st, /*need_arrive=*/false)) return r;
  if (cfg->B > REPLAYSSM_STATIC_SCRATCH_SEQS)
    return fail(REPLAYSSM_EINVAL, "B=%d above the %d sequences of the library's scratch counters", cfg->B,
                REPLAYSSM_STATIC_SCRATCH_SEQS);
  if (T < 1 || T > cfg->T_max) return fail(REPLAYSSM_EINVAL, "T=%d outside 1..T_max=%d", T, cfg->T_max);
  NEED(alpha);
  return append_common(cfg, st, T, alpha, nullptr, nullptr, nullptr, k, v, beta, stream, true);
}

int replayssm_append(const replayssm_config* cfg, const replayssm_state* st, int T,
                     const float* alpha, const float* k, const float* v, const float* beta,
                     void* stream) {
  if (int r = check_config(cfg)) return r;
  if (int r = check_state(cfg, st)) return r;
  if (T < 1 || T > cfg->T_max) return fail(REPLAYSSM_EINVAL, "T=%d outside 1..T_max=%d", T, cfg->T_max);
  NEED(alpha);
  return append_common(cfg, st, T, alpha, nullptr, nullptr, nullptr, k, v, beta, stream);
}

int replayssm_append_dt(const replayssm_config* cfg, const replayssm_state* st, int T, const float* dt,
                        const float* A, const float* dt_bias, const float* k, const float* v, const float* beta,
                        void* stream) {
  if (int r = check_config(cfg)) return r;
  if (int r = check_state(cfg, st)) return r;
  if (cfg->kind == REPLAYSSM_KDA)
    return fail(REPLAYSSM_ENOTSUP, "append_dt computes a scalar decay per record; KDA gates are per channel");
  if (T < 1 || T > cfg->T_max) return fail(REPLAYSSM_EINVAL, "T=%d outside 1..T_max=%d", T, cfg->T_max);
  NEED(dt);
  NEED(A);
  return append_common(cfg, st, T, nullptr, dt, A, dt_bias, k, v, beta, stream);
}

int replayssm_decode(const replayssm_config* cfg, const replayssm_state* st, const float* q,
                     float* out, void* stream) {
  if (int r = check_config(cfg)) return r;
  if (int r = check_state(cfg, st)) return r;
  NEED(q);
  NEED(out);
  const rs::ReplayArgs a = replay_args(cfg, st, 1, rs::kModeDecode, q, out);
  return replay(cfg, 1, a, as_stream(stream), "decode");
}

int replayssm_verify(const replayssm_config* cfg, const replayssm_state* st, int T, const float* q,
                     float* out, void* stream) {
  if (int r = check_config(cfg)) return r;
  if (int r = check_state(cfg, st)) return r;
  if (T < 1 || T > cfg->T_max) return fail(REPLAYSSM_EINVAL, "T=%d outside 1..T_max=%d", T, cfg->T_max);
  NEED(q);
  NEED(out);
  const rs::ReplayArgs a = replay_args(cfg, st, T, rs::kModeVerify, q, out);
  return replay(cfg, tmax_bucket(T), a, as_stream(stream), "verify");
}

static int fused_call(const replayssm_config* cfg, const replayssm_state* st, int T, int mode,
                      const float* alpha, const float* k, const float* v, const float* beta, const float* q,
                      float* out, void* stream, const char* what) {
  if (int r = check_config(cfg)) return r;
  if (int r = check_state(cfg, st)) return r;
  if (T < 1 || T > cfg->T_max) return fail(REPLAYSSM_EINVAL, "T=%d outside 1..T_max=%d", T, cfg->T_max);
  NEED(alpha);
  NEED(k);
  NEED(v);
  NEED(q);
  NEED(out);
  if (cfg->kind != REPLAYSSM_MAMBA2) NEED(beta);
  rs::ReplayArgs a = replay_args(cfg, st, T, mode, q, out);
  a.in_alpha = alpha;
  a.in_beta = cfg->kind != REPLAYSSM_MAMBA2 ? beta : nullptr;
  a.in_k = k;
  a.in_v = v;
  a.fused = 1;
  return replay(cfg, tmax_bucket(T), a, as_stream(stream), what);
}

int replayssm_decode_step(const replayssm_config* cfg, const replayssm_state* st, const float* alpha,
                          const float* k, const float* v, const float* beta, const float* q, float* out,
                          void* stream) {
  return fused_call(cfg, st, 1, rs::kModeDecode, alpha, k, v, beta, q, out, stream, "decode_step");
}

int replayssm_verify_step(const replayssm_config* cfg, const replayssm_state* st, int T, const float* alpha,
                          const float* k, const float* v, const float* beta, const float* q, float* out,
                          void* stream) {
  return fused_call(cfg, st, T, rs::kModeVerify, alpha, k, v, beta, q, out, stream, "verify_step");
}

int replayssm_accept(const replayssm_config* cfg, const replayssm_state* st,
                     const int32_t* accepted, void* stream) {
  if (int r = check_config(cfg)) return r;
  if (int r = check_state(cfg, st)) return r;
  NEED(accepted);
  return hip_result(
      rs::launch_accept(st->h, st->p, st->err, accepted, cfg->B, cfg->L, as_stream(stream)),
      "accept");
}

int replayssm_flush(const replayssm_config* cfg, const replayssm_state* st, void* stream) {
  if (int r = check_config(cfg)) return r;
  if (int r = check_state(cfg, st)) return r;
  const rs::ReplayArgs a = replay_args(cfg, st, 0, rs::kModeFlush, nullptr, nullptr);
  return replay(cfg, 1, a, as_stream(stream), "flush");
}

int replayssm_flush_selected(const replayssm_config* cfg, const replayssm_state* st,
                             const int32_t* select, void* stream) {
  if (int r = check_config(cfg)) return r;
  if (int r = check_state(cfg, st)) return r;
  NEED(select);
  rs::ReplayArgs a = replay_args(cfg, st, 0, rs::kModeFlush, nullptr, nullptr);
  a.select = select;
  return replay(cfg, 1, a, as_stream(stream), "flush_selected");
}

int replayssm_snapshot(const replayssm_config* cfg, const replayssm_state* st, int n,
                       const int32_t* seqs, float* dst, void* stream) {
  if (int r = check_config(cfg)) return r;
  if (int r = check_state(cfg, st)) return r;
  if (n < 0) return fail(REPLAYSSM_EINVAL, "n=%d < 0", n);
  if (n == 0) return REPLAYSSM_OK;
  NEED(seqs);
  NEED(dst);
  const float* hp = cfg->precision == REPLAYSSM_BF16_SHARED ? nullptr : st->hp;
  return hip_result(rs::launch_snapshot(hp, st->lp, st->h, st->err, seqs, n, dst, cfg->B, cfg->H, cfg->dv,
                                        cfg->dk, as_stream(stream)),
                    "snapshot");
}

int replayssm_restore(const replayssm_config* cfg, const replayssm_state* st, int n,
                      const int32_t* seqs, const float* src, void* stream) {
  if (int r = check_config(cfg)) return r;
  if (int r = check_state(cfg, st)) return r;
  if (n < 0) return fail(REPLAYSSM_EINVAL, "n=%d < 0", n);
  if (n == 0) return REPLAYSSM_OK;
  NEED(seqs);
  NEED(src);
  float* hp = cfg->precision == REPLAYSSM_BF16_SHARED ? nullptr : st->hp;
  uint16_t* lp = cfg->precision == REPLAYSSM_FP32 ? nullptr : st->lp;
  return hip_result(rs::launch_restore(hp, lp, st->head, st->h, st->p, st->folded, st->err, seqs, n, src, cfg->B,
                                       cfg->H, cfg->dv, cfg->dk, as_stream(stream)),
                    "restore");
}

int replayssm_eager_step(const replayssm_config* cfg, float* S, const float* alpha, const float* k,
                         const float* v, const float* beta, const float* q, float* out,
                         void* stream) {
  if (int r = check_config(cfg)) return r;
  if (cfg->precision != REPLAYSSM_FP32)
    return fail(REPLAYSSM_EINVAL, "the eager kernel keeps an fp32 state (precision must be FP32)");
  NEED(S);
  NEED(alpha);
  NEED(k);
  NEED(v);
  NEED(q);
  NEED(out);
  if (cfg->kind != REPLAYSSM_MAMBA2) NEED(beta);
  rs::EagerArgs a{};
  a.S = S;
  a.slot = nullptr;
  a.alpha = alpha;
  a.beta = beta;
  a.k = k;
  a.v = v;
  a.q = q;
  a.out = out;
  a.B = cfg->B;
  a.H = cfg->H;
  a.dv = cfg->dv;
  a.T = 1;
  a.nslots = 1;
  return hip_result(rs::launch_eager(cfg->kind, cfg->dk, a, as_stream(stream)), "eager_step");
}

int replayssm_eager_verify(const replayssm_config* cfg, float* pool, const int32_t* slot, int T,
                           const float* alpha, const float* k, const float* v, const float* beta,
                           const float* q, float* out, void* stream) {
  if (int r = check_config(cfg)) return r;
  if (cfg->precision != REPLAYSSM_FP32)
    return fail(REPLAYSSM_EINVAL, "the eager kernel keeps an fp32 state (precision must be FP32)");
  if (T < 1 || T > cfg->T_max) return fail(REPLAYSSM_EINVAL, "T=%d outside 1..T_max=%d", T, cfg->T_max);
  NEED(pool);
  NEED(slot);
  NEED(alpha);
  NEED(k);
  NEED(v);
  NEED(q);
  NEED(out);
  if (cfg->kind != REPLAYSSM_MAMBA2) NEED(beta);
  rs::EagerArgs a{};
  a.S = pool;
  a.slot = slot;
  a.alpha = alpha;
  a.beta = beta;
  a.k = k;
  a.v = v;
  a.q = q;
  a.out = out;
  a.B = cfg->B;
  a.H = cfg->H;
  a.dv = cfg->dv;
  a.T = T;
  a.nslots = T + 1;
  return hip_result(rs::launch_eager(cfg->kind, cfg->dk, a, as_stream(stream)), "eager_verify");
}

int replayssm_eager_accept(const replayssm_config* cfg, int32_t* slot, const int32_t* accepted, int T,
                           void* stream) {
  if (int r = check_config(cfg)) return r;
  if (T < 1 || T > cfg->T_max) return fail(REPLAYSSM_EINVAL, "T=%d outside 1..T_max=%d", T, cfg->T_max);
  NEED(slot);
  NEED(accepted);
  return hip_result(rs::launch_eager_accept(slot, accepted, cfg->B, T, as_stream(stream)),
                    "eager_accept");
}

int replayssm_set_tiling(int policy) {
  if (policy != REPLAYSSM_TILES_AUTO && policy != REPLAYSSM_TILES_ONE && policy != REPLAYSSM_TILES_TWO)
    return fail(REPLAYSSM_EINVAL, "tiling policy %d is not one of 0 (auto), 1 (one tile), 2 (two tiles)", policy);
  rs::set_tiling(policy);
  return REPLAYSSM_OK;
}

int replayssm_get_tiling(void) { return rs::get_tiling(); }

int replayssm_probe_read(const void* src, int64_t bytes, float* sink, void* stream) {
  NEED(src);
  if (sink == nullptr) return fail(REPLAYSSM_EINVAL, "sink is NULL");
  if (bytes <= 0 || bytes % 16 != 0)
    return fail(REPLAYSSM_EINVAL, "bytes=%lld must be a positive multiple of 16", (long long)bytes);
  return hip_result(rs::launch_probe_read(src, bytes, sink, as_stream(stream)), "probe_read");
}

}  // extern "C"

// ---- convolution input ring ----------------------------------------------

namespace {

int check_conv(const replayssm_conv_config* c) {
  if (c == nullptr) return fail(REPLAYSSM_EINVAL, "cfg is NULL");
  if (c->B < 1 || c->B > 65535) return fail(REPLAYSSM_EINVAL, "B=%d outside 1..65535", c->B);
  if (c->D < 4 || c->D % 4 != 0) return fail(REPLAYSSM_EINVAL, "D=%d must be a positive multiple of 4", c->D);
  if ((int64_t)c->D / 4 > (int64_t)256 * 65535) return fail(REPLAYSSM_EINVAL, "D=%d too large", c->D);
  if (c->W < 1 || c->W > rs::kConvMaxW) return fail(REPLAYSSM_EINVAL, "W=%d outside 1..%d", c->W, rs::kConvMaxW);
  if (c->T_max < 1 || c->T_max > rs::kMaxDrafts) return fail(REPLAYSSM_EINVAL, "T_max=%d outside 1..8", c->T_max);
  return REPLAYSSM_OK;
}

int check_conv_state(const replayssm_conv_state* s) {
  if (s == nullptr) return fail(REPLAYSSM_EINVAL, "state is NULL");
  NEED(s->ring);
  NEED(s->start);
  NEED(s->pend);
  NEED(s->arrive);
  NEED(s->err);
  return REPLAYSSM_OK;
}

rs::ConvArgs conv_args(const replayssm_conv_config* c, const replayssm_conv_state* s) {
  rs::ConvArgs a{};
  a.ring = s->ring;
  a.start = s->start;
  a.pend = s->pend;
  a.arrive = s->arrive;
  a.err = s->err;
  a.B = c->B;
  a.D = c->D;
  a.W = c->W;
  a.T_max = c->T_max;
  return a;
}

}  // namespace

extern "C" {

int replayssm_conv_sizes(const replayssm_conv_config* cfg, int64_t* ring_bytes, int64_t* ptr_bytes) {
  if (int r = check_conv(cfg)) return r;
  if (ring_bytes) *ring_bytes = (int64_t)cfg->B * (cfg->W - 1 + cfg->T_max) * cfg->D * 4;
  if (ptr_bytes) *ptr_bytes = (int64_t)cfg->B * 4;
  return REPLAYSSM_OK;
}

int replayssm_conv_init(const replayssm_conv_config* cfg, const replayssm_conv_state* st, void* stream) {
  if (int r = check_conv(cfg)) return r;
  if (int r = check_conv_state(st)) return r;
  return hip_result(rs::launch_conv_init(conv_args(cfg, st), as_stream(stream)), "conv_init");
}

int replayssm_conv_step(const replayssm_conv_config* cfg, const replayssm_conv_state* st, int T,
                        const float* x, const float* w, const float* bias, int silu, int commit,
                        float* y, void* stream) {
  if (int r = check_conv(cfg)) return r;
  if (int r = check_conv_state(st)) return r;
  if (T < 1 || T > cfg->T_max) return fail(REPLAYSSM_EINVAL, "T=%d outside 1..T_max=%d", T, cfg->T_max);
  NEED(x);
  NEED(w);
  NEED(y);
  if (bias && !aligned(bias)) return fail(REPLAYSSM_EINVAL, "bias is not 16-byte aligned");
  rs::ConvArgs a = conv_args(cfg, st);
  a.x = x;
  a.w = w;
  a.bias = bias;
  a.y = y;
  a.T = T;
  a.silu = silu ? 1 : 0;
  a.commit = commit ? 1 : 0;
  return hip_result(rs::launch_conv_step(a, as_stream(stream)), "conv_step");
}

int replayssm_conv_accept(const replayssm_conv_config* cfg, const replayssm_conv_state* st,
                          const int32_t* accepted, void* stream) {
  if (int r = check_conv(cfg)) return r;
  if (int r = check_conv_state(st)) return r;
  NEED(accepted);
  return hip_result(rs::launch_conv_accept(conv_args(cfg, st), accepted, as_stream(stream)), "conv_accept");
}

}  // extern "C"
