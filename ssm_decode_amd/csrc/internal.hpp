// Internal declarations shared by the HIP sources of libreplayssm (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "replayssm.h"

namespace rs {

// ---------------------------------------------------------------------------
// Checkpoint layout on the device (private to the library).
//
// A head's dv x dk fp32 state is cut into 16 x 16 tiles; tile (pt, nt) covers
// rows p = 16 pt .. 16 pt + 15 and columns n = 16 nt .. 16 nt + 15 and is stored
// as 1 KiB at float offset (pt * NT + nt) * 256, NT = dk / 16. Inside a tile,
// lane l (0..63) of a wavefront owns one float4:
//     row p = 16 pt + (l & 15), columns n = 16 nt + 4 (l >> 4) + {0, 1, 2, 3}
// This is exactly the accumulator layout of v_mfma_f32_16x16x4_f32 when the
// MFMA's M index runs over n and its N index over p, so a fold can seed the
// accumulators with one 16-byte load per lane and store them back the same
// way, and a wavefront's load of one tile is one contiguous 1 KiB.
//
// The bf16 copy pairs tiles (pt, 2m) and (pt, 2m + 1) into one 1 KiB chunk at
// bf16 offset (pt * NT/2 + m) * 512; lane l owns 8 bf16 (16 bytes): elements
// 0..3 are its float4 of tile 2m, elements 4..7 its float4 of tile 2m + 1.
// ---------------------------------------------------------------------------
constexpr int kWave = 64;
constexpr int kMaxDrafts = 8;
constexpr int kMaxL = 64;
constexpr int kMaxDv = 256;
constexpr int kStageRegs = 5;  // float4 record units per thread kept in flight at once

typedef float f32x4 __attribute__((ext_vector_type(4)));

enum Mode : int { kModeDecode = 0, kModeVerify = 1, kModeFlush = 2 };

// Kernel kinds: the two public kinds, plus GDN with the two-precision checkpoint,
// whose folds recompute the folded records' corrections (its own instantiation,
// so that the other GDN kernels do not carry that code's registers).
constexpr int kKindGdnExact = 3;
// Kinds whose records carry a correction u and a beta (the delta rule).
__host__ __device__ constexpr bool kind_gdn(int kind) { return kind != REPLAYSSM_MAMBA2; }

struct ReplayArgs {
  float* hp;
  uint16_t* lp;
  float* ring_alpha;
  float* ring_beta;
  float* ring_k;
  float* ring_v;
  int32_t* head;
  int32_t* h;
  int32_t* p;
  int64_t* folded;
  int32_t* arrive;
  int32_t* err;
  float* ring_vraw;  // GDN two-precision: raw v of every record, for the fold
  const int32_t* select;  // flush only: [B] nonzero = fold this sequence; NULL = all
  const float* q;  // [B][T][H][dk]
  float* out;      // [B][T][H][dv]
  // fused append: the T new records come from these inputs (and are written to
  // the ring by the same launch) instead of from the ring; p must be 0 on entry
  const float* in_alpha;  // [B][T][H]
  const float* in_beta;   // [B][T][H] (GDN)
  const float* in_k;      // [B][T][H][dk]
  const float* in_v;      // [B][T][H][dv]
  int fused;
  int lds_unpadded;  // set by the launcher: the LDS carve uses unpadded record rows
  int B, H, dv, L, C, T;
  int precision;
  int mode;
};

struct AppendArgs {
  float* ring_alpha;
  float* ring_beta;
  float* ring_k;
  float* ring_v;
  float* ring_vraw;  // or NULL
  int32_t* head;
  int32_t* h;
  int32_t* p;
  int32_t* arrive;
  int32_t* err;
  const float* alpha;
  const float* beta;
  const float* k;
  const float* v;
  // decay from the raw time step (replayssm_append_dt): alpha is NULL and
  // alpha = exp(-softplus(dt + dt_bias[h]) * A[h]); dt_bias may be NULL
  const float* dt;       // [B][T][H]
  const float* A;        // [H]
  const float* dt_bias;  // [H] or NULL
  int B, H, dv, dk, C, T, T_max;
  int units_per_seq;  // float4 units of k and v per sequence
};

struct EagerArgs {
  float* S;             // [B][H][slots][dv*dk] private layout
  const int32_t* slot;  // [B] or NULL (in-place step)
  const float* alpha;   // [B][T][H]
  const float* beta;
  const float* k;  // [B][T][H][dk]
  const float* v;  // [B][T][H][dv]
  const float* q;  // [B][T][H][dk]
  float* out;      // [B][T][H][dv]
  int B, H, dv, T, nslots;
};

// Dynamic LDS carve-up of the replay kernel, in floats. Every block starts on a
// 16-byte boundary. Row strides are padded so that the four 16-lane groups of a
// wavefront reading one column of four consecutive rows hit distinct banks,
// unless the launcher asks for unpadded rows (when they let more workgroups
// share a compute unit: long windows, whose padded carve is what limits the
// occupancy) or the padded carve passes kLdsPaddedBudget. The carve may exceed
// that budget up to what the device gives one workgroup (kArchMaxLdsBytes on
// gfx950, 160 KiB per compute unit; each launch checks the device's own figure).
// The kernel kind changes blocks: GDN with the two-precision checkpoint adds the
// Gram blocks k_i . k_j of the staged records and a table of S k_j (its exact fold); KDA has a gate
// row per record instead of a scalar, no decay-product tables, and adds the
// drafts' queries and keys scaled by the gates since the last committed record,
// and the committed records' column decay.
constexpr int kLdsPaddedBudget = 64 * 1024;
constexpr int kArchMaxLdsBytes = 160 * 1024;
struct ReplayLds {
  int dks, dvs;  // row strides of the k and v record rows
  int k, v, alpha, beta, q, gq, gk, cq, ck, gram, ytab, ys, qg, kg, pf, total;
  __host__ __device__ static int pad4(int x) { return (x + 3) & ~3; }
  __host__ __device__ static int row_stride(int d) { return ((d / 16) & 1) ? d : d + 16; }
  __host__ __device__ ReplayLds(int C, int dk, int dv, int tmax, int kind = REPLAYSSM_MAMBA2,
                                bool unpadded = false) {
    carve(C, dk, dv, tmax, row_stride(dk), row_stride(dv), kind);
    if (unpadded || total * 4 > kLdsPaddedBudget) carve(C, dk, dv, tmax, dk, dv, kind);
  }
  __host__ __device__ void carve(int C, int dk, int dv, int tmax, int kstride, int vstride, int kind) {
    const bool with_gram = kind == kKindGdnExact, kda = kind == REPLAYSSM_KDA;
    dks = kstride;
    dvs = vstride;
    k = 0;
    v = k + C * dks;
    alpha = v + C * dvs;
    beta = alpha + (kda ? C * dks : pad4(C));
    q = beta + pad4(C);
    gq = q + tmax * dk;
    gk = gq + (kda ? 0 : pad4((C + 1) * tmax));
    cq = gk + (kda ? 0 : pad4((C + 1) * tmax));
    ck = cq + pad4(C * tmax);
    gram = ck + pad4(C * tmax);
    // (exact-correction fold: the Gram matrix's diagonal 16 x 16 blocks, and S k_j of one
    // block of 16 records for every state row, row stride dv + 4)
    ytab = gram + (with_gram ? ((C + 15) / 16) * 256 : 0);
    ys = dv + 4;
    qg = ytab + (with_gram ? 16 * ys : 0);
    kg = qg + (kda ? tmax * dk : 0);
    pf = kg + (kda ? tmax * dk : 0);
    total = pf + (kda ? dk : 0);
  }
};

// Grid size for a persistent kernel: as many workgroups as can be resident on
// the current device at once (occupancy x compute units), at most `items`.
// The occupancy of each (kernel, block, LDS) triple is computed once and cached.
hipError_t persistent_grid(const void* kernel, int block, size_t smem, int items, int* grid);
// Workgroups of `kernel` that can be resident on one compute unit of the current device (cached).
hipError_t blocks_per_cu(const void* kernel, int block, size_t smem, int* per_cu);

// Largest dynamic LDS one workgroup may use on the current device, in bytes (cached per device).
hipError_t device_max_lds(int* bytes);

// Launchers (one per kernel family); they return hipError_t of the launch.
hipError_t launch_replay(int kind, int dk, int tmax, const ReplayArgs& a, hipStream_t s);
// Tiling policy of the replay kernel (REPLAYSSM_TILES_*), process-wide.
void set_tiling(int policy);
int get_tiling();
// Compute units of the current device (cached per device).
hipError_t device_cus(int* cus);
hipError_t launch_append(int kind, const AppendArgs& a, hipStream_t s);
// The same with the per-sequence arrival counters in the library's static device array
// (a.arrive is ignored; B <= kStaticScratchSeqs): clears them, then appends.
constexpr int kStaticScratchSeqs = REPLAYSSM_STATIC_SCRATCH_SEQS;
hipError_t launch_append_static(int kind, const AppendArgs& a, hipStream_t s);
hipError_t launch_accept(int32_t* h, int32_t* p, int32_t* err, const int32_t* acc, int B, int L,
                         hipStream_t s);
hipError_t launch_init(int32_t* head, int32_t* h, int32_t* p, int64_t* folded, int32_t* arrive,
                       int32_t* err, int B, hipStream_t s);
hipError_t launch_pack(const float* src, float* hp, uint16_t* lp, int64_t nheads, int dv, int dk,
                       hipStream_t s);
hipError_t launch_unpack(const float* hp, const uint16_t* lp, float* dst, int64_t nheads, int dv,
                         int dk, hipStream_t s);
// Prefix states: the listed sequences' checkpoints out to / in from the logical layout.
hipError_t launch_snapshot(const float* hp, const uint16_t* lp, const int32_t* h, int32_t* err,
                           const int32_t* seqs, int n, float* dst, int B, int H, int dv, int dk,
                           hipStream_t s);
hipError_t launch_restore(float* hp, uint16_t* lp, int32_t* head, int32_t* h, int32_t* p, int64_t* folded,
                          int32_t* err, const int32_t* seqs, int n, const float* src, int B, int H, int dv,
                          int dk, hipStream_t s);
hipError_t launch_eager(int kind, int dk, const EagerArgs& a, hipStream_t s);
hipError_t launch_eager_accept(int32_t* slot, const int32_t* acc, int B, int T, hipStream_t s);
hipError_t launch_probe_read(const void* src, int64_t bytes, float* sink, hipStream_t s);


}  // namespace rs
