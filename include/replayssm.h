/*
 * replayssm.h -- C ABI of the ReplaySSM decode path for AMD Instinct MI355X (gfx950).
 *
 * ReplaySSM keeps each head's SSM state as a checkpoint S_ck plus a circular
 * buffer of the most recent input records, computes decode outputs from the two
 * without writing the state back, and folds the buffer into the checkpoint only
 * when the window of L records is full ("ReplaySSM: Cache SSM Inputs, Not
 * State", How it works: Standard decoding; the paper abstract on the Lattice
 * page). With c the checkpoint position and records j = c+1..t in the buffer:
 *
 *     o_t = Gamma_t * S_ck q_t + sum_j gamma_{j,t} * v_j (k_j . q_t)
 *     Gamma_t = prod_{i=c+1..t} alpha_i,  gamma_{j,t} = prod_{i=j+1..t} alpha_i
 *
 * which equals the eager recurrence S_t = alpha_t S_{t-1} + v_t k_t^T,
 * o_t = S_t q_t up to floating-point rounding (same page, Limits).
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Every call returns an int status: REPLAYSSM_OK (0) or a negative code.
 *    Arguments are validated on the host before anything is enqueued; on a
 *    validation error nothing is enqueued and replayssm_last_error() gives text.
 *  - Device work is enqueued on `stream` (a hipStream_t passed as void*; NULL is
 *    the null stream) in stream order. Calls do not synchronise, do not allocate
 *    device memory and keep no pointer after they return.
 *  - All arrays are device memory owned by the caller (e.g. PyTorch tensors).
 *    Their sizes come from replayssm_get_sizes(); every pointer must be 16-byte
 *    aligned and arrays must not overlap.
 *  - Device-side contract violations that depend on device data (e.g. accepting
 *    more drafts than are pending) cannot be returned synchronously: the kernel
 *    leaves that sequence unchanged (or clamps, as documented per call) and ORs
 *    a REPLAYSSM_DEVERR_* bit into the sticky word `state->err`, which
 *    replayssm_read_error() returns.
 *  - The library keeps no per-layer state: calls on distinct states may run
 *    concurrently; calls on one state must be stream-ordered. Its only
 *    process-wide state is the kernel tiling policy (replayssm_set_tiling,
 *    shared by every thread and device; it never changes results), the
 *    per-device caches of compute-unit counts and kernel occupancies, and the
 *    per-device counter array of replayssm_append_static (whose calls on one
 *    GPU must not overlap).
 *
 * Shapes use B sequences, H heads, dv = value/head dim (Mamba-2 P, GDN d_v),
 * dk = key/state dim (Mamba-2 N, GDN d_k), ring capacity C = L + T_max.
 */
#ifndef REPLAYSSM_H
#define REPLAYSSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define REPLAYSSM_OK 0
#define REPLAYSSM_EINVAL (-1)  /* bad argument, size, pointer or alignment      */
#define REPLAYSSM_ENOTSUP (-2) /* valid request with no compiled kernel          */
#define REPLAYSSM_EHIP (-3)    /* the HIP runtime reported an error              */

/* ---- sticky device error bits (state->err) ----------------------------- */
#define REPLAYSSM_DEVERR_APPEND_OVERFLOW 1 /* append: p + T > T_max; sequence skipped     */
#define REPLAYSSM_DEVERR_PENDING 2         /* decode/verify: p != T; sequence skipped     */
#define REPLAYSSM_DEVERR_ACCEPT 4          /* accept: a < 0, a > p or h + a > L; clamped  */
#define REPLAYSSM_DEVERR_CORRUPT 8         /* head/h/p out of range; sequence skipped     */
#define REPLAYSSM_DEVERR_STALE 16          /* snapshot of a sequence with unfolded records */
#define REPLAYSSM_DEVERR_INDEX 32          /* sequence index outside 0..B-1; skipped       */

/* ---- configuration ------------------------------------------------------ */
enum replayssm_kind {
  REPLAYSSM_MAMBA2 = 0, /* S <- alpha S + v k^T                                  */
  REPLAYSSM_GDN = 1,    /* gated delta rule, stored as S <- alpha S + u k^T       */
  REPLAYSSM_KDA = 2     /* Kimi Delta Attention: the delta rule with a gate per key
                           channel, S <- S Diag(a) (I - beta k k^T) + beta v k^T,
                           stored as S <- S Diag(a) + u k^T with
                           u = beta (v - S (a * k)). Named compatible but not built
                           on the summary page (Limits); FP32 precision only.
                           Every alpha input below, [...][H] for the other kinds,
                           is [...][H][dk] for KDA (a gate row per record)         */
};

enum replayssm_precision {
  REPLAYSSM_FP32 = 0,          /* one fp32 checkpoint (HP), read every step          */
  REPLAYSSM_FP32_HP_BF16_LP = 1, /* non-fold steps read a bf16 copy (LP); folds read
                                    HP and write HP and LP. GDN: a fold recomputes
                                    every folded record's u from HP and the raw v
                                    (ring_vraw), so the bf16 rounding of the copy
                                    never enters the checkpoint                     */
  REPLAYSSM_BF16_SHARED = 2    /* one bf16 checkpoint for reads and folds (Mamba-2
                                  only); the comparison case for the two-precision
                                  mode                                              */
};

typedef struct replayssm_config {
  int32_t kind;      /* enum replayssm_kind                                        */
  int32_t precision; /* enum replayssm_precision                                   */
  int32_t B;         /* sequences, >= 1                                            */
  int32_t H;         /* heads per sequence, >= 1, B*H <= 2^30                      */
  int32_t dv;        /* 16..256, multiple of 16                                    */
  int32_t dk;        /* 16, 32, 64 or 128 (32, 64, 128 when a bf16 copy is kept)   */
  int32_t L;         /* window: records folded per checkpoint write, 1..64          */
  int32_t T_max;     /* largest number of drafts per round, 1..min(8, L)           */
} replayssm_config;

/* Device arrays of one layer's state. All are caller-owned device memory.
 *  hp          float  [B][H][dv*dk]  fp32 checkpoint, library-defined layout
 *                                    (NULL in BF16_SHARED mode)
 *  lp          uint16 [B][H][dv*dk]  bf16 checkpoint bits, library-defined
 *                                    layout (NULL in FP32 mode)
 *  ring_alpha  float  [B][H][C]      (KDA: [B][H][C][dk], one gate per key channel)
 *  ring_beta   float  [B][H][C]      GDN and KDA, else NULL
 *  ring_k      float  [B][H][C][dk]
 *  ring_v      float  [B][H][C][dv]  Mamba-2: v. GDN: v as appended, replaced by
 *                                    the correction u_t = beta_t (v_t - alpha_t
 *                                    S_{t-1} k_t) by the decode/verify call that
 *                                    consumes the record (computed from the
 *                                    checkpoint copy that call reads)
 *  ring_vraw   float  [B][H][C][dv]  GDN in FP32_HP_BF16_LP mode only, else NULL:
 *                                    v as appended, kept for the fold
 *  head, h, p  int32  [B]            ring slot of the oldest unfolded committed
 *                                    record; committed unfolded records; pending
 *                                    drafts
 *  folded      int64  [B]            tokens folded into the checkpoint so far
 *  arrive      int32  [B]            library scratch, zero between calls
 *  err         int32  [1]            sticky REPLAYSSM_DEVERR_* bits
 * The ring, pointer and error arrays have plain row-major layouts that callers
 * may read. The checkpoint layouts are private: use replayssm_pack_state /
 * replayssm_unpack_state to move between them and the logical [dv][dk] order. */
typedef struct replayssm_state {
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
  float* ring_vraw;
} replayssm_state;

typedef struct replayssm_sizes {
  int32_t C;               /* ring capacity L + T_max                         */
  int32_t alignment;       /* required alignment of every array, bytes        */
  int64_t hp_bytes;        /* 0 when not used by the precision mode           */
  int64_t lp_bytes;        /* 0 when not used by the precision mode           */
  int64_t ring_alpha_bytes;
  int64_t ring_beta_bytes; /* 0 for Mamba-2                                   */
  int64_t ring_k_bytes;
  int64_t ring_v_bytes;
  int64_t ptr_bytes;       /* each of head, h, p, arrive                       */
  int64_t folded_bytes;
  int64_t err_bytes;
  int64_t ring_vraw_bytes; /* GDN with FP32_HP_BF16_LP only, else 0            */
} replayssm_sizes;

/* ---- helpers ------------------------------------------------------------ */

/* Validates cfg and reports the size of every state array. Host only. */
int replayssm_get_sizes(const replayssm_config* cfg, replayssm_sizes* out);

/* Text for a status code (static storage). */
const char* replayssm_status_string(int status);

/* Text of the last host-side validation or HIP error of the calling thread. */
const char* replayssm_last_error(void);

/* Zeroes head, h, p, folded, arrive and err: an empty buffer whose checkpoint
 * sits at position 0. Does not touch hp/lp (use replayssm_pack_state). */
int replayssm_init(const replayssm_config* cfg, const replayssm_state* st, void* stream);

/* Converts B*H logical checkpoints src [B][H][dv][dk] fp32 (row p, column n)
 * into the private layouts: hp_dst gets the fp32 values, lp_dst their bf16
 * round-to-nearest-even (either may be NULL, not both). lp_dst needs dk % 32 == 0. */
int replayssm_pack_state(const replayssm_config* cfg, const float* src, float* hp_dst,
                         uint16_t* lp_dst, void* stream);

/* Inverse of replayssm_pack_state: reads hp_src if it is not NULL, else lp_src
 * (bf16 widened exactly), and writes dst [B][H][dv][dk] fp32. */
int replayssm_unpack_state(const replayssm_config* cfg, const float* hp_src,
                           const uint16_t* lp_src, float* dst, void* stream);

/* Copies the sticky error word to *err_out. Synchronises `stream` (tests and
 * debugging only, not for the hot path). */
int replayssm_read_error(const replayssm_state* st, int32_t* err_out, void* stream);

/* ---- the decode path ----------------------------------------------------- */

/* Append T input records per (sequence, head) as pending drafts: record i goes
 * to ring slot (head + h + p + i) mod C, then p += T ("How it works":
 * Standard decoding appends the token's (alpha, v, k); Speculative decoding
 * appends all T draft records; the buffer is circular with capacity L + T).
 *   alpha [B][T][H] (KDA: [B][T][H][dk]), k [B][T][H][dk], v [B][T][H][dv],
 *   beta [B][T][H] (GDN and KDA, else NULL)
 * 1 <= T <= T_max. A sequence with p + T > T_max is skipped and flagged
 * (REPLAYSSM_DEVERR_APPEND_OVERFLOW). */
int replayssm_append(const replayssm_config* cfg, const replayssm_state* st, int T,
                     const float* alpha, const float* k, const float* v, const float* beta,
                     void* stream);

/* replayssm_append with each record's decay computed on the GPU from the raw
 * time step instead of passed in: the discretisation of the layer just before
 * the path (Mamba-2; the same scalar gate form serves Gated DeltaNet), fused
 * into the append so that no separate elementwise pass writes alpha. Per
 * record (b, i, h):
 *     Delta = softplus(dt[b][i][h] + dt_bias[h]),  alpha = exp(-Delta * A[h])
 * with softplus(x) = log(1 + e^x), evaluated as max(x, 0) + log1p(e^-|x|) in
 * fp32. The pages give alpha as an input ("How it works": the buffer holds the
 * records (alpha, k, v)); this form of it is the reading taken for the step on
 * the path's input side (the thread's question on prefix caching and the
 * neighbouring layer steps is where the pages leave it open).
 *   dt [B][T][H]; A [H] (decay rate per head, A >= 0 gives alpha in (0, 1]);
 *   dt_bias [H] or NULL (zero); k, v, beta as for replayssm_append.
 * Scalar-gate kinds only: KDA returns REPLAYSSM_ENOTSUP. Everything else
 * (slots, p += T, overflow flag) is exactly replayssm_append. */
int replayssm_append_dt(const replayssm_config* cfg, const replayssm_state* st, int T,
                        const float* dt, const float* A, const float* dt_bias, const float* k,
                        const float* v, const float* beta, void* stream);

/* replayssm_append for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops and harnesses that forbid allocation): the
 * same call, except that the per-sequence arrival counters the append kernel
 * uses are taken from an array the library holds in device memory
 * (REPLAYSSM_STATIC_SCRATCH_SEQS int32 counters, 64 KiB, one copy per GPU for
 * the life of the process, its address looked up on the first call on each
 * device) instead of st->arrive, which may be NULL. Allocates nothing; each call
 * clears the counters it uses before the append. B above
 * REPLAYSSM_STATIC_SCRATCH_SEQS returns REPLAYSSM_EINVAL. Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (on different
 * streams without ordering) race on it and must not be issued; stream-ordered
 * calls are safe. Results are bit-identical to replayssm_append. */
#define REPLAYSSM_STATIC_SCRATCH_SEQS 16384
int replayssm_append_static(const replayssm_config* cfg, const replayssm_state* st, int T,
                            const float* alpha, const float* k, const float* v, const float* beta,
                            void* stream);

/* One standard decoding step: the single pending record (appended by
 * replayssm_append with T = 1) is the new token t.
 *   - if h + 1 > L, the h committed records are first folded into the
 *     checkpoint (S_ck <- Gamma S_ck + V diag(gamma) K^T; one checkpoint write
 *     per L tokens; "How it works": Standard decoding, and the author's reply
 *     on the flush route: the state comes from one V K^T product, the output
 *     from multiplying it with q_t);
 *   - o_t is computed output-only from the checkpoint and the buffer;
 *   - the token is committed: h += 1, p = 0.
 * In FP32_HP_BF16_LP mode non-fold steps read the bf16 copy and fold steps read
 * the fp32 checkpoint and write both ("How it works": Two precisions).
 * For GDN the record's v is replaced in the ring by u_t.
 *   q [B][H][dk], out [B][H][dv].
 * A sequence with p != 1 is skipped and flagged (REPLAYSSM_DEVERR_PENDING). */
int replayssm_decode(const replayssm_config* cfg, const replayssm_state* st, const float* q,
                     float* out, void* stream);

/* Output-only verification of the T pending drafts (p must equal T): if
 * h + T > L the committed records are folded first (they are known to be
 * committed, so this can run before acceptance; flowchart under "How it works"),
 * then o for every draft i = 1..T is computed from the checkpoint and the
 * buffer without materialising any intermediate state. h and p are not changed
 * except by the fold (head += h mod C, folded += h, h = 0).
 *   q [B][T][H][dk], out [B][T][H][dv].
 * A sequence with p != T is skipped and flagged (REPLAYSSM_DEVERR_PENDING). */
int replayssm_verify(const replayssm_config* cfg, const replayssm_state* st, int T,
                     const float* q, float* out, void* stream);

/* Accepts a prefix of the pending drafts: h += a[b], p = 0. No data moves;
 * rejected records stay in the ring until the next append overwrites them
 * ("How it works": Speculative decoding).
 *   accepted [B] int32, device memory.
 * a < 0, a > p or h + a > L is clamped into range and flagged
 * (REPLAYSSM_DEVERR_ACCEPT). */
int replayssm_accept(const replayssm_config* cfg, const replayssm_state* st,
                     const int32_t* accepted, void* stream);

/* Folds every committed record into the checkpoint now (a rank-h update,
 * written to HP and/or LP as the precision mode requires): head += h mod C,
 * folded += h, h = 0. Pending drafts are kept. Sequences with h = 0 are left
 * alone. Afterwards the checkpoint alone is the state at position `folded`.
 * This is the fold that decode and verify run on their flush route, on its
 * own: the checkpoint becomes the decayed checkpoint plus the buffered records
 * ("How it works": Standard decoding, the checkpoint is written when the buffer
 * is folded; the author's reply on the flush route in the thread "Songlin Yang
 * releases ReplaySSM": the new state is one product of the stacked v and k
 * vectors, V K^T, instead of a token-by-token recurrence). */
int replayssm_flush(const replayssm_config* cfg, const replayssm_state* st, void* stream);

/* ---- prefix states -------------------------------------------------------
 * The checkpoint alone is a sequence's state only once its committed records are
 * folded; until then it trails them (the staleness raised about prefix caching in
 * the replies of the thread on "ReplaySSM"). These calls let a state be shared
 * between sequences, e.g. a cached prompt prefix: fold, copy it out, start other
 * sequences from it. */

/* replayssm_flush for the sequences with select[b] != 0 only (select: [B] int32,
 * device memory); the others keep their checkpoints and pointers. */
int replayssm_flush_selected(const replayssm_config* cfg, const replayssm_state* st,
                             const int32_t* select, void* stream);

/* Copies the checkpoints of sequences seqs[0..n) (device int32) to dst
 * [n][H][dv][dk] fp32, logical layout (from the fp32 copy; from the bf16 one in
 * BF16_SHARED mode). The state is the sequence's at position `folded` only when
 * h = 0: a sequence with unfolded records is copied anyway and sets
 * REPLAYSSM_DEVERR_STALE (fold it first with replayssm_flush_selected). Indices
 * outside 0..B-1 are skipped and set REPLAYSSM_DEVERR_INDEX. n >= 0. */
int replayssm_snapshot(const replayssm_config* cfg, const replayssm_state* st, int n,
                       const int32_t* seqs, float* dst, void* stream);

/* Starts sequences seqs[0..n) from the states src [n][H][dv][dk] fp32: their
 * checkpoints (every copy the mode keeps; bf16 by round-to-nearest-even) are set
 * from src and their buffers emptied (head = h = p = 0, folded = 0). Indices
 * outside 0..B-1 are skipped and set REPLAYSSM_DEVERR_INDEX. n >= 0. */
int replayssm_restore(const replayssm_config* cfg, const replayssm_state* st, int n,
                      const int32_t* seqs, const float* src, void* stream);

/* The same two calls fused with the append that precedes them, in one launch
 * (the new records are read from the inputs and written to the ring by the
 * kernel that replays them, which saves the append launch and the re-read of
 * the records). Semantics are exactly replayssm_append followed by the
 * unfused call; p must be 0 on entry (else the sequence is skipped and
 * flagged REPLAYSSM_DEVERR_PENDING).
 *   decode_step: alpha, beta [B][H]; k, q [B][H][dk]; v [B][H][dv]; out [B][H][dv]
 *   verify_step: alpha, beta [B][T][H]; k, q [B][T][H][dk]; v [B][T][H][dv];
 *                out [B][T][H][dv]; afterwards p = T (accept follows). */
int replayssm_decode_step(const replayssm_config* cfg, const replayssm_state* st, const float* alpha,
                          const float* k, const float* v, const float* beta, const float* q, float* out,
                          void* stream);
int replayssm_verify_step(const replayssm_config* cfg, const replayssm_state* st, int T, const float* alpha,
                          const float* k, const float* v, const float* beta, const float* q, float* out,
                          void* stream);

/* ---- eager comparison kernels -------------------------------------------- */

/* The conventional decode step the method is measured against ("What it
 * claims": a conventional step loads and also stores the whole state, where
 * attention only loads its KV cache): for every
 * (sequence, head) load S, S <- alpha S + v k^T (GDN: the gated delta rule),
 * o = S q, store S. S uses the private fp32 layout (replayssm_pack_state).
 *   alpha, beta [B][H]; k, q [B][H][dk]; v [B][H][dv]; out [B][H][dv].
 * cfg->precision must be REPLAYSSM_FP32. */
int replayssm_eager_step(const replayssm_config* cfg, float* S, const float* alpha,
                         const float* k, const float* v, const float* beta, const float* q,
                         float* out, void* stream);

/* Eager speculative verification with one stored state per draft, as a
 * conventional engine does to be able to roll back (the thread's post [3/N]):
 * pool [B][H][T+1][dv*dk] private fp32 layout, slot [B] int32 selects the
 * committed state of each sequence. Draft i = 1..T is applied in order, its
 * state is stored to slot (slot + i) mod (T+1), and o_i = S_i q_i.
 *   alpha, beta [B][T][H]; k, q [B][T][H][dk]; v [B][T][H][dv]; out [B][T][H][dv]. */
int replayssm_eager_verify(const replayssm_config* cfg, float* pool, const int32_t* slot,
                           int T, const float* alpha, const float* k, const float* v,
                           const float* beta, const float* q, float* out, void* stream);

/* Commits the accepted draft's stored state: slot[b] = (slot[b] + a[b]) mod (T+1).
 * a is clamped to 0..T. */
int replayssm_eager_accept(const replayssm_config* cfg, int32_t* slot, const int32_t* accepted,
                           int T, void* stream);

/* ---- the convolution on the input side, kept as an input ring ------------
 * Mamba-2 passes the input projection's D channels (x, and the B and C that
 * become k and q) through a short causal depthwise convolution of width W with
 * a bias and SiLU before the state-space step:
 *     y_t[c] = act(bias[c] + sum_{j<W} w[c][j] x_{t-W+1+j}[c]),  x_s = 0 for s < 0.
 * The pages leave this neighbouring step open; taken the ReplaySSM way ("How it
 * works": cache the inputs, not the state; Speculative decoding: acceptance
 * moves a pointer), its state is its last W - 1 inputs, kept in a ring of
 * capacity Cc = W - 1 + T_max per sequence. A step appends T inputs after the
 * window and computes each one's output from the window that ends at it;
 * accepting a drafts moves the window's start by a; rejected inputs are
 * overwritten by the next step.
 *   W 1..4, D a multiple of 4, 1 <= T_max <= 8, B 1..65535.
 * State (caller-owned device memory, 16-byte aligned):
 *   ring  float [B][Cc][D] (row-major, callers may read it); start, pend, arrive
 *   int32 [B] (window start slot, pending inputs, library scratch); err int32 [1]. */
typedef struct replayssm_conv_config {
  int32_t B;
  int32_t D;
  int32_t W;
  int32_t T_max;
} replayssm_conv_config;

typedef struct replayssm_conv_state {
  float* ring;
  int32_t* start;
  int32_t* pend;
  int32_t* arrive;
  int32_t* err;
} replayssm_conv_state;

/* Validates cfg; ring bytes (B * Cc * D * 4) and bytes of each int32 [B] array. Host only. */
int replayssm_conv_sizes(const replayssm_conv_config* cfg, int64_t* ring_bytes, int64_t* ptr_bytes);

/* Zero window (x_s = 0 before the first token), start = pend = 0, err = 0. */
int replayssm_conv_init(const replayssm_conv_config* cfg, const replayssm_conv_state* st, void* stream);

/* Appends T inputs x [B][T][D] per sequence and writes y [B][T][D]: output i
 * from the window ending at input i. w [D][W] (PyTorch's conv1d weight
 * [D][1][W] squeezed), bias [D] or NULL, silu nonzero applies SiLU. With commit
 * nonzero the T inputs join the window at once (standard decoding); otherwise
 * they stay pending until replayssm_conv_accept. A sequence with pending inputs
 * is skipped and flagged (REPLAYSSM_DEVERR_PENDING). */
int replayssm_conv_step(const replayssm_conv_config* cfg, const replayssm_conv_state* st, int T,
                        const float* x, const float* w, const float* bias, int silu, int commit,
                        float* y, void* stream);

/* accepted [B] int32 device array: the first a_b pending inputs join the window;
 * a outside 0..pend is clamped and flagged (REPLAYSSM_DEVERR_ACCEPT); pend = 0. */
int replayssm_conv_accept(const replayssm_conv_config* cfg, const replayssm_conv_state* st,
                          const int32_t* accepted, void* stream);

/* ---- Kernel tiling (no effect on results) ----------------------------------------------
 * How the replay kernel (decode, verify, flush and the fused steps) maps the checkpoint onto
 * wavefronts when dk = 128, T_max <= 4 and dv is a multiple of 32: one 16-row tile
 * per wavefront, or two (half as many wavefronts per (sequence, head), more heads in flight
 * per compute unit). Both give the same bits in every output, copy and ring; the choice only
 * changes speed. REPLAYSSM_TILES_AUTO (the default) takes two tiles once a call has at least
 * 64 (dv < 128), 6 (dv >= 128) or 3 (dv >= 128, Gated DeltaNet with the two-precision
 * checkpoint) (sequence, head) items per compute unit of the current device, where their
 * throughput was measured higher, and one tile for smaller batches, whose latency one tile
 * keeps lower; and only where two tiles fit more workgroups on a compute unit than one (long
 * windows, whose record staging in LDS holds both to the same count, take one tile).
 * Process-wide; takes effect at the next launch. EINVAL for another value. */
#define REPLAYSSM_TILES_AUTO 0
#define REPLAYSSM_TILES_ONE 1
#define REPLAYSSM_TILES_TWO 2
int replayssm_set_tiling(int policy);
/* The current policy (one of the values above). */
int replayssm_get_tiling(void);

/* ---- Measurement helper (not a step of the method) -------------------------------------
 * Reads `bytes` bytes at device address `src` once, in the access pattern of the replay
 * kernel's checkpoint stream (persistent workgroups, 32 KiB per workgroup per pass, 16-byte
 * non-temporal loads), and discards them. Timing it gives the practical HBM read ceiling
 * the decode kernel's bandwidth is set beside. `src` must be 16-byte aligned and `bytes` a
 * positive multiple of 16; `sink` is a device float that is written only in the
 * (practically impossible) case that the loaded values sum to one specific NaN pattern.
 * Enqueued on `stream`; EINVAL on bad arguments, EHIP on a launch failure. */
int replayssm_probe_read(const void* src, int64_t bytes, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* REPLAYSSM_H */
