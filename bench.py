"""Benchmark of the ReplaySSM decode path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--quick] [--sweep]
                    [--window-sweep] [--flush-only] [--leg NAME]

A step of the headline workload is one standard decoding step of a Mamba-2 SSM
layer at B=256, H=128, P=64, N=128 (4 MiB fp32 state per sequence), L=16:
replayssm_append of the new token's record followed by replayssm_decode (which
folds the window into the checkpoint every 16th step). Inputs are seeded
synthetic tensors generated on the GPU before the timed region (a pool of
distinct steps, cycled when K + W exceeds it). Prints one JSON line:

  value      tokens/s of the whole step (B tokens per step), HIP-event timed over
             K steps after W warm-up steps, inputs already resident in HBM; a step
             is replayssm_append of the token's record, then replayssm_decode
  roofline   the decode kernel (the dominant one): algorithmic bytes per launch
             (checkpoint read, h+1 records, q, output, checkpoint write on fold
             steps) / its average launch duration, both measured live in a second
             pass with events around each launch, against 8 TB/s
  fused      the same step as one replayssm_decode_step launch
  decode_from_dt  the step with replayssm_append_dt (decay computed from the raw time step)
  eager      the conventional kernel that loads and stores the state every step
  flush      standalone replayssm_flush launches (16 records folded per head): HBM rate and
             MFMA rate against the fp32 matrix peak
  conv_input_ring  the input-side short convolution kept as an input ring (replayssm_conv_step)
             at the layer's 40,960 channels, width 4: standard steps and T=4 rounds
  workloads  speculative verify (T=4), Gated DeltaNet, two-precision checkpoint (with its
             small-batch rounds, B in {1, 32}, launched eagerly and replayed from a HIP graph);
             with --sweep the two-precision batch sweep B in {1, 32, 256, 512},
             each warm (one layer) and rotated (rounds cycle over layer instances
             holding >= 2 GiB of state, so the on-package cache cannot hold it)
  drift      output drift of the bf16-read checkpoints (two-precision and shared bf16) against
             an fp32-checkpoint layer on the same inputs: 1024 T=4 rounds at B=256, and the
             batch sweep B in {1, 32, 512}; per-head and per-token max and 99.9th percentile
  window_sweep  with --window-sweep: L in {4..64} x T in {1, 4, 8} at the headline shape
  ceilings   practical HBM ceilings measured on the device: a read-only probe in
             the checkpoint stream's access pattern, and a device-to-device copy
  cpu_baseline  the CPU oracle (fp32 eager recurrence, OpenMP over heads) on the
             headline workload at full shape, all cores: up to 32 timed decode steps on
             their own inputs; also on one core, in fp64, and on the Gated DeltaNet and
             KDA workloads
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SSM-layer decode tokens/sec at B=256 (+ achieved HBM GB/s vs MI355X peak)"
HBM_PEAK_GBS = 8000.0
MFMA_F32_PEAK_TFLOPS = 157.3  # dense fp32 matrix-core peak of MI355X
POOL_BYTES_MAX = 8 << 30


PMC_SUMMARY = os.path.join(ROOT, "profiles", "replay_kernel_mamba2_decode_b256_pmc.md")
KERNEL_SOURCES = ["ssm_decode_amd/csrc/replay.hip", "ssm_decode_amd/csrc/device.hpp",
                  "ssm_decode_amd/csrc/internal.hpp", "ssm_decode_amd/csrc/route.hpp"]


def counter_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter summary, or None when the
    kernel sources have changed since the counters were taken."""
    import hashlib

    try:
        text = open(PMC_SUMMARY).read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        if ":" in line and line.strip().split(":")[0] in ("traffic_bytes_per_launch", "kernel_sources_sha16"):
            k, v = line.strip().split(":", 1)
            vals[k] = v.strip()
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if vals.get("kernel_sources_sha16") != h.hexdigest()[:16] or "traffic_bytes_per_launch" not in vals:
        return None
    return float(vals["traffic_bytes_per_launch"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--workload", default="mamba2_decode_b256")
    ap.add_argument("--quick", action="store_true", help="headline workload only (no extras, no CPU baseline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-drift", action="store_true", help="skip the drift leg (1024-round comparisons)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="timed oracle seconds of the CPU baseline (each further figure under `more` a quarter)")
    ap.add_argument("--sweep", action="store_true", help="also run the batch sweep of the two-precision layer")
    ap.add_argument("--window-sweep", action="store_true", help="also run the window-size sweep L x T")
    ap.add_argument("--leg", choices=sorted(LEGS),
                    help="run one benchmark leg only and print its figures (for profiling)")
    ap.add_argument("--flush-only", action="store_true",
                    help="only the standalone flush leg (replayssm_flush folding L records per head); for profiling")
    return ap.parse_args()


# ----------------------------------------------------------------------------
# byte model (algorithmic bytes: what the method must move, per head)
# ----------------------------------------------------------------------------

def delta_rule(kind):
    """Kinds whose records carry a beta and whose drafts' corrections u replace v in the ring."""
    return kind in ("gdn", "kda")


def record_bytes(kind, P, N):
    gate = 4 * N if kind == "kda" else 4  # a gate row per record for KDA, else one scalar
    return gate + 4 * N + 4 * P + (4 if delta_rule(kind) else 0)


def ckpt_read_bytes(precision, P, N, fold):
    if precision == "fp32" or (precision == "fp32_hp_bf16_lp" and fold):
        return 4 * P * N
    return 2 * P * N


def ckpt_write_bytes(precision, P, N):
    return {"fp32": 4 * P * N, "fp32_hp_bf16_lp": 6 * P * N, "bf16_shared": 2 * P * N}[precision]


def replay_launch_bytes(kind, precision, P, N, h, T, fold, fused=False):
    """Bytes one head moves in one decode/verify launch with h committed records before it.

    A fused launch (append + decode / verify) also writes the drafts' records to the ring
    (k, alpha and v for Mamba-2; k, alpha and beta for GDN and KDA, whose u is counted below)."""
    b = ckpt_read_bytes(precision, P, N, fold)
    b += (h + T) * record_bytes(kind, P, N)  # committed records and the drafts' own records
    if fused:
        b += T * (record_bytes(kind, P, N) - (4 * P if delta_rule(kind) else 0))
    b += T * 4 * N + T * 4 * P  # q in, o out
    if delta_rule(kind):
        b += T * 4 * P  # u written back into the ring
    if fold:
        b += ckpt_write_bytes(precision, P, N)
    if kind == "gdn" and precision == "fp32_hp_bf16_lp":
        if fold:
            b += h * (4 * P + 4)  # the folded records' raw v and beta, to recompute their u
        if fused:
            b += T * 4 * P  # the drafts' raw v kept for the fold
    return b


def append_bytes(kind, P, N, T, precision="fp32"):
    extra = T * 4 * P if (kind == "gdn" and precision == "fp32_hp_bf16_lp") else 0  # raw v copy
    return 2 * T * record_bytes(kind, P, N) + extra  # read the inputs, write the ring


def eager_bytes(kind, P, N, T, snapshots):
    # load the state once, store it after every draft (snapshots) or once, plus inputs and outputs
    stores = T if snapshots else 1
    per_tok = record_bytes(kind, P, N) + 4 * N + 4 * P  # alpha, k, v (, beta), q, out
    return 4 * P * N * (1 + stores) + T * per_tok


# ----------------------------------------------------------------------------

class Timer:
    def __init__(self, torch):
        self.torch = torch

    def __enter__(self):
        self.torch.cuda.synchronize()
        self.e0 = self.torch.cuda.Event(enable_timing=True)
        self.e1 = self.torch.cuda.Event(enable_timing=True)
        self.e0.record()
        return self

    def __exit__(self, *a):
        self.e1.record()
        self.torch.cuda.synchronize()
        self.ms = self.e0.elapsed_time(self.e1)


def make_pool(torch, synth, shape, T, n_needed, seed, wid, bytes_per_set):
    n = int(max(1, min(n_needed, POOL_BYTES_MAX // max(bytes_per_set, 1))))
    return [synth.device_step(seed, wid, 1000 + i, shape, T, "cuda") for i in range(n)]


def run_standard_decode(torch, rs, synth, w, steps, warmup, seed, kernel_pass=True, fused=True, precision=None,
                        from_dt=False):
    """Standard-decoding steps (fused append + decode launches, or append then decode). With from_dt
    the append is replayssm_append_dt (each record's decay computed from its raw time step)."""
    sh = w.shape
    prec = precision or w.precision
    cfg = rs.make_config(sh.kind, prec, sh.B, sh.H, sh.P, sh.N, w.L, 1)
    layer = rs.LayerState(cfg)
    layer.import_state(synth.device_initial_state(seed, w.wid, sh, w.s0_sigma, "cuda"))
    rb = record_bytes(sh.kind, sh.P, sh.N)
    pool = make_pool(torch, synth, sh, 1, steps + warmup, seed, w.wid, sh.B * sh.H * (rb + 4 * (sh.N + sh.P)))
    if from_dt:
        A, bias = synth.device_decay_params(seed, w.wid, sh, "cuda")
        for i, x in enumerate(pool):
            x["dt"] = synth.device_time_steps(seed, w.wid, 1000 + i, sh, 1, "cuda")
    out = torch.empty((sh.B, sh.H, sh.P), dtype=torch.float32, device="cuda")
    st, stream = layer.struct, torch.cuda.current_stream()

    def step(i):
        x = pool[i % len(pool)]
        if fused:
            rs.decode_step(cfg, st, x["alpha"], x["k"], x["v"], x.get("beta"), x["q"], out, stream)
        else:
            if from_dt:
                rs.append_dt(cfg, st, 1, x["dt"], A, bias, x["k"], x["v"], x.get("beta"), stream)
            else:
                rs.append(cfg, st, 1, x["alpha"], x["k"], x["v"], x.get("beta"), stream)
            rs.decode(cfg, st, x["q"], out, stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    h0 = int(layer.h[0].item())
    with Timer(torch) as tm:
        for i in range(steps):
            step(warmup + i)
    # exact byte count of the timed steps from the pointer rule (all sequences move in step)
    h, kbytes, nfold = h0, 0, 0
    for _ in range(steps):
        fold = h + 1 > w.L
        kbytes += replay_launch_bytes(sh.kind, prec, sh.P, sh.N, h, 1, fold, fused)
        nfold += fold
        h = 1 if fold else h + 1
    res = {"ms": tm.ms, "steps": steps, "tokens": sh.B * steps, "decode_bytes": kbytes * sh.B * sh.H,
           "append_bytes": 0 if fused else append_bytes(sh.kind, sh.P, sh.N, 1, prec) * sh.B * sh.H * steps,
           "folds": nfold, "fused": fused}
    if kernel_pass:
        # second pass: events around every decode launch (same stream as the kernels)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        h1 = int(layer.h[0].item())
        for i in range(steps):
            x = pool[(warmup + steps + i) % len(pool)]
            if fused:
                evs[i][0].record(stream)
                rs.decode_step(cfg, st, x["alpha"], x["k"], x["v"], x.get("beta"), x["q"], out, stream)
                evs[i][1].record(stream)
            else:
                if from_dt:
                    rs.append_dt(cfg, st, 1, x["dt"], A, bias, x["k"], x["v"], x.get("beta"), stream)
                else:
                    rs.append(cfg, st, 1, x["alpha"], x["k"], x["v"], x.get("beta"), stream)
                evs[i][0].record(stream)
                rs.decode(cfg, st, x["q"], out, stream)
                evs[i][1].record(stream)
        torch.cuda.synchronize()
        durs = np.array([a.elapsed_time(b) for a, b in evs])
        h, kb, fold_ms, plain_ms, fold_b, plain_b = h1, 0, [], [], 0, 0
        for i in range(steps):
            fold = h + 1 > w.L
            bb = replay_launch_bytes(sh.kind, prec, sh.P, sh.N, h, 1, fold, fused) * sh.B * sh.H
            kb += bb
            (fold_ms if fold else plain_ms).append(durs[i])
            if fold:
                fold_b += bb
            else:
                plain_b += bb
            h = 1 if fold else h + 1
        by_h = {}
        hh = h1
        for i in range(steps):
            by_h.setdefault(hh, []).append(durs[i] * 1e3)
            hh = 1 if hh + 1 > w.L else hh + 1
        res["us_by_h"] = {int(k): round(float(np.mean(v)), 1) for k, v in sorted(by_h.items())}
        # Steady state: the timed window's decode launches replaced by one whole L-step cycle's
        # (h = 1..L before the step; the append's cost does not depend on h). Both figures come
        # from the same event-timed launches, so their event overhead cancels.
        t_of_h = {k: float(np.mean(v)) for k, v in by_h.items()}
        cycle = list(range(1, w.L + 1))
        if all(hh in t_of_h for hh in cycle):
            hh, timed = h0, []
            for _ in range(steps):
                timed.append(t_of_h.get(hh, np.nan))
                hh = 1 if hh + 1 > w.L else hh + 1
            if not np.isnan(timed).any():
                ms_step = tm.ms / steps - np.mean(timed) * 1e-3 + np.mean([t_of_h[c] for c in cycle]) * 1e-3
                res["steady_ms_per_step"] = ms_step
                res["steady_tokens_per_s"] = sh.B / (ms_step * 1e-3)
        res.update({"kernel_ms_total": float(durs.sum()), "kernel_launches": steps, "kernel_bytes": kb,
                    "kernel_avg_us": float(durs.mean() * 1e3),
                    "fold_avg_us": float(np.mean(fold_ms) * 1e3) if fold_ms else None,
                    "plain_avg_us": float(np.mean(plain_ms) * 1e3) if plain_ms else None,
                    "fold_gbs": fold_b / (np.sum(fold_ms) * 1e6) if fold_ms else None,
                    "plain_gbs": plain_b / (np.sum(plain_ms) * 1e6) if plain_ms else None})
    err = rs.read_error(st)
    if err:
        raise RuntimeError(f"device error word {err}")
    del layer, pool
    return res


def run_spec(torch, rs, synth, w, rounds, warmup, seed, precision=None, B=None, kernel_pass=True, fused=True,
             rotate_bytes=0):
    """Speculative rounds (verify T drafts, then accept). With rotate_bytes > 0 the rounds cycle over
    enough independent layer instances to hold that many bytes of state, as the layers of a model
    do, so that consecutive rounds do not find their state in the on-package cache."""
    sh = w.shape
    if B is not None:
        sh = synth.LayerShape(sh.kind, B, sh.H, sh.P, sh.N)
    prec = precision or w.precision
    T = w.T if w.T > 1 else int(w.extra.get("spec_T", 4))
    cfg = rs.make_config(sh.kind, prec, sh.B, sh.H, sh.P, sh.N, w.L, T)
    S0 = synth.device_initial_state(seed, w.wid, sh, w.s0_sigma, "cuda")
    lays = [rs.LayerState(cfg)]
    footprint = sum(t.numel() * t.element_size() for t in lays[0].tensors())
    layers = max(1, -(-int(rotate_bytes) // footprint))
    lays += [rs.LayerState(cfg) for _ in range(layers - 1)]
    for lay in lays:
        lay.import_state(S0)
    del S0
    rb = record_bytes(sh.kind, sh.P, sh.N)
    n = warmup + 2 * rounds  # both timed passes get their own acceptance draws
    pool = make_pool(torch, synth, sh, T, n, seed, w.wid, sh.B * sh.H * T * (rb + 4 * (sh.N + sh.P)))
    accs = [synth.device_accept(seed, w.wid, r, sh.B, T, "cuda") for r in range(n)]
    acc_host = [a.cpu().numpy() for a in accs]
    out = torch.empty((sh.B, T, sh.H, sh.P), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def rnd(i, evs=None):
        x = pool[i % len(pool)]
        st = lays[i % layers].struct
        if not fused:
            rs.append(cfg, st, T, x["alpha"], x["k"], x["v"], x.get("beta"), stream)
        if evs is not None:
            evs[0].record(stream)
        if fused:
            rs.verify_step(cfg, st, T, x["alpha"], x["k"], x["v"], x.get("beta"), x["q"], out, stream)
        else:
            rs.verify(cfg, st, T, x["q"], out, stream)
        if evs is not None:
            evs[1].record(stream)
        rs.accept(cfg, st, accs[i], stream)

    def launch_bytes(h, first):
        """Algorithmic bytes of rounds first.. with per-layer h arrays advanced in place."""
        fold = h + T > w.L
        kb = 0
        for f in (False, True):
            m = fold == f
            if m.any():
                kb += sum(replay_launch_bytes(sh.kind, prec, sh.P, sh.N, int(hh), T, f, fused) for hh in h[m]) * sh.H
        return kb, np.where(fold, 0, h) + acc_host[first]

    for i in range(warmup):
        rnd(i)
    torch.cuda.synchronize()
    hs = [lay.h.cpu().numpy().astype(np.int64) for lay in lays]
    with Timer(torch) as tm:
        for i in range(rounds):
            rnd(warmup + i)
    accepted = int(sum(acc_host[warmup + i].sum() for i in range(rounds)))
    kb = 0
    for i in range(rounds):
        b, hs[(warmup + i) % layers] = launch_bytes(hs[(warmup + i) % layers], warmup + i)
        kb += b
    res = {"ms": tm.ms, "rounds": rounds, "accepted_tokens": accepted, "drafts": sh.B * T * rounds,
           "verify_bytes": int(kb), "layers": layers, "layer_footprint_MiB": footprint / 2**20}
    if kernel_pass:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(rounds)]
        torch.cuda.synchronize()
        hs = [lay.h.cpu().numpy().astype(np.int64) for lay in lays]
        base = warmup + rounds
        for i in range(rounds):
            rnd(base + i, evs[i])
        torch.cuda.synchronize()
        durs = np.array([a.elapsed_time(b) for a, b in evs])
        kb2 = 0
        for i in range(rounds):
            b, hs[(base + i) % layers] = launch_bytes(hs[(base + i) % layers], base + i)
            kb2 += b
        res.update({"kernel_avg_us": float(durs.mean() * 1e3), "kernel_gbs": kb2 / (durs.sum() * 1e6)})
    for lay in lays:
        err = rs.read_error(lay.struct)
        if err:
            raise RuntimeError(f"device error word {err}")
    return res


def run_drift(torch, rs, synth, w, B, rounds, seed):
    """Output drift of the two bf16-read checkpoints over `rounds` speculative rounds (fused append +
    verify of T drafts, accepted prefix ~ U{0..T}): the two-precision layer (bf16 copy read off-fold)
    and the shared-bf16 layer run beside an fp32-checkpoint layer on identical inputs, and every
    draft output of every sequence and head is compared with the fp32 layer's (which the parity
    tests hold within 1e-4 of the fp64 oracle per head). Per head: max|o - o_fp32| / max|o_fp32|
    over the head's output vector; per token: the same over the token's whole layer output (all
    heads). Reported: max and 99.9th percentile over all vectors."""
    sh = synth.LayerShape(w.shape.kind, B, w.shape.H, w.shape.P, w.shape.N)
    T = w.T
    modes = ("fp32", "fp32_hp_bf16_lp", "bf16_shared")
    S0 = synth.device_initial_state(seed, w.wid, sh, w.s0_sigma, "cuda")
    cfgs = {m: rs.make_config(sh.kind, m, sh.B, sh.H, sh.P, sh.N, w.L, T) for m in modes}
    lays = {m: rs.LayerState(cfgs[m]) for m in modes}
    for m in modes:
        lays[m].import_state(S0)
    del S0
    outs = {m: torch.empty((sh.B, T, sh.H, sh.P), dtype=torch.float32, device="cuda") for m in modes}
    head = {m: torch.empty((rounds, sh.B, T, sh.H), dtype=torch.float32, device="cuda") for m in modes[1:]}
    tok = {m: torch.empty((rounds, sh.B, T), dtype=torch.float32, device="cuda") for m in modes[1:]}
    wid = w.wid + 7000
    for r in range(rounds):
        x = synth.device_step(seed, wid, r, sh, T, "cuda")
        acc = synth.device_accept(seed, wid, r, sh.B, T, "cuda")
        for m in modes:
            st = lays[m].struct
            rs.verify_step(cfgs[m], st, T, x["alpha"], x["k"], x["v"], x.get("beta"), x["q"], outs[m])
            rs.accept(cfgs[m], st, acc)
        ref = outs["fp32"]
        den_h = ref.abs().amax(-1).clamp_min(1e-30)
        den_t = ref.abs().amax((2, 3)).clamp_min(1e-30)
        for m in modes[1:]:
            d = (outs[m] - ref).abs()
            head[m][r] = d.amax(-1) / den_h
            tok[m][r] = d.amax((2, 3)) / den_t
    torch.cuda.synchronize()
    for m in modes:
        err = rs.read_error(lays[m].struct)
        if err:
            raise RuntimeError(f"device error word {err} ({m})")

    def stats(x):
        x = x.flatten()
        k = max(1, x.numel() // 1000)
        return {"max": float(x.max().item()), "p99_9": float(torch.topk(x, k).values.min().item()),
                "vectors": int(x.numel())}

    res = {"B": B, "rounds": rounds, "T": T, "L": w.L, "reference": "fp32-checkpoint layer on the same inputs"}
    for m in modes[1:]:
        res[m] = {"per_head": stats(head[m]), "per_token": stats(tok[m])}
    del lays, outs, head, tok
    torch.cuda.empty_cache()
    return res


def flush_launch_bytes(kind, precision, P, N, h):
    """Bytes one head moves in a replayssm_flush launch that folds h committed records: the
    checkpoint copy the fold reads, the h records, and the checkpoint copies it writes."""
    b = ckpt_read_bytes(precision, P, N, True) + h * record_bytes(kind, P, N) + ckpt_write_bytes(precision, P, N)
    # GDN with the two-precision checkpoint stages the raw v rows and beta (to recompute the
    # corrections) in place of the stored u; every other delta-rule fold stages no beta
    if delta_rule(kind) and not (kind == "gdn" and precision == "fp32_hp_bf16_lp"):
        b -= h * 4
    return b


def run_flush(torch, rs, synth, w, cycles, warmup, seed, precision=None):
    """Standalone checkpoint folds: every cycle is L standard decoding steps (append + decode; the
    window fills without a fold) followed by one replayssm_flush, which folds all L committed
    records of every sequence (rank-L update per head). Only the flush launches are timed, with
    events on the kernels' stream."""
    sh = w.shape
    prec = precision or w.precision
    cfg = rs.make_config(sh.kind, prec, sh.B, sh.H, sh.P, sh.N, w.L, 1)
    layer = rs.LayerState(cfg)
    layer.import_state(synth.device_initial_state(seed, w.wid, sh, w.s0_sigma, "cuda"))
    rb = record_bytes(sh.kind, sh.P, sh.N)
    pool = make_pool(torch, synth, sh, 1, w.L * 4, seed, w.wid, sh.B * sh.H * (rb + 4 * (sh.N + sh.P)))
    out = torch.empty((sh.B, sh.H, sh.P), dtype=torch.float32, device="cuda")
    st, stream = layer.struct, torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(cycles)]
    n = 0
    for c in range(warmup + cycles):
        for _ in range(w.L):
            x = pool[n % len(pool)]
            n += 1
            rs.append(cfg, st, 1, x["alpha"], x["k"], x["v"], x.get("beta"), stream)
            rs.decode(cfg, st, x["q"], out, stream)
        if c >= warmup:
            evs[c - warmup][0].record(stream)
        rs.flush(cfg, st, stream)
        if c >= warmup:
            evs[c - warmup][1].record(stream)
    torch.cuda.synchronize()
    h = int(layer.h[0].item())
    err = rs.read_error(st)
    if err:
        raise RuntimeError(f"device error word {err}")
    if h != 0:
        raise RuntimeError(f"flush left h = {h}")
    durs = np.array([a.elapsed_time(b) for a, b in evs])
    us = float(durs.mean() * 1e3)
    nbytes = flush_launch_bytes(sh.kind, prec, sh.P, sh.N, w.L) * sh.B * sh.H
    flops = 2 * sh.P * sh.N * w.L * sh.B * sh.H  # V diag(gamma) K^T over the L folded records
    del layer, pool
    return {"launches": cycles, "records_folded_per_head": w.L, "avg_us": us, "min_us": float(durs.min() * 1e3),
            "bytes_per_launch": nbytes, "gbs": nbytes / (us * 1e3), "hbm_frac": nbytes / (us * 1e3) / HBM_PEAK_GBS,
            "flops_per_launch": flops, "tflops": flops / (us * 1e6),
            "mfma_frac": flops / (us * 1e6) / MFMA_F32_PEAK_TFLOPS, "precision": prec}


def run_spec_graph(torch, rs, synth, w, B, K, reps, seed, precision=None):
    """Small-batch speculative rounds, eager against HIP-graph replay: K rounds (fused append +
    verify, then accept) captured once with torch.cuda.CUDAGraph around the library's calls and
    replayed `reps` times, against the same K rounds launched eagerly `reps` times."""
    sh = synth.LayerShape(w.shape.kind, B, w.shape.H, w.shape.P, w.shape.N)
    prec = precision or w.precision
    T = w.T if w.T > 1 else int(w.extra.get("spec_T", 4))
    cfg = rs.make_config(sh.kind, prec, sh.B, sh.H, sh.P, sh.N, w.L, T)
    layer = rs.LayerState(cfg)
    layer.import_state(synth.device_initial_state(seed, w.wid, sh, w.s0_sigma, "cuda"))
    xs = [synth.device_step(seed, w.wid, 3000 + r, sh, T, "cuda") for r in range(K)]
    accs = [synth.device_accept(seed, w.wid, 3000 + r, sh.B, T, "cuda") for r in range(K)]
    outs = [torch.empty((sh.B, T, sh.H, sh.P), dtype=torch.float32, device="cuda") for _ in range(K)]
    accepted = int(sum(int(a.sum().item()) for a in accs))

    def rounds():
        for r in range(K):
            x = xs[r]
            rs.verify_step(cfg, layer.struct, T, x["alpha"], x["k"], x["v"], x.get("beta"), x["q"], outs[r])
            rs.accept(cfg, layer.struct, accs[r])

    for _ in range(2):
        rounds()
    with Timer(torch) as te:
        for _ in range(reps):
            rounds()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        rounds()
    graph.replay()
    with Timer(torch) as tg:
        for _ in range(reps):
            graph.replay()
    err = rs.read_error(layer.struct)
    if err:
        raise RuntimeError(f"device error word {err}")
    n = reps * K
    return {"B": B, "T": T, "precision": prec, "rounds_per_graph": K,
            "eager_us_per_round": te.ms * 1e3 / n, "graph_us_per_round": tg.ms * 1e3 / n,
            "eager_accepted_tokens_per_s": reps * accepted / (te.ms * 1e-3),
            "graph_accepted_tokens_per_s": reps * accepted / (tg.ms * 1e-3)}


def conv_launch_bytes(D, W, T):
    """Bytes one sequence moves in a conv step: the W - 1 window inputs read, the T inputs read and
    written to the ring, the T outputs written (weights and bias, shared by all sequences, aside)."""
    return 4 * D * ((W - 1) + 3 * T)


def run_conv(torch, rs, synth, B, D, W, T, steps, warmup, seed, wid=20):
    """The input-side convolution ring at a Mamba-2 layer's channel count: T = 1 steps commit
    their input at once; T > 1 rounds leave the drafts pending and accept a prefix ~ U{0..T}.
    Events around every step launch give the kernel's time."""
    cfg = rs.make_conv_config(B, D, W, T)
    layer = rs.ConvLayer(cfg)
    wh, bh = synth.host_conv_params(seed, wid, D, W)
    w, b = torch.from_numpy(wh).cuda(), torch.from_numpy(bh).cuda()
    n = int(max(2, min(8, (1 << 30) // (B * T * D * 4))))
    xs = [synth.device_conv_inputs(seed, wid, i, B, T, D, "cuda") for i in range(n)]
    accs = [synth.device_accept(seed, wid, i, B, T, "cuda") for i in range(n)]
    y = torch.empty((B, T, D), dtype=torch.float32, device="cuda")
    st, stream = layer.struct, torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(warmup + steps):
        if i >= warmup:
            evs[i - warmup][0].record(stream)
        rs.conv_step(cfg, st, T, xs[i % n], w, b, True, T == 1, y, stream)
        if i >= warmup:
            evs[i - warmup][1].record(stream)
        if T > 1:
            rs.conv_accept(cfg, st, accs[i % n], stream)
    torch.cuda.synchronize()
    if int(layer.err[0].item()):
        raise RuntimeError(f"conv error word {int(layer.err[0].item())}")
    us = float(np.mean([a.elapsed_time(e) for a, e in evs]) * 1e3)
    nbytes = conv_launch_bytes(D, W, T) * B
    return {"B": B, "D": D, "W": W, "T": T, "step_us": us, "bytes_per_launch": nbytes, "gbs": nbytes / (us * 1e3),
            "hbm_frac": nbytes / (us * 1e3) / HBM_PEAK_GBS}


def run_eager(torch, rs, synth, w, steps, warmup, seed, T=1):
    sh = w.shape
    cfg = rs.make_config(sh.kind, "fp32", sh.B, sh.H, sh.P, sh.N, w.L, T)
    nslots = 1 if T == 1 else T + 1
    S = torch.empty((sh.B, sh.H, nslots, sh.P * sh.N), dtype=torch.float32, device="cuda")
    S0 = synth.device_initial_state(seed, w.wid, sh, w.s0_sigma, "cuda")
    packed = torch.empty((sh.B, sh.H, sh.P * sh.N), dtype=torch.float32, device="cuda")
    rs.pack_state(cfg, S0, packed, None)
    S[:, :, 0].copy_(packed)
    del S0, packed
    rb = record_bytes(sh.kind, sh.P, sh.N)
    pool = make_pool(torch, synth, sh, T, steps + warmup, seed, w.wid, sh.B * sh.H * T * (rb + 4 * (sh.N + sh.P)))
    out = torch.empty((sh.B, T, sh.H, sh.P), dtype=torch.float32, device="cuda")
    slot = torch.zeros(sh.B, dtype=torch.int32, device="cuda")
    acc = torch.full((sh.B,), T, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        x = pool[i % len(pool)]
        if T == 1:
            rs.eager_step(cfg, S, x["alpha"], x["k"], x["v"], x.get("beta"), x["q"], out, stream)
        else:
            rs.eager_verify(cfg, S, slot, T, x["alpha"], x["k"], x["v"], x.get("beta"), x["q"], out, stream)
            rs.eager_accept(cfg, slot, acc, T, stream)

    for i in range(warmup):
        step(i)
    with Timer(torch) as tm:
        for i in range(steps):
            step(warmup + i)
    b = eager_bytes(sh.kind, sh.P, sh.N, T, T > 1) * sh.B * sh.H * steps
    return {"ms": tm.ms, "steps": steps, "tokens": sh.B * T * steps, "bytes": b, "gbs": b / (tm.ms * 1e6)}


def window_sweep(torch, rs, synth, seed):
    """Window size L x drafts T at the headline layer shape (B=256, H=128, P=64, N=128, fp32):
    standard decoding (append + decode) for T = 1, verify rounds with accepted prefix ~ U{0..T}
    for T > 1. Per cell: throughput, the replay kernel's bandwidth, and algorithmic bytes per
    (accepted) token, split into checkpoint bytes and the rest."""
    import dataclasses

    base = synth.WORKLOADS["mamba2_spec_b256"]
    sh = base.shape
    cells = {}
    for L in (4, 8, 16, 32, 64):
        for T in (1, 4, 8):
            if T > L:
                continue
            key = f"L{L}_T{T}"
            w = dataclasses.replace(base, L=L, T=T, wid=base.wid + 1000 + 10 * L + T)
            if T == 1:
                r = run_standard_decode(torch, rs, synth, w, max(128, 2 * L), 16, seed, fused=False)
                toks = r["tokens"]
                cells[key] = {"tokens_per_s": toks / (r["ms"] * 1e-3),
                              "kernel_gbs": r["kernel_bytes"] / (r["kernel_ms_total"] * 1e6),
                              "kernel_avg_us": r["kernel_avg_us"],
                              "bytes_per_token": (r["decode_bytes"] + r["append_bytes"]) / toks,
                              "ckpt_bytes_per_token": 4 * sh.P * sh.N * (1 + 1.0 / L) * sh.H}
            else:
                r = run_spec(torch, rs, synth, w, 128, 16, seed, fused=False)
                cells[key] = {"accepted_tokens_per_s": r["accepted_tokens"] / (r["ms"] * 1e-3),
                              "drafts_per_s": r["drafts"] / (r["ms"] * 1e-3),
                              "kernel_gbs": r["kernel_gbs"], "kernel_avg_us": r["kernel_avg_us"],
                              "bytes_per_accepted_token": (r["verify_bytes"] + append_bytes(sh.kind, sh.P, sh.N, T)
                                                           * sh.B * sh.H * r["rounds"]) / max(r["accepted_tokens"], 1)}
    best = {}
    for T in (1, 4, 8):
        vals = {k: v.get("tokens_per_s", v.get("accepted_tokens_per_s")) for k, v in cells.items()
                if isinstance(v, dict) and k.endswith(f"_T{T}")}
        if vals:
            best[f"T{T}"] = max(vals, key=vals.get)
    return {"cells": cells, "best": best, "shape": "Mamba-2 B=256 H=128 P=64 N=128 fp32"}


def ceilings(torch, rs):
    """Practical HBM ceilings of the device: the read probe (the decode kernel's checkpoint access
    pattern, read-only) over 4 GiB, and a 2 GiB device-to-device copy (2 bytes moved per byte)."""
    src = torch.empty(1 << 30, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    src.fill_(1.0)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        rs.probe_read(src, sink, stream)
    reps = 20
    with Timer(torch) as tm:
        for _ in range(reps):
            rs.probe_read(src, sink, stream)
    read = src.numel() * 4 * reps / (tm.ms * 1e6)
    a = src[: 1 << 29]
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    with Timer(torch) as tm:
        for _ in range(reps):
            b.copy_(a)
    copy = 2 * a.numel() * 4 * reps / (tm.ms * 1e6)
    del src, a, b
    torch.cuda.empty_cache()
    return {"read_probe_gbs": read, "d2d_copy_gbs": copy, "unit": "GB/s",
            "read_probe": "replayssm_probe_read over 4 GiB (persistent workgroups, 32 KiB per pass, "
                          "non-temporal 16-byte loads)", "d2d_copy": "torch copy_ of 2 GiB (hipMemcpy D2D)"}


def host_cpu():
    """CPU model and the cores this process may use."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"model": model, "affinity_cores": len(os.sched_getaffinity(0))}


_CPU_INPUTS = {}


def cpu_baseline(synth, w, seed, seconds, threads=None, precision="f32", max_steps=4096, warmup=2, pool=16):
    """The oracle as it stands (the eager recurrence, OpenMP over heads) at the workload's full
    shape: every sequence and head, `warmup` untimed steps, then timed decode steps until
    `seconds` of oracle time are spent (at most `max_steps`). Step t takes the seeded inputs of
    step t mod `pool` (the recurrence's work does not depend on the values); their generation
    is not timed."""
    import oracle

    if threads is not None:
        prev = oracle.num_threads()
        oracle.set_num_threads(threads)
        try:
            return cpu_baseline(synth, w, seed, seconds, precision=precision, max_steps=max_steps, warmup=warmup,
                                pool=pool)
        finally:
            oracle.set_num_threads(prev)

    sh = w.shape
    nh = sh.B * sh.H
    dt = np.float64 if precision == "f64" else np.float32
    S = synth.host_initial_state(seed, w.wid, sh, w.s0_sigma).reshape(nh, sh.P, sh.N).astype(dt)
    acc = np.ones(nh, np.int32)
    steps, spent = 0, 0.0
    for t in range(warmup + max_steps):
        key = (w.name, seed, t % pool)
        if key not in _CPU_INPUTS:  # generated once per pool entry and shared by the runs (not timed)
            x = synth.host_step(seed, w.wid, t % pool, sh, 1)
            _CPU_INPUTS[key] = {k: np.ascontiguousarray(np.swapaxes(v, 1, 2)).reshape(nh, 1, *v.shape[3:])
                                for k, v in x.items()}
        args = _CPU_INPUTS[key]
        t0 = time.perf_counter()
        if sh.kind == "mamba2":
            oracle.mamba2_round(S, args["alpha"].reshape(nh, 1), args["k"], args["v"], args["q"], acc, precision)
        elif sh.kind == "kda":
            oracle.kda_round(S, args["alpha"], args["beta"].reshape(nh, 1), args["k"], args["v"], args["q"], acc,
                             precision)
        else:
            oracle.gdn_round(S, args["alpha"].reshape(nh, 1), args["beta"].reshape(nh, 1), args["k"], args["v"],
                             args["q"], acc, precision)
        if t >= warmup:
            spent += time.perf_counter() - t0
            steps += 1
            if spent >= seconds:
                break
    name = {"f32": "fp32", "f64": "fp64"}[precision]
    return {"value": sh.B * steps / spent, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "host": host_cpu(),
            "sample": f"{w.name} at full shape ({sh.B} sequences x {sh.H} heads, {sh.P}x{sh.N} state), "
                      f"{steps} decode steps after {warmup} warm-up steps (inputs cycling over {pool} seeded "
                      f"steps), {name} eager recurrence, "
                      f"{spent:.1f} s of oracle time (input generation excluded)"}


# Single legs (--leg NAME), each on its own workload: K steps or rounds after W warm-up ones.
LEGS = {
    "mamba2_decode": lambda torch, rs, synth, k, w, seed: run_standard_decode(
        torch, rs, synth, synth.WORKLOADS["mamba2_decode_b256"], k, w, seed, fused=False),
    "mamba2_decode_dt": lambda torch, rs, synth, k, w, seed: run_standard_decode(
        torch, rs, synth, synth.WORKLOADS["mamba2_decode_b256"], k, w, seed, fused=False, from_dt=True),
    "mamba2_decode_fused": lambda torch, rs, synth, k, w, seed: run_standard_decode(
        torch, rs, synth, synth.WORKLOADS["mamba2_decode_b256"], k, w, seed, fused=True),
    "mamba2_spec": lambda torch, rs, synth, k, w, seed: run_spec(
        torch, rs, synth, synth.WORKLOADS["mamba2_spec_b256"], k, w, seed),
    "mamba2_decode_two_precision": lambda torch, rs, synth, k, w, seed: run_standard_decode(
        torch, rs, synth, synth.WORKLOADS["mamba2_decode_b256"], k, w, seed, fused=False,
        precision="fp32_hp_bf16_lp"),
    "mamba2_spec_two_precision": lambda torch, rs, synth, k, w, seed: run_spec(
        torch, rs, synth, synth.WORKLOADS["mamba2_2prec_b256"], k, w, seed, precision="fp32_hp_bf16_lp"),
    "mamba2_spec_bf16_shared": lambda torch, rs, synth, k, w, seed: run_spec(
        torch, rs, synth, synth.WORKLOADS["mamba2_2prec_b256"], k, w, seed, precision="bf16_shared"),
    "gdn_decode": lambda torch, rs, synth, k, w, seed: run_standard_decode(
        torch, rs, synth, synth.WORKLOADS["gdn_decode_b256"], k, w, seed, fused=False),
    "gdn_spec": lambda torch, rs, synth, k, w, seed: run_spec(
        torch, rs, synth, synth.WORKLOADS["gdn_decode_b256"], k, w, seed),
    "gdn_spec_two_precision": lambda torch, rs, synth, k, w, seed: run_spec(
        torch, rs, synth, synth.WORKLOADS["gdn_decode_b256"], k, w, seed, precision="fp32_hp_bf16_lp"),
    "kda_decode": lambda torch, rs, synth, k, w, seed: run_standard_decode(
        torch, rs, synth, synth.WORKLOADS["kda_decode_b256"], k, w, seed, fused=False),
    "conv_decode": lambda torch, rs, synth, k, w, seed: run_conv(torch, rs, synth, 256, 40960, 4, 1, k, w, seed),
    "kda_spec": lambda torch, rs, synth, k, w, seed: run_spec(
        torch, rs, synth, synth.WORKLOADS["kda_decode_b256"], k, w, seed),
    "drift": lambda torch, rs, synth, k, w, seed: {f"B{B}": run_drift(
        torch, rs, synth, synth.WORKLOADS["mamba2_2prec_b256"], B, k, seed) for B in (256, 1, 32, 512)},
}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode path has no cross-GPU step (sequences and heads shard "
              "with no exchange). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch

    import ssm_decode_amd as rs
    import synth

    rs.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = synth.WORKLOADS[args.workload]
    sh = w.shape
    if args.flush_only:
        print(json.dumps({"flush": run_flush(torch, rs, synth, w, 16, 2, args.seed)}), flush=True)
        return
    if args.leg:
        res = LEGS[args.leg](torch, rs, synth, args.steps, args.warmup, args.seed)
        print(json.dumps({"leg": args.leg, **{k: v for k, v in res.items() if not isinstance(v, dict)}}), flush=True)
        return
    main_res = run_standard_decode(torch, rs, synth, w, args.steps, args.warmup, args.seed, fused=False)
    fold_flops = 2 * sh.P * sh.N * w.L * sh.B * sh.H  # V diag(gamma) K^T over the L folded records
    tok_s = main_res["tokens"] / (main_res["ms"] * 1e-3)
    achieved = main_res["kernel_bytes"] / (main_res["kernel_ms_total"] * 1e6)
    line = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms"] / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "kind": sh.kind, "B": sh.B, "H": sh.H, "P": sh.P, "N": sh.N, "L": w.L,
                   "T": 1, "precision": w.precision, "state_MiB_per_seq": sh.H * sh.P * sh.N * 4 / 2**20},
        "roofline": {"bound": "hbm", "kernel": "replay_kernel (decode)", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": counter_traffic(), "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled)",
                     "avg_launch_us": main_res["kernel_avg_us"],
                     "algorithmic_bytes_per_launch": main_res["kernel_bytes"] / main_res["kernel_launches"],
                     "plain_step_us": main_res["plain_avg_us"], "fold_step_us": main_res["fold_avg_us"],
                     "plain_step_gbs": main_res["plain_gbs"], "fold_step_gbs": main_res["fold_gbs"],
                     "us_by_h_before_step": main_res["us_by_h"],
                     "fold_mfma": None if not main_res["fold_avg_us"] else {
                         "tflops": fold_flops / (main_res["fold_avg_us"] * 1e6), "peak": MFMA_F32_PEAK_TFLOPS,
                         "frac": fold_flops / (main_res["fold_avg_us"] * 1e6) / MFMA_F32_PEAK_TFLOPS,
                         "flops_per_fold_step": fold_flops}},
        "step_gbs": (main_res["decode_bytes"] + main_res["append_bytes"]) / (main_res["ms"] * 1e6),
        "step": "replayssm_append then replayssm_decode",
        "steady_state_tokens_per_s": main_res.get("steady_tokens_per_s"),
        "steady_state_ms_per_step": main_res.get("steady_ms_per_step"),
        "steady_state": "the timed K steps with their decode launches replaced by one whole window of "
                        "L steps (h = 1..L before the step, one fold), from the per-h launch times in "
                        "us_by_h_before_step; value itself is the K steps as timed",
    }
    # the other standard-decoding legs time whole windows: a multiple of L steps after a warm-up of
    # L + 1 steps (one fold), so every timed window holds exactly one fold per L steps
    sec_steps = max(w.L, (min(args.steps, 256) // w.L) * w.L)
    sec_warm = w.L + 1
    if not args.quick:
        fu = run_standard_decode(torch, rs, synth, w, sec_steps, sec_warm, args.seed, fused=True)
        line["fused"] = {"tokens_per_s": fu["tokens"] / (fu["ms"] * 1e-3),
                         "kernel_gbs": fu["kernel_bytes"] / (fu["kernel_ms_total"] * 1e6),
                         "kernel_avg_us": fu["kernel_avg_us"], "steps": fu["steps"],
                         "unfused_steady_state_tokens_per_s": main_res.get("steady_tokens_per_s"),
                         "step": "replayssm_decode_step (append + decode in one launch)"}
    if not args.quick:
        tp = run_standard_decode(torch, rs, synth, w, sec_steps, sec_warm, args.seed, fused=False,
                                 precision="fp32_hp_bf16_lp")
        line["two_precision"] = {"tokens_per_s": tp["tokens"] / (tp["ms"] * 1e-3),
                                 "kernel_gbs": tp["kernel_bytes"] / (tp["kernel_ms_total"] * 1e6),
                                 "kernel_avg_us": tp["kernel_avg_us"], "plain_step_us": tp["plain_avg_us"],
                                 "fold_step_us": tp["fold_avg_us"], "steps": tp["steps"],
                                 "step": "replayssm_append then replayssm_decode, bf16 copy read off-fold"}
    if not args.quick:
        dtl = run_standard_decode(torch, rs, synth, w, sec_steps, sec_warm, args.seed, fused=False,
                                  kernel_pass=False, from_dt=True)
        line["decode_from_dt"] = {"tokens_per_s": dtl["tokens"] / (dtl["ms"] * 1e-3),
                                  "ms_per_step": dtl["ms"] / dtl["steps"], "steps": dtl["steps"],
                                  "headline_steady_state_ms_per_step": main_res.get("steady_ms_per_step"),
                                  "step": "replayssm_append_dt (decay from the raw time step) then replayssm_decode"}
    if not args.quick:
        eg = run_eager(torch, rs, synth, w, min(args.steps, 256), 16, args.seed)
        line["eager"] = {"tokens_per_s": eg["tokens"] / (eg["ms"] * 1e-3), "gbs": eg["gbs"],
                         "frac": eg["gbs"] / HBM_PEAK_GBS,
                         "speedup_of_replay": tok_s / (eg["tokens"] / (eg["ms"] * 1e-3)),
                         "state_bytes_per_step_eager": 2 * 4 * sh.P * sh.N,
                         "state_bytes_per_step_replay": 4 * sh.P * sh.N * (1 + 1.0 / w.L)}
        wl = {}
        w2 = synth.WORKLOADS["mamba2_spec_b256"]
        r2 = run_spec(torch, rs, synth, w2, 128, 8, args.seed)
        e2 = run_eager(torch, rs, synth, w2, 64, 4, args.seed, T=w2.T)
        wl[w2.name] = {"accepted_tokens_per_s": r2["accepted_tokens"] / (r2["ms"] * 1e-3),
                       "drafts_per_s": r2["drafts"] / (r2["ms"] * 1e-3),
                       "verify_kernel_gbs": r2["kernel_gbs"], "verify_avg_us": r2["kernel_avg_us"],
                       "eager_snapshot_drafts_per_s": e2["tokens"] / (e2["ms"] * 1e-3), "eager_snapshot_gbs": e2["gbs"]}
        w3 = synth.WORKLOADS["gdn_decode_b256"]
        r3 = run_standard_decode(torch, rs, synth, w3, 256, 16, args.seed)
        e3 = run_eager(torch, rs, synth, w3, 256, 16, args.seed)
        r3s = run_spec(torch, rs, synth, w3, 64, 8, args.seed)
        r3p = run_spec(torch, rs, synth, w3, 64, 8, args.seed, precision="fp32_hp_bf16_lp")
        wl[w3.name] = {"tokens_per_s": r3["tokens"] / (r3["ms"] * 1e-3),
                       "decode_kernel_gbs": r3["kernel_bytes"] / (r3["kernel_ms_total"] * 1e6),
                       "eager_tokens_per_s": e3["tokens"] / (e3["ms"] * 1e-3), "eager_gbs": e3["gbs"],
                       "verify_T4_accepted_tokens_per_s": r3s["accepted_tokens"] / (r3s["ms"] * 1e-3),
                       "verify_T4_kernel_gbs": r3s["kernel_gbs"], "verify_T4_avg_us": r3s["kernel_avg_us"],
                       "two_precision_verify_T4_accepted_tokens_per_s": r3p["accepted_tokens"] / (r3p["ms"] * 1e-3),
                       "two_precision_verify_T4_kernel_gbs": r3p["kernel_gbs"],
                       "two_precision_verify_T4_avg_us": r3p["kernel_avg_us"]}
        w5 = synth.WORKLOADS["kda_decode_b256"]
        r5 = run_standard_decode(torch, rs, synth, w5, 256, 16, args.seed, fused=False)
        r5f = run_standard_decode(torch, rs, synth, w5, 256, 16, args.seed, fused=True)
        e5 = run_eager(torch, rs, synth, w5, 256, 16, args.seed)
        r5s = run_spec(torch, rs, synth, w5, 64, 8, args.seed)
        wl[w5.name] = {"tokens_per_s": r5["tokens"] / (r5["ms"] * 1e-3),
                       "decode_kernel_gbs": r5["kernel_bytes"] / (r5["kernel_ms_total"] * 1e6),
                       "decode_kernel_avg_us": r5["kernel_avg_us"],
                       "fused_tokens_per_s": r5f["tokens"] / (r5f["ms"] * 1e-3),
                       "fused_kernel_gbs": r5f["kernel_bytes"] / (r5f["kernel_ms_total"] * 1e6),
                       "eager_tokens_per_s": e5["tokens"] / (e5["ms"] * 1e-3), "eager_gbs": e5["gbs"],
                       "verify_T4_accepted_tokens_per_s": r5s["accepted_tokens"] / (r5s["ms"] * 1e-3),
                       "verify_T4_kernel_gbs": r5s["kernel_gbs"], "verify_T4_avg_us": r5s["kernel_avg_us"]}
        fl = {"mamba2_fp32": run_flush(torch, rs, synth, w, 16, 2, args.seed),
              "mamba2_fp32_hp_bf16_lp": run_flush(torch, rs, synth, w, 16, 2, args.seed, precision="fp32_hp_bf16_lp"),
              "gdn_fp32": run_flush(torch, rs, synth, synth.WORKLOADS["gdn_decode_b256"], 16, 2, args.seed),
              "gdn_fp32_hp_bf16_lp": run_flush(torch, rs, synth, synth.WORKLOADS["gdn_decode_b256"], 16, 2,
                                               args.seed, precision="fp32_hp_bf16_lp")}
        line["flush"] = fl
        # the input side of the Mamba-2 layer: x (8192) and B, C (2 x 128 x 128) channels, width 4
        line["conv_input_ring"] = {f"T{T}": run_conv(torch, rs, synth, 256, 40960, 4, T, 64, 8, args.seed)
                                   for T in (1, 4)}
        w4 = synth.WORKLOADS["mamba2_2prec_b256"]
        r4 = {}
        for prec in ("fp32_hp_bf16_lp", "bf16_shared", "fp32"):
            r = run_spec(torch, rs, synth, w4, 128, 8, args.seed, precision=prec)
            r4[prec] = {"accepted_tokens_per_s": r["accepted_tokens"] / (r["ms"] * 1e-3),
                        "verify_kernel_gbs": r["kernel_gbs"], "verify_avg_us": r["kernel_avg_us"]}
        r4["small_batch_graph"] = {f"B{B}": run_spec_graph(torch, rs, synth, w4, B, 16, 20, args.seed)
                                   for B in (1, 32)}
        if not args.no_drift:
            line["drift"] = {f"B{B}": run_drift(torch, rs, synth, w4, B, w4.steps, args.seed)
                             for B in (256, 1, 32, 512)}
        if args.sweep:
            sweep = {}
            for B in (1, 32, 256, 512):
                for label, rot in (("warm", 0), ("rotated", 2 << 30)):
                    r = run_spec(torch, rs, synth, w4, 128, 16, args.seed, B=B, rotate_bytes=rot)
                    sweep[f"B{B}_{label}"] = {
                        "accepted_tokens_per_s": r["accepted_tokens"] / (r["ms"] * 1e-3),
                        "verify_kernel_gbs": r["kernel_gbs"], "verify_avg_us": r["kernel_avg_us"],
                        "layers": r["layers"], "layer_footprint_MiB": round(r["layer_footprint_MiB"], 1)}
            r4["batch_sweep_fp32_hp_bf16_lp"] = sweep
        wl[w4.name] = r4
        line["workloads"] = wl
        line["ceilings"] = ceilings(torch, rs)
    if args.window_sweep:
        line["window_sweep"] = window_sweep(torch, rs, synth, args.seed)
    if not (args.quick or args.no_cpu_baseline):
        line["cpu_baseline"] = cpu_baseline(synth, w, args.seed, args.cpu_seconds)
        if not args.quick:
            side = args.cpu_seconds / 4  # the further figures take a quarter of the budget each
            one = cpu_baseline(synth, w, args.seed, side, threads=1)
            f64 = cpu_baseline(synth, w, args.seed, side, precision="f64")
            g = synth.WORKLOADS["gdn_decode_b256"]
            gd = cpu_baseline(synth, g, args.seed, side)
            kd = synth.WORKLOADS["kda_decode_b256"]
            kc = cpu_baseline(synth, kd, args.seed, side)
            _CPU_INPUTS.clear()
            line["cpu_baseline"]["more"] = {
                "one_core": {"value": one["value"], "cores": one["cores"], "sample": one["sample"]},
                "fp64": {"value": f64["value"], "cores": f64["cores"], "sample": f64["sample"]},
                g.name: {"value": gd["value"], "cores": gd["cores"], "sample": gd["sample"]},
                kd.name: {"value": kc["value"], "cores": kc["cores"], "sample": kc["sample"]}}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
