"""Benchmark of the ReplaySSM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload large|fp8|nvfp4|prod|mtp|tiny] [--algo auto|monolith|split]
                    [--batch B] [--no-cpu-baseline] [--no-extra] [--no-fuse] [--separate]

One step = one pass of the hot path over one batch of synthetic input: the
replay step (dt' softplus, decay prefix, C.B, checkpoint replay and readout,
ring appends) and, for the flushing workloads, the flush (fold of the
accepted tokens, re-encode, ring_start advance).

The headline workload is the largest single-GPU configuration: 1024 active
entries of a 2048-slot cache (slot 0 padding, 256 B of padding between slot
pages), 128 heads in 8 groups, headdim 64, dstate 128, bf16 checkpoint,
varlen T_b ~ U{1..8} new tokens per entry, pnat ~ U{0..8} live ring tokens,
ring length 16.  The same JSON line carries, under "extra", the quantised-
checkpoint loop (fp8 e4m3 checkpoint with fp32 row scales, batch 256, T = 4,
k ~ U{1..4} accepted tokens folded every step inside the step), the only
configuration that runs every flush row.

Inputs are synthetic, drawn on the GPU (synth package) and resident in HBM
before timing.  To measure HBM rather than the 256 MB Infinity Cache the
cache holds disjoint sets of `batch` slots (>= 2 GiB in total) and
consecutive steps rotate through them.

Timing protocol: W eager warmup steps; a HIP graph of K steps is captured;
the graph is replayed for a settle phase of about --settle seconds (reported
on its own: a GPU that has been idle runs its first milliseconds at lower
clocks); then --trials replays of the K-step graph, each bracketed by HIP
events on the launch stream between two synchronisations.  ms_per_step is
the median trial / K (min and max reported).  The roofline of the dominant
kernel comes from the same timed replays (its launches per step are stated),
with the eager per-call event times beside it.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "replayed SSU tokens/sec and achieved HBM GB/s (% of MI355X peak) at 1 GPU"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published peak
HEADLINE = "large"
EXTRA = "fp8"

WORKLOADS = {
    "nvfp4": dict(nheads=128, ngroups=8, state_dtype="nvfp4", batch=256, T=4, pnat_max=0, out="bf16",
                  flush=(1, 4), varlen=False, slot_pad=0, separate=True,
                  desc="NVFP4 read checkpoint (e2m1, e4m3 block scales, f32 slot scale) + FP16 recurrence "
                       "checkpoint with stochastic rounding, batch 256, H128 G8, P64 N128, T=4, fold "
                       "k~U{1..4} every step, L=16"),
    "fp8": dict(nheads=128, ngroups=8, state_dtype="fp8", batch=256, T=4, pnat_max=0, out="bf16",
                flush=(1, 4), varlen=False, slot_pad=0,
                desc="fp8 e4m3 checkpoint + f32 row scales, batch 256, H128 G8, P64 N128, T=4, "
                     "replay step + flush k~U{1..4} every step, L=16"),
    "prod": dict(nheads=128, ngroups=8, state_dtype="f16", batch=256, T=8, pnat_max=8, out="bf16",
                 flush=None, varlen=False, slot_pad=0,
                 desc="production MTP decode, fp16 checkpoint, H128 G8, P64 N128, T=8, pnat~U{0..8}, "
                      "L=16, ring_start~U{0..15}"),
    "mtp": dict(nheads=64, ngroups=8, state_dtype="bf16", batch=64, T=4, pnat_max=4, out="bf16",
                flush=None, varlen=False, slot_pad=0,
                desc="MTP decode, bf16 checkpoint, batch 64 of 128 slots, H64 G8, P64 N128, T=4, "
                     "pnat~U{0..4}, L=16"),
    "large": dict(nheads=128, ngroups=8, state_dtype="bf16", batch=1024, T=8, pnat_max=8, out="bf16",
                  flush=None, varlen=True, slot_pad=256,
                  desc="large batch, bf16 checkpoint, 1024 active of 2048 slots, H128 G8, P64 N128, "
                       "varlen T_b~U{1..8}, pnat~U{0..8}, L=16, 256 B padding between slot pages"),
    "tiny": dict(nheads=8, ngroups=1, state_dtype="f32", batch=2, T=1, pnat_max=8, out="f32",
                 flush=None, varlen=False, slot_pad=0,
                 desc="tiny reference, fp32 checkpoint, batch 2 of 4 slots, H8 G1, T=1"),
}

# the arithmetic type of the readout products (MFMA inputs; every sum is fp32)
COMPUTE_DTYPE = {"f32": "f32", "bf16": "bf16", "f16": "f16", "fp8": "bf16", "nvfp4": "bf16"}

ELEM = {"f32": 4, "bf16": 2, "f16": 2, "fp8": 1, "nvfp4": 0.5}


def scale_bytes(spec, H):
    """Scale bytes read or written with one slot's checkpoint: fp8 an f32 per
    row, nvfp4 an e4m3 per 16 values and the slot's f32 scale."""
    if spec.state_dtype == "fp8":
        return H * 64 * 4
    if spec.state_dtype == "nvfp4":
        return H * (64 * 128 // 16) + 4
    return 0


def step_bytes(spec, H, G, pnat, Tb, out_bytes=2):
    """Algorithmic HBM bytes of one replay step (sum over entries): checkpoint
    (+ fp8 row scales) read, live-ring x/B/dt' read, new x/B/C/dt read, out
    written, x/B/dt' appended.  Scratch traffic of the split is excluded."""
    P, N = 64, 128
    per_state = int(H * P * N * ELEM[spec.state_dtype]) + scale_bytes(spec, H)
    tot = 0
    for p, t in zip(pnat, Tb):
        p, t = int(p), int(t)
        tot += per_state
        tot += p * (H * P * 2 + G * N * 2 + H * 4)              # live ring reads
        tot += t * (H * P * 2 + 2 * G * N * 2 + H * 4)          # new x, B, C, dt
        tot += t * H * P * out_bytes                            # out
        tot += t * (H * P * 2 + G * N * 2 + H * 4)              # appends
    return tot


def state_bytes(spec, H):
    """Checkpoint (+ fp8 row scales) bytes of one slot."""
    return int(H * 64 * 128 * ELEM[spec.state_dtype]) + scale_bytes(spec, H)


def fused_bytes(spec, H, G, k, Tb, out_bytes=2):
    """Algorithmic bytes of one fused flush-in-step with pnat = k = num_fold:
    a flush of k tokens and a step with no live tokens, minus the checkpoint
    read the fusion saves for every entry that folds."""
    saved = sum(state_bytes(spec, H) for kk in k if kk > 0)
    return step_bytes(spec, H, G, [0] * len(k), Tb, out_bytes) + flush_bytes(spec, H, G, k) - saved


def recur_bytes(H):
    """FP16 recurrence checkpoint bytes of one slot (separate checkpoints)."""
    return H * 64 * 128 * 2


def separate_extra_bytes(spec, H, k, G=8):
    """What separate checkpoints add to a fold of each entry with k > 0: the
    recurrence checkpoint is read and written, the read checkpoint (+ scales)
    only written.  An NVFP4 read checkpoint has one scale per slot over every
    head, so its fold first makes a pass that reads the recurrence checkpoint
    and the k ring tokens for the head maxima (4 B written per head), and the
    encode reads the slot's H maxima back."""
    extra = 0
    for kk in k:
        if kk <= 0:
            continue
        extra += 2 * recur_bytes(H) - state_bytes(spec, H)
        if spec.state_dtype == "nvfp4":
            extra += recur_bytes(H) + int(kk) * (H * 64 * 2 + G * 128 * 2 + H * 4) + 2 * H * 4
    return int(extra)


def flush_bytes(spec, H, G, k):
    """Algorithmic bytes of one flush: checkpoint read + write and the k ring
    tokens (x, B, dt') read, per entry with k > 0."""
    P, N = 64, 128
    per_state = int(H * P * N * ELEM[spec.state_dtype]) + scale_bytes(spec, H)
    return int(sum(2 * per_state + int(kk) * (H * P * 2 + G * N * 2 + H * 4) for kk in k if kk > 0))


# ---------------------------------------------------------------------------
# GPU clocks (amdsmi, when it imports on the box)
# ---------------------------------------------------------------------------

class Clocks:
    def __init__(self):
        self.h = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            hs = amdsmi.amdsmi_get_processor_handles()
            if hs:
                self.amdsmi, self.h = amdsmi, hs[0]
        except Exception:  # no amdsmi, or no permission: clocks are reported as null
            self.h = None

    def sample(self):
        if self.h is None:
            return None
        out = {}
        for name, kind in (("sclk_mhz", "GFX"), ("mclk_mhz", "MEM")):
            try:
                info = self.amdsmi.amdsmi_get_clock_info(self.h, getattr(self.amdsmi.AmdSmiClkType, kind))
                out[name] = info.get("clk")
                out[name.replace("_mhz", "_max_mhz")] = info.get("max_clk")
            except Exception:
                out[name] = None
        return out


# ---------------------------------------------------------------------------
# one workload: cache, steps, graph, timed trials
# ---------------------------------------------------------------------------

def run_workload(args, name, clocks, dev, batch=None, cpu=False):
    import speculative_replay_state_amd as ssu
    import synth
    from synth import device as sd

    wl = dict(WORKLOADS[name])
    wl_batch = wl["batch"]
    separate = bool(wl.get("separate")) or (args.separate and name == args.workload)
    fused = bool(wl["flush"]) and args.fuse
    if separate and (not wl["flush"] or wl["state_dtype"] not in ("fp8", "nvfp4")):
        raise SystemExit("--separate needs a workload with flushes and an fp8 checkpoint (fp8)")
    if batch:
        wl["batch"] = batch
    batch, H, G, T = wl["batch"], wl["nheads"], wl["ngroups"], wl["T"]

    # --- cache with rotating arenas (HBM, not the Infinity Cache) -----------
    probe = synth.CacheSpec(num_slots=2, nheads=H, ngroups=G, state_dtype=wl["state_dtype"],
                            slot_pad=wl["slot_pad"], separate=separate)
    slot_bytes = sum(probe.strides().values())
    if args.arenas is None:
        arenas = max(1, math.ceil(2.2 * 2 ** 30 / (slot_bytes * batch)))
        if name == "large" and batch == wl_batch:
            arenas = 2  # 2048 slots: 1024 active at a time, ~4.6 GB of checkpoints
    else:
        arenas = args.arenas
    num_slots = arenas * batch + 1
    spec = synth.CacheSpec(num_slots=num_slots, nheads=H, ngroups=G, state_dtype=wl["state_dtype"],
                           slot_pad=wl["slot_pad"], separate=separate)
    tcache = sd.make_cache_device(spec, args.seed, dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    dc = ssu.DeviceCache(num_slots, H, G, spec.ring_len, spec.state_dtype, tcache["state"],
                         tcache["scale"], tcache["x_cache"], tcache["B_cache"], tcache["dt_cache"],
                         tcache["ring_start"], status, recur=tcache.get("recur"), gscale=tcache.get("gscale"))

    rng = np.random.default_rng(args.seed)
    perm = rng.permutation(np.arange(1, num_slots, dtype=np.int32))
    steps_in, tsteps, flush_k, descs = [], [], [], []
    out_dt = torch.float32 if wl["out"] == "f32" else torch.bfloat16
    for a in range(arenas):
        slots = np.sort(perm[a * batch:(a + 1) * batch]).astype(np.int32)
        stp = synth.make_step(spec, batch, T, args.seed + 17 * a + 1, wl["pnat_max"], varlen=wl["varlen"],
                              slots=slots, pnat_fixed=0 if wl["pnat_max"] == 0 else None)
        if wl["flush"]:
            k = synth.flush_counts(batch, wl["flush"][0], wl["flush"][1], args.seed + 31 * a + 5)
            flush_k.append(torch.from_numpy(k).to(dev))
            if fused:  # the k accepted tokens of the previous step are the live prefix, folded first
                stp.pnat[:] = k
        steps_in.append(stp)
        t = sd.upload_step(stp, dev)
        t["out"] = torch.empty((stp.tokens, H, 64), dtype=out_dt, device=dev)
        tsteps.append(t)
    ws = None
    d0 = ssu.make_step_desc(batch, T, tsteps[0]["slot_idx"], tsteps[0]["pnat"], tsteps[0]["cu_seqlens"],
                            tsteps[0]["x"], tsteps[0]["B"], tsteps[0]["C"], tsteps[0]["dt"],
                            tsteps[0]["A"], tsteps[0]["D"], tsteps[0]["dt_bias"], tsteps[0]["out"],
                            wl["out"], None, args.algo, flush_k[0] if fused else None)
    resolved = ssu.ssu_resolve_algo(dc.desc(), d0)
    if resolved < 0:
        raise ssu.SsuError(resolved, ssu.ssu_last_error())
    algo_used = {ssu.SSU_ALGO_MONOLITH: "monolith", ssu.SSU_ALGO_SPLIT: "split"}[resolved]
    if algo_used == "split":
        ws = torch.empty(ssu.workspace_size(dc, batch, T) // 4 + 1, dtype=torch.float32, device=dev)
    for a, t in enumerate(tsteps):
        descs.append(ssu.make_step_desc(batch, T, t["slot_idx"], t["pnat"], t["cu_seqlens"], t["x"],
                                        t["B"], t["C"], t["dt"], t["A"], t["D"], t["dt_bias"], t["out"],
                                        wl["out"], ws, algo_used, flush_k[a] if fused else None))
    cdesc = dc.desc()

    def one_step(i, ev=None):
        stream = torch.cuda.current_stream()  # the capture stream inside torch.cuda.graph
        sh = stream.cuda_stream
        a = i % arenas
        if ev is not None:
            ev[0].record(stream)
        descs[a].sr_seed = i  # a new stochastic-rounding seed every call (separate checkpoints)
        rc = ssu.ssu_replay_step(cdesc, descs[a], sh)
        if rc:
            raise ssu.SsuError(rc, ssu.ssu_last_error())
        if ev is not None:
            ev[1].record(stream)
        if wl["flush"] and not fused:
            t = tsteps[a]
            rc = ssu.ssu_flush(cdesc, t["slot_idx"].data_ptr(), flush_k[a].data_ptr(), t["A"].data_ptr(),
                               batch, sr_seed=i, stream=sh)
            if rc:
                raise ssu.SsuError(rc, ssu.ssu_last_error())
            if ev is not None:
                ev[2].record(stream)

    # --- warmup (eager), then capture K steps in a graph --------------------
    for i in range(args.warmup):
        one_step(i)
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise RuntimeError("device status %d after warmup" % int(status.item()))

    K = args.steps
    graph = None
    stream = torch.cuda.current_stream()
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(K):
                one_step(args.warmup + i)
        torch.cuda.synchronize()

    def replay_once():
        if graph is not None:
            graph.replay()
        else:
            for i in range(K):
                one_step(args.warmup + i)

    # --- settle: replay until the GPU has run for about --settle seconds ----
    clk_before = clocks.sample()
    torch.cuda.synchronize()
    s0 = time.perf_counter()
    settle_replays = 0
    while True:
        replay_once()
        settle_replays += 1
        if settle_replays % 4 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - s0 >= args.settle:
                break
    torch.cuda.synchronize()
    settle_s = time.perf_counter() - s0

    # --- timed trials: each one replay of the K-step graph -------------------
    clk_settled = clocks.sample()
    trial_ms = []
    wall_timed = 0.0
    for _ in range(args.trials):
        ta = torch.cuda.Event(enable_timing=True)
        tb = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        ta.record(stream)
        replay_once()
        tb.record(stream)
        torch.cuda.synchronize()
        wall_timed += time.perf_counter() - w0
        trial_ms.append(ta.elapsed_time(tb))
    clk_after = clocks.sample()
    if int(status.item()) != 0:
        raise RuntimeError("device status %d after the timed replays" % int(status.item()))
    ms_med = float(np.median(trial_ms))
    ms_per_step = ms_med / K

    # --- eager per-call durations (HIP events around each call, same stream) -
    nrep = min(K, 8 * arenas)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(nrep)]
    torch.cuda.synchronize()
    for i in range(nrep):
        one_step(i, evs[i])
    torch.cuda.synchronize()
    step_ms = [e[0].elapsed_time(e[1]) for e in evs]
    flush_ms = [e[1].elapsed_time(e[2]) for e in evs] if (wl["flush"] and not fused) else []

    tokens_per_step = float(np.mean([s.tokens for s in steps_in]))
    # replayed positions: live ring tokens plus new tokens of every entry (the folded prefix included)
    positions_per_step = float(np.mean([int(np.sum(s.pnat)) + s.tokens for s in steps_in]))
    ob = 4 if wl["out"] == "f32" else 2
    tbs = [np.diff(s.cu_seqlens) if s.cu_seqlens is not None else [T] * batch for s in steps_in]
    if fused:
        sbytes = float(np.mean([fused_bytes(spec, H, G, k.cpu().numpy(), tb, ob)
                                + (separate_extra_bytes(spec, H, k.cpu().numpy(), G) if separate else 0)
                                for k, tb in zip(flush_k, tbs)]))
        fbytes = 0.0
    else:
        sbytes = float(np.mean([step_bytes(spec, H, G, s.pnat, tb, ob) for s, tb in zip(steps_in, tbs)]))
        fbytes = float(np.mean([flush_bytes(spec, H, G, k.cpu().numpy())
                                + (separate_extra_bytes(spec, H, k.cpu().numpy(), G) if separate else 0)
                                for k in flush_k])) if flush_k else 0.0
    # kernel launches per ssu_replay_step call (as dispatched for this workload)
    launches = 1
    if algo_used == "split":
        launches = 2
    elif fused:
        launches = 2  # the fused kernel and its ring advance
    step_avg = float(np.mean(step_ms))
    kernels = {"replay_step": {"algo": algo_used, "fused_flush": fused, "launches_per_call": launches,
                               "eager_call_us": 1e3 * step_avg, "bytes": sbytes,
                               "eager_GBps": sbytes / (step_avg * 1e6)}}
    dominant = "replay_step"
    if flush_ms:
        fl_avg = float(np.mean(flush_ms))
        kernels["flush"] = {"eager_call_us": 1e3 * fl_avg, "bytes": fbytes, "eager_GBps": fbytes / (fl_avg * 1e6)}
        if fl_avg > step_avg:
            dominant = "flush"
    # the roofline from the timed replays: a step that is one call (no separate
    # flush) spends the whole step time in that call's launches
    if not flush_ms:
        call_us = 1e3 * ms_per_step
        achieved = sbytes / (ms_per_step * 1e6)
        timed_from = "timed graph replays (median trial / K steps)"
    else:
        call_us = kernels[dominant]["eager_call_us"]
        achieved = kernels[dominant]["eager_GBps"]
        timed_from = "eager per-call HIP events (a step holds a step and a flush call)"
    value = tokens_per_step * K / (ms_med * 1e-3)

    res = {
        "name": name, "wl": wl, "spec": spec, "tcache": tcache, "steps_in": steps_in, "flush_k": flush_k,
        "fused": fused, "separate": separate, "batch": batch, "H": H, "G": G, "T": T,
        "value": value, "ms_per_step": ms_per_step, "trial_ms": trial_ms, "wall_timed": wall_timed,
        "settle_s": settle_s, "settle_replays": settle_replays,
        "clocks": {"before_settle": clk_before, "settled": clk_settled, "after_trials": clk_after},
        "tokens_per_step": tokens_per_step, "positions_per_step": positions_per_step,
        "sbytes": sbytes, "fbytes": fbytes, "algo": algo_used, "arenas": arenas, "num_slots": num_slots,
        "graph": graph is not None, "kernels": kernels, "dominant": dominant, "call_us": call_us,
        "achieved": achieved, "timed_from": timed_from, "launches": launches, "wl_batch": wl_batch,
    }
    if cpu and not args.no_cpu_baseline:
        c = cpu_baseline(args, res)
        c["effective_GBps"] = c["value"] * (sbytes + fbytes) / tokens_per_step / 1e9
        res["cpu"] = c
    return res


def summary(res, K):
    """The compact record of a workload run (the extra loop of the JSON line)."""
    return {
        "workload": res["name"] + ": " + res["wl"]["desc"],
        "value": res["value"], "unit": "tokens/s", "ms_per_step": res["ms_per_step"],
        "trials_ms_per_step": [t / K for t in res["trial_ms"]],
        "algorithmic_bytes_per_step": res["sbytes"] + res["fbytes"],
        "achieved_GBps_step": (res["sbytes"] + res["fbytes"]) / (res["ms_per_step"] * 1e6),
        "frac_step": (res["sbytes"] + res["fbytes"]) / (res["ms_per_step"] * 1e6) / HBM_PEAK_GBS,
        "kernels": res["kernels"],
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--trials", type=int, default=5, help="timed replays of the K-step graph (median)")
    ap.add_argument("--settle", type=float, default=2.0, help="seconds of graph replays before the trials")
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(WORKLOADS))
    ap.add_argument("--algo", default="auto", choices=["auto", "monolith", "split"])
    ap.add_argument("--batch", type=int, default=None)
    ap.add_argument("--arenas", type=int, default=None, help="disjoint slot sets rotated per step")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the fp8 flush loop in the same line")
    ap.add_argument("--no-streams", action="store_true", help="skip the plain HBM stream rates")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    ap.add_argument("--seed", type=int, default=1234)
    ap.add_argument("--fuse", action=argparse.BooleanOptionalAction, default=True,
                    help="flush workloads: fold the accepted tokens inside the replay step (one "
                         "ssu_replay_step with num_fold) instead of a separate ssu_flush call")
    ap.add_argument("--separate", action="store_true",
                    help="fp8 workload: separate FP16 recurrence checkpoint (stochastic rounding)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the ReplaySSM step has no cross-GPU exchange "
              "(slots and heads shard without communication); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X)", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.trials < 1:
        print("--steps and --trials must be >= 1", file=sys.stderr)
        sys.exit(2)

    dev = "cuda:0"
    clocks = Clocks()
    K = args.steps
    res = run_workload(args, args.workload, clocks, dev, batch=args.batch, cpu=True)
    cpu = res.pop("cpu", None)
    extra = None
    if not args.no_extra and args.workload == HEADLINE and not args.batch:
        # the headline's cache is freed first (the extra loop draws its own)
        head_keep = {k: v for k, v in res.items() if k not in ("tcache",)}
        del res
        torch.cuda.empty_cache()
        ex = run_workload(args, EXTRA, clocks, dev)
        extra = {EXTRA + "_fused_flush": summary(ex, K)}
        del ex
        torch.cuda.empty_cache()
        res = head_keep
    else:
        res.pop("tcache", None)

    # --- counter calibration copy (1 GiB), only when asked ------------------
    if args.calib_copy:
        src = torch.empty(2 ** 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # --- what plain streams reach on this GPU (context for the roofline) ----
    streams = None if args.no_streams else hbm_streams(dev)
    floor_us = None if args.no_streams else launch_floor_us(dev)

    wl, spec = res["wl"], res["spec"]
    batch, H, G, T = res["batch"], res["H"], res["G"], res["T"]
    name = res["name"]
    achieved = res["achieved"]
    fused, separate = res["fused"], res["separate"]
    line = {
        "metric": METRIC,
        "value": res["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": COMPUTE_DTYPE[wl["state_dtype"]],
        "data": "synthetic (seeded, drawn on the GPU; no dataset)",
        "config": {
            "workload": name + ": " + wl["desc"],
            "batch": batch, "nheads": H, "ngroups": G, "headdim": 64, "dstate": 128, "ring_len": 16,
            "T": T, "state_dtype": wl["state_dtype"], "out_dtype": wl["out"], "accumulate": "f32",
            "algo": res["algo"],
            "separate_checkpoints": (None if not separate else
                                     "FP16 recurrence checkpoint, stochastic rounding, %s read checkpoint"
                                     % wl["state_dtype"]),
            "flush": (None if not wl["flush"] else
                      "fused into the replay step (ssu_replay_step with num_fold = pnat = k)" if fused
                      else "separate ssu_flush after the step"),
            "arenas": res["arenas"], "cache_slots": res["num_slots"], "graph": res["graph"],
            "tokens_per_step": res["tokens_per_step"],
            "replayed_positions_per_s": res["positions_per_step"] * K / (res["ms_per_step"] * K * 1e-3),
            "algorithmic_bytes_per_step": res["sbytes"] + res["fbytes"],
            "achieved_GBps_step": (res["sbytes"] + res["fbytes"]) / (res["ms_per_step"] * 1e6),
        },
        "timing": {
            "trials": len(res["trial_ms"]),
            "steps_per_trial": K,
            "ms_per_step_median": res["ms_per_step"],
            "ms_per_step_min": min(res["trial_ms"]) / K,
            "ms_per_step_max": max(res["trial_ms"]) / K,
            "settle_s": res["settle_s"],
            "settle_replays": res["settle_replays"],
            "wall_s_timed": res["wall_timed"],
            "clocks": res["clocks"],
        },
        "roofline": {
            "bound": "hbm",
            "kernel": res["dominant"],
            "launches_per_call": res["launches"],
            "call_us": res["call_us"],
            "timed_from": res["timed_from"],
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": (measured_traffic(res["dominant"], name + ("_fused" if fused else "")
                                         + ("_separate" if separate else ""))
                        if batch == res["wl_batch"] and res["algo"] == "monolith" else None),
        },
        "kernels": res["kernels"],
        "hbm_stream": (None if streams is None else
                       dict(streams, frac_of_copy=achieved / streams["copy_GBps"],
                            frac_of_rmw=achieved / streams["rmw_GBps"])),
        "launch_floor_us": floor_us,
        "extra": extra,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def hbm_streams(dev, nbytes=2 ** 31, reps=5):
    """GB/s of plain PyTorch streams over 2 GiB buffers on this GPU: a device
    copy (half reads, half writes), an in-place read-modify-write of one
    buffer (x.mul_(1.0): every byte read and written back, as a checkpoint
    fold does), a fill (writes only) and row sums over rows of 2048 values
    (reads, with 1/2048 as many bytes written; a sum of the whole buffer to
    one value runs as a multi-pass reduction and reads far slower).  Best of
    `reps`."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    rows = src.view(-1, 2048)
    acc = torch.empty(rows.shape[0], dtype=torch.float32, device=dev)
    ops = {
        "copy_GBps": (lambda: dst.copy_(src), 2 * nbytes),
        "rmw_GBps": (lambda: src.mul_(1.0), 2 * nbytes),
        "write_GBps": (lambda: dst.fill_(2.0), nbytes),
        "read_GBps": (lambda: torch.sum(rows, dim=1, out=acc), nbytes + 4 * rows.shape[0]),
    }
    out = {"bytes_per_buffer": nbytes}
    for name, (fn, moved) in ops.items():
        fn()
        best = float("inf")
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            best = min(best, a.elapsed_time(b))
        out[name] = moved / (best * 1e6)
    del src, dst, rows, acc
    torch.cuda.empty_cache()
    return out


def launch_floor_us(dev, n=20, reps=5):
    """Microseconds per launch of a one-value PyTorch kernel, n launches in a
    row (each waiting for the one before) captured in one HIP graph and
    replayed as the steps are: the floor that a step of one launch pays on
    this GPU whatever it computes.  Median of `reps` replays."""
    t = torch.zeros(1, dtype=torch.float32, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            t.add_(1.0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            t.add_(1.0)
    g.replay()
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    del g, t
    return float(np.median(ms)) * 1e3 / n


def cpu_baseline(args, res):
    """The CPU oracle (as it stands) on a bounded sample: the first 64 entries
    of the first arena, step (+ flush), repeated until --cpu-seconds of work,
    once with every OpenMP thread the host offers and once with one thread."""
    from oracle import ssu_oracle as O
    from synth import device as sd

    spec, tcache, steps_in, flush_k, fused = (res["spec"], res["tcache"], res["steps_in"], res["flush_k"],
                                              res["fused"])
    step = steps_in[0]
    n = min(64, step.batch)
    entries = list(range(n))
    slots = [int(step.slot_idx[b]) for b in entries]
    host, smap = sd.download_subset(spec, tcache, slots)
    sub = sd.subset_step(step, entries, smap)
    k = flush_k[0].cpu().numpy()[:n] if flush_k else None

    def timed(seconds):
        tokens = reps = 0
        t0 = time.perf_counter()
        while True:
            c = host.copy()
            if fused:
                O.replay_step(c, sub, num_fold=k, seed=reps)
            else:
                O.replay_step(c, sub)
                if k is not None:
                    O.flush(c, sub.slot_idx, k, sub.A, reps)
            tokens += sub.tokens
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds or reps >= 1000:
                return tokens / el, reps, el

    threads = O.max_threads()
    v_all, reps, el = timed(args.cpu_seconds)
    O.set_threads(1)
    v_one, reps1, el1 = timed(args.cpu_seconds / 2)
    O.set_threads(threads)
    return {"value": v_all, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d entries of the first batch (%d new tokens), step%s, repeated %d times (%.1f s)" % (
                n, step.batch, sub.tokens,
                (" with fused flush" if fused else " + flush") if k is not None else "", reps, el),
            "single_thread": {"value": v_one, "cores": 1, "repeats": reps1, "seconds": el1},
            "host": {"os_cpu_count": os.cpu_count(), "cpu_model": _cpu_model()}}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def kernel_source_sha256():
    """Hash of the library's device and launch sources (file names and bytes)."""
    csrc = os.path.join(ROOT, "speculative_replay_state_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".cuh", ".hip", ".cpp", ".h")):
            h.update(name.encode())
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed counter summary
    profiles/<kernel>_<workload>_hbm_traffic.md, or None when that summary is
    missing or was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "%s_%s_hbm_traffic.md" % (kernel, workload))
    try:
        text = open(path).read()
        sha = kernel_source_sha256()
    except OSError:
        return None
    m_sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_val or m_sha.group(1) != sha:
        return None
    return float(m_val.group(1))


if __name__ == "__main__":
    main()
