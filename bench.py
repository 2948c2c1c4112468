#!/usr/bin/env python3
"""Decode benchmark of the ReplaySSM hot path on one MI355X.

Workload: one Mamba-2 SSM layer in decode, batch 256, 128 heads x P=64 x N=128
(a 4 MiB fp32 state per sequence), bf16 x/B/C, fp32 dt and A, flush window
W=16, synthetic seeded inputs (workloads.synth; 256 distinct decode steps
resident in HBM before timing, cycled when more steps are timed).

A step is one decode token for the whole batch through the replay path: the
replay decode kernel every step, and the checkpoint fold every W steps inside
the decode that fills the window (the fold's cost is part of the timed region).
`value` times exactly --steps steps; `steady_state` times whole windows, so
that it holds exactly one fold per W tokens whatever --steps is.

Output: one JSON line with tokens/s per layer (whole-job throughput, inputs
already in HBM), the dominant kernel's roofline (algorithmic bytes per launch
over the HIP-event-measured launch duration, against 8 TB/s), the HBM read
and copy rates this GPU achieves (the library's calibration kernels), the eager
GPU baseline, the further workloads (staggered folds, dual precision and its
window sweep, the low-precision comparison, speculative rounds at batch 512,
Gated DeltaNet, Kimi Delta Attention, a single B/C group), each timed over
whole windows, and the fp64 CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import concurrent.futures
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402
from workloads import synth  # noqa: E402

WORKLOAD = "mamba2_b256_h128_p64_n128_w16"
METRIC = "SSM decode tokens/s per layer + achieved HBM GB/s (% of peak), batch 256"
PEAK_HBM_GBS = 8000.0
COUNTERS_FILE = os.path.join(ROOT, "profiles", "replay_decode_b256_hbm_counters.txt")
KERNEL_SOURCES = ["replay.hip", "device.h", "limits.h", "launch.h", "lds.h", "fold.h", "verify_mfma.h",
                  "eager.hip"]
SWEEP_WINDOWS = (8, 16, 32)


# ---- algorithmic bytes (what the method must move, per (sequence, head)) ----
def replay_bytes(wl, n0: int) -> int:
    """Replay decode of one token with n0 entries already in the window."""
    P, N, ib = wl.headdim, wl.dstate, 2 if wl.in_dtype == "bf16" else 4
    tile = P * N * (2 if wl.read_copy in ("bf16", "bf16_state") else 4)
    entry = P * ib + N * ib + 8                     # x, B, (dt, dt*A)
    inputs = P * ib + 2 * N * ib + 4                 # x_t, B_t, C_t, dt_t
    return tile + n0 * entry + inputs + P * 4 + entry + 32 + 4   # + y, append, pointers, A


def flush_bytes(wl, n: int) -> int:
    """Fold of n window entries into one checkpoint tile (read + write)."""
    P, N, ib = wl.headdim, wl.dstate, 2 if wl.in_dtype == "bf16" else 4
    ring = n * (P * ib + N * ib + 8) + 32
    if wl.read_copy == "bf16_state":            # bf16 checkpoint read and written
        return 2 * P * N * 2 + ring
    lo = P * N * 2 if wl.read_copy == "bf16" else 0
    return 2 * P * N * 4 + lo + ring


def fused_bytes(wl) -> int:
    """Decode of the token that fills the window, with the fold in the same pass:
    the replay's bytes plus the new checkpoint written."""
    sb = 2 if wl.read_copy == "bf16_state" else 4
    return replay_bytes(wl, wl.window - 1) + wl.headdim * wl.dstate * sb


def dual_fused_bytes(wl) -> int:
    """Dual precision, the token that fills every window folded in one pass from
    the fp32 master: the replay's bytes with the master tile read instead of the
    bf16 copy, plus the new master and the new copy written."""
    P, N = wl.headdim, wl.dstate
    return replay_bytes(wl.replace(read_copy="none"), wl.window - 1) + P * N * 4 + P * N * 2


def eager_bytes(wl, state_bytes: int = 4) -> int:
    P, N, ib = wl.headdim, wl.dstate, 2 if wl.in_dtype == "bf16" else 4
    return 2 * P * N * state_bytes + P * ib + 2 * N * ib + 4 + P * 4 + 4


def verify_bytes(wl, n0: np.ndarray, fold: np.ndarray) -> int:
    """Verify of K+1 tokens per (sequence, head) with n0[b] committed entries in
    the window, summed over the batch and the heads; fold[b]: the committed
    window is folded in the same pass (its tile written back)."""
    P, N, K = wl.headdim, wl.dstate, wl.draft
    entry = 2 * P + 2 * N + 8
    per = (P * N * 4 + n0 * entry + (K + 1) * (2 * P + 4 * N + 4 + 4 * P + entry) + 36
           + fold.astype(np.int64) * P * N * 4)
    return int(np.sum(per)) * wl.nheads


def gdn_bytes(wl, n0: int) -> dict:
    """Algorithmic bytes per (sequence, head) of the GDN / KDA kernels (fp32)."""
    P, N = wl.headdim, wl.dstate
    if wl.kind == "kda":
        entry = 8 * N + 4 * P                       # k, u, log-gate row
        inputs = 4 * N * 3 + 4 * P + 4              # q, k, alpha row, v, beta
    else:
        entry = 4 * N + 4 * P + 8                   # k, u, (1, log alpha)
        inputs = 4 * N * 2 + 4 * P + 8              # q, k, v, beta, alpha
    replay = P * N * 4 + n0 * entry + inputs + 4 * P + entry + 32
    return {"replay": replay, "inputs": inputs,
            "fused": P * N * 4 * 2 + (wl.window - 1) * entry + inputs + 4 * P + entry + 32,
            "flush": 2 * P * N * 4 + wl.window * entry + 32,
            "eager": 2 * P * N * 4 + inputs + 4 * P}


def whole(steps: int, multiple: int, minimum: int) -> int:
    """`steps` rounded up to a whole number of windows, at least `minimum`."""
    return max(minimum, -(-steps // multiple) * multiple)


def kernel_source_hash() -> str:
    """Hash of the replay kernel's code (comments and blank space removed, so a
    comment edit does not retire the committed counter measurements)."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "recurrent_state_storage_amd", "csrc", f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def counter_traffic(key: str = "replay"):
    """HBM bytes per launch of the replay decode kernel ("replay"), the fused
    decode + fold ("fused") or the eager step ("eager") from the committed
    rocprofv3 counter summary, or None when the summary is absent, lacks the
    figure, or the replay kernel's code changed since."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    vals = {}
    with open(COUNTERS_FILE) as f:
        for line in f:
            m = re.match(r"^(\w+)\s*=\s*(\S+)", line.strip())
            if m:
                vals[m.group(1)] = m.group(2)
    if vals.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return float(vals[f"{key}_hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---- inputs (host generators; run before the device is touched) ----------------
def _gen_step(args):
    name, t = args
    s = synth.step_inputs(workloads.get(name), t)
    return t, s["x_bits"], s["B_bits"], s["C_bits"], s["dt"]


def gen_pool(wl, T: int, workers: int):
    xs = np.empty((T, wl.batch, wl.nheads, wl.headdim), np.uint16)
    Bs = np.empty((T, wl.batch, wl.ngroups, wl.dstate), np.uint16)
    Cs = np.empty_like(Bs)
    dts = np.empty((T, wl.batch, wl.nheads), np.float32)
    with concurrent.futures.ProcessPoolExecutor(max_workers=workers) as ex:
        for t, x, B, C, dt in ex.map(_gen_step, [(wl.name, t) for t in range(T)]):
            xs[t], Bs[t], Cs[t], dts[t] = x, B, C, dt
    return xs, Bs, Cs, dts


# ---- CPU baseline: the fp64 oracle as it stands ----------------------------------
_CPU_POOL = None       # (x, B, C, dt bits, A), inherited by forked workers


def _cpu_worker(args):
    """fp64 eager recurrence of the oracle on sequences [w*nseq, (w+1)*nseq),
    one BLAS thread, until the time budget or the pool's steps run out."""
    w, nseq, budget_s = args
    from threadpoolctl import threadpool_limits
    from oracle import mamba2
    xs, Bs, Cs, dts, A = _CPU_POOL
    lo, hi = w * nseq, (w + 1) * nseq
    S = np.zeros((nseq,) + xs.shape[2:] + (Bs.shape[-1],))
    bf = synth.bf16_value
    steps = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            i = steps % xs.shape[0]
            S, _ = mamba2.eager_step(S, A, bf(xs[i, lo:hi]), bf(Bs[i, lo:hi]), bf(Cs[i, lo:hi]),
                                     dts[i, lo:hi])
            steps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or steps >= xs.shape[0]:
                break
    return nseq * steps, el, steps


def cpu_baseline(wl, pool, budget_s: float, workers: int):
    """The oracle timed on the host: once on one core, then sharded over
    `workers` processes (sequences are independent), each with one thread."""
    import multiprocessing
    global _CPU_POOL
    _CPU_POOL = tuple(pool) + (synth.params(wl)["A"],)
    nseq = 16
    workers = max(1, min(workers, wl.batch // nseq))
    tok1, el1, st1 = _cpu_worker((0, nseq, budget_s / 3))
    with multiprocessing.get_context("fork").Pool(workers) as p:
        res = p.map(_cpu_worker, [(w, nseq, budget_s) for w in range(workers)])
    tokens = sum(r[0] for r in res)
    el = max(r[1] for r in res)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": tokens / el, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "one_core_tokens_per_s": tok1 / el1, "cpu_model": model,
            "sample": f"fp64 eager recurrence of the oracle, {workers} processes x 1 thread, each "
                      f"{nseq} sequences x {wl.nheads} heads ({workers * nseq} of {wl.batch} sequences), "
                      f"{min(r[2] for r in res)}-{max(r[2] for r in res)} decode steps in {el:.1f} s; "
                      f"one core alone: {st1} steps of {nseq} sequences in {el1:.1f} s"}


# ---- timing helpers --------------------------------------------------------------
def _timed(torch, fn, n, start=0):
    """Run fn(start + i) for i < n between two events on the current stream; ms."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(n):
        fn(start + i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


class Launches:
    """HIP events around individual launches on the current (launch) stream,
    grouped by a key; durations in microseconds."""

    def __init__(self, torch):
        self.torch = torch
        self.ev = {}

    def around(self, key, fn):
        a = self.torch.cuda.Event(enable_timing=True)
        b = self.torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.ev.setdefault(key, []).append((a, b))

    def us(self, key):
        return [a.elapsed_time(b) * 1e3 for a, b in self.ev.get(key, [])]


def rate(nbytes, us):
    return nbytes / (us * 1e-6) / 1e9 if us else None


# ---- calibration: what HBM delivers ---------------------------------------------
def run_calibration(torch, rss, dev):
    """Best of three grid sizes of the library's streaming-read and copy kernels
    over 1 GiB (16-byte non-temporal accesses, as the decode kernels use), and
    torch's elementwise copy for comparison."""
    n = 1 << 28                                        # 1 GiB of fp32
    src = torch.ones((n,), device=dev)
    dst = torch.empty_like(src)
    sink = torch.zeros((4,), device=dev)
    nbytes = n * 4
    read = {}
    for g in (2048, 4096, 8192):
        rss.rss_calib_read(src, sink, g)
        ms = _timed(torch, lambda i: rss.rss_calib_read(src, sink, g), 10) / 10
        read[g] = rate(nbytes, ms * 1e3)
    copy = {}
    for g in (4096, 8192, 16384):
        rss.rss_calib_copy(src, dst, g)
        ms = _timed(torch, lambda i: rss.rss_calib_copy(src, dst, g), 10) / 10
        copy[g] = rate(2 * nbytes, ms * 1e3)
    write = {}
    for g in (4096, 8192, 16384):
        rss.rss_calib_write(dst, g)
        ms = _timed(torch, lambda i: rss.rss_calib_write(dst, g), 10) / 10
        write[g] = rate(nbytes, ms * 1e3)
    torch.mul(src, 1.0, out=dst)
    ms = _timed(torch, lambda i: torch.mul(src, 1.0, out=dst), 10) / 10
    # The replay's shape of work without its arithmetic: one workgroup per
    # checkpoint tile, then the bytes a replay writes per tile (y, the appended
    # ring entry, the pointer word), rounded up to whole 16-byte vectors.
    wl = workloads.get(WORKLOAD)
    P, N = wl.headdim, wl.dstate
    tile = P * N * 4
    ntile = nbytes // tile
    wb = -(-(4 * P + (2 * P + 2 * N + 8) + 16) // 16) * 16
    wdst = torch.empty((ntile * wb // 4,), device=dev)

    def tiles(tb, nt, dst=None, w=0):
        """Milliseconds of rss_calib_tiles: the faster of the two workgroup
        orders (the decode kernels' runs of up to 512 KiB per XCD, or one
        contiguous range per XCD), and that order."""
        best = None
        for order in (0, 1):
            rss.rss_calib_tiles(src, tb, nt, dst, w, order)
            m = _timed(torch, lambda i: rss.rss_calib_tiles(src, tb, nt, dst, w, order), 10) / 10
            if best is None or m < best[0]:
                best = (m, order)
        return best

    (ms_t, o_t) = tiles(tile, ntile)
    (ms_tw, o_tw) = tiles(tile, ntile, wdst, wb)
    # the same with a verify's bytes written per tile (K + 1 outputs and
    # appended entries of the speculative workload, and the pointer word)
    sw = workloads.get("mamba2_spec_b512_h128_p64_n128_w16_k4")
    wbv = -(-((sw.draft + 1) * (4 * P + 2 * P + 2 * N + 8) + 16) // 16) * 16
    del wdst
    wdst = torch.empty((ntile * wbv // 4,), device=dev)
    (ms_tv, o_tv) = tiles(tile, ntile, wdst, wbv)
    # whole tiles read and written back (eager step, folds)
    del wdst
    wdst = torch.empty_like(src)
    (ms_tc, o_tc) = tiles(tile, ntile, wdst, tile)
    # Gated DeltaNet / KDA replays: 64 KiB tiles (d = 128 fp32), and the bytes
    # each writes per tile (output, appended k / u (/ log-gate) rows, pointer)
    delta = {}
    for name in ("gdn_b256_h32_d128_w16", "kda_b256_h32_d128_w16"):
        dw = workloads.get(name)
        dt_ = dw.headdim * dw.dstate * 4
        g = gdn_bytes(dw, 0)
        wbd = -(-(g["replay"] - dt_ - g["inputs"] - 16) // 16) * 16   # y + appended entry + pointer write
        nd = nbytes // dt_
        (ms_d, o_d) = tiles(dt_, nd, wdst, wbd)
        delta[dw.kind] = {"GBps": rate(nbytes + nd * wbd, ms_d * 1e3), "bytes_per_tile": [dt_, wbd],
                          "order": o_d}
    out = {"read_ceiling_GBps": max(read.values()), "copy_ceiling_GBps": max(copy.values()),
           "write_ceiling_GBps": max(write.values()),
           "tile_read_GBps": rate(nbytes, ms_t * 1e3),
           "tile_read_write_GBps": rate(nbytes + ntile * wb, ms_tw * 1e3),
           "tile_read_write_bytes_per_tile": [tile, wb],
           "tile_read_verify_writes_GBps": rate(nbytes + ntile * wbv, ms_tv * 1e3),
           "tile_read_verify_writes_bytes_per_tile": [tile, wbv],
           "tile_read_delta_rule_writes": delta,
           "tile_copy_GBps": rate(2 * nbytes, ms_tc * 1e3),
           "tile_orders": {"read": o_t, "read_write": o_tw, "read_verify_writes": o_tv, "copy": o_tc},
           "read_by_grid": read, "copy_by_grid": copy, "write_by_grid": write,
           "torch_elementwise_copy_GBps": rate(2 * nbytes, ms * 1e3),
           "how": "rss_calib_read / rss_calib_copy / rss_calib_write over 1 GiB, best of grids of 256-thread "
                  "workgroups; rss_calib_tiles over the same 1 GiB as 32 KiB tiles, one workgroup each, "
                  "without and with the replay's (or a verify's) bytes written per tile, and each tile copied back, "
                  "each the faster of two workgroup orders (tile_orders: 0 = the decode kernels' runs of up to "
                  "512 KiB per XCD, 1 = one contiguous range per XCD)"}
    del src, dst, sink, wdst
    return out


PHASES = ["main", "eager", "calibration", "staggered", "grouped", "dual", "dual_w8", "dual_w16",
          "dual_w32", "bf16_checkpoint", "eager_bf16", "speculative", "gdn", "kda"]


class PhaseMarker:
    """With --phase-markers, a tiny launch of the library's read kernel before
    each section, its grid size (1 + the section's index in PHASES) naming the
    section, so a profiler's per-dispatch records can be split by workload."""

    def __init__(self, torch, rss, dev, on):
        self.on, self.rss = on, rss
        if on:
            self.src = torch.zeros((4,), device=dev)
            self.sink = torch.zeros((4,), device=dev)

    def __call__(self, name):
        if self.on:
            self.rss.rss_calib_read(self.src, self.sink, 1 + PHASES.index(name))


def calibrate_counters(torch, rss, dev):
    """A plain 1 GiB -> 1 GiB copy by the library's copy kernel, run three
    times: the reference a profiler's HBM byte counters are scaled by."""
    src = torch.ones((1 << 28,), device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        rss.rss_calib_copy(src, dst, 8192)
    torch.cuda.synchronize()
    del src, dst


# ---- the benchmark workload ------------------------------------------------------
def run_main(torch, rss, dev, X, Bm, Cm, DT, A, args):
    wl = workloads.get(WORKLOAD)
    Bt, H, P, N, G, W = wl.batch, wl.nheads, wl.headdim, wl.dstate, wl.ngroups, wl.window
    cfg = rss.make_config(Bt, H, P, N, G, W, wl.capacity, 0, rss.RSS_DTYPE_BF16, rss.RSS_COPY_NONE)
    layer = rss.ReplayLayer(cfg, A, dev)
    y = torch.empty((Bt, H, P), device=dev)
    T = X.shape[0]
    fused = not args.separate_flush

    def step(k, lt=None):
        i = k % T
        fold = (k + 1) % W == 0
        if fused and fold:   # this token fills every window: decode and fold in one pass
            f = lambda: layer.decode_flush_step(W, X[i], Bm[i], Cm[i], DT[i], y)  # noqa: E731
            key = "fused"
        else:
            f = lambda: layer.decode_step(X[i], Bm[i], Cm[i], DT[i], y)  # noqa: E731
            key = f"replay{k % W}"
        if lt is None:
            f()
        else:
            lt.around(key, f)
        if fold and not fused:
            g = lambda: layer.flush_checkpoint(W)  # noqa: E731
            if lt is None:
                g()
            else:
                lt.around("flush", g)

    def repeats(nsteps, warm, reps):
        out = []
        for _ in range(reps):
            layer.init_state()
            for k in range(warm):
                step(k)
            out.append(_timed(torch, step, nsteps, start=warm))
        return out

    # value: exactly --steps steps after --warmup steps, median of the repeats
    reps_ms = repeats(args.steps, args.warmup, max(1, args.repeats))
    ms = float(np.median(reps_ms))
    # steady state: whole windows, starting at a window boundary
    ss_steps = whole(args.steps, W, 4 * W)
    ss_warm = whole(args.warmup, W, W)
    ss_ms = float(np.median(repeats(ss_steps, ss_warm, 3)))
    # per-launch durations (HIP events on the launch stream), in a further pass
    lt = Launches(torch)
    layer.init_state()
    for k in range(ss_warm):
        step(k)
    for k in range(ss_warm, ss_warm + ss_steps):
        step(k, lt)
    torch.cuda.synchronize()
    assert layer.device_error() == 0
    rep_us, rep_bytes = 0.0, 0
    n_rep = 0
    for n0 in range(W):
        d = lt.us(f"replay{n0}")
        rep_us += sum(d)
        rep_bytes += len(d) * replay_bytes(wl, n0) * Bt * H
        n_rep += len(d)
    fold_key, fold_b = ("fused", fused_bytes(wl)) if fused else ("flush", flush_bytes(wl, W))
    f_us = lt.us(fold_key)
    step_us = []
    kernels = {"replay_decode": {"avg_us": rep_us / n_rep, "GBps": rate(rep_bytes, rep_us),
                                 "frac_of_peak": rate(rep_bytes, rep_us) / PEAK_HBM_GBS,
                                 "launches": n_rep, "algorithmic_bytes_per_launch": rep_bytes / n_rep},
               ("fused_decode_fold" if fused else "flush"): {
                   "avg_us": float(np.mean(f_us)), "GBps": rate(fold_b * Bt * H * len(f_us), sum(f_us)),
                   "frac_of_peak": rate(fold_b * Bt * H * len(f_us), sum(f_us)) / PEAK_HBM_GBS,
                   "launches": len(f_us), "algorithmic_bytes_per_launch": fold_b * Bt * H}}
    for n0 in range(W):
        step_us += lt.us(f"replay{n0}")
    step_us += f_us
    return {"tokens_per_s": Bt * args.steps / (ms / 1e3), "ms": ms, "reps_ms": reps_ms,
            "steady": {"tokens_per_s": Bt * ss_steps / (ss_ms / 1e3), "steps": ss_steps,
                       "folds_timed": ss_steps // W, "ms_per_step": ss_ms / ss_steps},
            "kernels": kernels, "rep_us": rep_us / n_rep, "rep_gbs": rate(rep_bytes, rep_us),
            "rep_bytes": rep_bytes / n_rep, "step_us": step_us, "cfg": cfg, "fused": fused}


def run_eager(torch, rss, dev, X, Bm, Cm, DT, A, cfg, steps, warmup):
    wl = workloads.get(WORKLOAD)
    Bt, H, P, N, W = wl.batch, wl.nheads, wl.headdim, wl.dstate, wl.window
    T = X.shape[0]
    S = torch.zeros((Bt, H, P, N), device=dev)
    ye = torch.empty((Bt, H, P), device=dev)

    def eager_step(k):
        i = k % T
        rss.rss_eager_step(cfg, S, X[i], Bm[i], Cm[i], DT[i], A, ye)
    for k in range(warmup):
        eager_step(k)
    ems = _timed(torch, eager_step, steps, start=warmup)
    lt = Launches(torch)
    for k in range(steps):
        lt.around("e", lambda k=k: eager_step(k))
    torch.cuda.synchronize()
    e_us = lt.us("e")
    out = {"tokens_per_s": Bt * steps / (ems / 1e3), "ms_per_step": ems / steps,
           "kernel_avg_us": float(np.mean(e_us)),
           "kernel_GBps": rate(eager_bytes(wl) * Bt * H * len(e_us), sum(e_us)),
           "bytes_per_token": eager_bytes(wl) * H}
    # Parity of the timed path on the whole batch: a fresh replay layer (the
    # benchmark's schedule) and a fresh eager state run 2W steps side by side.
    S.zero_()
    y = torch.empty_like(ye)
    chk = rss.ReplayLayer(cfg, A, dev)
    chk.init_state()
    num = den = worst = 0.0
    for k in range(2 * W):
        i = k % T
        if (k + 1) % W == 0:
            chk.decode_flush_step(W, X[i], Bm[i], Cm[i], DT[i], y)
        else:
            chk.decode_step(X[i], Bm[i], Cm[i], DT[i], y)
        rss.rss_eager_step(cfg, S, X[i], Bm[i], Cm[i], DT[i], A, ye)
        d2 = float(torch.sum((y - ye).double() ** 2))
        r2 = float(torch.sum(ye.double() ** 2))
        num, den = num + d2, den + r2
        worst = max(worst, (d2 / r2) ** 0.5)
    assert chk.device_error() == 0
    out["parity_replay_vs_eager"] = {"steps": 2 * W, "run_rel_l2": (num / den) ** 0.5,
                                     "worst_step_rel_l2": worst}
    return out


# ---- further workloads, each over whole windows -----------------------------------
def run_stagger(torch, rss, dev, X, Bm, Cm, DT, A, steps, warmup):
    """The benchmark workload with staggered folds: sequence b's first window is
    1 + (b mod W) tokens long (per-sequence fold thresholds), W after that, so
    every step folds ~Bt/W sequences inside the fused decode instead of all of
    them on one step in W. Same inputs, same bytes per token."""
    wl = workloads.get(WORKLOAD)
    Bt, H, P, N, W = wl.batch, wl.nheads, wl.headdim, wl.dstate, wl.window
    cfg = rss.make_config(Bt, H, P, N, wl.ngroups, W, wl.capacity, 0, rss.RSS_DTYPE_BF16,
                          rss.RSS_COPY_NONE)
    layer = rss.ReplayLayer(cfg, A, dev)
    layer.init_state()
    y = torch.empty((Bt, H, P), device=dev)
    T = X.shape[0]
    first = 1 + np.arange(Bt) % W
    th = [torch.from_numpy(np.where(t < first, first, W).astype(np.int32)).to(dev) for t in range(W + 1)]

    def step(k):
        i = k % T
        layer.decode_flush_step_each(th[min(k, W)], X[i], Bm[i], Cm[i], DT[i], y)
    k0 = whole(warmup, W, W)
    for k in range(k0):
        step(k)
    ms = _timed(torch, step, steps, start=k0)
    lt = Launches(torch)
    for k in range(k0 + steps, k0 + 2 * steps):
        lt.around("s", lambda k=k: step(k))
    torch.cuda.synchronize()
    d = np.array(lt.us("s"))
    assert layer.device_error() == 0
    return {"tokens_per_s": Bt * steps / (ms / 1e3), "steps": steps,
            "step_us_median": float(np.median(d)), "step_us_max": float(d.max()),
            "step_us_min": float(d.min())}


def run_grouped(torch, rss, dev, X, Bm, Cm, DT, A, steps, warmup, groups=1):
    """The benchmark workload with B and C shared by groups of heads (G = 1: one
    B, C row per sequence, as in Mamba-2 models with a single group): the same x
    and dt, B and C taken from the first group of the same inputs. The ring's B
    rows shrink by H/G, so fewer bytes per token; replay + fused fold schedule,
    and the eager kernel on the same inputs."""
    wl = workloads.get(WORKLOAD)
    Bt, H, P, N, W = wl.batch, wl.nheads, wl.headdim, wl.dstate, wl.window
    B1 = Bm[:, :, :groups, :].contiguous()
    C1 = Cm[:, :, :groups, :].contiguous()
    cfg = rss.make_config(Bt, H, P, N, groups, W, wl.capacity, 0, rss.RSS_DTYPE_BF16,
                          rss.RSS_COPY_NONE)
    layer = rss.ReplayLayer(cfg, A, dev)
    layer.init_state()
    y = torch.empty((Bt, H, P), device=dev)
    T = X.shape[0]

    def step(k):
        i = k % T
        if (k + 1) % W == 0:
            layer.decode_flush_step(W, X[i], B1[i], C1[i], DT[i], y)
        else:
            layer.decode_step(X[i], B1[i], C1[i], DT[i], y)
    k0 = whole(warmup, W, W)
    for k in range(k0):
        step(k)
    ms = _timed(torch, step, steps, start=k0)
    S = torch.zeros((Bt, H, P, N), device=dev)
    ye = torch.empty_like(y)

    def eager(k):
        i = k % T
        rss.rss_eager_step(cfg, S, X[i], B1[i], C1[i], DT[i], A, ye)
    for k in range(k0):
        eager(k)
    ms_e = _timed(torch, eager, steps, start=k0)
    assert layer.device_error() == 0
    return {"groups": groups, "steps": steps, "tokens_per_s": Bt * steps / (ms / 1e3),
            "eager_tokens_per_s": Bt * steps / (ms_e / 1e3), "speedup": ms_e / ms}


def run_lowp(torch, rss, dev, X, Bm, Cm, DT, A, steps, warmup, mode="bf16", window=16, separate=False):
    """Replay with a bf16 tile read, W = window, same inputs: dual precision
    (fp32 master + bf16 read copy, mode "bf16"; the token that fills every
    window is decoded and folded in one pass from the fp32 master) or a single
    bf16 checkpoint ("bf16_state"; folded inside the two-wavefront decode that
    fills the window). `steps` is a whole number of windows, and the timed
    region starts at a window boundary. separate=True times the dual mode's
    other plan instead: the replay of the copy, then the flush launch."""
    wl = workloads.get(f"mamba2_dual_b256_h128_p64_n128_w{window}").replace(read_copy=mode)
    Bt, H, P, N, W = wl.batch, wl.nheads, wl.headdim, wl.dstate, wl.window
    assert steps % W == 0
    code = rss.RSS_COPY_BF16 if mode == "bf16" else rss.RSS_STATE_BF16
    cfg = rss.make_config(Bt, H, P, N, wl.ngroups, W, wl.capacity, 0, rss.RSS_DTYPE_BF16, code)
    layer = rss.ReplayLayer(cfg, A, dev)
    layer.init_state()
    y = torch.empty((Bt, H, P), device=dev)
    T = X.shape[0]
    fused = not separate

    def step(k, lt=None):
        i = k % T
        fold = (k + 1) % W == 0
        if fold and fused:
            f, key = (lambda: layer.decode_flush_step(W, X[i], Bm[i], Cm[i], DT[i], y)), "f"  # noqa: E731
        else:
            f, key = (lambda: layer.decode_step(X[i], Bm[i], Cm[i], DT[i], y)), f"r{k % W}"  # noqa: E731
        if lt is None:
            f()
        else:
            lt.around(key, f)
        if fold and not fused:
            g = lambda: layer.flush_checkpoint(W)  # noqa: E731
            if lt is None:
                g()
            else:
                lt.around("f", g)
    k0 = whole(warmup, W, W)
    for k in range(k0):
        step(k)
    ms = _timed(torch, step, steps, start=k0)
    lt = Launches(torch)
    for k in range(k0 + steps, k0 + 2 * steps):
        step(k, lt)
    torch.cuda.synchronize()
    r_us = r_b = 0
    n_r = 0
    for n0 in range(W):
        d = lt.us(f"r{n0}")
        r_us += sum(d)
        r_b += len(d) * replay_bytes(wl, n0) * Bt * H
        n_r += len(d)
    f_us = lt.us("f")
    per_fold = (fused_bytes(wl) if mode == "bf16_state" else dual_fused_bytes(wl)) if fused else flush_bytes(wl, W)
    assert layer.device_error() == 0
    return {"workload": wl.name if mode == "bf16" else wl.name + " with a bf16-only checkpoint",
            "steps": steps, "folds_timed": steps // W,
            "tokens_per_s": Bt * steps / (ms / 1e3),
            "replay_avg_us": r_us / n_r, "replay_GBps": rate(r_b, r_us),
            "fold": ("fused into the decode that fills the window" if mode == "bf16_state" else
                     "one pass from the fp32 master on the token that fills every window") if fused
                    else "separate flush launch",
            "fold_avg_us": float(np.mean(f_us)),
            "fold_GBps": rate(per_fold * Bt * H * len(f_us), sum(f_us)),
            "fold_frac_of_peak": rate(per_fold * Bt * H * len(f_us), sum(f_us)) / PEAK_HBM_GBS}


def run_eager_bf16(torch, rss, dev, X, Bm, Cm, DT, A, steps, warmup):
    """Eager decode with the state stored in bf16 (rounded every token): the
    low-precision eager point of comparison, same inputs and shape."""
    wl = workloads.get(WORKLOAD)
    Bt, H, P, N = wl.batch, wl.nheads, wl.headdim, wl.dstate
    cfg = rss.make_config(Bt, H, P, N, wl.ngroups, wl.window, wl.capacity, 0, rss.RSS_DTYPE_BF16,
                          rss.RSS_STATE_BF16)
    S = torch.zeros((Bt, H, P, N), dtype=torch.bfloat16, device=dev)
    y = torch.empty((Bt, H, P), device=dev)
    T = X.shape[0]

    def step(k):
        i = k % T
        rss.rss_eager_step(cfg, S, X[i], Bm[i], Cm[i], DT[i], A, y)
    for k in range(warmup):
        step(k)
    ms = _timed(torch, step, steps, start=warmup)
    return {"tokens_per_s": Bt * steps / (ms / 1e3), "kernel_avg_us": ms / steps * 1e3,
            "kernel_GBps": eager_bytes(wl, 2) * Bt * H * steps / (ms / 1e3) / 1e9,
            "bytes_per_token": eager_bytes(wl, 2) * H}


def run_spec(torch, rss, dev, warmup=8, rounds=None):
    """Speculative rounds at batch 512, K = 4, over the workload's 200 rounds
    (or `rounds`), each with its own draft inputs (drawn on the device) and
    accepted lengths: verify with the committed window's fold in the same pass
    + rollback, the same with a separate flush launch, and the eager kernel
    with a state snapshot per draft token."""
    wl = workloads.get("mamba2_spec_b512_h128_p64_n128_w16_k4")
    Bt, H, P, N, G, W, K = wl.batch, wl.nheads, wl.headdim, wl.dstate, wl.ngroups, wl.window, wl.draft
    R = rounds or wl.rounds
    D = [synth.device_draft_inputs(wl, r, dev) for r in range(R)]
    NACC = [synth.accepted_drafts(wl, r) for r in range(R)]
    NDROP = [torch.from_numpy((K - n).astype(np.int32)).to(dev) for n in NACC]
    SRC = [torch.from_numpy(n.astype(np.int32)).to(dev) for n in NACC]
    A = torch.from_numpy(synth.params(wl)["A"]).to(dev)
    cfg = rss.make_config(Bt, H, P, N, G, W, wl.capacity, K, rss.RSS_DTYPE_BF16, rss.RSS_COPY_NONE)
    layer = rss.ReplayLayer(cfg, A, dev)
    y = torch.empty((Bt, K + 1, H, P), device=dev)

    def sep_round(r, lt=None):   # verify, rollback, then a flush of the windows the accepted tokens filled
        d = D[r % R]
        f = lambda: layer.verify_k_tokens(K, d["x"], d["B"], d["C"], d["dt"], y)  # noqa: E731
        f() if lt is None else lt.around("v", f)
        layer.rollback(NDROP[r % R])
        layer.flush_checkpoint(W)

    def rep_round(r, lt=None):   # the fold of a full committed window rides on the next verify
        d = D[r % R]
        f = lambda: layer.verify_k_tokens_fold(W, K, d["x"], d["B"], d["C"], d["dt"], y)  # noqa: E731
        f() if lt is None else lt.around("vf", f)
        layer.rollback(NDROP[r % R])

    def timed_schedule(fn):
        layer.init_state()
        for r in range(warmup):
            fn(r)
        layer.init_state()
        return _timed(torch, fn, R)
    ms_rep = timed_schedule(rep_round)
    ms_sep = timed_schedule(sep_round)
    # per-launch durations and algorithmic bytes (window lengths replayed on the host)
    committed = sum(int(np.sum(n + 1)) for n in NACC)
    lt = Launches(torch)
    lens = np.zeros(Bt, np.int64)
    vbytes = 0
    layer.init_state()
    for r in range(R):
        sep_round(r, lt)
        vbytes += verify_bytes(wl, lens, np.zeros(Bt, bool))
        lens += NACC[r] + 1
        lens[lens >= W] = 0
    lens[:] = 0
    vfbytes = 0
    layer.init_state()
    for r in range(R):
        fold = lens >= W
        rep_round(r, lt)
        vfbytes += verify_bytes(wl, lens, fold)
        lens[fold] = 0
        lens += NACC[r] + 1
    torch.cuda.synchronize()
    assert layer.device_error() == 0
    v_us, vf_us = lt.us("v"), lt.us("vf")
    del layer
    # eager baseline: K+1 eager tokens from slot src, snapshot i -> slot i;
    # rolling back to n_acc accepted drafts = next round reads slot n_acc
    pool = torch.zeros((Bt, K + 1, H, P, N), device=dev)
    src = [torch.zeros((Bt,), dtype=torch.int32, device=dev)]

    def eag_round(r, lt=None):
        d = D[r % R]
        f = lambda: rss.rss_eager_verify(cfg, pool, src[0], K, d["x"], d["B"], d["C"], d["dt"], A, y)  # noqa: E731
        f() if lt is None else lt.around("e", f)
        src[0] = SRC[r % R]
    for r in range(warmup):
        eag_round(r)
    pool.zero_()
    src[0] = torch.zeros((Bt,), dtype=torch.int32, device=dev)
    ms_eag = _timed(torch, eag_round, R)
    lt2 = Launches(torch)
    for r in range(R):
        eag_round(r, lt2)
    torch.cuda.synchronize()
    e_us = lt2.us("e")
    ebytes = H * Bt * ((K + 2) * P * N * 4 + (K + 1) * (2 * P + 4 * N + 4 + 4 * P) + 4)
    # of which written: a state snapshot and a y row per token
    ewrite = H * Bt * (K + 1) * (P * N * 4 + 4 * P)
    del pool, D
    return {"workload": wl.name, "rounds": R, "inputs": "fresh draws every round (device generator)",
            "committed_tokens": committed,
            "replay_committed_tokens_per_s": committed / (ms_rep / 1e3),
            "schedule": "verify with the committed-window fold in the same pass, then rollback",
            "replay_separate_flush_committed_tokens_per_s": committed / (ms_sep / 1e3),
            "eager_snapshot_committed_tokens_per_s": committed / (ms_eag / 1e3),
            "speedup": ms_eag / ms_rep,
            "verify_avg_us": float(np.mean(v_us)), "verify_GBps": rate(vbytes, sum(v_us)),
            "verify_frac_of_peak": rate(vbytes, sum(v_us)) / PEAK_HBM_GBS,
            "verify_fold_avg_us": float(np.mean(vf_us)), "verify_fold_GBps": rate(vfbytes, sum(vf_us)),
            "verify_fold_frac_of_peak": rate(vfbytes, sum(vf_us)) / PEAK_HBM_GBS,
            "eager_verify_avg_us": float(np.mean(e_us)),
            "eager_verify_GBps": rate(ebytes * len(e_us), sum(e_us)),
            "eager_verify_read_bytes": ebytes - ewrite, "eager_verify_write_bytes": ewrite}


def run_gdn(torch, rss, dev, steps, warmup, name="gdn_b256_h32_d128_w16"):
    """Gated DeltaNet (or, with the KDA workload, Kimi Delta Attention) decode at
    batch 256, 32 heads, d_k = d_v = 128: replay with the fold inside the decode
    that fills the window (and with a separate flush launch), against the eager
    delta-rule kernel. `steps` distinct inputs, drawn on the device."""
    wl = workloads.get(name)
    kda = wl.kind == "kda"
    Bt, H, P, N, W = wl.batch, wl.nheads, wl.headdim, wl.dstate, wl.window
    assert steps % W == 0
    D = [synth.device_delta_inputs(wl, t, dev) for t in range(steps)]
    cfg = rss.make_config(Bt, H, P, N, H, W, wl.capacity, 0, rss.RSS_DTYPE_F32, rss.RSS_COPY_NONE,
                          rss.RSS_KIND_KDA if kda else rss.RSS_KIND_GDN)
    layer = rss.ReplayLayer(cfg, None, dev)
    decode = layer.kda_decode_step if kda else layer.gdn_decode_step
    decode_fold = layer.kda_decode_flush_step if kda else layer.gdn_decode_flush_step
    eager_step = rss.rss_kda_eager_step if kda else rss.rss_gdn_eager_step
    o = torch.empty((Bt, H, P), device=dev)

    def args(k):
        d = D[k % steps]
        return d["q"], d["k"], d["v"], d["beta"], d["alpha"], o

    def fused_step(k, lt=None):  # the window-filling token folds in the same pass
        if (k + 1) % W == 0:
            f, key = (lambda: decode_fold(W, *args(k))), "fused"  # noqa: E731
        else:
            f, key = (lambda: decode(*args(k))), f"r{k % W}"  # noqa: E731
        f() if lt is None else lt.around(key, f)

    def sep_step(k, lt=None):
        f = lambda: decode(*args(k))  # noqa: E731
        f() if lt is None else lt.around(f"r{k % W}", f)
        if (k + 1) % W == 0:
            g = lambda: layer.flush_checkpoint(W)  # noqa: E731
            g() if lt is None else lt.around("flush", g)

    k0 = whole(warmup, W, W)

    def timed(fn):
        layer.init_state()
        for k in range(k0):
            fn(k)
        return _timed(torch, fn, steps, start=k0)
    ms_fused = timed(fused_step)
    ms_sep = timed(sep_step)
    lt = Launches(torch)
    layer.init_state()
    for k in range(steps):
        fused_step(k, lt)
    layer.init_state()
    for k in range(steps):
        sep_step(k, lt)
    torch.cuda.synchronize()
    assert layer.device_error() == 0
    r_us = r_b = n_r = 0
    for n0 in range(W):
        d = lt.us(f"r{n0}")
        r_us += sum(d)
        r_b += len(d) * gdn_bytes(wl, n0)["replay"] * Bt * H
        n_r += len(d)
    fb = gdn_bytes(wl, W)
    fu_us, fl_us = lt.us("fused"), lt.us("flush")
    del layer, decode, decode_fold
    S = torch.zeros((Bt, H, P, N), device=dev)

    def eager(k):
        eager_step(cfg, S, *args(k))
    for k in range(k0):
        eager(k)
    ems = _timed(torch, eager, steps, start=k0)
    lt2 = Launches(torch)
    for k in range(steps):
        lt2.around("e", lambda k=k: eager(k))
    torch.cuda.synchronize()
    e_us = lt2.us("e")
    del D
    return {"workload": wl.name, "steps": steps, "folds_timed": steps // W,
            "replay_tokens_per_s": Bt * steps / (ms_fused / 1e3),
            "schedule": "replay, the window-filling token folds in the same pass",
            "replay_separate_flush_tokens_per_s": Bt * steps / (ms_sep / 1e3),
            "eager_tokens_per_s": Bt * steps / (ems / 1e3), "speedup": ems / ms_fused,
            "replay_avg_us": r_us / n_r, "replay_GBps": rate(r_b, r_us),
            "fused_avg_us": float(np.mean(fu_us)),
            "fused_GBps": rate(fb["fused"] * Bt * H * len(fu_us), sum(fu_us)),
            "fused_frac_of_peak": rate(fb["fused"] * Bt * H * len(fu_us), sum(fu_us)) / PEAK_HBM_GBS,
            "flush_avg_us": float(np.mean(fl_us)),
            "flush_GBps": rate(fb["flush"] * Bt * H * len(fl_us), sum(fl_us)),
            "eager_avg_us": float(np.mean(e_us)),
            "eager_GBps": rate(fb["eager"] * Bt * H * len(e_us), sum(e_us))}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--pool", type=int, default=256, help="distinct decode steps kept in HBM")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-eager", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 1 GiB -> 1 GiB copy with the library's copy kernel (counter scaling)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed repeats of --steps steps (each after a fresh init); median reported")
    ap.add_argument("--separate-flush", action="store_true",
                    help="fold with a separate flush launch instead of the fused decode+fold")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the further workloads (dual precision, speculative, GDN, ...)")
    ap.add_argument("--spec-rounds", type=int, default=0,
                    help="speculative rounds to run (default: the workload's 200)")
    ap.add_argument("--phase-markers", action="store_true",
                    help="launch a tiny marker kernel before each section (for profiler runs)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the decode path has no cross-GPU step, and every "
              "(sequence, head) shard runs the same kernel at a smaller batch. Run with --gpus 1.",
              file=sys.stderr)
        return 2

    wl = workloads.get(WORKLOAD)
    Bt, H, P, N, G, W = wl.batch, wl.nheads, wl.headdim, wl.dstate, wl.ngroups, wl.window
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    # Host-side work that forks (input pool, CPU baseline) runs before the device
    # is touched.
    t0 = time.perf_counter()
    pool = gen_pool(wl, args.pool, workers)
    gen_s = time.perf_counter() - t0
    cpu = None if args.no_cpu_baseline else cpu_baseline(wl, pool, args.cpu_seconds, workers)

    import torch
    from recurrent_state_storage_amd import rss

    dev = torch.device("cuda:0")
    X = torch.from_numpy(pool[0].view(np.int16)).view(torch.bfloat16).to(dev)
    Bm = torch.from_numpy(pool[1].view(np.int16)).view(torch.bfloat16).to(dev)
    Cm = torch.from_numpy(pool[2].view(np.int16)).view(torch.bfloat16).to(dev)
    DT = torch.from_numpy(pool[3]).to(dev)
    A = torch.from_numpy(synth.params(wl)["A"]).to(dev)

    mark = PhaseMarker(torch, rss, dev, args.phase_markers)
    mark("main")
    main_run = run_main(torch, rss, dev, X, Bm, Cm, DT, A, args)
    cfg, fused = main_run["cfg"], main_run["fused"]
    mark("eager")
    out_eager = None if args.no_eager else run_eager(torch, rss, dev, X, Bm, Cm, DT, A, cfg,
                                                     args.steps, args.warmup)
    mark("calibration")
    calib = run_calibration(torch, rss, dev)
    if args.calibrate_copy:
        calibrate_counters(torch, rss, dev)

    # Bytes per decoded token per layer (analytic): state tiles, and everything.
    st_eager = 2 * P * N * 4 * H
    if fused:
        tot_replay = (sum(replay_bytes(wl, n) for n in range(W - 1)) + fused_bytes(wl)) / W * H
    else:
        tot_replay = (sum(replay_bytes(wl, n) for n in range(W)) / W + flush_bytes(wl, W) / W) * H
    st_replay = P * N * 4 * H + (P * N * 4 * H / W if fused else 2 * P * N * 4 * H / W)
    traffic = counter_traffic()
    # Measured bytes per token over one window (W - 1 replay launches and the
    # fused one) against the eager launch, both from the HBM counters.
    c_fused, c_eager = counter_traffic("fused"), counter_traffic("eager")
    meas_replay = ((W - 1) * traffic + c_fused) / W / Bt if traffic and c_fused and fused else None
    meas_eager = c_eager / Bt if c_eager else None
    kern = main_run["kernels"]
    fk = "fused_decode_fold" if fused else "flush"
    rec = {
        "metric": METRIC,
        "value": main_run["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_run["ms"] / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "batch": Bt, "heads": H, "headdim": P, "dstate": N,
                   "groups": G, "window": W, "xBC_storage": "bf16", "state": "f32",
                   "fold": "fused into the window-filling decode" if fused else "separate flush",
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": main_run["rep_gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": main_run["rep_gbs"] / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": "replay decode", "avg_launch_us": main_run["rep_us"],
                     "algorithmic_bytes_per_launch": main_run["rep_bytes"]},
        "steady_state_tokens_per_s": main_run["steady"]["tokens_per_s"],
        "steady_state": main_run["steady"],
        "kernels": kern,
        "step_us": {"median": float(np.median(main_run["step_us"])),
                    "max": float(np.max(main_run["step_us"]))},
        "repeats_ms": main_run["reps_ms"],
        "context": dict(calib, **{
            "replay_frac_of_read_ceiling": main_run["rep_gbs"] / calib["read_ceiling_GBps"],
            "replay_frac_of_tile_read_write": main_run["rep_gbs"] / calib["tile_read_write_GBps"],
            "fold_frac_of_copy_ceiling": kern[fk]["GBps"] / calib["copy_ceiling_GBps"],
            "eager_frac_of_copy_ceiling": (out_eager["kernel_GBps"] / calib["copy_ceiling_GBps"]
                                           if out_eager else None),
            "fold_frac_of_tile_copy": kern[fk]["GBps"] / calib["tile_copy_GBps"],
            "eager_frac_of_tile_copy": (out_eager["kernel_GBps"] / calib["tile_copy_GBps"]
                                        if out_eager else None)}),
        "eager_baseline": out_eager,
        "bytes_per_token": {"replay_state": st_replay, "eager_state": st_eager,
                            "state_ratio": st_replay / st_eager, "replay_total": tot_replay,
                            "eager_total": eager_bytes(wl) * H,
                            "total_ratio": tot_replay / (eager_bytes(wl) * H),
                            "replay_decode_launch_analytic": main_run["rep_bytes"] / Bt,
                            "replay_decode_launch_counters": traffic / Bt if traffic else None,
                            "replay_window_counters": meas_replay,
                            "eager_counters": meas_eager,
                            "total_ratio_counters": (meas_replay / meas_eager
                                                     if meas_replay and meas_eager else None)},
        "input_generation_s": gen_s,
    }
    if out_eager:
        rec["speedup_vs_eager_gpu"] = main_run["tokens_per_s"] / out_eager["tokens_per_s"]
        rec["steady_state_speedup_vs_eager_gpu"] = (main_run["steady"]["tokens_per_s"] /
                                                    out_eager["tokens_per_s"])
    if not args.no_extra:
        sub = whole(args.steps, max(SWEEP_WINDOWS), 64)   # whole windows of every W swept
        rec["sub_measurement_steps"] = sub
        mark("staggered")
        rec["staggered_folds"] = run_stagger(torch, rss, dev, X, Bm, Cm, DT, A, sub, args.warmup)
        mark("grouped")
        rec["grouped_bc"] = run_grouped(torch, rss, dev, X, Bm, Cm, DT, A, sub, args.warmup)
        mark("dual")
        rec["dual_precision"] = run_lowp(torch, rss, dev, X, Bm, Cm, DT, A, sub, args.warmup)
        sep_dual = run_lowp(torch, rss, dev, X, Bm, Cm, DT, A, sub, args.warmup, separate=True)
        rec["dual_precision"]["separate_flush"] = {
            k: sep_dual[k] for k in ("tokens_per_s", "replay_avg_us", "fold", "fold_avg_us", "fold_GBps",
                                     "fold_frac_of_peak")}
        by_window = {}
        for w in SWEEP_WINDOWS:
            mark(f"dual_w{w}")
            by_window[w] = {k: v for k, v in run_lowp(torch, rss, dev, X, Bm, Cm, DT, A, sub, args.warmup,
                                                      window=w).items() if k != "workload"}
        rec["dual_precision"]["by_window"] = by_window
        mark("bf16_checkpoint")
        bf16_ckpt = run_lowp(torch, rss, dev, X, Bm, Cm, DT, A, sub, args.warmup, mode="bf16_state")
        mark("eager_bf16")
        rec["low_precision"] = {
            "bf16_checkpoint": bf16_ckpt,
            "eager_bf16_state": run_eager_bf16(torch, rss, dev, X, Bm, Cm, DT, A, sub, args.warmup)}
        mark("speculative")
        rec["speculative"] = sp = run_spec(torch, rss, dev, rounds=args.spec_rounds or None)
        # the eager verify writes ~4.6x what it reads: its bound is the read
        # bytes at the read ceiling plus the written bytes at the write ceiling
        bound_us = (sp["eager_verify_read_bytes"] / calib["read_ceiling_GBps"] +
                    sp["eager_verify_write_bytes"] / calib["write_ceiling_GBps"]) / 1e3
        sp["eager_verify_frac_of_read_write_ceilings"] = bound_us / sp["eager_verify_avg_us"]
        sp["verify_frac_of_tile_read_verify_writes"] = sp["verify_GBps"] / calib["tile_read_verify_writes_GBps"]
        mark("gdn")
        rec["gated_deltanet"] = run_gdn(torch, rss, dev, sub, args.warmup)
        mark("kda")
        rec["kimi_delta_attention"] = run_gdn(torch, rss, dev, sub, args.warmup,
                                              name="kda_b256_h32_d128_w16")
        for key, kind in (("gated_deltanet", "gdn"), ("kimi_delta_attention", "kda")):
            rec[key]["replay_frac_of_tile_read_write"] = (rec[key]["replay_GBps"] /
                                                          calib["tile_read_delta_rule_writes"][kind]["GBps"])
    if cpu is not None:
        rec["cpu_baseline"] = cpu
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
