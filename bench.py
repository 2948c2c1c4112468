#!/usr/bin/env python3
"""Decode benchmark of the ReplaySSM hot path on one MI355X.

Workload: one Mamba-2 SSM layer in decode, batch 256, 128 heads x P=64 x N=128
(a 4 MiB fp32 state per sequence), bf16 x/B/C, fp32 dt and A, flush window
W=16, synthetic seeded inputs (workloads.synth; 256 distinct decode steps
resident in HBM before timing, cycled when more steps are timed).

A step is one decode token for the whole batch through the replay path: the
replay decode kernel every step, plus the checkpoint fold every W steps (the
fold's cost is part of the timed region). The eager-rewrite kernel on the same
inputs is timed too, so the state-traffic cut is measured.

Output: one JSON line with tokens/s per layer (whole-job throughput, inputs
already in HBM), the dominant kernel's roofline (algorithmic bytes per launch
over the HIP-event-measured launch duration, against 8 TB/s), and the fp64 CPU
oracle timed on a bounded sample on this host's cores.
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
KERNEL_SOURCES = ["replay.hip", "device.h", "limits.h", "launch.h", "lds.h"]


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


def eager_bytes(wl, state_bytes: int = 4) -> int:
    P, N, ib = wl.headdim, wl.dstate, 2 if wl.in_dtype == "bf16" else 4
    return 2 * P * N * state_bytes + P * ib + 2 * N * ib + 4 + P * 4 + 4


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


# ---- inputs -------------------------------------------------------------------
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


def _timed(torch, fn, n):
    """Run fn(i) for i < n between two events on the current stream; ms."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(n):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def run_lowp(torch, rss, dev, X, Bm, Cm, DT, A, steps, warmup, mode="bf16", window=16):
    """Replay with a bf16 tile read, W = window (16 by default), same inputs: dual precision (fp32
    master + bf16 read copy, mode "bf16"; the fold of the master is a separate
    flush launch) or a single bf16 checkpoint ("bf16_state"; folded inside the
    decode that fills the window)."""
    wl = workloads.get(f"mamba2_dual_b256_h128_p64_n128_w{window}").replace(read_copy=mode)
    Bt, H, P, N, W = wl.batch, wl.nheads, wl.headdim, wl.dstate, wl.window
    code = rss.RSS_COPY_BF16 if mode == "bf16" else rss.RSS_STATE_BF16
    cfg = rss.make_config(Bt, H, P, N, wl.ngroups, W, wl.capacity, 0, rss.RSS_DTYPE_BF16, code)
    layer = rss.ReplayLayer(cfg, A, dev)
    layer.init_state()
    y = torch.empty((Bt, H, P), device=dev)
    T = X.shape[0]
    fused = mode == "bf16_state"
    ev = {"r": [], "f": []}

    def mark(key):
        ev[key].append((torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)))
        ev[key][-1][0].record()

    def step(k, rec=False):
        i = k % T
        fold = (k + 1) % W == 0
        key = "f" if fold and fused else "r"
        if rec:
            mark(key)
        if fold and fused:
            layer.decode_flush_step(W, X[i], Bm[i], Cm[i], DT[i], y)
        else:
            layer.decode_step(X[i], Bm[i], Cm[i], DT[i], y)
        if rec:
            ev[key][-1][1].record()
        if fold and not fused:
            if rec:
                mark("f")
            layer.flush_checkpoint(W)
            if rec:
                ev["f"][-1][1].record()
    for k in range(warmup):
        step(k)
    ms = _timed(torch, lambda j: step(warmup + j), steps)
    base = warmup + steps
    for j in range(steps):
        step(base + j, rec=True)
    torch.cuda.synchronize()
    r_ms = sum(a.elapsed_time(b) for a, b in ev["r"])
    f_ms = sum(a.elapsed_time(b) for a, b in ev["f"])
    phases = [(base + j) % W for j in range(steps)]
    rbytes = sum(replay_bytes(wl, n0) for n0 in phases if not (fused and n0 == W - 1)) * Bt * H
    per_fold = fused_bytes(wl) if fused else flush_bytes(wl, W)
    fbytes = per_fold * Bt * H * len(ev["f"])
    assert layer.device_error() == 0
    return {"workload": wl.name if mode == "bf16" else wl.name + " with a bf16-only checkpoint",
            "tokens_per_s": Bt * steps / (ms / 1e3),
            "replay_avg_us": r_ms / max(len(ev["r"]), 1) * 1e3,
            "replay_GBps": rbytes / (r_ms / 1e3) / 1e9,
            "fold": "fused into the decode that fills the window" if fused else "separate flush launch",
            "fold_avg_us": f_ms / max(len(ev["f"]), 1) * 1e3,
            "fold_GBps": fbytes / (f_ms / 1e3) / 1e9 if f_ms else None}


def _gen_round(args):
    name, r = args
    wl = workloads.get(name)
    d = synth.draft_inputs(wl, r)
    return r, d["x_bits"], d["B_bits"], d["C_bits"], d["dt"], synth.accepted_drafts(wl, r)


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
    for k in range(max(warmup, W)):
        step(k)
    k0 = max(warmup, W)
    ms = _timed(torch, lambda j: step(k0 + j), steps)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for j in range(steps):
        ev[j][0].record()
        step(k0 + steps + j)
        ev[j][1].record()
    torch.cuda.synchronize()
    d = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    assert layer.device_error() == 0
    return {"tokens_per_s": Bt * steps / (ms / 1e3), "step_us_median": float(np.median(d)),
            "step_us_max": float(d.max()), "step_us_min": float(d.min())}


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
    for k in range(warmup):
        step(k)
    ms = _timed(torch, lambda j: step(warmup + j), steps)
    S = torch.zeros((Bt, H, P, N), device=dev)
    ye = torch.empty_like(y)

    def eager(k):
        i = k % T
        rss.rss_eager_step(cfg, S, X[i], B1[i], C1[i], DT[i], A, ye)
    for k in range(warmup):
        eager(k)
    ms_e = _timed(torch, lambda j: eager(warmup + j), steps)
    assert layer.device_error() == 0
    return {"groups": groups, "tokens_per_s": Bt * steps / (ms / 1e3),
            "eager_tokens_per_s": Bt * steps / (ms_e / 1e3), "speedup": ms_e / ms}


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
    ms = _timed(torch, lambda j: step(warmup + j), steps)
    return {"tokens_per_s": Bt * steps / (ms / 1e3), "kernel_avg_us": ms / steps * 1e3,
            "kernel_GBps": eager_bytes(wl, 2) * Bt * H * steps / (ms / 1e3) / 1e9,
            "bytes_per_token": eager_bytes(wl, 2) * H}


def run_spec(torch, rss, dev, rounds, warmup, workers, distinct=6):
    """Speculative rounds at batch 512, K = 4: replay verify + rollback + flush,
    against the eager kernel with a state snapshot per draft token."""
    wl = workloads.get("mamba2_spec_b512_h128_p64_n128_w16_k4")
    Bt, H, P, N, G, W, K = wl.batch, wl.nheads, wl.headdim, wl.dstate, wl.ngroups, wl.window, wl.draft
    with concurrent.futures.ProcessPoolExecutor(max_workers=min(workers, distinct)) as ex:
        got = sorted(ex.map(_gen_round, [(wl.name, r) for r in range(distinct)]))
    bf = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    RX = [bf(g[1]) for g in got]
    RB = [bf(g[2]) for g in got]
    RC = [bf(g[3]) for g in got]
    RD = [torch.from_numpy(g[4]).to(dev) for g in got]
    NACC = [g[5] for g in got]
    NDROP = [torch.from_numpy((K - n).astype(np.int32)).to(dev) for n in NACC]
    SRC = [torch.from_numpy(n.astype(np.int32)).to(dev) for n in NACC]
    A = torch.from_numpy(synth.params(wl)["A"]).to(dev)
    cfg = rss.make_config(Bt, H, P, N, G, W, wl.capacity, K, rss.RSS_DTYPE_BF16, rss.RSS_COPY_NONE)
    layer = rss.ReplayLayer(cfg, A, dev)
    layer.init_state()
    y = torch.empty((Bt, K + 1, H, P), device=dev)

    def sep_round(r):   # verify, rollback, then a flush of the windows the accepted tokens filled
        i = r % distinct
        layer.verify_k_tokens(K, RX[i], RB[i], RC[i], RD[i], y)
        layer.rollback(NDROP[i])
        layer.flush_checkpoint(W)

    def rep_round(r):   # the fold of a full committed window rides on the next verify
        i = r % distinct
        layer.verify_k_tokens_fold(W, K, RX[i], RB[i], RC[i], RD[i], y)
        layer.rollback(NDROP[i])
    for r in range(warmup):
        sep_round(r)
    ms_sep = _timed(torch, lambda j: sep_round(warmup + j), rounds)
    layer.init_state()
    for r in range(warmup):
        rep_round(r)
    ms_rep = _timed(torch, lambda j: rep_round(warmup + j), rounds)
    # per-kernel duration of the plain verify (separate-flush schedule), and its
    # algorithmic bytes from the window lengths
    layer.init_state()
    for r in range(warmup + rounds):
        sep_round(r)
    lens = np.zeros(Bt, np.int64)
    for r in range(warmup + rounds):        # replay the integer pointer rule on the host
        lens += K + 1 - (K - NACC[r % distinct])
        lens[lens >= W] = 0
    vev = []
    vbytes = 0
    entry = 2 * P + 2 * N + 8
    for j in range(rounds):
        r = warmup + rounds + j
        i = r % distinct
        vev.append((torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)))
        vev[-1][0].record()
        layer.verify_k_tokens(K, RX[i], RB[i], RC[i], RD[i], y)
        vev[-1][1].record()
        vbytes += H * int(np.sum(P * N * 4 + lens * entry + (K + 1) * (2 * P + 4 * N + 4 + 4 * P + entry) + 36))
        layer.rollback(NDROP[i])
        layer.flush_checkpoint(W)
        lens += K + 1 - (K - NACC[i])
        lens[lens >= W] = 0
    torch.cuda.synchronize()
    v_ms = sum(a.elapsed_time(b) for a, b in vev)
    assert layer.device_error() == 0
    committed = sum(int(np.sum(NACC[(warmup + j) % distinct] + 1)) for j in range(rounds))
    del layer
    # eager baseline: K+1 eager tokens from slot src, snapshot i -> slot i;
    # rolling back to n_acc accepted drafts = next round reads slot n_acc
    pool = torch.zeros((Bt, K + 1, H, P, N), device=dev)
    src = [torch.zeros((Bt,), dtype=torch.int32, device=dev)]

    def eag_round(r):
        i = r % distinct
        rss.rss_eager_verify(cfg, pool, src[0], K, RX[i], RB[i], RC[i], RD[i], A, y)
        src[0] = SRC[i]
    for r in range(warmup):
        eag_round(r)
    ms_eag = _timed(torch, lambda j: eag_round(warmup + j), rounds)
    eev = []
    for j in range(rounds):
        eev.append((torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)))
        eev[-1][0].record()
        eag_round(warmup + rounds + j)
        eev[-1][1].record()
    torch.cuda.synchronize()
    e_ms = sum(a.elapsed_time(b) for a, b in eev)
    ebytes = H * Bt * ((K + 2) * P * N * 4 + (K + 1) * (2 * P + 4 * N + 4 + 4 * P) + 4)
    del pool
    return {"workload": wl.name, "rounds": rounds,
            "replay_committed_tokens_per_s": committed / (ms_rep / 1e3),
            "schedule": "verify with the committed-window fold in the same pass, then rollback",
            "replay_separate_flush_committed_tokens_per_s": committed / (ms_sep / 1e3),
            "eager_snapshot_committed_tokens_per_s": committed / (ms_eag / 1e3),
            "speedup": ms_eag / ms_rep,
            "verify_avg_us": v_ms / rounds * 1e3, "verify_GBps": vbytes / (v_ms / 1e3) / 1e9,
            "eager_verify_avg_us": e_ms / rounds * 1e3,
            "eager_verify_GBps": ebytes / (e_ms / rounds / 1e3) / 1e9}


def gdn_bytes(wl, n0: int) -> dict:
    """Algorithmic bytes per (sequence, head) of the GDN / KDA kernels (fp32)."""
    P, N = wl.headdim, wl.dstate
    if wl.kind == "kda":
        entry = 8 * N + 4 * P                       # k, u, log-gate row
        inputs = 4 * N * 3 + 4 * P + 4              # q, k, alpha row, v, beta
    else:
        entry = 4 * N + 4 * P + 8                   # k, u, (1, log alpha)
        inputs = 4 * N * 2 + 4 * P + 8              # q, k, v, beta, alpha
    return {"replay": P * N * 4 + n0 * entry + inputs + 4 * P + entry + 32,
            "flush": 2 * P * N * 4 + wl.window * entry + 32,
            "eager": 2 * P * N * 4 + inputs + 4 * P}


def _gen_gdn(args):
    name, t = args
    wl = workloads.get(name)
    s = (synth.kda_step_inputs if wl.kind == "kda" else synth.gdn_step_inputs)(wl, t)
    return t, s


def run_gdn(torch, rss, dev, steps, warmup, workers, distinct=64, name="gdn_b256_h32_d128_w16"):
    """Gated DeltaNet (or, with the KDA workload, Kimi Delta Attention) decode at
    batch 256, 32 heads, d_k = d_v = 128: replay (+ flush every W) against the
    eager delta-rule kernel."""
    wl = workloads.get(name)
    kda = wl.kind == "kda"
    Bt, H, P, N, W = wl.batch, wl.nheads, wl.headdim, wl.dstate, wl.window
    with concurrent.futures.ProcessPoolExecutor(max_workers=min(workers, 16)) as ex:
        got = sorted(ex.map(_gen_gdn, [(wl.name, t) for t in range(distinct)]), key=lambda g: g[0])
    D = [{k: torch.from_numpy(v).to(dev) for k, v in g[1].items()} for g in got]
    cfg = rss.make_config(Bt, H, P, N, H, W, wl.capacity, 0, rss.RSS_DTYPE_F32, rss.RSS_COPY_NONE,
                          rss.RSS_KIND_KDA if kda else rss.RSS_KIND_GDN)
    layer = rss.ReplayLayer(cfg, None, dev)
    decode = layer.kda_decode_step if kda else layer.gdn_decode_step
    decode_fold = layer.kda_decode_flush_step if kda else layer.gdn_decode_flush_step
    eager_step = rss.rss_kda_eager_step if kda else rss.rss_gdn_eager_step
    layer.init_state()
    o = torch.empty((Bt, H, P), device=dev)
    evs = []

    def step(k, rec=False):
        d = D[k % distinct]
        if rec:
            evs.append([torch.cuda.Event(enable_timing=True) for _ in range(4)])
            evs[-1][0].record()
        decode(d["q"], d["k"], d["v"], d["beta"], d["alpha"], o)
        if rec:
            evs[-1][1].record()
        if (k + 1) % W == 0:
            if rec:
                evs[-1][2].record()
            layer.flush_checkpoint(W)
            if rec:
                evs[-1][3].record()
    def fused_step(k):  # the window-filling token folds in the same pass
        d = D[k % distinct]
        if (k + 1) % W == 0:
            decode_fold(W, d["q"], d["k"], d["v"], d["beta"], d["alpha"], o)
        else:
            decode(d["q"], d["k"], d["v"], d["beta"], d["alpha"], o)
    for k in range(warmup):
        fused_step(k)
    ms_fused = _timed(torch, lambda j: fused_step(warmup + j), steps)
    layer.init_state()
    for k in range(warmup):
        step(k)
    ms = _timed(torch, lambda j: step(warmup + j), steps)
    base = warmup + steps
    for j in range(steps):
        step(base + j, rec=True)
    torch.cuda.synchronize()
    r_ms = sum(e[0].elapsed_time(e[1]) for e in evs)
    f_list = [e[2].elapsed_time(e[3]) for j, e in enumerate(evs) if (base + j + 1) % W == 0]
    rbytes = sum(gdn_bytes(wl, (base + j) % W)["replay"] for j in range(steps)) * Bt * H
    assert layer.device_error() == 0
    del layer, decode, decode_fold
    S = torch.zeros((Bt, H, P, N), device=dev)

    def eager(k):
        d = D[k % distinct]
        eager_step(cfg, S, d["q"], d["k"], d["v"], d["beta"], d["alpha"], o)
    for k in range(warmup):
        eager(k)
    ems = _timed(torch, lambda j: eager(warmup + j), steps)
    eev = []
    for j in range(steps):
        eev.append((torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)))
        eev[-1][0].record()
        eager(j)
        eev[-1][1].record()
    torch.cuda.synchronize()
    e_ms = sum(a.elapsed_time(b) for a, b in eev)
    fb = gdn_bytes(wl, W)
    return {"workload": wl.name, "replay_tokens_per_s": Bt * steps / (ms_fused / 1e3),
            "schedule": "replay, the window-filling token folds in the same pass",
            "replay_separate_flush_tokens_per_s": Bt * steps / (ms / 1e3),
            "eager_tokens_per_s": Bt * steps / (ems / 1e3), "speedup": ems / ms_fused,
            "replay_avg_us": r_ms / steps * 1e3, "replay_GBps": rbytes / (r_ms / 1e3) / 1e9,
            "flush_avg_us": sum(f_list) / max(len(f_list), 1) * 1e3,
            "flush_GBps": fb["flush"] * Bt * H * len(f_list) / (sum(f_list) / 1e3) / 1e9 if f_list else None,
            "eager_avg_us": e_ms / steps * 1e3,
            "eager_GBps": fb["eager"] * Bt * H * steps / (e_ms / 1e3) / 1e9}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--pool", type=int, default=256, help="distinct decode steps kept in HBM")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-eager", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 1 GiB read + 1 GiB write elementwise kernel (counter scaling)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed repeats of --steps steps (each after a fresh init); median reported")
    ap.add_argument("--separate-flush", action="store_true",
                    help="fold with a separate flush launch instead of the fused decode+fold")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the dual-precision and speculative-verify measurements")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the decode path has no cross-GPU step, and every "
              "(sequence, head) shard runs the same kernel at a smaller batch. Run with --gpus 1.",
              file=sys.stderr)
        return 2

    import torch
    from recurrent_state_storage_amd import rss

    wl = workloads.get(WORKLOAD)
    Bt, H, P, N, G, W = wl.batch, wl.nheads, wl.headdim, wl.dstate, wl.ngroups, wl.window
    dev = torch.device("cuda:0")
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    t0 = time.perf_counter()
    pool = gen_pool(wl, args.pool, workers)
    gen_s = time.perf_counter() - t0
    # The host baseline runs before the device is touched (its workers are forked).
    cpu = None if args.no_cpu_baseline else cpu_baseline(wl, pool, args.cpu_seconds, workers)
    X = torch.from_numpy(pool[0].view(np.int16)).view(torch.bfloat16).to(dev)
    Bm = torch.from_numpy(pool[1].view(np.int16)).view(torch.bfloat16).to(dev)
    Cm = torch.from_numpy(pool[2].view(np.int16)).view(torch.bfloat16).to(dev)
    DT = torch.from_numpy(pool[3]).to(dev)
    A = torch.from_numpy(synth.params(wl)["A"]).to(dev)
    cfg = rss.make_config(Bt, H, P, N, G, W, wl.capacity, 0, rss.RSS_DTYPE_BF16, rss.RSS_COPY_NONE)
    layer = rss.ReplayLayer(cfg, A, dev)
    layer.init_state()
    y = torch.empty((Bt, H, P), device=dev)
    T = args.pool

    fused = not args.separate_flush

    def replay_step(k, ev=None):
        i = k % T
        fold = (k + 1) % W == 0
        if ev is not None:
            ev[0].record()
        if fold and fused:   # this token fills every window: decode and fold in one pass
            layer.decode_flush_step(W, X[i], Bm[i], Cm[i], DT[i], y)
        else:
            layer.decode_step(X[i], Bm[i], Cm[i], DT[i], y)
        if ev is not None:
            ev[1].record()
        if fold and not fused:
            if ev is not None:
                ev[2].record()
            layer.flush_checkpoint(W)
            if ev is not None:
                ev[3].record()

    # Repeats: each starts from a fresh init_state and W warm-up steps (untimed),
    # then exactly `steps` steps between two events; the median repeat is reported.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps_ms = []
    for _ in range(max(1, args.repeats)):
        layer.init_state()
        k = 0
        for _ in range(args.warmup):
            replay_step(k)
            k += 1
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            replay_step(k)
            k += 1
        e1.record()
        torch.cuda.synchronize()
        reps_ms.append(e0.elapsed_time(e1))
    ms = float(np.median(reps_ms))
    tok_s = Bt * args.steps / (ms / 1e3)

    # Per-kernel durations: HIP events around every launch on the launch stream,
    # in a second pass of the same length (so the timed pass above is unperturbed).
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    phase = []
    for j in range(args.steps):
        phase.append(k % W)
        replay_step(k, ev[j])
        k += 1
    torch.cuda.synchronize()
    # "replay decode" = the plain decode launches (window positions 0..W-2, and
    # W-1 too when the flush runs separately); the fold launches are reported apart.
    rep_ms, rep_bytes, n_rep, fl_ms, fl_bytes, n_fl = 0.0, 0, 0, 0.0, 0, 0
    for j in range(args.steps):
        d = ev[j][0].elapsed_time(ev[j][1])
        if phase[j] == W - 1 and fused:
            fl_ms += d
            fl_bytes += fused_bytes(wl) * Bt * H
            n_fl += 1
            continue
        rep_ms += d
        rep_bytes += replay_bytes(wl, phase[j]) * Bt * H
        n_rep += 1
        if phase[j] == W - 1:
            fl_ms += ev[j][2].elapsed_time(ev[j][3])
            fl_bytes += flush_bytes(wl, W) * Bt * H
            n_fl += 1
    step_us = [ev[j][0].elapsed_time(ev[j][1]) * 1e3 + (ev[j][2].elapsed_time(ev[j][3]) * 1e3
               if phase[j] == W - 1 and not fused else 0.0) for j in range(args.steps)]
    rep_avg_us = rep_ms / n_rep * 1e3
    rep_gbs = rep_bytes / (rep_ms / 1e3) / 1e9
    assert layer.device_error() == 0

    out_eager = None
    if not args.no_eager:
        S = torch.zeros((Bt, H, P, N), device=dev)
        ye = torch.empty_like(y)

        def eager_step(k):
            i = k % T
            rss.rss_eager_step(cfg, S, X[i], Bm[i], Cm[i], DT[i], A, ye)
        for j in range(args.warmup):
            eager_step(j)
        torch.cuda.synchronize()
        e0.record()
        for j in range(args.steps):
            eager_step(j)
        e1.record()
        torch.cuda.synchronize()
        ems = e0.elapsed_time(e1)
        eev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for j in range(args.steps):
            eev[j][0].record()
            eager_step(j)
            eev[j][1].record()
        torch.cuda.synchronize()
        eag_ms = sum(a.elapsed_time(b) for a, b in eev)
        out_eager = {
            "tokens_per_s": Bt * args.steps / (ems / 1e3), "ms_per_step": ems / args.steps,
            "kernel_avg_us": eag_ms / args.steps * 1e3,
            "kernel_GBps": eager_bytes(wl) * Bt * H * args.steps / (eag_ms / 1e3) / 1e9,
            "bytes_per_token": eager_bytes(wl) * H,
        }
        # Parity of the timed path on the whole batch: a fresh replay layer (the
        # benchmark's schedule) and a fresh eager state run 2W steps side by side.
        S.zero_()
        chk = rss.ReplayLayer(cfg, A, dev)
        chk.init_state()
        num = den = 0.0
        worst = 0.0
        for k in range(2 * W):
            i = k % T
            if (k + 1) % W == 0 and fused:
                chk.decode_flush_step(W, X[i], Bm[i], Cm[i], DT[i], y)
            else:
                chk.decode_step(X[i], Bm[i], Cm[i], DT[i], y)
                if (k + 1) % W == 0:
                    chk.flush_checkpoint(W)
            rss.rss_eager_step(cfg, S, X[i], Bm[i], Cm[i], DT[i], A, ye)
            d2 = float(torch.sum((y - ye).double() ** 2))
            r2 = float(torch.sum(ye.double() ** 2))
            num, den = num + d2, den + r2
            worst = max(worst, (d2 / r2) ** 0.5)
        assert chk.device_error() == 0
        out_eager["parity_replay_vs_eager"] = {"steps": 2 * W, "run_rel_l2": (num / den) ** 0.5,
                                               "worst_step_rel_l2": worst}
        del S, chk

    # Context: a plain device copy, 1 GiB read + 1 GiB written (torch's vectorised
    # elementwise kernel multiplying by 1, the faster of torch's copy paths here).
    csrc = torch.ones((1 << 28,), device=dev)
    cdst = torch.empty_like(csrc)
    torch.mul(csrc, 1.0, out=cdst)
    copy_ms = _timed(torch, lambda j: torch.mul(csrc, 1.0, out=cdst), 10) / 10
    copy_gbs = 2 * (1 << 30) / (copy_ms / 1e3) / 1e9
    del csrc, cdst

    if args.calibrate_copy:
        src = torch.ones((1 << 28,), device=dev)      # 1 GiB fp32
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

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
    rec = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "batch": Bt, "heads": H, "headdim": P, "dstate": N,
                   "groups": G, "window": W, "xBC_storage": "bf16", "state": "f32",
                   "fold": "fused into the window-filling decode" if fused else "separate flush",
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": rep_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": rep_gbs / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": "replay decode", "avg_launch_us": rep_avg_us,
                     "algorithmic_bytes_per_launch": rep_bytes / n_rep},
        "kernels": {
            "replay_decode": {"avg_us": rep_avg_us, "GBps": rep_gbs},
            ("fused_decode_fold" if fused else "flush"): {
                "avg_us": fl_ms / max(n_fl, 1) * 1e3,
                "GBps": fl_bytes / (fl_ms / 1e3) / 1e9 if n_fl else None, "launches": n_fl},
        },
        "step_us": {"median": float(np.median(step_us)), "max": float(np.max(step_us))},
        "repeats_ms": reps_ms,
        "context": {"device_copy_GBps": copy_gbs, "replay_frac_of_copy": rep_gbs / copy_gbs},
        "eager_baseline": out_eager,
        "bytes_per_token": {"replay_state": st_replay, "eager_state": st_eager,
                            "state_ratio": st_replay / st_eager, "replay_total": tot_replay,
                            "eager_total": eager_bytes(wl) * H,
                            "total_ratio": tot_replay / (eager_bytes(wl) * H),
                            "replay_decode_launch_analytic": rep_bytes / n_rep / Bt,
                            "replay_decode_launch_counters": traffic / Bt if traffic else None,
                            "replay_window_counters": meas_replay,
                            "eager_counters": meas_eager,
                            "total_ratio_counters": (meas_replay / meas_eager
                                                     if meas_replay and meas_eager else None)},
        "input_generation_s": gen_s,
    }
    if out_eager:
        rec["speedup_vs_eager_gpu"] = tok_s / out_eager["tokens_per_s"]
    if not args.no_extra:
        rec["staggered_folds"] = run_stagger(torch, rss, dev, X, Bm, Cm, DT, A, args.steps,
                                             args.warmup)
        rec["grouped_bc"] = run_grouped(torch, rss, dev, X, Bm, Cm, DT, A, args.steps, args.warmup)
        rec["dual_precision"] = run_lowp(torch, rss, dev, X, Bm, Cm, DT, A, args.steps, args.warmup)
        # the dual-precision window sweep (W = 8, 16, 32; R = W), same inputs
        rec["dual_precision"]["by_window"] = {
            w: {k: v for k, v in run_lowp(torch, rss, dev, X, Bm, Cm, DT, A, args.steps, args.warmup,
                                          window=w).items() if k != "workload"}
            for w in (8, 16, 32)}
        rec["low_precision"] = {
            "bf16_checkpoint": run_lowp(torch, rss, dev, X, Bm, Cm, DT, A, args.steps, args.warmup,
                                        mode="bf16_state"),
            "eager_bf16_state": run_eager_bf16(torch, rss, dev, X, Bm, Cm, DT, A, args.steps,
                                               args.warmup)}
        rec["speculative"] = run_spec(torch, rss, dev, rounds=48, warmup=8, workers=workers)
        rec["gated_deltanet"] = run_gdn(torch, rss, dev, steps=args.steps, warmup=args.warmup,
                                        workers=workers)
        rec["kimi_delta_attention"] = run_gdn(torch, rss, dev, steps=args.steps, warmup=args.warmup,
                                              workers=workers, name="kda_b256_h32_d128_w16")
    if cpu is not None:
        rec["cpu_baseline"] = cpu
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
