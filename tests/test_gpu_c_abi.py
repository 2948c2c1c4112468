"""The C ABI from a plain C++ caller: tests/c_abi/rss_c_driver (built by
__graft_entry__.build(); no torch, no Python) allocates every buffer from
rss_buffer_sizes with hipMalloc, binds a layer and runs init + decode (+ fold),
then speculative rounds (verify with fold, rollback), through the C entry
points, for each checkpoint precision. Its outputs, final checkpoint and pointers are checked here against
the fp64 oracle and the integer ring model."""
import os
import subprocess

import numpy as np
import pytest

from oracle import gdn, kda, mamba2
from oracle.lowp import round_bf16_from_f32
from oracle.ring import PointerModel
import workloads
from workloads import synth
from gpu_util import rel_l2, log

pytestmark = pytest.mark.gpu

DRIVER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "rss_c_driver")
BASE = workloads.get("tiny_b2_h4_p16_n16_w8")
COPY = {"none": 0, "bf16": 1, "bf16_state": 2}   # rss_config.read_copy codes (include/rss.h)
KIND = {"mamba2": 0, "gdn": 1, "kda": 2}           # rss_config.kind codes


def _write_tokens(f, s, bf16):
    for k in ("x", "B", "C"):
        if bf16:
            f.write(np.ascontiguousarray(s[k + "_bits"]).astype(np.uint16).tobytes())
        else:
            f.write(np.ascontiguousarray(s[k], dtype=np.float32).tobytes())
    f.write(np.ascontiguousarray(s["dt"], dtype=np.float32).tobytes())


def _run_driver(tmp_path, wl, T, fused, rounds=0):
    """Run the C++ caller: T decode steps, then `rounds` speculative rounds of
    wl.draft drafts with the seeded acceptances."""
    delta = wl.kind in ("gdn", "kda")
    A = np.zeros(wl.nheads, np.float32) if delta else synth.params(wl)["A"].astype(np.float32)
    S0 = synth.initial_state(wl).astype(np.float32)
    has_s0 = int(np.any(S0 != 0))
    bf16 = int(wl.in_dtype == "bf16")
    K = wl.draft if rounds else 0
    copy = COPY[wl.read_copy]
    hdr = np.array([0x52535334, wl.batch, wl.nheads, wl.headdim, wl.dstate, wl.ngroups, wl.window,
                    wl.capacity, T, has_s0, int(fused), K, rounds, bf16, copy, KIND[wl.kind]], dtype=np.int32)
    gen = {"gdn": synth.gdn_step_inputs, "kda": synth.kda_step_inputs}.get(wl.kind, synth.step_inputs)
    steps = [gen(wl, t) for t in range(T)]
    rins = [synth.draft_inputs(wl, r) for r in range(rounds)]
    naccs = [synth.accepted_drafts(wl, r) for r in range(rounds)]
    with open(tmp_path / "in.bin", "wb") as f:
        f.write(hdr.tobytes())
        f.write(A.tobytes())
        if has_s0:
            f.write(np.ascontiguousarray(S0).tobytes())
        for s in steps:
            if delta:
                for k in ("q", "k", "v", "beta", "alpha"):
                    f.write(np.ascontiguousarray(s[k], dtype=np.float32).tobytes())
            else:
                _write_tokens(f, s, bf16)
        for rin, nacc in zip(rins, naccs):
            _write_tokens(f, rin, bf16)
            f.write((K - nacc).astype(np.int32).tobytes())
    if not os.path.exists(DRIVER):
        pytest.fail(f"{DRIVER} is not built; run __graft_entry__.build() first")
    r = subprocess.run([DRIVER, str(tmp_path / "in.bin"), str(tmp_path / "out.bin")],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    Bt, H, P, N = wl.batch, wl.nheads, wl.headdim, wl.dstate
    raw = open(tmp_path / "out.bin", "rb").read()
    ny, nyr, nS, nptr = T * Bt * H * P, rounds * Bt * (K + 1) * H * P, Bt * H * P * N, Bt * H * 4
    ck_bytes = nS * (2 if copy == 2 else 4)       # fp32 checkpoint, or the bf16-stored one
    lo_bytes = nS * 2 if copy == 1 else 0         # bf16 read copy
    assert len(raw) == 4 * (ny + nyr + nptr + 1) + ck_bytes + lo_bytes
    y = np.frombuffer(raw, np.float32, ny).reshape(T, Bt, H, P)
    yr = np.frombuffer(raw, np.float32, nyr, offset=4 * ny).reshape(rounds, Bt, K + 1, H, P)
    o = 4 * (ny + nyr)

    def bf16_at(off):  # bf16 words -> float32 values
        return (np.frombuffer(raw, np.uint16, nS, offset=off).astype(np.uint32) << 16).view(np.float32)
    ck = bf16_at(o) if copy == 2 else np.frombuffer(raw, np.float32, nS, offset=o)
    ck_lo = bf16_at(o + ck_bytes).reshape(Bt, H, P, N) if copy == 1 else None
    o += ck_bytes + lo_bytes
    ptr = np.frombuffer(raw, np.int32, nptr, offset=o).reshape(Bt, H, 4)
    err = int(np.frombuffer(raw, np.int32, 1, offset=o + 4 * nptr)[0])
    return dict(steps=steps, rins=rins, naccs=naccs, A=A, S0=S0, y=y, yr=yr, ck=ck.reshape(Bt, H, P, N),
                ck_lo=ck_lo, ptr=ptr, err=err)


@pytest.mark.parametrize("shape,fused", [
    ((2, 4, 16, 16, 4, 8, 8), False),
    ((2, 4, 16, 16, 2, 8, 8), True),
    ((3, 4, 64, 128, 4, 16, 16), True),
    ((2, 3, 37, 32, 1, 5, 7), False),
], ids=["tiny", "tiny-G2-fused", "P64N128-fused", "P37N32-G1"])
def test_c_caller_matches_oracle(tmp_path, shape, fused):
    Bt, H, P, N, G, W, R = shape
    wl = BASE.replace(name="c-abi", batch=Bt, nheads=H, headdim=P, dstate=N, ngroups=G, window=W,
                      capacity=R, s0="normal", seed=7000 + P + N + G)
    T = 3 * W + 2
    log(f"[c-abi] Bt={Bt} H={H} P={P} N={N} G={G} W={W} R={R} fused={fused}, {T} steps")
    out = _run_driver(tmp_path, wl, T, fused)
    steps, A, S0, y, ck, ptr = (out[k] for k in ("steps", "A", "S0", "y", "ck", "ptr"))
    assert out["err"] == 0
    S = S0.astype(np.float64)
    pm = PointerModel(Bt, R)
    worst, ys, refs = 0.0, [], []
    for t, s in enumerate(steps):
        S, y_ref = mamba2.eager_step(S, A, s["x"], s["B"], s["C"], s["dt"])
        worst = max(worst, rel_l2(y[t].astype(np.float64), y_ref))
        ys.append(y[t])
        refs.append(y_ref)
        for b in range(Bt):
            pm.append(b, 1)
            pm.flush(b, W)
    run = rel_l2(np.stack(ys).astype(np.float64), np.stack(refs))
    log(f"  worst step {worst:.2e}, run {run:.2e}")
    assert worst < 1e-5 and run < 1e-5
    for h in range(H):
        assert np.array_equal(ptr[:, h, :3], pm.as_array())
    # the last fold was at step T - (T mod W); replay the oracle to that point
    S_f = S0.astype(np.float64)
    for s in steps[:T - T % W]:
        S_f, _ = mamba2.eager_step(S_f, A, s["x"], s["B"], s["C"], s["dt"])
    assert rel_l2(ck.astype(np.float64), S_f) < 1e-5


# Decode steps, then speculative rounds of rss_verify_k_tokens_fold(W, K) and
# rss_rollback from the C++ caller. bf16 inputs take the matrix-core ring
# terms; grouped B rows need R >= W + 2K + 1, one B row set per head R >= W + K.
@pytest.mark.parametrize("shape,in_dtype", [
    ((2, 4, 16, 16, 4, 8, 12, 4), "f32"),
    ((3, 4, 64, 128, 2, 8, 15, 3), "bf16"),
    ((2, 3, 37, 32, 3, 5, 12, 7), "bf16"),
    ((2, 2, 64, 128, 1, 16, 25, 4), "f32"),
], ids=["tiny-f32", "P64N128-G2-bf16", "P37N32-K7-bf16", "P64N128-G1-f32"])
def test_c_caller_speculative_rounds(tmp_path, shape, in_dtype):
    Bt, H, P, N, G, W, R, K = shape
    wl = BASE.replace(name="c-abi-spec", batch=Bt, nheads=H, headdim=P, dstate=N, ngroups=G, window=W,
                      capacity=R, max_draft=K, draft=K, in_dtype=in_dtype, s0="normal",
                      seed=7100 + P + N + G + K)
    out = _spec_run(tmp_path, wl)
    assert out["worst"] < 1e-5 and out["run"] < 1e-5
    assert rel_l2(out["ck"].astype(np.float64), out["ck_ref"]) < 1e-5


# The other checkpoint precisions through the same raw-pointer calls: dual
# precision (fp32 master for the fold, bf16 read copy for the outputs) and a
# single bf16-stored checkpoint. Outputs against the exact recurrence at the
# bf16-read bar (2e-2); the dual master at the fp32 bar and its read copy
# bit for bit the round-to-nearest-even of the master.
@pytest.mark.parametrize("copy,in_dtype", [("bf16", "bf16"), ("bf16", "f32"), ("bf16_state", "bf16"),
                                           ("bf16_state", "f32")])
def test_c_caller_checkpoint_precisions(tmp_path, copy, in_dtype):
    Bt, H, P, N, G, W, R, K = 2, 4, 64, 128, 2, 8, 15, 3
    wl = BASE.replace(name="c-abi-prec", batch=Bt, nheads=H, headdim=P, dstate=N, ngroups=G, window=W,
                      capacity=R, max_draft=K, draft=K, in_dtype=in_dtype, read_copy=copy, s0="normal",
                      seed=7200 + COPY[copy] + (in_dtype == "bf16"))
    out = _spec_run(tmp_path, wl)
    assert out["run"] < 2e-2
    if copy == "bf16":
        assert rel_l2(out["ck"].astype(np.float64), out["ck_ref"]) < 1e-5
        assert np.array_equal(out["ck_lo"], round_bf16_from_f32(out["ck"]).astype(np.float32))
    else:
        assert rel_l2(out["ck"].astype(np.float64), out["ck_ref"]) < 2e-2


def _spec_run(tmp_path, wl):
    """W + 3 decode steps, then 10 rounds of verify-with-fold and rollback, from
    the C++ caller; returns its outputs with the oracle's errors: worst round
    and whole-run rel-L2 of the outputs, and each sequence's state just before
    its open window (ck_ref). Pointers are checked against the ring model."""
    Bt, H, R, K, W = wl.batch, wl.nheads, wl.capacity, wl.draft, wl.window
    T, rounds = W + 3, 10
    log(f"[c-abi spec] Bt={Bt} H={H} P={wl.headdim} N={wl.dstate} G={wl.ngroups} W={W} R={R} K={K} "
        f"{wl.in_dtype} read_copy={wl.read_copy}, {T} steps + {rounds} rounds")
    out = _run_driver(tmp_path, wl, T, True, rounds)
    assert out["err"] == 0
    A = out["A"]
    S = out["S0"].astype(np.float64)
    hist = [[S[b]] for b in range(Bt)]     # committed states of each sequence
    pm = PointerModel(Bt, R)
    ys, refs = [], []
    for t, s in enumerate(out["steps"]):
        S, y_ref = mamba2.eager_step(S, A, s["x"], s["B"], s["C"], s["dt"])
        ys.append(out["y"][t])
        refs.append(y_ref)
        for b in range(Bt):
            hist[b].append(S[b])
            pm.append(b, 1)
            pm.flush(b, W)
    worst = 0.0
    for r, (rin, nacc) in enumerate(zip(out["rins"], out["naccs"])):
        states, y_ref = [], []
        Sr = S
        for i in range(K + 1):
            Sr, yi = mamba2.eager_step(Sr, A, rin["x"][:, i], rin["B"][:, i], rin["C"][:, i], rin["dt"][:, i])
            states.append(Sr)
            y_ref.append(yi)
        y_ref = np.stack(y_ref, axis=1)
        worst = max(worst, rel_l2(out["yr"][r].astype(np.float64), y_ref))
        ys.append(out["yr"][r])
        refs.append(y_ref)
        S = np.stack([states[nacc[b]][b] for b in range(Bt)])
        for b in range(Bt):
            pm.flush(b, W)
            pm.append(b, K + 1)
            pm.mark_tentative(b, K + 1)
            pm.rollback(b, int(K - nacc[b]))
            hist[b].extend(states[i][b] for i in range(nacc[b] + 1))
    run = rel_l2(np.concatenate([a.ravel() for a in ys]).astype(np.float64),
                 np.concatenate([a.ravel() for a in refs]))
    log(f"  worst round {worst:.2e}, run {run:.2e}")
    for h in range(H):
        assert np.array_equal(out["ptr"][:, h, :3], pm.as_array())
    # each checkpoint holds the state before its sequence's open window
    out["ck_ref"] = np.stack([hist[b][len(hist[b]) - 1 - int(pm.len[b])] for b in range(Bt)])
    out["worst"], out["run"] = worst, run
    return out


# The delta rules through their own C entry points: Gated DeltaNet (scalar gate)
# and Kimi Delta Attention (one gate per key channel), decode with the fold in
# the same pass or a separate flush each step. Outputs at every step and the
# final checkpoint against the fp64 eager rule; pointers against the ring model.
@pytest.mark.parametrize("kind,fused", [("gdn", True), ("gdn", False), ("kda", True), ("kda", False)])
def test_c_caller_delta_rules(tmp_path, kind, fused):
    Bt, H, P, N, W = 2, 3, 64, 128, 6
    wl = workloads.get("gdn_b256_h32_d128_w16").replace(
        name="c-abi-delta", kind=kind, batch=Bt, nheads=H, ngroups=H, headdim=P, dstate=N, window=W,
        capacity=W, s0="normal", seed=7300 + KIND[kind] + int(fused))
    T = 3 * W + 2
    log(f"[c-abi {kind}] Bt={Bt} H={H} dv={P} dk={N} W={W} fused={fused}, {T} steps")
    out = _run_driver(tmp_path, wl, T, fused)
    assert out["err"] == 0
    rule = gdn if kind == "gdn" else kda
    S = out["S0"].astype(np.float64)
    pm = PointerModel(Bt, W)
    worst, ys, refs, S_fold = 0.0, [], [], S
    for t, s in enumerate(out["steps"]):
        S, o_ref = rule.eager_step(S, s["q"], s["k"], s["v"], s["beta"], s["alpha"])
        worst = max(worst, rel_l2(out["y"][t].astype(np.float64), o_ref))
        ys.append(out["y"][t])
        refs.append(o_ref)
        for b in range(Bt):
            pm.append(b, 1)
            if pm.flush(b, W) and b == 0:
                S_fold = S
    run = rel_l2(np.stack(ys).astype(np.float64), np.stack(refs))
    log(f"  worst step {worst:.2e}, run {run:.2e}")
    assert worst < 1e-5 and run < 1e-5
    for h in range(H):
        assert np.array_equal(out["ptr"][:, h, :3], pm.as_array())
    assert rel_l2(out["ck"].astype(np.float64), S_fold) < 1e-5
