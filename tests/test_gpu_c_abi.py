"""The C ABI from a plain C++ caller: tests/c_abi/rss_c_driver (built by
__graft_entry__.build(); no torch, no Python) allocates every buffer from
rss_buffer_sizes with hipMalloc, binds a layer and runs init + decode (+ fold)
through the C entry points. Its outputs, final checkpoint and pointers are
checked here against the fp64 oracle and the integer ring model."""
import os
import subprocess

import numpy as np
import pytest

from oracle import mamba2
from oracle.ring import PointerModel
import workloads
from workloads import synth
from gpu_util import rel_l2, log

pytestmark = pytest.mark.gpu

DRIVER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "rss_c_driver")
BASE = workloads.get("tiny_b2_h4_p16_n16_w8")


def _run_driver(tmp_path, wl, T, fused):
    A = synth.params(wl)["A"].astype(np.float32)
    S0 = synth.initial_state(wl).astype(np.float32)
    has_s0 = int(np.any(S0 != 0))
    hdr = np.array([0x52535331, wl.batch, wl.nheads, wl.headdim, wl.dstate, wl.ngroups, wl.window,
                    wl.capacity, T, has_s0, int(fused)], dtype=np.int32)
    steps = [synth.step_inputs(wl, t) for t in range(T)]
    with open(tmp_path / "in.bin", "wb") as f:
        f.write(hdr.tobytes())
        f.write(A.tobytes())
        if has_s0:
            f.write(np.ascontiguousarray(S0).tobytes())
        for s in steps:
            for k in ("x", "B", "C", "dt"):
                f.write(np.ascontiguousarray(s[k], dtype=np.float32).tobytes())
    if not os.path.exists(DRIVER):
        pytest.fail(f"{DRIVER} is not built; run __graft_entry__.build() first")
    r = subprocess.run([DRIVER, str(tmp_path / "in.bin"), str(tmp_path / "out.bin")],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    Bt, H, P, N = wl.batch, wl.nheads, wl.headdim, wl.dstate
    raw = open(tmp_path / "out.bin", "rb").read()
    ny, nS, nptr = T * Bt * H * P, Bt * H * P * N, Bt * H * 4
    y = np.frombuffer(raw, np.float32, ny).reshape(T, Bt, H, P)
    ck = np.frombuffer(raw, np.float32, nS, offset=4 * ny).reshape(Bt, H, P, N)
    ptr = np.frombuffer(raw, np.int32, nptr, offset=4 * (ny + nS)).reshape(Bt, H, 4)
    err = int(np.frombuffer(raw, np.int32, 1, offset=4 * (ny + nS + nptr))[0])
    return steps, A, S0, y, ck, ptr, err


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
    steps, A, S0, y, ck, ptr, err = _run_driver(tmp_path, wl, T, fused)
    assert err == 0
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
