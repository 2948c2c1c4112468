"""Host logic of bench.py, without a GPU: the algorithmic byte model behind
`roofline.achieved` (counted here by hand from the layouts in include/rss.h),
the whole-window step rounding, the counter-summary lookup, and the one-GPU
guard."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
WL = workloads.get(bench.WORKLOAD)


def test_workload_is_the_headline_shape():
    assert (WL.batch, WL.nheads, WL.headdim, WL.dstate, WL.ngroups, WL.window) == (256, 128, 64, 128, 128, 16)
    assert WL.in_dtype == "bf16" and WL.read_copy == "none"


def test_replay_bytes_by_hand():
    # per (sequence, head), P = 64, N = 128, bf16 x / B / C, fp32 dt, A, y and state
    tile = 64 * 128 * 4                  # checkpoint tile read once
    entry = 64 * 2 + 128 * 2 + 8         # one ring entry: x row, B row, (dt, l)
    inputs = 64 * 2 + 128 * 2 * 2 + 4    # x_t, B_t, C_t, dt_t
    y = 64 * 4
    ptr = 16 + 16                        # pointer word read and written
    A = 4
    for n0 in range(WL.window):
        want = tile + n0 * entry + inputs + y + entry + ptr + A
        assert bench.replay_bytes(WL, n0) == want == 34096 + 392 * n0


def test_dual_one_pass_fold_bytes_by_hand():
    # the window-filling token of a dual-precision layer (W = 16): the fp32
    # master tile read, 15 ring entries, the inputs, y, the appended entry,
    # pointers and A, then the new master (fp32) and copy (bf16) written
    wl = workloads.get("mamba2_dual_b256_h128_p64_n128_w16")
    entry = 64 * 2 + 128 * 2 + 8
    want = 64 * 128 * 4 + 15 * entry + (64 * 2 + 128 * 2 * 2 + 4) + 64 * 4 + entry + 32 + 4 + 64 * 128 * (4 + 2)
    assert bench.dual_fused_bytes(wl) == want == 89128


def test_replay_launch_bytes_of_the_fused_schedule():
    # plain replays run at n0 = 0..W-2; the window-filling token is the fused launch
    per_launch = sum(bench.replay_bytes(WL, n0) for n0 in range(WL.window - 1)) / (WL.window - 1)
    assert per_launch * WL.batch * WL.nheads == 1_207_173_120
    # the fused launch also writes the new tile
    assert bench.fused_bytes(WL) == bench.replay_bytes(WL, 15) + 64 * 128 * 4 == 72_744


def test_eager_bytes_and_ratio():
    e = bench.eager_bytes(WL)
    assert e == 2 * 64 * 128 * 4 + (64 * 2 + 2 * 128 * 2 + 4) + 64 * 4 + 4
    # bytes per token over a window: 15 replays + 1 fused vs 16 eager steps
    rep = (sum(bench.replay_bytes(WL, n0) for n0 in range(15)) + bench.fused_bytes(WL)) / 16
    assert 0.58 < rep / e < 0.60


def test_verify_bytes_match_the_replay_model_at_one_token():
    wl = WL.replace(draft=0)
    n0 = np.array([3, 7], np.int64)
    got = bench.verify_bytes(wl.replace(batch=2), n0, np.zeros(2, bool))
    # one token: exactly the decode's bytes (pointers and A: 36 in both)
    want = sum(bench.replay_bytes(wl, int(k)) for k in n0) * wl.nheads
    assert got == want
    folded = bench.verify_bytes(wl.replace(batch=2), n0, np.array([True, False]))
    assert folded - got == 64 * 128 * 4 * wl.nheads


@pytest.mark.parametrize("steps,mult,minimum,want", [(20, 16, 64, 64), (70, 16, 64, 80), (256, 32, 0, 256),
                                                      (257, 32, 0, 288), (0, 16, 16, 16)])
def test_whole_windows(steps, mult, minimum, want):
    assert bench.whole(steps, mult, minimum) == want


def test_counter_traffic_follows_the_kernel_hash():
    """The committed counters are used only for the kernel code they measured."""
    with open(bench.COUNTERS_FILE) as f:
        text = f.read()
    recorded = [ln.split("=")[1].strip() for ln in text.splitlines() if ln.startswith("kernel_source_hash")]
    assert len(recorded) == 1
    t = bench.counter_traffic("replay")
    if recorded[0] == bench.kernel_source_hash():
        alg = 1_207_173_120
        assert t is not None and abs(t / alg - 1) < 0.01
    else:
        assert t is None


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       timeout=120, env={**os.environ, **env}, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
