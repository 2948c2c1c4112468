"""GPU parity of the fused decode + fold entry point: bit for bit the same
outputs, checkpoint, read copy, ring and pointers as rss_decode_step followed by
rss_flush_checkpoint, in lockstep decode and with per-sequence windows left
uneven by speculative rounds; and against the fp64 oracle."""
import numpy as np
import pytest
import torch

from oracle import mamba2
import workloads
from workloads import synth
from recurrent_state_storage_amd import rss
from gpu_util import DEV, cfg_of, dev_inputs, rel_l2, log

pytestmark = pytest.mark.gpu

BASE = workloads.get("tiny_b2_h4_p16_n16_w8")


def _pair(wl):
    cfg = cfg_of(wl)
    A = torch.from_numpy(synth.params(wl)["A"]).to(DEV)
    S0 = torch.from_numpy(synth.initial_state(wl)).to(DEV)
    out = []
    for _ in range(2):
        L = rss.ReplayLayer(cfg, A, DEV)
        L.init_state(S0)
        out.append(L)
    return out


def _same(L1, L2):
    torch.cuda.synchronize()
    assert torch.equal(L1.ckpt, L2.ckpt)
    assert torch.equal(L1.ptr, L2.ptr)
    assert torch.equal(L1.ring_x, L2.ring_x) and torch.equal(L1.ring_B, L2.ring_B)
    assert torch.equal(L1.ring_dl, L2.ring_dl)
    if L1.ckpt_lo is not None:
        assert torch.equal(L1.ckpt_lo, L2.ckpt_lo)


SHAPES = [
    # P, N, H, G, W, R, in_dtype, copy
    (64, 128, 4, 4, 16, 16, "bf16", "none"),
    (37, 32, 3, 1, 5, 7, "f32", "none"),
    (100, 256, 2, 2, 4, 4, "f32", "none"),
    (128, 128, 2, 2, 8, 8, "bf16", "none"),
    (64, 128, 4, 4, 16, 16, "bf16", "bf16"),
    (1, 16, 1, 1, 1, 1, "f32", "none"),
    # dual precision: the bf16 copy is read, the fp32 master folded in the same launch
    (37, 32, 3, 1, 5, 7, "f32", "bf16"),
    (100, 256, 2, 2, 4, 4, "f32", "bf16"),
    (128, 128, 2, 2, 8, 8, "bf16", "bf16"),
    (1, 16, 1, 1, 1, 1, "f32", "bf16"),
    # a bf16-stored checkpoint, folded inside the two-wavefront decode
    (64, 128, 4, 4, 16, 16, "bf16", "bf16_state"),
    (37, 32, 3, 1, 5, 7, "f32", "bf16_state"),
    (100, 256, 2, 2, 4, 4, "f32", "bf16_state"),
    (128, 128, 2, 2, 8, 8, "bf16", "bf16_state"),
    (256, 64, 1, 1, 3, 3, "bf16", "bf16_state"),
    (1, 16, 1, 1, 1, 1, "f32", "bf16_state"),
    # windows past 16 entries: the bf16 fold's second and third groups of 16,
    # a grouped layer, N = 256 (4-row hand-over), and the fp32-input fold
    (64, 128, 2, 2, 20, 20, "bf16", "bf16_state"),
    (48, 64, 2, 1, 40, 44, "bf16", "bf16_state"),
    (256, 256, 1, 1, 24, 24, "bf16", "bf16_state"),
    (64, 128, 2, 2, 20, 20, "f32", "bf16_state"),
    # tile counts past whole groups of the workgroup-to-tile order with a ragged
    # tail: 144 fp32 tiles (groups of 128), 288 bf16 tiles (groups of 256)
    (64, 128, 48, 48, 8, 8, "bf16", "none"),
    (64, 128, 96, 96, 8, 8, "bf16", "bf16_state"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "P%dN%dH%dG%dW%dR%d-%s-%s" % s)
def test_fused_equals_separate_and_oracle(shape):
    P, N, H, G, W, R, idt, copy = shape
    wl = BASE.replace(name="fused", batch=3, headdim=P, dstate=N, nheads=H, ngroups=G, window=W,
                      capacity=R, in_dtype=idt, read_copy=copy, s0="normal", seed=5000 + P + N)
    log(f"[fused] {shape}")
    sep, fus = _pair(wl)
    A_np = synth.params(wl)["A"]
    S_ref = synth.initial_state(wl).astype(np.float64)
    ys, refs = [], []
    for t in range(3 * W + 1):
        s = synth.step_inputs(wl, t)
        d = dev_inputs(s, idt)
        y1 = torch.empty((wl.batch, H, P), device=DEV)
        y2 = torch.empty_like(y1)
        sep.decode_step(d["x"], d["B"], d["C"], d["dt"], y1)
        sep.flush_checkpoint(W)
        fus.decode_flush_step(W, d["x"], d["B"], d["C"], d["dt"], y2)
        if copy == "bf16" and (t + 1) % W == 0:
            # dual precision, every window filled (lockstep from init): one pass
            # from the fp32 master, outputs from its bf16 rounding, summed in the
            # fp32 kernel's order
            assert rel_l2(y2.double().cpu().numpy(), y1.double().cpu().numpy()) < 1e-5, t
        else:
            assert torch.equal(y1, y2), t
        S_ref, y_ref = mamba2.eager_step(S_ref, A_np, s["x"], s["B"], s["C"], s["dt"])
        ys.append(y2.double().cpu().numpy())
        refs.append(y_ref)
        if (t + 1) % W == 0:
            _same(sep, fus)
            if copy == "none":
                assert rel_l2(fus.ckpt.double().cpu().numpy(), S_ref) < 1e-5
    _same(sep, fus)
    assert fus.device_error() == 0
    assert rel_l2(np.stack(ys), np.stack(refs)) < (1e-5 if copy == "none" else 2e-2)


def test_dual_fold_plan_follows_what_the_handle_knows():
    """Dual precision: the fused entry point reads the fp32 master in one pass
    only while every window is known to fill together (from init, and again
    after rss_flush_checkpoint(1)); after a verify round it falls back to the
    replay of the copy plus the flush. Either way the checkpoint, copy, ring and
    pointers equal decode + flush bit for bit, the outputs bit for bit or, on a
    one-pass fold, up to rounding."""
    wl = BASE.replace(name="fused-dual-plan", batch=4, headdim=64, dstate=128, nheads=4, ngroups=4,
                      window=6, capacity=10, max_draft=4, draft=4, in_dtype="bf16", s0="normal",
                      read_copy="bf16", seed=5300)
    sep, fus = _pair(wl)
    W, K = wl.window, wl.draft
    Bt, H, P = wl.batch, wl.nheads, wl.headdim
    t = 0
    one_pass = 0

    def decode(n, lock_known):
        nonlocal t, one_pass
        for _ in range(n):
            d = dev_inputs(synth.step_inputs(wl, t), "bf16")
            y1 = torch.empty((Bt, H, P), device=DEV)
            y2 = torch.empty_like(y1)
            fills = int(fus.ptr[0, 0, 1]) + 1 >= W
            sep.decode_step(d["x"], d["B"], d["C"], d["dt"], y1)
            sep.flush_checkpoint(W)
            fus.decode_flush_step(W, d["x"], d["B"], d["C"], d["dt"], y2)
            torch.cuda.synchronize()
            if lock_known and fills:
                one_pass += 1
                assert rel_l2(y2.double().cpu().numpy(), y1.double().cpu().numpy()) < 1e-5, t
            else:
                assert torch.equal(y1, y2), t
            _same(sep, fus)
            t += 1

    decode(2 * W + 2, True)                  # lockstep from init
    rin = dev_inputs(synth.draft_inputs(wl, 0), "bf16")
    nd = torch.from_numpy((K - synth.accepted_drafts(wl, 0)).astype(np.int32)).to(DEV)
    yv = torch.empty((Bt, K + 1, H, P), device=DEV)
    for L in (sep, fus):
        L.verify_k_tokens(K, rin["x"], rin["B"], rin["C"], rin["dt"], yv)
        L.rollback(nd)
        L.flush_checkpoint(W)
    _same(sep, fus)
    decode(2 * W, False)                     # windows uneven: replay of the copy + flush
    for L in (sep, fus):
        L.flush_checkpoint(1)                # every window folded: in step again
    _same(sep, fus)
    decode(2 * W + 1, True)
    assert one_pass >= 4
    assert fus.device_error() == 0 and sep.device_error() == 0


@pytest.mark.parametrize("copy", ["none", "bf16", "bf16_state"])
def test_fused_folds_only_full_windows(copy):
    """After speculative rounds the sequences' windows differ; a fused decode
    folds exactly those that reach the threshold, like decode + flush."""
    wl = BASE.replace(name="fused-spec", batch=6, headdim=64, dstate=128, nheads=4, ngroups=4,
                      window=8, capacity=12, max_draft=4, draft=4, in_dtype="bf16", s0="normal",
                      read_copy=copy, seed=5100)
    sep, fus = _pair(wl)
    K = wl.draft
    for r in range(9):
        rin = dev_inputs(synth.draft_inputs(wl, r), "bf16")
        nd = torch.from_numpy((K - synth.accepted_drafts(wl, r)).astype(np.int32)).to(DEV)
        y = torch.empty((wl.batch, K + 1, wl.nheads, wl.headdim), device=DEV)
        for L in (sep, fus):
            L.verify_k_tokens(K, rin["x"], rin["B"], rin["C"], rin["dt"], y)
            L.rollback(nd)
            L.flush_checkpoint(wl.window)
        lens = fus.ptr[:, 0, 1].cpu().numpy()
        for t in range(3):
            d = dev_inputs(synth.step_inputs(wl, 100 * r + t), "bf16")
            y1 = torch.empty((wl.batch, wl.nheads, wl.headdim), device=DEV)
            y2 = torch.empty_like(y1)
            sep.decode_step(d["x"], d["B"], d["C"], d["dt"], y1)
            sep.flush_checkpoint(wl.window)
            fus.decode_flush_step(wl.window, d["x"], d["B"], d["C"], d["dt"], y2)
            assert torch.equal(y1, y2)
        _same(sep, fus)
        if r == 0:
            log(f"  window lengths after round 0: {lens.tolist()}")
    assert fus.device_error() == 0 and sep.device_error() == 0


@pytest.mark.parametrize("copy", ["none", "bf16", "bf16_state"])
def test_staggered_folds(copy):
    """Per-sequence thresholds 1 + (b mod W) until a sequence's first fold, W
    after: each step folds only the sequences at their phase. The fused entry
    point with per-sequence thresholds equals decode + per-sequence flush bit
    for bit, folds exactly the sequences the integer schedule names, and matches
    the oracle (driven with the same thresholds) at every step."""
    W = 4
    wl = BASE.replace(name="stagger", batch=7, headdim=64, dstate=128, nheads=3, ngroups=3,
                      window=W, capacity=W, in_dtype="bf16", read_copy=copy, s0="normal", seed=5200)
    log(f"[fused] staggered folds, Bt=7, W=4, copy={copy}")
    sep, fus = _pair(wl)
    A_np = synth.params(wl)["A"]
    model = mamba2.ReplayModel(synth.initial_state(wl), A_np, wl.ngroups, wl.capacity, read_copy=copy)
    first = 1 + np.arange(wl.batch) % W
    worst = 0.0
    for t in range(4 * W + 3):
        th_np = np.where(t < first, first, W).astype(np.int32)
        th = torch.from_numpy(th_np).to(DEV)
        s = synth.step_inputs(wl, t)
        d = dev_inputs(s, "bf16")
        y1 = torch.empty((wl.batch, wl.nheads, wl.headdim), device=DEV)
        y2 = torch.empty_like(y1)
        sep.decode_step(d["x"], d["B"], d["C"], d["dt"], y1)
        sep.flush_checkpoint_each(th)
        fus.decode_flush_step_each(th, d["x"], d["B"], d["C"], d["dt"], y2)
        assert torch.equal(y1, y2), t
        y_m = model.decode(s["x"], s["B"], s["C"], s["dt"])
        folded = model.flush(th_np)
        want = [b for b in range(wl.batch) if t + 1 >= first[b] and (t + 1 - first[b]) % W == 0]
        assert folded == want, t
        lens = fus.ptr[:, :, 1].cpu().numpy()
        assert np.array_equal(lens, np.repeat(model.ptr.len[:, None], wl.nheads, axis=1)), t
        worst = max(worst, rel_l2(y2.double().cpu().numpy(), y_m))
    _same(sep, fus)
    log(f"  worst vs oracle {worst:.2e}")
    assert worst < (1e-5 if copy == "none" else 1e-3)
    assert fus.device_error() == 0 and sep.device_error() == 0
