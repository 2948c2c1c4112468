"""GPU parity of Gated DeltaNet decode: replay (checkpoint + ring of (k, u,
log alpha)) and the eager gated-delta-rule kernel against the fp64 oracle at
every step; flush folds GDN windows; full size on sampled (sequence, head)
pairs, replay against eager on the whole batch."""
import numpy as np
import pytest
import torch

from oracle import gdn
from oracle.ring import PointerModel
import workloads
from workloads import synth
from recurrent_state_storage_amd import rss
from gpu_util import DEV, cfg_of, rel_l2, sample_pairs, log

pytestmark = pytest.mark.gpu

GDN = workloads.get("gdn_b256_h32_d128_w16")


def _dev(s):
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to(DEV) for k, v in s.items()}


def _run(wl, steps, flush_every_step=True):
    log(f"[gdn] Bt={wl.batch} H={wl.nheads} dv={wl.headdim} dk={wl.dstate} W={wl.window} R={wl.capacity} s0={wl.s0}")
    cfg = cfg_of(wl)
    layer = rss.ReplayLayer(cfg, None, DEV)
    S0 = synth.initial_state(wl)
    layer.init_state(torch.from_numpy(S0).to(DEV))
    S_eag = torch.from_numpy(S0).to(DEV).clone()
    S_ref = S0.astype(np.float64)
    pm = PointerModel(wl.batch, wl.capacity)
    Bt, H, P = wl.batch, wl.nheads, wl.headdim
    worst = {"step": 0.0, "eager": 0.0, "ckpt": 0.0}
    os_, refs = [], []
    for t in range(steps):
        s = synth.gdn_step_inputs(wl, t)
        d = _dev(s)
        o = torch.full((Bt, H, P), float("nan"), device=DEV)
        oe = torch.full_like(o, float("nan"))
        layer.gdn_decode_step(d["q"], d["k"], d["v"], d["beta"], d["alpha"], o)
        rss.rss_gdn_eager_step(cfg, S_eag, d["q"], d["k"], d["v"], d["beta"], d["alpha"], oe)
        S_ref, o_ref = gdn.eager_step(S_ref, s["q"], s["k"], s["v"], s["beta"], s["alpha"])
        for b in range(Bt):
            pm.append(b, 1)
        og = o.double().cpu().numpy()
        assert np.isfinite(og).all(), t
        worst["step"] = max(worst["step"], rel_l2(og, o_ref))
        worst["eager"] = max(worst["eager"], rel_l2(oe.double().cpu().numpy(), o_ref))
        os_.append(og)
        refs.append(o_ref)
        flushed = False
        if flush_every_step or (t + 1) % wl.window == 0:
            layer.flush_checkpoint(wl.window)
            for b in range(Bt):
                flushed |= pm.flush(b, wl.window)
        ptr = layer.ptr.cpu().numpy()
        for h in range(H):
            assert np.array_equal(ptr[:, h, :3], pm.as_array()), (t, h)
        if flushed:
            worst["ckpt"] = max(worst["ckpt"], rel_l2(layer.ckpt.double().cpu().numpy(), S_ref))
    assert layer.device_error() == 0
    worst["run"] = rel_l2(np.stack(os_), np.stack(refs))
    worst["eager_state"] = rel_l2(S_eag.double().cpu().numpy(), S_ref)
    log(f"  worst {worst}")
    return worst


SHAPES = [
    # dv, dk, H, W, R, s0
    (16, 32, 3, 4, 5, "normal"),
    (37, 16, 2, 3, 3, "normal"),
    (128, 128, 2, 8, 8, "zeros"),
    (128, 128, 2, 5, 7, "normal"),
    (100, 64, 2, 6, 6, "normal"),
    (64, 256, 2, 4, 4, "normal"),
    (256, 32, 1, 3, 4, "normal"),
    (128, 128, 24, 5, 6, "normal"),   # 72 tiles of 64 KiB: one group of the tile order (64) + a tail
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "dv%ddk%dH%dW%dR%d-%s" % s)
def test_gdn_every_step(shape):
    dv, dk, H, W, R, s0 = shape
    wl = GDN.replace(name="gdn-sweep", batch=3, nheads=H, ngroups=H, headdim=dv, dstate=dk, window=W,
                     capacity=R, s0=s0, seed=6000 + dv + dk)
    w = _run(wl, 3 * W + 2)
    assert w["step"] < 1e-5 and w["run"] < 1e-5
    assert w["eager"] < 1e-5 and w["eager_state"] < 1e-5
    assert w["ckpt"] < 1e-5


def test_gdn_flush_only_at_window():
    wl = GDN.replace(name="gdn-win", batch=2, nheads=4, ngroups=4, headdim=32, dstate=64, window=6,
                     capacity=9, s0="normal", seed=6100)
    w = _run(wl, 20, flush_every_step=False)
    assert w["run"] < 1e-5 and w["ckpt"] < 1e-5


@pytest.mark.slow
def test_gdn_b256_full_size():
    wl = GDN
    log(f"[gdn full] {wl.name}: {wl.steps} steps")
    cfg = cfg_of(wl)
    layer = rss.ReplayLayer(cfg, None, DEV)
    layer.init_state()
    S_eag = torch.zeros((wl.batch, wl.nheads, wl.headdim, wl.dstate), device=DEV)
    pairs = sample_pairs(wl, 24, seed=21)
    pb = np.array([p[0] for p in pairs])
    ph = np.array([p[1] for p in pairs])
    S_ref = np.zeros((1, len(pairs), wl.headdim, wl.dstate))
    o = torch.empty((wl.batch, wl.nheads, wl.headdim), device=DEV)
    oe = torch.empty_like(o)
    bi, hi = torch.as_tensor(pb, device=DEV), torch.as_tensor(ph, device=DEV)
    worst_pair = worst_eager = 0.0
    got, refs = [], []
    for t in range(wl.steps):
        s = synth.gdn_step_inputs(wl, t)
        d = _dev(s)
        if (t + 1) % wl.window == 0:      # the benchmark's schedule: fold in the same pass
            layer.gdn_decode_flush_step(wl.window, d["q"], d["k"], d["v"], d["beta"], d["alpha"], o)
        else:
            layer.gdn_decode_step(d["q"], d["k"], d["v"], d["beta"], d["alpha"], o)
        rss.rss_gdn_eager_step(cfg, S_eag, d["q"], d["k"], d["v"], d["beta"], d["alpha"], oe)
        ps = {k: v[pb, ph][None] for k, v in s.items()}
        S_ref, o_ref = gdn.eager_step(S_ref, ps["q"], ps["k"], ps["v"], ps["beta"], ps["alpha"])
        g = o[bi, hi].double().cpu().numpy()[None]
        worst_pair = max(worst_pair, rel_l2(g, o_ref))
        got.append(g)
        refs.append(o_ref)
        worst_eager = max(worst_eager, float(torch.linalg.vector_norm(o - oe) / torch.linalg.vector_norm(oe)))
    run = rel_l2(np.stack(got), np.stack(refs))
    log(f"  pairs worst/run {worst_pair:.3e}/{run:.3e}; replay vs eager {worst_eager:.3e}")
    assert layer.device_error() == 0
    assert worst_pair < 1e-5 and run < 1e-5 and worst_eager < 1e-5
    ck = layer.ckpt[bi, hi].double().cpu().numpy()[None]
    assert rel_l2(ck, S_ref) < 1e-5          # 256 = 16 W: the last step folded every window


@pytest.mark.parametrize("shape", [(128, 128, 2, 8, 8), (37, 16, 2, 3, 3), (256, 256, 1, 4, 5),
                                   (64, 32, 3, 1, 1)], ids=lambda s: "dv%ddk%dH%dW%dR%d" % s)
def test_gdn_fused_fold_equals_separate(shape):
    """rss_gdn_decode_flush_step against rss_gdn_decode_step + rss_flush_checkpoint:
    outputs, checkpoint, ring and pointers bit for bit at every step (including
    a head dimension that spans several tile chunks)."""
    dv, dk, H, W, R = shape
    wl = GDN.replace(name="gdn-fused", batch=3, nheads=H, ngroups=H, headdim=dv, dstate=dk, window=W,
                     capacity=R, s0="normal", seed=6300 + dv + dk)
    log(f"[gdn] fused fold {shape}")
    cfg = cfg_of(wl)
    sep, fus = rss.ReplayLayer(cfg, None, DEV), rss.ReplayLayer(cfg, None, DEV)
    S0 = torch.from_numpy(synth.initial_state(wl)).to(DEV)
    sep.init_state(S0)
    fus.init_state(S0)
    o1 = torch.empty((wl.batch, H, dv), device=DEV)
    o2 = torch.empty_like(o1)
    for t in range(3 * W + 2):
        d = _dev(synth.gdn_step_inputs(wl, t))
        sep.gdn_decode_step(d["q"], d["k"], d["v"], d["beta"], d["alpha"], o1)
        sep.flush_checkpoint(W)
        fus.gdn_decode_flush_step(W, d["q"], d["k"], d["v"], d["beta"], d["alpha"], o2)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), t
        assert torch.equal(sep.ckpt, fus.ckpt), t
        assert torch.equal(sep.ptr, fus.ptr), t
        assert torch.equal(sep.ring_x, fus.ring_x) and torch.equal(sep.ring_B, fus.ring_B), t
        assert torch.equal(sep.ring_dl, fus.ring_dl), t
    assert sep.device_error() == 0 and fus.device_error() == 0
