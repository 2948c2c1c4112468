"""GPU parity of Kimi Delta Attention decode: replay (checkpoint + ring of (k, u,
per-channel log-gate rows)) and the eager kernel against the fp64 KDA oracle at
every step; the flush folds KDA windows with per-channel decays; with equal
gates on every channel the KDA kernels agree with the gated-DeltaNet ones; full
size on sampled (sequence, head) pairs, replay against eager on the whole batch."""
import numpy as np
import pytest
import torch

from oracle import kda
from oracle.ring import PointerModel
import workloads
from workloads import synth
from recurrent_state_storage_amd import rss
from gpu_util import DEV, cfg_of, rel_l2, sample_pairs, log

pytestmark = pytest.mark.gpu

KDA = workloads.get("kda_b256_h32_d128_w16")


def _dev(s):
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to(DEV) for k, v in s.items()}


def _run(wl, steps, flush_every_step=True):
    log(f"[kda] Bt={wl.batch} H={wl.nheads} dv={wl.headdim} dk={wl.dstate} W={wl.window} "
        f"R={wl.capacity} s0={wl.s0}")
    cfg = cfg_of(wl)
    layer = rss.ReplayLayer(cfg, None, DEV)
    S0 = synth.initial_state(wl)
    layer.init_state(torch.from_numpy(S0).to(DEV))
    S_eag = torch.from_numpy(S0).to(DEV).clone()
    S_ref = S0.astype(np.float64)
    model = kda.KDAReplayModel(S0, wl.capacity)
    pm = PointerModel(wl.batch, wl.capacity)
    Bt, H, P = wl.batch, wl.nheads, wl.headdim
    worst = {"step": 0.0, "eager": 0.0, "ckpt": 0.0, "model": 0.0}
    os_, refs = [], []
    for t in range(steps):
        s = synth.kda_step_inputs(wl, t)
        d = _dev(s)
        o = torch.full((Bt, H, P), float("nan"), device=DEV)
        oe = torch.full_like(o, float("nan"))
        layer.kda_decode_step(d["q"], d["k"], d["v"], d["beta"], d["alpha"], o)
        rss.rss_kda_eager_step(cfg, S_eag, d["q"], d["k"], d["v"], d["beta"], d["alpha"], oe)
        S_ref, o_ref = kda.eager_step(S_ref, s["q"], s["k"], s["v"], s["beta"], s["alpha"])
        o_mod = model.decode(s["q"], s["k"], s["v"], s["beta"], s["alpha"])
        for b in range(Bt):
            pm.append(b, 1)
        og = o.double().cpu().numpy()
        assert np.isfinite(og).all(), t
        worst["step"] = max(worst["step"], rel_l2(og, o_ref))
        worst["model"] = max(worst["model"], rel_l2(og, o_mod))
        worst["eager"] = max(worst["eager"], rel_l2(oe.double().cpu().numpy(), o_ref))
        os_.append(og)
        refs.append(o_ref)
        flushed = False
        if flush_every_step or (t + 1) % wl.window == 0:
            layer.flush_checkpoint(wl.window)
            model.flush(wl.window)
            for b in range(Bt):
                flushed |= pm.flush(b, wl.window)
        ptr = layer.ptr.cpu().numpy()
        for h in range(H):
            assert np.array_equal(ptr[:, h, :3], pm.as_array()), (t, h)
        if flushed:
            worst["ckpt"] = max(worst["ckpt"], rel_l2(layer.ckpt.double().cpu().numpy(), S_ref))
    # the ring's log-gate rows hold fp32 log(alpha) of every committed entry
    g = layer.ring_dl.double().cpu().numpy()
    for b in range(Bt):
        for j in range(int(pm.len[b])):
            slot = pm.slot(b, j)
            t = steps - int(pm.len[b]) + j
            want = np.log(synth.kda_step_inputs(wl, t)["alpha"][b].astype(np.float64))
            assert np.allclose(g[b, slot], want, rtol=1e-6, atol=1e-6), (b, j)
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
    (32, 64, 2, 1, 1, "normal"),
    (128, 128, 24, 5, 6, "normal"),   # 72 tiles of 64 KiB: one group of the tile order (64) + a tail
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "dv%ddk%dH%dW%dR%d-%s" % s)
def test_kda_every_step(shape):
    dv, dk, H, W, R, s0 = shape
    wl = KDA.replace(name="kda-sweep", batch=3, nheads=H, ngroups=H, headdim=dv, dstate=dk, window=W,
                     capacity=R, s0=s0, seed=7000 + dv + dk)
    w = _run(wl, 3 * W + 2)
    assert w["step"] < 1e-5 and w["run"] < 1e-5 and w["model"] < 1e-5
    assert w["eager"] < 1e-5 and w["eager_state"] < 1e-5
    assert w["ckpt"] < 1e-5


def test_kda_flush_only_at_window():
    wl = KDA.replace(name="kda-win", batch=2, nheads=4, ngroups=4, headdim=32, dstate=64, window=6,
                     capacity=9, s0="normal", seed=7100)
    w = _run(wl, 20, flush_every_step=False)
    assert w["run"] < 1e-5 and w["ckpt"] < 1e-5


def test_kda_with_equal_gates_matches_gdn_kernels():
    """One gate value repeated over every channel: the KDA replay, fold and eager
    kernels give the gated-DeltaNet kernels' results (different arithmetic
    order, so to 1e-5)."""
    wl = KDA.replace(name="kda-eq", batch=2, nheads=3, ngroups=3, headdim=64, dstate=128, window=5,
                     capacity=5, s0="normal", seed=7200)
    log(f"[kda] equal gates vs GDN kernels, {wl.name}")
    ck = cfg_of(wl)
    cg = cfg_of(wl.replace(kind="gdn"))
    lk, lg = rss.ReplayLayer(ck, None, DEV), rss.ReplayLayer(cg, None, DEV)
    S0 = torch.from_numpy(synth.initial_state(wl)).to(DEV)
    lk.init_state(S0)
    lg.init_state(S0)
    Ek, Eg = S0.clone(), S0.clone()
    shape = (wl.batch, wl.nheads, wl.headdim)
    ok, og, oek, oeg = (torch.empty(shape, device=DEV) for _ in range(4))
    worst = 0.0
    for t in range(17):
        s = synth.gdn_step_inputs(wl.replace(kind="gdn"), t)
        d = _dev(s)
        a_vec = d["alpha"][..., None].expand(-1, -1, wl.dstate).contiguous()
        lk.kda_decode_step(d["q"], d["k"], d["v"], d["beta"], a_vec, ok)
        lg.gdn_decode_step(d["q"], d["k"], d["v"], d["beta"], d["alpha"], og)
        rss.rss_kda_eager_step(ck, Ek, d["q"], d["k"], d["v"], d["beta"], a_vec, oek)
        rss.rss_gdn_eager_step(cg, Eg, d["q"], d["k"], d["v"], d["beta"], d["alpha"], oeg)
        lk.flush_checkpoint(wl.window)
        lg.flush_checkpoint(wl.window)
        for a, b in ((ok, og), (oek, oeg), (lk.ckpt, lg.ckpt), (Ek, Eg)):
            worst = max(worst, float(torch.linalg.vector_norm(a - b) / torch.linalg.vector_norm(b)))
    log(f"  worst relative difference {worst:.2e}")
    assert worst < 1e-5
    assert lk.device_error() == 0 and lg.device_error() == 0


@pytest.mark.slow
def test_kda_b256_full_size():
    wl = KDA
    log(f"[kda full] {wl.name}: {wl.steps} steps")
    cfg = cfg_of(wl)
    layer = rss.ReplayLayer(cfg, None, DEV)
    layer.init_state()
    S_eag = torch.zeros((wl.batch, wl.nheads, wl.headdim, wl.dstate), device=DEV)
    pairs = sample_pairs(wl, 24, seed=23)
    pb = np.array([p[0] for p in pairs])
    ph = np.array([p[1] for p in pairs])
    S_ref = np.zeros((1, len(pairs), wl.headdim, wl.dstate))
    o = torch.empty((wl.batch, wl.nheads, wl.headdim), device=DEV)
    oe = torch.empty_like(o)
    bi, hi = torch.as_tensor(pb, device=DEV), torch.as_tensor(ph, device=DEV)
    worst_pair = worst_eager = 0.0
    got, refs = [], []
    for t in range(wl.steps):
        s = synth.kda_step_inputs(wl, t)
        d = _dev(s)
        if (t + 1) % wl.window == 0:      # the benchmark's schedule: fold in the same pass
            layer.kda_decode_flush_step(wl.window, d["q"], d["k"], d["v"], d["beta"], d["alpha"], o)
        else:
            layer.kda_decode_step(d["q"], d["k"], d["v"], d["beta"], d["alpha"], o)
        rss.rss_kda_eager_step(cfg, S_eag, d["q"], d["k"], d["v"], d["beta"], d["alpha"], oe)
        ps = {k: v[pb, ph][None] for k, v in s.items()}
        S_ref, o_ref = kda.eager_step(S_ref, ps["q"], ps["k"], ps["v"], ps["beta"], ps["alpha"])
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
    assert rel_l2(ck, S_ref) < 1e-5


@pytest.mark.parametrize("shape", [(128, 128, 2, 8, 8), (37, 16, 2, 3, 3), (256, 256, 1, 4, 5),
                                   (64, 32, 3, 1, 1)], ids=lambda s: "dv%ddk%dH%dW%dR%d" % s)
def test_kda_fused_fold_equals_separate(shape):
    """rss_kda_decode_flush_step against rss_kda_decode_step + rss_flush_checkpoint:
    outputs, checkpoint, ring and pointers bit for bit at every step."""
    dv, dk, H, W, R = shape
    wl = KDA.replace(name="kda-fused", batch=3, nheads=H, ngroups=H, headdim=dv, dstate=dk, window=W,
                     capacity=R, s0="normal", seed=7300 + dv + dk)
    log(f"[kda] fused fold {shape}")
    cfg = cfg_of(wl)
    sep, fus = rss.ReplayLayer(cfg, None, DEV), rss.ReplayLayer(cfg, None, DEV)
    S0 = torch.from_numpy(synth.initial_state(wl)).to(DEV)
    sep.init_state(S0)
    fus.init_state(S0)
    o1 = torch.empty((wl.batch, H, dv), device=DEV)
    o2 = torch.empty_like(o1)
    for t in range(3 * W + 2):
        d = _dev(synth.kda_step_inputs(wl, t))
        sep.kda_decode_step(d["q"], d["k"], d["v"], d["beta"], d["alpha"], o1)
        sep.flush_checkpoint(W)
        fus.kda_decode_flush_step(W, d["q"], d["k"], d["v"], d["beta"], d["alpha"], o2)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), t
        assert torch.equal(sep.ckpt, fus.ckpt), t
        assert torch.equal(sep.ptr, fus.ptr), t
        assert torch.equal(sep.ring_x, fus.ring_x) and torch.equal(sep.ring_B, fus.ring_B), t
        assert torch.equal(sep.ring_dl, fus.ring_dl), t
    assert sep.device_error() == 0 and fus.device_error() == 0
