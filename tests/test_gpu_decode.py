"""GPU parity of plain decode: replay + flush and the eager kernel against the
fp64 oracle at every step, pointers bit-exact against the ring model, ring
contents bit-exact against the inputs, across shapes, dtypes and both
precision modes. All calls go through the C ABI."""
import numpy as np
import pytest
import torch

from oracle import mamba2
from oracle.ring import PointerModel
import workloads
from workloads import synth
from recurrent_state_storage_amd import rss
from gpu_util import DEV, cfg_of, dev_inputs, rel_l2, log

pytestmark = pytest.mark.gpu

TINY = workloads.get("tiny_b2_h4_p16_n16_w8")


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.contiguous().cpu()
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)).numpy()


def _run_decode(wl, steps, flush_every_step=True, check_ring=True, check_eager=True):
    """Drive replay (+eager) for `steps` tokens; compare with the oracle each step.

    Returns a dict of the worst errors seen."""
    log(f"[decode] {wl.name} P={wl.headdim} N={wl.dstate} H={wl.nheads} G={wl.ngroups} "
        f"W={wl.window} R={wl.capacity} in={wl.in_dtype} copy={wl.read_copy} s0={wl.s0}")
    cfg = cfg_of(wl)
    A_np = synth.params(wl)["A"]
    A = torch.from_numpy(A_np).to(DEV)
    S0 = synth.initial_state(wl)
    layer = rss.ReplayLayer(cfg, A, DEV)
    layer.init_state(torch.from_numpy(S0).to(DEV))
    S_eag = torch.from_numpy(S0).to(DEV).clone()
    S_ref = S0.astype(np.float64)
    dual_ref = mamba2.ReplayModel(S0, A_np, wl.ngroups, wl.capacity, read_copy=wl.read_copy) \
        if wl.read_copy == "bf16" else None
    pm = PointerModel(wl.batch, wl.capacity)
    Bt, H, P = wl.batch, wl.nheads, wl.headdim
    hist = []
    worst = {"step": 0.0, "eager": 0.0, "ckpt": 0.0, "dual_emul": 0.0}
    ys, yrefs = [], []
    for t in range(steps):
        s = synth.step_inputs(wl, t)
        hist.append(s)
        d = dev_inputs(s, wl.in_dtype)
        y = torch.full((Bt, H, P), float("nan"), device=DEV)
        layer.decode_step(d["x"], d["B"], d["C"], d["dt"], y)
        for b in range(Bt):
            pm.append(b, 1)
        S_ref, y_ref = mamba2.eager_step(S_ref, A_np, s["x"], s["B"], s["C"], s["dt"])
        if check_eager:
            ye = torch.full((Bt, H, P), float("nan"), device=DEV)
            rss.rss_eager_step(cfg, S_eag, d["x"], d["B"], d["C"], d["dt"], A, ye)
            worst["eager"] = max(worst["eager"], rel_l2(ye.double().cpu().numpy(), y_ref))
        yg = y.double().cpu().numpy()
        assert np.isfinite(yg).all(), f"non-finite output at step {t}"
        worst["step"] = max(worst["step"], rel_l2(yg, y_ref))
        ys.append(yg)
        yrefs.append(y_ref)
        if dual_ref is not None:
            y_em = dual_ref.decode(s["x"], s["B"], s["C"], s["dt"])
            worst["dual_emul"] = max(worst["dual_emul"], rel_l2(yg, y_em))
        flushed = False
        if flush_every_step or (t + 1) % wl.window == 0:
            layer.flush_checkpoint(wl.window)
            for b in range(Bt):
                flushed |= pm.flush(b, wl.window)
            if dual_ref is not None:
                dual_ref.flush(wl.window)
        # pointers: every head holds the sequence's values
        ptr = layer.ptr.cpu().numpy()
        want = pm.as_array()
        for h in range(H):
            assert np.array_equal(ptr[:, h, :3], want), f"pointers differ at step {t}, head {h}"
        assert (ptr[:, :, 3] == 0).all()
        if flushed:
            worst["ckpt"] = max(worst["ckpt"], rel_l2(layer.ckpt.double().cpu().numpy(), S_ref))
            if dual_ref is not None:   # the copy is torch's RNE bf16 cast of the master
                assert torch.equal(layer.ckpt_lo.cpu(), layer.ckpt.cpu().to(torch.bfloat16)), \
                    "read copy is not RNE-bf16 of the master"
        if check_ring:
            rx, rB = _bits(layer.ring_x), _bits(layer.ring_B)
            for b in range(Bt):
                c = t + 1 - int(pm.len[b])
                for j in range(int(pm.len[b])):
                    slot = pm.slot(b, j)
                    src = hist[c + j]
                    xb = src["x_bits"] if wl.in_dtype == "bf16" else src["x"]
                    Bb = src["B_bits"] if wl.in_dtype == "bf16" else src["B"]
                    assert np.array_equal(rx[b, slot].view(xb.dtype), xb[b]), (t, b, j)
                    assert np.array_equal(rB[b, slot].view(Bb.dtype), Bb[b]), (t, b, j)
    assert layer.device_error() == 0
    worst["run"] = rel_l2(np.stack(ys), np.stack(yrefs))
    return worst, layer


@pytest.mark.parametrize("groups", [4, 2, 1])
@pytest.mark.parametrize("s0", ["zeros", "normal"])
def test_tiny_workload_every_step(s0, groups):
    wl = TINY.replace(s0=s0, ngroups=groups)
    w, _ = _run_decode(wl, wl.steps)
    log(f"  worst {w}")
    assert w["step"] < 1e-5 and w["run"] < 1e-5
    assert w["eager"] < 1e-5
    assert w["ckpt"] < 1e-5


def test_tiny_flush_only_at_window():
    wl = TINY.replace(s0="normal", capacity=11)
    w, _ = _run_decode(wl, wl.steps, flush_every_step=False)
    assert w["step"] < 1e-5 and w["ckpt"] < 1e-5


SHAPES = [
    # P, N, H, G, W, R, in_dtype, copy
    (37, 32, 3, 1, 5, 7, "f32", "none"),
    (64, 128, 4, 2, 16, 16, "bf16", "none"),
    (64, 128, 4, 4, 16, 16, "bf16", "bf16"),
    (100, 64, 2, 2, 6, 9, "bf16", "none"),
    (100, 256, 2, 2, 4, 4, "f32", "none"),
    (128, 128, 2, 2, 8, 8, "f32", "bf16"),
    (256, 16, 2, 1, 3, 3, "f32", "none"),
    (1, 16, 1, 1, 1, 1, "f32", "none"),
    (64, 32, 8, 2, 8, 12, "bf16", "none"),
    (48, 256, 2, 1, 7, 8, "bf16", "bf16"),
    # tile counts past whole groups of the workgroup-to-tile order (8 runs of up
    # to 512 KiB of tiles) with a ragged tail: 144 fp32 tiles of 32 KiB (one
    # group of 128), 288 bf16 read-copy tiles of 16 KiB (one group of 256)
    (64, 128, 48, 48, 8, 8, "bf16", "none"),
    (64, 128, 96, 96, 8, 8, "bf16", "bf16"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "P%dN%dH%dG%dW%dR%d-%s-%s" % s)
def test_shapes(shape):
    P, N, H, G, W, R, idt, copy = shape
    wl = TINY.replace(name="sweep", batch=3, headdim=P, dstate=N, nheads=H, ngroups=G, window=W,
                      capacity=R, in_dtype=idt, read_copy=copy, s0="normal", seed=2000 + P + N)
    w, layer = _run_decode(wl, 3 * W + 2)
    log(f"  worst {w}")
    if copy == "none":
        assert w["step"] < 1e-5 and w["run"] < 1e-5
    else:
        assert w["run"] < 2e-2 and w["dual_emul"] < 1e-3
    assert w["eager"] < 1e-5
    assert w["ckpt"] < 1e-5       # the fp32 master is exact in both modes


@pytest.mark.parametrize("fused", [False, True], ids=["decode+flush", "fused"])
def test_dual_master_equals_fp32_checkpoint(fused):
    """The bf16 read copy never feeds back: the dual-mode master is bitwise the
    fp32-mode checkpoint after the same tokens, and the copy is RNE-bf16 of it;
    also through the fused entry point, where a dual-precision layer in step
    folds the window-filling token in one pass from the master."""
    base = TINY.replace(name="dual", batch=4, headdim=64, dstate=128, nheads=4, ngroups=4,
                        window=8, capacity=8, in_dtype="bf16", s0="normal", seed=3001)
    layers = {}
    for copy in ("none", "bf16"):
        wl = base.replace(read_copy=copy)
        cfg = cfg_of(wl)
        A = torch.from_numpy(synth.params(wl)["A"]).to(DEV)
        L = rss.ReplayLayer(cfg, A, DEV)
        L.init_state(torch.from_numpy(synth.initial_state(wl)).to(DEV))
        layers[copy] = (L, A)
    y = torch.empty((4, 4, 64), device=DEV)
    for t in range(27):
        d = dev_inputs(synth.step_inputs(base, t), "bf16")
        for L, _ in layers.values():
            if fused:
                L.decode_flush_step(8, d["x"], d["B"], d["C"], d["dt"], y)
            else:
                L.decode_step(d["x"], d["B"], d["C"], d["dt"], y)
                L.flush_checkpoint(8)
    torch.cuda.synchronize()
    master, dual = layers["none"][0], layers["bf16"][0]
    assert torch.equal(master.ckpt, dual.ckpt)
    assert torch.equal(master.ptr, dual.ptr)
    assert torch.equal(dual.ckpt_lo, dual.ckpt.to(torch.bfloat16))   # torch's cast rounds to nearest even


def test_deterministic():
    wl = TINY.replace(name="det", batch=4, headdim=64, dstate=128, nheads=8, ngroups=8,
                      window=16, capacity=16, in_dtype="bf16", s0="normal", seed=3002)
    outs = []
    for _ in range(2):
        cfg = cfg_of(wl)
        A = torch.from_numpy(synth.params(wl)["A"]).to(DEV)
        L = rss.ReplayLayer(cfg, A, DEV)
        L.init_state(torch.from_numpy(synth.initial_state(wl)).to(DEV))
        ys = []
        for t in range(40):
            d = dev_inputs(synth.step_inputs(wl, t), "bf16")
            y = torch.empty((4, 8, 64), device=DEV)
            L.decode_step(d["x"], d["B"], d["C"], d["dt"], y)
            L.flush_checkpoint(16)
            ys.append(y)
        outs.append((torch.stack(ys).cpu(), L.ckpt.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_explicit_streams():
    """Every call enqueues on the stream it is given: two layers driven on two
    side streams (passed explicitly, default priority), their inputs produced on
    the default stream and handed over with events, equal one layer driven on the
    default stream, bit for bit."""
    wl = TINY.replace(name="streams", batch=3, headdim=64, dstate=128, nheads=4, ngroups=4,
                      window=8, capacity=12, max_draft=4, draft=4, in_dtype="bf16", s0="normal",
                      seed=3003)
    cfg = cfg_of(wl)
    A = torch.from_numpy(synth.params(wl)["A"]).to(DEV)
    S0 = torch.from_numpy(synth.initial_state(wl)).to(DEV)
    ref, a, b = (rss.ReplayLayer(cfg, A, DEV) for _ in range(3))
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    ref.init_state(S0)
    torch.cuda.synchronize()
    a.init_state(S0, stream=sa)
    b.init_state(S0, stream=sb)
    K = wl.draft
    outs = {0: [], 1: [], 2: []}
    keep = []      # inputs stay referenced until the side streams are done with them
    for t in range(20):
        ready = torch.cuda.Event()
        if t % 6 == 5:
            rin = dev_inputs(synth.draft_inputs(wl, t), "bf16")
            nd = torch.from_numpy((K - synth.accepted_drafts(wl, t)).astype(np.int32)).to(DEV)
            keep.append((rin, nd))
            ready.record()
            for idx, (L, s) in enumerate(((ref, None), (a, sa), (b, sb))):
                y = torch.empty((wl.batch, K + 1, wl.nheads, wl.headdim), device=DEV)
                if s is not None:
                    s.wait_event(ready)
                L.verify_k_tokens_fold(wl.window, K, rin["x"], rin["B"], rin["C"], rin["dt"], y, stream=s)
                L.rollback(nd, stream=s)
                outs[idx].append(y)
        else:
            d = dev_inputs(synth.step_inputs(wl, t), "bf16")
            keep.append(d)
            ready.record()
            for idx, (L, s) in enumerate(((ref, None), (a, sa), (b, sb))):
                y = torch.empty((wl.batch, wl.nheads, wl.headdim), device=DEV)
                if s is not None:
                    s.wait_event(ready)
                L.decode_flush_step(wl.window, d["x"], d["B"], d["C"], d["dt"], y, stream=s)
                outs[idx].append(y)
    torch.cuda.synchronize()
    for idx in (1, 2):
        for y0, y1 in zip(outs[0], outs[idx]):
            assert torch.equal(y0, y1)
    for L in (a, b):
        assert torch.equal(L.ckpt, ref.ckpt) and torch.equal(L.ptr, ref.ptr)
        assert torch.equal(L.ring_x, ref.ring_x) and torch.equal(L.ring_B, ref.ring_B)
        assert L.device_error(stream=sa) == 0
    assert ref.device_error() == 0


@pytest.mark.parametrize("copy", ["none", "bf16", "bf16_state"])
def test_empty_batch_every_entry_point(copy):
    """Zero sequences: every Mamba-2 entry point (init, decode, the fused and
    per-sequence folds, flush, verify with and without the fold, rollback, the
    eager baselines) returns OK on empty tensors and launches nothing that could
    touch memory; the device error word stays clear."""
    code = {"none": rss.RSS_COPY_NONE, "bf16": rss.RSS_COPY_BF16, "bf16_state": rss.RSS_STATE_BF16}[copy]
    H, P, N, K = 4, 16, 16, 2
    cfg = rss.make_config(0, H, P, N, H, 4, 6, K, rss.RSS_DTYPE_F32, code)
    A = torch.full((H,), -0.5, device=DEV)
    layer = rss.ReplayLayer(cfg, A, DEV)
    layer.init_state()
    e = lambda *s, dt=torch.float32: torch.empty(s, dtype=dt, device=DEV)
    x, B, C, dt, y = e(0, H, P), e(0, H, N), e(0, H, N), e(0, H), e(0, H, P)
    th = e(0, dt=torch.int32)
    layer.decode_step(x, B, C, dt, y)
    layer.decode_flush_step(4, x, B, C, dt, y)
    layer.decode_flush_step_each(th, x, B, C, dt, y)
    layer.flush_checkpoint(4)
    layer.flush_checkpoint_each(th)
    xs, Bs, Cs, dts, ys = e(0, K + 1, H, P), e(0, K + 1, H, N), e(0, K + 1, H, N), e(0, K + 1, H), e(0, K + 1, H, P)
    layer.verify_k_tokens(K, xs, Bs, Cs, dts, ys)
    layer.rollback(th)
    layer.verify_k_tokens_fold(4, K, xs, Bs, Cs, dts, ys)
    layer.rollback(th)
    S = e(0, H, P, N, dt=torch.bfloat16 if copy == "bf16_state" else torch.float32)
    rss.rss_eager_step(cfg, S, x, B, C, dt, A, y)
    if copy != "bf16_state":
        rss.rss_eager_verify(cfg, e(0, K + 1, H, P, N), th, K, xs, Bs, Cs, dts, A, ys)
    assert layer.device_error() == 0


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_empty_batch_delta_rules(kind):
    """Zero sequences for the delta-rule layers: decode, fused fold, flush and the
    eager baseline return OK on empty tensors."""
    code = rss.RSS_KIND_GDN if kind == "gdn" else rss.RSS_KIND_KDA
    H, P, N = 2, 16, 16
    cfg = rss.make_config(0, H, P, N, H, 4, 4, 0, rss.RSS_DTYPE_F32, rss.RSS_COPY_NONE, code)
    layer = rss.ReplayLayer(cfg, None, DEV)
    layer.init_state()
    e = lambda *s: torch.empty(s, device=DEV)
    q, k, v, beta, o = e(0, H, N), e(0, H, N), e(0, H, P), e(0, H), e(0, H, P)
    alpha = e(0, H, N) if kind == "kda" else e(0, H)
    dec = layer.kda_decode_step if kind == "kda" else layer.gdn_decode_step
    fused = layer.kda_decode_flush_step if kind == "kda" else layer.gdn_decode_flush_step
    dec(q, k, v, beta, alpha, o)
    fused(4, q, k, v, beta, alpha, o)
    layer.flush_checkpoint(4)
    eager = rss.rss_kda_eager_step if kind == "kda" else rss.rss_gdn_eager_step
    eager(cfg, e(0, H, P, N), q, k, v, beta, alpha, o)
    assert layer.device_error() == 0
