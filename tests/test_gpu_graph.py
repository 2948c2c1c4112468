"""The decode entry points under HIP graph capture: one window of decode steps
(plain replay launches and the fused decode + fold) captured once and replayed
with fresh inputs copied into the captured buffers, eager work and
synchronisations between the replays; every replay's outputs, checkpoint and
pointers equal those of the same calls made without a graph, bit for bit; and
one speculative round (verify with the fold, rollback) captured and replayed
round after round. No entry point on these paths issues a memset or a host
synchronisation."""
import numpy as np
import pytest
import torch

import workloads
from workloads import synth
from recurrent_state_storage_amd import rss
from gpu_util import DEV, cfg_of, dev_inputs, log

pytestmark = pytest.mark.gpu


# every checkpoint precision: fp32 (fold fused into the replay), dual (replay of
# the bf16 copy, then the flush of the master), a bf16-stored checkpoint (folded
# on the bf16 matrix cores inside the two-wavefront decode)
@pytest.mark.parametrize("copy", ["none", "bf16", "bf16_state"])
def test_captured_window_replays_match_eager_calls(copy):
    wl = workloads.get("tiny_b2_h4_p16_n16_w8").replace(
        name="graph", batch=4, nheads=4, ngroups=2, headdim=64, dstate=128, window=4, capacity=4,
        in_dtype="bf16", read_copy=copy, s0="normal", seed=9100)
    W = wl.window
    log(f"[graph] {copy}: capture {W} decode steps (the last fused with the fold), replay 3 times")
    cfg = cfg_of(wl)
    A = torch.from_numpy(synth.params(wl)["A"]).to(DEV)
    S0 = torch.from_numpy(synth.initial_state(wl)).to(DEV)
    ref, cap = rss.ReplayLayer(cfg, A, DEV), rss.ReplayLayer(cfg, A, DEV)
    ref.init_state(S0)
    cap.init_state(S0)
    Bt, H, P = wl.batch, wl.nheads, wl.headdim
    # static input and output buffers of the captured window
    inp = [dev_inputs(synth.step_inputs(wl, t), "bf16") for t in range(W)]
    ys = [torch.empty((Bt, H, P), device=DEV) for _ in range(W)]

    def window(layer, xs, outs):
        for t in range(W):
            d = xs[t]
            if t == W - 1:
                layer.decode_flush_step(W, d["x"], d["B"], d["C"], d["dt"], outs[t])
            else:
                layer.decode_step(d["x"], d["B"], d["C"], d["dt"], outs[t])

    # warm up on a side stream (no capture), then restore the start state
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        window(cap, inp, ys)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    cap.init_state(S0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        window(cap, inp, ys)
    torch.cuda.synchronize()
    for rep in range(3):
        fresh = [dev_inputs(synth.step_inputs(wl, 100 * rep + t), "bf16") for t in range(W)]
        for t in range(W):
            for k in inp[t]:
                inp[t][k].copy_(fresh[t][k])
        g.replay()
        y_ref = [torch.empty_like(ys[0]) for _ in range(W)]
        window(ref, fresh, y_ref)       # the same calls, not captured
        torch.cuda.synchronize()
        for t in range(W):
            assert torch.equal(ys[t], y_ref[t]), (rep, t)
        assert torch.equal(cap.ckpt, ref.ckpt), rep
        if copy == "bf16":
            assert torch.equal(cap.ckpt_lo, ref.ckpt_lo), rep
        assert torch.equal(cap.ptr, ref.ptr), rep
        assert torch.equal(cap.ring_x, ref.ring_x) and torch.equal(cap.ring_B, ref.ring_B), rep
        _ = torch.ones(1000, device=DEV).sum().item()   # eager work between replays
    assert cap.device_error() == 0 and ref.device_error() == 0


def test_captured_dual_fold_step_replayed_at_every_phase():
    """A dual-precision rss_decode_flush_step captured on the token that fills
    every window (so the one-pass fold from the fp32 master is recorded), then
    replayed on every token: the kernel decides each fold on the device, so on
    the replays where no window fills it only decodes. Checkpoint, copy, ring
    and pointers equal rss_decode_step + rss_flush_checkpoint bit for bit after
    every replay; outputs up to rounding (the copy's values, summed in the fp32
    kernel's order)."""
    wl = workloads.get("tiny_b2_h4_p16_n16_w8").replace(
        name="graph-dual", batch=4, nheads=4, ngroups=4, headdim=64, dstate=128, window=4, capacity=4,
        in_dtype="bf16", read_copy="bf16", s0="normal", seed=9300)
    W = wl.window
    cfg = cfg_of(wl)
    A = torch.from_numpy(synth.params(wl)["A"]).to(DEV)
    S0 = torch.from_numpy(synth.initial_state(wl)).to(DEV)
    ref, cap = rss.ReplayLayer(cfg, A, DEV), rss.ReplayLayer(cfg, A, DEV)
    Bt, H, P = wl.batch, wl.nheads, wl.headdim
    inp = dev_inputs(synth.step_inputs(wl, 0), "bf16")
    y = torch.empty((Bt, H, P), device=DEV)

    def lead_in(layer):                      # W - 1 plain decodes: the next token fills every window
        layer.init_state(S0)
        for t in range(W - 1):
            d = dev_inputs(synth.step_inputs(wl, t), "bf16")
            layer.decode_step(d["x"], d["B"], d["C"], d["dt"], y)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        lead_in(cap)
        cap.decode_flush_step(W, inp["x"], inp["B"], inp["C"], inp["dt"], y)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    lead_in(cap)
    lead_in(ref)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap.decode_flush_step(W, inp["x"], inp["B"], inp["C"], inp["dt"], y)
    torch.cuda.synchronize()
    folds = 0
    for t in range(W - 1, W - 1 + 3 * W + 2):
        fresh = dev_inputs(synth.step_inputs(wl, t), "bf16")
        for k in inp:
            inp[k].copy_(fresh[k])
        g.replay()
        y_ref = torch.empty_like(y)
        ref.decode_step(fresh["x"], fresh["B"], fresh["C"], fresh["dt"], y_ref)
        ref.flush_checkpoint(W)
        torch.cuda.synchronize()
        folds += int((ref.ptr[:, 0, 1] == 0).all())
        rel = float(torch.linalg.vector_norm(y - y_ref) / torch.linalg.vector_norm(y_ref))
        assert rel < 1e-5, (t, rel)
        assert torch.equal(cap.ckpt, ref.ckpt), t
        assert torch.equal(cap.ckpt_lo, ref.ckpt_lo), t
        assert torch.equal(cap.ptr, ref.ptr), t
        assert torch.equal(cap.ring_x, ref.ring_x) and torch.equal(cap.ring_B, ref.ring_B), t
        assert torch.equal(cap.ring_dl, ref.ring_dl), t
        _ = torch.ones(1000, device=DEV).sum().item()   # eager work between replays
    log(f"[graph] dual one-pass fold step replayed {3 * W + 2} times, {folds} of them folding")
    assert folds >= 3
    assert cap.device_error() == 0 and ref.device_error() == 0


def test_captured_speculative_round_replays_match_eager_calls():
    """One speculative round (verify K+1 tokens with the committed-window fold,
    then rollback by a device n_drop array) captured once and replayed for eight
    rounds with fresh drafts and acceptance counts copied into the captured
    buffers: outputs, checkpoint, ring and pointers equal the uncaptured calls
    bit for bit after every round, folds included."""
    wl = workloads.get("mamba2_spec_b512_h128_p64_n128_w16_k4").replace(
        name="graph-spec", batch=4, nheads=4, ngroups=4, s0="normal", seed=9200)
    K, W = wl.draft, wl.window
    log(f"[graph] capture one speculative round (K={K}, W={W}, R={wl.capacity}), replay 8 rounds")
    cfg = cfg_of(wl)
    A = torch.from_numpy(synth.params(wl)["A"]).to(DEV)
    S0 = torch.from_numpy(synth.initial_state(wl)).to(DEV)
    ref, cap = rss.ReplayLayer(cfg, A, DEV), rss.ReplayLayer(cfg, A, DEV)
    ref.init_state(S0)
    cap.init_state(S0)
    Bt, H, P = wl.batch, wl.nheads, wl.headdim
    d = dev_inputs(synth.draft_inputs(wl, 0), "bf16")
    y = torch.empty((Bt, K + 1, H, P), device=DEV)
    nd = torch.zeros((Bt,), dtype=torch.int32, device=DEV)

    def round_(layer, inp, out, n_drop):
        layer.verify_k_tokens_fold(W, K, inp["x"], inp["B"], inp["C"], inp["dt"], out)
        layer.rollback(n_drop)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        round_(cap, d, y, nd)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    cap.init_state(S0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        round_(cap, d, y, nd)
    torch.cuda.synchronize()
    folded = 0
    for r in range(8):
        fresh = dev_inputs(synth.draft_inputs(wl, r), "bf16")
        nd_r = torch.from_numpy((K - synth.accepted_drafts(wl, r)).astype(np.int32)).to(DEV)
        for k in d:
            d[k].copy_(fresh[k])
        nd.copy_(nd_r)
        g.replay()
        y_ref = torch.empty_like(y)
        before = ref.ptr[:, 0, 1].clone()
        round_(ref, fresh, y_ref, nd_r)
        torch.cuda.synchronize()
        folded += int((ref.ptr[:, 0, 1] < before).sum())
        assert torch.equal(y, y_ref), r
        assert torch.equal(cap.ckpt, ref.ckpt), r
        assert torch.equal(cap.ptr, ref.ptr), r
        assert torch.equal(cap.ring_x, ref.ring_x) and torch.equal(cap.ring_B, ref.ring_B), r
        assert torch.equal(cap.ring_dl, ref.ring_dl), r
        _ = torch.ones(1000, device=DEV).sum().item()   # eager work between replays
    log(f"  sequence folds over the 8 rounds: {folded}")
    assert folded > 0
    assert cap.device_error() == 0 and ref.device_error() == 0
