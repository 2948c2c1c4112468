"""GPU parity of speculative verify + rollback (replay) and of the eager
snapshot baseline, against the eager recurrence run on the committed stream;
pointers bit-exact against the ring model; checkpoint bytes untouched by
verify and rollback. Also mixes plain decode steps between rounds."""
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

BASE = workloads.get("tiny_b2_h4_p16_n16_w8")


def _spec_wl(**kw):
    d = dict(name="spec", batch=5, nheads=4, ngroups=2, headdim=32, dstate=64, window=8,
             capacity=12, max_draft=4, draft=4, rounds=14, in_dtype="bf16", s0="normal", seed=4001)
    d.update(kw)
    return BASE.replace(**d)


def _eager_round(S, A, r_in, b_sel=None):
    """Outputs of the round's K+1 tokens and the states after each, from S."""
    states, ys = [], []
    Kp1 = r_in["x"].shape[1]
    for i in range(Kp1):
        S, y = mamba2.eager_step(S, A, r_in["x"][:, i], r_in["B"][:, i], r_in["C"][:, i], r_in["dt"][:, i])
        states.append(S)
        ys.append(y)
    return np.stack(ys, axis=1), states


@pytest.mark.parametrize("copy", ["none", "bf16"])
def test_verify_rollback_matches_committed_stream(copy):
    _rounds_against_oracle(_spec_wl(read_copy=copy))


# The matrix-core ring terms of a bf16 verify at the shapes their blocking
# meets: N = 16 (half of each 32-wide K slice empty), N = 256, row counts that
# leave a partial 16-row block (P = 17, 100, 1), K + 1 = 8 outputs, a window
# of 27 positions (two 16-entry blocks), and grouped B rows; and 144 tiles of
# 32 KiB (batch 3 x 48 heads), past one whole group of the workgroup-to-tile
# order (8 runs of 16 tiles) with a ragged tail.
@pytest.mark.parametrize("P,N,H,G,W,R,K", [(17, 16, 2, 1, 6, 14, 7), (100, 256, 2, 2, 5, 10, 3),
                                           (64, 128, 3, 3, 20, 27, 7), (1, 32, 2, 1, 1, 3, 2),
                                           (64, 128, 48, 48, 8, 12, 4)])
def test_verify_ring_term_shapes(P, N, H, G, W, R, K):
    _rounds_against_oracle(_spec_wl(headdim=P, dstate=N, nheads=H, ngroups=G, window=W, capacity=R,
                                    max_draft=K, draft=K, rounds=8, batch=3, seed=4100 + P + N))


def _rounds_against_oracle(wl):
    copy = wl.read_copy
    log(f"[spec] {wl} ")
    cfg = cfg_of(wl)
    A_np = synth.params(wl)["A"]
    A = torch.from_numpy(A_np).to(DEV)
    S0 = synth.initial_state(wl)
    layer = rss.ReplayLayer(cfg, A, DEV)
    layer.init_state(torch.from_numpy(S0).to(DEV))
    pm = PointerModel(wl.batch, wl.capacity)
    S_ref = S0.astype(np.float64)
    Bt, H, P, K = wl.batch, wl.nheads, wl.headdim, wl.draft
    tol = 1e-5 if copy == "none" else 2e-2
    worst = 0.0
    ys_all, refs_all = [], []
    for r in range(wl.rounds):
        rin = synth.draft_inputs(wl, r)
        nacc = synth.accepted_drafts(wl, r)
        d = dev_inputs(rin, wl.in_dtype)
        y = torch.full((Bt, K + 1, H, P), float("nan"), device=DEV)
        ck_before = layer.ckpt.clone()
        layer.verify_k_tokens(K, d["x"], d["B"], d["C"], d["dt"], y)
        for b in range(Bt):
            pm.append(b, K + 1)
            pm.mark_tentative(b, K + 1)
        assert np.array_equal(layer.ptr.cpu().numpy()[:, 0, :3], pm.as_array())
        y_ref, states = _eager_round(S_ref, A_np, rin)
        yg = y.double().cpu().numpy()
        worst = max(worst, rel_l2(yg, y_ref))
        ys_all.append(yg)
        refs_all.append(y_ref)
        n_drop = torch.from_numpy((K - nacc).astype(np.int32)).to(DEV)
        layer.rollback(n_drop)
        for b in range(Bt):
            pm.rollback(b, int(K - nacc[b]))
        torch.cuda.synchronize()
        assert torch.equal(layer.ckpt, ck_before), "verify/rollback touched the checkpoint"
        ptr = layer.ptr.cpu().numpy()
        for h in range(H):
            assert np.array_equal(ptr[:, h, :3], pm.as_array()), f"round {r} head {h}"
        S_ref = np.stack([states[nacc[b]][b] for b in range(Bt)])
        layer.flush_checkpoint(wl.window)
        for b in range(Bt):
            pm.flush(b, wl.window)
        assert np.array_equal(layer.ptr.cpu().numpy()[:, 0, :3], pm.as_array())
        if r % 5 == 4:   # a few plain decode tokens between rounds
            for t in range(3):
                s = synth.step_inputs(wl, 1000 * r + t)
                dd = dev_inputs(s, wl.in_dtype)
                yd = torch.empty((Bt, H, P), device=DEV)
                layer.decode_step(dd["x"], dd["B"], dd["C"], dd["dt"], yd)
                for b in range(Bt):
                    pm.append(b, 1)
                S_ref, y1 = mamba2.eager_step(S_ref, A_np, s["x"], s["B"], s["C"], s["dt"])
                worst = max(worst, rel_l2(yd.double().cpu().numpy(), y1))
                layer.flush_checkpoint(wl.window)
                for b in range(Bt):
                    pm.flush(b, wl.window)
    assert layer.device_error() == 0
    run = rel_l2(np.stack(ys_all), np.stack(refs_all))
    log(f"  worst step rel-L2 {worst:.3e}, run {run:.3e}")
    assert run < tol
    if copy == "none":
        assert worst < 1e-5


def test_eager_snapshot_baseline():
    """Eager verify with a snapshot per draft token: outputs and every snapshot
    equal the eager recurrence; rollback = next round reads slot n_acc."""
    wl = _spec_wl(rounds=6)
    cfg = cfg_of(wl)
    A_np = synth.params(wl)["A"]
    A = torch.from_numpy(A_np).to(DEV)
    Bt, H, P, N, K = wl.batch, wl.nheads, wl.headdim, wl.dstate, wl.draft
    S0 = synth.initial_state(wl)
    pool = torch.zeros((Bt, K + 1, H, P, N), device=DEV)
    src = torch.full((Bt,), 2, dtype=torch.int32, device=DEV)   # any slot can hold the start
    pool[:, 2] = torch.from_numpy(S0).to(DEV)
    S_ref = S0.astype(np.float64)
    for r in range(wl.rounds):
        rin = synth.draft_inputs(wl, r)
        nacc = synth.accepted_drafts(wl, r)
        d = dev_inputs(rin, wl.in_dtype)
        y = torch.full((Bt, K + 1, H, P), float("nan"), device=DEV)
        rss.rss_eager_verify(cfg, pool, src, K, d["x"], d["B"], d["C"], d["dt"], A, y)
        y_ref, states = _eager_round(S_ref, A_np, rin)
        assert rel_l2(y.double().cpu().numpy(), y_ref) < 1e-5, r
        snaps = pool.double().cpu().numpy()
        for i in range(K + 1):
            assert rel_l2(snaps[:, i], states[i]) < 1e-5
        S_ref = np.stack([states[nacc[b]][b] for b in range(Bt)])
        src = torch.from_numpy(nacc.astype(np.int32)).to(DEV)


def test_verify_with_zero_drafts_equals_decode():
    """K = 0 verify + rollback(0) is a plain decode step."""
    wl = _spec_wl(in_dtype="f32")
    cfg = cfg_of(wl)
    A = torch.from_numpy(synth.params(wl)["A"]).to(DEV)
    S0 = torch.from_numpy(synth.initial_state(wl)).to(DEV)
    L1, L2 = rss.ReplayLayer(cfg, A, DEV), rss.ReplayLayer(cfg, A, DEV)
    L1.init_state(S0)
    L2.init_state(S0)
    zero = torch.zeros((wl.batch,), dtype=torch.int32, device=DEV)
    for t in range(19):
        d = dev_inputs(synth.step_inputs(wl, t), "f32")
        y1 = torch.empty((wl.batch, wl.nheads, wl.headdim), device=DEV)
        y2 = torch.empty((wl.batch, 1, wl.nheads, wl.headdim), device=DEV)
        L1.decode_step(d["x"], d["B"], d["C"], d["dt"], y1)
        L2.verify_k_tokens(0, d["x"].unsqueeze(1), d["B"].unsqueeze(1), d["C"].unsqueeze(1),
                           d["dt"].unsqueeze(1), y2)
        L2.rollback(zero)
        for L in (L1, L2):
            L.flush_checkpoint(wl.window)
        assert torch.equal(y1, y2[:, 0])
    assert torch.equal(L1.ckpt, L2.ckpt) and torch.equal(L1.ptr, L2.ptr)


def test_device_errors_and_order():
    wl = _spec_wl(batch=2, window=4, capacity=8, max_draft=4)
    cfg = cfg_of(wl)
    A = torch.from_numpy(synth.params(wl)["A"]).to(DEV)
    L = rss.ReplayLayer(cfg, A, DEV)
    L.init_state()
    Bt, H, P, K = wl.batch, wl.nheads, wl.headdim, 4
    # order errors are host-side and leave everything untouched
    with pytest.raises(rss.RssError) as e:
        L.rollback(torch.zeros((Bt,), dtype=torch.int32, device=DEV))
    assert e.value.status == rss.RSS_E_ORDER
    rin = dev_inputs(synth.draft_inputs(wl, 0), wl.in_dtype)
    y = torch.empty((Bt, K + 1, H, P), device=DEV)
    L.verify_k_tokens(K, rin["x"], rin["B"], rin["C"], rin["dt"], y)
    s = dev_inputs(synth.step_inputs(wl, 0), wl.in_dtype)
    yd = torch.empty((Bt, H, P), device=DEV)
    for call in (lambda: L.decode_step(s["x"], s["B"], s["C"], s["dt"], yd),
                 lambda: L.flush_checkpoint(4),
                 lambda: L.verify_k_tokens(K, rin["x"], rin["B"], rin["C"], rin["dt"], y)):
        with pytest.raises(rss.RssError) as e:
            call()
        assert e.value.status == rss.RSS_E_ORDER
    # rollback beyond the tentative count: device error, sequence unchanged
    before = L.ptr.clone()
    L.rollback(torch.tensor([6, 1], dtype=torch.int32, device=DEV))
    assert L.device_error() == rss.RSS_DEV_ROLLBACK_RANGE
    after = L.ptr.cpu()
    assert torch.equal(after[0], before.cpu()[0])                 # seq 0 untouched
    assert after[1, :, 1].tolist() == [4] * H and after[1, :, 2].tolist() == [0] * H
    # ring overflow: seq 0 still holds 5 tentative entries; decode until full
    L.init_state()
    for t in range(8):
        L.decode_step(s["x"], s["B"], s["C"], s["dt"], yd)
    assert L.device_error() == 0
    yd.zero_()
    L.decode_step(s["x"], s["B"], s["C"], s["dt"], yd)       # 9th entry into R = 8
    assert L.device_error() == rss.RSS_DEV_RING_OVERFLOW
    assert torch.isnan(yd).all()
    assert L.ptr.cpu()[:, :, 1].unique().tolist() == [8]
    # flush recovers
    L.flush_checkpoint(4)
    L.decode_step(s["x"], s["B"], s["C"], s["dt"], yd)
    assert torch.isfinite(yd).all()


def test_empty_batch_is_a_no_op():
    wl = _spec_wl(batch=0)
    cfg = cfg_of(wl)
    A = torch.from_numpy(synth.params(wl)["A"]).to(DEV)
    L = rss.ReplayLayer(cfg, A, DEV)
    L.init_state()
    e = torch.empty((0, wl.nheads, wl.headdim), device=DEV)
    eB = torch.empty((0, wl.ngroups, wl.dstate), dtype=torch.bfloat16, device=DEV)
    L.decode_step(e.to(torch.bfloat16), eB, eB, torch.empty((0, wl.nheads), device=DEV), e)
    L.flush_checkpoint(1)
    assert L.device_error() == 0


@pytest.mark.parametrize("copy,K,G", [("none", 4, 4), ("bf16", 4, 4), ("none", 0, 4), ("none", 7, 4),
                                     ("none", 4, 2), ("bf16", 4, 2)])
def test_verify_with_fold_equals_flush_then_verify(copy, K, G):
    """rss_verify_k_tokens_fold(W) against rss_flush_checkpoint(W) followed by
    rss_verify_k_tokens: checkpoint, read copy, ring and pointers bit for bit
    after every round; outputs equal up to rounding and match the eager
    recurrence on the committed stream; no flush call in the fused loop."""
    # one B row set per head: R = W + K_max (the fold frees slots in the same
    # pass); grouped B rows: R = W + 2K + 1, no slot reuse within a call
    R = 8 + max(K, 1) if G == 4 else 8 + 2 * K + 1
    wl = _spec_wl(read_copy=copy, ngroups=G, max_draft=max(K, 1), draft=K, capacity=R, rounds=12,
                  seed=4100 + K + G)
    log(f"[spec] verify+fold vs flush+verify, copy={copy}, K={K}, G={G}, R={R}")
    cfg = cfg_of(wl)
    A_np = synth.params(wl)["A"]
    A = torch.from_numpy(A_np).to(DEV)
    S0 = torch.from_numpy(synth.initial_state(wl)).to(DEV)
    sep, fus = rss.ReplayLayer(cfg, A, DEV), rss.ReplayLayer(cfg, A, DEV)
    sep.init_state(S0)
    fus.init_state(S0)
    S_ref = synth.initial_state(wl).astype(np.float64)
    Bt, H, P, W = wl.batch, wl.nheads, wl.headdim, wl.window
    tol = 1e-5 if copy == "none" else 2e-2
    worst = worst_pair = 0.0
    folds = 0
    for r in range(wl.rounds):
        rin = synth.draft_inputs(wl, r)
        nacc = synth.accepted_drafts(wl, r) if K > 0 else np.zeros(Bt, np.int32)
        d = dev_inputs(rin, wl.in_dtype)
        y1 = torch.empty((Bt, K + 1, H, P), device=DEV)
        y2 = torch.empty_like(y1)
        lens = sep.ptr[:, 0, 1].cpu().numpy()
        folds += int(np.sum(lens >= W))
        sep.flush_checkpoint(W)
        sep.verify_k_tokens(K, d["x"], d["B"], d["C"], d["dt"], y1)
        fus.verify_k_tokens_fold(W, K, d["x"], d["B"], d["C"], d["dt"], y2)
        torch.cuda.synchronize()
        assert torch.equal(sep.ckpt, fus.ckpt), r
        if copy == "bf16":
            assert torch.equal(sep.ckpt_lo, fus.ckpt_lo), r
            assert torch.equal(y1, y2), r          # same launches in this mode
        assert torch.equal(sep.ptr, fus.ptr), r
        assert torch.equal(sep.ring_x, fus.ring_x) and torch.equal(sep.ring_B, fus.ring_B), r
        assert torch.equal(sep.ring_dl, fus.ring_dl), r
        worst_pair = max(worst_pair, float(torch.linalg.vector_norm(y1 - y2) / torch.linalg.vector_norm(y1)))
        y_ref, states = _eager_round(S_ref, A_np, rin)
        worst = max(worst, rel_l2(y2.double().cpu().numpy(), y_ref))
        nd = torch.from_numpy((K - nacc).astype(np.int32)).to(DEV)
        sep.rollback(nd)
        fus.rollback(nd)
        S_ref = np.stack([states[nacc[b]][b] for b in range(Bt)])
    log(f"  folds {folds}, fused vs separate {worst_pair:.2e}, vs oracle {worst:.2e}")
    assert folds > 0
    assert worst_pair < 1e-5 and worst < tol
    assert sep.device_error() == 0 and fus.device_error() == 0
