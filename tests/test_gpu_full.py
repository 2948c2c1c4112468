"""Full-size parity, in the launch configuration the benchmark times.

Sizes: batch 256 x 128 heads x P=64 x N=128 (4 MiB fp32 state per sequence),
bf16 x/B/C, W=16; batch 512 speculative rounds with K=4; dual precision over
1024 steps. The oracle checks sampled (sequence, head) pairs one by one (pairs
are independent); properties that hold at any size (replay == eager on the
whole batch, pointers on every sequence, untouched checkpoint bytes) are
checked in full."""
import numpy as np
import pytest
import torch

from oracle import mamba2
from oracle.ring import PointerModel
import workloads
from workloads import synth
from recurrent_state_storage_amd import rss
from gpu_util import DEV, PairGather, cfg_of, dev_inputs, rel_l2, sample_pairs, log

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.mark.parametrize("schedule", ["separate", "fused", "staggered", "fused-G1"])
def test_decode_b256_full_size(schedule):
    """The benchmark workload in each fold schedule the benchmark times: decode +
    flush every W steps, the fused decode + fold, and staggered per-sequence folds;
    and the fused schedule with B and C shared by all heads (G = 1)."""
    wl = workloads.get("mamba2_b256_h128_p64_n128_w16")
    if schedule == "fused-G1":
        wl, schedule = wl.replace(ngroups=1), "fused"
    log(f"[full] {wl.name}: {wl.steps} steps, {schedule} folds every {wl.window}")
    cfg = cfg_of(wl)
    A_np = synth.params(wl)["A"]
    A = torch.from_numpy(A_np).to(DEV)
    layer = rss.ReplayLayer(cfg, A, DEV)
    layer.init_state()
    S_eag = torch.zeros((wl.batch, wl.nheads, wl.headdim, wl.dstate), device=DEV)
    pg = PairGather(wl, sample_pairs(wl, 24, seed=11))
    S_ref = np.zeros((1, len(pg.pairs), wl.headdim, wl.dstate))      # S0 = 0
    A_pair = pg.A(A_np)
    y = torch.empty((wl.batch, wl.nheads, wl.headdim), device=DEV)
    ye = torch.empty_like(y)
    worst_pair = worst_eager = worst_ckpt = 0.0
    ys, refs = [], []
    W = wl.window
    first = 1 + np.arange(wl.batch) % W
    lens = np.zeros(wl.batch, np.int64)
    for t in range(wl.steps):
        s = synth.step_inputs(wl, t)
        d = dev_inputs(s, wl.in_dtype)
        if schedule == "separate" or (schedule == "fused" and (t + 1) % W != 0):
            layer.decode_step(d["x"], d["B"], d["C"], d["dt"], y)
        elif schedule == "fused":
            layer.decode_flush_step(W, d["x"], d["B"], d["C"], d["dt"], y)
        else:
            th = np.where(t < first, first, W).astype(np.int32)
            layer.decode_flush_step_each(torch.from_numpy(th).to(DEV), d["x"], d["B"], d["C"], d["dt"], y)
            lens += 1
            lens[lens >= th] = 0
            assert np.array_equal(layer.ptr[:, :, 1].cpu().numpy(), np.repeat(lens[:, None], wl.nheads, 1)), t
        rss.rss_eager_step(cfg, S_eag, d["x"], d["B"], d["C"], d["dt"], A, ye)
        ps = pg.step(s)
        S_ref, y_ref = mamba2.eager_step(S_ref, A_pair, ps["x"], ps["B"], ps["C"], ps["dt"])
        got = pg.out(y)
        worst_pair = max(worst_pair, rel_l2(got, y_ref))
        ys.append(got)
        refs.append(y_ref)
        worst_eager = max(worst_eager, float(torch.linalg.vector_norm(y - ye) / torch.linalg.vector_norm(ye)))
        if (t + 1) % wl.window == 0 and schedule != "staggered":
            if schedule == "separate":
                layer.flush_checkpoint(wl.window)
            ck = layer.ckpt[torch.as_tensor(pg.b, device=DEV), torch.as_tensor(pg.h, device=DEV)]
            worst_ckpt = max(worst_ckpt, rel_l2(ck.double().cpu().numpy()[None], S_ref))
            st = layer.ptr.cpu()
            assert (st[:, :, 1] == 0).all() and (st[:, :, 0] == 0).all()   # R = W: head returns to 0
        if t % 64 == 0:
            log(f"  step {t}: pair rel-L2 {worst_pair:.2e}, replay vs eager {worst_eager:.2e}")
    run = rel_l2(np.stack(ys), np.stack(refs))
    log(f"  pairs worst/run {worst_pair:.3e}/{run:.3e}; replay vs eager {worst_eager:.3e}; ckpt {worst_ckpt:.3e}")
    assert layer.device_error() == 0
    assert worst_pair < 1e-5 and run < 1e-5
    assert worst_eager < 1e-5
    assert worst_ckpt < 1e-5
    # the eager kernel's own state against the oracle on the pairs
    se = S_eag[torch.as_tensor(pg.b, device=DEV), torch.as_tensor(pg.h, device=DEV)]
    assert rel_l2(se.double().cpu().numpy()[None], S_ref) < 1e-5


def test_spec_b512_full_size():
    wl = workloads.get("mamba2_spec_b512_h128_p64_n128_w16_k4")
    rounds = 6
    log(f"[full] {wl.name}: {rounds} rounds")
    cfg = cfg_of(wl)
    A_np = synth.params(wl)["A"]
    A = torch.from_numpy(A_np).to(DEV)
    Bt, H, P, N, K = wl.batch, wl.nheads, wl.headdim, wl.dstate, wl.draft
    layer = rss.ReplayLayer(cfg, A, DEV)
    layer.init_state()
    pool = torch.zeros((Bt, K + 1, H, P, N), device=DEV)
    src = torch.zeros((Bt,), dtype=torch.int32, device=DEV)
    pm = PointerModel(Bt, wl.capacity)
    pg = PairGather(wl, sample_pairs(wl, 24, seed=12))
    S_ref = np.zeros((1, len(pg.pairs), P, N))
    A_pair = pg.A(A_np)
    y = torch.empty((Bt, K + 1, H, P), device=DEV)
    ye = torch.empty_like(y)
    bidx, hidx = torch.as_tensor(pg.b, device=DEV), torch.as_tensor(pg.h, device=DEV)
    for r in range(rounds):
        rin = synth.draft_inputs(wl, r)
        nacc = synth.accepted_drafts(wl, r)
        d = dev_inputs(rin, wl.in_dtype)
        ck = layer.ckpt.clone()
        layer.verify_k_tokens(K, d["x"], d["B"], d["C"], d["dt"], y)
        rss.rss_eager_verify(cfg, pool, src, K, d["x"], d["B"], d["C"], d["dt"], A, ye)
        # oracle on the pairs: K+1 eager steps from the committed state
        pr = pg.draft(rin)
        states, refs = [], []
        S_run = S_ref
        for i in range(K + 1):
            S_run, yi = mamba2.eager_step(S_run, A_pair, pr["x"][:, i], pr["B"][:, i], pr["C"][:, i], pr["dt"][:, i])
            states.append(S_run)
            refs.append(yi)
        y_ref = np.stack(refs, axis=1)                                   # (1,K+1,n,P)
        got = y[bidx, :, hidx].permute(1, 0, 2).double().cpu().numpy()[None]
        goe = ye[bidx, :, hidx].permute(1, 0, 2).double().cpu().numpy()[None]
        e1, e2 = rel_l2(got, y_ref), rel_l2(goe, y_ref)
        log(f"  round {r}: replay {e1:.2e}, eager+snapshots {e2:.2e}")
        assert e1 < 1e-5 and e2 < 1e-5
        n_drop = torch.from_numpy((K - nacc).astype(np.int32)).to(DEV)
        layer.rollback(n_drop)
        for b in range(Bt):
            pm.append(b, K + 1)
            pm.mark_tentative(b, K + 1)
            pm.rollback(b, int(K - nacc[b]))
        assert torch.equal(layer.ckpt, ck), "verify/rollback changed checkpoint bytes"
        del ck
        ptr = layer.ptr.cpu().numpy()
        want = pm.as_array()
        assert all(np.array_equal(ptr[:, h, :3], want) for h in range(H))
        layer.flush_checkpoint(wl.window)
        for b in range(Bt):
            pm.flush(b, wl.window)
        ptr = layer.ptr.cpu().numpy()
        assert all(np.array_equal(ptr[:, h, :3], pm.as_array()) for h in range(H))
        keep = nacc[pg.b]
        S_ref = np.stack([states[keep[i]][0, i] for i in range(len(pg.pairs))])[None]
        src = torch.from_numpy(nacc.astype(np.int32)).to(DEV)
    assert layer.device_error() == 0


@pytest.mark.parametrize("window", [8, 16, 32])
def test_dual_precision_drift(window):
    """fp32 master + bf16 read copy over 1024 steps on 16 sequences of the
    batch-256 shape: output drift vs the fp64 recurrence stays within 2e-2, the
    master matches the recurrence to 1e-5, and is bitwise the fp32-mode checkpoint."""
    wl = workloads.get(f"mamba2_dual_b256_h128_p64_n128_w{window}").replace(batch=16)
    log(f"[full] {wl.name} (16 sequences), {wl.steps} steps")
    A_np = synth.params(wl)["A"]
    A = torch.from_numpy(A_np).to(DEV)
    dual = rss.ReplayLayer(cfg_of(wl), A, DEV)
    ref32 = rss.ReplayLayer(cfg_of(wl.replace(read_copy="none")), A, DEV)
    dual.init_state()
    ref32.init_state()
    pg = PairGather(wl, sample_pairs(wl, 24, seed=13))
    S_ref = np.zeros((1, len(pg.pairs), wl.headdim, wl.dstate))
    A_pair = pg.A(A_np)
    y = torch.empty((wl.batch, wl.nheads, wl.headdim), device=DEV)
    y32 = torch.empty_like(y)
    drift, ys, refs, master = 0.0, [], [], 0.0
    bidx, hidx = torch.as_tensor(pg.b, device=DEV), torch.as_tensor(pg.h, device=DEV)
    for t in range(wl.steps):
        s = synth.step_inputs(wl, t)
        d = dev_inputs(s, wl.in_dtype)
        dual.decode_step(d["x"], d["B"], d["C"], d["dt"], y)
        ref32.decode_step(d["x"], d["B"], d["C"], d["dt"], y32)
        ps = pg.step(s)
        S_ref, y_ref = mamba2.eager_step(S_ref, A_pair, ps["x"], ps["B"], ps["C"], ps["dt"])
        got = pg.out(y)
        drift = max(drift, rel_l2(got, y_ref))
        ys.append(got)
        refs.append(y_ref)
        if (t + 1) % window == 0:
            dual.flush_checkpoint(window)
            ref32.flush_checkpoint(window)
            ck = dual.ckpt[bidx, hidx].double().cpu().numpy()[None]
            master = max(master, rel_l2(ck, S_ref))
    torch.cuda.synchronize()
    final = rel_l2(ys[-1], refs[-1])
    run = rel_l2(np.stack(ys), np.stack(refs))
    log(f"  W={window}: drift max {drift:.3e}, final {final:.3e}, run {run:.3e}, master {master:.3e}")
    assert torch.equal(dual.ckpt, ref32.ckpt)
    assert drift < 2e-2 and run < 2e-2
    assert master < 1e-5


def test_spec_b512_fold_verify_full_size():
    """The benchmark's speculative schedule at full size: verify with the
    committed-window fold in the same pass, then rollback, no flush call.
    Outputs on sampled pairs against the committed-stream recurrence, every
    (sequence, head) pointer against the integer model, and every folded
    checkpoint (sampled pairs) against the recurrence's state."""
    wl = workloads.get("mamba2_spec_b512_h128_p64_n128_w16_k4")
    rounds = 12
    log(f"[full] {wl.name} with fold in verify: {rounds} rounds")
    cfg = cfg_of(wl)
    A_np = synth.params(wl)["A"]
    A = torch.from_numpy(A_np).to(DEV)
    Bt, H, P, N, K, W = wl.batch, wl.nheads, wl.headdim, wl.dstate, wl.draft, wl.window
    layer = rss.ReplayLayer(cfg, A, DEV)
    layer.init_state()
    pm = PointerModel(Bt, wl.capacity)
    pg = PairGather(wl, sample_pairs(wl, 24, seed=14))
    S_ref = np.zeros((1, len(pg.pairs), P, N))
    A_pair = pg.A(A_np)
    y = torch.empty((Bt, K + 1, H, P), device=DEV)
    bidx, hidx = torch.as_tensor(pg.b, device=DEV), torch.as_tensor(pg.h, device=DEV)
    folds = 0
    for r in range(rounds):
        rin = synth.draft_inputs(wl, r)
        nacc = synth.accepted_drafts(wl, r)
        d = dev_inputs(rin, wl.in_dtype)
        folded = np.array([pm.len[b] >= W for b in range(Bt)])
        for b in range(Bt):
            pm.flush(b, W)
        layer.verify_k_tokens_fold(W, K, d["x"], d["B"], d["C"], d["dt"], y)
        folds += int(folded.sum())
        fp = folded[pg.b]
        if fp.any():
            ck = layer.ckpt[bidx, hidx].double().cpu().numpy()
            assert rel_l2(ck[fp], S_ref[0][fp]) < 1e-5, r
        pr = pg.draft(rin)
        states, refs = [], []
        S_run = S_ref
        for i in range(K + 1):
            S_run, yi = mamba2.eager_step(S_run, A_pair, pr["x"][:, i], pr["B"][:, i], pr["C"][:, i], pr["dt"][:, i])
            states.append(S_run)
            refs.append(yi)
        y_ref = np.stack(refs, axis=1)
        got = y[bidx, :, hidx].permute(1, 0, 2).double().cpu().numpy()[None]
        e1 = rel_l2(got, y_ref)
        assert e1 < 1e-5, r
        layer.rollback(torch.from_numpy((K - nacc).astype(np.int32)).to(DEV))
        for b in range(Bt):
            pm.append(b, K + 1)
            pm.mark_tentative(b, K + 1)
            pm.rollback(b, int(K - nacc[b]))
        ptr = layer.ptr.cpu().numpy()
        assert all(np.array_equal(ptr[:, h, :3], pm.as_array()) for h in range(H)), r
        keep = nacc[pg.b]
        S_ref = np.stack([states[keep[i]][0, i] for i in range(len(pg.pairs))])[None]
    log(f"  {folds} sequence folds over {rounds} rounds")
    assert folds > Bt        # most sequences folded at least once
    assert layer.device_error() == 0


@pytest.mark.parametrize("copy", ["bf16", "bf16_state"])
def test_bf16_tile_modes_b256_full_size(copy):
    """The bf16-tile modes the benchmark times at batch 256 (dual precision and
    the bf16-only checkpoint, W = 16, the two-wavefront replay launch): 48 steps,
    sampled pairs against their fp64 emulators (1e-3) and the exact recurrence
    (2e-2); the eager bf16-stored state beside them, against its emulator."""
    wl = workloads.get("mamba2_dual_b256_h128_p64_n128_w16").replace(read_copy=copy)
    steps = 48
    log(f"[full] {wl.name} read_copy={copy}: {steps} steps")
    cfg = cfg_of(wl)
    A_np = synth.params(wl)["A"]
    A = torch.from_numpy(A_np).to(DEV)
    layer = rss.ReplayLayer(cfg, A, DEV)
    layer.init_state()
    pg = PairGather(wl, sample_pairs(wl, 24, seed=15))
    A_pair = pg.A(A_np)
    Z = np.zeros((1, len(pg.pairs), wl.headdim, wl.dstate))
    emu = mamba2.ReplayModel(Z, A_pair, len(pg.pairs), wl.capacity, read_copy=copy)
    S_ref, S_eb = Z.copy(), Z.copy()
    Se = torch.zeros((wl.batch, wl.nheads, wl.headdim, wl.dstate), dtype=torch.bfloat16, device=DEV)
    ecfg = cfg_of(wl, read_copy=rss.RSS_STATE_BF16)
    y = torch.empty((wl.batch, wl.nheads, wl.headdim), device=DEV)
    ye = torch.empty_like(y)
    got, emus, refs, egot, eemu = [], [], [], [], []
    for t in range(steps):
        s = synth.step_inputs(wl, t)
        d = dev_inputs(s, wl.in_dtype)
        layer.decode_flush_step(wl.window, d["x"], d["B"], d["C"], d["dt"], y)
        rss.rss_eager_step(ecfg, Se, d["x"], d["B"], d["C"], d["dt"], A, ye)
        ps = pg.step(s)
        S_ref, y_ref = mamba2.eager_step(S_ref, A_pair, ps["x"], ps["B"], ps["C"], ps["dt"])
        emus.append(emu.decode(ps["x"], ps["B"], ps["C"], ps["dt"]))
        emu.flush(wl.window)
        S_new, y_eb = mamba2.eager_step(S_eb, A_pair, ps["x"], ps["B"], ps["C"], ps["dt"])
        S_eb = mamba2.lowp.round_bf16(S_new)
        got.append(pg.out(y))
        egot.append(pg.out(ye))
        eemu.append(y_eb)
        refs.append(y_ref)
    vs_emu = rel_l2(np.stack(got), np.stack(emus))
    vs_exact = rel_l2(np.stack(got), np.stack(refs))
    eager_vs_emu = rel_l2(np.stack(egot), np.stack(eemu))
    log(f"  replay vs emulator {vs_emu:.2e}, vs exact {vs_exact:.2e}; eager bf16 vs emulator {eager_vs_emu:.2e}")
    assert vs_emu < 1e-3 and vs_exact < 2e-2 and eager_vs_emu < 1e-3
    assert layer.device_error() == 0


def test_spec_b512_fold_verify_200_rounds():
    """The speculative workload at its stated length: batch 512, K = 4, all 200
    seeded rounds of the verify-with-fold + rollback schedule, each round with
    its own draft inputs (drawn on the device by the workload's seeded
    generator; the oracle reads back the sampled pairs' exact input bits) and
    accepted lengths. After every round: all K+1 outputs of 24 sampled
    (sequence, head) pairs against the fp64 recurrence on the committed stream
    (<= 1e-5), every (sequence, head) pointer against the integer ring model
    (bit-exact), and every folded checkpoint of a sampled pair against the
    recurrence's state (<= 1e-5)."""
    wl = workloads.get("mamba2_spec_b512_h128_p64_n128_w16_k4")
    rounds = wl.rounds
    log(f"[full] {wl.name}: {rounds} rounds, verify with fold + rollback")
    cfg = cfg_of(wl)
    A_np = synth.params(wl)["A"]
    A = torch.from_numpy(A_np).to(DEV)
    Bt, H, P, N, K, W = wl.batch, wl.nheads, wl.headdim, wl.dstate, wl.draft, wl.window
    layer = rss.ReplayLayer(cfg, A, DEV)
    layer.init_state()
    pm = PointerModel(Bt, wl.capacity)
    pg = PairGather(wl, sample_pairs(wl, 24, seed=17))
    S_ref = np.zeros((1, len(pg.pairs), P, N))
    A_pair = pg.A(A_np)
    y = torch.empty((Bt, K + 1, H, P), device=DEV)
    bidx, hidx = torch.as_tensor(pg.b, device=DEV), torch.as_tensor(pg.h, device=DEV)
    gidx = torch.as_tensor(pg.g, device=DEV)

    def host(t):  # (n, K+1, ...) device gather -> (1, K+1, n, ...) exact fp64 values
        a = t.double().cpu().numpy()
        return np.moveaxis(a, 1, 0)[None]

    folds, worst = 0, 0.0
    for r in range(rounds):
        d = synth.device_draft_inputs(wl, r, DEV)
        nacc = synth.accepted_drafts(wl, r)
        folded = pm.len >= W
        for b in np.nonzero(folded)[0]:
            pm.flush(int(b), W)
        layer.verify_k_tokens_fold(W, K, d["x"], d["B"], d["C"], d["dt"], y)
        folds += int(folded.sum())
        fp = folded[pg.b]
        if fp.any():
            ck = layer.ckpt[bidx, hidx].double().cpu().numpy()
            assert rel_l2(ck[fp], S_ref[0][fp]) < 1e-5, r
        px, pB, pC = host(d["x"][bidx, :, hidx]), host(d["B"][bidx, :, gidx]), host(d["C"][bidx, :, gidx])
        pdt = host(d["dt"][bidx, :, hidx])
        states, refs = [], []
        S_run = S_ref
        for i in range(K + 1):
            S_run, yi = mamba2.eager_step(S_run, A_pair, px[:, i], pB[:, i], pC[:, i], pdt[:, i])
            states.append(S_run)
            refs.append(yi)
        y_ref = np.stack(refs, axis=1)
        got = y[bidx, :, hidx].permute(1, 0, 2).double().cpu().numpy()[None]
        e = rel_l2(got, y_ref)
        worst = max(worst, e)
        assert e < 1e-5, r
        layer.rollback(torch.from_numpy((K - nacc).astype(np.int32)).to(DEV))
        pm.len += K + 1                     # verify appends K+1 tentative entries, the
        pm.len -= K - nacc                  # rollback keeps the accepted ones (n_tent back to 0)
        assert np.all(pm.len <= wl.capacity)
        ptr = layer.ptr.cpu().numpy()
        assert all(np.array_equal(ptr[:, h, :3], pm.as_array()) for h in range(H)), r
        keep = nacc[pg.b]
        S_ref = np.stack([states[keep[i]][0, i] for i in range(len(pg.pairs))])[None]
    log(f"  {folds} sequence folds over {rounds} rounds; worst round rel-L2 {worst:.2e}")
    assert folds > 10 * Bt
    assert layer.device_error() == 0
