"""The oracle's replay model (checkpoint + ring) against its eager recurrence,
the ring pointer model, speculative rounds and the dual-precision emulator."""
import numpy as np
import pytest

from oracle import mamba2, lowp
from oracle.ring import PointerModel, RingError
import oracle_pins as pins
import workloads
from workloads import synth

TINY = "tiny_b2_h4_p16_n16_w8"


def _tiny_inputs(wl):
    A = synth.params(wl)["A"]
    st = [synth.step_inputs(wl, t) for t in range(wl.steps)]
    return A, st


@pytest.mark.parametrize("s0", ["zeros", "normal"])
@pytest.mark.parametrize("groups", [4, 2, 1])
def test_replay_equals_eager_every_step(s0, groups):
    """Outputs from checkpoint + buffered inputs equal the eager outputs at every
    step, and each flush leaves the checkpoint equal to the eager state."""
    wl = workloads.get(TINY).replace(s0=s0, ngroups=groups)
    A, st = _tiny_inputs(wl)
    S0 = synth.initial_state(wl)
    model = mamba2.ReplayModel(S0, A, wl.ngroups, wl.capacity)
    S = S0.astype(np.float64)
    for t, s in enumerate(st):
        S, y_e = mamba2.eager_step(S, A, s["x"], s["B"], s["C"], s["dt"])
        y_r = model.decode(s["x"], s["B"], s["C"], s["dt"])
        assert pins.rel_err(y_r, y_e) < 1e-12, t
        for b in range(wl.batch):
            assert pins.rel_err(model.implied_state(b), S[b]) < 1e-12
        folded = model.flush(wl.window)
        if (t + 1) % wl.window == 0:
            assert folded == list(range(wl.batch))
            assert pins.rel_err(model.ckpt, S) < 1e-12
            assert list(model.ptr.len) == [0] * wl.batch
        else:
            assert folded == []
            assert list(model.ptr.len) == [(t + 1) % wl.window] * wl.batch


def test_ring_slots_hold_the_inputs():
    """After any number of steps, window position j holds token (c + j)'s input."""
    wl = workloads.get(TINY).replace(capacity=11, window=8)
    A, st = _tiny_inputs(wl)
    model = mamba2.ReplayModel(synth.initial_state(wl), A, wl.ngroups, wl.capacity)
    for t, s in enumerate(st[:29]):
        model.decode(s["x"], s["B"], s["C"], s["dt"])
        model.flush(wl.window)
        c = t + 1 - int(model.ptr.len[0])   # tokens folded so far
        for j in range(int(model.ptr.len[0])):
            slot = model.ptr.slot(0, j)
            assert np.array_equal(model.ring_x[0, slot], st[c + j]["x"][0])
            assert np.array_equal(model.ring_B[0, slot], st[c + j]["B"][0])
    assert model.ptr.head[0] == (29 // 8 * 8) % 11


def test_pointer_model_rules():
    pm = PointerModel(2, 5)
    assert pm.append(0, 3) == [0, 1, 2]
    pm.mark_tentative(0, 3)
    with pytest.raises(RingError):
        pm.flush(0, 1)
    with pytest.raises(RingError):
        pm.rollback(0, 4)
    pm.rollback(0, 2)
    assert (pm.len[0], pm.n_tent[0]) == (1, 0)
    assert pm.flush(0, 1) and pm.head[0] == 1 and pm.len[0] == 0
    assert pm.append(0, 5) == [1, 2, 3, 4, 0]
    with pytest.raises(RingError):
        pm.append(0, 1)
    with pytest.raises(RingError):
        pm.rollback(1, 1)          # nothing tentative
    assert pm.flush(0, 5) and pm.head[0] == 1
    assert pm.as_array().tolist() == [[1, 0, 0], [0, 0, 0]]


def _spec_case(rounds=12, seed_wl="tiny_b2_h4_p16_n16_w8"):
    wl = workloads.get(seed_wl).replace(window=8, capacity=8 + 4, max_draft=4, draft=4,
                                        rounds=rounds, s0="normal")
    A = synth.params(wl)["A"]
    rin = [synth.draft_inputs(wl, r) for r in range(rounds)]
    nacc = [synth.accepted_drafts(wl, r) for r in range(rounds)]
    return wl, A, rin, nacc


def test_verify_rollback_equals_committed_stream():
    """Each round's K+1 outputs equal the eager recurrence over (committed prefix +
    the round's tokens); rollback and verify never touch the checkpoint."""
    wl, A, rin, nacc = _spec_case()
    S0 = synth.initial_state(wl)
    ref, S_fin = mamba2.speculative_reference(S0, A, rin, nacc)
    model = mamba2.ReplayModel(S0, A, wl.ngroups, wl.capacity)
    pm = PointerModel(wl.batch, wl.capacity)
    for r in range(len(rin)):
        ck = model.ckpt.copy()
        y = model.verify(rin[r]["x"], rin[r]["B"], rin[r]["C"], rin[r]["dt"])
        assert pins.rel_err(y, ref[r]) < 1e-12, r
        model.rollback(wl.draft - nacc[r])
        assert np.array_equal(model.ckpt, ck)
        # the pointers follow the integer model
        for b in range(wl.batch):
            pm.append(b, wl.draft + 1)
            pm.mark_tentative(b, wl.draft + 1)
            pm.rollback(b, int(wl.draft - nacc[r][b]))
            pm.flush(b, wl.window)
        model.flush(wl.window)
        assert np.array_equal(model.ptr.as_array(), pm.as_array())
        assert int(model.ptr.len.max()) <= wl.window - 1
    for b in range(wl.batch):
        assert pins.rel_err(model.implied_state(b), S_fin[b]) < 1e-12


def test_dual_precision_emulator():
    """bf16 read copy: the master is untouched by the copy's rounding, the output
    error obeys |dy| <= exp(Lam_c) ||S_c - copy||_F ||C_t|| per head, and the
    whole run stays within 2e-2 of the fp64 recurrence."""
    wl = workloads.get(TINY).replace(s0="normal")
    A, st = _tiny_inputs(wl)
    S0 = synth.initial_state(wl)
    exact = mamba2.ReplayModel(S0, A, wl.ngroups, wl.capacity)
    dual = mamba2.ReplayModel(S0, A, wl.ngroups, wl.capacity, read_copy="bf16")
    S = S0.astype(np.float64)
    ys_e, ys_d = [], []
    g = mamba2.group_index(wl.nheads, wl.ngroups)
    for t, s in enumerate(st):
        S, y_ref = mamba2.eager_step(S, A, s["x"], s["B"], s["C"], s["dt"])
        y_e = exact.decode(s["x"], s["B"], s["C"], s["dt"])
        y_d = dual.decode(s["x"], s["B"], s["C"], s["dt"])
        for b in range(wl.batch):
            n = int(dual.ptr.len[b])
            _, _, _, ell = dual._window(b, n)
            total = ell.sum(axis=0)
            for h in range(wl.nheads):
                bound = (np.exp(total[h]) * np.linalg.norm(dual.ckpt[b, h] - dual.copy[b, h])
                         * np.linalg.norm(np.asarray(s["C"], np.float64)[b, g[h]]))
                assert np.linalg.norm(y_d[b, h] - y_e[b, h]) <= bound * (1 + 1e-9) + 1e-300
        exact.flush(wl.window)
        dual.flush(wl.window)
        assert np.array_equal(dual.ckpt, exact.ckpt)
        assert np.array_equal(dual.copy, lowp.round_bf16(dual.ckpt))
        ys_e.append(y_ref)
        ys_d.append(y_d)
    err = pins.rel_err(np.stack(ys_d), np.stack(ys_e))
    assert 1e-5 < err < 2e-2


def test_decode_refuses_uncommitted_round():
    wl, A, rin, nacc = _spec_case(rounds=1)
    model = mamba2.ReplayModel(synth.initial_state(wl), A, wl.ngroups, wl.capacity)
    model.verify(rin[0]["x"], rin[0]["B"], rin[0]["C"], rin[0]["dt"])
    s = synth.step_inputs(wl, 0)
    with pytest.raises(RingError):
        model.decode(s["x"], s["B"], s["C"], s["dt"])
    with pytest.raises(RingError):
        model.flush(1)


def test_staggered_thresholds_fold_each_sequence_on_its_own_phase():
    """Per-sequence fold thresholds: 1 + (b mod W) until sequence b's first fold,
    W after it, so sequence b folds after tokens 1 + (b mod W) + k W; every
    output still equals the eager one, and every fold leaves that sequence's
    checkpoint at its eager state."""
    wl = workloads.get(TINY).replace(batch=6, ngroups=2, s0="normal")
    W = 4
    A, st = _tiny_inputs(wl)
    S0 = synth.initial_state(wl)
    model = mamba2.ReplayModel(S0, A, wl.ngroups, W)
    S = S0.astype(np.float64)
    first = 1 + np.arange(wl.batch) % W
    for t, s in enumerate(st[:20]):
        S, y_e = mamba2.eager_step(S, A, s["x"], s["B"], s["C"], s["dt"])
        assert pins.rel_err(model.decode(s["x"], s["B"], s["C"], s["dt"]), y_e) < 1e-12, t
        th = np.where(t < first, first, W)
        folded = model.flush(th)
        want = [b for b in range(wl.batch) if (t + 1 - first[b]) % W == 0 and t + 1 >= first[b]]
        assert folded == want, t
        for b in folded:
            assert pins.rel_err(model.ckpt[b], S[b]) < 1e-12
    # one value per sequence, all equal, is the scalar threshold
    m1 = mamba2.ReplayModel(S0, A, wl.ngroups, W)
    m2 = mamba2.ReplayModel(S0, A, wl.ngroups, W)
    for s in st[:9]:
        m1.decode(s["x"], s["B"], s["C"], s["dt"])
        m2.decode(s["x"], s["B"], s["C"], s["dt"])
        assert m1.flush(W) == m2.flush(np.full(wl.batch, W))
    assert np.array_equal(m1.ckpt, m2.ckpt)
