"""Property tests of the oracle itself (CPU, hypothesis): random small shapes
and random schedules of decode, speculative rounds (verify + rollback) and
flushes with random thresholds. Whatever the schedule, the replay model's
outputs equal the eager recurrence over the committed stream, its checkpoint
plus window equal the eager state, rollback never touches the checkpoint, and
its pointers follow the integer ring rules."""
import numpy as np
from hypothesis import given, settings, HealthCheck, strategies as st

from oracle import mamba2
import oracle_pins as pins


@st.composite
def schedules(draw):
    Bt = draw(st.integers(1, 3))
    G = draw(st.integers(1, 2))
    H = G * draw(st.integers(1, 2))
    P = draw(st.integers(1, 6))
    N = draw(st.integers(1, 6))
    K = draw(st.integers(0, 3))
    W = draw(st.integers(1, 6))
    R = W + K + draw(st.integers(0, 2))
    ops = draw(st.lists(st.sampled_from(["decode", "round", "flush"]), min_size=1, max_size=24))
    seed = draw(st.integers(0, 2**31 - 1))
    return dict(Bt=Bt, G=G, H=H, P=P, N=N, K=K, W=W, R=R, ops=ops, seed=seed)


@settings(max_examples=200, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(schedules())
def test_replay_model_matches_eager_under_any_schedule(c):
    rng = np.random.default_rng(c["seed"])
    Bt, G, H, P, N, K, W, R = (c[k] for k in ("Bt", "G", "H", "P", "N", "K", "W", "R"))
    A = -np.exp(rng.uniform(0, 1, H))
    S0 = rng.standard_normal((Bt, H, P, N))
    model = mamba2.ReplayModel(S0, A, G, R)
    S = S0.copy()                                   # eager state over the committed stream

    def toks(n):
        return (rng.standard_normal((Bt, n, H, P)), rng.standard_normal((Bt, n, G, N)),
                rng.standard_normal((Bt, n, G, N)), np.log1p(np.exp(rng.standard_normal((Bt, n, H)) - 2)))

    for op in c["ops"]:
        lens = model.ptr.len.copy()
        if op == "decode":
            if np.any(lens >= R):                    # a full ring must be flushed first
                model.flush(W)
                lens = model.ptr.len.copy()
            x, B, C, dt = toks(1)
            y = model.decode(x[:, 0], B[:, 0], C[:, 0], dt[:, 0])
            S, y_ref = mamba2.eager_step(S, A, x[:, 0], B[:, 0], C[:, 0], dt[:, 0])
            assert pins.rel_err(y, y_ref) < 1e-10
        elif op == "round":
            if np.any(lens + K + 1 > R):
                model.flush(W)
                lens = model.ptr.len.copy()
                if np.any(lens + K + 1 > R):
                    continue
            x, B, C, dt = toks(K + 1)
            ck = model.ckpt.copy()
            y = model.verify(x, B, C, dt)
            n_acc = rng.integers(0, K + 1, Bt)
            ys, states, S_run = [], [], S
            for i in range(K + 1):
                S_run, yi = mamba2.eager_step(S_run, A, x[:, i], B[:, i], C[:, i], dt[:, i])
                ys.append(yi)
                states.append(S_run)
            assert pins.rel_err(y, np.stack(ys, axis=1)) < 1e-10
            model.rollback(K - n_acc)
            assert np.array_equal(model.ckpt, ck)
            assert np.array_equal(model.ptr.len, lens + n_acc + 1)
            assert not np.any(model.ptr.n_tent)
            S = np.stack([states[n_acc[b]][b] for b in range(Bt)])
        else:
            th = rng.integers(1, W + 1, Bt)
            before = model.ptr.as_array().copy()
            folded = model.flush(th)
            for b in range(Bt):
                assert (b in folded) == (before[b, 1] >= th[b])
                if b in folded:
                    assert model.ptr.len[b] == 0
                    assert model.ptr.head[b] == (before[b, 0] + before[b, 1]) % R
        for b in range(Bt):
            assert pins.rel_err(model.implied_state(b), S[b]) < 1e-10
