"""bf16 rounding (oracle side and the input generator) against torch's CPU cast,
a library routine with round-to-nearest-even."""
import numpy as np
import torch

from oracle import lowp
from workloads import synth


def _cases():
    rng = np.random.default_rng(0)
    v = rng.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    # exact ties between two bf16 neighbours, both parities of the kept bit
    u = rng.integers(0, 2**31 - 2**24, 4000, dtype=np.int64).astype(np.uint32)
    ties = ((u & ~np.uint32(0xFFFF)) | np.uint32(0x8000)).view(np.float32)
    tiny = np.array([1e-40, -1e-40, 0.0, -0.0, 3.4e38, -3.4e38], np.float32)
    return np.concatenate([v, ties[np.isfinite(ties)], tiny])


def test_oracle_bf16_matches_torch():
    a = _cases()
    want = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    got = lowp.round_bf16_from_f32(a)
    assert np.array_equal(got, want)


def test_generator_bf16_matches_torch():
    a = _cases()
    bits = synth.bf16_bits(a)
    want = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, want)
    assert np.array_equal(synth.bf16_value(bits).astype(np.float64),
                          torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy())


def test_round_f32_then_bf16():
    rng = np.random.default_rng(1)
    a = rng.standard_normal(1000)
    want = torch.from_numpy(a).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(lowp.round_bf16(a), want)


# ---- stored-bf16 state: per-token rounding vs once per fold -----------------
# Closed form (swamping): a state of exact value 1 receiving +2^-9 per token
# with no decay. In bf16 (8 significant bits, spacing 2^-7 just above 1) the
# sum 1 + 2^-9 lies below the midpoint and rounds back to 1, so a state stored
# after every token never moves, while the exact state is 1 + t 2^-9. Folding
# once per window of 8 tokens adds 8 * 2^-9 = 2^-6, an exact bf16 step, so
# the once-per-fold checkpoint stays exact (P1, "Trois ennuis nés de la même
# fusion" and "Tenir le journal plutôt que le solde").
def _swamp_inputs(T, P=2, N=2):
    xs = np.full((T, 1, 1, P), 2.0 ** -9)
    Bs = np.ones((T, 1, 1, N))
    Cs = np.zeros((T, 1, 1, N))
    Cs[..., 0] = 1.0
    dts = np.ones((T, 1, 1))
    S0 = np.ones((1, 1, P, N))
    return S0, np.zeros(1), xs, Bs, Cs, dts


def test_eager_bf16_state_swamping_closed_form():
    from oracle import mamba2
    T = 64
    S0, A, xs, Bs, Cs, dts = _swamp_inputs(T)
    ys, S_T = mamba2.eager_scan_bf16_state(S0, A, xs, Bs, Cs, dts)
    assert np.all(S_T == 1.0)                               # never moves
    assert np.all(ys == 1.0 + 2.0 ** -9)                    # y from the unrounded new state
    ye, _, _ = mamba2.eager_scan(S0, A, xs, Bs, Cs, dts)
    t = np.arange(1, T + 1)[:, None, None, None]
    assert np.all(ye == 1.0 + t * 2.0 ** -9)                # the exact recurrence


def test_bf16_checkpoint_rounds_once_per_fold():
    from oracle import mamba2
    T, W = 64, 8
    S0, A, xs, Bs, Cs, dts = _swamp_inputs(T)
    m = mamba2.ReplayModel(S0, A, 1, W, read_copy="bf16_state")
    for t in range(T):
        y = m.decode(xs[t], Bs[t], Cs[t], dts[t])
        assert np.all(y == 1.0 + (t + 1) * 2.0 ** -9)        # exact: no rounding lost
        if m.flush(W):
            assert np.all(m.ckpt == 1.0 + ((t + 1) // W) * 2.0 ** -6)
    # with a window of one token the fold happens every token: the eager bf16 state
    m1 = mamba2.ReplayModel(S0, A, 1, 1, read_copy="bf16_state")
    for t in range(T):
        y = m1.decode(xs[t], Bs[t], Cs[t], dts[t])
        m1.flush(1)
        assert np.all(y == 1.0 + 2.0 ** -9) and np.all(m1.ckpt == 1.0)


def test_bf16_checkpoint_window_one_equals_eager_bf16_state():
    """Random inputs: a bf16-only checkpoint folded after every token is the
    bf16-stored eager state, step by step (same rounding points)."""
    from oracle import mamba2
    rng = np.random.default_rng(7)
    Bt, H, G, P, N, T = 2, 4, 2, 5, 8, 40
    A = -np.exp(rng.random(H))
    xs = rng.standard_normal((T, Bt, H, P))
    Bs = rng.standard_normal((T, Bt, G, N))
    Cs = rng.standard_normal((T, Bt, G, N))
    dts = np.log1p(np.exp(rng.standard_normal((T, Bt, H)) - 2))
    S0 = rng.standard_normal((Bt, H, P, N))
    ye, Se = mamba2.eager_scan_bf16_state(S0, A, xs, Bs, Cs, dts)
    m = mamba2.ReplayModel(S0, A, G, 1, read_copy="bf16_state")
    for t in range(T):
        y = m.decode(xs[t], Bs[t], Cs[t], dts[t])
        m.flush(1)
        np.testing.assert_allclose(y, ye[t], rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(m.ckpt, Se)
    assert np.array_equal(lowp.round_bf16(Se), Se)           # stored values are bf16


def test_bf16_checkpoint_error_bounded_by_its_roundings():
    """Each stored checkpoint differs from the exact state by at most the
    accumulated bf16 rounding: per fold and element at most half an ulp, i.e.
    2^-8 of the unrounded value (8 significant bits), carried forward decayed."""
    from oracle import mamba2
    rng = np.random.default_rng(8)
    Bt, H, P, N, T, W = 1, 2, 4, 8, 48, 8
    A = -np.exp(rng.random(H))
    xs = rng.standard_normal((T, Bt, H, P))
    Bs = rng.standard_normal((T, Bt, H, N))
    Cs = rng.standard_normal((T, Bt, H, N))
    dts = np.log1p(np.exp(rng.standard_normal((T, Bt, H)) - 2))
    S0 = np.zeros((Bt, H, P, N))
    _, _, kept = mamba2.eager_scan(S0, A, xs, Bs, Cs, dts, keep=range(0, T + 1, W))
    m = mamba2.ReplayModel(S0, A, H, W, read_copy="bf16_state")
    bound = np.zeros((Bt, H, P, N))
    for t in range(T):
        m.decode(xs[t], Bs[t], Cs[t], dts[t])
        if (t + 1) % W == 0:
            dec = np.exp(np.sum(dts[t + 1 - W:t + 1] * A[None, None, :], axis=0))[..., None, None]
            m.flush(W)
            exact = kept[t + 1]
            # error <= decayed previous error + this fold's rounding (<= 2^-8 |unrounded|)
            bound = dec * bound + 2.0 ** -8 * np.abs(m.ckpt) * (1 + 2.0 ** -7)
            err = np.abs(m.ckpt - exact)
            assert np.all(err <= bound + 1e-15), float(np.max(err - bound))
            assert np.any(m.ckpt != exact)                  # rounding did happen
