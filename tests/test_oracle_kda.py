"""The oracle's Kimi-Delta-Attention rule (per-channel gated delta rule):
reduction to the scalar-gate rule, textbook special cases, exact rational
arithmetic on a scalar case, and replay == eager."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import gdn, kda
import oracle_pins as pins
import workloads
from workloads import synth


def _rand_inputs(rng, Bt, H, dk, dv, scalar_gate=False):
    q = rng.standard_normal((Bt, H, dk))
    k = rng.standard_normal((Bt, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    za = rng.standard_normal((Bt, H, 1) if scalar_gate else (Bt, H, dk))
    alpha = np.exp(-np.log1p(np.exp(za))) * np.ones((Bt, H, dk))
    return {"q": q, "k": k, "v": rng.standard_normal((Bt, H, dv)),
            "beta": 1 / (1 + np.exp(-rng.standard_normal((Bt, H)))), "alpha": alpha}


def test_scalar_gate_is_gated_deltanet():
    """Every channel with the same gate: the KDA rule is the gated DeltaNet
    rule (a separately pinned reference), state and output, over 12 steps, and
    so is the KDA replay model."""
    rng = np.random.default_rng(3)
    Bt, H, dk, dv = 2, 3, 6, 4
    S0 = rng.standard_normal((Bt, H, dv, dk))
    Sk, Sg = S0.copy(), S0.copy()
    model = kda.KDAReplayModel(S0, 4)
    for t in range(12):
        inp = _rand_inputs(rng, Bt, H, dk, dv, scalar_gate=True)
        Sk, ok = kda.eager_step(Sk, inp["q"], inp["k"], inp["v"], inp["beta"], inp["alpha"])
        Sg, og = gdn.eager_step(Sg, inp["q"], inp["k"], inp["v"], inp["beta"], inp["alpha"][..., 0])
        orp = model.decode(inp["q"], inp["k"], inp["v"], inp["beta"], inp["alpha"])
        model.flush(4)
        assert pins.rel_err(Sk, Sg) < 1e-13 and pins.rel_err(ok, og) < 1e-13, t
        assert pins.rel_err(orp, og) < 1e-12, t


def test_beta_zero_is_per_channel_decay():
    """beta = 0: S_t = S_0 Diag(prod of the gates), each key channel (column)
    decayed on its own; o_t = S_t q_t."""
    rng = np.random.default_rng(4)
    S0 = rng.standard_normal((2, 3, 4, 5))
    S = S0.copy()
    prod = np.ones((2, 3, 5))
    for _ in range(5):
        inp = _rand_inputs(rng, 2, 3, 5, 4)
        S, o = kda.eager_step(S, inp["q"], inp["k"], inp["v"], np.zeros((2, 3)), inp["alpha"])
        prod = prod * inp["alpha"]
        assert pins.rel_err(S, S0 * prod[:, :, None, :]) < 1e-14
        assert pins.rel_err(o, np.matmul(S, inp["q"][..., None])[..., 0]) < 1e-14


def test_unit_rate_writes_the_value_at_its_key():
    """beta = 1 and a unit key: whatever the gates, the new state maps k_t to v_t
    exactly (the delta rule replaces the value stored under k_t)."""
    rng = np.random.default_rng(5)
    S = rng.standard_normal((2, 2, 3, 7))
    for _ in range(6):
        inp = _rand_inputs(rng, 2, 2, 7, 3)
        S, _ = kda.eager_step(S, inp["q"], inp["k"], inp["v"], np.ones((2, 2)), inp["alpha"])
        got = np.matmul(S, inp["k"][..., None])[..., 0]
        assert np.allclose(got, inp["v"], atol=1e-13, rtol=0)


def test_scalar_case_in_exact_rationals():
    """d_k = d_v = 1: S_t = alpha S (1 - beta k^2) + beta v k and o = S q, run in
    exact fractions on dyadic inputs; the fp64 eager step is exact there too."""
    steps = [(Fraction(1, 2), Fraction(3, 4), Fraction(-5, 8), Fraction(1, 4), Fraction(3, 8)),
             (Fraction(7, 8), Fraction(1, 2), Fraction(3, 2), Fraction(1, 2), Fraction(-1, 4)),
             (Fraction(1, 4), Fraction(1, 1), Fraction(-1, 8), Fraction(3, 4), Fraction(5, 4))]
    S_ex = Fraction(3, 2)
    S = np.full((1, 1, 1, 1), 1.5)
    for a, k, v, b, q in steps:
        S_ex = a * S_ex * (1 - b * k * k) + b * v * k
        o_ex = S_ex * q
        S, o = kda.eager_step(S, np.full((1, 1, 1), float(q)), np.full((1, 1, 1), float(k)),
                              np.full((1, 1, 1), float(v)), np.full((1, 1), float(b)),
                              np.full((1, 1, 1), float(a)))
        assert S[0, 0, 0, 0] == float(S_ex) and o[0, 0, 0] == float(o_ex)


@pytest.mark.parametrize("W,dk,dv", [(1, 5, 3), (4, 8, 5), (6, 4, 9), (16, 16, 16)])
def test_replay_equals_eager_kda(W, dk, dv):
    """The checkpoint + ring model gives the eager outputs at every step and its
    fold gives the eager state at every flush."""
    rng = np.random.default_rng(6 + W)
    Bt, H = 2, 3
    S0 = rng.standard_normal((Bt, H, dv, dk))
    model = kda.KDAReplayModel(S0, W)
    S = S0.copy()
    for t in range(3 * W + 5):
        inp = _rand_inputs(rng, Bt, H, dk, dv)
        S, o_e = kda.eager_step(S, inp["q"], inp["k"], inp["v"], inp["beta"], inp["alpha"])
        o_r = model.decode(inp["q"], inp["k"], inp["v"], inp["beta"], inp["alpha"])
        assert pins.rel_err(o_r, o_e) < 1e-12, t
        if model.flush(W):
            assert pins.rel_err(model.ckpt, S) < 1e-12, t


def test_channel_suffix_sums():
    g = np.arange(1.0, 13.0).reshape(4, 1, 3)            # entries 0..3, channels 0..2
    lam, total = kda.channel_suffix(g)
    assert np.array_equal(total[0], g[:, 0].sum(axis=0))
    for j in range(4):
        assert np.array_equal(lam[j, 0], g[j + 1:, 0].sum(axis=0))


def test_generator_shapes_and_ranges():
    wl = workloads.get("kda_b256_h32_d128_w16").replace(batch=2)
    s = synth.kda_step_inputs(wl, 0)
    assert s["alpha"].shape == (2, 32, 128) and s["beta"].shape == (2, 32)
    assert np.all((s["alpha"] > 0) & (s["alpha"] < 1))
    assert np.allclose(np.linalg.norm(s["k"].astype(np.float64), axis=-1), 1, atol=1e-6)
    assert len(np.unique(s["alpha"][0, 0])) > 100        # gates differ per channel
