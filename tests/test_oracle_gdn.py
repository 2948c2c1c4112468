"""The oracle's gated-DeltaNet rule: textbook special cases and replay == eager."""
import numpy as np

from oracle import gdn
import oracle_pins as pins
import workloads
from workloads import synth


def _rand_inputs(rng, Bt, H, dk, dv):
    q = rng.standard_normal((Bt, H, dk))
    k = rng.standard_normal((Bt, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    return {"q": q, "k": k, "v": rng.standard_normal((Bt, H, dv)),
            "beta": 1 / (1 + np.exp(-rng.standard_normal((Bt, H)))),
            "alpha": np.exp(-np.log1p(np.exp(rng.standard_normal((Bt, H)))))}


def test_beta_zero_is_pure_decay():
    rng = np.random.default_rng(0)
    S0 = rng.standard_normal((2, 3, 4, 5))
    inp = _rand_inputs(rng, 2, 3, 5, 4)
    S, o = gdn.eager_step(S0, inp["q"], inp["k"], inp["v"], np.zeros((2, 3)), inp["alpha"])
    assert pins.rel_err(S, inp["alpha"][..., None, None] * S0) < 1e-15
    assert pins.rel_err(o, np.einsum("bhvk,bhk->bhv", S, inp["q"])) < 1e-14


def test_delta_rule_retrieves_orthonormal_keys():
    """alpha = beta = 1 with orthonormal keys: after writing (k_i, v_i) pairs the
    state maps every k_i to v_i exactly (the textbook delta rule), and rewriting
    a key replaces its value."""
    rng = np.random.default_rng(1)
    dk, dv = 6, 3
    Q, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Q.T                                   # rows orthonormal
    vals = rng.standard_normal((dk, dv))
    S = rng.standard_normal((1, 1, dv, dk)) * 0.0
    one = np.ones((1, 1))
    for i in range(dk):
        S, _ = gdn.eager_step(S, keys[i][None, None], keys[i][None, None], vals[i][None, None], one, one)
    for i in range(dk):
        assert np.allclose(S[0, 0] @ keys[i], vals[i], atol=1e-13)
    new = rng.standard_normal(dv)
    S, o = gdn.eager_step(S, keys[2][None, None], keys[2][None, None], new[None, None], one, one)
    assert np.allclose(o[0, 0], new, atol=1e-13)
    assert np.allclose(S[0, 0] @ keys[4], vals[4], atol=1e-13)


def test_replay_equals_eager_gdn():
    rng = np.random.default_rng(2)
    Bt, H, dk, dv, W = 2, 3, 8, 5, 4
    S0 = rng.standard_normal((Bt, H, dv, dk))
    model = gdn.GDNReplayModel(S0, W)
    S = S0.copy()
    for t in range(19):
        inp = _rand_inputs(rng, Bt, H, dk, dv)
        S, o_e = gdn.eager_step(S, inp["q"], inp["k"], inp["v"], inp["beta"], inp["alpha"])
        o_r = model.decode(inp["q"], inp["k"], inp["v"], inp["beta"], inp["alpha"])
        assert pins.rel_err(o_r, o_e) < 1e-12, t
        for b in range(Bt):
            assert pins.rel_err(model.implied_state(b), S[b]) < 1e-12
        model.flush(W)
        if (t + 1) % W == 0:
            assert pins.rel_err(model.ckpt, S) < 1e-12


def test_gdn_workload_inputs():
    wl = workloads.get("gdn_b256_h32_d128_w16").replace(batch=2)
    s = synth.gdn_step_inputs(wl, 0)
    assert np.allclose(np.linalg.norm(s["q"].astype(np.float64), axis=-1), 1, atol=1e-6)
    assert np.allclose(np.linalg.norm(s["k"].astype(np.float64), axis=-1), 1, atol=1e-6)
    assert (s["beta"] > 0).all() and (s["beta"] < 1).all()
    assert (s["alpha"] > 0).all() and (s["alpha"] < 1).all()
    S0 = np.zeros((2, wl.nheads, wl.headdim, wl.dstate))
    o_e = gdn.eager_scan(S0, [synth.gdn_step_inputs(wl, t) for t in range(3)])[0]
    assert np.isfinite(o_e).all()
