"""Planted mistakes in the oracle (on the CPU) must each fail at least one pin.

Every mutant below is a plausible slip when writing the recurrence or the
replay model; the test shows the pins are strong enough to notice it."""
import numpy as np
import pytest

from oracle import mamba2
import oracle_pins as pins
import workloads
from workloads import synth


def _step_variant(kind):
    def step(S, A, x, B, C, dt):
        S, A, x, B, C, dt = (np.asarray(v, np.float64) for v in (S, A, x, B, C, dt))
        H, G = S.shape[1], B.shape[1]
        g = np.arange(H) // (H // G)
        if kind == "group_mod":
            g = np.arange(H) % G
        Bh, Ch = B[:, g], C[:, g]
        if kind == "swap_BC":
            Bh, Ch = Ch, Bh
        a = np.exp(dt * A[None])
        if kind == "decay_no_dt":
            a = np.exp(A[None] + 0 * dt)
        if kind == "decay_sign":
            a = np.exp(-dt * A[None])
        scale = dt
        if kind == "drop_dt":
            scale = np.ones_like(dt)
        if kind == "dt_squared":
            scale = dt * dt
        upd = scale[:, :, None, None] * x[:, :, :, None] * Bh[:, :, None, :]
        if kind == "decay_after_update":
            S_new = a[:, :, None, None] * (S + upd)
        else:
            S_new = a[:, :, None, None] * S + upd
        read = S if kind == "output_before_update" else S_new
        y = np.matmul(read, Ch[..., None])[..., 0]
        return S_new, y
    return step


def _scan_of(step):
    def scan(S0, A, xs, Bs, Cs, dts):
        S = np.asarray(S0, np.float64)
        ys = []
        for t in range(len(xs)):
            S, y = step(S, A, xs[t], Bs[t], Cs[t], dts[t])
            ys.append(y)
        return np.stack(ys), S
    return scan


def _all_pins(step):
    scan = _scan_of(step)
    return {
        "one_step": pins.pin_one_step(step) < 1e-12,
        "two_steps": pins.pin_two_steps(step) < 1e-12,
        "geometric": pins.pin_geometric(step) < 1e-12,
        "linear_attention": pins.pin_linear_attention(scan) < 1e-12,
        "exact_rational": pins.pin_exact_rational(scan) == 0.0,
        "golden": pins.pin_golden_two_tokens(step) < 1e-12,
        "unrolled": pins.pin_unrolled(scan, mamba2.unrolled_outputs) < 1e-12,
    }


def test_unmutated_variant_passes_every_pin():
    assert all(_all_pins(_step_variant("none")).values())


@pytest.mark.parametrize("kind", ["group_mod", "swap_BC", "decay_no_dt", "decay_sign", "drop_dt",
                                  "dt_squared", "decay_after_update", "output_before_update"])
def test_eager_mutant_fails_a_pin(kind):
    res = _all_pins(_step_variant(kind))
    assert not all(res.values()), res


# ---- replay-model mutants: caught by replay == eager --------------------------
class _ReplayOffByOne(mamba2.ReplayModel):
    def _output(self, b, C_t, n):          # forgets the newest (current) entry
        return super()._output(b, C_t, n - 1) if n > 1 else super()._output(b, C_t, n)


class _ReplayNoCkptDecay(mamba2.ReplayModel):
    def implied_state(self, b):            # fold without decaying the checkpoint
        n = int(self.ptr.len[b])
        x, Bh, dt, ell = self._window(b, n)
        lam, _ = mamba2.suffix_decay(ell)
        S = self.ckpt[b].copy()
        for j in range(n):
            S = S + (np.exp(lam[j]) * dt[j])[:, None, None] * x[j][:, :, None] * Bh[j][:, None, :]
        return S


_SUFFIX = mamba2.suffix_decay


def _prefix_decay(ell):                    # includes entry j's own decay
    lam, total = _SUFFIX(ell)
    return lam + ell, total


def _replay_vs_eager(model_cls, monkeypatch=None, patch=None) -> float:
    wl = workloads.get("tiny_b2_h4_p16_n16_w8").replace(s0="normal")
    A = synth.params(wl)["A"]
    S0 = synth.initial_state(wl)
    model = model_cls(S0, A, wl.ngroups, wl.capacity)
    S = S0.astype(np.float64)
    worst = 0.0
    for t in range(20):
        s = synth.step_inputs(wl, t)
        S, y_e = mamba2.eager_step(S, A, s["x"], s["B"], s["C"], s["dt"])
        worst = max(worst, pins.rel_err(model.decode(s["x"], s["B"], s["C"], s["dt"]), y_e))
        model.flush(wl.window)
    return worst


def test_replay_model_passes():
    assert _replay_vs_eager(mamba2.ReplayModel) < 1e-12


@pytest.mark.parametrize("cls", [_ReplayOffByOne, _ReplayNoCkptDecay])
def test_replay_mutant_fails(cls):
    assert _replay_vs_eager(cls) > 1e-6


def test_suffix_sum_mutant_fails(monkeypatch):
    monkeypatch.setattr(mamba2, "suffix_decay", _prefix_decay)
    assert _replay_vs_eager(mamba2.ReplayModel) > 1e-6


def test_bf16_state_without_per_token_rounding_fails_the_swamping_pin(monkeypatch):
    """A bf16-stored eager state that forgets to round after each token (only
    the initial store rounds) is caught by the swamping closed form."""
    import test_oracle_lowp as tl
    calls = {"n": 0}
    real = mamba2.lowp.round_bf16

    def first_only(a):
        calls["n"] += 1
        return real(a) if calls["n"] == 1 else np.asarray(a, np.float64)
    monkeypatch.setattr(mamba2.lowp, "round_bf16", first_only)
    with pytest.raises(AssertionError):
        tl.test_eager_bf16_state_swamping_closed_form()


def test_bf16_checkpoint_rounding_every_token_fails_the_fold_pin(monkeypatch):
    """A bf16-only checkpoint that rounds every token (folding after each
    decode) loses the increments the once-per-window pin requires."""
    import test_oracle_lowp as tl
    real_flush = mamba2.ReplayModel.flush
    monkeypatch.setattr(mamba2.ReplayModel, "flush", lambda self, th: real_flush(self, 1))
    with pytest.raises(AssertionError):
        tl.test_bf16_checkpoint_rounds_once_per_fold()


def _kda_gate_on_rows(S, q, k, v, beta, alpha):
    """Mutant: the per-channel gate applied to the value rows instead of the
    key channels (only meaningful when d_v == d_k)."""
    S = np.asarray(S, np.float64) * np.asarray(alpha, np.float64)[..., :, None]
    ones = np.ones_like(np.asarray(alpha, np.float64))
    return _KDA_STEP(S, q, k, v, beta, ones)


def test_kda_gate_on_the_wrong_side_fails_a_pin(monkeypatch):
    from oracle import kda
    import test_oracle_kda as tk
    monkeypatch.setattr(kda, "eager_step", _kda_gate_on_rows)
    rng = np.random.default_rng(4)
    S0 = rng.standard_normal((1, 1, 5, 5))
    inp = tk._rand_inputs(rng, 1, 1, 5, 5)
    S, _ = kda.eager_step(S0, inp["q"], inp["k"], inp["v"], np.zeros((1, 1)), inp["alpha"])
    assert pins.rel_err(S, S0 * inp["alpha"][:, :, None, :]) > 1e-3   # the beta = 0 pin's check


def test_kda_replay_without_the_new_gate_fails(monkeypatch):
    from oracle import kda
    import test_oracle_kda as tk
    real = kda.KDAReplayModel._apply
    monkeypatch.setattr(kda.KDAReplayModel, "_apply",
                        lambda self, b, vec, n, g_next=None: real(self, b, vec, n))
    with pytest.raises(AssertionError):
        tk.test_replay_equals_eager_kda(4, 8, 5)


from oracle import kda as _kda_mod  # noqa: E402
_KDA_STEP = _kda_mod.eager_step
