"""The oracle's eager recurrence against closed forms, exact arithmetic, the
hand-worked golden example and invariants (CPU only)."""
import numpy as np
import pytest

from oracle import mamba2
import oracle_pins as pins
import workloads
from workloads import synth


def _scan(S0, A, xs, Bs, Cs, dts):
    return mamba2.eager_scan(S0, A, xs, Bs, Cs, dts)


def test_one_step_closed_form():
    assert pins.pin_one_step(mamba2.eager_step) < 1e-14


def test_two_steps_closed_form():
    assert pins.pin_two_steps(mamba2.eager_step) < 1e-14


def test_geometric_series():
    assert pins.pin_geometric(mamba2.eager_step) < 1e-13


def test_no_decay_is_causal_linear_attention():
    assert pins.pin_linear_attention(_scan) < 1e-13


def test_exact_rational_arithmetic():
    assert pins.pin_exact_rational(_scan) == 0.0


def test_golden_two_tokens():
    assert pins.pin_golden_two_tokens(mamba2.eager_step) < 1e-14


def test_recurrence_equals_unrolled_form():
    assert pins.pin_unrolled(_scan, mamba2.unrolled_outputs) < 1e-12


def test_fp64_error_bounded_by_50_digit_run():
    assert pins.pin_mpmath(_scan) < 1e-13


def test_unrolled_form_on_tiny_workload():
    """Recurrence == semiseparable-matrix form on the whole tiny workload (64 steps),
    with S0 = 0 and with S0 ~ N(0,1)."""
    for s0 in ("zeros", "normal"):
        wl = workloads.get("tiny_b2_h4_p16_n16_w8").replace(s0=s0)
        A = synth.params(wl)["A"]
        st = [synth.step_inputs(wl, t) for t in range(wl.steps)]
        xs, Bs, Cs, dts = (np.stack([s[k] for s in st]) for k in ("x", "B", "C", "dt"))
        S0 = synth.initial_state(wl)
        ys = mamba2.eager_scan(S0, A, xs, Bs, Cs, dts)[0]
        yu = mamba2.unrolled_outputs(S0, A, xs, Bs, Cs, dts)
        assert pins.rel_err(ys, yu) < 1e-12


def test_state_size_matches_pages():
    g = pins.load_golden("state_size.txt")
    wl = workloads.get("mamba2_b256_h128_p64_n128_w16")
    assert wl.state_bytes_per_seq == int(g["state_bytes_per_seq"][0]) == 4 * 2**20
    tokens = wl.state_bytes_per_seq / g["kv_bytes_per_token"][0]
    assert abs(tokens - g["equivalent_tokens_approx"][0]) / tokens < 0.05


# ---- invariants -----------------------------------------------------------
def _random_case(seed, T=7, Bt=3, H=4, G=2, P=5, N=6):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, Bt, H, P)), rng.standard_normal((T, Bt, G, N)),
            rng.standard_normal((T, Bt, G, N)), np.log1p(np.exp(rng.standard_normal((T, Bt, H)) - 2)),
            -np.exp(rng.random(H)))


def test_linear_in_x_from_zero_state():
    xs, Bs, Cs, dts, A = _random_case(10)
    S0 = np.zeros(xs.shape[1:] + (Bs.shape[-1],))
    y1 = mamba2.eager_scan(S0, A, xs, Bs, Cs, dts)[0]
    y2 = mamba2.eager_scan(S0, A, 2.5 * xs, Bs, Cs, dts)[0]
    assert pins.rel_err(y2, 2.5 * y1) < 1e-14


def test_batch_and_head_permutation_equivariance():
    xs, Bs, Cs, dts, A = _random_case(11, G=4)
    rng = np.random.default_rng(12)
    S0 = rng.standard_normal(xs.shape[1:] + (Bs.shape[-1],))
    y = mamba2.eager_scan(S0, A, xs, Bs, Cs, dts)[0]
    pb, ph = rng.permutation(xs.shape[1]), rng.permutation(xs.shape[2])
    yp = mamba2.eager_scan(S0[pb][:, ph], A[ph], xs[:, pb][:, :, ph], Bs[:, pb][:, :, ph],
                           Cs[:, pb][:, :, ph], dts[:, pb][:, :, ph])[0]
    assert np.array_equal(yp, y[:, pb][:, :, ph])


def test_groups_equal_broadcast_per_head():
    """G = 1 equals G = H with B, C copied to every head."""
    xs, Bs, Cs, dts, A = _random_case(13, G=1)
    S0 = np.zeros(xs.shape[1:] + (Bs.shape[-1],))
    H = xs.shape[2]
    y1 = mamba2.eager_scan(S0, A, xs, Bs, Cs, dts)[0]
    yH = mamba2.eager_scan(S0, A, xs, np.repeat(Bs, H, axis=2), np.repeat(Cs, H, axis=2), dts)[0]
    assert np.array_equal(y1, yH)


def test_group_index():
    assert list(mamba2.group_index(8, 2)) == [0, 0, 0, 0, 1, 1, 1, 1]
    assert list(mamba2.group_index(4, 4)) == [0, 1, 2, 3]
    with pytest.raises(ValueError):
        mamba2.group_index(6, 4)
