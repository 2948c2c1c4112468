"""Seeded generators: determinism, shapes, and the stated distributions."""
import numpy as np

import workloads
from workloads import synth


def test_deterministic_and_independent_of_order():
    wl = workloads.get("tiny_b2_h4_p16_n16_w8")
    a = synth.step_inputs(wl, 5)
    _ = synth.step_inputs(wl, 3)
    b = synth.step_inputs(wl, 5)
    for k in ("x", "B", "C", "dt"):
        assert np.array_equal(a[k], b[k])
    assert not np.array_equal(a["x"], synth.step_inputs(wl, 6)["x"])


def test_shapes_and_dtypes():
    wl = workloads.get("mamba2_b256_h128_p64_n128_w16").replace(batch=3)
    s = synth.step_inputs(wl, 0)
    assert s["x"].shape == (3, 128, 64) and s["B"].shape == (3, 128, 128)
    assert s["C"].shape == (3, 128, 128) and s["dt"].shape == (3, 128)
    assert s["x_bits"].dtype == np.uint16
    assert np.array_equal(synth.bf16_value(s["x_bits"]), s["x"])
    d = synth.draft_inputs(workloads.get("mamba2_spec_b512_h128_p64_n128_w16_k4").replace(batch=2), 0)
    assert d["x"].shape == (2, 5, 128, 64) and d["dt"].shape == (2, 5, 128)


def test_distributions():
    wl = workloads.get("mamba2_b256_h128_p64_n128_w16").replace(batch=16)
    s = synth.step_inputs(wl, 1)
    assert abs(float(s["x"].mean())) < 0.01 and abs(float(s["x"].std()) - 1) < 0.01
    z = np.log(np.expm1(s["dt"].astype(np.float64))) + 2.0      # invert softplus(z - 2)
    assert abs(z.mean()) < 0.03 and abs(z.std() - 1) < 0.03
    A = synth.params(wl)["A"]
    assert A.shape == (128,) and (A <= -1).all() and (A >= -np.e).all()
    n = np.concatenate([synth.accepted_drafts(workloads.get("mamba2_spec_b512_h128_p64_n128_w16_k4"), r)
                        for r in range(20)])
    assert set(np.unique(n)) == {0, 1, 2, 3, 4}
    assert abs(n.mean() - 2.0) < 0.05


def test_workload_table():
    for name, wl in workloads.WORKLOADS.items():
        assert wl.name == name
        assert wl.nheads % wl.ngroups == 0
        assert wl.capacity >= wl.window + wl.max_draft
