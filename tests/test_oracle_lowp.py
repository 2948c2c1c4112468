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
