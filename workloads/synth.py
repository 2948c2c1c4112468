"""Seeded input generators (NumPy PCG64), shared by the oracle's tests and the HIP path.

Every draw comes from ``numpy.random.default_rng([seed, stream, index])`` so any
step or round can be regenerated on its own, in any order:

  stream 0            A = -exp(U(0,1)) per head (computed in fp64, stored fp32),
                      times a_scale (0.01 for the long-memory workloads)
  stream 1, step t    x (Bt,H,P), B (Bt,G,N), C (Bt,G,N), z (Bt,H): standard
                      normals drawn in that order as float32; dt = softplus(z - 2)
                      computed in fp64 and stored fp32
  stream 2, round r   the same four draws for a speculative round, shaped
                      (Bt,K+1,H,P), (Bt,K+1,G,N), (Bt,K+1,G,N), (Bt,K+1,H)
  stream 3, round r   accepted drafts n_acc ~ Uniform{0..K}, one per sequence
  stream 4            S0 ~ N(0,1) (Bt,H,P,N) float32, for the "normal" S0 variant
  stream 5, step t    gated-DeltaNet inputs (see ``gdn_step_inputs``)
  stream 6, step t    Kimi-Delta-Attention inputs (see ``kda_step_inputs``)

Long runs whose inputs would take minutes to draw on the host (200 speculative
rounds at batch 512 are 42 GB of inputs) draw them on the device instead, with
torch's counter-based (Philox) generator seeded per round or step (streams 7-9,
``device_*`` below): the same distributions, rounded to the same storage types.
A consumer on the host (the oracle's tests) copies back the exact bits it needs.

Inputs stored as bf16 are rounded from the float32 draw with round-to-nearest-
even; the returned float32 arrays are the exact values of those bf16 numbers, so
an fp64 consumer sees the very bits the device reads.

Nothing here is part of the method: no decay, update or output is computed.
"""
from __future__ import annotations

import numpy as np

from .shapes import Workload


def _rng(seed: int, stream: int, idx: int | None = None) -> np.random.Generator:
    key = [seed, stream] if idx is None else [seed, stream, idx]
    return np.random.default_rng(key)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Adds half of the dropped 16 bits (minus one when the kept part is even) and
    truncates. Exact for every finite value (overflow rounds to Inf); NaN inputs
    are not handled (the generators never draw them)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return u.astype(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> their exact float32 values."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _softplus64(u: np.ndarray) -> np.ndarray:
    u = u.astype(np.float64)
    return np.maximum(u, 0.0) + np.log1p(np.exp(-np.abs(u)))


def _store(a: np.ndarray, dtype: str) -> dict:
    """Round a float32 draw to the storage dtype; return values (+ bits for bf16)."""
    if dtype == "f32":
        return {"val": np.ascontiguousarray(a, dtype=np.float32), "bits": None}
    if dtype == "bf16":
        bits = bf16_bits(a)
        return {"val": bf16_value(bits), "bits": bits}
    raise ValueError(dtype)


def params(wl: Workload) -> dict:
    """Per-head parameters: A (H,) float32, A = -a_scale * exp(U(0,1)) (fp64, then
    rounded to fp32; a_scale = 1 except for the long-memory workloads)."""
    u = _rng(wl.seed, 0).random(wl.nheads)
    return {"A": (-wl.a_scale * np.exp(u)).astype(np.float32)}


def initial_state(wl: Workload) -> np.ndarray:
    """S0 (Bt,H,P,N) float32: zeros, or N(0,1) for the "normal" variant."""
    shape = (wl.batch, wl.nheads, wl.headdim, wl.dstate)
    if wl.s0 == "zeros":
        return np.zeros(shape, np.float32)
    return _rng(wl.seed, 4).standard_normal(shape, dtype=np.float32)


def _draw_tokens(rng: np.random.Generator, wl: Workload, lead: tuple) -> dict:
    Bt, H, P, N, G = wl.batch, wl.nheads, wl.headdim, wl.dstate, wl.ngroups
    x = rng.standard_normal((Bt, *lead, H, P), dtype=np.float32)
    B = rng.standard_normal((Bt, *lead, G, N), dtype=np.float32)
    C = rng.standard_normal((Bt, *lead, G, N), dtype=np.float32)
    z = rng.standard_normal((Bt, *lead, H), dtype=np.float32)
    out = {}
    for k, v in (("x", x), ("B", B), ("C", C)):
        s = _store(v, wl.in_dtype)
        out[k] = s["val"]
        out[k + "_bits"] = s["bits"]
    out["dt"] = _softplus64(z.astype(np.float64) - 2.0).astype(np.float32)
    return out


def step_inputs(wl: Workload, t: int) -> dict:
    """Inputs of plain decode step t (0-based).

    Returns float32 arrays x (Bt,H,P), B (Bt,G,N), C (Bt,G,N), dt (Bt,H) holding
    the exact stored values, and x_bits/B_bits/C_bits (uint16) when stored bf16."""
    return _draw_tokens(_rng(wl.seed, 1, t), wl, ())


def draft_inputs(wl: Workload, r: int) -> dict:
    """Inputs of speculative round r: K+1 tokens per sequence (the last sampled
    token followed by K drafts), shaped (Bt,K+1,...)."""
    return _draw_tokens(_rng(wl.seed, 2, r), wl, (wl.draft + 1,))


def accepted_drafts(wl: Workload, r: int) -> np.ndarray:
    """n_acc (Bt,) int32 ~ Uniform{0..K}: drafts the target model accepts in round r."""
    return _rng(wl.seed, 3, r).integers(0, wl.draft + 1, wl.batch).astype(np.int32)


def gdn_step_inputs(wl: Workload, t: int) -> dict:
    """Gated-DeltaNet inputs of step t (0-based), all float32.

    q, k (Bt,H,d_k): N(0,1) draws scaled to unit L2 norm (in fp64);
    v (Bt,H,d_v) ~ N(0,1); beta = sigmoid(N(0,1)); alpha = exp(-softplus(N(0,1))),
    beta and alpha shaped (Bt,H). Draw order: q, k, v, beta's normal, alpha's."""
    Bt, H, dk, dv = wl.batch, wl.nheads, wl.dstate, wl.headdim
    rng = _rng(wl.seed, 5, t)
    q = rng.standard_normal((Bt, H, dk), dtype=np.float32).astype(np.float64)
    k = rng.standard_normal((Bt, H, dk), dtype=np.float32).astype(np.float64)
    v = rng.standard_normal((Bt, H, dv), dtype=np.float32)
    zb = rng.standard_normal((Bt, H), dtype=np.float32).astype(np.float64)
    za = rng.standard_normal((Bt, H), dtype=np.float32).astype(np.float64)
    q = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True))
    k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True))
    return {
        "q": q.astype(np.float32),
        "k": k.astype(np.float32),
        "v": v,
        "beta": (1.0 / (1.0 + np.exp(-zb))).astype(np.float32),
        "alpha": np.exp(-_softplus64(za)).astype(np.float32),
    }


def kda_step_inputs(wl: Workload, t: int) -> dict:
    """Kimi-Delta-Attention inputs of step t (0-based), all float32: as
    ``gdn_step_inputs`` but the gate has one value per key channel,
    alpha = exp(-softplus(N(0,1))) shaped (Bt,H,d_k). Draw order: q, k, v,
    beta's normal, alpha's normals."""
    Bt, H, dk, dv = wl.batch, wl.nheads, wl.dstate, wl.headdim
    rng = _rng(wl.seed, 6, t)
    q = rng.standard_normal((Bt, H, dk), dtype=np.float32).astype(np.float64)
    k = rng.standard_normal((Bt, H, dk), dtype=np.float32).astype(np.float64)
    v = rng.standard_normal((Bt, H, dv), dtype=np.float32)
    zb = rng.standard_normal((Bt, H), dtype=np.float32).astype(np.float64)
    za = rng.standard_normal((Bt, H, dk), dtype=np.float32).astype(np.float64)
    q = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True))
    k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True))
    return {
        "q": q.astype(np.float32),
        "k": k.astype(np.float32),
        "v": v,
        "beta": (1.0 / (1.0 + np.exp(-zb))).astype(np.float32),
        "alpha": np.exp(-_softplus64(za)).astype(np.float32),
    }


# ---- device-side draws (torch, Philox), for long runs ---------------------------
def _device_gen(seed: int, stream: int, idx: int, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + stream) * 1_000_003 + idx)
    return g


def device_draft_inputs(wl: Workload, r: int, device) -> dict:
    """Speculative round r drawn on `device` (stream 7): x (Bt,K+1,H,P), B and
    C (Bt,K+1,G,N) ~ N(0,1) drawn as float32 and rounded to the storage dtype
    (bf16: round to nearest even), dt (Bt,K+1,H) = softplus(z - 2) with
    z ~ N(0,1), computed in float32. Draw order: x, B, C, z."""
    import torch
    g = _device_gen(wl.seed, 7, r, device)
    Bt, H, P, N, G, T = wl.batch, wl.nheads, wl.headdim, wl.dstate, wl.ngroups, wl.draft + 1
    st = torch.bfloat16 if wl.in_dtype == "bf16" else torch.float32
    out = {}
    for k, shape in (("x", (Bt, T, H, P)), ("B", (Bt, T, G, N)), ("C", (Bt, T, G, N))):
        out[k] = torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(st)
    z = torch.randn((Bt, T, H), generator=g, device=device, dtype=torch.float32)
    out["dt"] = torch.nn.functional.softplus(z - 2.0)
    return out


def device_delta_inputs(wl: Workload, t: int, device) -> dict:
    """Gated-DeltaNet (stream 8) or Kimi-Delta-Attention (stream 9) inputs of
    step t drawn on `device`, float32, with the recipe of ``gdn_step_inputs`` /
    ``kda_step_inputs`` evaluated in float32: q, k unit-L2-normalised N(0,1)
    draws, v ~ N(0,1), beta = sigmoid(N(0,1)), alpha = exp(-softplus(N(0,1)))
    (per key channel for KDA). Draw order: q, k, v, beta's normal, alpha's."""
    import torch
    kda = wl.kind == "kda"
    g = _device_gen(wl.seed, 9 if kda else 8, t, device)
    Bt, H, dk, dv = wl.batch, wl.nheads, wl.dstate, wl.headdim
    f = torch.float32
    q = torch.randn((Bt, H, dk), generator=g, device=device, dtype=f)
    k = torch.randn((Bt, H, dk), generator=g, device=device, dtype=f)
    v = torch.randn((Bt, H, dv), generator=g, device=device, dtype=f)
    zb = torch.randn((Bt, H), generator=g, device=device, dtype=f)
    za = torch.randn((Bt, H, dk) if kda else (Bt, H), generator=g, device=device, dtype=f)
    return {"q": q / q.norm(dim=-1, keepdim=True), "k": k / k.norm(dim=-1, keepdim=True), "v": v,
            "beta": torch.sigmoid(zb), "alpha": torch.exp(-torch.nn.functional.softplus(za))}
