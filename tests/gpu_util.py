"""Helpers for the GPU tests: device tensors from the seeded generators, and
gathers of sampled (sequence, head) pairs for the oracle.

The HIP path is always called through the C ABI binding; the oracle only ever
sees the generators' exact input values, never anything the GPU produced."""
from __future__ import annotations

import sys

import numpy as np
import torch

from recurrent_state_storage_amd import rss

DEV = torch.device("cuda:0")


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def cfg_of(wl, **kw):
    d = dict(batch=wl.batch, nheads=wl.nheads, headdim=wl.headdim, dstate=wl.dstate,
             ngroups=wl.ngroups, window=wl.window, capacity=wl.capacity, max_draft=wl.max_draft,
             in_dtype=rss.RSS_DTYPE_BF16 if wl.in_dtype == "bf16" else rss.RSS_DTYPE_F32,
             read_copy={"none": rss.RSS_COPY_NONE, "bf16": rss.RSS_COPY_BF16,
                        "bf16_state": rss.RSS_STATE_BF16}[wl.read_copy],
             kind={"mamba2": rss.RSS_KIND_MAMBA2, "gdn": rss.RSS_KIND_GDN,
                   "kda": rss.RSS_KIND_KDA}[wl.kind])
    d.update(kw)
    return rss.rss_config(**d)


def dev_inputs(s: dict, in_dtype: str) -> dict:
    """Generator outputs -> device tensors with the exact same bits."""
    out = {}
    for k in ("x", "B", "C"):
        if in_dtype == "bf16":
            bits = np.ascontiguousarray(s[k + "_bits"]).view(np.int16)
            out[k] = torch.from_numpy(bits).view(torch.bfloat16).to(DEV)
        else:
            out[k] = torch.from_numpy(np.ascontiguousarray(s[k])).to(DEV)
    out["dt"] = torch.from_numpy(np.ascontiguousarray(s["dt"])).to(DEV)
    return out


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    n = np.linalg.norm(ref.ravel())
    d = np.linalg.norm((got - ref).ravel())
    return float(d / n) if n > 0 else float(d)


class PairGather:
    """Sampled (b, h) pairs laid out for the oracle as one sequence with one
    head (and one group) per pair, so any pair set runs as a single batch."""

    def __init__(self, wl, pairs):
        self.pairs = list(pairs)
        self.b = np.array([p[0] for p in self.pairs])
        self.h = np.array([p[1] for p in self.pairs])
        self.g = self.h // (wl.nheads // wl.ngroups)

    def A(self, A):
        return np.asarray(A)[self.h]

    def state(self, S):          # (Bt,H,P,N) -> (1, n, P, N)
        return np.asarray(S)[self.b, self.h][None]

    def step(self, s: dict) -> dict:   # per-step inputs (Bt,...) -> (1, n, ...)
        return {"x": s["x"][self.b, self.h][None], "B": s["B"][self.b, self.g][None],
                "C": s["C"][self.b, self.g][None], "dt": s["dt"][self.b, self.h][None]}

    def draft(self, d: dict) -> dict:  # round inputs (Bt,K+1,...) -> (1, K+1, n, ...)
        return {"x": d["x"][self.b, :, self.h].transpose(1, 0, 2)[None],
                "B": d["B"][self.b, :, self.g].transpose(1, 0, 2)[None],
                "C": d["C"][self.b, :, self.g].transpose(1, 0, 2)[None],
                "dt": d["dt"][self.b, :, self.h].T[None]}

    def out(self, y) -> np.ndarray:    # device (Bt,H,P) -> (1, n, P)
        return y[torch.as_tensor(self.b, device=y.device), torch.as_tensor(self.h, device=y.device)] \
            .double().cpu().numpy()[None]


def sample_pairs(wl, n, seed):
    rng = np.random.default_rng(seed)
    bs = rng.integers(0, wl.batch, n)
    hs = rng.integers(0, wl.nheads, n)
    pairs = {(0, 0), (wl.batch - 1, wl.nheads - 1)}
    pairs.update(zip(bs.tolist(), hs.tolist()))
    return sorted(pairs)
