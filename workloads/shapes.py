"""Named decode workloads (shapes, dtypes, seeds).

Notation: batch Bt, heads H, head dimension P, state dimension N, groups G
(B and C are shared by the H/G heads of a group), flush window W, ring capacity
R (entries per sequence and head), largest draft K_max.

The state of one layer for one sequence at 128 heads x P=64 x N=128 in fp32 is
4 MiB, the size the pages quote for Nemotron-3-Super at batch 256 (P1, section
"La fiche qu'on réécrit à chaque token"); batch 512 is the speculative-decoding
batch of P4's table ("Co się zmieniło?").
"""
from __future__ import annotations

import dataclasses


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str             # "mamba2", "gdn" or "kda"
    batch: int            # Bt
    nheads: int           # H
    headdim: int          # P   (GDN: d_v)
    dstate: int           # N   (GDN: d_k)
    ngroups: int          # G
    window: int           # W
    capacity: int         # R
    max_draft: int        # K_max
    steps: int            # plain decode tokens (T)
    in_dtype: str         # "f32" or "bf16": storage type of x, B, C
    read_copy: str        # "none" or "bf16"
    seed: int
    draft: int = 0        # K for speculative rounds
    rounds: int = 0       # speculative rounds
    s0: str = "zeros"     # "zeros" or "normal"
    a_scale: float = 1.0  # A_h = -a_scale * exp(U(0,1)); < 1 gives long-memory heads

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def state_bytes_per_seq(self) -> int:
        return self.nheads * self.headdim * self.dstate * 4


def _mk() -> dict:
    w = {}
    w["tiny_b2_h4_p16_n16_w8"] = Workload(
        "tiny_b2_h4_p16_n16_w8", "mamba2", 2, 4, 16, 16, 4, 8, 8, 0, 64,
        "f32", "none", 1000)
    w["mamba2_b256_h128_p64_n128_w16"] = Workload(
        "mamba2_b256_h128_p64_n128_w16", "mamba2", 256, 128, 64, 128, 128, 16,
        16, 0, 256, "bf16", "none", 1001)
    for win in (8, 16, 32):
        n = f"mamba2_dual_b256_h128_p64_n128_w{win}"
        w[n] = Workload(n, "mamba2", 256, 128, 64, 128, 128, win, win, 0, 1024,
                        "bf16", "bf16", 1002)
    # Long-memory heads (decay per token ~0.997 instead of ~0.8), same shapes:
    # the regime where per-token rounding of a stored state accumulates.
    for win in (8, 16, 32):
        n = f"mamba2_slowdecay_b256_h128_p64_n128_w{win}"
        w[n] = Workload(n, "mamba2", 256, 128, 64, 128, 128, win, win, 0, 1024,
                        "bf16", "bf16", 1005, a_scale=0.01)
    w["mamba2_spec_b512_h128_p64_n128_w16_k4"] = Workload(
        "mamba2_spec_b512_h128_p64_n128_w16_k4", "mamba2", 512, 128, 64, 128,
        128, 16, 20, 4, 0, "bf16", "none", 1003, draft=4, rounds=200)
    w["gdn_b256_h32_d128_w16"] = Workload(
        "gdn_b256_h32_d128_w16", "gdn", 256, 32, 128, 128, 32, 16, 16, 0, 256,
        "f32", "none", 1004)
    # Kimi Delta Attention at the gated-DeltaNet shape (per-channel gates).
    w["kda_b256_h32_d128_w16"] = Workload(
        "kda_b256_h32_d128_w16", "kda", 256, 32, 128, 128, 32, 16, 16, 0, 256,
        "f32", "none", 1006)
    return w


WORKLOADS = _mk()


def get(name: str) -> Workload:
    return WORKLOADS[name]
