"""bf16 rounding for the dual-precision emulator (oracle side).

The low-precision read copy is a bf16 image of the fp32 master checkpoint (P2,
section "Deux précisions pour le prix d'une"; P4, the accuracy row of the table
in "Co się zmieniło?"). The pages do not name a rounding mode; the reading taken
is round to nearest, ties to even (IEEE default).
"""
from __future__ import annotations

import numpy as np


def round_f32(a) -> np.ndarray:
    """fp64 -> nearest fp32 (ties to even), returned as float64."""
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_bf16_from_f32(a) -> np.ndarray:
    """Round fp32 values to bf16 (8 significant bits, ties to even); float64 out.

    bf16 keeps the top 16 bits of an fp32 word. Rounding adds half of the
    dropped range, minus one when the kept part is even so that an exact tie
    goes to the even neighbour, then truncates."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> 16) & 1
    u = ((u + 0x7FFF + keep_lsb) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def round_bf16(a) -> np.ndarray:
    """fp64 -> fp32 -> bf16, both steps to nearest even (the device holds an
    fp32 master and rounds that to bf16)."""
    return round_bf16_from_f32(np.asarray(a, dtype=np.float64).astype(np.float32))
