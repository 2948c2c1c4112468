"""Integer model of the per-sequence input ring (oracle side).

ReplaySSM keeps, beside a checkpoint, a buffer of the recent inputs; the
checkpoint is rewritten only when that buffer is full (P1, section "Tenir le
journal plutôt que le solde"; P3, "Решение ReplaySSM"). Rolling back rejected
speculative tokens is a pointer operation on that buffer (P2, section "Un retour
en arrière qui devient trivial"); rejected tokens leave the buffer without
touching the checkpoint (P1, "Tenir le journal plutôt que le solde").

Readings taken where the pages are silent:
  * the buffer is a ring of R slots per sequence, addressed by (head, len):
    slot of window position j is (head + j) mod R;
  * a speculative round appends K+1 entries as tentative (n_tent = K+1);
  * rollback(n) drops the n newest entries, requires 0 <= n <= n_tent, and
    commits the rest (n_tent = 0);
  * flush(threshold) folds every committed entry of a sequence whose window
    holds at least `threshold` entries: head advances by len, len = 0.

Violations are reported, and the sequence is left unchanged.
"""
from __future__ import annotations

import numpy as np


class RingError(Exception):
    pass


class PointerModel:
    """Pointers (head, len, n_tent) of Bt sequences, each ring holding R slots."""

    def __init__(self, batch: int, capacity: int):
        self.R = int(capacity)
        self.head = np.zeros(batch, np.int64)
        self.len = np.zeros(batch, np.int64)
        self.n_tent = np.zeros(batch, np.int64)

    def slot(self, b: int, j: int) -> int:
        """Ring slot of window position j (0 = oldest) of sequence b."""
        return int((self.head[b] + j) % self.R)

    def window_slots(self, b: int) -> list:
        return [self.slot(b, j) for j in range(int(self.len[b]))]

    def append(self, b: int, n: int = 1) -> list:
        """Reserve n new window positions at the tail; return their slots."""
        if self.len[b] + n > self.R:
            raise RingError(f"ring overflow: seq {b} len {self.len[b]} + {n} > R={self.R}")
        slots = [self.slot(b, int(self.len[b]) + i) for i in range(n)]
        self.len[b] += n
        return slots

    def mark_tentative(self, b: int, n: int) -> None:
        self.n_tent[b] = n

    def rollback(self, b: int, n_drop: int) -> None:
        if not (0 <= n_drop <= self.n_tent[b]):
            raise RingError(f"rollback {n_drop} outside [0, {self.n_tent[b]}] for seq {b}")
        self.len[b] -= n_drop
        self.n_tent[b] = 0

    def flush(self, b: int, threshold: int) -> bool:
        """Fold-and-advance if the window holds >= threshold entries."""
        if self.n_tent[b] != 0:
            raise RingError(f"flush with {self.n_tent[b]} uncommitted entries on seq {b}")
        if self.len[b] >= threshold:
            self.head[b] = (self.head[b] + self.len[b]) % self.R
            self.len[b] = 0
            return True
        return False

    def as_array(self) -> np.ndarray:
        """(Bt, 3) int64: head, len, n_tent."""
        return np.stack([self.head, self.len, self.n_tent], axis=1)
