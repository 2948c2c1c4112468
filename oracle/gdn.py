"""Gated DeltaNet decode in fp64: the gated delta rule and its replay model.

P1 ("La fiche qu'on réécrit à chaque token") says GDN and KDA add a delta-rule
correction but write their updates in the same form as Mamba-2; P2 ("Des
chiffres qui parlent d'eux-mêmes") says the method runs for Mamba-2 and Gated
DeltaNet. The pages give no GDN formula. The reading taken is the standard gated
delta rule with a scalar gate per head; S is d_v x d_k:

    S_t = alpha_t * S_{t-1} @ (I - beta_t * k_t k_t^T) + beta_t * v_t k_t^T
    o_t = S_t @ q_t

Rearranged, with u_t = beta_t * (v_t - alpha_t * S_{t-1} @ k_t):

    S_t = alpha_t * S_{t-1} + outer(u_t, k_t)

which is the Mamba-2 step with x -> u, B -> k, C -> q, dt -> 1 and decay
log(alpha). The replay model keeps (k_t, u_t, log alpha_t) in the ring; u_t needs
S_{t-1} @ k_t, which replay forms from the checkpoint and the window without
materialising S_{t-1}. No q/k scale factor (inputs arrive L2-normalised).
"""
from __future__ import annotations

import numpy as np

from .ring import PointerModel, RingError
from .mamba2 import suffix_decay


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def eager_step(S, q, k, v, beta, alpha):
    """Matrix form of the gated delta rule. S (Bt,H,dv,dk); q,k (Bt,H,dk);
    v (Bt,H,dv); beta, alpha (Bt,H). Returns (S_new, o (Bt,H,dv))."""
    S, q, k, v, beta, alpha = map(_f64, (S, q, k, v, beta, alpha))
    dk = k.shape[-1]
    proj = np.eye(dk) - beta[..., None, None] * k[..., :, None] * k[..., None, :]
    S_new = (alpha[..., None, None] * np.matmul(S, proj)
             + beta[..., None, None] * v[..., :, None] * k[..., None, :])
    o = np.matmul(S_new, q[..., None])[..., 0]
    return S_new, o


def eager_scan(S0, steps):
    """steps: list of dicts (q, k, v, beta, alpha). Returns (o (T,Bt,H,dv), S_T)."""
    S = _f64(S0).copy()
    outs = []
    for inp in steps:
        S, o = eager_step(S, inp["q"], inp["k"], inp["v"], inp["beta"], inp["alpha"])
        outs.append(o)
    return np.stack(outs), S


class GDNReplayModel:
    """Checkpoint + ring of (k, u, log alpha) for gated DeltaNet decode."""

    def __init__(self, S0, capacity: int):
        S0 = _f64(S0)
        Bt, H, dv, dk = S0.shape
        self.Bt, self.H, self.dv, self.dk = Bt, H, dv, dk
        self.ckpt = S0.copy()
        self.ptr = PointerModel(Bt, capacity)
        self.ring_k = np.zeros((Bt, capacity, H, dk))
        self.ring_u = np.zeros((Bt, capacity, H, dv))
        self.ring_ell = np.zeros((Bt, capacity, H))

    def _window(self, b, n):
        slots = [self.ptr.slot(b, j) for j in range(n)]
        return self.ring_k[b, slots], self.ring_u[b, slots], self.ring_ell[b, slots]

    def _apply(self, b, vec, n):
        """(state after window entries 0..n-1) @ vec, per head; vec (H,dk)."""
        k, u, ell = self._window(b, n)
        lam, total = suffix_decay(ell) if n else (np.zeros((0, self.H)), np.zeros(self.H))
        out = np.exp(total)[:, None] * np.matmul(self.ckpt[b], vec[..., None])[..., 0]
        for j in range(n):
            out = out + (np.exp(lam[j]) * np.sum(k[j] * vec, axis=-1))[:, None] * u[j]
        return out

    def decode(self, q, k, v, beta, alpha):
        q, k, v, beta, alpha = map(_f64, (q, k, v, beta, alpha))
        o = np.zeros((self.Bt, self.H, self.dv))
        for b in range(self.Bt):
            if self.ptr.n_tent[b]:
                raise RingError("decode while a verify round is uncommitted")
            n = int(self.ptr.len[b])
            Sk = self._apply(b, k[b], n)                     # S_{t-1} @ k_t
            u = beta[b][:, None] * (v[b] - alpha[b][:, None] * Sk)
            slot = self.ptr.append(b, 1)[0]
            self.ring_k[b, slot] = k[b]
            self.ring_u[b, slot] = u
            self.ring_ell[b, slot] = np.log(alpha[b])
            o[b] = self._apply(b, q[b], n + 1)
        return o

    def implied_state(self, b):
        n = int(self.ptr.len[b])
        k, u, ell = self._window(b, n)
        lam, total = suffix_decay(ell) if n else (np.zeros((0, self.H)), np.zeros(self.H))
        S = np.exp(total)[:, None, None] * self.ckpt[b]
        for j in range(n):
            S = S + np.exp(lam[j])[:, None, None] * u[j][:, :, None] * k[j][:, None, :]
        return S

    def flush(self, threshold: int):
        folded = []
        for b in range(self.Bt):
            if self.ptr.len[b] >= threshold:
                self.ckpt[b] = self.implied_state(b)
                self.ptr.flush(b, threshold)
                folded.append(b)
        return folded
