"""Kimi Delta Attention (KDA) decode in fp64: the per-channel gated delta rule
and its replay model.

P1 ("Des couches rapides sur le papier") names KDA as the third SSM layer type of
hybrid models, and ("La fiche qu'on réécrit à chaque token") says GDN and KDA add
a delta-rule correction to an update of the same form. The pages give no KDA
formula. The reading taken is the gated delta rule with a fine-grained gate: one
decay per key channel instead of one per head. With S of size d_v x d_k, per head:

    S_t = S_{t-1} @ Diag(alpha_t) @ (I - beta_t * k_t k_t^T) + beta_t * v_t k_t^T
    o_t = S_t @ q_t                                  alpha_t in (0,1)^{d_k}

A scalar gate (every channel equal) gives the gated DeltaNet rule of ``gdn``.

Rearranged, with S' = S_{t-1} Diag(alpha_t) and u_t = beta_t (v_t - S' k_t):

    S_t = S' + outer(u_t, k_t),      o_t = S' q_t + (k_t . q_t) u_t

so the state after window entries 0..t is the checkpoint with every key channel
n decayed by exp(Lam[n]) plus, per entry j, outer(u_j, k_j * exp(lam_j)), where
lam_j[n] sums log alpha_i[n] over the entries i after j and Lam[n] over all of
them: per-channel suffix sums instead of the scalar ones of Mamba-2 and GDN. The
replay model keeps (k_t, u_t, log alpha_t) in the ring.
"""
from __future__ import annotations

import numpy as np

from .ring import PointerModel, RingError


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def eager_step(S, q, k, v, beta, alpha):
    """Matrix form of the per-channel gated delta rule. S (Bt,H,dv,dk); q, k,
    alpha (Bt,H,dk); v (Bt,H,dv); beta (Bt,H). Returns (S_new, o (Bt,H,dv))."""
    S, q, k, v, beta, alpha = map(_f64, (S, q, k, v, beta, alpha))
    dk = k.shape[-1]
    gate = alpha[..., :, None] * np.eye(dk)                       # Diag(alpha)
    proj = np.eye(dk) - beta[..., None, None] * k[..., :, None] * k[..., None, :]
    S_new = (np.matmul(np.matmul(S, gate), proj)
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


def channel_suffix(g):
    """g (n,H,dk): per-entry per-channel log-decays, oldest first. Returns
    lam (n,H,dk) with lam[j] = sum_{i>j} g[i], and total = sum_i g[i], summed
    from the newest entry backwards (never differences of prefix sums)."""
    n = g.shape[0]
    lam = np.zeros_like(g)
    acc = np.zeros(g.shape[1:])
    for j in range(n - 1, -1, -1):
        lam[j] = acc
        acc = acc + g[j]
    return lam, acc


class KDAReplayModel:
    """Checkpoint + ring of (k, u, log alpha) rows for KDA decode."""

    def __init__(self, S0, capacity: int):
        S0 = _f64(S0)
        Bt, H, dv, dk = S0.shape
        self.Bt, self.H, self.dv, self.dk = Bt, H, dv, dk
        self.ckpt = S0.copy()
        self.ptr = PointerModel(Bt, capacity)
        self.ring_k = np.zeros((Bt, capacity, H, dk))
        self.ring_u = np.zeros((Bt, capacity, H, dv))
        self.ring_g = np.zeros((Bt, capacity, H, dk))

    def _window(self, b, n):
        slots = [self.ptr.slot(b, j) for j in range(n)]
        return self.ring_k[b, slots], self.ring_u[b, slots], self.ring_g[b, slots]

    def _apply(self, b, vec, n, g_next=None):
        """(state after window entries 0..n-1, then decayed by g_next if given) @ vec;
        vec (H,dk)."""
        k, u, g = self._window(b, n)
        if g_next is not None:
            g = np.concatenate([g, g_next[None]], axis=0)
        lam, total = channel_suffix(g)
        out = np.matmul(self.ckpt[b], (np.exp(total) * vec)[..., None])[..., 0]
        for j in range(n):
            w = np.sum(k[j] * np.exp(lam[j]) * vec, axis=-1)      # (H,)
            out = out + w[:, None] * u[j]
        return out

    def decode(self, q, k, v, beta, alpha):
        q, k, v, beta, alpha = map(_f64, (q, k, v, beta, alpha))
        o = np.zeros((self.Bt, self.H, self.dv))
        for b in range(self.Bt):
            if self.ptr.n_tent[b]:
                raise RingError("decode while a verify round is uncommitted")
            n = int(self.ptr.len[b])
            g_t = np.log(alpha[b])
            Sk = self._apply(b, k[b], n, g_next=g_t)            # S_{t-1} Diag(alpha_t) k_t
            Sq = self._apply(b, q[b], n, g_next=g_t)            # S_{t-1} Diag(alpha_t) q_t
            u = beta[b][:, None] * (v[b] - Sk)
            slot = self.ptr.append(b, 1)[0]
            self.ring_k[b, slot] = k[b]
            self.ring_u[b, slot] = u
            self.ring_g[b, slot] = g_t
            o[b] = Sq + np.sum(k[b] * q[b], axis=-1)[:, None] * u
        return o

    def implied_state(self, b):
        n = int(self.ptr.len[b])
        k, u, g = self._window(b, n)
        lam, total = channel_suffix(g)
        S = self.ckpt[b] * np.exp(total)[:, None, :]
        for j in range(n):
            S = S + u[j][:, :, None] * (k[j] * np.exp(lam[j]))[:, None, :]
        return S

    def flush(self, threshold: int):
        folded = []
        for b in range(self.Bt):
            if self.ptr.len[b] >= threshold:
                self.ckpt[b] = self.implied_state(b)
                self.ptr.flush(b, threshold)
                folded.append(b)
        return folded
