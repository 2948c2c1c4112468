"""Mamba-2 decode in fp64: eager recurrence, unrolled form, replay model.

The eager step (P1, section "La fiche qu'on réécrit à chaque token"): read the
previous state, apply a decay factor and a rank-1 update, compute the output,
write the whole state back. The pages give no formula; the reading taken is the
Mamba-2 scalar-decay form, per head h of sequence b:

    a_t = exp(dt_t * A_h)
    S_t = a_t * S_{t-1} + dt_t * outer(x_t, B_t)        S is P x N
    y_t = S_t @ C_t                                      y is length P

B_t and C_t belong to the group g(h) = h // (H/G) of the head. The output is
read from the *updated* state: the step order on P1, and P5's ``ssm_step`` (in
"Comment fonctionnent réellement les modèles à espace d'états") computes y from
the new hidden state. No D skip, gate or norm: none of them touches the state.

Tokens are indexed 0..T-1 here; S0 is the state before token 0.
"""
from __future__ import annotations

import numpy as np

from . import lowp
from .ring import PointerModel, RingError


def group_index(H: int, G: int) -> np.ndarray:
    """g(h) = h // (H/G) for every head: consecutive blocks of H/G heads share a group."""
    if G <= 0 or H % G:
        raise ValueError(f"H={H} must be a multiple of G={G}")
    return np.arange(H) // (H // G)


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# The reference result: the eager recurrence.
# --------------------------------------------------------------------------
def eager_step(S, A, x, B, C, dt):
    """One eager step for every (sequence, head).

    S (Bt,H,P,N), A (H,), x (Bt,H,P), B and C (Bt,G,N), dt (Bt,H).
    Returns (S_new, y) with y (Bt,H,P), all float64."""
    S, A, x, B, C, dt = map(_f64, (S, A, x, B, C, dt))
    g = group_index(S.shape[1], B.shape[1])
    Bh = B[:, g, :]
    Ch = C[:, g, :]
    a = np.exp(dt * A[None, :])
    S_new = (a[:, :, None, None] * S
             + dt[:, :, None, None] * x[:, :, :, None] * Bh[:, :, None, :])
    y = np.matmul(S_new, Ch[..., None])[..., 0]
    return S_new, y


def eager_scan(S0, A, xs, Bs, Cs, dts, keep=()):
    """Run T eager steps. xs (T,Bt,H,P), Bs/Cs (T,Bt,G,N), dts (T,Bt,H).

    Returns (ys (T,Bt,H,P), S_T, {n: state after n tokens for n in keep})."""
    S = _f64(S0).copy()
    T = len(xs)
    ys = np.zeros((T,) + np.shape(xs)[1:], np.float64)
    kept = {0: S.copy()} if 0 in keep else {}
    for t in range(T):
        S, ys[t] = eager_step(S, A, xs[t], Bs[t], Cs[t], dts[t])
        if t + 1 in keep:
            kept[t + 1] = S.copy()
    return ys, S, kept


def eager_scan_bf16_state(S0, A, xs, Bs, Cs, dts):
    """The eager recurrence with its state *stored* in bf16 (a quantised state
    rewritten at every token, P1 "Trois ennuis nés de la même fusion": each
    rewrite adds a rounding). Each step starts from the stored bf16 values, is
    computed exactly, gives y from that unrounded new state, and stores the new
    state rounded to nearest (via fp32, ties to even). The initial state is
    stored the same way. Returns (ys (T,Bt,H,P), stored S_T)."""
    S = lowp.round_bf16(S0)
    T = len(xs)
    ys = np.zeros((T,) + np.shape(xs)[1:], np.float64)
    for t in range(T):
        S_new, ys[t] = eager_step(S, A, xs[t], Bs[t], Cs[t], dts[t])
        S = lowp.round_bf16(S_new)
    return ys, S


# --------------------------------------------------------------------------
# The recurrence unrolled: closed form and semiseparable matrix.
# --------------------------------------------------------------------------
def semiseparable_matrix(A_h, B_seq, C_seq, dt_seq) -> np.ndarray:
    """M (T,T) of one (sequence, head): Y = M @ X + (initial-state term).

    M[t, j] = exp(sum_{i=j+1..t} dt_i*A_h) * dt_j * (C_t . B_j) for j <= t, else 0.
    This is the recurrence unrolled, which is what ReplaySSM does (P2, section
    "L'astuce du checkpoint et du tampon"); the same lower-triangular matrix is
    the structured-SSM / linear-attention duality P5 mentions (section "De Mamba
    à Mamba-3"). B_seq, C_seq (T,N), dt_seq (T,)."""
    A_h = float(A_h)
    B_seq, C_seq, dt_seq = map(_f64, (B_seq, C_seq, dt_seq))
    T = len(dt_seq)
    ell = dt_seq * A_h
    M = np.zeros((T, T))
    for t in range(T):
        for j in range(t + 1):
            M[t, j] = np.exp(np.sum(ell[j + 1:t + 1])) * dt_seq[j] * np.dot(C_seq[t], B_seq[j])
    return M


def unrolled_outputs(S0, A, xs, Bs, Cs, dts) -> np.ndarray:
    """Closed form of every output (no state is formed):

    y_t = exp(sum_{i<=t} l_i) * S0 @ C_t + sum_{j<=t} M[t,j] * x_j,  l_i = dt_i*A_h.
    Dense O(T^2) per (sequence, head); for small T only."""
    S0, A, xs, Bs, Cs, dts = map(_f64, (S0, A, xs, Bs, Cs, dts))
    T, Bt, H, P = xs.shape
    g = group_index(H, Bs.shape[2])
    ys = np.zeros((T, Bt, H, P))
    for b in range(Bt):
        for h in range(H):
            Bq, Cq, dq = Bs[:, b, g[h]], Cs[:, b, g[h]], dts[:, b, h]
            M = semiseparable_matrix(A[h], Bq, Cq, dq)
            d0 = np.array([np.exp(np.sum(dq[:t + 1] * A[h])) for t in range(T)])
            ys[:, b, h] = M @ xs[:, b, h] + d0[:, None] * (Cq @ S0[b, h].T)
    return ys


# --------------------------------------------------------------------------
# The method: checkpoint + ring of recent inputs, outputs by replay.
# --------------------------------------------------------------------------
def suffix_decay(ell: np.ndarray):
    """For window entries 0..n-1 (oldest first) with log-decays ell (n,H):

    lam[j] = sum_{i=j+1..n-1} ell[i]  (decay from entry j to the newest entry),
    total  = sum_{i=0..n-1} ell[i]    (decay of the checkpoint to the newest).
    Summed from the newest entry backwards: suffix sums, never differences of
    prefix sums, which cancel once the window's total decay is large."""
    n = ell.shape[0]
    lam = np.zeros_like(ell)
    acc = np.zeros(ell.shape[1:])
    for j in range(n - 1, -1, -1):
        lam[j] = acc
        acc = acc + ell[j]
    return lam, acc


class ReplayModel:
    """fp64 model of ReplaySSM's state storage for Bt sequences.

    The state is a checkpoint plus a buffer of recent inputs; the output is
    computed from both without touching a full state, and the checkpoint is
    rewritten only when the buffer is full (P1, "Tenir le journal plutôt que le
    solde"; P2, "L'astuce du checkpoint et du tampon"; P3, "Решение ReplaySSM";
    P4's table, row "Ruch pamięci stanu": checkpoint read every step, written
    only on flush).

    Each ring entry holds (x_t, B_t, dt_t, l_t = dt_t*A) — C_t is needed only at
    step t and is not kept. The pages list the buffer's contents only loosely
    (P3, "Решение ReplaySSM", names the recent inputs (v_t, k_t)).

    Output of the newest window entry t, window entries j = 0..t:
        y_t = exp(Lam_c) * S_c @ C_t + sum_j exp(lam_j) * dt_j * (B_j . C_t) * x_j
    Flush (fold the window into the checkpoint):
        S_c <- exp(Lam_c) * S_c + sum_j exp(lam_j) * dt_j * outer(x_j, B_j)

    read_copy="bf16" is the dual-precision mode (P2, "Deux précisions pour le
    prix d'une"): outputs read a bf16 copy of the checkpoint, refreshed from the
    high-precision master after each fold; the fold itself only ever reads the
    master, so the copy's rounding never feeds back.

    read_copy="bf16_state" is the single shared low-precision checkpoint that
    P2 compares the dual mode with: the checkpoint itself is stored in bf16
    (rounded at init and after every fold), outputs and folds start from those
    stored values. It rounds once per fold instead of once per token (P1, "Tenir
    le journal plutôt que le solde": the quantised state is rewritten only at
    spaced intervals).
    """

    def __init__(self, S0, A, ngroups: int, capacity: int, read_copy: str = "none"):
        S0 = _f64(S0)
        Bt, H, P, N = S0.shape
        self.Bt, self.H, self.P, self.N, self.G = Bt, H, P, N, ngroups
        self.g = group_index(H, ngroups)
        self.A = _f64(A)
        self.R = capacity
        if read_copy not in ("none", "bf16", "bf16_state"):
            raise ValueError(read_copy)
        self.ckpt = lowp.round_bf16(S0) if read_copy == "bf16_state" else S0.copy()
        self.read_copy = read_copy
        self.copy = lowp.round_bf16(self.ckpt) if read_copy == "bf16" else None
        self.ptr = PointerModel(Bt, capacity)
        self.ring_x = np.zeros((Bt, capacity, H, P))
        self.ring_B = np.zeros((Bt, capacity, ngroups, N))
        self.ring_dt = np.zeros((Bt, capacity, H))
        self.ring_ell = np.zeros((Bt, capacity, H))

    # -- ring access ------------------------------------------------------
    def _put(self, b, slot, x, B, dt):
        self.ring_x[b, slot] = x
        self.ring_B[b, slot] = B
        self.ring_dt[b, slot] = dt
        self.ring_ell[b, slot] = dt * self.A

    def _window(self, b, n):
        slots = [self.ptr.slot(b, j) for j in range(n)]
        return (self.ring_x[b, slots], self.ring_B[b, slots][:, self.g],
                self.ring_dt[b, slots], self.ring_ell[b, slots])

    def _output(self, b, C_t, n):
        """Output for the n-th window entry of sequence b (entries 0..n-1)."""
        Ch = _f64(C_t)[self.g]                                   # (H,N)
        x, Bh, dt, ell = self._window(b, n)
        lam, total = suffix_decay(ell)
        base = self.copy[b] if self.copy is not None else self.ckpt[b]
        y = np.exp(total)[:, None] * np.matmul(base, Ch[..., None])[..., 0]
        for j in range(n):
            coef = np.exp(lam[j]) * dt[j] * np.sum(Bh[j] * Ch, axis=-1)
            y = y + coef[:, None] * x[j]
        return y

    def implied_state(self, b):
        """The state checkpoint + window stand for (a fold, without storing it)."""
        n = int(self.ptr.len[b])
        x, Bh, dt, ell = self._window(b, n)
        lam, total = suffix_decay(ell)
        S = np.exp(total)[:, None, None] * self.ckpt[b]
        for j in range(n):
            c = np.exp(lam[j]) * dt[j]
            S = S + c[:, None, None] * x[j][:, :, None] * Bh[j][:, None, :]
        return S

    # -- the calls ----------------------------------------------------------
    def decode(self, x, B, C, dt):
        """Plain decode step for all sequences: append, then replay the output."""
        x, B, C, dt = map(_f64, (x, B, C, dt))
        y = np.zeros((self.Bt, self.H, self.P))
        for b in range(self.Bt):
            if self.ptr.n_tent[b]:
                raise RingError("decode while a verify round is uncommitted")
            slot = self.ptr.append(b, 1)[0]
            self._put(b, slot, x[b], B[b], dt[b])
            y[b] = self._output(b, C[b], int(self.ptr.len[b]))
        return y

    def flush(self, threshold):
        """Fold every sequence whose window holds >= threshold entries; the
        threshold may be one value or one per sequence (values below 1 act as 1)."""
        folded = []
        for b in range(self.Bt):
            if self.ptr.n_tent[b]:
                raise RingError("flush while a verify round is uncommitted")
            th = max(1, int(threshold[b] if np.ndim(threshold) else threshold))
            if self.ptr.len[b] >= th:
                self.ckpt[b] = self.implied_state(b)
                if self.read_copy == "bf16_state":
                    self.ckpt[b] = lowp.round_bf16(self.ckpt[b])
                self.ptr.flush(b, th)
                if self.copy is not None:
                    self.copy[b] = lowp.round_bf16(self.ckpt[b])
                folded.append(b)
        return folded

    def verify(self, xs, Bs, Cs, dts):
        """Append K+1 tentative tokens per sequence and return their K+1 outputs,
        each causal over the committed window and the earlier drafts.
        xs (Bt,K+1,H,P), Bs/Cs (Bt,K+1,G,N), dts (Bt,K+1,H)."""
        xs, Bs, Cs, dts = map(_f64, (xs, Bs, Cs, dts))
        Kp1 = xs.shape[1]
        y = np.zeros((self.Bt, Kp1, self.H, self.P))
        for b in range(self.Bt):
            if self.ptr.n_tent[b]:
                raise RingError("verify while a verify round is uncommitted")
            n0 = int(self.ptr.len[b])
            slots = self.ptr.append(b, Kp1)
            for i, s in enumerate(slots):
                self._put(b, s, xs[b, i], Bs[b, i], dts[b, i])
            self.ptr.mark_tentative(b, Kp1)
            for i in range(Kp1):
                y[b, i] = self._output(b, Cs[b, i], n0 + i + 1)
        return y

    def rollback(self, n_drop):
        """Drop the n_drop[b] newest tentative entries; commit the rest."""
        for b in range(self.Bt):
            self.ptr.rollback(b, int(n_drop[b]))


# --------------------------------------------------------------------------
# Speculative decoding, by its plain definition.
# --------------------------------------------------------------------------
def speculative_reference(S0, A, rounds, n_acc):
    """The eager recurrence run over the committed stream.

    Each round feeds K+1 tokens (the last sampled token, then K drafts); the
    target keeps the first n_acc+1 of them. The round's K+1 outputs are those of
    the eager recurrence on (committed prefix + the round's tokens); the next
    round starts from the state after the kept tokens only.

    rounds: list of dicts with x (Bt,K+1,H,P), B, C (Bt,K+1,G,N), dt (Bt,K+1,H);
    n_acc: list of (Bt,) ints. Returns (list of y (Bt,K+1,H,P), final state)."""
    S = _f64(S0).copy()
    outs = []
    for r, inp in enumerate(rounds):
        Kp1 = inp["x"].shape[1]
        states = []
        ys = np.zeros((S.shape[0], Kp1, S.shape[1], S.shape[2]))
        S_run = S
        for i in range(Kp1):
            S_run, ys[:, i] = eager_step(S_run, A, inp["x"][:, i], inp["B"][:, i],
                                         inp["C"][:, i], inp["dt"][:, i])
            states.append(S_run)
        keep = np.asarray(n_acc[r]) + 1
        S = np.stack([states[keep[b] - 1][b] for b in range(S.shape[0])])
        outs.append(ys)
    return outs, S
