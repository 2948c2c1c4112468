"""Pins for the oracle: checks that tie it to facts other than itself.

Each pin takes the oracle function(s) under test as arguments and returns the
worst error it sees, so ``test_oracle_pins`` can run it on the real oracle and
``test_oracle_mutations`` on planted mistakes (which must fail at least one).

What fixes each value:
  * one and two steps from S0 = 0 have short closed forms (dt*(B.C)*x, and the
    same plus the decayed first token);
  * P = N = 1 with constant a and b = dt*x*B is a geometric series;
  * A = 0 (no decay) is unnormalised causal linear attention, a dense lower-
    triangular matmul (the running key-value sum of P5's linear-attention
    example, "Attention linéaire et convergence avec les SSM", without its
    normaliser);
  * with A = 0 and dyadic inputs every operation is exact, so the fp64 result
    must equal exact rational arithmetic bit for bit;
  * a hand-worked example (tests/golden/two_tokens_dyadic.txt);
  * the unrolled closed form (a different formula, no state);
  * a 50-digit mpmath evaluation bounds the fp64 rounding.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rel_err(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    d = np.linalg.norm((a - b).ravel())
    n = np.linalg.norm(b.ravel())
    return float(d / n) if n > 0 else float(d)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _dt(rng, *shape):
    return np.log1p(np.exp(rng.standard_normal(shape) - 2.0))


def _A(rng, H):
    return -np.exp(rng.random(H))


def _heads_of(H, G):
    return np.arange(H) // (H // G)


def pin_one_step(step, seed=1) -> float:
    """From S0 = 0 one step gives y = dt * (B.C) * x (B, C of the head's group)."""
    rng = np.random.default_rng(seed)
    Bt, H, G, P, N = 2, 4, 2, 3, 5
    x, B, C = _rand(rng, Bt, H, P), _rand(rng, Bt, G, N), _rand(rng, Bt, G, N)
    dt, A = _dt(rng, Bt, H), _A(rng, H)
    _, y = step(np.zeros((Bt, H, P, N)), A, x, B, C, dt)
    g = _heads_of(H, G)
    want = np.zeros((Bt, H, P))
    for b in range(Bt):
        for h in range(H):
            want[b, h] = dt[b, h] * np.dot(B[b, g[h]], C[b, g[h]]) * x[b, h]
    return rel_err(y, want)


def pin_two_steps(step, seed=2) -> float:
    """y_2 = dt_2 (B_2.C_2) x_2 + exp(dt_2 A) dt_1 (B_1.C_2) x_1 from S0 = 0."""
    rng = np.random.default_rng(seed)
    Bt, H, G, P, N = 2, 4, 2, 3, 5
    xs, Bs, Cs = _rand(rng, 2, Bt, H, P), _rand(rng, 2, Bt, G, N), _rand(rng, 2, Bt, G, N)
    dts, A = _dt(rng, 2, Bt, H), _A(rng, H)
    S, _ = step(np.zeros((Bt, H, P, N)), A, xs[0], Bs[0], Cs[0], dts[0])
    _, y2 = step(S, A, xs[1], Bs[1], Cs[1], dts[1])
    g = _heads_of(H, G)
    want = np.zeros((Bt, H, P))
    for b in range(Bt):
        for h in range(H):
            B1, B2, C2 = Bs[0, b, g[h]], Bs[1, b, g[h]], Cs[1, b, g[h]]
            a2 = math.exp(dts[1, b, h] * A[h])
            want[b, h] = (dts[1, b, h] * np.dot(B2, C2) * xs[1, b, h]
                          + a2 * dts[0, b, h] * np.dot(B1, C2) * xs[0, b, h])
    return rel_err(y2, want)


def pin_geometric(step, T=25) -> float:
    """Scalar case P = N = 1, constant a = exp(dt A), C = 1, b = dt x B:
    s_t = b (1 - a^t) / (1 - a) from s_0 = 0, and y_t = s_t."""
    dt, A, x, Bv = 0.7, -0.4, 1.3, -0.9
    a, bb = math.exp(dt * A), dt * x * Bv
    S = np.zeros((1, 1, 1, 1))
    worst = 0.0
    for t in range(1, T + 1):
        S, y = step(S, np.array([A]), np.full((1, 1, 1), x), np.full((1, 1, 1), Bv),
                    np.ones((1, 1, 1)), np.full((1, 1), dt))
        want = bb * (1 - a ** t) / (1 - a)
        worst = max(worst, abs(float(y[0, 0, 0]) - want) / abs(want))
    return worst


def pin_linear_attention(scan, seed=3) -> float:
    """A = 0: Y = tril(C B^T) diag(dt) X + C S0^T for every (sequence, head)."""
    rng = np.random.default_rng(seed)
    T, Bt, H, G, P, N = 9, 2, 2, 1, 3, 4
    xs, Bs, Cs = _rand(rng, T, Bt, H, P), _rand(rng, T, Bt, G, N), _rand(rng, T, Bt, G, N)
    dts, S0 = _dt(rng, T, Bt, H), _rand(rng, Bt, H, P, N)
    ys = scan(S0, np.zeros(H), xs, Bs, Cs, dts)[0]
    worst = 0.0
    for b in range(Bt):
        for h in range(H):
            Cm, Bm = Cs[:, b, 0], Bs[:, b, 0]
            Y = np.tril(Cm @ Bm.T) @ np.diag(dts[:, b, h]) @ xs[:, b, h] + Cm @ S0[b, h].T
            worst = max(worst, rel_err(ys[:, b, h], Y))
    return worst


def pin_exact_rational(scan, seed=4) -> float:
    """A = 0 and small dyadic inputs: the fp64 recurrence is exact, so it must
    equal a Fraction evaluation of y_t = sum_{j<=t} dt_j (B_j.C_t) x_j + S0 C_t
    bit for bit (returns the largest absolute difference, 0 when exact)."""
    rng = np.random.default_rng(seed)
    T, P, N = 6, 3, 4
    q = lambda *s: rng.integers(-8, 9, size=s) / 8.0  # noqa: E731
    xs, Bs, Cs = q(T, 1, 1, P), q(T, 1, 1, N), q(T, 1, 1, N)
    dts = rng.integers(1, 9, size=(T, 1, 1)) / 4.0
    S0 = q(1, 1, P, N)
    ys = scan(S0, np.zeros(1), xs, Bs, Cs, dts)[0]
    F = Fraction
    worst = 0.0
    for t in range(T):
        for p in range(P):
            acc = sum(F(S0[0, 0, p, n]) * F(Cs[t, 0, 0, n]) for n in range(N))
            for j in range(t + 1):
                bc = sum(F(Bs[j, 0, 0, n]) * F(Cs[t, 0, 0, n]) for n in range(N))
                acc += F(dts[j, 0, 0]) * bc * F(xs[j, 0, 0, p])
            worst = max(worst, abs(float(F(ys[t, 0, 0, p]) - acc)))
    return worst


def load_golden(name: str) -> dict:
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            vals[k] = np.array([float(t) for t in v.split()])
    return vals


def pin_golden_two_tokens(step) -> float:
    g = load_golden("two_tokens_dyadic.txt")
    A = g["A"]
    worst = 0.0
    for suffix, S0 in (("", g["S0"].reshape(1, 1, 2, 2)), ("_zero_init", np.zeros((1, 1, 2, 2)))):
        S = S0
        for t in (0, 1):
            S, y = step(S, A, g[f"x{t}"].reshape(1, 1, 2), g[f"B{t}"].reshape(1, 1, 2),
                        g[f"C{t}"].reshape(1, 1, 2), g[f"dt{t}"].reshape(1, 1))
            worst = max(worst, float(np.max(np.abs(y.ravel() - g[f"y{t}{suffix}"]))))
        worst = max(worst, float(np.max(np.abs(S.ravel() - g[f"S2{suffix}"]))))
    return worst


def pin_unrolled(scan, unrolled, seed=5) -> float:
    """The recurrence against its unrolled closed form (no state formed)."""
    rng = np.random.default_rng(seed)
    T, Bt, H, G, P, N = 24, 2, 4, 2, 5, 3
    xs, Bs, Cs = _rand(rng, T, Bt, H, P), _rand(rng, T, Bt, G, N), _rand(rng, T, Bt, G, N)
    dts, A, S0 = _dt(rng, T, Bt, H), _A(rng, H), _rand(rng, Bt, H, P, N)
    return rel_err(scan(S0, A, xs, Bs, Cs, dts)[0], unrolled(S0, A, xs, Bs, Cs, dts))


def pin_mpmath(scan, seed=6) -> float:
    """fp64 recurrence against the same recurrence in 50-digit arithmetic."""
    import mpmath as mp
    mp.mp.dps = 50
    rng = np.random.default_rng(seed)
    T, P, N = 8, 3, 4
    xs, Bs, Cs = _rand(rng, T, 1, 1, P), _rand(rng, T, 1, 1, N), _rand(rng, T, 1, 1, N)
    dts, A = _dt(rng, T, 1, 1), _A(rng, 1)
    S0 = _rand(rng, 1, 1, P, N)
    ys = scan(S0, A, xs, Bs, Cs, dts)[0]
    S = [[mp.mpf(float(S0[0, 0, p, n])) for n in range(N)] for p in range(P)]
    worst = 0.0
    for t in range(T):
        a = mp.exp(mp.mpf(float(dts[t, 0, 0])) * mp.mpf(float(A[0])))
        d = mp.mpf(float(dts[t, 0, 0]))
        S = [[a * S[p][n] + d * mp.mpf(float(xs[t, 0, 0, p])) * mp.mpf(float(Bs[t, 0, 0, n]))
              for n in range(N)] for p in range(P)]
        yt = [mp.fsum(S[p][n] * mp.mpf(float(Cs[t, 0, 0, n])) for n in range(N)) for p in range(P)]
        scale = max(abs(v) for v in yt)
        for p in range(P):
            worst = max(worst, float(abs(yt[p] - mp.mpf(float(ys[t, 0, 0, p]))) / scale))
    return worst
