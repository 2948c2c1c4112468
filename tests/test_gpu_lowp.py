"""GPU low-precision modes beside dual precision: a single bf16 checkpoint
(replay; rounded once per fold) and a bf16-stored eager state (rounded every
token). Each is checked against its fp64 emulator in the oracle, a closed form
tells the two rounding schedules apart bit for bit, and drift curves over 1024
steps are measured against the exact recurrence for both decay regimes.

Tolerances. Device and emulator round the same values to bf16, but the device
forms them in fp32 and the emulator in fp64, so a value within ~1e-7 relative
of a rounding midpoint can land on the other side: such flips are one bf16 ulp
(2^-8 relative) on a few elements in ten thousand. Outputs and checkpoints of a
mode therefore match its emulator to rel-L2 <= 1e-3 per step, and drift figures
to 10 % of the emulator's; the exact-recurrence bar for bf16 reads is 2e-2.
"""
import numpy as np
import pytest
import torch

from oracle import mamba2
import workloads
from workloads import synth
from recurrent_state_storage_amd import rss
from gpu_util import DEV, PairGather, cfg_of, dev_inputs, rel_l2, sample_pairs, log

pytestmark = pytest.mark.gpu

TINY = workloads.get("tiny_b2_h4_p16_n16_w8")
EMU_TOL = 1e-3


def _eager_cfg(wl):
    return cfg_of(wl, read_copy=rss.RSS_STATE_BF16)


# ---- closed form: rounding every token vs once per fold -----------------------
def test_swamping_closed_form_all_modes():
    """S0 = 1, no decay (A = 0), +2^-9 per token on every element, C = e_0.
    bf16 stored every token never moves (1 + 2^-9 rounds to 1); a bf16
    checkpoint folded every 8 tokens gains exactly 2^-6 per fold; fp32 and dual
    are exact. All values are dyadic, so every comparison is exact."""
    P = N = 16
    T, W = 64, 8
    log("[lowp] swamping closed form, P=N=16, W=8, 64 tokens")
    base = TINY.replace(batch=1, nheads=1, ngroups=1, headdim=P, dstate=N, window=W, capacity=W)
    A = torch.zeros(1, device=DEV)
    x = torch.full((1, 1, P), 2.0 ** -9, device=DEV)
    B = torch.ones((1, 1, N), device=DEV)
    C = torch.zeros((1, 1, N), device=DEV)
    C[..., 0] = 1.0
    dt = torch.ones((1, 1), device=DEV)
    S0 = torch.ones((1, 1, P, N), device=DEV)
    layers = {m: rss.ReplayLayer(cfg_of(base.replace(read_copy=m)), A, DEV)
              for m in ("none", "bf16", "bf16_state")}
    for layer in layers.values():
        layer.init_state(S0)
    Sb = torch.ones((1, 1, P, N), dtype=torch.bfloat16, device=DEV)
    S32 = S0.clone()
    y = torch.empty((1, 1, P), device=DEV)
    for t in range(T):
        exact = 1.0 + (t + 1) * 2.0 ** -9
        for m, layer in layers.items():
            if m == "bf16_state":
                layer.decode_flush_step(W, x, B, C, dt, y)
            else:
                layer.decode_step(x, B, C, dt, y)
                layer.flush_checkpoint(W)
            assert torch.all(y == exact), (m, t)
        rss.rss_eager_step(_eager_cfg(base), Sb, x, B, C, dt, A, y)
        assert torch.all(y == 1.0 + 2.0 ** -9) and torch.all(Sb == 1.0), t
        rss.rss_eager_step(cfg_of(base), S32, x, B, C, dt, A, y)
        assert torch.all(y == exact), t
        if (t + 1) % W == 0:
            k = (t + 1) // W
            assert layers["bf16_state"].ckpt.dtype == torch.bfloat16
            assert torch.all(layers["bf16_state"].ckpt.float() == 1.0 + k * 2.0 ** -6), t
            assert torch.all(layers["none"].ckpt == 1.0 + k * 2.0 ** -6)
            assert torch.all(layers["bf16"].ckpt_lo.float() == 1.0 + k * 2.0 ** -6)
    for layer in layers.values():
        assert layer.device_error() == 0


# ---- both bf16-state modes against their emulators ----------------------------
SHAPES = [
    TINY.replace(read_copy="bf16_state"),
    TINY.replace(read_copy="bf16_state", s0="normal", ngroups=1),
    TINY.replace(name="p37_n64_g2_w5", read_copy="bf16_state", batch=3, nheads=4, ngroups=2,
                 headdim=37, dstate=64, window=5, capacity=7, in_dtype="bf16", s0="normal"),
    TINY.replace(name="p64_n128_w16", read_copy="bf16_state", batch=2, nheads=3, ngroups=3,
                 headdim=64, dstate=128, window=16, capacity=16, in_dtype="bf16"),
    TINY.replace(name="p100_n256_w4", read_copy="bf16_state", batch=1, nheads=2, ngroups=1,
                 headdim=100, dstate=256, window=4, capacity=6, s0="normal"),
]


@pytest.mark.parametrize("wl", SHAPES, ids=lambda w: f"{w.name}-{w.s0}-G{w.ngroups}")
def test_bf16_state_modes_match_emulators(wl):
    steps = 3 * wl.window + 3
    log(f"[lowp] {wl.name} P={wl.headdim} N={wl.dstate} G={wl.ngroups} W={wl.window} "
        f"in={wl.in_dtype} s0={wl.s0}: {steps} steps")
    A_np = synth.params(wl)["A"]
    A = torch.from_numpy(A_np).to(DEV)
    S0 = synth.initial_state(wl)
    layer = rss.ReplayLayer(cfg_of(wl), A, DEV)
    layer.init_state(torch.from_numpy(S0).to(DEV))
    Se = torch.from_numpy(S0).to(DEV).to(torch.bfloat16)       # RNE, as the emulator stores it
    emu = mamba2.ReplayModel(S0, A_np, wl.ngroups, wl.capacity, read_copy="bf16_state")
    assert np.array_equal(layer.ckpt.double().cpu().numpy(), emu.ckpt)
    S_ref = S0.astype(np.float64)
    Bt, H, P = wl.batch, wl.nheads, wl.headdim
    hist = {k: [] for k in ("x", "B", "C", "dt")}
    ye_all, worst = [], {"replay": 0.0, "ckpt": 0.0, "exact": 0.0, "eager": 0.0}
    y = torch.empty((Bt, H, P), device=DEV)
    ye = torch.empty_like(y)
    for t in range(steps):
        s = synth.step_inputs(wl, t)
        for k in hist:
            hist[k].append(s[k])
        d = dev_inputs(s, wl.in_dtype)
        layer.decode_step(d["x"], d["B"], d["C"], d["dt"], y)
        rss.rss_eager_step(_eager_cfg(wl), Se, d["x"], d["B"], d["C"], d["dt"], A, ye)
        y_em = emu.decode(s["x"], s["B"], s["C"], s["dt"])
        S_ref, y_ref = mamba2.eager_step(S_ref, A_np, s["x"], s["B"], s["C"], s["dt"])
        yg = y.double().cpu().numpy()
        assert np.isfinite(yg).all()
        worst["replay"] = max(worst["replay"], rel_l2(yg, y_em))
        worst["exact"] = max(worst["exact"], rel_l2(yg, y_ref))
        ye_all.append(ye.double().cpu().numpy())
        layer.flush_checkpoint(wl.window)
        if emu.flush(wl.window):
            worst["ckpt"] = max(worst["ckpt"], rel_l2(layer.ckpt.double().cpu().numpy(), emu.ckpt))
    ys_em, S_em = mamba2.eager_scan_bf16_state(S0, A_np, *(np.stack(hist[k]) for k in hist))
    for t in range(steps):
        worst["eager"] = max(worst["eager"], rel_l2(ye_all[t], ys_em[t]))
    state_err = rel_l2(Se.double().cpu().numpy(), S_em)
    log("  " + ", ".join(f"{k} {v:.2e}" for k, v in worst.items()) + f", eager state {state_err:.2e}")
    assert worst["replay"] <= EMU_TOL and worst["ckpt"] <= EMU_TOL
    assert worst["eager"] <= EMU_TOL and state_err <= EMU_TOL
    assert worst["exact"] <= 2e-2
    assert layer.device_error() == 0


def test_bf16_state_verify_and_rollback():
    """Speculative rounds on a bf16-only checkpoint: verify outputs match the
    emulator, and rollback leaves the stored bf16 checkpoint bytes unchanged."""
    wl = TINY.replace(name="spec_bf16_state", read_copy="bf16_state", batch=3, nheads=4, ngroups=2,
                      headdim=32, dstate=64, window=8, capacity=12, max_draft=4, in_dtype="bf16",
                      s0="normal", draft=4)
    log(f"[lowp] {wl.name}: 6 verify rounds, K=4")
    A_np = synth.params(wl)["A"]
    A = torch.from_numpy(A_np).to(DEV)
    S0 = synth.initial_state(wl)
    layer = rss.ReplayLayer(cfg_of(wl), A, DEV)
    layer.init_state(torch.from_numpy(S0).to(DEV))
    emu = mamba2.ReplayModel(S0, A_np, wl.ngroups, wl.capacity, read_copy="bf16_state")
    K = wl.draft
    worst = 0.0
    for r in range(6):
        dr = synth.draft_inputs(wl, r)
        nacc = synth.accepted_drafts(wl, r)
        d = dev_inputs(dr, wl.in_dtype)
        y = torch.empty((wl.batch, K + 1, wl.nheads, wl.headdim), device=DEV)
        before = layer.ckpt.clone()
        layer.verify_k_tokens(K, d["x"], d["B"], d["C"], d["dt"], y)
        y_em = emu.verify(dr["x"], dr["B"], dr["C"], dr["dt"])
        worst = max(worst, rel_l2(y.double().cpu().numpy(), y_em))
        ndrop = (K - nacc).astype(np.int32)
        layer.rollback(torch.from_numpy(ndrop).to(DEV))
        emu.rollback(ndrop)
        assert torch.equal(layer.ckpt.view(torch.int16), before.view(torch.int16))
        layer.flush_checkpoint(wl.window)
        emu.flush(wl.window)
    log(f"  verify vs emulator {worst:.2e}")
    assert worst <= EMU_TOL
    assert layer.device_error() == 0


# ---- drift curves: the low-precision comparison --------------------------------
@pytest.mark.slow
@pytest.mark.parametrize("family", ["dual", "slowdecay"])
def test_low_precision_drift_curves(family):
    """16 sequences of the batch-256 shape, 1024 steps, W = 8, 16, 32 side by
    side: eager with a bf16-stored state, replay with a single bf16 checkpoint,
    and dual precision, each against the exact fp64 recurrence on 24 sampled
    (sequence, head) pairs and against its own emulator. `dual` draws the
    dual-precision workload's inputs (decay ~0.8 per token); `slowdecay` scales
    A by 0.01 (decay ~0.997, long memory), where per-token rounding piles up."""
    wins = (8, 16, 32)
    wls = {w: workloads.get(f"mamba2_{family}_b256_h128_p64_n128_w{w}").replace(batch=16) for w in wins}
    wl = wls[16]
    log(f"[lowp] drift curves {family}: 16 sequences, {wl.steps} steps, W = 8/16/32")
    A_np = synth.params(wl)["A"]
    A = torch.from_numpy(A_np).to(DEV)
    modes = [("bf16_state", w) for w in wins] + [("bf16", w) for w in wins]
    layers = {m: rss.ReplayLayer(cfg_of(wls[m[1]].replace(read_copy=m[0])), A, DEV) for m in modes}
    for layer in layers.values():
        layer.init_state()
    Se = torch.zeros((wl.batch, wl.nheads, wl.headdim, wl.dstate), dtype=torch.bfloat16, device=DEV)
    pg = PairGather(wl, sample_pairs(wl, 24, seed=17))
    A_pair = pg.A(A_np)
    Z = np.zeros((1, len(pg.pairs), wl.headdim, wl.dstate))
    emus = {m: mamba2.ReplayModel(Z, A_pair, len(pg.pairs), wls[m[1]].capacity, read_copy=m[0])
            for m in modes}
    S_ref, S_emb = Z.copy(), Z.copy()
    y = torch.empty((wl.batch, wl.nheads, wl.headdim), device=DEV)
    got = {m: [] for m in modes + [("eager_bf16", 0)]}
    emu_y = {m: [] for m in got}
    refs = []
    for t in range(wl.steps):
        s = synth.step_inputs(wl, t)
        d = dev_inputs(s, wl.in_dtype)
        ps = pg.step(s)
        S_ref, y_ref = mamba2.eager_step(S_ref, A_pair, ps["x"], ps["B"], ps["C"], ps["dt"])
        refs.append(y_ref)
        for m in modes:
            layers[m].decode_step(d["x"], d["B"], d["C"], d["dt"], y)
            got[m].append(pg.out(y))
            layers[m].flush_checkpoint(m[1])
            emu_y[m].append(emus[m].decode(ps["x"], ps["B"], ps["C"], ps["dt"]))
            emus[m].flush(m[1])
        rss.rss_eager_step(_eager_cfg(wl), Se, d["x"], d["B"], d["C"], d["dt"], A, y)
        got[("eager_bf16", 0)].append(pg.out(y))
        S_new, y_eb = mamba2.eager_step(S_emb, A_pair, ps["x"], ps["B"], ps["C"], ps["dt"])
        S_emb = mamba2.lowp.round_bf16(S_new)
        emu_y[("eager_bf16", 0)].append(y_eb)
    torch.cuda.synchronize()
    ref = np.stack(refs)
    res = {}
    for m in got:
        g, e = np.stack(got[m]), np.stack(emu_y[m])
        curve = [rel_l2(g[t0:t0 + 128], ref[t0:t0 + 128]) for t0 in range(0, wl.steps, 128)]
        res[m] = {"run": rel_l2(g, ref), "emu_run": rel_l2(e, ref), "vs_emu": rel_l2(g, e),
                  "last256": rel_l2(g[-256:], ref[-256:]), "curve": curve}
        log(f"  {m[0]:10s} W={m[1]:2d}: run {res[m]['run']:.3e} (emulator {res[m]['emu_run']:.3e}, "
            f"vs emulator {res[m]['vs_emu']:.1e}), last 256 {res[m]['last256']:.3e}, per 128 steps "
            + " ".join(f"{c:.2e}" for c in curve))
    for m, r in res.items():
        assert r["vs_emu"] <= EMU_TOL, m
        assert abs(r["run"] - r["emu_run"]) <= 0.1 * r["emu_run"], m
    eb = res[("eager_bf16", 0)]["run"]
    for w in wins:
        single, dual = res[("bf16_state", w)]["run"], res[("bf16", w)]["run"]
        assert dual <= 2e-2
        assert eb > single >= 0.9 * dual, w          # per-token rounding is worst
        if family == "slowdecay":
            assert single > 1.5 * dual, w            # a shared bf16 checkpoint accumulates
    if family == "slowdecay":                         # fewer folds, fewer roundings
        assert res[("bf16_state", 8)]["run"] > res[("bf16_state", 16)]["run"] > res[("bf16_state", 32)]["run"]
    for layer in layers.values():
        assert layer.device_error() == 0


# ---- the bf16 rounding itself ---------------------------------------------------
def _edge_patterns(n, seed=77):
    """fp32 bit patterns that stress a round-to-nearest-even conversion: exact
    ties with even and odd kept parts (both signs), values just above and below
    a tie, denormals (smallest, largest, ties), the largest finite values (which
    round up to infinity), infinities, signed zeros, NaNs with a quiet bit and
    with only low payload bits, then random patterns to fill n."""
    edges = []
    for hi in (0x3F80, 0x3F81, 0x0001, 0x007F, 0x0080, 0x7F7E, 0x7F7F, 0x4B00, 0x3400):
        for lo in (0x8000, 0x7FFF, 0x8001, 0x0000, 0xFFFF, 0x0001):
            for sign in (0, 0x80000000):
                edges.append(((hi << 16) | lo) | sign)
    edges += [0x00000001, 0x007FFFFF, 0x00400000, 0x00008000, 0x00018000, 0x7F800000, 0xFF800000,
              0x00000000, 0x80000000, 0x7FC00000, 0xFFC00001, 0x7F800001, 0x7FBFFFFF, 0xFF80FFFF,
              0x7FFFFFFF, 0x7F808000]
    rng = np.random.default_rng(seed)
    rest = rng.integers(0, 2 ** 32, size=n - len(edges), dtype=np.uint64).astype(np.uint32)
    return np.concatenate([np.array(edges, dtype=np.uint32), rest])


def _rne_bits(u):
    """Expected bf16 bits, written from the definition: NaN -> top half with the
    quiet bit set; otherwise the oracle's round-to-nearest-even."""
    from oracle import lowp
    u = np.asarray(u, dtype=np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    f = u.copy()
    f[nan] = 0                                   # the oracle rounds finite values and infinities
    r = lowp.round_bf16_from_f32(f.view(np.float32)).astype(np.float32).view(np.uint32) >> 16
    return np.where(nan, (u >> 16) | 0x40, r).astype(np.uint16)


@pytest.mark.parametrize("copy", ["bf16", "bf16_state"])
def test_bf16_rounding_bit_exact_on_edge_patterns(copy):
    """init_state stores the bf16 image of S0 (the read copy in dual mode, the
    checkpoint itself with a bf16-only checkpoint) through the same packed
    conversion every bf16 store uses; its bits must be round-to-nearest-even of
    the fp32 input, ties, denormals, overflow to infinity and NaNs included."""
    P, N = 64, 128
    code = rss.RSS_COPY_BF16 if copy == "bf16" else rss.RSS_STATE_BF16
    cfg = rss.make_config(2, 3, P, N, 3, 4, 4, 0, rss.RSS_DTYPE_F32, code)
    u = _edge_patterns(2 * 3 * P * N)
    S0 = torch.from_numpy(u.view(np.float32).reshape(2, 3, P, N).copy()).to(DEV)
    layer = rss.ReplayLayer(cfg, torch.zeros(3, device=DEV), DEV)
    layer.init_state(S0)
    lo = layer.ckpt_lo if copy == "bf16" else layer.ckpt
    got = lo.cpu().view(torch.int16).numpy().view(np.uint16).reshape(-1)
    want = _rne_bits(u)
    bad = np.nonzero(got != want)[0]
    log(f"[lowp] {copy}: {len(u)} patterns, {len(bad)} mismatches")
    assert len(bad) == 0, [(hex(u[i]), hex(got[i]), hex(want[i])) for i in bad[:8]]
    if copy == "bf16":   # the fp32 master keeps the input bits
        assert np.array_equal(layer.ckpt.cpu().numpy().view(np.uint32).reshape(-1), u)
