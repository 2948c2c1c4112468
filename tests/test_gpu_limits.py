"""The largest supported shapes on the GPU: P = N = 256 with the longest ring the
LDS budget allows (R = 64, or 58 with fp32 x/B/C and drafts, 48 for KDA), the
longest draft (K = 7), a window that fills the ring, and head groups shared by
two heads. Every output against the fp64 recurrence over the committed stream,
pointers against the integer ring model."""
import numpy as np
import pytest
import torch

from oracle import gdn, kda, mamba2
from oracle.ring import PointerModel
import workloads
from workloads import synth
from recurrent_state_storage_amd import rss
from gpu_util import DEV, cfg_of, dev_inputs, rel_l2, log

pytestmark = pytest.mark.gpu

BASE = workloads.get("tiny_b2_h4_p16_n16_w8")


@pytest.mark.parametrize("in_dtype,copy,R", [("bf16", "none", 64), ("f32", "none", 58),
                                              ("bf16", "bf16", 64),
                                              # bf16-stored checkpoint: the fold inside the decode
                                              # (R = 16), and the separate fold its LDS budget
                                              # forces at R = 64
                                              ("bf16", "bf16_state", 16), ("bf16", "bf16_state", 64)])
def test_mamba2_largest_shape(in_dtype, copy, R):
    K = 7
    W = R - K
    wl = BASE.replace(name="max", batch=2, nheads=2, ngroups=1, headdim=256, dstate=256, window=W,
                      capacity=R, max_draft=K, draft=K, in_dtype=in_dtype, read_copy=copy,
                      s0="normal", seed=8000 + R)
    log(f"[limits] mamba2 P=N=256 R={R} W={W} K={K} in={in_dtype} copy={copy}")
    A_np = synth.params(wl)["A"]
    A = torch.from_numpy(A_np).to(DEV)
    S0 = synth.initial_state(wl)
    L = rss.ReplayLayer(cfg_of(wl), A, DEV)
    L.init_state(torch.from_numpy(S0).to(DEV))
    pm = PointerModel(wl.batch, R)
    S = S0.astype(np.float64)
    tol = 1e-5 if copy == "none" else 2e-2
    worst = 0.0
    y = torch.empty((wl.batch, wl.nheads, wl.headdim), device=DEV)

    def decode(t):
        nonlocal S, worst
        s = synth.step_inputs(wl, t)
        d = dev_inputs(s, in_dtype)
        L.decode_flush_step(W, d["x"], d["B"], d["C"], d["dt"], y)
        for b in range(wl.batch):
            pm.append(b, 1)
            pm.flush(b, W)
        S, yr = mamba2.eager_step(S, A_np, s["x"], s["B"], s["C"], s["dt"])
        worst = max(worst, rel_l2(y.double().cpu().numpy(), yr))

    for t in range(W - 1):                     # the window one short of full
        decode(t)
    rin = synth.draft_inputs(wl, 0)            # K+1 = 8 tentative entries fill the ring
    nacc = synth.accepted_drafts(wl, 0)
    d = dev_inputs(rin, in_dtype)
    yv = torch.empty((wl.batch, K + 1, wl.nheads, wl.headdim), device=DEV)
    L.verify_k_tokens(K, d["x"], d["B"], d["C"], d["dt"], yv)
    Sr = S
    yg = yv.double().cpu().numpy()
    for i in range(K + 1):
        Sr, yr = mamba2.eager_step(Sr, A_np, rin["x"][:, i], rin["B"][:, i], rin["C"][:, i],
                                   rin["dt"][:, i])
        worst = max(worst, rel_l2(yg[:, i], yr))
    L.rollback(torch.from_numpy((K - nacc).astype(np.int32)).to(DEV))
    L.flush_checkpoint(W)
    for b in range(wl.batch):
        pm.append(b, K + 1)
        pm.mark_tentative(b, K + 1)
        pm.rollback(b, int(K - nacc[b]))
        pm.flush(b, W)
    # continue from the committed stream: the accepted drafts, per sequence
    Sn = np.empty_like(S)
    for b in range(wl.batch):
        Sb = S[b:b + 1]
        for i in range(int(nacc[b]) + 1):
            Sb, _ = mamba2.eager_step(Sb, A_np, rin["x"][b:b + 1, i], rin["B"][b:b + 1, i],
                                      rin["C"][b:b + 1, i], rin["dt"][b:b + 1, i])
        Sn[b] = Sb[0]
    S = Sn
    for t in range(1000, 1000 + W + 3):        # a full window more: every sequence folds again
        decode(t)
    ptr = L.ptr.cpu().numpy()
    for h in range(wl.nheads):
        assert np.array_equal(ptr[:, h, :3], pm.as_array())
    log(f"  worst rel-L2 {worst:.2e}")
    assert worst < tol
    assert L.device_error() == 0


@pytest.mark.parametrize("kind,R", [("gdn", 64), ("kda", 48)])
def test_delta_rule_largest_shape(kind, R):
    wl = workloads.get(f"{kind}_b256_h32_d128_w16").replace(
        batch=2, nheads=2, ngroups=2, headdim=256, dstate=256, window=R, capacity=R, s0="normal",
        seed=8100 + R)
    log(f"[limits] {kind} d_v=d_k=256 R=W={R}")
    L = rss.ReplayLayer(cfg_of(wl), None, DEV)
    S0 = synth.initial_state(wl)
    L.init_state(torch.from_numpy(S0).to(DEV))
    S = S0.astype(np.float64)
    mod, gen = (kda, synth.kda_step_inputs) if kind == "kda" else (gdn, synth.gdn_step_inputs)
    step = L.kda_decode_step if kind == "kda" else L.gdn_decode_step
    o = torch.empty((wl.batch, wl.nheads, wl.headdim), device=DEV)
    worst = 0.0
    for t in range(R + 5):
        s = gen(wl, t)
        d = {k: torch.from_numpy(np.ascontiguousarray(v)).to(DEV) for k, v in s.items()}
        step(d["q"], d["k"], d["v"], d["beta"], d["alpha"], o)
        L.flush_checkpoint(R)
        S, orf = mod.eager_step(S, s["q"], s["k"], s["v"], s["beta"], s["alpha"])
        worst = max(worst, rel_l2(o.double().cpu().numpy(), orf))
        if t == R - 1:
            assert rel_l2(L.ckpt.double().cpu().numpy(), S) < 1e-5
    log(f"  worst rel-L2 {worst:.2e}")
    assert worst < 1e-5
    assert L.device_error() == 0
