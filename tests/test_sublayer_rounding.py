"""Why the attention-sublayer gradients are judged by their own bar (R24).

The GPU computes the attention sublayer's backward in the absorbed form of
[LLaTTE] Appendix A.3 with bf16 operands: the recomputed forward rounds H,
the latent C, q, the latent queries, the latent output and o to bf16 (and
the attention core takes its operands and P in fp16), and the backward
rounds d_out, do, the latent-query gradient, dq and the latent gradient to
bf16 before they enter products. This file emulates exactly those rounding
points in fp64, all other arithmetic exact, and compares with the oracle's
exact gradients (non-absorbed definition):

- with every rounding switched off, the emulation equals the oracle to
  1e-9 (this pins the emulation's own gradient formulas: the absorbed and
  non-absorbed forms have the same derivative);
- with the roundings, some gradient tensor exceeds the forward's bar
  max|g - r| <= 2e-2 RMS(r) on these shapes (each gradient is dominated by a
  few rows: a causal user's early query rows attend few keys), while every
  tensor stays within max|g - r| <= 1.5e-2 max|r| and RMS(g - r) <=
  1e-2 RMS(r), the bar the GPU test of the sublayer backward applies.

The inputs are the GPU test's (synth.sublayer_case, same seeds).
"""
import math
from types import SimpleNamespace

import numpy as np
import pytest

import synth
from oracle import llatte_oracle as O
from synth.sublayer import sublayer_case

LOG2E = 1.0 / math.log(2.0)


def bf16(x):
    return synth.round_bf16(x).astype(np.float64)


def fp16(x):
    return np.asarray(x, np.float64).astype(np.float16).astype(np.float64)


def ident(x):
    return np.asarray(x, np.float64)


def emulate(Rh, Rc, n, W, cfg, dRq, rb, rh):
    """Sublayer backward for one user with rounding functions rb (the bf16
    points) and rh (the fp16 operands of the attention core's forward).
    Returns (dRh, dRc, grads) like O.attention_sublayer_backward."""
    d, h, dk, r, eps = cfg.d, cfg.h, cfg.dk, cfg.r, cfg.eps
    K, nc = Rh.shape[0], Rc.shape[0]
    H = rb(O.rmsnorm(Rh, W["g1"], eps))
    Hc = rb(O.rmsnorm(Rc, W["g1"], eps))
    C0 = H @ W["W_dkv"]
    C = rb(O.rmsnorm(C0, W["g_c"], eps) if cfg.latent_norm else C0)
    Hq = np.concatenate([H[K - n:], Hc], axis=0)
    M = Hq.shape[0]
    q = rb(Hq @ W["W_uq"])
    allowed = O.history_query_mask(K, n, nc)
    scale = 1.0 / math.sqrt(dk)
    Wuk = W["W_uk"].reshape(r, h, dk)
    Wuv = W["W_uv"].reshape(r, h, dk)
    qt, ot, Pb = [], [], []
    for j in range(h):
        qt.append(rb(q[:, j * dk:(j + 1) * dk] @ Wuk[:, j, :].T))
        # forward core: scores in log2 units from fp16 operands, P in fp16,
        # the sums exact; lse from the running max and the sum of P
        s2 = np.where(allowed, rh(qt[j] * scale * LOG2E) @ rh(C).T, -np.inf)
        m = np.max(s2, axis=1, keepdims=True)
        p = np.where(allowed, rh(np.exp2(s2 - m)), 0.0)
        l = np.sum(p, axis=1, keepdims=True)
        ot.append((p @ rh(C)) / l)
        lse = (m + np.log2(l)) / LOG2E
        # the backward core recomputes P from its (bf16) operands and lse
        Pb.append(np.where(allowed, np.exp(scale * (qt[j] @ C.T) - lse), 0.0))
    otb = [rb(x) for x in ot]
    o = np.concatenate([rb(otb[j] @ Wuv[:, j, :]) for j in range(h)], axis=1)
    g = {}
    dRb = rb(dRq)
    g["W_o"] = o.T @ dRb
    dob = rb(dRb @ W["W_o"].T)
    dWuv = np.zeros((r, h, dk))
    dWuk = np.zeros((r, h, dk))
    dC = np.zeros_like(C)
    dq = np.zeros((M, h * dk))
    for j in range(h):
        do_j = dob[:, j * dk:(j + 1) * dk]
        dWuv[:, j, :] = otb[j].T @ do_j
        dot = do_j @ Wuv[:, j, :].T
        D = np.sum(dot * ot[j], axis=1, keepdims=True)
        ds = Pb[j] * (dot @ C.T - D)
        dC += Pb[j].T @ dot + scale * (ds.T @ qt[j])
        dqt = rb(scale * (ds @ C))
        dq[:, j * dk:(j + 1) * dk] = rb(dqt @ Wuk[:, j, :])
        dWuk[:, j, :] = dqt.T @ q[:, j * dk:(j + 1) * dk]
    g["W_uk"] = dWuk.reshape(r, h * dk)
    g["W_uv"] = dWuv.reshape(r, h * dk)
    g["W_uq"] = Hq.T @ dq
    dHq = dq @ W["W_uq"].T
    if cfg.latent_norm:
        dC0, g["g_c"] = O.rmsnorm_backward(C0, W["g_c"], dC, eps)
    else:
        dC0 = dC
    dC0 = rb(dC0)
    g["W_dkv"] = H.T @ dC0
    dH = dC0 @ W["W_dkv"].T
    dH[K - n:] += dHq[:n]
    dRh, dg1h = O.rmsnorm_backward(Rh, W["g1"], dH, eps)
    dRc, dg1c = O.rmsnorm_backward(Rc, W["g1"], dHq[n:], eps)
    g["g1"] = dg1h + dg1c
    dRh[K - n:] += dRq[:n]
    dRc = dRc + dRq[n:]
    return dRh, dRc, g


def run(case, rb, rh):
    d, h, dk, r, n_cand, K, n, ln = case
    cfg = SimpleNamespace(d=d, h=h, dk=dk, r=r, eps=1e-6, latent_norm=ln, norm_mode="pre")
    W, Rh, Rc, dout, kv, hq = sublayer_case(d, h, dk, r, n_cand, K, n, 0)
    B, nc = len(K), len(K) * n_cand
    out = {"emu": [], "ref": []}
    for which, fn in (("emu", lambda *a: emulate(*a, rb, rh)),
                      ("ref", O.attention_sublayer_backward)):
        dRh_all, dRc_all, gsum = [], [], {}
        for u in range(B):
            dq_u = np.concatenate([dout[nc + hq[u]:nc + hq[u + 1]],
                                   dout[u * n_cand:(u + 1) * n_cand]]).astype(np.float64)
            dRh, dRc, g = fn(Rh[u].astype(np.float64), Rc[u].astype(np.float64), int(n[u]), W, cfg,
                             dq_u)
            dRh_all.append(dRh)
            dRc_all.append(dRc)
            for k, v in g.items():
                gsum[k] = gsum.get(k, 0.0) + v
        t = {"d_r_kv": np.concatenate(dRh_all)}
        if n_cand:
            t["d_r_cand"] = np.concatenate(dRc_all)
        t.update(gsum)
        out[which] = t
    return out["emu"], out["ref"]


def metrics(g, r):
    e = np.abs(g - r)
    rms = math.sqrt(float(np.mean(r * r)))
    return (float(np.max(e)) / rms, float(np.max(e)) / float(np.max(np.abs(r))),
            math.sqrt(float(np.mean(e * e))) / rms)


# the shapes of the GPU test of the sublayer backward (its upstream-size case
# aside): d, h, dk, r, n_cand, K per user, n per user, latent norm
CASES = [
    (64, 2, 32, 64, 3, [20, 70, 1], [20, 35, 1], True),
    (128, 4, 32, 128, 0, [130, 65], [130, 64], False),
    (256, 4, 64, 128, 2, [300, 200, 90], [150, 200, 0], True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"d{c[0]}-h{c[1]}-r{c[3]}-nc{c[4]}")
def test_emulation_without_rounding_is_the_oracle(case):
    emu, ref = run(case, ident, ident)
    for k in ref:
        scale = max(float(np.max(np.abs(ref[k]))), 1e-30)
        assert np.max(np.abs(emu[k] - ref[k])) <= 1e-9 * scale, k


def test_rounding_points_exceed_the_forward_bar_but_not_the_sublayer_bar():
    worst_rms = 0.0
    for case in CASES:
        emu, ref = run(case, bf16, fp16)
        for k in ref:
            if k == "g_c" and not case[7]:
                continue
            max_rms, max_rel, rms_rel = metrics(emu[k], ref[k])
            print(f"{case[:5]} {k:8s} max/RMS {max_rms:.2e}  max/max {max_rel:.2e}  "
                  f"RMS/RMS {rms_rel:.2e}", flush=True)
            worst_rms = max(worst_rms, max_rms)
            assert max_rel <= 1.5e-2 and rms_rel <= 1e-2, (case, k, max_rel, rms_rel)
    assert worst_rms > 2e-2, worst_rms
