"""Pins of the sequence-summary oracle (LoRAMLP_k over the flattened
readout, oracle.llatte_oracle.lora_mlp_summaries) against torch's linear /
GELU routines in other groupings, the no-adapter and adapter-only special
cases, and a scalar brute force; plus the raw-readout option of the forward
(no W_p) against the projected readout.

Source: "LLaTTE: Scaling Laws for Multi-Stage Sequence Modeling in
Large-Scale Ads Recommendation" (annotated translation), Appendix A.2 item 4
(sequence summaries: LoRAMLP_k of Flatten(Z_raw)).
"""
import math

import numpy as np
import pytest

import synth
from oracle import llatte_oracle as O
from synth.summaries import generate_summaries, get_summary_config


def _small(name="s_small", seed=0):
    cfg = get_summary_config(name)
    p = generate_summaries(cfg, seed)
    return cfg, p["weights"], p["inputs"]["z"]


def test_unmerged_adapters_in_torch_match():
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    cfg, L, z = _small()
    got = O.lora_mlp_summaries(z, L)
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    zt = t(z)
    for k in range(cfg.K):
        # the adapters applied as separate low-rank products (x A) B, not merged
        pre = F.linear(zt, t(L["W1"]).T) + F.linear(F.linear(zt, t(L["A1"][k]).T), t(L["B1"][k]).T)
        h = F.gelu(pre, approximate="none")
        y = F.linear(h, t(L["W2"]).T) + F.linear(F.linear(h, t(L["A2"][k]).T), t(L["B2"][k]).T)
        np.testing.assert_allclose(got[k], y.numpy(), rtol=1e-12, atol=1e-12)


def test_zero_adapters_give_the_plain_mlp():
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    cfg, L, z = _small(seed=1)
    L = dict(L)
    L["B1"] = np.zeros_like(L["B1"])
    L["B2"] = np.zeros_like(L["B2"])
    got = O.lora_mlp_summaries(z, L)
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    y = F.linear(F.gelu(F.linear(t(z), t(L["W1"]).T), approximate="none"), t(L["W2"]).T).numpy()
    for k in range(cfg.K):
        np.testing.assert_allclose(got[k], y, rtol=1e-12, atol=1e-12)
    # and the summaries then coincide
    np.testing.assert_array_equal(got[0], got[cfg.K - 1])


def test_adapters_only_when_the_base_is_zero():
    cfg, L, z = _small(seed=2)
    L = dict(L)
    L["W1"] = np.zeros_like(L["W1"])
    L["W2"] = np.zeros_like(L["W2"])
    got = O.lora_mlp_summaries(z, L)
    for k in range(cfg.K):
        a = np.asarray(z, np.float64) @ np.asarray(L["A1"][k], np.float64)
        pre = a @ np.asarray(L["B1"][k], np.float64)
        h = np.array([[0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in row] for row in pre])
        y = (h @ np.asarray(L["A2"][k], np.float64)) @ np.asarray(L["B2"][k], np.float64)
        np.testing.assert_allclose(got[k], y, rtol=1e-12, atol=1e-12)


def test_brute_force_on_tiny_inputs():
    cfg, L, z = _small(seed=3)
    got = O.lora_mlp_summaries(z, L)
    for k in (0, cfg.K - 1):
        for b in (0, cfg.B - 1):
            x = [float(v) for v in z[b]]
            h = []
            for j in range(cfg.d_hidden):
                s = 0.0
                for i in range(cfg.d_z):
                    w = float(L["W1"][i][j])
                    for r in range(cfg.rank):
                        w += float(L["A1"][k][i][r]) * float(L["B1"][k][r][j])
                    s += x[i] * w
                h.append(0.5 * s * (1.0 + math.erf(s / math.sqrt(2.0))))
            for c in (0, 17, cfg.d_seq - 1):
                s = 0.0
                for j in range(cfg.d_hidden):
                    w = float(L["W2"][j][c])
                    for r in range(cfg.rank):
                        w += float(L["A2"][k][j][r]) * float(L["B2"][k][r][c])
                    s += h[j] * w
                assert got[k, b, c] == pytest.approx(s, rel=1e-11, abs=1e-12)


def test_forward_without_projection_returns_the_flattened_readout():
    cfg = synth.get_config("c1")
    cfg = synth.Config("c1_ro", B=3, L=12, len_range=None, d=16, h=2, dk=8, r=8, n_q=2,
                       d_c=8, N=1, pyramid=cfg.pyramid, dtype="f32", n_seeds=2, d_out=12)
    p = synth.generate(cfg, seed=0)
    W, I = p["weights"], p["inputs"]
    a = O.forward(cfg, W, I["hist"], I["offsets"], I["cand"], I["ctx"])
    W2 = dict(W)
    W2["W_p"] = None
    b = O.forward(cfg, W2, I["hist"], I["offsets"], I["cand"], I["ctx"])
    for u in range(cfg.B):
        assert b["emb"][u].shape == (cfg.n_seeds * cfg.d,)
        np.testing.assert_allclose(b["emb"][u] @ np.asarray(W["W_p"], np.float64), a["emb"][u],
                                   rtol=1e-12, atol=1e-12)
