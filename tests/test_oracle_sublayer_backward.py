"""Pins of the attention-sublayer backward oracle (oracle.llatte_oracle.
attention_sublayer_backward, and its rmsnorm_backward) against torch
autograd on an independent torch forward, central finite differences of
the oracle's own pinned layer forward (mla_layer with W1 = W2 = 0, whose
output is then the sublayer's), and the one-key closed form.

Source: "LLaTTE: Scaling Laws for Multi-Stage Sequence Modeling in
Large-Scale Ads Recommendation" (annotated translation), Appendix A.3 (MLA,
non-absorbed form) and Appendix A.2 (layer equation, pre-norm reading); the
backward is the derivative of that definition.
"""
import math
from types import SimpleNamespace

import numpy as np
import pytest

from oracle import llatte_oracle as O

NAMES = ("g1", "W_dkv", "g_c", "W_uq", "W_uk", "W_uv", "W_o")


def _case(seed, K=9, n=5, n_c=2, d=16, h=2, dk=4, r=6, latent_norm=True):
    rng = np.random.default_rng(seed)
    cfg = SimpleNamespace(d=d, h=h, dk=dk, r=r, eps=1e-6, latent_norm=latent_norm,
                          norm_mode="pre")
    W = {"g1": 1 + 0.1 * rng.standard_normal(d), "W_dkv": rng.standard_normal((d, r)) / math.sqrt(d),
         "g_c": 1 + 0.1 * rng.standard_normal(r), "W_uq": rng.standard_normal((d, h * dk)) / math.sqrt(d),
         "W_uk": rng.standard_normal((r, h * dk)) / math.sqrt(r),
         "W_uv": rng.standard_normal((r, h * dk)) / math.sqrt(r),
         "W_o": rng.standard_normal((h * dk, d)) / math.sqrt(h * dk),
         "g2": np.ones(d), "W1": np.zeros((d, 4 * d)), "W2": np.zeros((4 * d, d))}
    Rh = rng.standard_normal((K, d))
    Rc = rng.standard_normal((n_c, d))
    dRq = rng.standard_normal((n + n_c, d))
    return cfg, W, Rh, Rc, n, dRq


def _torch_sublayer(torch, cfg, T, Rh, Rc, n):
    F_ = torch.nn.functional
    K, n_c = Rh.shape[0], Rc.shape[0]
    H = F_.rms_norm(Rh, (cfg.d,), weight=T["g1"], eps=cfg.eps)
    Hc = F_.rms_norm(Rc, (cfg.d,), weight=T["g1"], eps=cfg.eps)
    C = H @ T["W_dkv"]
    if cfg.latent_norm:
        C = F_.rms_norm(C, (cfg.r,), weight=T["g_c"], eps=cfg.eps)
    Hq = torch.cat([H[K - n:], Hc])
    q = (Hq @ T["W_uq"]).reshape(-1, cfg.h, cfg.dk)
    pos = torch.tensor([K - n + t for t in range(n)] + [K - 1] * n_c)
    mask = torch.arange(K)[None, :] > pos[:, None]
    outs = []
    for hh in range(cfg.h):
        Kh = C @ T["W_uk"][:, hh * cfg.dk:(hh + 1) * cfg.dk]
        Vh = C @ T["W_uv"][:, hh * cfg.dk:(hh + 1) * cfg.dk]
        s = (q[:, hh, :] @ Kh.T) / math.sqrt(cfg.dk)
        outs.append(torch.softmax(s.masked_fill(mask, float("-inf")), dim=1) @ Vh)
    o = torch.stack(outs, dim=1).reshape(-1, cfg.h * cfg.dk)
    return torch.cat([Rh[K - n:], Rc]) + o @ T["W_o"]


@pytest.mark.parametrize("latent_norm", [True, False])
def test_matches_torch_autograd(latent_norm):
    torch = pytest.importorskip("torch")
    cfg, W, Rh, Rc, n, dRq = _case(0, latent_norm=latent_norm)
    T = {k: torch.tensor(W[k], requires_grad=True) for k in NAMES}
    th = torch.tensor(Rh, requires_grad=True)
    tc = torch.tensor(Rc, requires_grad=True)
    _torch_sublayer(torch, cfg, T, th, tc, n).backward(torch.tensor(dRq))
    dRh, dRc, g = O.attention_sublayer_backward(Rh, Rc, n, W, cfg, dRq)
    np.testing.assert_allclose(dRh, th.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dRc, tc.grad.numpy(), rtol=1e-10, atol=1e-12)
    for k in NAMES:
        if k == "g_c" and not latent_norm:
            assert k not in g
            continue
        np.testing.assert_allclose(g[k], T[k].grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=k)


def test_central_finite_differences_of_the_layer_forward():
    # W1 = W2 = 0: mla_layer's output is R1 = Rq + A exactly
    cfg, W, Rh, Rc, n, dRq = _case(1)
    dRh, dRc, g = O.attention_sublayer_backward(Rh, Rc, n, W, cfg, dRq)

    def loss(Rh_, Rc_, W_):
        oh, oc = O.mla_layer(Rh_, Rc_, n, W_, cfg)
        return float(np.sum(dRq * np.concatenate([oh, oc])))

    eps = 1e-6
    for idx in [(0, 0), (4, 7), (8, 15)]:
        a, b = Rh.copy(), Rh.copy()
        a[idx] += eps
        b[idx] -= eps
        assert (loss(a, Rc, W) - loss(b, Rc, W)) / (2 * eps) == pytest.approx(dRh[idx], rel=1e-6, abs=1e-8)
    for idx in [(0, 3), (1, 12)]:
        a, b = Rc.copy(), Rc.copy()
        a[idx] += eps
        b[idx] -= eps
        assert (loss(Rh, a, W) - loss(Rh, b, W)) / (2 * eps) == pytest.approx(dRc[idx], rel=1e-6, abs=1e-8)
    for k, idx in [("g1", (3,)), ("W_dkv", (2, 5)), ("g_c", (1,)), ("W_uq", (7, 6)),
                   ("W_uk", (4, 3)), ("W_uv", (0, 7)), ("W_o", (5, 11))]:
        a, b = dict(W), dict(W)
        a[k] = W[k].copy()
        b[k] = W[k].copy()
        a[k][idx] += eps
        b[k][idx] -= eps
        fd = (loss(Rh, Rc, a) - loss(Rh, Rc, b)) / (2 * eps)
        assert fd == pytest.approx(g[k][idx], rel=1e-6, abs=1e-8), k


def test_one_key_has_no_score_gradient():
    # one key, one history query, no candidates: the softmax is 1 whatever
    # the scores, so nothing reaches the query and key projections
    cfg, W, Rh, Rc, n, dRq = _case(2, K=1, n=1, n_c=0)
    dRh, dRc, g = O.attention_sublayer_backward(Rh, Rc, n, W, cfg, dRq)
    np.testing.assert_array_equal(g["W_uq"], 0.0)
    np.testing.assert_array_equal(g["W_uk"], 0.0)
    assert dRc.shape == (0, cfg.d)
    assert np.max(np.abs(g["W_uv"])) > 0


def test_rmsnorm_backward_matches_torch_autograd():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(4)
    x, g, dy = rng.standard_normal((6, 10)), 1 + 0.1 * rng.standard_normal(10), rng.standard_normal((6, 10))
    tx, tg = torch.tensor(x, requires_grad=True), torch.tensor(g, requires_grad=True)
    torch.nn.functional.rms_norm(tx, (10,), weight=tg, eps=1e-6).backward(torch.tensor(dy))
    dx, dg = O.rmsnorm_backward(x, g, dy, 1e-6)
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dg, tg.grad.numpy(), rtol=1e-11, atol=1e-13)
