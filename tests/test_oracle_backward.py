"""Pins of the latent-attention backward oracle
(oracle.llatte_oracle.latent_attention_backward) against torch autograd on
an independent torch forward, central finite differences, and closed forms
(one allowed key, identical keys).

Source: "LLaTTE: Scaling Laws for Multi-Stage Sequence Modeling in
Large-Scale Ads Recommendation" (annotated translation), Appendix A.3 (the
absorbed MLA form: attention on the latent, C both key and value); the
backward is the derivative of that definition.
"""
import numpy as np
import pytest

from oracle import llatte_oracle as O


def _case(seed, B=3, h=2, r=8, n_cand=2, lengths=(5, 1, 9), keep=(3, 1, 9)):
    rng = np.random.default_rng(seed)
    lengths = np.array(lengths)
    keep = np.array(keep)
    kv = np.concatenate([[0], np.cumsum(lengths)])
    hq = np.concatenate([[0], np.cumsum(keep)])
    Mtot = B * n_cand + int(hq[-1])
    q = rng.standard_normal((Mtot, h, r))
    C = rng.standard_normal((int(kv[-1]), r))
    g = rng.standard_normal((Mtot, h, r))
    return q, C, kv, hq, n_cand, 0.3, g


def _torch_forward(torch, q, C, kv, hq, n_cand, scale):
    """The attention written with torch ops (masked_fill + softmax)."""
    B = len(kv) - 1
    nc = B * n_cand
    out = torch.zeros_like(q)
    for u in range(B):
        Cu = C[kv[u]:kv[u + 1]]
        K = Cu.shape[0]
        n = int(hq[u + 1] - hq[u])
        rows = list(range(nc + hq[u], nc + hq[u + 1])) + list(range(u * n_cand, (u + 1) * n_cand))
        pos = torch.tensor([K - n + t for t in range(n)] + [K - 1] * n_cand)
        mask = torch.arange(K)[None, :] > pos[:, None]
        for hh in range(q.shape[1]):
            s = (q[rows, hh, :] @ Cu.T) * scale
            p = torch.softmax(s.masked_fill(mask, float("-inf")), dim=1)
            out = out.index_put((torch.tensor(rows), torch.tensor(hh)), p @ Cu)
    return out


def test_matches_torch_autograd():
    torch = pytest.importorskip("torch")
    q, C, kv, hq, nc, scale, g = _case(0)
    qt = torch.tensor(q, requires_grad=True)
    Ct = torch.tensor(C, requires_grad=True)
    out = _torch_forward(torch, qt, Ct, kv, hq, nc, scale)
    out.backward(torch.tensor(g))
    dq, dc = O.latent_attention_backward(q, C, kv, hq, nc, scale, g)
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dc, Ct.grad.numpy(), rtol=1e-11, atol=1e-12)
    # the oracle's own forward agrees with the torch one
    o_ref, _ = O.latent_attention(q, C, kv, hq, nc, scale)
    np.testing.assert_allclose(out.detach().numpy(), o_ref, rtol=1e-12, atol=1e-12)


def test_central_finite_differences():
    q, C, kv, hq, nc, scale, g = _case(1)
    dq, dc = O.latent_attention_backward(q, C, kv, hq, nc, scale, g)
    loss = lambda q_, C_: float(np.sum(g * O.latent_attention(q_, C_, kv, hq, nc, scale)[0]))
    eps = 1e-6
    for idx in [(0, 0, 0), (7, 1, 5), (q.shape[0] - 1, 1, 7)]:
        qp, qm = q.copy(), q.copy()
        qp[idx] += eps
        qm[idx] -= eps
        assert (loss(qp, C) - loss(qm, C)) / (2 * eps) == pytest.approx(dq[idx], rel=1e-6, abs=1e-8)
    for idx in [(0, 0), (5, 3), (C.shape[0] - 1, 7)]:
        Cp, Cm = C.copy(), C.copy()
        Cp[idx] += eps
        Cm[idx] -= eps
        assert (loss(q, Cp) - loss(q, Cm)) / (2 * eps) == pytest.approx(dc[idx], rel=1e-6, abs=1e-8)


def test_one_allowed_key_passes_the_gradient_straight_to_it():
    # one user, one key, one history query row, no candidates: out = C_0 for
    # every head whatever q is, so d_q = 0 and d_C_0 = sum over heads of d_out
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 3, 4))
    C = rng.standard_normal((1, 4))
    g = rng.standard_normal((1, 3, 4))
    dq, dc = O.latent_attention_backward(q, C, [0, 1], [0, 1], 0, 0.5, g)
    np.testing.assert_allclose(dq, 0.0, atol=1e-14)
    np.testing.assert_allclose(dc[0], g[0].sum(axis=0), rtol=1e-14, atol=1e-14)


def test_identical_keys_give_no_query_gradient():
    # all keys equal: the softmax is uniform whatever the scores, out = C_0
    rng = np.random.default_rng(3)
    q = rng.standard_normal((4, 2, 6))
    C = np.tile(rng.standard_normal((1, 6)), (4, 1))
    g = rng.standard_normal((4, 2, 6))
    dq, dc = O.latent_attention_backward(q, C, [0, 4], [0, 4], 0, 0.7, g)
    np.testing.assert_allclose(dq, 0.0, atol=1e-12)
    # the value gradient sums to the total of d_out over rows and heads
    np.testing.assert_allclose(dc.sum(axis=0), g.sum(axis=(0, 1)), rtol=1e-12, atol=1e-12)
