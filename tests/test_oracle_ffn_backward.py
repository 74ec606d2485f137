"""Pins of the FFN-sublayer backward oracle (oracle.llatte_oracle.
ffn_block_backward) against torch autograd on an independent torch forward
(torch's own rms_norm and exact GELU), central finite differences, the
W2 = 0 special case, and the scale invariance of RMSNorm.

Source: "LLaTTE: Scaling Laws for Multi-Stage Sequence Modeling in
Large-Scale Ads Recommendation" (annotated translation), Appendix A.2 (the
layer equation, pre-norm reading: R2 = R1 + FFN(RMSNorm(R1))); the backward
is the derivative of that definition.
"""
import numpy as np
import pytest

from oracle import llatte_oracle as O


def _case(seed, M=7, d=12, F=20, eps=1e-6):
    rng = np.random.default_rng(seed)
    R1 = rng.standard_normal((M, d)) * 1.5
    g2 = 1 + 0.1 * rng.standard_normal(d)
    W1 = rng.standard_normal((d, F)) / np.sqrt(d)
    W2 = rng.standard_normal((F, d)) / np.sqrt(F)
    dout = rng.standard_normal((M, d))
    return R1, g2, W1, W2, dout, eps


def test_matches_torch_autograd():
    torch = pytest.importorskip("torch")
    F_ = torch.nn.functional
    R1, g2, W1, W2, dout, eps = _case(0)
    t = [torch.tensor(x, requires_grad=True) for x in (R1, g2, W1, W2)]
    h = F_.rms_norm(t[0], (R1.shape[1],), weight=t[1], eps=eps)
    R2 = t[0] + F_.gelu(h @ t[2], approximate="none") @ t[3]
    R2.backward(torch.tensor(dout))
    got = O.ffn_block_backward(R1, g2, W1, W2, dout, eps)
    for g, tt in zip(got, t):
        np.testing.assert_allclose(g, tt.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_central_finite_differences():
    R1, g2, W1, W2, dout, eps = _case(1)
    dR1, dg2, dW1, dW2 = O.ffn_block_backward(R1, g2, W1, W2, dout, eps)

    def loss(R1_, g2_, W1_, W2_):
        H2 = O.rmsnorm(R1_, g2_, eps)
        return float(np.sum(dout * (R1_ + O.gelu(H2 @ W1_) @ W2_)))

    h = 1e-6
    args = [R1, g2, W1, W2]
    for which, grad, idxs in [(0, dR1, [(0, 0), (3, 7), (6, 11)]), (1, dg2, [(0,), (5,)]),
                              (2, dW1, [(0, 0), (4, 13)]), (3, dW2, [(2, 3), (19, 11)])]:
        for idx in idxs:
            ap, am = [a.copy() for a in args], [a.copy() for a in args]
            ap[which][idx] += h
            am[which][idx] -= h
            fd = (loss(*ap) - loss(*am)) / (2 * h)
            assert fd == pytest.approx(grad[idx], rel=1e-6, abs=1e-8)


def test_zero_second_weight_passes_the_gradient_through():
    # W2 = 0: the FFN branch is zero whatever its input, so dR1 = d_out and
    # nothing reaches W1 or g2; dW2 is GELU(H2 W1)^T d_out
    R1, g2, W1, W2, dout, eps = _case(2)
    dR1, dg2, dW1, dW2 = O.ffn_block_backward(R1, g2, W1, np.zeros_like(W2), dout, eps)
    np.testing.assert_array_equal(dR1, dout)
    np.testing.assert_array_equal(dg2, 0.0)
    np.testing.assert_array_equal(dW1, 0.0)
    H2 = O.rmsnorm(R1, g2, eps)
    np.testing.assert_allclose(dW2, O.gelu(H2 @ W1).T @ dout, rtol=1e-13, atol=1e-13)


def test_norm_branch_is_orthogonal_to_the_row():
    # with eps = 0, RMSNorm(a x) = RMSNorm(x) for a > 0: the gradient that
    # goes through the norm has no component along the row itself
    R1, g2, W1, W2, dout, _ = _case(3)
    dR1, _, _, _ = O.ffn_block_backward(R1, g2, W1, W2, dout, 0.0)
    through = dR1 - dout
    assert np.max(np.abs(np.sum(through * R1, axis=1))) < 1e-12 * np.max(np.abs(through))
    assert np.max(np.abs(through)) > 1e-3
