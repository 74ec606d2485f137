"""GPU parity of llatte_ffn_backward (the pre-norm FFN sublayer backward)
against the oracle's ffn_block_backward in fp64 on the same inputs (weights
rounded to bf16 on both sides), from a few rows through a ragged row count
to the upstream layer-1 shape (64 users x 1600 rows, d = 512, d_ff = 2048),
plus the no-row and W2 = 0 cases.

Tolerance (the bf16 path's): max|g - r| / RMS(r) <= 2e-2 per gradient.
A weight gradient over fewer than 64 rows is a short sum of outer products
of two bf16-rounded vectors (relative rounding 2^-9 each): its largest
entries sit about (max/RMS of one vector)^2 ~ 10 times above its RMS, and
the rounding error scales with them, so there the bar is
max|g - r| <= 1e-2 max|r| (about twice the two roundings plus dA's own).
"""
import numpy as np
import pytest

import synth
from oracle import llatte_oracle as O

pytestmark = pytest.mark.gpu


def _err(g, r):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    return float(np.max(np.abs(g - r)) / np.sqrt(np.mean(r ** 2)))


def make_inputs(M, d, F, seed):
    rng = np.random.default_rng(seed)
    R1 = rng.standard_normal((M, d)).astype(np.float32)
    g2 = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    W1 = synth.round_bf16(rng.standard_normal((d, F)) / np.sqrt(d))
    W2 = synth.round_bf16(rng.standard_normal((F, d)) / np.sqrt(F))
    dout = rng.standard_normal((M, d)).astype(np.float32)
    return R1, g2, W1, W2, dout


def run_gpu(R1, g2, W1, W2, dout, eps=1e-6):
    import torch
    from target_aware_latent_amd import llatte as C
    M, d = R1.shape
    F = W1.shape[1]
    f = C.llatte_ffn_desc(d, F, C.LLATTE_BF16, eps)
    dev = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda().to(dt)
    ws = torch.empty(max(C.llatte_ffn_backward_workspace_size(f, M), 256), dtype=torch.uint8,
                     device="cuda")
    nan = lambda *s: torch.full(s, float("nan"), device="cuda")
    dr1, dg2, dw1, dw2 = nan(M, d), nan(d), nan(d, F), nan(F, d)
    C.llatte_ffn_backward(f, dev(R1), dev(g2), dev(W1, torch.bfloat16), dev(W2, torch.bfloat16),
                          dev(dout), M, dr1, dg2, dw1, dw2, ws)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (dr1, dg2, dw1, dw2)]


CASES = [
    # M, d, F
    (1, 64, 256),
    (7, 64, 128),
    (333, 128, 512),
    (1000, 64, 256),
    (4099, 512, 2048),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"M{c[0]}-d{c[1]}-F{c[2]}")
def test_ffn_backward_matches_oracle(case):
    M, d, F = case
    print(f"ffn backward {case}", flush=True)
    R1, g2, W1, W2, dout = make_inputs(M, d, F, seed=M)
    got = run_gpu(R1, g2, W1, W2, dout)
    ref = O.ffn_block_backward(*(x.astype(np.float64) for x in (R1, g2, W1, W2, dout)))
    for name, g, r in zip(("d_r1", "d_g2", "d_w1", "d_w2"), got, ref):
        assert np.isfinite(g).all(), name
        if M < 64 and name in ("d_w1", "d_w2"):
            e = float(np.max(np.abs(g - r)) / np.max(np.abs(r)))
            assert e <= 1e-2, f"{name}: error {e:.3e} of the largest entry"
        else:
            e = _err(g, r)
            assert e <= 2e-2, f"{name}: error {e:.3e}"


def test_upstream_layer_one_shape():
    M, d, F = 64 * 1600, 512, 2048
    print("ffn backward 102400 x 512 x 2048", flush=True)
    R1, g2, W1, W2, dout = make_inputs(M, d, F, seed=7)
    got = run_gpu(R1, g2, W1, W2, dout)
    ref = O.ffn_block_backward(*(x.astype(np.float64) for x in (R1, g2, W1, W2, dout)))
    for name, g, r in zip(("d_r1", "d_g2", "d_w1", "d_w2"), got, ref):
        e = _err(g, r)
        assert e <= 2e-2, f"{name}: error {e:.3e}"


def test_zero_second_weight_passes_the_gradient_through():
    R1, g2, W1, W2, dout = make_inputs(200, 128, 512, seed=3)
    dr1, dg2, dw1, dw2 = run_gpu(R1, g2, W1, np.zeros_like(W2), dout)
    np.testing.assert_array_equal(dr1, dout)
    assert np.count_nonzero(dg2) == 0 and np.count_nonzero(dw1) == 0
    ref = O.ffn_block_backward(*(x.astype(np.float64) for x in (R1, g2, W1, np.zeros_like(W2), dout)))
    assert _err(dw2, ref[3]) <= 2e-2


def test_no_rows_zero_the_weight_gradients():
    import torch
    from target_aware_latent_amd import llatte as C
    d, F = 64, 256
    f = C.llatte_ffn_desc(d, F, C.LLATTE_BF16, 1e-6)
    g2 = torch.ones(d, device="cuda")
    w1 = torch.ones(d, F, device="cuda").to(torch.bfloat16)
    w2 = torch.ones(F, d, device="cuda").to(torch.bfloat16)
    nan = lambda *s: torch.full(s, float("nan"), device="cuda")
    dg2, dw1, dw2 = nan(d), nan(d, F), nan(F, d)
    C.llatte_ffn_backward(f, None, g2, w1, w2, None, 0, None, dg2, dw1, dw2, None)
    torch.cuda.synchronize()
    for t in (dg2, dw1, dw2):
        assert torch.count_nonzero(t).item() == 0
