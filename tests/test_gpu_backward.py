"""GPU parity of llatte_mla_attention_backward against the oracle's
latent_attention_backward (fp64 on the same bf16-rounded q_lat and C), for
jagged users with pyramid-style query subsets and candidates, one-key
histories, and the upstream layer-1 shape of two users. The GPU backward
takes the GPU forward's out and lse.

Tolerance (the bf16 path's): max|g - r| / RMS(r) <= 2e-2 per tensor.
"""
import math

import numpy as np
import pytest

import synth
from oracle import llatte_oracle as O

pytestmark = pytest.mark.gpu


def _err(g, r):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    return float(np.max(np.abs(g - r)) / np.sqrt(np.mean(r ** 2)))


def run_backward(h, r, K, n, n_cand, seed=0):
    import torch
    from target_aware_latent_amd import llatte as C
    rng = np.random.default_rng(seed)
    K, n = np.asarray(K), np.asarray(n)
    B = K.size
    kv = np.concatenate([[0], np.cumsum(K)]).astype(np.int32)
    hq = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    Mtot = int(B * n_cand + hq[-1])
    q = synth.round_bf16(rng.standard_normal((Mtot, h, r)) * 0.5)
    Cl = synth.round_bf16(rng.standard_normal((int(kv[-1]), r)))
    g = rng.standard_normal((Mtot, h, r)).astype(np.float32)
    scale = 1.0 / math.sqrt(64)
    dev = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda().to(dt)
    idev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()
    ad = C.llatte_attn_desc(h, r, n_cand, C.LLATTE_BF16, scale)
    Ktot = int(kv[-1])
    ws = torch.empty(C.llatte_mla_attention_workspace_size(ad, B, Mtot, Ktot), dtype=torch.uint8,
                     device="cuda")
    qd, cd = dev(q, torch.bfloat16), dev(Cl, torch.bfloat16)
    out = torch.empty((Mtot, h, r), device="cuda")
    lse = torch.empty((Mtot, h), device="cuda")
    C.llatte_mla_attention(ad, qd, cd, idev(kv), idev(hq), B, Mtot, Ktot, out, lse, ws)
    d_q = torch.full((Mtot, h, r), float("nan"), device="cuda")
    d_c = torch.full((Ktot, r), float("nan"), device="cuda")
    bws = torch.empty(C.llatte_mla_attention_backward_workspace_size(ad, Mtot), dtype=torch.uint8,
                      device="cuda")
    C.llatte_mla_attention_backward(ad, qd, cd, idev(kv), idev(hq), B, Mtot, Ktot, int(K.max()),
                                    out, lse, dev(g), d_q, d_c, bws)
    torch.cuda.synchronize()
    rq, rc = O.latent_attention_backward(q.astype(np.float64), Cl.astype(np.float64), kv, hq,
                                         n_cand, scale, g.astype(np.float64))
    return d_q.cpu().numpy(), d_c.cpu().numpy(), rq, rc, g


CASES = [
    # h, r, K per user, n per user, n_cand
    (4, 64, [1, 63, 64, 65, 200, 333], [1, 63, 10, 65, 0, 200], 16),
    (8, 128, [300, 129, 1], [300, 64, 1], 0),
    (8, 128, [700, 50], [300, 50], 5),
    (2, 64, [90, 260], [90, 17], 2),
    (3, 128, [130, 5, 257], [100, 5, 0], 3),   # odd head count: one head group
    (1, 64, [64, 129], [64, 129], 0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"h{c[0]}-r{c[1]}-nc{c[4]}-B{len(c[2])}")
def test_backward_matches_oracle(case):
    h, r, K, n, nc = case
    print(f"attention backward {case}", flush=True)
    dq, dc, rq, rc, _ = run_backward(h, r, K, n, nc)
    assert np.isfinite(dq).all() and np.isfinite(dc).all()
    e_q, e_c = _err(dq, rq), _err(dc, rc)
    assert e_q <= 2e-2, f"d_q error {e_q:.3e}"
    assert e_c <= 2e-2, f"d_c error {e_c:.3e}"


def test_one_key_history():
    # users with one key and one history row: d_c[key] = sum of d_out over
    # the heads (and the user's candidates), d_q = 0
    dq, dc, rq, rc, g = run_backward(8, 128, [1, 1, 1], [1, 0, 1], 2, seed=3)
    assert np.max(np.abs(dq)) <= 1e-3 * np.max(np.abs(g))
    assert _err(dc, rc) <= 2e-2


def test_upstream_layer_one_shape():
    # two users of the upstream layer 1: 1600 keys, 1600 causal query rows, 8 heads
    print("attention backward 2 x 1600", flush=True)
    dq, dc, rq, rc, _ = run_backward(8, 128, [1600, 1600], [1600, 1600], 0, seed=1)
    assert _err(dq, rq) <= 2e-2
    assert _err(dc, rc) <= 2e-2


def test_no_query_rows_zero_the_latent_gradient():
    # every user with n = 0 and no candidates: Mtot = 0, d_c = 0, and the
    # row buffers may be NULL
    import torch
    from target_aware_latent_amd import llatte as C
    ad = C.llatte_attn_desc(4, 128, 0, C.LLATTE_BF16, 0.125)
    kv = torch.tensor([0, 5, 14], dtype=torch.int32, device="cuda")
    hq = torch.zeros(3, dtype=torch.int32, device="cuda")
    cl = torch.randn(14, 128, device="cuda").to(torch.bfloat16)
    d_c = torch.full((14, 128), float("nan"), device="cuda")
    C.llatte_mla_attention_backward(ad, None, cl, kv, hq, 2, 0, 14, 9, None, None, None, None,
                                    d_c, None)
    torch.cuda.synchronize()
    assert torch.count_nonzero(d_c).item() == 0


def test_full_upstream_layer_one_sampled_users():
    # the bench's launch configuration: 64 users x 1600 keys and causal query
    # rows, 8 heads, r = 128; users are independent, so the oracle checks the
    # d_q rows and d_C rows of sampled users one by one
    import torch
    from target_aware_latent_amd import llatte as C
    B, L, h, r = 64, 1600, 8, 128
    print("attention backward 64 x 1600 (sampled users)", flush=True)
    rng = np.random.default_rng(21)
    kv = (np.arange(B + 1) * L).astype(np.int32)
    q = synth.round_bf16(rng.standard_normal((B * L, h, r)) * 0.5)
    Cl = synth.round_bf16(rng.standard_normal((B * L, r)))
    g = rng.standard_normal((B * L, h, r)).astype(np.float32)
    dev = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda().to(dt)
    ad = C.llatte_attn_desc(h, r, 0, C.LLATTE_BF16, 0.125)
    kvd = torch.from_numpy(kv).cuda()
    qd, cd = dev(q, torch.bfloat16), dev(Cl, torch.bfloat16)
    out = torch.empty((B * L, h, r), device="cuda")
    lse = torch.empty((B * L, h), device="cuda")
    ws = torch.empty(C.llatte_mla_attention_workspace_size(ad, B, B * L, B * L), dtype=torch.uint8,
                     device="cuda")
    C.llatte_mla_attention(ad, qd, cd, kvd, kvd, B, B * L, B * L, out, lse, ws)
    d_q = torch.empty((B * L, h, r), device="cuda")
    d_c = torch.empty((B * L, r), device="cuda")
    bws = torch.empty(C.llatte_mla_attention_backward_workspace_size(ad, B * L), dtype=torch.uint8,
                      device="cuda")
    C.llatte_mla_attention_backward(ad, qd, cd, kvd, kvd, B, B * L, B * L, L, out, lse, dev(g), d_q,
                                    d_c, bws)
    torch.cuda.synchronize()
    d_q, d_c = d_q.cpu().numpy(), d_c.cpu().numpy()
    assert np.isfinite(d_q).all() and np.isfinite(d_c).all()
    for u in (0, 29, 63):
        s = slice(u * L, (u + 1) * L)
        rq, rc = O.latent_attention_backward(q[s].astype(np.float64), Cl[s].astype(np.float64),
                                             [0, L], [0, L], 0, 0.125, g[s].astype(np.float64))
        assert _err(d_q[s], rq) <= 2e-2, f"user {u} d_q"
        assert _err(d_c[s], rc) <= 2e-2, f"user {u} d_c"
