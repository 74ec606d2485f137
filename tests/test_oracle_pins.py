"""Pins of the CPU oracle against things other than itself (CPU only).

Each test names what it pins: a library routine (torch CPU in fp64), a closed
form, an invariant the pages imply, a hand-worked table, or the independent
scalar-loop brute force on tiny inputs.
"""
import dataclasses
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import brute
from oracle import llatte_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny_cfg(**kw):
    base = dict(name="tiny", B=3, L=None, len_range=None, d=8, h=2, dk=4, r=3,
                n_q=2, d_c=3, N=2,
                pyramid=synth.PyramidRule("fixed", (5, 3)), dtype="f32",
                gain_jitter=0.1)
    base.update(kw)
    return synth.Config(**base)


def rand_layer(rng, cfg):
    d, hd, r, rq = cfg.d, cfg.h * cfg.dk, cfg.r, cfg.r_q
    qin = rq if rq else d
    n = lambda *s: rng.standard_normal(s)
    L = {"g1": 1 + 0.1 * n(d), "W_dkv": n(d, r) / math.sqrt(d),
         "g_c": 1 + 0.1 * n(r), "W_uq": n(qin, hd) / math.sqrt(qin),
         "W_uk": n(r, hd) / math.sqrt(r), "W_uv": n(r, hd) / math.sqrt(r),
         "W_o": n(hd, d) / math.sqrt(hd), "g2": 1 + 0.1 * n(d),
         "W1": n(d, 4 * d) / math.sqrt(d), "W2": n(4 * d, d) / math.sqrt(4 * d)}
    if rq:
        L["W_dq"] = n(d, rq) / math.sqrt(d)
        L["g_q"] = 1 + 0.1 * n(rq)
    return L


def rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ------------------------------------------------------- primitives vs torch

def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 33)) * 3
    g = 1 + 0.2 * rng.standard_normal(33)
    ref = F.rms_norm(torch.tensor(x), (33,), weight=torch.tensor(g), eps=1e-6)
    assert rel(O.rmsnorm(x, g, 1e-6), ref.numpy()) < 1e-14


def test_rmsnorm_scale_invariance_exact():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 16))
    g = np.ones(16)
    # eps is negligible only relative to mean(x^2); use eps=0 for exactness
    a = O.rmsnorm(x, g, 0.0)
    b = O.rmsnorm(x * 8.0, g, 0.0)
    assert np.array_equal(a, b)


def test_gelu_matches_erf_and_torch():
    xs = np.linspace(-6, 6, 101)
    ref = np.array([0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in xs])
    assert rel(O.gelu(xs), ref) < 1e-14
    tref = F.gelu(torch.tensor(xs), approximate="none").numpy()
    assert rel(O.gelu(xs), tref) < 1e-14


# ------------------------------------------------------- layer vs torch.nn

def torch_layer(Rh, Rc, n, W, cfg):
    """The layer built from torch.nn parts: RMSNorm, MultiheadAttention with
    separate key/value input width r (the latent), GELU. Pins head split,
    mask, scale, residual placement and norms of the oracle's layer."""
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64))
    d, h = cfg.d, cfg.h
    K = Rh.shape[0]
    norm = lambda x, g: F.rms_norm(x, (x.shape[-1],), weight=t(g), eps=cfg.eps)
    pre = cfg.norm_mode == "pre"
    Rh_t, Rc_t = t(Rh), t(Rc)
    Hh = norm(Rh_t, W["g1"]) if pre else Rh_t
    Hc = norm(Rc_t, W["g1"]) if pre else Rc_t
    C = Hh @ t(W["W_dkv"])
    if cfg.latent_norm:
        C = norm(C, W["g_c"])
    mha = torch.nn.MultiheadAttention(d, h, bias=False, kdim=cfg.r, vdim=cfg.r,
                                      batch_first=True, dtype=torch.float64)
    with torch.no_grad():
        if "W_dq" not in W:
            mha.q_proj_weight.copy_(t(W["W_uq"]).T)
        mha.k_proj_weight.copy_(t(W["W_uk"]).T)
        mha.v_proj_weight.copy_(t(W["W_uv"]).T)
        mha.out_proj.weight.copy_(t(W["W_o"]).T)
    Hq = torch.cat([Hh[K - n:], Hc])
    if "W_dq" in W:
        # low-rank query path: the query enters already projected,
        # RMSNorm(Hq W_dq) g_q W_uq, through an identity q_proj (h*dk == d)
        with torch.no_grad():
            mha.q_proj_weight.copy_(torch.eye(d, dtype=torch.float64))
        Qin = norm(Hq @ t(W["W_dq"]), W["g_q"]) @ t(W["W_uq"])
    else:
        Qin = Hq
    mha.eval()
    Rq = torch.cat([Rh_t[K - n:], Rc_t])
    M = Hq.shape[0]
    blocked = torch.ones(M, K, dtype=torch.bool)
    for i in range(n):
        blocked[i, :K - n + i + 1] = False
    blocked[n:, :] = False
    with torch.no_grad():
        A = mha(Qin[None], C[None], C[None], attn_mask=blocked,
                need_weights=False)[0][0]
    gelu = lambda x: F.gelu(x, approximate="none")
    if pre:
        R1 = Rq + A
        R2 = R1 + gelu(norm(R1, W["g2"]) @ t(W["W1"])) @ t(W["W2"])
    else:
        R1 = norm(Rq + A, W["g1"])
        R2 = norm(R1 + gelu(R1 @ t(W["W1"])) @ t(W["W2"]), W["g2"])
    return R2[:n].numpy(), R2[n:].numpy()


@pytest.mark.parametrize("norm_mode", ["pre", "post"])
@pytest.mark.parametrize("latent_norm", [True, False])
@pytest.mark.parametrize("K,n,nc", [(9, 9, 3), (9, 4, 2), (6, 0, 4), (1, 1, 2),
                                    (12, 5, 0)])
def test_layer_matches_torch_nn(norm_mode, latent_norm, K, n, nc):
    cfg = tiny_cfg(d=16, h=4, dk=4, r=6, norm_mode=norm_mode,
                   latent_norm=latent_norm)
    rng = np.random.default_rng(K * 100 + n * 10 + nc)
    W = rand_layer(rng, cfg)
    Rh = rng.standard_normal((K, cfg.d))
    Rc = rng.standard_normal((nc, cfg.d))
    ah, ac = O.mla_layer(Rh, Rc, n, W, cfg)
    bh, bc = torch_layer(Rh, Rc, n, W, cfg)
    assert ah.shape == (n, cfg.d) and ac.shape == (nc, cfg.d)
    if n:
        assert rel(ah, bh) < 1e-12
    if nc:
        assert rel(ac, bc) < 1e-12


@pytest.mark.parametrize("norm_mode", ["pre", "post"])
@pytest.mark.parametrize("K,n,nc,rq", [(9, 9, 3, 5), (9, 4, 2, 24), (6, 0, 4, 3)])
def test_low_rank_query_layer_matches_torch_nn(norm_mode, K, n, nc, rq):
    cfg = tiny_cfg(d=16, h=4, dk=4, r=6, norm_mode=norm_mode, r_q=rq)
    rng = np.random.default_rng(K * 100 + n * 10 + nc + rq)
    W = rand_layer(rng, cfg)
    Rh = rng.standard_normal((K, cfg.d))
    Rc = rng.standard_normal((nc, cfg.d))
    ah, ac = O.mla_layer(Rh, Rc, n, W, cfg)
    bh, bc = torch_layer(Rh, Rc, n, W, cfg)
    if n:
        assert rel(ah, bh) < 1e-12
    if nc:
        assert rel(ac, bc) < 1e-12


def test_low_rank_query_with_identity_down_projection_is_full_rank():
    # With eps = 0, g1 = 1, W_dq = I and g_q = 1 the query norm acts on rows
    # that are already unit-RMS, so the low-rank path returns H W_uq exactly
    # (up to rounding) and the layer equals the full-rank layer.
    cfg = tiny_cfg(d=16, h=4, dk=4, r=6, eps=0.0, r_q=16)
    cfg_full = dataclasses.replace(cfg, r_q=0)
    rng = np.random.default_rng(77)
    W = rand_layer(rng, cfg)
    W["g1"] = np.ones(cfg.d)
    W["W_dq"] = np.eye(cfg.d)
    W["g_q"] = np.ones(cfg.d)
    Wf = {k: v for k, v in W.items() if k not in ("W_dq", "g_q")}
    Rh = rng.standard_normal((7, cfg.d))
    Rc = rng.standard_normal((2, cfg.d))
    ah, ac = O.mla_layer(Rh, Rc, 4, W, cfg)
    bh, bc = O.mla_layer(Rh, Rc, 4, Wf, cfg_full)
    assert rel(ah, bh) < 1e-12 and rel(ac, bc) < 1e-12


# ------------------------------------------------------- MLA invariants

@pytest.mark.parametrize("norm_mode", ["pre", "post"])
def test_absorbed_equals_non_absorbed(norm_mode):
    cfg = tiny_cfg(d=32, h=4, dk=8, r=12, norm_mode=norm_mode)
    rng = np.random.default_rng(5)
    W = rand_layer(rng, cfg)
    Rh = rng.standard_normal((20, cfg.d))
    Rc = rng.standard_normal((3, cfg.d))
    a = O.mla_layer(Rh, Rc, 7, W, cfg, absorbed=False)
    b = O.mla_layer(Rh, Rc, 7, W, cfg, absorbed=True)
    assert rel(a[0], b[0]) < 1e-12 and rel(a[1], b[1]) < 1e-12


def test_softmax_rows_sum_to_one_and_mask_respected():
    cfg = tiny_cfg(d=16, h=4, dk=4, r=5)
    rng = np.random.default_rng(6)
    W = rand_layer(rng, cfg)
    K, n, nc = 11, 6, 3
    _, p = O.mla_layer(rng.standard_normal((K, 16)), rng.standard_normal((nc, 16)),
                       n, W, cfg, return_probs=True)
    assert np.allclose(p.sum(axis=-1), 1.0, atol=1e-14, rtol=0)
    for i in range(n):          # history row i sits at key position K-n+i
        assert np.all(p[:, i, K - n + i + 1:] == 0)
        assert np.all(p[:, i, :K - n + i + 1] > 0)
    assert np.all(p[:, n:, :] > 0)


def test_latent_attention_matches_torch_sdpa():
    """Special case reducing to a library routine: per head, the latent core
    is single-head attention with key = value = C (torch SDPA, bool mask)."""
    rng = np.random.default_rng(7)
    B, h, r, nc = 3, 2, 5, 2
    K = np.array([4, 9, 1])
    n = np.array([4, 3, 1])
    kv_off = np.concatenate([[0], np.cumsum(K)])
    hq_off = np.concatenate([[0], np.cumsum(n)])
    Mtot = hq_off[-1] + B * nc
    q = rng.standard_normal((Mtot, h, r))
    C = rng.standard_normal((kv_off[-1], r))
    scale = 0.37
    out, lse = O.latent_attention(q, C, kv_off, hq_off, nc, scale)
    for u in range(B):
        rows = list(range(B * nc + hq_off[u], B * nc + hq_off[u + 1])) + \
            list(range(u * nc, (u + 1) * nc))
        Cu = torch.tensor(C[kv_off[u]:kv_off[u + 1]])
        allowed = torch.tensor(O.history_query_mask(K[u], n[u], nc))
        for hh in range(h):
            qt = torch.tensor(q[rows, hh, :])
            ref = F.scaled_dot_product_attention(qt[None], Cu[None], Cu[None],
                                                 attn_mask=allowed[None],
                                                 scale=scale)[0]
            assert rel(out[rows, hh, :], ref.numpy()) < 1e-12
            s = (qt @ Cu.T) * scale
            s = s.masked_fill(~allowed, -math.inf)
            assert rel(lse[rows, hh], torch.logsumexp(s, -1).numpy()) < 1e-12


def test_one_key_history_returns_that_row():
    rng = np.random.default_rng(8)
    C = rng.standard_normal((1, 6))
    q = rng.standard_normal((1 + 3, 2, 6)) * 5
    out, lse = O.latent_attention(q, C, [0, 1], [0, 1], 3, 0.5)
    assert np.array_equal(out, np.broadcast_to(C[0], out.shape))
    # layer level: every query of a one-key history has probability 1 on it
    cfg = tiny_cfg(d=16, h=4, dk=4, r=5)
    W = rand_layer(rng, cfg)
    _, p = O.mla_layer(rng.standard_normal((1, 16)), rng.standard_normal((3, 16)),
                       1, W, cfg, return_probs=True)
    assert np.array_equal(p, np.ones_like(p))


def test_identical_keys_long_history_return_that_row():
    rng = np.random.default_rng(9)
    row = rng.standard_normal(8)
    C = np.tile(row, (1600, 1))
    n = 50
    q = rng.standard_normal((n + 2, 3, 8)) * 4
    out, lse = O.latent_attention(q, C, [0, 1600], [0, n], 2, 1.0 / 8)
    assert np.max(np.abs(out - row)) < 1e-12
    # lse = s + log(number of allowed keys) since all scores are equal;
    # rows: the 2 candidates first, then the n history queries
    s = (q @ row) / 8
    cnt = np.concatenate([[1600, 1600], 1600 - n + np.arange(n) + 1])
    assert rel(lse, s + np.log(cnt)[:, None]) < 1e-12


def test_causality_future_rows_do_not_leak():
    cfg = tiny_cfg(d=16, h=4, dk=4, r=5)
    rng = np.random.default_rng(10)
    W = rand_layer(rng, cfg)
    K = 10
    Rh = rng.standard_normal((K, 16))
    Rc = rng.standard_normal((2, 16))
    a, ac = O.mla_layer(Rh, Rc, K, W, cfg)
    Rh2 = Rh.copy()
    Rh2[6:] += rng.standard_normal((4, 16))
    b, bc = O.mla_layer(Rh2, Rc, K, W, cfg)
    assert np.array_equal(a[:6], b[:6])
    assert not np.allclose(a[6:], b[6:]) and not np.allclose(ac, bc)


def test_candidate_independence():
    cfg = tiny_cfg(d=16, h=4, dk=4, r=5)
    rng = np.random.default_rng(11)
    W = rand_layer(rng, cfg)
    Rh = rng.standard_normal((9, 16))
    Rc = rng.standard_normal((4, 16))
    a, ac = O.mla_layer(Rh, Rc, 5, W, cfg)
    b, bc = O.mla_layer(Rh, Rc[1:3], 5, W, cfg)
    c, cc = O.mla_layer(Rh, np.zeros((0, 16)), 5, W, cfg)
    assert rel(ac[1:3], bc) < 1e-13
    assert rel(a, b) < 1e-13 and rel(a, c) < 1e-13


# ------------------------------------------------------- pyramid

@pytest.mark.parametrize("n", [0, 3, 8])
def test_extraction_equals_full_then_slice(n):
    cfg = tiny_cfg(d=16, h=4, dk=4, r=5)
    rng = np.random.default_rng(12 + n)
    W = rand_layer(rng, cfg)
    Rh = rng.standard_normal((8, 16))
    Rc = rng.standard_normal((3, 16))
    fh, fc = O.mla_layer(Rh, Rc, 8, W, cfg)     # n_l = K: full attention
    eh, ec = O.mla_layer(Rh, Rc, n, W, cfg)
    assert eh.shape[0] == n
    if n:
        assert rel(eh, fh[8 - n:]) < 1e-13
    assert rel(ec, fc) < 1e-13


def _golden_schedules():
    out = []
    with open(os.path.join(GOLDEN, "pyramid_schedules.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = line.split(":")
            out.append((lhs.split(), [int(v) for v in rhs.split()]))
    return out


@pytest.mark.parametrize("lhs,expect", _golden_schedules())
def test_pyramid_schedules_golden(lhs, expect):
    kind = lhs[0]
    if kind == "halving":
        F_, N, L = map(int, lhs[1:])
        rule = synth.PyramidRule("halving", floor=F_)
    elif kind == "geometric":
        S, E, N, L = map(int, lhs[1:])
        rule = synth.PyramidRule("geometric", start=S, end=E)
    else:
        vals = tuple(int(v) for v in lhs[1].split(","))
        N, L = int(lhs[2]), int(lhs[3])
        rule = synth.PyramidRule("fixed", vals)
    keep = O.pyramid_counts(rule, [L], N)[:, 0]
    assert list(keep) == expect
    cfg = tiny_cfg(N=N, pyramid=rule)
    assert brute.keep_counts(cfg, L) == expect


def test_compaction_indices_exact():
    rng = np.random.default_rng(13)
    lens = rng.integers(1, 40, 17)
    off = np.concatenate([[0], np.cumsum(lens)])
    keep = np.array([rng.integers(0, l + 1) for l in lens])
    vals = rng.standard_normal((off[-1], 5))
    out, noff, src = O.compact(vals, off, keep)
    expect = np.concatenate([off[u] + np.arange(lens[u] - keep[u], lens[u])
                             for u in range(17)])
    assert np.array_equal(src, expect)
    assert np.array_equal(noff, np.concatenate([[0], np.cumsum(keep)]))
    assert np.array_equal(out, vals[expect])
    with pytest.raises(ValueError):
        O.compact(vals, off, lens + 1)


def test_jagged_lengths_of_c4_workload():
    L = synth.generate(synth.get_config("c4"))["inputs"]["lengths"]
    assert int(L.sum()) == 117132 and L.min() == 203 and L.max() == 1597


def test_unmasked_pairs_closed_form():
    """Pairs of a layer with K keys, n history queries, n_q candidates:
    n*(K-n) + n*(n+1)/2 + n_q*K (causal staircase plus full candidate rows)."""
    cfg = tiny_cfg(N=3, n_q=2, pyramid=synth.PyramidRule("fixed", (30, 17, 4)))
    L = np.array([30, 25, 3])
    keep = O.pyramid_counts(cfg.pyramid, L, 3)
    got = O.unmasked_pairs(cfg, L)
    exp = np.zeros(3, dtype=np.int64)
    for u in range(3):
        K = L[u]
        for l in range(3):
            n = keep[l, u]
            exp[l] += n * (K - n) + n * (n + 1) // 2 + 2 * K
            K = n
    assert np.array_equal(got, exp)


# ------------------------------------------------------- whole stack

BRUTE_CASES = [
    dict(N=1, n_q=0, d_c=0, pyramid=synth.PyramidRule("fixed", (8,)), L=(1, 2, 8)),
    dict(N=2, n_q=1, d_c=3, pyramid=synth.PyramidRule("fixed", (5, 3)), L=(5, 2, 8)),
    dict(N=3, n_q=2, d_c=3, pyramid=synth.PyramidRule("halving", floor=2), L=(1, 3, 8)),
    dict(N=3, n_q=2, d_c=0, pyramid=synth.PyramidRule("geometric", start=8, end=2),
         L=(8, 5, 2)),
    dict(N=2, n_q=2, d_c=3, pyramid=synth.PyramidRule("fixed", (8, 0)), L=(8, 3, 1)),
    dict(N=2, n_q=1, d_c=3, pyramid=synth.PyramidRule("fixed", (4, 2)), L=(5, 4, 2),
         n_seeds=2, d_out=5),
    dict(N=2, n_q=2, d_c=3, pyramid=synth.PyramidRule("fixed", (4, 2)), L=(6, 4, 3),
         norm_mode="post", latent_norm=False),
    dict(N=2, n_q=2, d_c=3, pyramid=synth.PyramidRule("fixed", (5, 3)), L=(5, 2, 8),
         r_q=5),
    dict(N=2, n_q=1, d_c=3, pyramid=synth.PyramidRule("fixed", (4, 2)), L=(5, 4, 2),
         n_seeds=2, d_out=5, r_q=3, norm_mode="post"),
]


@pytest.mark.parametrize("case", BRUTE_CASES)
def test_forward_matches_brute_force(case):
    case = dict(case)
    lengths = case.pop("L")
    cfg = tiny_cfg(**case)
    rng = np.random.default_rng(sum(lengths) + cfg.N)
    W = {"layers": [rand_layer(rng, cfg) for _ in range(cfg.N)]}
    if cfg.n_q:
        W["W_q"] = rng.standard_normal((cfg.d + cfg.d_c, cfg.d)) / 3
    if cfg.n_seeds:
        W["seeds"] = rng.standard_normal((cfg.n_seeds, cfg.d))
        W["readout"] = rand_layer(rng, cfg)
        W["W_p"] = rng.standard_normal((cfg.n_seeds * cfg.d, cfg.d_out)) / 4
    off = np.concatenate([[0], np.cumsum(lengths)])
    hist = rng.standard_normal((off[-1], cfg.d))
    cand = rng.standard_normal((3 * cfg.n_q, cfg.d)) if cfg.n_q else None
    ctx = rng.standard_normal((3, cfg.d_c)) if cfg.d_c else None
    res = O.forward(cfg, W, hist, off, cand, ctx)
    resa = O.forward(cfg, W, hist, off, cand, ctx, absorbed=True)
    for u in range(3):
        bh, bc, be = brute.forward_user(
            cfg, W, hist[off[u]:off[u + 1]],
            cand[u * cfg.n_q:(u + 1) * cfg.n_q] if cfg.n_q else None,
            ctx[u] if cfg.d_c else None)
        for got in (res, resa):
            if len(bh):
                assert rel(got["hist"][u], bh) < 1e-12
            else:
                assert got["hist"][u].shape[0] == 0
            if len(bc):
                assert rel(got["cand"][u], bc) < 1e-12
            if cfg.n_seeds:
                assert rel(got["emb"][u], be) < 1e-12


def test_user_independence_and_subset():
    cfg = tiny_cfg(N=2, pyramid=synth.PyramidRule("halving", floor=2))
    rng = np.random.default_rng(21)
    W = {"layers": [rand_layer(rng, cfg) for _ in range(2)],
         "W_q": rng.standard_normal((cfg.d + cfg.d_c, cfg.d)) / 3}
    lengths = [7, 1, 4]
    off = np.concatenate([[0], np.cumsum(lengths)])
    hist = rng.standard_normal((off[-1], cfg.d))
    cand = rng.standard_normal((3 * cfg.n_q, cfg.d))
    ctx = rng.standard_normal((3, cfg.d_c))
    full = O.forward(cfg, W, hist, off, cand, ctx)
    for u in range(3):
        one = O.forward(cfg, W, hist[off[u]:off[u + 1]], [0, lengths[u]],
                        cand[u * 2:(u + 1) * 2], ctx[u:u + 1])
        assert np.array_equal(one["hist"][0], full["hist"][u])
        assert np.array_equal(one["cand"][0], full["cand"][u])
    sub = O.forward(cfg, W, hist, off, cand, ctx, users=[2])
    assert np.array_equal(sub["hist"][0], full["hist"][2])


def test_token_embed_is_row_plus_projection():
    rng = np.random.default_rng(22)
    T = rng.standard_normal((10, 4))
    S = rng.standard_normal((10, 3))
    Ws = rng.standard_normal((3, 4))
    ref = torch.tensor(T) + torch.tensor(S) @ torch.tensor(Ws)
    assert rel(O.token_embed(T, S, Ws), ref.numpy()) < 1e-14


def test_c1_digest_regression():
    """Regression only (not a pin): the fp64 c1 output digest written by
    tests/golden/make_golden.py from the oracle after the pins above pass."""
    path = os.path.join(GOLDEN, "c1_digest.txt")
    vals = {}
    with open(path) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            k, v = line.split("=")
            vals[k.strip()] = float(v)
    cfg = synth.get_config("c1")
    p = synth.generate(cfg)
    I = p["inputs"]
    res = O.forward(cfg, p["weights"], I["hist"], I["offsets"], I.get("cand"),
                    I.get("ctx"))
    H = np.concatenate(res["hist"])
    C = np.concatenate(res["cand"])
    assert abs(H.sum() - vals["hist_sum"]) < 1e-9
    assert abs(np.abs(H).sum() - vals["hist_abs_sum"]) < 1e-9
    assert abs(C.sum() - vals["cand_sum"]) < 1e-9
    assert abs(np.abs(C).sum() - vals["cand_abs_sum"]) < 1e-9
