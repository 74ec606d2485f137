"""GPU parity of llatte_attn_sublayer_backward (the attention sublayer of a
pre-norm MLA layer: norms, latent projection, query, key/value absorption,
masked softmax, output projection, residual) against the oracle's
attention_sublayer_backward in fp64 (non-absorbed form), per user, with the
weight gradients summed over users: jagged users with candidates, latent
norm on and off, r = 64 and 128, and two users of the upstream layer-1
shape (1600 keys and query rows, d = 512, 8 x 64 heads, r = 128).

Tolerance, per gradient tensor: max|g - r| <= 1.5e-2 max|r| and
RMS(g - r) <= 1e-2 RMS(r). The max/RMS bar of the forward does not fit
these gradients: each is dominated by a few rows (the early query rows of a
causal user attend few keys, so their attention outputs and gradients are
much larger than the rest), and an fp64 emulation of this path's bf16
rounding points (operands of every product, the recomputed forward
included; test_sublayer_rounding.py) already reaches 2.1-2.9 % of the RMS
on the first three shapes below while staying within 0.55 % of the largest
entry and 0.56 % in RMS.
"""
import math
from types import SimpleNamespace

import numpy as np
import pytest

import synth
from oracle import llatte_oracle as O
from synth.sublayer import sublayer_case

pytestmark = pytest.mark.gpu

KEYS = ("g1", "w_dkv", "g_c", "w_uq", "w_uk", "w_uv", "w_o")
ONAME = {"g1": "g1", "w_dkv": "W_dkv", "g_c": "g_c", "w_uq": "W_uq", "w_uk": "W_uk",
         "w_uv": "W_uv", "w_o": "W_o"}


def _errs(g, r):
    """(max|g - r| / max|r|, RMS(g - r) / RMS(r))"""
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    return (float(np.max(np.abs(g - r)) / np.max(np.abs(r))),
            float(np.sqrt(np.mean((g - r) ** 2)) / np.sqrt(np.mean(r ** 2))))


def run_case(d, h, dk, r, n_cand, K, n, latent_norm, seed=0):
    import torch
    from target_aware_latent_amd import llatte as C
    B = len(K)
    cfg = SimpleNamespace(d=d, h=h, dk=dk, r=r, eps=1e-6, latent_norm=latent_norm, norm_mode="pre")
    W, Rh, Rc, dout, kv, hq = sublayer_case(d, h, dk, r, n_cand, K, n, seed)
    Mtot = dout.shape[0]
    Ktot = int(kv[-1])

    dev = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda().to(dt)
    desc = C.llatte_attn_sublayer_desc(d, h, dk, r, n_cand, C.LLATTE_BF16, int(latent_norm), 1e-6)
    wd = {"g1": dev(W["g1"]), "g_c": dev(W["g_c"])}
    for k in ("w_dkv", "w_uq", "w_uk", "w_uv", "w_o"):
        wd[k] = dev(W[ONAME[k]], torch.bfloat16)
    nan = lambda *s: torch.full(s, float("nan"), device="cuda")
    gd = {"g1": nan(d), "w_dkv": nan(d, r), "g_c": nan(r), "w_uq": nan(d, h * dk),
          "w_uk": nan(r, h * dk), "w_uv": nan(r, h * dk), "w_o": nan(h * dk, d)}
    d_r_kv = nan(Ktot, d)
    d_r_c = nan(max(B * n_cand, 1), d)
    ws = torch.empty(C.llatte_attn_sublayer_backward_workspace_size(desc, B, Mtot, Ktot),
                     dtype=torch.uint8, device="cuda")
    r_c = dev(np.concatenate(Rc)) if n_cand else None
    C.llatte_attn_sublayer_backward(desc, wd, dev(np.concatenate(Rh)), r_c,
                                    torch.from_numpy(kv).cuda(), torch.from_numpy(hq).cuda(), B, Mtot,
                                    Ktot, int(max(K)), dev(dout), d_r_kv,
                                    d_r_c if n_cand else None, gd, ws)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in gd.items()}
    got_rkv = d_r_kv.cpu().numpy()
    got_rc = d_r_c.cpu().numpy()

    # oracle per user; d_out rows: candidates user-major, then history rows
    nc = B * n_cand
    ref = {ONAME[k]: 0.0 for k in KEYS}
    ref_rkv, ref_rc = [], []
    for u in range(B):
        dq_u = np.concatenate([dout[nc + hq[u]:nc + hq[u + 1]], dout[u * n_cand:(u + 1) * n_cand]])
        dRh, dRc, g = O.attention_sublayer_backward(Rh[u].astype(np.float64), Rc[u].astype(np.float64),
                                                    int(n[u]), W, cfg, dq_u.astype(np.float64))
        ref_rkv.append(dRh)
        ref_rc.append(dRc)
        for k, v in g.items():
            ref[k] = ref[k] + v
    return got, got_rkv, got_rc, ref, np.concatenate(ref_rkv), np.concatenate(ref_rc)


CASES = [
    # d, h, dk, r, n_cand, K per user, n per user, latent_norm
    (64, 2, 32, 64, 3, [20, 70, 1], [20, 35, 1], True),
    (128, 4, 32, 128, 0, [130, 65], [130, 64], False),
    (256, 4, 64, 128, 2, [300, 200, 90], [150, 200, 0], True),
    (512, 8, 64, 128, 0, [1600, 1600], [1600, 1600], True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"d{c[0]}-h{c[1]}-r{c[3]}-nc{c[4]}-B{len(c[5])}-ln{int(c[7])}")
def test_sublayer_backward_matches_oracle(case):
    print(f"attention sublayer backward {case}", flush=True)
    got, got_rkv, got_rc, ref, ref_rkv, ref_rc = run_case(*case)
    latent_norm, n_cand = case[7], case[4]
    assert np.isfinite(got_rkv).all()
    pairs = {"d_r_kv": (got_rkv, ref_rkv)}
    if n_cand:
        pairs["d_r_cand"] = (got_rc[:len(ref_rc)], ref_rc)
    for k in KEYS:
        if k == "g_c" and not latent_norm:
            continue
        pairs[k] = (got[k], ref[ONAME[k]])
    errs = {k: _errs(*v) for k, v in pairs.items()}
    print({k: "%.2e / %.2e" % e for k, e in errs.items()}, flush=True)
    bad = {k: e for k, e in errs.items() if e[0] > 1.5e-2 or e[1] > 1e-2}
    assert not bad, f"errors above the bar: {bad}"


def test_no_query_rows_zero_every_gradient():
    import torch
    from target_aware_latent_amd import llatte as C
    d, h, dk, r = 64, 2, 32, 64
    desc = C.llatte_attn_sublayer_desc(d, h, dk, r, 0, C.LLATTE_BF16, 1, 1e-6)
    kv = torch.tensor([0, 5, 12], dtype=torch.int32, device="cuda")
    hq = torch.zeros(3, dtype=torch.int32, device="cuda")
    one = lambda *s, dt=torch.float32: torch.ones(s, device="cuda").to(dt)
    wd = {"g1": one(d), "g_c": one(r), "w_dkv": one(d, r, dt=torch.bfloat16),
          "w_uq": one(d, h * dk, dt=torch.bfloat16), "w_uk": one(r, h * dk, dt=torch.bfloat16),
          "w_uv": one(r, h * dk, dt=torch.bfloat16), "w_o": one(h * dk, d, dt=torch.bfloat16)}
    nan = lambda *s: torch.full(s, float("nan"), device="cuda")
    gd = {"g1": nan(d), "w_dkv": nan(d, r), "g_c": nan(r), "w_uq": nan(d, h * dk),
          "w_uk": nan(r, h * dk), "w_uv": nan(r, h * dk), "w_o": nan(h * dk, d)}
    d_r_kv = nan(12, d)
    ws = torch.empty(max(C.llatte_attn_sublayer_backward_workspace_size(desc, 2, 0, 12), 256),
                     dtype=torch.uint8, device="cuda")
    C.llatte_attn_sublayer_backward(desc, wd, one(12, d), None, kv, hq, 2, 0, 12, 7, None, d_r_kv,
                                    None, gd, ws)
    torch.cuda.synchronize()
    for t in [d_r_kv] + list(gd.values()):
        assert torch.count_nonzero(t).item() == 0


def test_full_upstream_layer_one():
    # the bench's launch configuration for layer 1 (64 users x 1600 rows,
    # d = 512, 8 x 64 heads, r = 128): the input-row gradients of sampled
    # users against the oracle one by one (users are independent), and the
    # weight gradients, which sum over users, against the sum of the GPU's
    # own single-user runs of every user (a property that holds at any size),
    # after the weight gradients of a two-user batch against the oracle
    import torch
    from target_aware_latent_amd import llatte as C
    B, L, d, h, dk, r = 64, 1600, 512, 8, 64, 128
    print("attention sublayer backward 64 x 1600", flush=True)
    rng = np.random.default_rng(8)
    cfg = SimpleNamespace(d=d, h=h, dk=dk, r=r, eps=1e-6, latent_norm=True, norm_mode="pre")
    W = {"g1": (1 + 0.1 * rng.standard_normal(d)).astype(np.float32).astype(np.float64),
         "g_c": (1 + 0.1 * rng.standard_normal(r)).astype(np.float32).astype(np.float64)}
    for k, shp, fan in (("W_dkv", (d, r), d), ("W_uq", (d, h * dk), d), ("W_uk", (r, h * dk), r),
                        ("W_uv", (r, h * dk), r), ("W_o", (h * dk, d), h * dk)):
        W[k] = np.asarray(synth.round_bf16(rng.standard_normal(shp) / math.sqrt(fan)),
                          np.float32).astype(np.float64)
    R = rng.standard_normal((B * L, d)).astype(np.float32)
    dout = rng.standard_normal((B * L, d)).astype(np.float32)
    dev = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda().to(dt)
    desc = C.llatte_attn_sublayer_desc(d, h, dk, r, 0, C.LLATTE_BF16, 1, 1e-6)
    wd = {"g1": dev(W["g1"]), "g_c": dev(W["g_c"])}
    for k in ("w_dkv", "w_uq", "w_uk", "w_uv", "w_o"):
        wd[k] = dev(W[ONAME[k]], torch.bfloat16)
    shapes = {"g1": (d,), "w_dkv": (d, r), "g_c": (r,), "w_uq": (d, h * dk), "w_uk": (r, h * dk),
              "w_uv": (r, h * dk), "w_o": (h * dk, d)}
    Rd, dod = dev(R), dev(dout)

    def run(b0, nb, rows=None, grads=None):
        off = torch.from_numpy((np.arange(nb + 1) * L).astype(np.int32)).cuda()
        gd = {k: torch.empty(s, device="cuda") for k, s in shapes.items()}
        drkv = torch.empty((nb * L, d), device="cuda")
        ws = torch.empty(C.llatte_attn_sublayer_backward_workspace_size(desc, nb, nb * L, nb * L),
                         dtype=torch.uint8, device="cuda")
        if rows is None:
            rows, grads = Rd[b0 * L:(b0 + nb) * L], dod[b0 * L:(b0 + nb) * L]
        C.llatte_attn_sublayer_backward(desc, wd, rows, None, off, off, nb, nb * L, nb * L, L,
                                        grads, drkv, None, gd, ws)
        return drkv, gd

    drkv, gd = run(0, B)
    torch.cuda.synchronize()
    drkv = drkv.cpu().numpy()
    assert np.isfinite(drkv).all()
    sampled = (0, 41)
    ref_sum = {}
    for u in sampled:
        s = slice(u * L, (u + 1) * L)
        ref, _, g = O.attention_sublayer_backward(R[s].astype(np.float64), np.zeros((0, d)), L, W,
                                                  cfg, dout[s].astype(np.float64))
        e = _errs(drkv[s], ref)
        assert e[0] <= 1.5e-2 and e[1] <= 1e-2, f"user {u} d_r_kv {e}"
        for k, v in g.items():
            ref_sum[k] = ref_sum.get(k, 0.0) + v
    # the weight gradients of a batch of the sampled users alone against the
    # oracle's sum over the same users
    pick = np.concatenate([np.arange(u * L, (u + 1) * L) for u in sampled])
    _, g2 = run(0, len(sampled), dev(R[pick]), dev(dout[pick]))
    torch.cuda.synchronize()
    for k in shapes:
        e = _errs(g2[k].cpu().numpy(), ref_sum[ONAME[k]])
        assert e[0] <= 1.5e-2 and e[1] <= 1e-2, f"users {sampled} {k} {e}"
    total = {k: torch.zeros(s, device="cuda", dtype=torch.float64) for k, s in shapes.items()}
    for u in range(B):
        _, gu = run(u, 1)
        for k in shapes:
            total[k] += gu[k].double()
    torch.cuda.synchronize()
    for k in shapes:
        a, b = gd[k].double().cpu().numpy(), total[k].cpu().numpy()
        e = float(np.max(np.abs(a - b)) / np.max(np.abs(b)))
        assert e <= 1e-5, f"{k}: batch vs sum of single-user runs {e:.2e}"
