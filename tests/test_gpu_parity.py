"""Parity of the HIP library (through its C ABI) with the CPU oracle.

Tolerances (from the build contract): fp32 path max |g - r| / max(|r|, RMS(r))
<= 1e-4 per element; bf16 path max |g - r| / RMS(r) <= 2e-2 per output
tensor; integer and index outputs bit-exact. The oracle runs in fp64 on the
same (bf16-rounded where applicable) inputs.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import synth
from oracle import llatte_oracle as O

pytestmark = pytest.mark.gpu

F32_TOL = 1e-4
BF16_TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from target_aware_latent_amd import llatte
    llatte.lib()
    yield
    torch.cuda.synchronize()


def L():
    from target_aware_latent_amd import llatte
    return llatte


def err_f32(g, r):
    g, r = np.asarray(g, np.float64), np.asarray(r, np.float64)
    rms = math.sqrt(float(np.mean(r * r))) if r.size else 1.0
    return float(np.max(np.abs(g - r) / np.maximum(np.abs(r), rms))) if r.size else 0.0


def err_bf16(g, r):
    g, r = np.asarray(g, np.float64), np.asarray(r, np.float64)
    if r.size == 0:
        return 0.0
    rms = math.sqrt(float(np.mean(r * r)))
    return float(np.max(np.abs(g - r)) / rms)


def check(g, r, dtype, what=""):
    e = err_f32(g, r) if dtype == "f32" else err_bf16(g, r)
    tol = F32_TOL if dtype == "f32" else BF16_TOL
    print(f"  {what}: err={e:.3e} (tol {tol})", flush=True)
    assert e <= tol, f"{what}: error {e:.3e} > {tol}"
    return e


def dev(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dtype)


def idev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")


# ---------------------------------------------------------------- pyramid

@pytest.mark.parametrize("rule,N", [
    (synth.PyramidRule("halving", floor=64), 4),
    (synth.PyramidRule("geometric", start=1600, end=50), 12),
    (synth.PyramidRule("fixed", (400, 200, 100)), 3),
    (synth.PyramidRule("fixed", (30, 30, 7, 0)), 4),
])
def test_pyramid_counts_device(rule, N):
    from target_aware_latent_amd.model import make_desc
    rng = np.random.default_rng(11)
    lengths = np.concatenate([[1, 2, 63, 64, 65, 1600], rng.integers(1, 2000, 3000)])
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    cfg = synth.Config("x", B=1, L=1, len_range=None, d=8, h=1, dk=8, r=8,
                       n_q=0, d_c=0, N=N, pyramid=rule, dtype="f32")
    keep = torch.empty(N * lengths.size, dtype=torch.int32, device="cuda")
    L().llatte_pyramid_counts(make_desc(cfg).pyramid, N, idev(off), lengths.size, keep)
    got = keep.cpu().numpy().reshape(N, -1)
    assert np.array_equal(got, O.pyramid_counts(rule, lengths, N))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("row_elems", [8, 64, 512, 1030])
def test_pyramid_compact_bit_exact(dt, row_elems):
    rng = np.random.default_rng(row_elems)
    lengths = np.concatenate([[1, 5, 64], rng.integers(1, 300, 40)])
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    keep = np.array([rng.integers(0, l + 1) for l in lengths])
    keep[0], keep[1], keep[2] = 1, 0, 64
    vals = rng.standard_normal((off[-1], row_elems)).astype(np.float32)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    v = dev(vals, tdt)
    out = torch.zeros(max(int(keep.sum()), 1), row_elems, dtype=tdt, device="cuda")
    noff = torch.empty(lengths.size + 1, dtype=torch.int32, device="cuda")
    src = torch.empty(max(int(keep.sum()), 1), dtype=torch.int32, device="cuda")
    code = L().LLATTE_BF16 if dt == "bf16" else L().LLATTE_F32
    L().llatte_pyramid_compact(v, row_elems, code, idev(off), lengths.size,
                               int(off[-1]), idev(keep), out, noff, src)
    ref_vals, ref_off, ref_src = O.compact(v.float().cpu().numpy(), off, keep)
    n = int(keep.sum())
    assert np.array_equal(noff.cpu().numpy(), ref_off)
    assert np.array_equal(src.cpu().numpy()[:n], ref_src)
    assert torch.equal(out[:n].float().cpu(), torch.from_numpy(ref_vals))


def test_pyramid_compact_many_users():
    """3000 users: more than the offsets scan's 1024 threads, so each thread
    scans a chunk of users; offsets, source rows and values bit-exact."""
    rng = np.random.default_rng(7)
    lengths = rng.integers(1, 20, 3000)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    keep = np.array([rng.integers(0, l + 1) for l in lengths])
    vals = rng.standard_normal((off[-1], 8)).astype(np.float32)
    v = dev(vals, torch.float32)
    n = int(keep.sum())
    out = torch.zeros(n, 8, device="cuda")
    noff = torch.empty(lengths.size + 1, dtype=torch.int32, device="cuda")
    src = torch.empty(n, dtype=torch.int32, device="cuda")
    L().llatte_pyramid_compact(v, 8, L().LLATTE_F32, idev(off), lengths.size, int(off[-1]),
                               idev(keep), out, noff, src)
    ref_vals, ref_off, ref_src = O.compact(vals, off, keep)
    assert np.array_equal(noff.cpu().numpy(), ref_off)
    assert np.array_equal(src.cpu().numpy(), ref_src)
    assert torch.equal(out.cpu(), torch.from_numpy(ref_vals))


def test_pyramid_compact_full_size_upstream():
    """Upstream shape: 64 users x 1600 rows of 512 floats, keep the last 800."""
    B, Lu, d = 64, 1600, 512
    off = (np.arange(B + 1) * Lu).astype(np.int32)
    keep = np.full(B, 800)
    v = torch.randn(B * Lu, d, device="cuda", generator=torch.Generator("cuda").manual_seed(0))
    out = torch.empty(B * 800, d, device="cuda")
    noff = torch.empty(B + 1, dtype=torch.int32, device="cuda")
    src = torch.empty(B * 800, dtype=torch.int32, device="cuda")
    L().llatte_pyramid_compact(v, d, L().LLATTE_F32, idev(off), B, B * Lu,
                               idev(keep), out, noff, src)
    exp_src = np.concatenate([u * Lu + np.arange(800, 1600) for u in range(B)])
    assert np.array_equal(src.cpu().numpy(), exp_src)
    assert torch.equal(out, v[torch.from_numpy(exp_src).cuda().long()])


# ---------------------------------------------------------------- attention

def run_attention(dt, h, r, K, n, n_cand, scale=None, seed=0, q=None, C=None):
    rng = np.random.default_rng(seed)
    K, n = np.asarray(K), np.asarray(n)
    B = K.size
    kv_off = np.concatenate([[0], np.cumsum(K)]).astype(np.int32)
    hq_off = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    Mtot = int(B * n_cand + hq_off[-1])
    if q is None:
        q = rng.standard_normal((Mtot, h, r)) * 0.5
    if C is None:
        C = rng.standard_normal((kv_off[-1], r))
    if dt == "bf16":
        q, C = synth.round_bf16(q), synth.round_bf16(C)
    q = np.asarray(q, np.float32)
    C = np.asarray(C, np.float32)
    scale = scale or 1.0 / math.sqrt(64)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    code = L().LLATTE_BF16 if dt == "bf16" else L().LLATTE_F32
    ad = L().llatte_attn_desc(h, r, n_cand, code, scale)
    ws = torch.empty(L().llatte_mla_attention_workspace_size(ad, B, Mtot, int(kv_off[-1])),
                     dtype=torch.uint8, device="cuda")
    out = torch.full((max(Mtot, 1), h, r), float("nan"), device="cuda")
    lse = torch.full((max(Mtot, 1), h), float("nan"), device="cuda")
    L().llatte_mla_attention(ad, dev(q, tdt), dev(C, tdt), idev(kv_off), idev(hq_off),
                             B, Mtot, int(kv_off[-1]), out, lse, ws)
    ref, ref_lse = O.latent_attention(q.astype(np.float64), C.astype(np.float64),
                                      kv_off, hq_off, n_cand, scale)
    return out[:Mtot].float().cpu().numpy(), lse[:Mtot].cpu().numpy(), ref, ref_lse, q, C, kv_off, hq_off


ATTN_CASES = [
    # dtype, h, r, K per user, n per user, n_cand
    ("f32", 2, 16, [32, 32, 32, 32], [32, 32, 32, 32], 4),
    ("f32", 4, 64, [1, 65, 130, 7], [1, 30, 130, 0], 3),
    ("f32", 3, 40, [200, 5], [77, 5], 0),
    ("bf16", 4, 64, [1, 63, 64, 65, 200, 333], [1, 63, 10, 65, 0, 200], 16),
    ("bf16", 8, 128, [1600, 129, 1], [1600, 64, 1], 0),
    ("bf16", 8, 128, [700, 50], [300, 50], 5),
    ("bf16", 16, 256, [300, 1, 97], [150, 1, 97], 16),
    ("bf16", 2, 64, [90, 260], [90, 17], 2),
    ("bf16", 16, 128, [100, 70], [33, 70], 1),
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=lambda c: f"{c[0]}-h{c[1]}-r{c[2]}-nc{c[5]}")
def test_latent_attention_matches_oracle(case):
    dt, h, r, K, n, nc = case
    print(f"attention {case}", flush=True)
    out, lse, ref, ref_lse, *_ = run_attention(dt, h, r, K, n, nc)
    check(out, ref, dt, "out")
    assert np.max(np.abs(lse - ref_lse)) < (1e-4 if dt == "f32" else 2e-3)


def test_softmax_rows_sum_to_one_via_lse():
    """sum_j exp(scale * q . C_j - lse) = 1 for every row, scores recomputed
    in fp64 from the (bf16) inputs and the GPU's lse."""
    K, n, nc, h, r = [500, 64], [250, 64], 4, 8, 128
    out, lse, ref, ref_lse, q, C, kv_off, hq_off = run_attention("bf16", h, r, K, n, nc)
    scale = 1.0 / 8
    B = 2
    for u in range(B):
        Cu = C[kv_off[u]:kv_off[u + 1]].astype(np.float64)
        Ku = Cu.shape[0]
        nu = hq_off[u + 1] - hq_off[u]
        rows = list(range(u * nc, (u + 1) * nc)) + \
            list(range(B * nc + hq_off[u], B * nc + hq_off[u + 1]))
        allowed = np.concatenate([np.ones((nc, Ku), bool),
                                  O.history_query_mask(Ku, nu, 0)])
        for hh in range(h):
            s = (q[rows, hh, :].astype(np.float64) @ Cu.T) * scale
            tot = np.where(allowed, np.exp(s - lse[rows, hh][:, None]), 0).sum(1)
            assert np.max(np.abs(tot - 1)) < 2e-3


@pytest.mark.parametrize("dt,h,r", [("bf16", 8, 128), ("bf16", 4, 64), ("f32", 2, 16)])
def test_one_key_history_returns_that_row(dt, h, r):
    rng = np.random.default_rng(5)
    out, lse, ref, *_ = run_attention(dt, h, r, [1, 1, 1], [1, 0, 1], 3)
    _, _, _, _, q, C, _, _ = run_attention(dt, h, r, [1, 1, 1], [1, 0, 1], 3)
    # candidate rows of user u and its one history row equal C_u exactly
    for u in range(3):
        for i in [u * 3, u * 3 + 1, u * 3 + 2]:
            assert np.array_equal(out[i], np.broadcast_to(C[u], (h, r)))


def test_identical_keys_over_many_tiles():
    rng = np.random.default_rng(6)
    row = synth.round_bf16(rng.standard_normal(128))
    C = np.tile(row, (1600, 1))
    out, *_ = run_attention("bf16", 8, 128, [1600], [1600], 2, C=C)
    assert np.max(np.abs(out - row)) <= 1e-2 * np.max(np.abs(row))


# ---------------------------------------------------------------- token build

@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_token_embed_matches_oracle(dt):
    rng = np.random.default_rng(7)
    V, d, ds, n = 5000, 256, 384, 777
    q = synth.round_bf16 if dt == "bf16" else (lambda a: np.asarray(a, np.float32))
    table = q(rng.standard_normal((V, d)))
    sem = q(rng.standard_normal((n, ds)))
    Ws = q(rng.standard_normal((ds, d)) / math.sqrt(ds))
    rows = rng.integers(0, V, n).astype(np.int32)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    code = L().LLATTE_BF16 if dt == "bf16" else L().LLATTE_F32
    out = torch.empty(n, d, device="cuda")
    ws = torch.empty(L().llatte_token_embed_workspace_size(d, ds, code),
                     dtype=torch.uint8, device="cuda")
    L().llatte_token_embed(dev(table, tdt), V, idev(rows), dev(sem, tdt), dev(Ws, tdt),
                           n, d, ds, code, out, ws)
    ref = O.token_embed(table[rows].astype(np.float64), sem.astype(np.float64),
                        Ws.astype(np.float64))
    check(out.cpu().numpy(), ref, dt, "token_embed")


# ---------------------------------------------------------------- whole stack

def gpu_forward(prob, hist=None, cand=None, packed=True):
    from target_aware_latent_amd.model import DeviceModel
    cfg = prob["cfg"]
    I = prob["inputs"]
    model = DeviceModel(cfg, prob["weights"])
    if packed:
        model.pack()
    lengths = [int(x) for x in I["lengths"]]
    h = dev(I["hist"] if hist is None else hist)
    c = None
    if cfg.n_q:
        c = dev(I["cand"] if cand is None else cand)
    ctx = dev(I["ctx"]) if (cfg.n_q and cfg.d_c) else None
    out = model.forward(h, idev(I["offsets"]), lengths, c, ctx)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.cpu().numpy()) for k, v in out.items()}


def oracle_forward(prob, users=None, hist=None, cand=None):
    cfg = prob["cfg"]
    I = prob["inputs"]
    return O.forward(cfg, prob["weights"], I["hist"] if hist is None else hist,
                     I["offsets"], I.get("cand") if cand is None else cand,
                     I.get("ctx"), users=users)


def compare_stack(prob, got, ref, users):
    cfg = prob["cfg"]
    lengths = prob["inputs"]["lengths"]
    keep = O.pyramid_counts(cfg.pyramid, lengths, cfg.N)[-1]
    hoff = np.concatenate([[0], np.cumsum(keep)])
    assert np.array_equal(got["hist_offsets"], hoff)
    gh, rh, gc, rc, ge, re_ = [], [], [], [], [], []
    for k, u in enumerate(users):
        gh.append(got["hist"][hoff[u]:hoff[u + 1]])
        rh.append(ref["hist"][k])
        if cfg.n_q:
            gc.append(got["cand"][u * cfg.n_q:(u + 1) * cfg.n_q])
            rc.append(ref["cand"][k])
        if cfg.n_seeds:
            ge.append(got["emb"][u])
            re_.append(ref["emb"][k])
    if sum(len(x) for x in rh):
        check(np.concatenate(gh), np.concatenate(rh), cfg.dtype, "out_hist")
    if cfg.n_q:
        check(np.concatenate(gc), np.concatenate(rc), cfg.dtype, "out_cand")
    if cfg.n_seeds:
        check(np.stack(ge), np.stack(re_), cfg.dtype, "out_emb")


def small(name, lengths, **kw):
    cfg = synth.get_config(name, B=len(lengths), **kw)
    return synth.generate(cfg, seed=1, lengths=lengths)


SMALL_CASES = {
    "c1": lambda: synth.generate(synth.get_config("c1")),
    "c1_jagged_post": lambda: small("c1", [1, 32, 17, 70, 5], norm_mode="post",
                                    pyramid=synth.PyramidRule("fixed", (40,))),
    "c1_f32_3layers_readout": lambda: small(
        "c1", [9, 70, 33], N=3, n_seeds=2, d_out=64, gain_jitter=0.1,
        pyramid=synth.PyramidRule("fixed", (50, 20, 8))),
    "c2_jagged": lambda: small("c2", [1, 70, 130, 400, 65, 401]),
    "c2_post_nolatent": lambda: small("c2", [33, 257, 4], norm_mode="post",
                                      latent_norm=False, gain_jitter=0.1),
    "c3_small": lambda: small("c3", [300, 150, 64, 1],
                              pyramid=synth.PyramidRule("fixed", (300, 129, 64, 33, 17, 5))),
    # the upstream widths under the halving rule, without the latent norm
    "c3_small_halving_nolatent": lambda: small("c3", [300, 150, 64, 1], latent_norm=False,
                                               pyramid=synth.PyramidRule("halving", floor=8)),
    "c4_small": lambda: small("c4", [1, 64, 65, 129, 300, 513, 200]),
    "c4_cross_last": lambda: small("c4", [90, 12, 300], N=2,
                                   pyramid=synth.PyramidRule("fixed", (200, 0))),
    "c5_small": lambda: small("c5", [200, 37], semantic=None, N=3,
                              pyramid=synth.PyramidRule("geometric", start=150, end=20)),
    # low-rank query path (A.3): fp32; bf16 with the query norm in the GEMM
    # epilogue for 64-, 128- and 256-wide ranks; wider ranks and post-norm
    # through a separate norm pass
    "c1_lowrank_f32": lambda: small("c1", [9, 32, 21], r_q=24, gain_jitter=0.1),
    "c2_lowrank_64": lambda: small("c2", [70, 130, 1], r_q=64, gain_jitter=0.1),
    "c3_small_lowrank": lambda: small("c3", [300, 150, 64, 1], r_q=128,
                                      pyramid=synth.PyramidRule("fixed", (300, 129, 64, 33, 17, 5))),
    "c5_small_lowrank": lambda: small("c5", [200, 37], semantic=None, N=3, r_q=256,
                                      pyramid=synth.PyramidRule("geometric", start=150, end=20)),
    "c4_lowrank_wide": lambda: small("c4", [65, 300, 129], r_q=384, gain_jitter=0.1),
    "c2_post_lowrank": lambda: small("c2", [33, 257, 4], norm_mode="post", r_q=96,
                                     gain_jitter=0.1),
    # more users than the planning scans' 1024 threads (several users per
    # thread), on the fp32 and the bf16 path
    "c1_many_users": lambda: small("c1", np.random.default_rng(5).integers(1, 13, 1100).tolist()),
    "c2_many_users": lambda: small("c2", np.random.default_rng(6).integers(1, 17, 1100).tolist(),
                                   pyramid=synth.PyramidRule("fixed", (12, 6, 3))),
}


@pytest.mark.parametrize("name", list(SMALL_CASES))
def test_forward_small_matches_oracle(name):
    print(f"forward {name}", flush=True)
    prob = SMALL_CASES[name]()
    got = gpu_forward(prob)
    B = prob["cfg"].B
    ref = oracle_forward(prob)
    compare_stack(prob, got, ref, list(range(B)))


def test_forward_is_deterministic():
    prob = small("c4", [1, 64, 65, 129, 300, 513, 200])
    a = gpu_forward(prob)
    b = gpu_forward(prob, packed=False)   # weights packed inside the call
    for k in a:
        if a[k] is not None:
            assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("name,users,over", [
    ("c1", None, {}),
    ("c2", None, {}),
    ("c3", [0, 7, 31, 63], {}),
    ("c4", None, {}),
    ("c3", [0, 40], {"r_q": 256}),
    # the upstream shape without the latent norm, under the halving rule,
    # and with a first layer that keeps 1200 of the 1600 rows
    ("c3", [3, 50], {"latent_norm": False}),
    ("c3", [5, 62], {"pyramid": synth.PyramidRule("halving", floor=64)}),
    ("c3", [1, 63], {"pyramid": synth.PyramidRule("fixed", (1200, 800, 400, 200, 100, 50))}),
])
def test_forward_full_size(name, users, over):
    print(f"forward full {name} {over}", flush=True)
    prob = synth.generate(synth.get_config(name, **over))
    got = gpu_forward(prob)
    B = prob["cfg"].B
    users = list(range(B)) if users is None else users
    ref = oracle_forward(prob, users=users)
    compare_stack(prob, got, ref, users)


def build_semantic_tokens(cfg, prob, seed=0):
    """Device table (streamed block by block) and the GPU token build of the
    history and candidate tokens through llatte_token_embed."""
    sp = cfg.semantic
    I, W = prob["inputs"], prob["weights"]
    table = torch.empty(sp.vocab, cfg.d, dtype=torch.bfloat16, device="cuda")
    for row0, blk in synth.full_table(cfg, seed):
        table[row0:row0 + blk.shape[0]] = torch.from_numpy(blk).to("cuda").to(torch.bfloat16)
    Ws = dev(W["W_s"], torch.bfloat16)
    ws = torch.empty(L().llatte_token_embed_workspace_size(cfg.d, sp.d_sem, L().LLATTE_BF16),
                     dtype=torch.uint8, device="cuda")
    out = {}
    for key in ("hist", "cand"):
        ids, sem = I[f"{key}_ids"], I[f"{key}_sem"]
        o = torch.empty(ids.size, cfg.d, device="cuda")
        L().llatte_token_embed(table, sp.vocab, idev(ids), dev(sem, torch.bfloat16), Ws,
                               ids.size, cfg.d, sp.d_sem, L().LLATTE_BF16, o, ws)
        out[key] = o
    torch.cuda.synchronize()
    return out


@pytest.mark.timeout(900)
def test_forward_full_size_semantic_tokens():
    """12 layers, d=1024, r=256, 16 candidates: token build from the 1M x 1024
    hashed-ID table plus W_s times the semantic vector, then the stack; the
    token build is checked on sampled rows and the stack on sampled users."""
    print("forward full c5", flush=True)
    cfg = synth.get_config("c5")
    prob = synth.generate(cfg)
    I, W = prob["inputs"], prob["weights"]
    tok = build_semantic_tokens(cfg, prob)
    users = [0, 17, 31]
    off = I["offsets"]
    # token build, sampled users' rows, against the oracle's token build
    hist_ref, cand_ref = {}, {}
    for u in users:
        rows = I["hist_ids"][off[u]:off[u + 1]]
        hist_ref[u] = O.token_embed(synth.table_rows(cfg, 0, rows).astype(np.float64),
                                    I["hist_sem"][off[u]:off[u + 1]].astype(np.float64),
                                    W["W_s"].astype(np.float64))
        crow = I["cand_ids"][u * cfg.n_q:(u + 1) * cfg.n_q]
        cand_ref[u] = O.token_embed(synth.table_rows(cfg, 0, crow).astype(np.float64),
                                    I["cand_sem"][u * cfg.n_q:(u + 1) * cfg.n_q].astype(np.float64),
                                    W["W_s"].astype(np.float64))
        check(tok["hist"][off[u]:off[u + 1]].cpu().numpy(), hist_ref[u], "bf16",
              f"token_embed user {u}")
    from target_aware_latent_amd.model import DeviceModel
    model = DeviceModel(cfg, W)
    model.pack()
    lengths = [int(x) for x in I["lengths"]]
    got = model.forward(tok["hist"], idev(off), lengths, tok["cand"], dev(I["ctx"]))
    torch.cuda.synchronize()
    got = {k: (None if v is None else v.cpu().numpy()) for k, v in got.items()}
    # oracle on the oracle's own tokens for the sampled users
    hist_o = np.zeros((off[-1], cfg.d))
    cand_o = np.zeros((cfg.B * cfg.n_q, cfg.d))
    for u in users:
        hist_o[off[u]:off[u + 1]] = hist_ref[u]
        cand_o[u * cfg.n_q:(u + 1) * cfg.n_q] = cand_ref[u]
    ref = O.forward(cfg, W, hist_o, off, cand_o, I["ctx"], users=users)
    compare_stack(prob, got, ref, users)
