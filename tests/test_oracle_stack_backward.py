"""Pins of the oracle's whole-stack backward (forward_backward).

The oracle writes the chain rule out by hand: sublayer derivatives, the
pyramid's routing of row gradients (layer l's input rows are layer l-1's
output rows; trimmed rows only get key/value terms), the readout (seeds and
W_p) and the fusion of the candidate tokens. Two independent checks:

- torch autograd through a forward written here from the definition
  ([LLaTTE] A.2 layer equation in its pre-norm reading, A.3 non-absorbed MLA,
  the pyramidal schedule, the A.2 fusion of query tokens and the readout
  with seeds), whose outputs are first checked against oracle.forward;
- central differences of oracle.forward itself (pinned to brute force
  elsewhere) along random directions of inputs and weights.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import llatte_oracle as O


def _case(ln, pyramid, raw=False, seed=0):
    cfg = synth.get_config("c2", B=3, N=3, d=16, h=2, dk=8, r=8, n_q=2, d_c=4,
                           n_seeds=2, d_out=8, latent_norm=ln, pyramid=pyramid,
                           gain_jitter=0.1, dtype="f32")
    prob = synth.generate(cfg, seed=seed, lengths=[7, 3, 1])
    W = prob["weights"]
    if raw:
        W = dict(W)
        W["W_p"] = None
    I = prob["inputs"]
    rng = np.random.default_rng(100 + seed)
    fw = O.forward(cfg, W, I["hist"], I["offsets"], I["cand"], I["ctx"])
    d_hist = [rng.standard_normal(h.shape) for h in fw["hist"]]
    d_cand = rng.standard_normal((cfg.B * cfg.n_q, cfg.d))
    d_emb = rng.standard_normal((cfg.B, np.asarray(fw["emb"][0]).size))
    return cfg, W, I, fw, d_hist, d_cand, d_emb


# ------------------------------------------------------------ torch forward

def _t_layer(Rh, Rc, n, W, cfg):
    eps = cfg.eps
    rms = lambda x, g: x * torch.rsqrt((x * x).mean(-1, keepdim=True) + eps) * g
    K, nc, h, dk = Rh.shape[0], Rc.shape[0], cfg.h, cfg.dk
    H, Hc = rms(Rh, W["g1"]), rms(Rc, W["g1"])
    C = H @ W["W_dkv"]
    if cfg.latent_norm:
        C = rms(C, W["g_c"])
    Hq = torch.cat([H[K - n:], Hc])
    Rq = torch.cat([Rh[K - n:], Rc])
    M = Hq.shape[0]
    q = (Hq @ W["W_uq"]).reshape(M, h, dk)
    k = (C @ W["W_uk"]).reshape(K, h, dk)
    v = (C @ W["W_uv"]).reshape(K, h, dk)
    key = torch.arange(K)[None, :]
    limit = torch.cat([torch.arange(K - n, K), torch.full((nc,), K - 1)])[:, None]
    allowed = key <= limit
    s = torch.einsum("mhd,khd->hmk", q, k) / math.sqrt(dk)
    p = torch.softmax(s.masked_fill(~allowed, float("-inf")), dim=-1)
    o = torch.einsum("hmk,khd->mhd", p, v).reshape(M, h * dk)
    R1 = Rq + o @ W["W_o"]
    R2 = R1 + F.gelu(rms(R1, W["g2"]) @ W["W1"]) @ W["W2"]
    return R2[:n], R2[n:]


def _t_loss(cfg, Wt, hist, cand, ctx, offsets, keep, d_hist, d_cand, d_emb):
    loss = 0.0
    for u in range(cfg.B):
        Rh = hist[offsets[u]:offsets[u + 1]]
        xc = torch.cat([cand[u * cfg.n_q:(u + 1) * cfg.n_q],
                        ctx[u].expand(cfg.n_q, cfg.d_c)], dim=1)
        Rc = xc @ Wt["W_q"]
        for l in range(cfg.N):
            Rh, Rc = _t_layer(Rh, Rc, int(keep[l, u]), Wt["layers"][l], cfg)
        loss = loss + (Rh * torch.from_numpy(d_hist[u])).sum()
        loss = loss + (Rc * torch.from_numpy(d_cand[u * cfg.n_q:(u + 1) * cfg.n_q])).sum()
        _, S = _t_layer(Rh, Wt["seeds"], 0, Wt["readout"], cfg)
        emb = S.reshape(-1) if Wt["W_p"] is None else S.reshape(-1) @ Wt["W_p"]
        loss = loss + (emb * torch.from_numpy(d_emb[u])).sum()
    return loss


def _leaf(a):
    return torch.tensor(np.asarray(a, np.float64), dtype=torch.float64, requires_grad=True)


@pytest.mark.parametrize("ln,pyr,raw", [
    (True, synth.PyramidRule("fixed", (5, 3, 2)), False),
    (False, synth.PyramidRule("halving", floor=1), False),
    (True, synth.PyramidRule("fixed", (6, 6, 1)), True),
], ids=["fixed-latentnorm", "halving-nolatent", "fixed-raw-readout"])
def test_stack_backward_matches_torch_autograd(ln, pyr, raw):
    cfg, W, I, fw, d_hist, d_cand, d_emb = _case(ln, pyr, raw)
    offsets = I["offsets"].astype(np.int64)
    keep = O.pyramid_counts(cfg.pyramid, offsets[1:] - offsets[:-1], cfg.N)
    Wt = {"layers": [{k: _leaf(v) for k, v in lw.items()} for lw in W["layers"]],
          "readout": {k: _leaf(v) for k, v in W["readout"].items()},
          "seeds": _leaf(W["seeds"]), "W_q": _leaf(W["W_q"]),
          "W_p": None if W["W_p"] is None else _leaf(W["W_p"])}
    hist, cand, ctx = _leaf(I["hist"]), _leaf(I["cand"]), _leaf(I["ctx"])
    # the torch forward reproduces the oracle's outputs
    with torch.no_grad():
        for u in range(cfg.B):
            Rh = hist[offsets[u]:offsets[u + 1]]
            xc = torch.cat([cand[u * 2:(u + 1) * 2], ctx[u].expand(2, cfg.d_c)], dim=1)
            Rc = xc @ Wt["W_q"]
            for l in range(cfg.N):
                Rh, Rc = _t_layer(Rh, Rc, int(keep[l, u]), Wt["layers"][l], cfg)
            assert np.allclose(Rh.numpy(), fw["hist"][u], rtol=0, atol=1e-10)
            assert np.allclose(Rc.numpy(), fw["cand"][u], rtol=0, atol=1e-10)
    loss = _t_loss(cfg, Wt, hist, cand, ctx, offsets, keep, d_hist, d_cand, d_emb)
    loss.backward()
    g = O.forward_backward(cfg, W, I["hist"], I["offsets"], I["cand"], I["ctx"],
                           d_hist, d_cand, d_emb)

    def close(a, t, what):
        t = t.grad.numpy()
        scale = max(float(np.max(np.abs(t))), 1e-30)
        err = float(np.max(np.abs(np.asarray(a) - t))) / scale
        assert err <= 1e-9, f"{what}: {err:.2e}"

    for l in range(cfg.N):
        for k, t in Wt["layers"][l].items():
            if k == "g_c" and not ln:
                assert float(np.max(np.abs(g["layers"][l][k]))) == 0.0
                continue
            close(g["layers"][l][k], t, f"layer {l} {k}")
    for k, t in Wt["readout"].items():
        if k == "g_c" and not ln:
            continue
        close(g["readout"][k], t, f"readout {k}")
    close(g["seeds"], Wt["seeds"], "seeds")
    close(g["W_q"], Wt["W_q"], "W_q")
    if Wt["W_p"] is not None:
        close(g["W_p"], Wt["W_p"], "W_p")
    else:
        assert "W_p" not in g
    close(g["hist"], hist, "hist")
    close(g["cand"], cand, "cand")
    close(g["ctx"], ctx, "ctx")


def test_stack_backward_matches_central_differences():
    cfg, W, I, fw, d_hist, d_cand, d_emb = _case(True, synth.PyramidRule("fixed", (5, 2, 2)),
                                                 seed=3)
    g = O.forward_backward(cfg, W, I["hist"], I["offsets"], I["cand"], I["ctx"],
                           d_hist, d_cand, d_emb)

    def loss(Wx, hist, cand, ctx):
        f = O.forward(cfg, Wx, hist, I["offsets"], cand, ctx)
        L = sum(float(np.sum(a * b)) for a, b in zip(f["hist"], d_hist))
        L += float(np.sum(np.concatenate(f["cand"]) * d_cand))
        L += sum(float(np.sum(np.asarray(e) * de)) for e, de in zip(f["emb"], d_emb))
        return L

    f64 = lambda a: np.asarray(a, np.float64)
    Wd = {"layers": [{k: f64(v) for k, v in lw.items()} for lw in W["layers"]],
          "readout": {k: f64(v) for k, v in W["readout"].items()},
          "seeds": f64(W["seeds"]), "W_q": f64(W["W_q"]), "W_p": f64(W["W_p"])}
    X = {"hist": f64(I["hist"]), "cand": f64(I["cand"]), "ctx": f64(I["ctx"])}
    rng = np.random.default_rng(7)
    # (where, key, gradient): weights of the first, middle and last layer, the
    # readout, the seeds, the fusion and projection matrices and the inputs
    probes = [(("layers", 0), "W_dkv", g["layers"][0]["W_dkv"]),
              (("layers", 0), "g1", g["layers"][0]["g1"]),
              (("layers", 1), "W_uk", g["layers"][1]["W_uk"]),
              (("layers", 1), "W1", g["layers"][1]["W1"]),
              (("layers", 2), "g_c", g["layers"][2]["g_c"]),
              (("layers", 2), "W_o", g["layers"][2]["W_o"]),
              (("readout",), "W_uq", g["readout"]["W_uq"]),
              ((), "seeds", g["seeds"]), ((), "W_q", g["W_q"]), ((), "W_p", g["W_p"]),
              (None, "hist", g["hist"]), (None, "cand", g["cand"]), (None, "ctx", g["ctx"])]
    eps = 1e-6
    for where, key, grad in probes:
        V = rng.standard_normal(np.shape(grad))

        def shifted(t):
            Wx = {"layers": [dict(lw) for lw in Wd["layers"]], "readout": dict(Wd["readout"]),
                  "seeds": Wd["seeds"], "W_q": Wd["W_q"], "W_p": Wd["W_p"]}
            Xx = dict(X)
            if where is None:
                Xx[key] = X[key] + t * V
            elif where == ():
                Wx[key] = Wd[key] + t * V
            elif where[0] == "readout":
                Wx["readout"][key] = Wd["readout"][key] + t * V
            else:
                Wx["layers"][where[1]][key] = Wd["layers"][where[1]][key] + t * V
            return loss(Wx, Xx["hist"], Xx["cand"], Xx["ctx"])

        fd = (shifted(eps) - shifted(-eps)) / (2 * eps)
        an = float(np.sum(grad * V))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (where, key, fd, an)


def test_trimmed_rows_still_get_key_value_gradients():
    # user 0 has 7 rows and layer 0 keeps the last 5: rows 0 and 1 leave the
    # stack after layer 0, where they were keys and values of every query,
    # so their gradient is nonzero although no output row descends from them;
    # with every output gradient zero, every gradient is zero
    cfg, W, I, fw, d_hist, d_cand, d_emb = _case(True, synth.PyramidRule("fixed", (5, 3, 2)))
    g = O.forward_backward(cfg, W, I["hist"], I["offsets"], I["cand"], I["ctx"],
                           d_hist, d_cand, d_emb)
    assert np.all(np.abs(g["hist"][0:2]) > 0)
    # with every output gradient zero, every gradient is zero
    z = O.forward_backward(cfg, W, I["hist"], I["offsets"], I["cand"], I["ctx"],
                           [np.zeros_like(x) for x in d_hist], np.zeros_like(d_cand),
                           np.zeros_like(d_emb))
    assert float(np.max(np.abs(z["hist"]))) == 0.0
    assert all(float(np.max(np.abs(v))) == 0.0 for lw in z["layers"] for v in lw.values())
