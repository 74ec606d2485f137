"""Scalar-loop brute force of the LLaTTE sequence-module forward, tiny inputs.

TEST INFRASTRUCTURE ONLY. A second, deliberately naive implementation of the
same definition as ``llatte_oracle.forward``: plain Python floats and explicit
index loops, no array library, one user at a time. It exists to catch slips in
the vectorised oracle (a transposed operand, a wrong head slice, a misplaced
mask bound) on inputs small enough for loops.

Sources: [LLaTTE] "LLaTTE: Scaling Laws for Multi-Stage Sequence Modeling in
Large-Scale Ads Recommendation", Appendix A.2 (fusion, layer equations,
pyramidal schedule, summaries) and A.3 (MLA); [Repro] "LLaTTE: Multi-stage
sequence scaling", core formula (q = W_Q [x; c]). Same readings as the
vectorised oracle.
"""
import math


def _mat(a):
    return [list(map(float, row)) for row in a]


def _vec(a):
    return list(map(float, a))


def _matvec_row(x, W):
    """x [n] times W [n][m] -> [m]."""
    n, m = len(W), len(W[0])
    out = [0.0] * m
    for i in range(n):
        xi = x[i]
        Wi = W[i]
        for j in range(m):
            out[j] += xi * Wi[j]
    return out


def _rms(x, g, eps):
    s = 0.0
    for v in x:
        s += v * v
    inv = 1.0 / math.sqrt(s / len(x) + eps)
    return [x[i] * inv * g[i] for i in range(len(x))]


def _gelu(v):
    return 0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0)))


def _layer(Rh, Rc, n, W, cfg):
    d, h, dk, r = cfg.d, cfg.h, cfg.dk, cfg.r
    eps = cfg.eps
    g1, g2, gc = _vec(W["g1"]), _vec(W["g2"]), _vec(W["g_c"])
    Wdkv, Wuq, Wuk = _mat(W["W_dkv"]), _mat(W["W_uq"]), _mat(W["W_uk"])
    Wuv, Wo, W1, W2 = _mat(W["W_uv"]), _mat(W["W_o"]), _mat(W["W1"]), _mat(W["W2"])
    pre = cfg.norm_mode == "pre"
    K = len(Rh)
    nc = len(Rc)
    Hh = [_rms(x, g1, eps) if pre else list(x) for x in Rh]
    Hc = [_rms(x, g1, eps) if pre else list(x) for x in Rc]
    # latent, then per-head keys and values of every history row
    C = []
    for x in Hh:
        c = _matvec_row(x, Wdkv)
        C.append(_rms(c, gc, eps) if cfg.latent_norm else c)
    Kf = [_matvec_row(c, Wuk) for c in C]       # [K][h*dk]
    Vf = [_matvec_row(c, Wuv) for c in C]
    # queries: the last n history rows (positions K-n..K-1), then candidates
    qrows = [(Hh[K - n + t], Rh[K - n + t], K - n + t) for t in range(n)]
    qrows += [(Hc[j], Rc[j], K - 1) for j in range(nc)]
    out = []
    for Hx, Rx, pos in qrows:
        if "W_dq" in W:  # low-rank query path: RMSNorm(x W_dq) g_q W_uq
            q = _matvec_row(_rms(_matvec_row(Hx, _mat(W["W_dq"])), _vec(W["g_q"]), eps), Wuq)
        else:
            q = _matvec_row(Hx, Wuq)
        o = [0.0] * (h * dk)
        for hh in range(h):
            sc = []
            for j in range(pos + 1):
                s = 0.0
                for e in range(dk):
                    s += q[hh * dk + e] * Kf[j][hh * dk + e]
                sc.append(s / math.sqrt(dk))
            mx = max(sc)
            ex = [math.exp(s - mx) for s in sc]
            tot = sum(ex)
            for j in range(pos + 1):
                w = ex[j] / tot
                for e in range(dk):
                    o[hh * dk + e] += w * Vf[j][hh * dk + e]
        a = _matvec_row(o, Wo)
        if pre:
            r1 = [Rx[i] + a[i] for i in range(d)]
            f = [_gelu(v) for v in _matvec_row(_rms(r1, g2, eps), W1)]
            f2 = _matvec_row(f, W2)
            r2 = [r1[i] + f2[i] for i in range(d)]
        else:
            r1 = _rms([Rx[i] + a[i] for i in range(d)], g1, eps)
            f = [_gelu(v) for v in _matvec_row(r1, W1)]
            f2 = _matvec_row(f, W2)
            r2 = _rms([r1[i] + f2[i] for i in range(d)], g2, eps)
        out.append(r2)
    return out[:n], out[n:]


def keep_counts(cfg, L):
    """Per-layer keep counts of one user (loop form of the pyramid rule)."""
    rule = cfg.pyramid
    res = []
    prev = L
    for l in range(cfg.N):
        if rule.kind == "halving":
            k = max(min(rule.floor, L), L // (2 ** l))
        elif rule.kind == "fixed":
            k = rule.values[l]
        else:  # geometric
            if cfg.N == 1:
                k = rule.start
            else:
                k = int(math.floor(rule.start * (rule.end / rule.start)
                                   ** (l / (cfg.N - 1)) + 0.5))
        k = min(k, prev)
        res.append(k)
        prev = k
    return res


def forward_user(cfg, W, hist_u, cand_u=None, ctx_u=None):
    """One user's forward: returns (hist_out, cand_out, emb or None)."""
    Rh = _mat(hist_u)
    Rc = []
    if cfg.n_q > 0:
        Wq = _mat(W["W_q"])
        for x in _mat(cand_u):
            xc = x + (_vec(ctx_u) if (ctx_u is not None and cfg.d_c > 0) else [])
            Rc.append(_matvec_row(xc, Wq))
    for l, n in enumerate(keep_counts(cfg, len(Rh))):
        Rh, Rc = _layer(Rh, Rc, n, W["layers"][l], cfg)
    emb = None
    if cfg.n_seeds > 0:
        _, S = _layer(Rh, _mat(W["seeds"]), 0, W["readout"], cfg)
        flat = [v for row in S for v in row]
        emb = _matvec_row(flat, _mat(W["W_p"]))
    return Rh, Rc, emb
