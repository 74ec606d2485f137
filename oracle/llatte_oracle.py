"""CPU oracle of the LLaTTE target-aware MLA sequence-module forward.

TEST INFRASTRUCTURE ONLY. This module is the slow, plain reference that the
GPU library is checked against. Only the tests, the package smoke check and
the CPU-baseline leg of the benchmark may import it; the product path never
does. It shares no code with the HIP library.

Sources (cited by page title and section):
  [LLaTTE]  "LLaTTE: Scaling Laws for Multi-Stage Sequence Modeling in
            Large-Scale Ads Recommendation" (annotated translation):
            section 1.3.2 (five-step sequence module), Appendix A.2 (query
            tokens and fusion, the layer equations, the pyramidal schedule
            and its cost, the three attention modes, sequence summaries),
            Appendix A.3 (MLA, non-absorbed and absorbed forms).
  [Repro]   "LLaTTE: Multi-stage sequence scaling" (reproduction note),
            section "core formula" (target-aware query q = W_Q [x; c]).

Readings taken where the pages are silent or disagree (each is also listed
with its reason in the design notes):
  * pre-norm layer by default (the A.2 layer equation is written post-norm;
    both placements are implemented, 'post' follows A.2 literally);
  * RMSNorm on the latent C (A.3) on by default, switchable off;
  * queries: a full-rank per-layer W_uq by default, or the A.3 low-rank path
    RMSNorm(H W_dq) g_q W_uq when the layer carries W_dq (the pages give no
    query rank; it is a workload parameter);
  * softmax scale 1/sqrt(head_dim) in both MLA forms (A.3's absorbed form
    writes sqrt(d_c); the two forms are only equal with one common scale);
  * candidate query tokens attend every history key and nothing else;
    history rows attend causally and never see candidates;
  * the pyramid keeps history rows only; candidates are always kept; layer
    l's keys are all rows kept by layer l-1, its queries the last n_l rows
    (output extraction; equal to computing all rows then slicing, A.2);
  * GELU with the exact erf, FFN width 4d, no biases; RMSNorm eps inside the
    square root; no final norm after the stack;
  * readout: one more layer in cross-attention mode whose queries are the
    learned seeds, flattened seed-major and multiplied by W_p (the A.2
    summary as a plain linear map); without W_p the flattened readout itself
    is returned, for the low-rank adapted MLP summaries
    (lora_mlp_summaries: one hidden layer, exact-erf GELU, no biases, base
    weights shared by the summaries plus rank-rho adapters per summary).

Numbers are fp64 by default; ``dtype=np.float32`` gives the same code in
single precision (used only as the timed CPU baseline).
"""
import math

import numpy as np
from scipy.special import erf as _erf

__all__ = [
    "rmsnorm", "gelu", "softmax_masked", "pyramid_list", "pyramid_counts",
    "compact", "history_query_mask", "mla_layer", "fuse_queries", "forward",
    "token_embed", "latent_attention", "unmasked_pairs", "flop_count",
    "lora_mlp_summaries", "latent_attention_backward", "ffn_block_backward",
    "rmsnorm_backward", "attention_sublayer_backward", "forward_backward",
]


# ---------------------------------------------------------------- primitives

def rmsnorm(x, g, eps=1e-6):
    """RMS normalisation over the last axis, times the gain g.

    [LLaTTE] A.2 layer equations use RMSNorm (Root Mean Square Layer
    Normalization): x / sqrt(mean(x^2) + eps) * g.
    """
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def gelu(x):
    """Exact GELU, x * Phi(x) with Phi the standard normal CDF (erf form).

    The FFN of the [LLaTTE] A.2 layer equation has no stated activation; the
    exact-erf GELU is the reading used throughout.
    """
    return 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0)))


def softmax_masked(s, allowed):
    """Row softmax over the last axis of s, with disallowed entries removed.

    [LLaTTE] A.3: softmax(Q K^T / sqrt(d_k)); masked entries get probability 0.
    The row maximum is subtracted before exponentiation. Every row must have
    at least one allowed entry.
    """
    z = np.where(allowed, s, -np.inf)
    m = np.max(z, axis=-1, keepdims=True)
    e = np.where(allowed, np.exp(z - m), 0.0)
    return e / np.sum(e, axis=-1, keepdims=True)


# ---------------------------------------------------------------- pyramid

def pyramid_list(rule, n_layers):
    """Per-layer keep list of a 'fixed' or 'geometric' rule.

    [LLaTTE] A.2 pyramidal schedule: T_{l+1} <= T_l. A geometric rule runs
    from rule.start to rule.end over the layers, rounded half up.
    """
    if rule.kind == "fixed":
        assert len(rule.values) == n_layers
        return [int(v) for v in rule.values]
    if rule.kind == "geometric":
        if n_layers == 1:
            return [int(rule.start)]
        out = []
        for l in range(n_layers):
            v = rule.start * (rule.end / rule.start) ** (l / (n_layers - 1))
            out.append(int(math.floor(v + 0.5)))
        return out
    raise ValueError(rule.kind)


def pyramid_counts(rule, lengths, n_layers):
    """keep[l, u]: history rows of user u kept as queries/outputs at layer l+1.

    [LLaTTE] A.2 pyramidal schedule: the next layer works on the most recent
    T_{l+1} <= T_l rows. Counts never exceed the previous layer's count.
    'halving': keep = max(min(floor, L_u), L_u >> l) for the 0-based layer l.
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    keep = np.zeros((n_layers, lengths.size), dtype=np.int64)
    prev = lengths.copy()
    if rule.kind == "halving":
        for l in range(n_layers):
            keep[l] = np.maximum(np.minimum(rule.floor, lengths), lengths >> l)
            keep[l] = np.minimum(keep[l], prev)
            prev = keep[l]
        return keep
    lst = pyramid_list(rule, n_layers)
    for l in range(n_layers):
        keep[l] = np.minimum(lst[l], prev)
        prev = keep[l]
    return keep


def compact(values, offsets, keep):
    """Keep the last keep[u] rows of each user's segment, in order.

    [LLaTTE] A.2: R^{(l+1)} = X^{(l)}[:, -T_{l+1}:, :]. Returns the kept rows,
    the exclusive scan of keep as new offsets, and the global source row of
    every kept row.
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    keep = np.asarray(keep, dtype=np.int64)
    B = keep.size
    lens = offsets[1:] - offsets[:-1]
    if np.any(keep < 0) or np.any(keep > lens):
        raise ValueError("keep must lie in [0, L_u]")
    src = []
    for u in range(B):
        src.extend(range(offsets[u + 1] - keep[u], offsets[u + 1]))
    src = np.asarray(src, dtype=np.int64)
    new_off = np.zeros(B + 1, dtype=np.int64)
    new_off[1:] = np.cumsum(keep)
    return values[src], new_off, src


def history_query_mask(K, n, n_c):
    """Allowed (query, key) pairs of one user at one layer, shape [n+n_c, K].

    Query rows 0..n-1 are the last n history rows (key positions K-n .. K-1)
    and attend causally ([LLaTTE] A.2 causal transformer). Rows n..n+n_c-1
    are candidate tokens and attend every history key (reading of the
    target-aware query of [Repro], core formula).
    """
    j = np.arange(K)[None, :]
    pos = (K - n + np.arange(n))[:, None]
    hist = j <= pos
    cand = np.ones((n_c, K), dtype=bool)
    return np.concatenate([hist, cand], axis=0)


# ---------------------------------------------------------------- one layer

def _split_heads(x, h):
    M = x.shape[0]
    return x.reshape(M, h, -1)


def mla_layer(Rh, Rc, n, W, cfg, absorbed=False, return_probs=False, return_r1=False):
    """One transformer layer with MLA on one user.

    Rh: the K history rows entering the layer (oldest first); Rc: the n_c
    candidate/seed rows; n: history rows kept as queries (0 <= n <= K).
    Returns (Rh_out [n, d], Rc_out [n_c, d]) and, on request, the attention
    probabilities [h, n+n_c, K] and then R1, the rows after the attention
    sublayer ([n+n_c, d]: query history rows, then candidates).

    [LLaTTE] A.3 non-absorbed MLA: C = RMSNorm(H W_down^KV) (the latent),
    K, V = split(C W_up^KV), attention softmax(Q K^T / sqrt(d_k)) V W_out.
    Queries: Q = H W_uq (full rank), or, when the layer has W_dq, the A.3
    low-rank path Q = RMSNorm(H W_down^Q) W_up^Q with gain g_q.
    With ``absorbed`` the A.3 rewritten form is used instead: per head the
    query is moved into latent space (q W_uk^T), scores are taken against C
    itself and the output is mapped back through W_uv.
    [LLaTTE] A.2 layer equation (post-norm) or its pre-norm reading.
    """
    d, h, dk = cfg.d, cfg.h, cfg.dk
    eps = cfg.eps
    K = Rh.shape[0]
    n_c = Rc.shape[0]
    if K < 1 or not (0 <= n <= K):
        raise ValueError("need K >= 1 and 0 <= n <= K")
    pre = cfg.norm_mode == "pre"
    Hh = rmsnorm(Rh, W["g1"], eps) if pre else Rh
    Hc = rmsnorm(Rc, W["g1"], eps) if pre else Rc

    C = Hh @ W["W_dkv"]
    if cfg.latent_norm:
        C = rmsnorm(C, W["g_c"], eps)

    Hq = np.concatenate([Hh[K - n:], Hc], axis=0)
    Rq = np.concatenate([Rh[K - n:], Rc], axis=0)
    M = Hq.shape[0]
    if "W_dq" in W:                                  # low-rank query path
        q = _split_heads(rmsnorm(Hq @ W["W_dq"], W["g_q"], eps) @ W["W_uq"], h)
    else:
        q = _split_heads(Hq @ W["W_uq"], h)          # [M, h, dk]
    allowed = history_query_mask(K, n, n_c)          # [M, K]
    scale = 1.0 / math.sqrt(dk)

    Wuk = W["W_uk"].reshape(cfg.r, h, dk)
    Wuv = W["W_uv"].reshape(cfg.r, h, dk)
    o = np.empty((M, h, dk), dtype=Rh.dtype)
    probs = np.empty((h, M, K), dtype=Rh.dtype) if return_probs else None
    for hh in range(h):
        if absorbed:
            q_lat = q[:, hh, :] @ Wuk[:, hh, :].T    # [M, r]
            s = (q_lat @ C.T) * scale
            p = softmax_masked(s, allowed)
            o[:, hh, :] = (p @ C) @ Wuv[:, hh, :]
        else:
            Kh = C @ Wuk[:, hh, :]                   # [K, dk]
            Vh = C @ Wuv[:, hh, :]
            s = (q[:, hh, :] @ Kh.T) * scale
            p = softmax_masked(s, allowed)
            o[:, hh, :] = p @ Vh
        if return_probs:
            probs[hh] = p
    A = o.reshape(M, h * dk) @ W["W_o"]

    if pre:
        R1 = Rq + A
        R2 = R1 + gelu(rmsnorm(R1, W["g2"], eps) @ W["W1"]) @ W["W2"]
    else:
        R1 = rmsnorm(Rq + A, W["g1"], eps)
        R2 = rmsnorm(R1 + gelu(R1 @ W["W1"]) @ W["W2"], W["g2"], eps)
    out = (R2[:n], R2[n:])
    extra = ((probs,) if return_probs else ()) + ((R1,) if return_r1 else ())
    return (out,) + extra if extra else out


# ---------------------------------------------------------------- the stack

def fuse_queries(cand, ctx, W_q):
    """Candidate query tokens Q0 = [x_j ; c_u] W_q for one user.

    [Repro] core formula q = W_Q [x; c]; [LLaTTE] A.2 query tokens appended
    after the history (Concat(X_seq, Q)). cand: [n_q, d]; ctx: [d_c] or None.
    """
    if ctx is None or ctx.size == 0:
        xc = cand
    else:
        xc = np.concatenate([cand, np.broadcast_to(ctx, (cand.shape[0], ctx.size))],
                            axis=1)
    return xc @ W_q


def forward(cfg, W, hist, offsets, cand=None, ctx=None, users=None,
            absorbed=False, dtype=np.float64, trace=None):
    """The sequence-module forward for each user in ``users`` (all if None).

    [LLaTTE] section 1.3.2: fusion of the query tokens, N layers of MLA with
    the pyramidal schedule, then the readout. Returns a dict with per-user
    lists 'hist' ([n_N(u), d]), 'cand' ([n_q, d]) and, with a readout,
    'emb' ([d_out]). With ``trace`` (a list), one entry per user is appended:
    the list of each layer's outputs (history rows, candidate rows), then,
    with a readout, the readout layer's seed rows (no history rows) - the
    values only, for localising a disagreement layer by layer.
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    lengths = offsets[1:] - offsets[:-1]
    B = lengths.size
    if np.any(lengths < 1):
        raise ValueError("every user needs at least one history row")
    keep = pyramid_counts(cfg.pyramid, lengths, cfg.N)
    users = range(B) if users is None else users
    cast = lambda a: None if a is None else np.asarray(a, dtype=dtype)
    Wc = {k: (v if k == "layers" or k == "readout" else cast(v))
          for k, v in W.items()}
    layers = [{k: cast(v) for k, v in lw.items()} for lw in W["layers"]]
    readout = ({k: cast(v) for k, v in W["readout"].items()}
               if cfg.n_seeds > 0 else None)
    res = {"users": list(users), "hist": [], "cand": [], "emb": []}
    for u in users:
        Rh = cast(hist[offsets[u]:offsets[u + 1]])
        if cfg.n_q > 0:
            cu = cast(cand[u * cfg.n_q:(u + 1) * cfg.n_q])
            xu = cast(ctx[u]) if (ctx is not None and cfg.d_c > 0) else None
            Rc = fuse_queries(cu, xu, Wc["W_q"])
        else:
            Rc = np.zeros((0, cfg.d), dtype=dtype)
        steps = []
        for l in range(cfg.N):
            Rh, Rc = mla_layer(Rh, Rc, int(keep[l, u]), layers[l], cfg, absorbed)
            steps.append((Rh, Rc))
        res["hist"].append(Rh)
        res["cand"].append(Rc)
        if readout is not None:
            _, S = mla_layer(Rh, Wc["seeds"], 0, readout, cfg, absorbed)
            steps.append((Rh[:0], S))
            flat = S.reshape(-1)   # Flatten(Z_raw), seed-major
            res["emb"].append(flat if Wc.get("W_p") is None else flat @ Wc["W_p"])
        if trace is not None:
            trace.append(steps)
    return res


def lora_mlp_summaries(z, L, dtype=np.float64):
    """Sequence summaries [K, B, d_seq] from flattened readouts z [B, d_z].

    [LLaTTE] Appendix A.2 item 4: each summary k is LoRAMLP_k applied to
    Flatten(Z_raw), a low-rank adapted MLP. Reading (the internals are not
    given): one hidden layer, exact-erf GELU, no biases, with base weights
    W1 [d_z, d_h], W2 [d_h, d_seq] shared by the summaries and rank-rho
    adapters per summary on both matrices:
        LoRAMLP_k(x) = GELU(x (W1 + A1_k B1_k)) (W2 + A2_k B2_k),
    A1 [K, d_z, rho], B1 [K, rho, d_h], A2 [K, d_h, rho], B2 [K, rho, d_seq].
    """
    f = lambda a: np.asarray(a, dtype=dtype)
    z = f(z)
    out = []
    for k in range(f(L["A1"]).shape[0]):
        W1k = f(L["W1"]) + f(L["A1"][k]) @ f(L["B1"][k])
        W2k = f(L["W2"]) + f(L["A2"][k]) @ f(L["B2"][k])
        out.append(gelu(z @ W1k) @ W2k)
    return np.stack(out)


def token_embed(table_rows, sem, W_s):
    """Token = hashed-ID table row + semantic vector times W_s.

    [LLaTTE] section 1.3 features: sparse-ID embeddings plus dense content
    embeddings per event (section 1.5.3 content-aware scaling adds the
    semantic representation to the token).
    """
    return table_rows + sem @ W_s


# ------------------------------------------------- the exported latent core

def latent_attention(q_lat, c_lat, kv_offsets, hq_offsets, n_cand, scale):
    """Attention in latent space, the core of the absorbed MLA form.

    [LLaTTE] A.3 absorbed form: queries already multiplied into latent space
    (q_lat [Mtot, h, r]) score against the shared latent C ([Ktot, r]) and the
    output is sum_j softmax_j(scale * q_lat . C_j) * C_j, per head.
    Candidate rows come first: user u's are rows u*n_cand + j, and see all
    K_u keys. History query rows of user u follow at
    B*n_cand + hq_offsets[u] .. B*n_cand + hq_offsets[u+1]-1; row t sits at
    key position K_u - n_u + t and sees keys 0..that position.
    Returns (out [Mtot, h, r], lse [Mtot, h]) with lse the natural-log
    log-sum-exp of the scaled scores.
    """
    kv_offsets = np.asarray(kv_offsets, dtype=np.int64)
    hq_offsets = np.asarray(hq_offsets, dtype=np.int64)
    B = kv_offsets.size - 1
    nc = B * n_cand
    Mtot = nc + int(hq_offsets[-1])
    h, r = q_lat.shape[1], q_lat.shape[2]
    out = np.zeros((Mtot, h, r), dtype=q_lat.dtype)
    lse = np.zeros((Mtot, h), dtype=q_lat.dtype)
    for u in range(B):
        C = c_lat[kv_offsets[u]:kv_offsets[u + 1]]
        K = C.shape[0]
        n = int(hq_offsets[u + 1] - hq_offsets[u])
        rows = list(range(nc + hq_offsets[u], nc + hq_offsets[u + 1])) + \
            list(range(u * n_cand, (u + 1) * n_cand))
        allowed = history_query_mask(K, n, n_cand)
        for hh in range(h):
            s = (q_lat[rows, hh, :] @ C.T) * scale
            z = np.where(allowed, s, -np.inf)
            m = np.max(z, axis=1, keepdims=True)
            e = np.where(allowed, np.exp(z - m), 0.0)
            tot = e.sum(axis=1, keepdims=True)
            out[rows, hh, :] = (e / tot) @ C
            lse[rows, hh] = (m + np.log(tot))[:, 0]
    return out, lse


def latent_attention_backward(q_lat, c_lat, kv_offsets, hq_offsets, n_cand, scale,
                              d_out):
    """Gradients of latent_attention's output with respect to q_lat and c_lat.

    [LLaTTE] mentions training with FlashAttention; this is the backward of
    the attention core in latent space (the derivative of the definition,
    written out): per user and head, with p = softmax over the allowed keys
    of s = scale * q . C_j and out = sum_j p_j C_j,
        dp_j = d_out . C_j,   D = d_out . out,   ds_j = p_j (dp_j - D),
        d_q  = scale * sum_j ds_j C_j,
        d_C_j += p_j d_out + scale * ds_j q      (over every query row and
                                                  head that sees key j; C is
                                                  both key and value).
    Returns (d_q [Mtot, h, r], d_c [Ktot, r]).
    """
    kv_offsets = np.asarray(kv_offsets, dtype=np.int64)
    hq_offsets = np.asarray(hq_offsets, dtype=np.int64)
    B = kv_offsets.size - 1
    nc = B * n_cand
    h = q_lat.shape[1]
    d_q = np.zeros_like(q_lat)
    d_c = np.zeros_like(c_lat)
    for u in range(B):
        C = c_lat[kv_offsets[u]:kv_offsets[u + 1]]
        K = C.shape[0]
        n = int(hq_offsets[u + 1] - hq_offsets[u])
        rows = list(range(nc + hq_offsets[u], nc + hq_offsets[u + 1])) + \
            list(range(u * n_cand, (u + 1) * n_cand))
        allowed = history_query_mask(K, n, n_cand)
        for hh in range(h):
            q = q_lat[rows, hh, :]
            g = d_out[rows, hh, :]
            s = (q @ C.T) * scale
            z = np.where(allowed, s, -np.inf)
            m = np.max(z, axis=1, keepdims=True)
            e = np.where(allowed, np.exp(z - m), 0.0)
            p = e / e.sum(axis=1, keepdims=True)
            o = p @ C
            dp = g @ C.T
            D = np.sum(g * o, axis=1, keepdims=True)
            ds = p * (dp - D)
            d_q[rows, hh, :] = scale * (ds @ C)
            d_c[kv_offsets[u]:kv_offsets[u + 1]] += p.T @ g + scale * (ds.T @ q)
    return d_q, d_c


# ---------------------------------------------------------------- counting

def ffn_block_backward(R1, g2, W1, W2, d_out, eps=1e-6):
    """Gradients of the pre-norm FFN sublayer of the [LLaTTE] A.2 layer
    equation (pre-norm reading), R2 = R1 + GELU(RMSNorm(R1) g2 W1) W2,
    row-wise over the rows of R1 [M, d], given d_out = dL/dR2 [M, d].

    [LLaTTE] trains the model (FlashAttention on H100s is mentioned); this
    is the derivative of the definition, written out step by step:
        s = (mean(R1^2) + eps)^-1/2 per row,  xh = R1 s,  H2 = xh g2,
        A = H2 W1,  G = GELU(A),
        dW2 = G^T d_out,          dG = d_out W2^T,
        dA  = dG * GELU'(A),      GELU'(a) = Phi(a) + a phi(a),
        dW1 = H2^T dA,            dH2 = dA W1^T,
        dg2 = sum over rows of dH2 * xh,   dxh = dH2 * g2,
        dR1 = d_out + s (dxh - xh mean(dxh * xh))   (per row).
    Returns (dR1 [M, d], dg2 [d], dW1 [d, d_ff], dW2 [d_ff, d]).
    """
    ms = np.mean(R1 * R1, axis=-1, keepdims=True)
    s = 1.0 / np.sqrt(ms + eps)
    xh = R1 * s
    H2 = xh * g2
    A = H2 @ W1
    G = gelu(A)
    dW2 = G.T @ d_out
    dG = d_out @ W2.T
    phi = np.exp(-0.5 * A * A) / math.sqrt(2.0 * math.pi)
    Phi = 0.5 * (1.0 + _erf(A / math.sqrt(2.0)))
    dA = dG * (Phi + A * phi)
    dW1 = H2.T @ dA
    dH2 = dA @ W1.T
    dg2 = np.sum(dH2 * xh, axis=0)
    dxh = dH2 * g2
    dR1 = d_out + s * (dxh - xh * np.mean(dxh * xh, axis=-1, keepdims=True))
    return dR1, dg2, dW1, dW2


def rmsnorm_backward(x, g, dy, eps=1e-6):
    """Gradients of y = RMSNorm(x) g (rmsnorm above) over the last axis:
    with s = (mean(x^2) + eps)^-1/2 and xh = x s per row,
        dg = sum over rows of dy * xh,
        dx = s (dy g - xh mean(dy g xh))   (per row).
    Returns (dx, dg)."""
    s = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    xh = x * s
    dxh = dy * g
    dx = s * (dxh - xh * np.mean(dxh * xh, axis=-1, keepdims=True))
    dg = np.sum((dy * xh).reshape(-1, x.shape[-1]), axis=0)
    return dx, dg


def attention_sublayer_backward(Rh, Rc, n, W, cfg, dRq):
    """Gradients of the attention sublayer of one pre-norm MLA layer on one
    user, R1 = Rq + MLA(RMSNorm(R) g1) (the first half of mla_layer, full-rank
    queries), given dRq = dL/dR1 for the query rows (the last n history rows,
    then the n_c candidate rows).

    [LLaTTE] A.3 non-absorbed MLA: C = RMSNorm(H W_dkv) g_c (or H W_dkv
    without the latent norm), per head K = C W_uk, V = C W_uv,
    P = softmax(q K^T / sqrt(d_k)) over the allowed keys, o = P V, then
    A = o W_o; A.2 layer equation (pre-norm reading) for the residual. The
    derivative written out, per head:
        dV = P^T do,  dP = do V^T,  dS = P (dP - rowsum(dP P)),
        dq = dS K / sqrt(d_k),  dK = dS^T q / sqrt(d_k),
        dW_uv += C^T dV,  dW_uk += C^T dK,  dC += dV W_uv^T + dK W_uk^T;
    then dW_uq = Hq^T dq, dH(query rows) += dq W_uq^T, the latent norm's
    backward, dW_dkv = H^T dC0, dH += dC0 W_dkv^T, and the pre-attention
    norm's backward plus the residual.
    Returns (dRh [K, d], dRc [n_c, d], grads) with grads holding g1, W_dkv,
    g_c (when the latent norm is on), W_uq, W_uk, W_uv, W_o.
    """
    d, h, dk, r = cfg.d, cfg.h, cfg.dk, cfg.r
    eps = cfg.eps
    K = Rh.shape[0]
    n_c = Rc.shape[0]
    H = rmsnorm(Rh, W["g1"], eps)
    Hc = rmsnorm(Rc, W["g1"], eps)
    C0 = H @ W["W_dkv"]
    C = rmsnorm(C0, W["g_c"], eps) if cfg.latent_norm else C0
    Hq = np.concatenate([H[K - n:], Hc], axis=0)
    M = Hq.shape[0]
    q = (Hq @ W["W_uq"]).reshape(M, h, dk)
    allowed = history_query_mask(K, n, n_c)
    scale = 1.0 / math.sqrt(dk)
    Wuk = W["W_uk"].reshape(r, h, dk)
    Wuv = W["W_uv"].reshape(r, h, dk)
    o = np.empty((M, h, dk))
    P, Kh, Vh = [], [], []
    for hh in range(h):
        Kh.append(C @ Wuk[:, hh, :])
        Vh.append(C @ Wuv[:, hh, :])
        P.append(softmax_masked((q[:, hh, :] @ Kh[hh].T) * scale, allowed))
        o[:, hh, :] = P[hh] @ Vh[hh]
    g = {}
    g["W_o"] = o.reshape(M, h * dk).T @ dRq
    do = (dRq @ W["W_o"].T).reshape(M, h, dk)
    dq = np.empty((M, h, dk))
    dWuk = np.zeros((r, h, dk))
    dWuv = np.zeros((r, h, dk))
    dC = np.zeros_like(C)
    for hh in range(h):
        dV = P[hh].T @ do[:, hh, :]
        dP = do[:, hh, :] @ Vh[hh].T
        dS = P[hh] * (dP - np.sum(dP * P[hh], axis=1, keepdims=True))
        dq[:, hh, :] = dS @ Kh[hh] * scale
        dK = dS.T @ q[:, hh, :] * scale
        dWuv[:, hh, :] = C.T @ dV
        dWuk[:, hh, :] = C.T @ dK
        dC += dV @ Wuv[:, hh, :].T + dK @ Wuk[:, hh, :].T
    g["W_uk"] = dWuk.reshape(r, h * dk)
    g["W_uv"] = dWuv.reshape(r, h * dk)
    dq = dq.reshape(M, h * dk)
    g["W_uq"] = Hq.T @ dq
    dHq = dq @ W["W_uq"].T
    if cfg.latent_norm:
        dC0, g["g_c"] = rmsnorm_backward(C0, W["g_c"], dC, eps)
    else:
        dC0 = dC
    g["W_dkv"] = H.T @ dC0
    dH = dC0 @ W["W_dkv"].T
    dH[K - n:] += dHq[:n]
    dRh, dg1h = rmsnorm_backward(Rh, W["g1"], dH, eps)
    dRc, dg1c = rmsnorm_backward(Rc, W["g1"], dHq[n:], eps)
    g["g1"] = dg1h + dg1c
    dRh[K - n:] += dRq[:n]
    dRc = dRc + dRq[n:]
    return dRh, dRc, g


def forward_backward(cfg, W, hist, offsets, cand=None, ctx=None, d_hist=None,
                     d_cand=None, d_emb=None):
    """Gradients of L = sum <d_hist, out_hist> + <d_cand, out_cand> +
    <d_emb, emb> through the whole forward above (pre-norm layers, full-rank
    queries), for every user.

    [LLaTTE] trains the sequence module end to end (section 1.5.1); this is
    the chain rule through section 1.3.2's steps, using the sublayer
    derivatives above ([LLaTTE] A.2 layer equation, A.3 MLA):
      readout: emb = flatten(S) W_p, so dS = (d_emb W_p^T) reshaped and
        dW_p = flatten(S)^T d_emb; the readout layer is a layer with n = 0
        whose candidate rows are the seeds: its input-row gradients go to
        the last layer's history outputs and (summed over users) the seeds;
      layer l (last to first): the output rows are the layer's query rows
        (last n_l history rows, then candidates); the FFN sublayer's
        backward gives dR1, the attention sublayer's backward the gradients
        of all K_l input rows and of the candidates. Layer l's input rows
        are layer l-1's output rows (the pyramid keeps the last rows), so
        they are layer l-1's output gradients; rows trimmed by the pyramid
        get only the key/value terms of the layer that saw them last;
      fusion: Q0 = [x ; c] W_q, so dW_q = [x ; c]^T dQ0 and d[x ; c] =
        dQ0 W_q^T (the context part summed over the user's candidates).
    d_hist: per-user list of [n_N(u), d] (None = zeros); d_cand [B*n_q, d];
    d_emb [B, d_out] (or [B, n_seeds*d] without W_p). Returns a dict: 'layers'
    (per layer: g1, W_dkv, g_c, W_uq, W_uk, W_uv, W_o, g2, W1, W2), and,
    where present, 'readout', 'seeds', 'W_p', 'W_q', then 'hist'
    [total_rows, d], 'cand' [B*n_q, d], 'ctx' [B, d_c].
    """
    if cfg.norm_mode != "pre":
        raise ValueError("the backward follows the pre-norm layer")
    offsets = np.asarray(offsets, dtype=np.int64)
    lengths = offsets[1:] - offsets[:-1]
    B = lengths.size
    keep = pyramid_counts(cfg.pyramid, lengths, cfg.N)
    f64 = lambda a: None if a is None else np.asarray(a, dtype=np.float64)
    layers = [{k: f64(v) for k, v in lw.items()} for lw in W["layers"]]
    if any("W_dq" in lw for lw in layers):
        raise ValueError("the backward follows the full-rank query path")
    ro = {k: f64(v) for k, v in W["readout"].items()} if cfg.n_seeds > 0 else None
    W_q = f64(W.get("W_q"))
    W_p = f64(W.get("W_p")) if cfg.n_seeds > 0 else None
    seeds = f64(W.get("seeds"))
    keys = ("g1", "W_dkv", "g_c", "W_uq", "W_uk", "W_uv", "W_o", "g2", "W1", "W2")
    zeros_like = lambda lw: {k: np.zeros_like(lw[k]) for k in keys if k in lw}
    g_layers = [zeros_like(lw) for lw in layers]
    res = {"layers": g_layers, "hist": np.zeros((int(offsets[-1]), cfg.d)),
           "cand": np.zeros((B * cfg.n_q, cfg.d)), "ctx": np.zeros((B, cfg.d_c))}
    if ro is not None:
        res["readout"] = zeros_like(ro)
        res["seeds"] = np.zeros_like(seeds)
        if W_p is not None:
            res["W_p"] = np.zeros_like(W_p)
    if cfg.n_q > 0:
        res["W_q"] = np.zeros_like(W_q)

    def layer_backward(Rh, Rc, n, lw, gw, dR2):
        R1 = mla_layer(Rh, Rc, n, lw, cfg, return_r1=True)[1]
        dR1, dg2, dW1, dW2 = ffn_block_backward(R1, lw["g2"], lw["W1"], lw["W2"], dR2, cfg.eps)
        dRh, dRc, g = attention_sublayer_backward(Rh, Rc, n, lw, cfg, dR1)
        g.update(g2=dg2, W1=dW1, W2=dW2)
        for k, v in g.items():
            gw[k] += v
        return dRh, dRc

    for u in range(B):
        Rh = f64(hist[offsets[u]:offsets[u + 1]])
        xc = None
        if cfg.n_q > 0:
            xu = f64(cand[u * cfg.n_q:(u + 1) * cfg.n_q])
            cu = f64(ctx[u]) if (ctx is not None and cfg.d_c > 0) else None
            xc = xu if cu is None else np.concatenate(
                [xu, np.broadcast_to(cu, (cfg.n_q, cu.size))], axis=1)
            Rc = xc @ W_q
        else:
            Rc = np.zeros((0, cfg.d))
        ins = []
        for l in range(cfg.N):
            n = int(keep[l, u])
            ins.append((Rh, Rc, n))
            Rh, Rc = mla_layer(Rh, Rc, n, layers[l], cfg)
        dRh = np.zeros_like(Rh) if d_hist is None else f64(d_hist[u]).copy()
        dRc = (np.zeros((cfg.n_q, cfg.d)) if d_cand is None
               else f64(d_cand[u * cfg.n_q:(u + 1) * cfg.n_q]).copy())
        if ro is not None:
            _, S = mla_layer(Rh, seeds, 0, ro, cfg)
            de = np.zeros(S.size) if d_emb is None else f64(d_emb[u])
            if W_p is not None:
                res["W_p"] += np.outer(S.reshape(-1), de)
                de = W_p @ de
            dRh_ro, dS = layer_backward(Rh, seeds, 0, ro, res["readout"], de.reshape(S.shape))
            dRh = dRh + dRh_ro
            res["seeds"] += dS
        for l in range(cfg.N - 1, -1, -1):
            Rh_in, Rc_in, n = ins[l]
            dRh, dRc = layer_backward(Rh_in, Rc_in, n, layers[l], g_layers[l],
                                      np.concatenate([dRh, dRc], axis=0))
        res["hist"][offsets[u]:offsets[u + 1]] = dRh
        if cfg.n_q > 0:
            res["W_q"] += xc.T @ dRc
            dxc = dRc @ W_q.T
            res["cand"][u * cfg.n_q:(u + 1) * cfg.n_q] = dxc[:, :cfg.d]
            if cfg.d_c > 0:
                res["ctx"][u] = dxc[:, cfg.d:].sum(axis=0)
    return res


def unmasked_pairs(cfg, lengths):
    """Allowed (query, key) pairs per layer, counted from the explicit masks."""
    lengths = np.asarray(lengths, dtype=np.int64)
    keep = pyramid_counts(cfg.pyramid, lengths, cfg.N)
    per_layer = np.zeros(cfg.N + (1 if cfg.n_seeds else 0), dtype=np.int64)
    for u, Lu in enumerate(lengths):
        K = int(Lu)
        for l in range(cfg.N):
            n = int(keep[l, u])
            per_layer[l] += int(history_query_mask(K, n, cfg.n_q).sum())
            K = n
        if cfg.n_seeds:
            per_layer[cfg.N] += int(history_query_mask(K, 0, cfg.n_seeds).sum())
    return per_layer


def flop_count(cfg, lengths, absorbed=True):
    """Algorithmic FLOPs of one batch: 2mnk per matrix product, plus per
    allowed (query, key) pair 4*r*h (absorbed) or 4*d_k*h (non-absorbed).

    Matrix products per layer, with K history rows in and M = n + n_q query
    rows: W_dkv (K x d x r), W_uq (M x d x h*dk; low-rank: W_dq M x d x r_q
    and W_uq M x r_q x h*dk), then absorbed W_uk and W_uv
    on the queries (M x dk x r per head, each) or non-absorbed W_uk and W_uv on
    the keys (K x r x h*dk, each), W_o (M x h*dk x d), W1 and W2 (M x d x 4d).
    Plus the fusion (B*n_q x (d+d_c) x d), the readout projection
    (B x n_s*d x d_out) and the W_s token build (rows x d_sem x d).
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    keep = pyramid_counts(cfg.pyramid, lengths, cfg.N)
    d, h, dk, r = cfg.d, cfg.h, cfg.dk, cfg.r
    pairs = unmasked_pairs(cfg, lengths)
    total = 0
    Ks = lengths.copy()
    nl = cfg.N + (1 if cfg.n_seeds else 0)
    for l in range(nl):
        if l < cfg.N:
            n = keep[l]
            nq = cfg.n_q
        else:
            n = np.zeros_like(Ks)
            nq = cfg.n_seeds
        Kt = int(Ks.sum())
        Mt = int(n.sum()) + nq * cfg.B
        if getattr(cfg, "r_q", 0):
            total += 2 * Kt * d * r + 2 * Mt * d * cfg.r_q + 2 * Mt * cfg.r_q * h * dk
        else:
            total += 2 * Kt * d * r + 2 * Mt * d * h * dk
        if absorbed:
            total += 2 * (2 * Mt * h * dk * r) + 4 * r * h * int(pairs[l])
        else:
            total += 2 * (2 * Kt * r * h * dk) + 4 * dk * h * int(pairs[l])
        total += 2 * Mt * h * dk * d + 2 * (2 * Mt * d * cfg.d_ff)
        Ks = n
    if cfg.n_q > 0:
        total += 2 * cfg.B * cfg.n_q * (d + cfg.d_c) * d
    if cfg.n_seeds:
        total += 2 * cfg.B * cfg.n_seeds * d * cfg.d_out
    if cfg.semantic is not None:
        rows = int(lengths.sum()) + cfg.B * cfg.n_q
        total += 2 * rows * cfg.semantic.d_sem * d
    return total
