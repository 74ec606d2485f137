"""Seeded synthetic weights and inputs (numpy, host).

Everything is drawn from ``numpy.random.default_rng(seed)`` in a fixed order:
lengths (jagged workloads), then per layer (g1, W_dkv, g_c, W_uq, W_uk, W_uv,
W_o, g2, W1, W2), then W_q, seeds, the readout layer, W_p, W_s, then the
inputs (history tokens or ids + semantic vectors, candidate tokens, context).

Distributions: tokens, candidate features, context, semantic vectors, table
rows and seeds are N(0, 1); a weight matrix with fan-in f is N(0, 1/f); gains
are 1 (or 1 + jitter * N(0, 1) when a test asks for it). For bf16 workloads
every drawn value is rounded once to bf16 (round to nearest even) and kept in
a float32 array, so both sides read the same numbers.

The hashed-ID table (1M x d) is drawn in independent blocks of TABLE_BLOCK
rows, each from its own seed sequence, so that any subset of rows can be
regenerated without drawing the whole table.
"""
import numpy as np

TABLE_BLOCK = 8192
_HASH_MUL = 2654435761  # odd multiplier; coprime with 10**6, so a bijection


def round_bf16(x):
    """Round to the nearest bf16 value (ties to even); returns float32."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).reshape(f.shape)


def _q(cfg, a):
    a = np.asarray(a, dtype=np.float32)
    return round_bf16(a) if cfg.dtype == "bf16" else a


def _w(rng, cfg, fan_in, shape):
    return _q(cfg, rng.standard_normal(shape) / np.sqrt(fan_in))


def _gain(rng, cfg, n):
    if cfg.gain_jitter:
        return (1.0 + cfg.gain_jitter * rng.standard_normal(n)).astype(np.float32)
    return np.ones(n, dtype=np.float32)


def _layer(rng, cfg):
    d, hd, r, rq = cfg.d, cfg.h * cfg.dk, cfg.r, cfg.r_q
    qin = rq if rq else d  # input width of W_uq
    L = {
        "g1": _gain(rng, cfg, d),
        "W_dkv": _w(rng, cfg, d, (d, r)),
        "g_c": _gain(rng, cfg, r),
        "W_uq": _w(rng, cfg, qin, (qin, hd)),
        "W_uk": _w(rng, cfg, r, (r, hd)),
        "W_uv": _w(rng, cfg, r, (r, hd)),
        "W_o": _w(rng, cfg, hd, (hd, d)),
        "g2": _gain(rng, cfg, d),
        "W1": _w(rng, cfg, d, (d, cfg.d_ff)),
        "W2": _w(rng, cfg, cfg.d_ff, (cfg.d_ff, d)),
    }
    if rq:  # low-rank query path, drawn after the rest of the layer
        L["W_dq"] = _w(rng, cfg, d, (d, rq))
        L["g_q"] = _gain(rng, cfg, rq)
    return L


def _lengths(rng, cfg):
    if cfg.len_range is not None:
        lo, hi = cfg.len_range
        return rng.integers(lo, hi + 1, cfg.B).astype(np.int64)
    return np.full(cfg.B, cfg.L, dtype=np.int64)


def _zipf_rows(rng, spec, n):
    """Zipf(s) ranks over 1..vocab by inverse CDF, hashed to table rows."""
    k = np.arange(1, spec.vocab + 1, dtype=np.float64)
    cdf = np.cumsum(k ** (-spec.zipf_s))
    cdf /= cdf[-1]
    u = rng.random(n)
    rank = np.minimum(np.searchsorted(cdf, u, side="right"), spec.vocab - 1)
    rows = (rank.astype(np.int64) * _HASH_MUL) % spec.vocab
    return rows.astype(np.int32)


def generate(cfg, seed=0, lengths=None):
    """All lengths, weights and inputs of one workload, in the fixed order.

    ``lengths`` replaces the workload's own per-user lengths (used for edge
    cases); when given, no lengths are drawn."""
    rng = np.random.default_rng(seed)
    if lengths is None:
        lengths = _lengths(rng, cfg)
    else:
        lengths = np.asarray(lengths, dtype=np.int64)
        assert lengths.size == cfg.B
    offsets = np.zeros(cfg.B + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(lengths)
    W = {"layers": [_layer(rng, cfg) for _ in range(cfg.N)]}
    if cfg.n_q > 0:
        W["W_q"] = _w(rng, cfg, cfg.d + cfg.d_c, (cfg.d + cfg.d_c, cfg.d))
    if cfg.n_seeds > 0:
        W["seeds"] = _q(cfg, rng.standard_normal((cfg.n_seeds, cfg.d)))
        W["readout"] = _layer(rng, cfg)
        W["W_p"] = _w(rng, cfg, cfg.n_seeds * cfg.d,
                      (cfg.n_seeds * cfg.d, cfg.d_out))
    if cfg.semantic is not None:
        W["W_s"] = _w(rng, cfg, cfg.semantic.d_sem, (cfg.semantic.d_sem, cfg.d))

    total = int(offsets[-1])
    nc = cfg.B * cfg.n_q
    I = {"lengths": lengths, "offsets": offsets}
    if cfg.semantic is None:
        I["hist"] = _q(cfg, rng.standard_normal((total, cfg.d)))
        if cfg.n_q > 0:
            I["cand"] = _q(cfg, rng.standard_normal((nc, cfg.d)))
    else:
        sp = cfg.semantic
        I["hist_ids"] = _zipf_rows(rng, sp, total)
        I["hist_sem"] = _q(cfg, rng.standard_normal((total, sp.d_sem)))
        if cfg.n_q > 0:
            I["cand_ids"] = _zipf_rows(rng, sp, nc)
            I["cand_sem"] = _q(cfg, rng.standard_normal((nc, sp.d_sem)))
    if cfg.n_q > 0 and cfg.d_c > 0:
        I["ctx"] = _q(cfg, rng.standard_normal((cfg.B, cfg.d_c)))
    return {"cfg": cfg, "seed": seed, "weights": W, "inputs": I}


def make_weights(cfg, seed=0):
    return generate(cfg, seed)["weights"]


def make_inputs(cfg, seed=0):
    return generate(cfg, seed)["inputs"]


def _table_block(cfg, seed, b):
    ss = np.random.SeedSequence([int(seed), 0x7AB1E, int(b)])
    blk = np.random.default_rng(ss).standard_normal(
        (TABLE_BLOCK, cfg.d), dtype=np.float32)
    return _q(cfg, blk)


def table_rows(cfg, seed, rows):
    """Rows of the hashed-ID table, regenerated block by block."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, cfg.d), dtype=np.float32)
    blocks = rows // TABLE_BLOCK
    for b in np.unique(blocks):
        sel = np.nonzero(blocks == b)[0]
        blk = _table_block(cfg, seed, b)
        out[sel] = blk[rows[sel] - b * TABLE_BLOCK]
    return out


def full_table(cfg, seed):
    """Yield (row0, block) for the whole table, TABLE_BLOCK rows at a time."""
    V = cfg.semantic.vocab
    for b in range((V + TABLE_BLOCK - 1) // TABLE_BLOCK):
        blk = _table_block(cfg, seed, b)
        n = min(TABLE_BLOCK, V - b * TABLE_BLOCK)
        yield b * TABLE_BLOCK, blk[:n]
