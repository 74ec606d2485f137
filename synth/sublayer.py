"""Seeded inputs of one attention sublayer (for its backward): weights with
fan-in scaling rounded to bf16, gains 1 + 0.1 N(0, 1) in float32, history
and candidate rows and the output gradient N(0, 1) in float32. Draw order:
g1, W_dkv, g_c, W_uq, W_uk, W_uv, W_o, history rows per user, candidate rows
per user, then the output gradient of all query rows. No arithmetic of the
method happens here."""
import math

import numpy as np

from .gen import round_bf16


def sublayer_case(d, h, dk, r, n_cand, K, n, seed=0):
    """Returns W (float64 arrays holding the bf16 / float32 values), the
    history rows Rh and candidate rows Rc (lists per user, float32), the
    output gradient dout ([Mtot, d] float32, rows: candidates user-major,
    then the history query rows user-major) and the kv / hq offsets."""
    rng = np.random.default_rng(seed)
    B = len(K)
    W = {"g1": 1 + 0.1 * rng.standard_normal(d),
         "W_dkv": round_bf16(rng.standard_normal((d, r)) / math.sqrt(d)),
         "g_c": 1 + 0.1 * rng.standard_normal(r),
         "W_uq": round_bf16(rng.standard_normal((d, h * dk)) / math.sqrt(d)),
         "W_uk": round_bf16(rng.standard_normal((r, h * dk)) / math.sqrt(r)),
         "W_uv": round_bf16(rng.standard_normal((r, h * dk)) / math.sqrt(r)),
         "W_o": round_bf16(rng.standard_normal((h * dk, d)) / math.sqrt(h * dk))}
    W = {k: np.asarray(v, np.float32).astype(np.float64) for k, v in W.items()}
    Rh = [rng.standard_normal((k, d)).astype(np.float32) for k in K]
    Rc = [rng.standard_normal((n_cand, d)).astype(np.float32) for _ in K]
    Mtot = B * n_cand + int(sum(n))
    dout = rng.standard_normal((Mtot, d)).astype(np.float32)
    kv = np.concatenate([[0], np.cumsum(K)]).astype(np.int32)
    hq = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    return W, Rh, Rc, dout, kv, hq
