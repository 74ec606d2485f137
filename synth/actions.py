"""Seeded synthetic workloads of the action tokenization.

Shapes, sizes and random draws only (ids, timestamps, dense meta features,
tables and weights); none of the method's arithmetic. The page gives no
feature schema, so the one below is a stated choice: five fields per action
(timestamp, type, item, surface, dense meta vector), with the item ids drawn
Zipf(1.1)-distributed over a hashed table as in the token-build workload.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

from .gen import _HASH_MUL, round_bf16


@dataclass(frozen=True)
class ActionConfig:
    name: str
    B: int
    lengths: Optional[Tuple[int, ...]]  # per user; None: all equal to L
    L: int
    d: int
    d_type: int
    d_item: int
    d_surf: int
    d_time: int
    d_meta: int
    d_meta_emb: int
    d_hidden: int
    d_enc: int
    V_type: int
    V_item: int
    V_surf: int
    n_buckets: int
    dtype: str
    zipf_s: float = 1.1
    future_frac: float = 0.0   # share of actions stamped after the request
    mean_gap_s: float = 3600.0

    @property
    def d_in(self):
        return self.d_type + self.d_item + self.d_surf + self.d_time + self.d_meta_emb


ACTION_CONFIGS = {
    # small, ragged, several users; every field narrow
    "a_small": ActionConfig("a_small", B=5, lengths=(1, 37, 64, 130, 3), L=0, d=64,
                            d_type=8, d_item=16, d_surf=8, d_time=8, d_meta=4,
                            d_meta_emb=8, d_hidden=96, d_enc=16, V_type=7,
                            V_item=1000, V_surf=5, n_buckets=24, dtype="f32",
                            future_frac=0.05),
    "a_small_bf16": ActionConfig("a_small_bf16", B=5, lengths=(1, 37, 64, 130, 3), L=0,
                                 d=64, d_type=8, d_item=16, d_surf=8, d_time=8,
                                 d_meta=8, d_meta_emb=8, d_hidden=96, d_enc=16,
                                 V_type=7, V_item=1000, V_surf=5, n_buckets=24,
                                 dtype="bf16", future_frac=0.05),
    # the upstream shape: 64 users x 1600 actions into d = 512 tokens
    "a_c3": ActionConfig("a_c3", B=64, lengths=None, L=1600, d=512, d_type=32,
                         d_item=128, d_surf=32, d_time=32, d_meta=16,
                         d_meta_emb=32, d_hidden=1024, d_enc=64, V_type=32,
                         V_item=1_000_000, V_surf=16, n_buckets=32, dtype="bf16"),
}


def get_action_config(name):
    return ACTION_CONFIGS[name]


def _q(cfg, a):
    a = np.asarray(a, dtype=np.float32)
    return round_bf16(a) if cfg.dtype == "bf16" else a


def _zipf_ids(rng, vocab, s, n):
    k = np.arange(1, vocab + 1, dtype=np.float64)
    cdf = np.cumsum(k ** (-s))
    cdf /= cdf[-1]
    rank = np.minimum(np.searchsorted(cdf, rng.random(n), side="right"), vocab - 1)
    return ((rank.astype(np.int64) * _HASH_MUL) % vocab).astype(np.int32)


def generate_actions(cfg, seed=0):
    """Weights, then inputs, in a fixed draw order."""
    rng = np.random.default_rng(seed)
    w = lambda fan_in, shape: _q(cfg, rng.standard_normal(shape) / np.sqrt(fan_in))
    W = {
        "E_type": _q(cfg, rng.standard_normal((cfg.V_type, cfg.d_type))),
        "E_item": _q(cfg, rng.standard_normal((cfg.V_item, cfg.d_item), dtype=np.float32)),
        "E_surf": _q(cfg, rng.standard_normal((cfg.V_surf, cfg.d_surf))),
        "E_time": _q(cfg, rng.standard_normal((cfg.n_buckets, cfg.d_time))),
        "W_meta": w(cfg.d_meta, (cfg.d_meta, cfg.d_meta_emb)),
        "W_a": w(cfg.d_in, (cfg.d_in, cfg.d_hidden)),
        "W_b": w(cfg.d_hidden, (cfg.d_hidden, cfg.d)),
    }
    lengths = np.array(cfg.lengths if cfg.lengths is not None else [cfg.L] * cfg.B,
                       dtype=np.int64)
    offsets = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    n = int(offsets[-1])
    t_req = (1_700_000_000 + 3600 * np.arange(cfg.B)).astype(np.int32)
    tau = np.empty(n, dtype=np.int32)
    for u in range(cfg.B):
        Lu = int(lengths[u])
        gaps = rng.exponential(cfg.mean_gap_s, Lu)
        age = np.cumsum(gaps)[::-1]          # oldest first, newest last
        tau[offsets[u]:offsets[u + 1]] = t_req[u] - np.floor(age).astype(np.int64)
    if cfg.future_frac:
        fut = rng.random(n) < cfg.future_frac
        tau[fut] = t_req[np.searchsorted(offsets, np.nonzero(fut)[0], side="right") - 1] \
            + rng.integers(1, 600, int(fut.sum()))
    I = {
        "offsets": offsets, "t_req": t_req, "tau": tau,
        "type_id": rng.integers(0, cfg.V_type, n).astype(np.int32),
        "item_id": _zipf_ids(rng, cfg.V_item, cfg.zipf_s, n),
        "surf_id": rng.integers(0, cfg.V_surf, n).astype(np.int32),
        "meta": _q(cfg, rng.standard_normal((n, cfg.d_meta))),
    }
    return {"weights": W, "inputs": I}
