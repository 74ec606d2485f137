"""Seeded synthetic workloads of the sequence summaries (LoRAMLP_k over the
flattened readout): base weights, per-summary rank-rho adapters and the
flattened readouts z. Shapes and random draws only."""
from dataclasses import dataclass

import numpy as np

from .gen import round_bf16


@dataclass(frozen=True)
class SummaryConfig:
    name: str
    B: int
    d_z: int        # n_seeds * d
    d_hidden: int
    d_seq: int
    rank: int
    K: int          # number of summaries
    dtype: str


SUMMARY_CONFIGS = {
    "s_small": SummaryConfig("s_small", B=5, d_z=64, d_hidden=96, d_seq=48, rank=4, K=3,
                             dtype="f32"),
    "s_small_bf16": SummaryConfig("s_small_bf16", B=5, d_z=64, d_hidden=96, d_seq=48,
                                  rank=8, K=3, dtype="bf16"),
    # the upstream readout: 4 seeds x 512 flattened to 2048, summaries of 2048
    "s_c3": SummaryConfig("s_c3", B=64, d_z=2048, d_hidden=2048, d_seq=2048, rank=16, K=2,
                          dtype="bf16"),
}


def get_summary_config(name):
    return SUMMARY_CONFIGS[name]


def generate_summaries(cfg, seed=0):
    rng = np.random.default_rng(seed)
    q = lambda a: round_bf16(a) if cfg.dtype == "bf16" else np.asarray(a, dtype=np.float32)
    w = lambda fan_in, shape, scale=1.0: q(scale * rng.standard_normal(shape) / np.sqrt(fan_in))
    K, r = cfg.K, cfg.rank
    L = {
        "W1": w(cfg.d_z, (cfg.d_z, cfg.d_hidden)),
        "W2": w(cfg.d_hidden, (cfg.d_hidden, cfg.d_seq)),
        "A1": w(cfg.d_z, (K, cfg.d_z, r)),
        "B1": w(r, (K, r, cfg.d_hidden), 0.5),
        "A2": w(cfg.d_hidden, (K, cfg.d_hidden, r)),
        "B2": w(r, (K, r, cfg.d_seq), 0.5),
    }
    z = q(rng.standard_normal((cfg.B, cfg.d_z)))
    return {"weights": L, "inputs": {"z": z}}
