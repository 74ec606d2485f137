"""The five synthetic workloads of the LLaTTE sequence-module forward.

Shapes follow the workloads the pages describe: an online ranker reading about
400 recent events with candidate query tokens (LLaTTE, section 1.6 on the
multi-stage design) and a deep upstream model over 200-1600 events with a
fixed-size readout (LLaTTE, section 1.5.2 sequence-length sweep; Appendix A.2
sequence summaries). Sizes are the ones fixed for this build's workloads:

  c1  correctness case, fp32, one layer
  c2  online-ranker shape, 3 layers, 16 candidate tokens
  c3  upstream user model, 6 layers, L=1600, readout to a 2048-d embedding
  c4  jagged batch, lengths uniform in [200, 1600], halving pyramid, floor 64
  c5  width/depth scale-up with hashed-ID + semantic token build, 12 layers
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class PyramidRule:
    """How many history rows stay as queries at each layer.

    kind 'fixed':     values[l] is the keep count of layer l+1 (capped by the
                      previous layer's count for short users).
    kind 'halving':   keep = max(min(floor, L_u), L_u >> l) at layer l+1.
    kind 'geometric': keep list interpolates start -> end geometrically over
                      the layers (rounded half-up), capped like 'fixed'.
    """
    kind: str
    values: Tuple[int, ...] = ()
    floor: int = 0
    start: int = 0
    end: int = 0


@dataclass(frozen=True)
class SemanticSpec:
    """Token build from a hashed-ID table plus a projected semantic vector."""
    vocab: int = 1_000_000
    d_sem: int = 384
    zipf_s: float = 1.1


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    L: Optional[int]                 # fixed history length, or None if jagged
    len_range: Optional[Tuple[int, int]]  # inclusive [lo, hi] when jagged
    d: int
    h: int
    dk: int
    r: int
    n_q: int
    d_c: int
    N: int
    pyramid: PyramidRule
    dtype: str                       # 'f32' or 'bf16'
    norm_mode: str = "pre"           # 'pre' or 'post'
    latent_norm: bool = True
    eps: float = 1e-6
    n_seeds: int = 0                 # readout: learned seed queries (0 = none)
    d_out: int = 0                   # readout: embedding width
    semantic: Optional[SemanticSpec] = None
    gain_jitter: float = 0.0         # gains = 1 + jitter * N(0,1)
    r_q: int = 0                     # query rank: 0 = full-rank W_uq [d, h*dk];
                                     # > 0 = RMSNorm(H W_dq) g_q W_uq [r_q, h*dk]

    @property
    def d_ff(self) -> int:
        return 4 * self.d


CONFIGS = {
    "c1": Config("c1", B=4, L=32, len_range=None, d=64, h=2, dk=32, r=16,
                 n_q=4, d_c=32, N=1, pyramid=PyramidRule("fixed", (32,)),
                 dtype="f32"),
    "c2": Config("c2", B=256, L=400, len_range=None, d=256, h=4, dk=64, r=64,
                 n_q=16, d_c=128, N=3,
                 pyramid=PyramidRule("fixed", (400, 200, 100)), dtype="bf16"),
    "c3": Config("c3", B=64, L=1600, len_range=None, d=512, h=8, dk=64,
                 r=128, n_q=0, d_c=0, N=6,
                 pyramid=PyramidRule("fixed", (1600, 800, 400, 200, 100, 50)),
                 dtype="bf16", n_seeds=4, d_out=2048),
    "c4": Config("c4", B=128, L=None, len_range=(200, 1600), d=256, h=4,
                 dk=64, r=64, n_q=8, d_c=128, N=4,
                 pyramid=PyramidRule("halving", floor=64), dtype="bf16"),
    "c5": Config("c5", B=32, L=1600, len_range=None, d=1024, h=16, dk=64,
                 r=256, n_q=16, d_c=128, N=12,
                 pyramid=PyramidRule("geometric", start=1600, end=50),
                 dtype="bf16", semantic=SemanticSpec()),
}


def get_config(name: str, **overrides) -> Config:
    """A named workload, optionally with fields replaced (smaller B, etc.)."""
    import dataclasses
    cfg = CONFIGS[name]
    return dataclasses.replace(cfg, **overrides) if overrides else cfg
