"""Host-side checks of the benchmark's accounting (CPU only)."""
import numpy as np
import pytest

import synth
from oracle import llatte_oracle as O


@pytest.mark.parametrize("name,r_q", [("c1", 0), ("c2", 0), ("c3", 0), ("c4", 0),
                                      ("c3", 256), ("c2", 96)])
def test_bench_flop_count_matches_oracle_count(name, r_q):
    import bench
    cfg = synth.get_config(name, r_q=r_q)
    lengths = synth.generate(cfg)["inputs"]["lengths"] if cfg.len_range else \
        np.full(cfg.B, cfg.L)
    assert bench.absorbed_flops(cfg, lengths) == O.flop_count(cfg, lengths, True)
    assert bench.non_absorbed_flops(cfg, lengths) == O.flop_count(cfg, lengths, False)


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr
