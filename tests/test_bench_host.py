"""Host-side checks of the benchmark's accounting (CPU only)."""
import numpy as np
import pytest

import synth
from oracle import llatte_oracle as O


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_bench_flop_count_matches_oracle_count(name):
    import bench
    cfg = synth.get_config(name)
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
