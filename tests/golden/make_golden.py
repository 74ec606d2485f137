"""Write tests/golden/c1_digest.txt from the oracle (and nothing else).

The digest is a regression check of the fp64 oracle on the c1 workload; it is
written only after the oracle's pins pass. Run: python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import llatte_oracle as O  # noqa: E402


def main():
    cfg = synth.get_config("c1")
    p = synth.generate(cfg)
    I = p["inputs"]
    res = O.forward(cfg, p["weights"], I["hist"], I["offsets"], I.get("cand"),
                    I.get("ctx"))
    H = np.concatenate(res["hist"])
    C = np.concatenate(res["cand"])
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c1_digest.txt")
    with open(path, "w") as f:
        f.write("# fp64 oracle output digest, workload c1 (seed 0); regression only.\n")
        f.write("# Written by tests/golden/make_golden.py, which calls oracle/ only.\n")
        f.write(f"hist_sum = {H.sum():.17g}\n")
        f.write(f"hist_abs_sum = {np.abs(H).sum():.17g}\n")
        f.write(f"cand_sum = {C.sum():.17g}\n")
        f.write(f"cand_abs_sum = {np.abs(C).sum():.17g}\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
