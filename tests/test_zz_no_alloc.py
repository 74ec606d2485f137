"""The no-allocation attention entry (fixed device scratch) against the
workspace entry it shares its kernels with, through the C ABI: the same
outputs on the same inputs, over two calls in a row where the second is
smaller (the scratch keeps the first call's plan), and against the oracle."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import llatte_oracle as O

pytestmark = pytest.mark.gpu


def L():
    from target_aware_latent_amd import llatte
    return llatte


def _inputs(dt, h, r, K, n, n_cand, seed):
    rng = np.random.default_rng(seed)
    K, n = np.asarray(K), np.asarray(n)
    B = K.size
    kv_off = np.concatenate([[0], np.cumsum(K)]).astype(np.int32)
    hq_off = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    Mtot = int(B * n_cand + hq_off[-1])
    q = rng.standard_normal((Mtot, h, r)) * 0.5
    C = rng.standard_normal((int(kv_off[-1]), r))
    if dt == "bf16":
        q, C = synth.round_bf16(q), synth.round_bf16(C)
    return B, kv_off, hq_off, Mtot, np.asarray(q, np.float32), np.asarray(C, np.float32)


def _run(dt, h, r, K, n, n_cand, seed):
    B, kv_off, hq_off, Mtot, q, C = _inputs(dt, h, r, K, n, n_cand, seed)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    code = L().LLATTE_BF16 if dt == "bf16" else L().LLATTE_F32
    scale = 1.0 / math.sqrt(64)
    ad = L().llatte_attn_desc(h, r, n_cand, code, scale)
    qd = torch.from_numpy(q).cuda().to(tdt)
    Cd = torch.from_numpy(C).cuda().to(tdt)
    kvd = torch.from_numpy(kv_off).cuda()
    hqd = torch.from_numpy(hq_off).cuda()
    Ktot = int(kv_off[-1])
    # the entry with a caller workspace
    ws = torch.empty(L().llatte_mla_attention_workspace_size(ad, B, Mtot, Ktot),
                     dtype=torch.uint8, device="cuda")
    out_ws = torch.full((Mtot, h, r), float("nan"), device="cuda")
    lse_ws = torch.full((Mtot, h), float("nan"), device="cuda")
    L().llatte_mla_attention(ad, qd, Cd, kvd, hqd, B, Mtot, Ktot, out_ws, lse_ws, ws)
    # the entry with the fixed scratch
    out_na = torch.full((Mtot, h, r), float("nan"), device="cuda")
    lse_na = torch.full((Mtot, h), float("nan"), device="cuda")
    L().llatte_mla_attention_noalloc(ad, qd, Cd, kvd, hqd, B, Mtot, Ktot, out_na, lse_na)
    torch.cuda.synchronize()
    ref, ref_lse = O.latent_attention(q.astype(np.float64), C.astype(np.float64),
                                      kv_off, hq_off, n_cand, scale)
    return (out_ws.cpu().numpy(), lse_ws.cpu().numpy(), out_na.cpu().numpy(),
            lse_na.cpu().numpy(), ref, ref_lse)


def _bar(dt, g, r):
    g, r = np.asarray(g, np.float64), np.asarray(r, np.float64)
    rms = math.sqrt(float(np.mean(r * r)))
    if dt == "f32":
        return float(np.max(np.abs(g - r) / np.maximum(np.abs(r), rms))), 1e-4
    return float(np.max(np.abs(g - r)) / rms), 2e-2


@pytest.mark.parametrize("dt,h,r", [("bf16", 8, 128), ("bf16", 4, 64), ("f32", 2, 32)])
def test_noalloc_matches_workspace_entry_over_two_calls(dt, h, r):
    # first call the larger batch, then a smaller one: the second plan is
    # written over the first in the same fixed scratch
    cases = [([700, 50, 1, 333], [300, 50, 1, 120], 5, 1),
             ([90, 33], [90, 3], 2, 2)]
    for K, n, nc, seed in cases:
        print(f"noalloc {dt} h{h} r{r} K={K} n={n} nc={nc}", flush=True)
        out_ws, lse_ws, out_na, lse_na, ref, ref_lse = _run(dt, h, r, K, n, nc, seed)
        assert np.isfinite(out_na).all() and np.isfinite(lse_na).all()
        # same kernels on the same inputs: identical results
        assert np.array_equal(out_na, out_ws)
        assert np.array_equal(lse_na, lse_ws)
        e, tol = _bar(dt, out_na, ref)
        print(f"  err vs oracle {e:.3e} (tol {tol})", flush=True)
        assert e <= tol
        assert np.max(np.abs(lse_na - ref_lse)) < (1e-4 if dt == "f32" else 2e-3)
