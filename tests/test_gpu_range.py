"""The bf16 attention core with values beyond fp16's range, through the C
ABI. The kernel computes in fp16 (more mantissa than bf16); the standalone
entry scales its bf16 inputs by powers of two into range first, so finite
inputs of any magnitude give finite results equal to the oracle's. The
cases keep the scores moderate (large latent rows with small queries, and
the reverse) or near zero (both small), so that what is checked is the
range handling: the common exponent that gives the scores exactly, and the
separate scaling of each side where there is none."""
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


# scores of standard deviation ~1, as in the other attention tests:
# sqrt(r) sigma_q sigma_c / 8 ~ 1
CASES = [
    # name, sigma of C, sigma of q, entry
    ("large_latent", 3e5, 2.4e-6, "workspace"),
    ("large_scaled_queries", 1.8e-6, 4e5, "workspace"),
    ("large_latent_noalloc", 2e6, 3.5e-7, "noalloc"),
    ("tiny_inputs", 1e-6, 7e5, "workspace"),
    # both small: the product of the two largest magnitudes (~2^-16) leaves
    # no common exponent for exact scores, so each side is scaled on its own
    # and the scores are scaled back (near-uniform softmax)
    ("tiny_product", 2e-3, 2e-3, "workspace"),
]


@pytest.mark.parametrize("name,cs,qs,entry", CASES, ids=[c[0] for c in CASES])
def test_large_finite_inputs_match_oracle(name, cs, qs, entry):
    rng = np.random.default_rng(11)
    h, r, nc = 8, 128, 3
    K = np.array([300, 65, 1])
    n = np.array([120, 65, 1])
    B = K.size
    kv_off = np.concatenate([[0], np.cumsum(K)]).astype(np.int32)
    hq_off = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    Mtot = int(B * nc + hq_off[-1])
    q = synth.round_bf16(rng.standard_normal((Mtot, h, r)) * qs).astype(np.float32)
    C = synth.round_bf16(rng.standard_normal((int(kv_off[-1]), r)) * cs).astype(np.float32)
    scale = 1.0 / math.sqrt(64)
    big = max(np.abs(C).max(), np.abs(q).max() * scale * 1.4427)
    assert big > 65504 or name in ("tiny_inputs", "tiny_product")  # beyond fp16's range
    if name == "tiny_inputs":
        assert np.abs(C).max() < 6.1e-5            # fp16 subnormals unscaled
    if name == "tiny_product":
        assert np.abs(C).max() * np.abs(q).max() * scale * 1.4427 < 2.0 ** -6
    ad = L().llatte_attn_desc(h, r, nc, L().LLATTE_BF16, scale)
    qd = torch.from_numpy(q).cuda().to(torch.bfloat16)
    Cd = torch.from_numpy(C).cuda().to(torch.bfloat16)
    kvd, hqd = torch.from_numpy(kv_off).cuda(), torch.from_numpy(hq_off).cuda()
    out = torch.full((Mtot, h, r), float("nan"), device="cuda")
    lse = torch.full((Mtot, h), float("nan"), device="cuda")
    print(f"range {name}: max|C|={np.abs(C).max():.3g} max|q|={np.abs(q).max():.3g}", flush=True)
    if entry == "workspace":
        ws = torch.empty(L().llatte_mla_attention_workspace_size(ad, B, Mtot, int(kv_off[-1])),
                         dtype=torch.uint8, device="cuda")
        L().llatte_mla_attention(ad, qd, Cd, kvd, hqd, B, Mtot, int(kv_off[-1]), out, lse, ws)
    else:
        L().llatte_mla_attention_noalloc(ad, qd, Cd, kvd, hqd, B, Mtot, int(kv_off[-1]), out, lse)
    torch.cuda.synchronize()
    g, gl = out.cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(g).all() and np.isfinite(gl).all()
    ref, ref_lse = O.latent_attention(q.astype(np.float64), C.astype(np.float64), kv_off, hq_off,
                                      nc, scale)
    rms = math.sqrt(float(np.mean(ref * ref)))
    e = float(np.max(np.abs(g - ref))) / rms
    print(f"  err {e:.3e} (tol 2e-2), lse err {np.max(np.abs(gl - ref_lse)):.3e}", flush=True)
    assert e <= 2e-2
    assert np.max(np.abs(gl - ref_lse)) < 2e-3
