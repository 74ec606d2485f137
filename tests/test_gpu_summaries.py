"""GPU parity of the sequence summaries (llatte_summary_pack +
llatte_summaries) against the oracle's LoRAMLP_k, standalone in fp32 and
bf16 and at the upstream size, and chained after llatte_mla_forward with
LLATTE_FLAG_RAW_READOUT (the readout returns Flatten(Z_raw)).

Tolerances (the stack's): fp32 max|g - r| / max(|r|, RMS(r)) <= 1e-4; bf16
max|g - r| / RMS(r) <= 2e-2, per summary tensor.
"""
import numpy as np
import pytest

import synth
from oracle import llatte_oracle as O
from synth.summaries import generate_summaries, get_summary_config

pytestmark = pytest.mark.gpu


def _check(dtype, got, ref, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    if dtype == "f32":
        e, tol = float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), rms))), 1e-4
    else:
        e, tol = float(np.max(np.abs(got - ref)) / rms), 2e-2
    assert e <= tol, f"{what}: error {e:.3e} > {tol}"


def _summaries(cfg, L, z):
    import torch
    from target_aware_latent_amd.summaries import DeviceSummaries
    ds = DeviceSummaries(cfg, L)
    out = ds(torch.from_numpy(np.ascontiguousarray(z, dtype=np.float32)).cuda())
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("name", ["s_small", "s_small_bf16", "s_c3"])
def test_summaries_match_oracle(name):
    cfg = get_summary_config(name)
    p = generate_summaries(cfg, 0)
    L, z = p["weights"], p["inputs"]["z"]
    print(f"summaries {name}", flush=True)
    got = _summaries(cfg, L, z)
    ref = O.lora_mlp_summaries(z, L)
    assert got.shape == (cfg.K, cfg.B, cfg.d_seq)
    for k in range(cfg.K):
        _check(cfg.dtype, got[k], ref[k], f"summary {k}")


def test_zero_adapters_make_the_summaries_equal():
    cfg = get_summary_config("s_small_bf16")
    p = generate_summaries(cfg, 1)
    L = dict(p["weights"])
    L["B1"] = np.zeros_like(L["B1"])
    L["B2"] = np.zeros_like(L["B2"])
    got = _summaries(cfg, L, p["inputs"]["z"])
    for k in range(1, cfg.K):
        np.testing.assert_array_equal(got[k], got[0])


def test_empty_batch_enqueues_nothing():
    import torch
    from target_aware_latent_amd import llatte as C
    from target_aware_latent_amd.summaries import DeviceSummaries
    cfg = get_summary_config("s_small")
    p = generate_summaries(cfg, 0)
    ds = DeviceSummaries(cfg, p["weights"])
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    C.llatte_summaries(ds.desc, ds.packed, None, 0, None, ws)
    torch.cuda.synchronize()


@pytest.mark.parametrize("base,lengths,kw", [
    ("c1", [9, 70, 33], dict(N=3, n_seeds=2, d_out=64, gain_jitter=0.1,
                             pyramid=synth.PyramidRule("fixed", (50, 20, 8)))),
    ("c3", [300, 150, 64, 1], dict(pyramid=synth.PyramidRule("fixed", (300, 129, 64, 33, 17, 5)))),
])
def test_raw_readout_then_summaries(base, lengths, kw):
    import torch
    from target_aware_latent_amd.model import DeviceModel
    from synth.summaries import SummaryConfig
    cfg = synth.get_config(base, B=len(lengths), **kw)
    prob = synth.generate(cfg, seed=1, lengths=lengths)
    W, I = prob["weights"], prob["inputs"]
    print(f"raw readout {base} {lengths}", flush=True)
    model = DeviceModel(cfg, W, raw_readout=True)
    model.pack()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    h = dev(I["hist"])
    c = dev(I["cand"]) if cfg.n_q else None
    ctx = dev(I["ctx"]) if (cfg.n_q and cfg.d_c) else None
    offs = torch.from_numpy(I["offsets"].astype(np.int32)).cuda()
    out = model.forward(h, offs, [int(x) for x in I["lengths"]], c, ctx)
    torch.cuda.synchronize()
    z_gpu = out["emb"]
    W2 = dict(W)
    W2["W_p"] = None
    ref = O.forward(cfg, W2, I["hist"], I["offsets"], I.get("cand"), I.get("ctx"))
    z_ref = np.stack(ref["emb"])
    assert z_gpu.shape == (cfg.B, cfg.n_seeds * cfg.d)
    _check(cfg.dtype, z_gpu.cpu().numpy(), z_ref, "flattened readout")
    # the summaries on the GPU's readout, against the oracle's on its own
    scfg = SummaryConfig("chain", B=cfg.B, d_z=cfg.n_seeds * cfg.d, d_hidden=2 * cfg.d,
                         d_seq=cfg.d, rank=8, K=2, dtype=cfg.dtype)
    L = generate_summaries(scfg, 5)["weights"]
    from target_aware_latent_amd.summaries import DeviceSummaries
    got = DeviceSummaries(scfg, L)(z_gpu).cpu().numpy()
    want = O.lora_mlp_summaries(z_ref, L)
    for k in range(scfg.K):
        _check(cfg.dtype, got[k], want[k], f"summary {k}")
