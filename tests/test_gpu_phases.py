"""The attention kernel's phase stamps (llatte_attention_phases_enable /
_read), a diagnostic of the absorbed form's three parts ([LLaTTE] App. A.3:
the W_uk absorption of the queries, latent flash attention over the key
tiles, the W_uv map of the output).

The instrumented kernel copy must compute exactly what the normal one does
(same outputs, bit for bit) and give one record per attention launch: every
layer's, then the readout's.
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def L():
    from target_aware_latent_amd import llatte
    return llatte


def _run(m, prob):
    cfg, I = prob["cfg"], prob["inputs"]
    lengths = [int(x) for x in I["lengths"]]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    out = m.forward(dev(I["hist"]), dev(np.asarray(I["offsets"], np.int32)), lengths,
                    dev(I["cand"]) if cfg.n_q else None,
                    dev(I["ctx"]) if (cfg.n_q and cfg.d_c) else None)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items() if v is not None}


@pytest.mark.parametrize("name,lengths,kw", [
    ("c2", [5, 40, 17, 300, 1], dict(N=3, n_seeds=2, d_out=64,
                                     pyramid=synth.PyramidRule("fixed", (200, 20, 10)))),
    ("c3", [64, 700, 3], dict(B=3)),
    # r = 256: the eight-wave kernel (16 rows per wave, two W_uk batches)
    ("c3", [40, 300], dict(N=2, r=256, n_seeds=0, pyramid=synth.PyramidRule("fixed", (300, 40)))),
])
def test_phase_stamps_change_nothing_and_cover_every_launch(name, lengths, kw):
    from target_aware_latent_amd.model import DeviceModel
    kw = dict(kw)
    kw.pop("B", None)
    cfg = synth.get_config(name, B=len(lengths), **kw)
    prob = synth.generate(cfg, seed=5, lengths=lengths)
    m = DeviceModel(cfg, prob["weights"])
    m.pack()
    print(f"phases {name} lengths={lengths}", flush=True)
    ref = _run(m, prob)
    C = L()
    C.llatte_attention_phases_enable(1 << 16)
    try:
        got = _run(m, prob)
        recs = C.llatte_attention_phases_read()
    finally:
        C.llatte_attention_phases_enable(0)
    for k in ref:
        assert np.array_equal(got[k], ref[k], equal_nan=True), k
    assert len(recs) == cfg.N + (1 if cfg.n_seeds else 0)
    for r in recs:
        assert r["workgroups"] >= 1
        assert r["loop_us"] > 0 and r["prologue_us"] > 0 and r["epilogue_us"] > 0
        assert r["span_us"] >= r["longest_us"] > 0
    # off again: no more records, normal kernel
    again = _run(m, prob)
    assert C.llatte_attention_phases_read() == []
    for k in ref:
        assert np.array_equal(again[k], ref[k], equal_nan=True), k


def test_gemm_phase_stamps_change_nothing():
    """The matrix products' phase stamps (llatte_gemm_phases_enable / _read):
    the instrumented copy of the 128 x 128 tile computes the same outputs bit
    for bit, and every launch on that tile gives one record whose shape is
    one of the layer's products and whose phases add up within the span."""
    from target_aware_latent_amd.model import DeviceModel
    lengths = [1600, 1500, 1600, 1400, 1600, 1600]
    cfg = synth.get_config("c3", B=len(lengths), N=2,
                           pyramid=synth.PyramidRule("fixed", (1600, 700)))
    prob = synth.generate(cfg, seed=7, lengths=lengths)
    m = DeviceModel(cfg, prob["weights"])
    m.pack()
    print(f"gemm phases c3 lengths={lengths}", flush=True)
    ref = _run(m, prob)
    C = L()
    C.llatte_gemm_phases_enable(1 << 16)
    try:
        got = _run(m, prob)
        recs = C.llatte_gemm_phases_read()
    finally:
        C.llatte_gemm_phases_enable(0)
    for k in ref:
        assert np.array_equal(got[k], ref[k], equal_nan=True), k
    d, hd, r, dff = cfg.d, cfg.h * cfg.dk, cfg.r, 4 * cfg.d
    shapes = {(r, d), (hd, d), (d, hd), (dff, d), (d, dff)}
    # layer 1 has 9300 rows: its W_uq, W_o, W1 and W2 launches are on the tile
    assert len(recs) >= 4, recs
    for rc in recs:
        assert (int(rc["N"]), int(rc["K"])) in shapes, rc
        assert rc["workgroups"] >= 1
        assert min(rc["first_us"], rc["loop_us"], rc["epilogue_us"]) >= 0, rc
        assert 0 < rc["longest_us"] <= rc["span_us"] + 1e-6, rc
        per_wg = (rc["first_us"] + rc["loop_us"] + rc["epilogue_us"]) / rc["workgroups"]
        assert per_wg <= rc["longest_us"] + 1e-6, rc
