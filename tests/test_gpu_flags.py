"""The forward's opt-in descriptor flags, through the C ABI.

LLATTE_FLAG_VALIDATE: the history offsets are checked on the device before
anything else runs ([LLaTTE] Appendix A.2, sequence module item 1: every S_u
is a non-empty, ordered action sequence). Malformed offsets that stay inside
the buffers must give LLATTE_ERR_INVALID_ARG and leave every output
untouched (no other kernel ran); valid ones give the same outputs as
without the flag.

LLATTE_FLAG_DEBUG_DUMP: every layer's query rows land in the caller's
buffer; each section is compared with the oracle's per-layer outputs (the
same bars as the forward's outputs), and the last layer's section with the
forward's own outputs, exactly.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import llatte_oracle as O

pytestmark = pytest.mark.gpu

F32_TOL = 1e-4
BF16_TOL = 2e-2


def L():
    from target_aware_latent_amd import llatte
    return llatte


def _err(g, r, dtype):
    g, r = np.asarray(g, np.float64), np.asarray(r, np.float64)
    rms = math.sqrt(float(np.mean(r * r)))
    if dtype == "f32":
        return float(np.max(np.abs(g - r) / np.maximum(np.abs(r), rms))), F32_TOL
    return float(np.max(np.abs(g - r)) / rms), BF16_TOL


def _model(prob):
    from target_aware_latent_amd.model import DeviceModel
    m = DeviceModel(prob["cfg"], prob["weights"])
    m.pack()
    return m


def _dev(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dtype)


def _prob(name, lengths, **kw):
    cfg = synth.get_config(name, B=len(lengths), **kw)
    return synth.generate(cfg, seed=3, lengths=lengths)


def _run(m, prob, offsets=None, total=None, max_len=None):
    """One forward with outputs pre-filled with NaN; returns (status, message,
    outputs)."""
    cfg, I = prob["cfg"], prob["inputs"]
    lengths = [int(x) for x in I["lengths"]]
    B = len(lengths)
    total = int(sum(lengths)) if total is None else total
    max_len = int(max(lengths)) if max_len is None else max_len
    out = m.alloc_outputs(lengths)
    for v in out.values():
        if v is not None and v.dtype == torch.float32:
            v.fill_(float("nan"))
    out["hist_offsets"].fill_(-7)
    off = I["offsets"] if offsets is None else offsets
    ws = m.workspace(B, max(total, int(sum(lengths))), max(max_len, int(max(lengths))))
    hist = _dev(I["hist"])
    cand = _dev(I["cand"]) if cfg.n_q else None
    ctx = _dev(I["ctx"]) if (cfg.n_q and cfg.d_c) else None
    import ctypes
    lib = L().lib()
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    st = lib.llatte_mla_forward(ctypes.byref(m.desc), ctypes.byref(m.weights), p(m.packed), p(hist),
                                p(torch.from_numpy(np.asarray(off, np.int32)).cuda()), B, total,
                                max_len, p(cand), p(ctx), p(out["cand"]), p(out["hist"]),
                                p(out["hist_offsets"]), p(out["emb"]), p(ws),
                                ws.numel(), None)
    torch.cuda.synchronize()
    msg = L().llatte_last_error() if st else ""
    return st, msg, {k: (None if v is None else v.cpu().numpy()) for k, v in out.items()}


def test_validate_accepts_good_offsets_with_identical_outputs():
    prob = _prob("c2", [5, 40, 17, 400], pyramid=synth.PyramidRule("fixed", (300, 20, 10)))
    m = _model(prob)
    st0, _, ref = _run(m, prob)
    assert st0 == 0
    m.desc.flags |= L().LLATTE_FLAG_VALIDATE
    st1, _, got = _run(m, prob)
    assert st1 == 0
    for k in ("cand", "hist", "hist_offsets"):
        assert np.array_equal(got[k], ref[k]), k


@pytest.mark.parametrize("case", ["non_monotone", "empty_user", "too_long", "wrong_total", "nonzero_start"])
def test_validate_rejects_malformed_offsets_before_any_launch(case):
    lengths = [5, 40, 17, 30]
    prob = _prob("c2", lengths, pyramid=synth.PyramidRule("fixed", (300, 20, 10)))
    m = _model(prob)
    m.desc.flags |= L().LLATTE_FLAG_VALIDATE
    good = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    total, max_len = int(good[-1]), 40
    off = good.copy()
    expect = {"non_monotone": "empty history", "empty_user": "empty history",
              "too_long": "longer than max_len", "wrong_total": "!= total_rows",
              "nonzero_start": "[0] != 0"}[case]
    if case == "non_monotone":
        off[2] = off[1] - 3            # user 1 has a negative length
    elif case == "empty_user":
        off[2] = off[1]                # user 1 empty
    elif case == "too_long":
        max_len = 30                   # user 1 holds 40 rows
    elif case == "wrong_total":
        total = total - 1              # offsets[B] = total + 1
    else:
        off[0] = 1
    print(f"validate {case}: offsets={off.tolist()} total={total} max_len={max_len}", flush=True)
    st, msg, got = _run(m, prob, offsets=off, total=total, max_len=max_len)
    assert st == L().LLATTE_ERR_INVALID_ARG, (st, msg)
    assert expect in msg, msg
    # nothing but the check ran: every output still holds its fill value
    assert np.isnan(got["cand"]).all() and np.isnan(got["hist"]).all()
    assert (got["hist_offsets"] == -7).all()


@pytest.mark.parametrize("name,lengths,kw", [
    ("c2", [5, 40, 17, 300, 1], dict(pyramid=synth.PyramidRule("fixed", (200, 20, 10)))),
    ("c1", [9, 70, 33], dict(N=3, n_seeds=2, d_out=64, gain_jitter=0.1,
                             pyramid=synth.PyramidRule("fixed", (50, 20, 4)))),
    ("c4", [64, 130, 7], dict(norm_mode="post", latent_norm=0)),
])
def test_debug_dump_matches_oracle_layer_by_layer(name, lengths, kw):
    prob = _prob(name, lengths, **kw)
    cfg, I = prob["cfg"], prob["inputs"]
    m = _model(prob)
    B, total, max_len = len(lengths), int(sum(lengths)), int(max(lengths))
    secs = L().llatte_mla_forward_debug_layout(m.desc, B, total, max_len)
    assert len(secs) == cfg.N + (2 if cfg.n_seeds else 1)
    dump = torch.full((secs[-1], cfg.d), float("nan"), device="cuda")
    m.desc.flags |= L().LLATTE_FLAG_DEBUG_DUMP
    m.desc.debug_dump = dump.data_ptr()
    m.desc.debug_dump_bytes = dump.numel() * 4
    st, msg, out = _run(m, prob)
    assert st == 0, msg
    D = dump.cpu().numpy()
    trace = []
    O.forward(cfg, prob["weights"], I["hist"], I["offsets"], I.get("cand"), I.get("ctx"),
              trace=trace)
    keep = O.pyramid_counts(cfg.pyramid, np.asarray(lengths), cfg.N)
    n_layers = cfg.N + (1 if cfg.n_seeds else 0)
    for l in range(n_layers):
        nq = cfg.n_q if l < cfg.N else cfg.n_seeds
        n_u = keep[l] if l < cfg.N else np.zeros(B, np.int64)
        rows = B * nq + int(np.sum(n_u))
        assert secs[l] + rows <= secs[l + 1]
        sec = D[secs[l]:secs[l] + rows]
        ref_c = np.concatenate([trace[u][l][1] for u in range(B)]) if nq else np.zeros((0, cfg.d))
        ref_h = np.concatenate([trace[u][l][0] for u in range(B)])
        ref = np.concatenate([ref_c, ref_h])
        e, tol = _err(sec, ref, cfg.dtype)
        print(f"  layer {l}: {rows} rows, err {e:.3e} (tol {tol})", flush=True)
        assert e <= tol, f"layer {l}"
    # the last stack layer's section is the forward's output, bit for bit
    l = cfg.N - 1
    last = D[secs[l]:secs[l] + B * cfg.n_q + int(np.sum(keep[l]))]
    if cfg.n_q:
        assert np.array_equal(last[:B * cfg.n_q], out["cand"])
    assert np.array_equal(last[B * cfg.n_q:], out["hist"][:int(np.sum(keep[l]))])
