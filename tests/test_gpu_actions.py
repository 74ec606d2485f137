"""GPU parity of llatte_action_tokenize against the action oracle (element by
element on the same seeded inputs), at small ragged sizes in fp32 and bf16
and at the upstream size on sampled rows, plus the edge cases: ids at and
beyond the table bounds, actions stamped after the request, a one-action
user, an empty batch.

Tolerances (the stack's): fp32 max|g - r| / max(|r|, RMS(r)) <= 1e-4; bf16
max|g - r| / RMS(r) <= 2e-2.
"""
import numpy as np
import pytest

from oracle import actions as A
from synth.actions import generate_actions, get_action_config

pytestmark = pytest.mark.gpu


def _err(cfg, got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    if cfg.dtype == "f32":
        return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), rms))), 1e-4
    return float(np.max(np.abs(got - ref)) / rms), 2e-2


def _oracle(cfg, W, I, rows=None):
    return A.action_tokens(W, I["t_req"], I["tau"], I["offsets"], I["type_id"],
                           I["item_id"], I["surf_id"], I["meta"], cfg.n_buckets,
                           cfg.d_enc, rows=rows)


def _run(cfg, W, I):
    import torch
    from target_aware_latent_amd.actions import DeviceActions
    dev = DeviceActions(cfg, W)
    out = dev.tokenize(dev.inputs(I))
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("name", ["a_small", "a_small_bf16"])
@pytest.mark.parametrize("seed", [0, 1])
def test_small_matches_oracle(name, seed):
    cfg = get_action_config(name)
    p = generate_actions(cfg, seed)
    W, I = p["weights"], p["inputs"]
    print(f"action tokenize {name} seed {seed} n={len(I['tau'])}", flush=True)
    got = _run(cfg, W, I)
    e, tol = _err(cfg, got, _oracle(cfg, W, I))
    assert e <= tol, f"error {e:.3e} > {tol}"


def test_ids_at_and_beyond_table_bounds():
    cfg = get_action_config("a_small")
    p = generate_actions(cfg, 3)
    W, I = p["weights"], dict(p["inputs"])
    n = len(I["tau"])
    for k, V in (("type_id", cfg.V_type), ("item_id", cfg.V_item), ("surf_id", cfg.V_surf)):
        ids = I[k].copy()
        ids[0::4] = 0
        ids[1::4] = V - 1
        I[k] = ids
    got = _run(cfg, W, I)
    e, tol = _err(cfg, got, _oracle(cfg, W, I))
    assert e <= tol, f"error {e:.3e} > {tol}"
    # ids outside a table read its nearest row (documented clamp)
    J = dict(I)
    for k, V in (("type_id", cfg.V_type), ("item_id", cfg.V_item), ("surf_id", cfg.V_surf)):
        ids = I[k].copy()
        ids[0::4] = -5
        ids[1::4] = V + 3
        J[k] = ids
    np.testing.assert_array_equal(_run(cfg, W, J), got)
    assert n > 8


def test_future_timestamps_and_one_action_user():
    cfg = get_action_config("a_small")
    p = generate_actions(cfg, 4)
    W, I = p["weights"], dict(p["inputs"])
    tau = I["tau"].copy()
    tau[0] = I["t_req"][0] + 100        # user 0 has one action, after the request
    tau[5] = I["t_req"][1] + 1
    I["tau"] = tau
    ref = _oracle(cfg, W, I)
    got = _run(cfg, W, I)
    e, tol = _err(cfg, got, ref)
    assert e <= tol, f"error {e:.3e} > {tol}"
    # age 0: the encoding is sin 0 = 0 / cos 0 = 1 on the leading dims
    W0 = dict(W)
    W0["W_b"] = np.zeros_like(W["W_b"])
    z = _run(cfg, W0, I)
    want = np.tile([0.0, 1.0], cfg.d_enc // 2)
    np.testing.assert_allclose(z[0, :cfg.d_enc], want, atol=1e-6)
    np.testing.assert_array_equal(z[:, cfg.d_enc:], 0.0)


def test_empty_batch_enqueues_nothing():
    import torch
    from target_aware_latent_amd import llatte as C
    from target_aware_latent_amd.actions import DeviceActions
    cfg = get_action_config("a_small")
    p = generate_actions(cfg, 0)
    dev = DeviceActions(cfg, p["weights"])
    offs = torch.zeros(3, dtype=torch.int32, device="cuda")
    t_req = torch.zeros(2, dtype=torch.int32, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    C.llatte_action_tokenize(dev.desc, dev.w, offs, 2, 0, t_req, None, None, None, None,
                             None, None, ws)
    torch.cuda.synchronize()


def test_deterministic():
    cfg = get_action_config("a_small_bf16")
    p = generate_actions(cfg, 7)
    a = _run(cfg, p["weights"], p["inputs"])
    b = _run(cfg, p["weights"], p["inputs"])
    np.testing.assert_array_equal(a, b)


def test_upstream_size_sampled_rows():
    import torch
    from target_aware_latent_amd.actions import DeviceActions
    cfg = get_action_config("a_c3")
    p = generate_actions(cfg, 0)
    W, I = p["weights"], p["inputs"]
    n = len(I["tau"])
    print(f"action tokenize a_c3 n={n}", flush=True)
    dev = DeviceActions(cfg, W)
    out = dev.tokenize(dev.inputs(I))
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    offs = I["offsets"]
    rows = np.unique(np.concatenate([offs[:-1], offs[1:] - 1, rng.integers(0, n, 256)]))
    got = out[torch.from_numpy(rows).cuda()].cpu().numpy()
    ref = _oracle(cfg, W, I, rows=rows)
    e, tol = _err(cfg, got, ref)
    assert e <= tol, f"error {e:.3e} > {tol}"
    assert np.isfinite(out.cpu().numpy()).all()
