"""Pins of the action-tokenization oracle (oracle/actions.py) against facts
fixed outside it: hand-computed ages and buckets, textbook values of sin and
cos, torch's embedding / linear / GELU routines, the identity-MLP special
case and a scalar brute force on tiny inputs.

Source: "LLaTTE: Scaling Laws for Multi-Stage Sequence Modeling in
Large-Scale Ads Recommendation" (annotated translation), Appendix A.2,
Sequence Module item 1 (action embeddings, MLP_act, additive timestamp
encodings on a subset of the hidden dimensions).
"""
import math

import numpy as np
import pytest

from oracle import actions as A
from synth.actions import generate_actions, get_action_config


def test_ages_per_user_and_clamped_at_zero():
    # offsets [0, 2, 5]: rows 0-1 are user 0 (t_req 100), rows 2-4 user 1 (1000)
    age = A.action_ages([100, 1000], [90, 101, 1000, 999, 1001], [0, 2, 5])
    assert age.tolist() == [10, 0, 0, 1, 0]


def test_time_bucket_is_floor_log2_of_one_plus_age():
    ages = [0, 1, 2, 3, 6, 7, 8, 1022, 1023, 1024, 2 ** 20 - 1, 2 ** 20, 2 ** 31 - 2]
    want = [0, 1, 1, 2, 2, 3, 3, 9, 10, 10, 20, 20, 30]
    assert A.time_bucket(ages, 64).tolist() == want
    # clamped to the last bucket
    assert A.time_bucket([2 ** 20], 8).tolist() == [7]
    # against the real logarithm away from powers of two
    rng = np.random.default_rng(3)
    for a in rng.integers(0, 2 ** 30, 200):
        v = int(a) + 1
        if v & (v - 1):
            assert A.time_bucket([int(a)], 64)[0] == math.floor(math.log2(v))


def test_time_encoding_textbook_values():
    # d_enc = 2: one frequency, 1 rad per hour
    enc = A.time_encoding([3600, 0], 2, 4)
    assert enc[0, 0] == pytest.approx(0.8414709848078965, abs=1e-15)  # sin 1
    assert enc[0, 1] == pytest.approx(0.5403023058681398, abs=1e-15)  # cos 1
    assert enc[1].tolist() == [0.0, 1.0, 0.0, 0.0]
    assert np.all(enc[:, 2:] == 0)


def test_time_encoding_matches_complex_exponential():
    rng = np.random.default_rng(0)
    age = rng.integers(0, 10 ** 7, 50)
    d_enc, d = 16, 24
    enc = A.time_encoding(age, d_enc, d)
    for i in range(d_enc // 2):
        z = np.exp(1j * (age / 3600.0) / 10000.0 ** (2 * i / d_enc))
        np.testing.assert_allclose(enc[:, 2 * i], z.imag, atol=1e-12)
        np.testing.assert_allclose(enc[:, 2 * i + 1], z.real, atol=1e-12)
    assert np.all(enc[:, d_enc:] == 0)
    np.testing.assert_allclose(enc[:, 0:d_enc:2] ** 2 + enc[:, 1:d_enc:2] ** 2, 1.0, atol=1e-12)


def _small(seed=0):
    cfg = get_action_config("a_small")
    p = generate_actions(cfg, seed)
    return cfg, p["weights"], p["inputs"]


def _tokens(cfg, W, I, **kw):
    return A.action_tokens(W, I["t_req"], I["tau"], I["offsets"], I["type_id"],
                           I["item_id"], I["surf_id"], I["meta"], cfg.n_buckets,
                           cfg.d_enc, **kw)


def test_tokens_match_torch_composition():
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    cfg, W, I = _small()
    x = _tokens(cfg, W, I)
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    ids = lambda a: torch.from_numpy(np.asarray(a, dtype=np.int64))
    age = np.maximum(np.repeat(I["t_req"].astype(np.int64), np.diff(I["offsets"]))
                     - I["tau"].astype(np.int64), 0)
    bucket = np.minimum(np.floor(np.log2(age + 1.0) + 1e-9).astype(np.int64), cfg.n_buckets - 1)
    u = torch.cat([F.embedding(ids(I["type_id"]), t(W["E_type"])),
                   F.embedding(ids(I["item_id"]), t(W["E_item"])),
                   F.embedding(ids(I["surf_id"]), t(W["E_surf"])),
                   F.embedding(ids(bucket), t(W["E_time"])),
                   F.linear(t(I["meta"]), t(W["W_meta"]).T)], dim=1)
    y = F.linear(F.gelu(F.linear(u, t(W["W_a"]).T), approximate="none"), t(W["W_b"]).T)
    ang = (age / 3600.0)[:, None] / 10000.0 ** (np.arange(0, cfg.d_enc, 2) / cfg.d_enc)[None, :]
    y = y.numpy()
    y[:, 0:cfg.d_enc:2] += np.sin(ang)
    y[:, 1:cfg.d_enc:2] += np.cos(ang)
    np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-12)


def test_identity_mlp_gives_gelu_of_the_concatenated_fields():
    cfg, W, I = _small()
    W = dict(W)
    d_in = cfg.d_in
    W["W_a"] = np.eye(d_in)
    W["W_b"] = np.eye(d_in)
    x = A.action_tokens(W, I["t_req"], I["tau"], I["offsets"], I["type_id"], I["item_id"],
                        I["surf_id"], I["meta"], cfg.n_buckets, 0)
    for i in (0, 1, 40, 200, 234):
        user = int(np.searchsorted(I["offsets"], i, side="right")) - 1
        age = max(int(I["t_req"][user]) - int(I["tau"][i]), 0)
        b = min(int(age + 1).bit_length() - 1, cfg.n_buckets - 1)
        meta = [sum(float(I["meta"][i][k]) * float(W["W_meta"][k][j]) for k in range(cfg.d_meta))
                for j in range(cfg.d_meta_emb)]
        u = (list(W["E_type"][I["type_id"][i]]) + list(W["E_item"][I["item_id"][i]])
             + list(W["E_surf"][I["surf_id"][i]]) + list(W["E_time"][b]) + meta)
        want = [0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in map(float, u)]
        np.testing.assert_allclose(x[i], want, rtol=1e-12, atol=1e-13)


def _brute(cfg, W, I, rows):
    """Scalar loops, written separately from the oracle."""
    out = []
    for i in rows:
        user = 0
        while not (I["offsets"][user] <= i < I["offsets"][user + 1]):
            user += 1
        age = int(I["t_req"][user]) - int(I["tau"][i])
        if age < 0:
            age = 0
        b, v = 0, age + 1
        while v > 1:
            v //= 2
            b += 1
        b = min(b, cfg.n_buckets - 1)
        u = [float(z) for z in W["E_type"][I["type_id"][i]]]
        u += [float(z) for z in W["E_item"][I["item_id"][i]]]
        u += [float(z) for z in W["E_surf"][I["surf_id"][i]]]
        u += [float(z) for z in W["E_time"][b]]
        for j in range(cfg.d_meta_emb):
            s = 0.0
            for k in range(cfg.d_meta):
                s += float(I["meta"][i][k]) * float(W["W_meta"][k][j])
            u.append(s)
        h = []
        for j in range(cfg.d_hidden):
            s = 0.0
            for k in range(cfg.d_in):
                s += u[k] * float(W["W_a"][k][j])
            h.append(s * 0.5 * (1.0 + math.erf(s / math.sqrt(2.0))))
        x = []
        for j in range(cfg.d):
            s = 0.0
            for k in range(cfg.d_hidden):
                s += h[k] * float(W["W_b"][k][j])
            if j < cfg.d_enc:
                f = (age / 3600.0) * 10000.0 ** (-(j - j % 2) / cfg.d_enc)
                s += math.sin(f) if j % 2 == 0 else math.cos(f)
            x.append(s)
        out.append(x)
    return np.array(out)


def test_brute_force_on_tiny_rows():
    cfg, W, I = _small(seed=5)
    rows = [0, 1, 37, 38, 100, 233, 234]
    np.testing.assert_allclose(_tokens(cfg, W, I, rows=rows), _brute(cfg, W, I, rows),
                               rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(_tokens(cfg, W, I)[rows], _brute(cfg, W, I, rows),
                               rtol=1e-11, atol=1e-11)


def test_rows_are_independent_and_only_age_matters_for_time():
    cfg, W, I = _small(seed=2)
    x = _tokens(cfg, W, I)
    # shifting every timestamp and request time by the same amount changes nothing
    I2 = dict(I)
    I2["t_req"] = I["t_req"] - 12345
    I2["tau"] = I["tau"] - 12345
    np.testing.assert_array_equal(_tokens(cfg, W, I2), x)
    # a token depends on its own row only: perturb every other field of row 5
    I3 = dict(I)
    I3["meta"] = I["meta"].copy()
    I3["meta"][5] += 1.0
    y = _tokens(cfg, W, I3)
    changed = np.nonzero(np.any(y != x, axis=1))[0]
    assert changed.tolist() == [5]


def test_flop_count_of_the_upstream_shape():
    cfg = get_action_config("a_c3")
    n = cfg.B * cfg.L
    assert A.action_flops(n, cfg.d_meta, cfg.d_meta_emb, cfg.d_in, cfg.d_hidden, cfg.d) == \
        2 * 102400 * (16 * 32 + 256 * 1024 + 1024 * 512)
