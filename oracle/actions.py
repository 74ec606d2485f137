"""CPU oracle of the LLaTTE action tokenization (one token per user action).

TEST INFRASTRUCTURE ONLY, like the rest of this package: the tests, the
package smoke check and the CPU leg of the benchmark may import it; the
product path never does. It shares no code with the HIP library.

Source: "LLaTTE: Scaling Laws for Multi-Stage Sequence Modeling in
Large-Scale Ads Recommendation" (annotated translation), Appendix A.2,
"Sequence Module", item 1 (action embeddings): each action (timestamp,
type, item, surface, meta) is embedded per field, the five embeddings go
through MLP_act to one d-wide token, the tokens of a user's actions are
stacked oldest first, and additive timestamp encodings are applied to a
subset of the hidden dimensions.

The page fixes neither the field embeddings, nor MLP_act, nor the encoding.
Readings taken (each also listed in the design notes):
  * type, item and surface are ids looked up in learned tables;
  * the time field is the action's age at the user's request time,
    age = max(0, t_req(u) - tau) in seconds, embedded through a learned
    table indexed by the logarithmic bucket floor(log2(1 + age)) (clamped
    to the last bucket);
  * meta is a dense vector, embedded linearly (meta W_meta, no bias);
  * MLP_act takes the five embeddings concatenated in the page's order
    (type, item, surface, time, meta) through one hidden layer with the
    exact-erf GELU and no biases, as the stack's FFN;
  * the timestamp encoding is the sinusoidal encoding of the age in hours
    (sin on even, cos on odd dimensions, frequencies 10000^(-2i/d_enc))
    added to the first d_enc dimensions of the token.
Numbers are fp64 by default; dtype=np.float32 runs the same code in single
precision.
"""
import math

import numpy as np
from scipy.special import erf as _erf

__all__ = ["action_ages", "time_bucket", "time_encoding", "action_concat",
           "action_tokens", "action_flops"]


def action_ages(t_req, tau, offsets):
    """Age in seconds of every action at its user's request time.

    Row i belongs to user u with offsets[u] <= i < offsets[u+1]; the age is
    t_req[u] - tau[i], negative ages (an action stamped after the request)
    taken as 0. Integer (int64), exact.
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    tau = np.asarray(tau, dtype=np.int64)
    t_req = np.asarray(t_req, dtype=np.int64)
    user = np.repeat(np.arange(len(offsets) - 1), np.diff(offsets))
    return np.maximum(t_req[user] - tau, 0)


def time_bucket(age, n_buckets):
    """floor(log2(1 + age)) for integer ages >= 0, clamped to n_buckets - 1.

    Integer arithmetic only: floor(log2(v)) of a positive integer v is its
    bit length minus one.
    """
    out = np.empty(len(age), dtype=np.int64)
    for i, a in enumerate(np.asarray(age, dtype=np.int64)):
        out[i] = min(int(a + 1).bit_length() - 1, n_buckets - 1)
    return out


def time_encoding(age, d_enc, d, dtype=np.float64):
    """[n, d] additive encoding: columns 2i, 2i+1 (2i < d_enc) hold
    sin and cos of (age / 3600) * 10000^(-2i / d_enc); other columns 0."""
    age_h = np.asarray(age, dtype=np.float64) / 3600.0
    enc = np.zeros((len(age_h), d), dtype=np.float64)
    for i in range(d_enc // 2):
        w = 10000.0 ** (-(2.0 * i) / d_enc)
        enc[:, 2 * i] = np.sin(age_h * w)
        enc[:, 2 * i + 1] = np.cos(age_h * w)
    return enc.astype(dtype)


def action_concat(W, type_id, item_id, surf_id, bucket, meta, dtype=np.float64):
    """The five field embeddings side by side, in the page's field order."""
    f = lambda a: np.asarray(a, dtype=dtype)
    return np.concatenate([
        f(W["E_type"])[type_id],
        f(W["E_item"])[item_id],
        f(W["E_surf"])[surf_id],
        f(W["E_time"])[bucket],
        f(meta) @ f(W["W_meta"]),
    ], axis=1)


def action_tokens(W, t_req, tau, offsets, type_id, item_id, surf_id, meta,
                  n_buckets, d_enc, dtype=np.float64, rows=None):
    """Tokens [n, d] of every action (or of the listed rows only).

    x = GELU(concat W_a) W_b + time_encoding(age), GELU with the exact erf.
    """
    age = action_ages(t_req, tau, offsets)
    if rows is not None:
        rows = np.asarray(rows)
        age, type_id, item_id, surf_id, meta = (
            age[rows], np.asarray(type_id)[rows], np.asarray(item_id)[rows],
            np.asarray(surf_id)[rows], np.asarray(meta)[rows])
    u = action_concat(W, type_id, item_id, surf_id, time_bucket(age, n_buckets),
                      meta, dtype)
    h = u @ np.asarray(W["W_a"], dtype=dtype)
    h = (0.5 * h * (1.0 + _erf(h / math.sqrt(2.0)))).astype(dtype)
    x = h @ np.asarray(W["W_b"], dtype=dtype)
    d = x.shape[1]
    return x + time_encoding(age, d_enc, d, dtype)


def action_flops(n, d_meta, d_meta_emb, d_in, d_hidden, d):
    """2mnk over the three products of the tokenizer (meta, W_a, W_b)."""
    return 2 * n * (d_meta * d_meta_emb + d_in * d_hidden + d_hidden * d)
