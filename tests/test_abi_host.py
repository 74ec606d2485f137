"""C-ABI library checks that need no GPU: it loads, exports every symbol the
header declares, validates arguments before launching anything, and its host
pyramid evaluation agrees with the oracle."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth
from oracle import llatte_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "llatte.h")


@pytest.fixture(scope="module")
def L():
    from target_aware_latent_amd import llatte
    llatte.lib()
    return llatte


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(llatte_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for must in ("llatte_mla_forward", "llatte_mla_attention",
                 "llatte_pyramid_compact", "llatte_pyramid_counts",
                 "llatte_token_embed", "llatte_mla_forward_workspace_size"):
        assert must in names


def test_library_exports_every_declared_symbol(L):
    lib = L.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in L._SIGS, f"binding lacks {name}"


def test_no_symbol_is_named_after_the_oracle():
    so = open(os.path.join(ROOT, "target_aware_latent_amd", "libllatte.so"), "rb").read()
    assert b"oracle" not in so


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_workspace_size_positive_for_workloads(L, name):
    from target_aware_latent_amd.model import make_desc
    cfg = synth.get_config(name)
    d = make_desc(cfg)
    L_ = cfg.L or cfg.len_range[1]
    assert L.llatte_mla_forward_workspace_size(d, cfg.B, cfg.B * L_, L_) > 0


def test_invalid_descriptors_rejected_on_host(L):
    from target_aware_latent_amd.model import make_desc
    cfg = synth.get_config("c2")
    good = make_desc(cfg)
    assert L.llatte_mla_forward_workspace_size(good, 4, 100, 50) > 0
    for field, val in [("d_ff", 3 * cfg.d), ("rank", 96), ("dtype", 7),
                       ("n_layers", 0), ("head_dim", 12), ("head_dim", 48),
                       ("flags", 8), ("q_rank", 12), ("q_rank", -8),
                       ("q_rank", 1032)]:
        d = make_desc(cfg)
        setattr(d, field, val)
        assert L.llatte_mla_forward_workspace_size(d, 4, 100, 50) == 0, field
    d = make_desc(cfg)
    d.pyramid.values[0] = 0     # zero before the last layer
    assert L.llatte_mla_forward_workspace_size(d, 4, 100, 50) == 0
    # total_rows < B (some user would be empty)
    assert L.llatte_mla_forward_workspace_size(good, 4, 3, 50) == 0
    assert L.llatte_packed_weights_size(good) > 0
    # a low-rank query path adds W_dq and g_q to the packed blob
    lr = make_desc(cfg)
    lr.q_rank = 96
    assert L.llatte_mla_forward_workspace_size(lr, 4, 100, 50) > 0
    assert L.llatte_packed_weights_size(lr) > L.llatte_packed_weights_size(good) - \
        cfg.N * cfg.d * cfg.h * cfg.dk * 2


def test_forward_argument_errors_return_status_without_launch(L):
    from target_aware_latent_amd.model import make_desc
    cfg = synth.get_config("c2")
    d = make_desc(cfg)
    w = L.llatte_weights()
    st = L.lib().llatte_mla_forward(ctypes.byref(d), ctypes.byref(w), None,
                                    None, None, 4, 100, 50, None, None, None,
                                    None, None, None, None, 0, None)
    assert st == L.LLATTE_ERR_INVALID_ARG
    assert "NULL" in L.llatte_last_error()
    ad = L.llatte_attn_desc(4, 96, 0, L.LLATTE_BF16, 0.125)
    st = L.lib().llatte_mla_attention(ctypes.byref(ad), None, None, None, None,
                                      2, 10, 10, None, None, None, 0, None)
    assert st == L.LLATTE_ERR_UNSUPPORTED
    st = L.lib().llatte_pyramid_compact(None, 8, L.LLATTE_F32, None, 2, 10,
                                        None, None, None, None, None)
    assert st == L.LLATTE_ERR_INVALID_ARG


def test_forward_flags_host_side(L):
    """VALIDATE and DEBUG_DUMP are accepted; the dump layout has one section
    per layer (and the readout) sized by the host row bounds; a missing or
    short dump buffer is rejected before anything is enqueued."""
    from target_aware_latent_amd.model import make_desc
    cfg = synth.get_config("c3")
    d = make_desc(cfg)
    d.flags = L.LLATTE_FLAG_VALIDATE | L.LLATTE_FLAG_DEBUG_DUMP
    B, total, max_len = 64, 64 * 1600, 1600
    assert L.llatte_mla_forward_workspace_size(d, B, total, max_len) > 0
    secs = L.llatte_mla_forward_debug_layout(d, B, total, max_len)
    sched = [1600, 800, 400, 200, 100, 50]
    assert secs == [0] + list(np.cumsum([B * n for n in sched] + [B * cfg.n_seeds]))
    fake = ctypes.c_void_p(0x100000)
    w = L.llatte_weights()
    args = lambda: (ctypes.byref(d), ctypes.byref(w), fake, fake, fake, B, total, max_len,
                    None, None, None, None, None, fake, fake, 1 << 40, None)
    d.debug_dump = None
    assert L.lib().llatte_mla_forward(*args()) == L.LLATTE_ERR_INVALID_ARG
    assert "debug_dump" in L.llatte_last_error()
    d.debug_dump = 0x200000
    d.debug_dump_bytes = secs[-1] * cfg.d * 4 - 4
    assert L.lib().llatte_mla_forward(*args()) == L.LLATTE_ERR_WORKSPACE
    # n_layers bounds as documented: 1 .. LLATTE_MAX_LAYERS - 1
    d2 = make_desc(cfg)
    d2.n_layers = L.LLATTE_MAX_LAYERS
    assert L.llatte_mla_forward_workspace_size(d2, B, total, max_len) == 0
    d2.n_layers = L.LLATTE_MAX_LAYERS - 1
    d2.pyramid.kind = L.LLATTE_PYR_HALVING
    d2.pyramid.floor = 16
    assert L.llatte_mla_forward_workspace_size(d2, B, total, max_len) > 0


def test_noalloc_attention_host_validation(L):
    """The fixed-scratch attention entry checks everything on the host before
    it touches the device: sizes whose plan exceeds the fixed scratch, bad
    ranks and NULL pointers are rejected (fake pointers, never dereferenced)."""
    fake = ctypes.c_void_p(0x100000)
    fn = L.lib().llatte_mla_attention_noalloc
    cap = L.llatte_mla_attention_noalloc_max_scratch()
    assert cap == 8 << 20
    ad = L.llatte_attn_desc(8, 128, 0, L.LLATTE_BF16, 0.125)
    big = 1_000_000
    assert L.llatte_mla_attention_workspace_size(ad, 1, big, big) > cap
    st = fn(ctypes.byref(ad), fake, fake, fake, fake, 1, big, big, fake, None, None)
    assert st == L.LLATTE_ERR_WORKSPACE
    assert "fixed scratch" in L.llatte_last_error()
    assert L.llatte_mla_attention_workspace_size(ad, 64, 102400, 102400) <= cap
    bad = L.llatte_attn_desc(4, 96, 0, L.LLATTE_BF16, 0.125)
    st = fn(ctypes.byref(bad), fake, fake, fake, fake, 2, 10, 10, fake, None, None)
    assert st == L.LLATTE_ERR_UNSUPPORTED
    st = fn(ctypes.byref(ad), None, fake, fake, fake, 2, 10, 10, fake, None, None)
    assert st == L.LLATTE_ERR_INVALID_ARG


def test_attention_backward_argument_errors(L):
    # every case fails validation before anything is enqueued (fake pointers
    # are never dereferenced on these paths)
    bw = L.lib().llatte_mla_attention_backward
    fake = ctypes.c_void_p(1 << 20)
    ad = L.llatte_attn_desc(8, 96, 0, L.LLATTE_BF16, 0.125)
    args = [fake] * 4 + [2, 10, 10, 5] + [fake] * 6
    assert bw(ctypes.byref(ad), *args, 1 << 30, None) == L.LLATTE_ERR_UNSUPPORTED
    ad = L.llatte_attn_desc(8, 128, 0, L.LLATTE_F32, 0.125)
    assert bw(ctypes.byref(ad), *args, 1 << 30, None) == L.LLATTE_ERR_UNSUPPORTED
    ad = L.llatte_attn_desc(8, 128, 0, L.LLATTE_BF16, 0.125)
    need = L.llatte_mla_attention_backward_workspace_size(ad, 10)
    assert need >= 10 * 8 * 128 * 4 + 10 * 8 * 4
    assert bw(ctypes.byref(ad), *args, need - 1, None) == L.LLATTE_ERR_WORKSPACE
    nul = [fake] * 4 + [2, 10, 10, 5] + [fake] * 4 + [None, fake]
    assert bw(ctypes.byref(ad), *nul, need, None) == L.LLATTE_ERR_INVALID_ARG
    assert "NULL" in L.llatte_last_error()
    mis = [fake] * 4 + [2, 10, 10, 5] + [fake] * 5 + [ctypes.c_void_p((1 << 20) + 4)]
    assert bw(ctypes.byref(ad), *mis, need, None) == L.LLATTE_ERR_INVALID_ARG
    assert "aligned" in L.llatte_last_error()
    bad = [fake] * 4 + [0, 10, 10, 5] + [fake] * 6
    assert bw(ctypes.byref(ad), *bad, need, None) == L.LLATTE_ERR_INVALID_ARG


def test_sublayer_and_ffn_backward_argument_errors(L):
    fake = ctypes.c_void_p(1 << 20)
    keys = ("g1", "w_dkv", "g_c", "w_uq", "w_uk", "w_uv", "w_o")
    w = L.llatte_attn_sublayer_weights(*[fake] * 7)
    g = L.llatte_attn_sublayer_grads(*[fake] * 7)
    sb = L.lib().llatte_attn_sublayer_backward
    args = lambda B=2, M=10, K=10: [fake, fake, fake, fake, B, M, K, 5, fake, fake, fake]
    d = L.llatte_attn_sublayer_desc(64, 2, 32, 96, 0, L.LLATTE_BF16, 1, 1e-6)
    assert sb(ctypes.byref(d), ctypes.byref(w), *args(), ctypes.byref(g), fake, 1 << 40, None) == \
        L.LLATTE_ERR_UNSUPPORTED
    d = L.llatte_attn_sublayer_desc(64, 2, 30, 64, 0, L.LLATTE_BF16, 1, 1e-6)
    assert sb(ctypes.byref(d), ctypes.byref(w), *args(), ctypes.byref(g), fake, 1 << 40, None) == \
        L.LLATTE_ERR_INVALID_ARG
    d = L.llatte_attn_sublayer_desc(64, 2, 32, 64, 0, L.LLATTE_BF16, 1, 1e-6)
    need = L.llatte_attn_sublayer_backward_workspace_size(d, 2, 10, 10)
    assert need > 0
    assert sb(ctypes.byref(d), ctypes.byref(w), *args(), ctypes.byref(g), fake, need - 1, None) == \
        L.LLATTE_ERR_WORKSPACE
    assert sb(ctypes.byref(d), ctypes.byref(w), *args(B=0), ctypes.byref(g), fake, need, None) == \
        L.LLATTE_ERR_INVALID_ARG
    w0 = L.llatte_attn_sublayer_weights(*([fake] * 6 + [None]))
    assert sb(ctypes.byref(d), ctypes.byref(w0), *args(), ctypes.byref(g), fake, need, None) == \
        L.LLATTE_ERR_INVALID_ARG
    f = L.llatte_ffn_desc(64, 256, L.LLATTE_F32, 1e-6)
    fb = L.lib().llatte_ffn_backward
    fa = [fake] * 5 + [10] + [fake] * 5
    assert fb(ctypes.byref(f), *fa, 1 << 40, None) == L.LLATTE_ERR_UNSUPPORTED
    f = L.llatte_ffn_desc(60, 256, L.LLATTE_BF16, 1e-6)
    assert fb(ctypes.byref(f), *fa, 1 << 40, None) == L.LLATTE_ERR_INVALID_ARG
    f = L.llatte_ffn_desc(64, 256, L.LLATTE_BF16, 1e-6)
    need = L.llatte_ffn_backward_workspace_size(f, 10)
    assert fb(ctypes.byref(f), *fa, need - 1, None) == L.LLATTE_ERR_WORKSPACE


def _rule(L, r):
    from target_aware_latent_amd.model import make_desc
    cfg = synth.Config("x", B=1, L=1, len_range=None, d=8, h=1, dk=8, r=8,
                       n_q=0, d_c=0, N=1, pyramid=r, dtype="f32")
    return make_desc(cfg).pyramid


@pytest.mark.parametrize("rule,N", [
    (synth.PyramidRule("halving", floor=64), 4),
    (synth.PyramidRule("halving", floor=3), 7),
    (synth.PyramidRule("geometric", start=1600, end=50), 12),
    (synth.PyramidRule("fixed", (1600, 800, 400, 200, 100, 50)), 6),
    (synth.PyramidRule("fixed", (30, 30, 7, 0)), 4),
])
def test_host_pyramid_counts_match_oracle(L, rule, N):
    rng = np.random.default_rng(3)
    lengths = np.concatenate([[1, 2, 63, 64, 65, 1600], rng.integers(1, 2000, 200)])
    got = np.array(L.llatte_pyramid_counts_host(_rule(L, rule), N, lengths))
    assert np.array_equal(got, O.pyramid_counts(rule, lengths, N))


def test_host_pyramid_counts_c4_lengths(L):
    cfg = synth.get_config("c4")
    lengths = synth.generate(cfg)["inputs"]["lengths"]
    got = np.array(L.llatte_pyramid_counts_host(_rule(L, cfg.pyramid), cfg.N, lengths))
    assert np.array_equal(got, O.pyramid_counts(cfg.pyramid, lengths, cfg.N))


def test_action_tokenize_host_validation(L):
    from synth.actions import get_action_config
    from target_aware_latent_amd.actions import make_action_desc
    lib = L.lib()
    good = make_action_desc(get_action_config("a_c3"))
    assert L.llatte_action_tokenize_workspace_size(good, 102400) > 102400 * 256 * 2
    assert L.llatte_action_tokenize_workspace_size(
        make_action_desc(get_action_config("a_small")), 235) > 0
    for field, val, code in [("dtype", 5, L.LLATTE_ERR_UNSUPPORTED),
                             ("d_item", 12, L.LLATTE_ERR_UNSUPPORTED),   # bf16: multiple of 8
                             ("d_enc", 3, L.LLATTE_ERR_INVALID_ARG),
                             ("d_enc", 1024, L.LLATTE_ERR_INVALID_ARG),
                             ("V_item", 0, L.LLATTE_ERR_INVALID_ARG),
                             ("n_buckets", 65, L.LLATTE_ERR_INVALID_ARG),
                             ("d_meta", 0, L.LLATTE_ERR_INVALID_ARG)]:
        d = make_action_desc(get_action_config("a_c3"))
        setattr(d, field, val)
        assert L.llatte_action_tokenize_workspace_size(d, 10) == 0, field
        w = L.llatte_action_weights()
        st = lib.llatte_action_tokenize(ctypes.byref(d), ctypes.byref(w), None, 2, 10, None,
                                        None, None, None, None, None, None, None, 0, None)
        assert st == code, (field, st)
    w = L.llatte_action_weights()
    # n = 0: valid, nothing to read, nothing launched
    assert lib.llatte_action_tokenize(ctypes.byref(good), ctypes.byref(w), None, 2, 0, None,
                                      None, None, None, None, None, None, None, 0, None) == 0
    # B < 1, NULL pointers with rows to do
    assert lib.llatte_action_tokenize(ctypes.byref(good), ctypes.byref(w), None, 0, 0, None,
                                      None, None, None, None, None, None, None, 0,
                                      None) == L.LLATTE_ERR_INVALID_ARG
    assert lib.llatte_action_tokenize(ctypes.byref(good), ctypes.byref(w), None, 2, 10, None,
                                      None, None, None, None, None, None, None, 0,
                                      None) == L.LLATTE_ERR_INVALID_ARG
    # every pointer present and aligned but the workspace too small: refused
    # before anything is enqueued (the addresses are never touched)
    fake = ctypes.c_void_p(1 << 20)
    for k in ("E_type", "E_item", "E_surf", "E_time", "W_meta", "W_a", "W_b"):
        setattr(w, k, 1 << 20)
    st = lib.llatte_action_tokenize(ctypes.byref(good), ctypes.byref(w), fake, 2, 10, fake,
                                    fake, fake, fake, fake, fake, fake, fake, 64, None)
    assert st == L.LLATTE_ERR_WORKSPACE
    assert "workspace" in L.llatte_last_error()


def test_stack_backward_host_validation(L):
    """llatte_mla_backward: supported set (BF16, pre-norm, full-rank queries,
    rank 64 / 128), workspace sizing, and argument errors before any launch."""
    from target_aware_latent_amd.model import make_desc
    for name in ("c2", "c3", "c4"):
        cfg = synth.get_config(name)
        L_ = cfg.L or cfg.len_range[1]
        assert L.llatte_mla_backward_workspace_size(make_desc(cfg), cfg.B, cfg.B * L_, L_) > 0
    cfg = synth.get_config("c2")
    B, total, max_len = 3, 30, 20
    for field, val in [("norm_mode", L.LLATTE_NORM_POST), ("dtype", L.LLATTE_F32),
                       ("q_rank", 64), ("rank", 256), ("flags", L.LLATTE_FLAG_VALIDATE)]:
        d = make_desc(cfg)
        setattr(d, field, val)
        assert L.llatte_mla_backward_workspace_size(d, B, total, max_len) == 0, field
    d = make_desc(cfg)
    fake = 0x100000
    lw = L.llatte_layer_weights(*([fake] * 10 + [None, None]))
    layers = (L.llatte_layer_weights * cfg.N)(*([lw] * cfg.N))
    w = L.llatte_weights(ctypes.cast(layers, ctypes.POINTER(L.llatte_layer_weights)), fake, fake,
                         lw, fake)
    lg = L.llatte_layer_grads(*([fake] * 10))
    glayers = (L.llatte_layer_grads * cfg.N)(*([lg] * cfg.N))
    g = L.llatte_grads(ctypes.cast(glayers, ctypes.POINTER(L.llatte_layer_grads)), fake, fake, lg,
                       fake)
    off = (ctypes.c_int * (B + 1))(0, 10, 20, 30)
    f = ctypes.c_void_p(fake)

    def call(desc=d, weights=w, offs=off, grads=g, wsb=1 << 40, dcand=f):
        return L.lib().llatte_mla_backward(
            ctypes.byref(desc), ctypes.byref(weights), f, f, offs, B, total, max_len, f, f, dcand,
            None, f, ctypes.byref(grads), f, f, f, f, wsb, None)

    post = make_desc(cfg)
    post.norm_mode = L.LLATTE_NORM_POST
    assert call(desc=post) == L.LLATTE_ERR_UNSUPPORTED
    assert "pre-norm" in L.llatte_last_error()
    assert call(weights=L.llatte_weights()) == L.LLATTE_ERR_INVALID_ARG
    assert call(dcand=None) == L.LLATTE_ERR_INVALID_ARG     # n_q > 0 needs d_out_cand
    assert call(offs=(ctypes.c_int * (B + 1))(0, 10, 20, 29)) == L.LLATTE_ERR_INVALID_ARG
    assert "total_rows" in L.llatte_last_error()
    assert call(offs=(ctypes.c_int * (B + 1))(0, 25, 26, 30)) == L.LLATTE_ERR_INVALID_ARG
    assert "max_len" in L.llatte_last_error()
    assert call(wsb=1024) == L.LLATTE_ERR_WORKSPACE
    nog = L.llatte_grads(ctypes.cast(glayers, ctypes.POINTER(L.llatte_layer_grads)), fake, None,
                         lg, fake)
    dr = make_desc(cfg)
    dr.n_seeds, dr.d_out = 2, 64
    assert call(desc=dr, grads=nog) == L.LLATTE_ERR_INVALID_ARG  # readout: the seeds' gradient
    assert "seeds" in L.llatte_last_error()


def test_attention_phase_diagnostic_off_by_default(L):
    # no GPU needed: nothing is allocated while the diagnostic is off
    assert L.llatte_attention_phases_read() == []
    L.llatte_attention_phases_enable(0)
    assert L.llatte_attention_phases_read() == []
    assert L.LLATTE_ATTN_PHASE_FIELDS == len(L.ATTN_PHASE_KEYS)


def test_gemm_phase_diagnostic_off_by_default(L):
    # no GPU needed: nothing is allocated while the diagnostic is off
    assert L.llatte_gemm_phases_read() == []
    L.llatte_gemm_phases_enable(0)
    assert L.llatte_gemm_phases_read() == []
    assert L.LLATTE_GEMM_PHASE_FIELDS == len(L.GEMM_PHASE_KEYS)
