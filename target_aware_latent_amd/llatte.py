"""Thin Python binding of libllatte.so (ctypes). Argument marshalling only.

Every function here forwards to the C ABI declared in include/llatte.h under
the same name; every step of the forward pass runs in the library's HIP
kernels. PyTorch provides device memory and the stream. If the library is
not built, or the GPU path is unavailable, calls raise: there is no fallback.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# LLATTE_LIBRARY selects another build of the library (the host-sanitized
# copy of build.py --sanitize); the default is the in-place build.
LIB_PATH = os.environ.get("LLATTE_LIBRARY") or os.path.join(HERE, "libllatte.so")

LLATTE_OK = 0
LLATTE_ERR_INVALID_ARG = -1
LLATTE_ERR_UNSUPPORTED = -2
LLATTE_ERR_WORKSPACE = -3
LLATTE_ERR_HIP = -4
LLATTE_F32 = 0
LLATTE_BF16 = 1
LLATTE_NORM_PRE = 0
LLATTE_NORM_POST = 1
LLATTE_PYR_FIXED = 0
LLATTE_PYR_HALVING = 1
LLATTE_PYR_GEOMETRIC = 2
LLATTE_MAX_LAYERS = 64
LLATTE_FLAG_RAW_READOUT = 1
LLATTE_FLAG_VALIDATE = 2
LLATTE_FLAG_DEBUG_DUMP = 4

_c_int = ctypes.c_int32
_vp = ctypes.c_void_p


class llatte_pyramid_rule(ctypes.Structure):
    _fields_ = [("kind", _c_int), ("floor", _c_int), ("start", _c_int),
                ("end", _c_int), ("values", _c_int * LLATTE_MAX_LAYERS)]


class llatte_model_desc(ctypes.Structure):
    _fields_ = [("d", _c_int), ("n_heads", _c_int), ("head_dim", _c_int),
                ("rank", _c_int), ("d_ff", _c_int), ("n_layers", _c_int),
                ("n_q", _c_int), ("d_ctx", _c_int), ("dtype", _c_int),
                ("norm_mode", _c_int), ("latent_norm", _c_int),
                ("eps", ctypes.c_float), ("pyramid", llatte_pyramid_rule),
                ("n_seeds", _c_int), ("d_out", _c_int),
                ("flags", ctypes.c_uint32), ("q_rank", _c_int),
                ("debug_dump", _vp), ("debug_dump_bytes", ctypes.c_size_t)]


class llatte_layer_weights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("g1", "W_dkv", "g_c", "W_uq", "W_uk",
                                   "W_uv", "W_o", "g2", "W1", "W2", "W_dq",
                                   "g_q")]


class llatte_weights(ctypes.Structure):
    _fields_ = [("layers", ctypes.POINTER(llatte_layer_weights)),
                ("W_q", _vp), ("seeds", _vp),
                ("readout", llatte_layer_weights), ("W_p", _vp)]


class llatte_attn_desc(ctypes.Structure):
    _fields_ = [("n_heads", _c_int), ("rank", _c_int), ("n_cand", _c_int),
                ("dtype", _c_int), ("scale", ctypes.c_float)]


class llatte_ffn_desc(ctypes.Structure):
    _fields_ = [("d", _c_int), ("d_ff", _c_int), ("dtype", _c_int), ("eps", ctypes.c_float)]


class llatte_attn_sublayer_desc(ctypes.Structure):
    _fields_ = [(n, _c_int) for n in ("d", "n_heads", "head_dim", "rank", "n_cand", "dtype",
                                      "latent_norm")] + [("eps", ctypes.c_float)]


class llatte_attn_sublayer_weights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("g1", "w_dkv", "g_c", "w_uq", "w_uk", "w_uv", "w_o")]


class llatte_attn_sublayer_grads(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("g1", "w_dkv", "g_c", "w_uq", "w_uk", "w_uv", "w_o")]


class llatte_layer_grads(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("g1", "W_dkv", "g_c", "W_uq", "W_uk", "W_uv", "W_o", "g2",
                                   "W1", "W2")]


class llatte_grads(ctypes.Structure):
    _fields_ = [("layers", ctypes.POINTER(llatte_layer_grads)), ("W_q", _vp), ("seeds", _vp),
                ("readout", llatte_layer_grads), ("W_p", _vp)]


class llatte_action_desc(ctypes.Structure):
    _fields_ = [(n, _c_int) for n in (
        "d", "d_hidden", "d_enc", "d_type", "d_item", "d_surf", "d_time",
        "d_meta", "d_meta_emb", "V_type", "V_item", "V_surf", "n_buckets",
        "dtype")]


class llatte_action_weights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("E_type", "E_item", "E_surf", "E_time",
                                   "W_meta", "W_a", "W_b")]


class llatte_summary_desc(ctypes.Structure):
    _fields_ = [(n, _c_int) for n in ("d_z", "d_hidden", "d_seq", "rank",
                                      "n_summaries", "dtype")]


class llatte_summary_weights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("W1", "W2", "A1", "B1", "A2", "B2")]


# name -> (restype, argtypes)
_SIGS = {
    "llatte_mla_forward": (_c_int, [
        ctypes.POINTER(llatte_model_desc), ctypes.POINTER(llatte_weights),
        _vp, _vp, _vp, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _vp,
        _vp, ctypes.c_size_t, _vp]),
    "llatte_packed_weights_size": (ctypes.c_size_t, [
        ctypes.POINTER(llatte_model_desc)]),
    "llatte_pack_weights": (_c_int, [
        ctypes.POINTER(llatte_model_desc), ctypes.POINTER(llatte_weights), _vp,
        ctypes.c_size_t, _vp]),
    "llatte_mla_forward_workspace_size": (ctypes.c_size_t, [
        ctypes.POINTER(llatte_model_desc), _c_int, _c_int, _c_int]),
    "llatte_mla_forward_debug_layout": (_c_int, [
        ctypes.POINTER(llatte_model_desc), _c_int, _c_int, _c_int,
        ctypes.POINTER(ctypes.c_int64)]),
    "llatte_mla_attention": (_c_int, [
        ctypes.POINTER(llatte_attn_desc), _vp, _vp, _vp, _vp, _c_int, _c_int,
        _c_int, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "llatte_mla_attention_workspace_size": (ctypes.c_size_t, [
        ctypes.POINTER(llatte_attn_desc), _c_int, _c_int, _c_int]),
    "llatte_mla_attention_noalloc": (_c_int, [
        ctypes.POINTER(llatte_attn_desc), _vp, _vp, _vp, _vp, _c_int, _c_int,
        _c_int, _vp, _vp, _vp]),
    "llatte_mla_attention_noalloc_max_scratch": (ctypes.c_size_t, []),
    "llatte_pyramid_compact": (_c_int, [
        _vp, _c_int, _c_int, _vp, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp]),
    "llatte_pyramid_counts": (_c_int, [
        ctypes.POINTER(llatte_pyramid_rule), _c_int, _vp, _c_int, _vp, _vp]),
    "llatte_pyramid_counts_host": (_c_int, [
        ctypes.POINTER(llatte_pyramid_rule), _c_int,
        ctypes.POINTER(_c_int), _c_int, ctypes.POINTER(_c_int)]),
    "llatte_token_embed": (_c_int, [
        _vp, _c_int, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp,
        ctypes.c_size_t, _vp]),
    "llatte_token_embed_workspace_size": (ctypes.c_size_t, [
        _c_int, _c_int, _c_int]),
    "llatte_action_tokenize": (_c_int, [
        ctypes.POINTER(llatte_action_desc), ctypes.POINTER(llatte_action_weights),
        _vp, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
        ctypes.c_size_t, _vp]),
    "llatte_action_tokenize_workspace_size": (ctypes.c_size_t, [
        ctypes.POINTER(llatte_action_desc), _c_int]),
    "llatte_summary_packed_size": (ctypes.c_size_t, [ctypes.POINTER(llatte_summary_desc)]),
    "llatte_summary_pack": (_c_int, [
        ctypes.POINTER(llatte_summary_desc), ctypes.POINTER(llatte_summary_weights), _vp,
        ctypes.c_size_t, _vp]),
    "llatte_summaries_workspace_size": (ctypes.c_size_t, [
        ctypes.POINTER(llatte_summary_desc), _c_int]),
    "llatte_summaries": (_c_int, [
        ctypes.POINTER(llatte_summary_desc), _vp, _vp, _c_int, _vp, _vp, ctypes.c_size_t, _vp]),
    "llatte_mla_attention_backward": (_c_int, [
        ctypes.POINTER(llatte_attn_desc), _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int,
        _c_int, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "llatte_mla_attention_backward_workspace_size": (ctypes.c_size_t, [
        ctypes.POINTER(llatte_attn_desc), _c_int]),
    "llatte_ffn_backward": (_c_int, [
        ctypes.POINTER(llatte_ffn_desc), _vp, _vp, _vp, _vp, _vp, _c_int, _vp, _vp, _vp, _vp,
        _vp, ctypes.c_size_t, _vp]),
    "llatte_ffn_backward_workspace_size": (ctypes.c_size_t, [
        ctypes.POINTER(llatte_ffn_desc), _c_int]),
    "llatte_attn_sublayer_backward": (_c_int, [
        ctypes.POINTER(llatte_attn_sublayer_desc), ctypes.POINTER(llatte_attn_sublayer_weights),
        _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp,
        ctypes.POINTER(llatte_attn_sublayer_grads), _vp, ctypes.c_size_t, _vp]),
    "llatte_attn_sublayer_backward_workspace_size": (ctypes.c_size_t, [
        ctypes.POINTER(llatte_attn_sublayer_desc), _c_int, _c_int, _c_int]),
    "llatte_mla_backward": (_c_int, [
        ctypes.POINTER(llatte_model_desc), ctypes.POINTER(llatte_weights), _vp, _vp,
        ctypes.POINTER(_c_int), _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp,
        ctypes.POINTER(llatte_grads), _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "llatte_mla_backward_workspace_size": (ctypes.c_size_t, [
        ctypes.POINTER(llatte_model_desc), _c_int, _c_int, _c_int]),
    "llatte_last_error": (ctypes.c_char_p, []),
    "llatte_version": (_c_int, []),
    "llatte_kernel_timing_enable": (None, [_c_int]),
    "llatte_kernel_timing_read": (_c_int, [
        ctypes.c_char_p, _c_int, ctypes.POINTER(_c_int),
        ctypes.POINTER(ctypes.c_double), _c_int]),
    "llatte_kernel_timing_reset": (None, []),
    "llatte_attention_phases_enable": (_c_int, [_c_int]),
    "llatte_attention_phases_read": (_c_int, [ctypes.POINTER(ctypes.c_double), _c_int]),
    "llatte_gemm_phases_enable": (_c_int, [_c_int]),
    "llatte_gemm_phases_read": (_c_int, [ctypes.POINTER(ctypes.c_double), _c_int]),
}

_lib = None


def lib():
    """Load libllatte.so (built in place by target_aware_latent_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run "
                "`python -m target_aware_latent_amd.build` first")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class LlatteError(RuntimeError):
    def __init__(self, status, where):
        msg = lib().llatte_last_error().decode(errors="replace")
        super().__init__(f"{where} returned {status}: {msg}")
        self.status = status


def _check(status, where):
    if status != LLATTE_OK:
        raise LlatteError(status, where)


def _p(t):
    """Device pointer of a tensor (or NULL for None)."""
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ------------------------------------------------------------------ C ABI

def llatte_mla_forward_workspace_size(desc, B, total_rows, max_len):
    return lib().llatte_mla_forward_workspace_size(ctypes.byref(desc), B,
                                                   total_rows, max_len)


def llatte_mla_forward_debug_layout(desc, B, total_rows, max_len):
    """Row offsets of the LLATTE_FLAG_DEBUG_DUMP sections (list of ints)."""
    buf = (ctypes.c_int64 * (LLATTE_MAX_LAYERS + 2))()
    n = lib().llatte_mla_forward_debug_layout(ctypes.byref(desc), B, total_rows,
                                              max_len, buf)
    if n <= 0:
        raise RuntimeError("llatte_mla_forward_debug_layout: invalid arguments")
    return [int(buf[i]) for i in range(n)]


def llatte_mla_forward(desc, weights, packed_weights, hist_values,
                       hist_offsets, B, total_rows, max_len, cand_x, ctx,
                       out_cand, out_hist, out_hist_offsets, out_emb,
                       workspace, stream=None):
    st = lib().llatte_mla_forward(
        ctypes.byref(desc), None if weights is None else ctypes.byref(weights),
        _p(packed_weights), _p(hist_values), _p(hist_offsets), B, total_rows,
        max_len, _p(cand_x), _p(ctx), _p(out_cand), _p(out_hist),
        _p(out_hist_offsets), _p(out_emb), _p(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "llatte_mla_forward")


def llatte_packed_weights_size(desc):
    return lib().llatte_packed_weights_size(ctypes.byref(desc))


def llatte_pack_weights(desc, weights, packed, stream=None):
    st = lib().llatte_pack_weights(
        ctypes.byref(desc), ctypes.byref(weights), _p(packed),
        packed.numel() * packed.element_size(), _stream(stream))
    _check(st, "llatte_pack_weights")


def llatte_mla_attention_workspace_size(adesc, B, Mtot, Ktot):
    return lib().llatte_mla_attention_workspace_size(ctypes.byref(adesc), B,
                                                     Mtot, Ktot)


def llatte_mla_attention(adesc, q_lat, c_lat, kv_offsets, hq_offsets, B, Mtot,
                         Ktot, out, lse, workspace, stream=None):
    st = lib().llatte_mla_attention(
        ctypes.byref(adesc), _p(q_lat), _p(c_lat), _p(kv_offsets),
        _p(hq_offsets), B, Mtot, Ktot, _p(out), _p(lse), _p(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "llatte_mla_attention")


def llatte_mla_attention_noalloc(adesc, q_lat, c_lat, kv_offsets, hq_offsets,
                                 B, Mtot, Ktot, out, lse, stream=None):
    st = lib().llatte_mla_attention_noalloc(
        ctypes.byref(adesc), _p(q_lat), _p(c_lat), _p(kv_offsets),
        _p(hq_offsets), B, Mtot, Ktot, _p(out), _p(lse), _stream(stream))
    _check(st, "llatte_mla_attention_noalloc")


def llatte_mla_attention_noalloc_max_scratch():
    return lib().llatte_mla_attention_noalloc_max_scratch()


def llatte_pyramid_compact(values, row_elems, dt, offsets_in, B, total_rows,
                           keep, values_out, offsets_out, src_index,
                           stream=None):
    st = lib().llatte_pyramid_compact(
        _p(values), row_elems, dt, _p(offsets_in), B, total_rows, _p(keep),
        _p(values_out), _p(offsets_out), _p(src_index), _stream(stream))
    _check(st, "llatte_pyramid_compact")


def llatte_pyramid_counts(rule, n_layers, offsets_in, B, keep_out, stream=None):
    st = lib().llatte_pyramid_counts(ctypes.byref(rule), n_layers,
                                     _p(offsets_in), B, _p(keep_out),
                                     _stream(stream))
    _check(st, "llatte_pyramid_counts")


def llatte_pyramid_counts_host(rule, n_layers, lengths):
    """Host evaluation of a pyramid rule: returns a list of n_layers lists."""
    B = len(lengths)
    arr = (_c_int * B)(*[int(x) for x in lengths])
    out = (_c_int * (B * n_layers))()
    st = lib().llatte_pyramid_counts_host(ctypes.byref(rule), n_layers, arr, B,
                                          out)
    _check(st, "llatte_pyramid_counts_host")
    return [list(out[l * B:(l + 1) * B]) for l in range(n_layers)]


def llatte_token_embed_workspace_size(d, d_sem, dt):
    return lib().llatte_token_embed_workspace_size(d, d_sem, dt)


def llatte_token_embed(table, V, rows, sem, W_s, n, d, d_sem, dt, out,
                       workspace, stream=None):
    st = lib().llatte_token_embed(
        _p(table), V, _p(rows), _p(sem), _p(W_s), n, d, d_sem, dt, _p(out),
        _p(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(st, "llatte_token_embed")


def llatte_action_tokenize_workspace_size(desc, n):
    return lib().llatte_action_tokenize_workspace_size(ctypes.byref(desc), n)


def llatte_action_tokenize(desc, w, offsets, B, n, t_req, tau, type_id,
                           item_id, surf_id, meta, out, workspace, stream=None):
    st = lib().llatte_action_tokenize(
        ctypes.byref(desc), ctypes.byref(w), _p(offsets), B, n, _p(t_req),
        _p(tau), _p(type_id), _p(item_id), _p(surf_id), _p(meta), _p(out),
        _p(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(st, "llatte_action_tokenize")


def llatte_summary_packed_size(desc):
    return lib().llatte_summary_packed_size(ctypes.byref(desc))


def llatte_summary_pack(desc, w, packed, stream=None):
    st = lib().llatte_summary_pack(ctypes.byref(desc), ctypes.byref(w), _p(packed),
                                   packed.numel() * packed.element_size(), _stream(stream))
    _check(st, "llatte_summary_pack")


def llatte_summaries_workspace_size(desc, B):
    return lib().llatte_summaries_workspace_size(ctypes.byref(desc), B)


def llatte_summaries(desc, packed, z, B, out, workspace, stream=None):
    st = lib().llatte_summaries(ctypes.byref(desc), _p(packed), _p(z), B, _p(out),
                                _p(workspace), workspace.numel() * workspace.element_size(),
                                _stream(stream))
    _check(st, "llatte_summaries")


def llatte_mla_attention_backward_workspace_size(desc, Mtot):
    return lib().llatte_mla_attention_backward_workspace_size(ctypes.byref(desc), Mtot)


def llatte_mla_attention_backward(desc, q_lat, c_lat, kv_offsets, hq_offsets, B, Mtot,
                                  Ktot, max_len, out, lse, d_out, d_q, d_c, workspace,
                                  stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().llatte_mla_attention_backward(
        ctypes.byref(desc), _p(q_lat), _p(c_lat), _p(kv_offsets), _p(hq_offsets), B, Mtot,
        Ktot, max_len, _p(out), _p(lse), _p(d_out), _p(d_q), _p(d_c), _p(workspace), nbytes,
        _stream(stream))
    _check(st, "llatte_mla_attention_backward")


def llatte_ffn_backward_workspace_size(desc, M):
    return lib().llatte_ffn_backward_workspace_size(ctypes.byref(desc), M)


def llatte_ffn_backward(desc, r1, g2, w1, w2, d_out, M, d_r1, d_g2, d_w1, d_w2, workspace,
                        stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().llatte_ffn_backward(
        ctypes.byref(desc), _p(r1), _p(g2), _p(w1), _p(w2), _p(d_out), M, _p(d_r1), _p(d_g2),
        _p(d_w1), _p(d_w2), _p(workspace), nbytes, _stream(stream))
    _check(st, "llatte_ffn_backward")


def llatte_attn_sublayer_backward_workspace_size(desc, B, Mtot, Ktot):
    return lib().llatte_attn_sublayer_backward_workspace_size(ctypes.byref(desc), B, Mtot, Ktot)


def llatte_attn_sublayer_backward(desc, weights, r_kv, r_cand, kv_offsets, hq_offsets, B, Mtot,
                                  Ktot, max_len, d_out, d_r_kv, d_r_cand, grads, workspace,
                                  stream=None):
    """weights / grads: dicts of tensors keyed g1, w_dkv, g_c, w_uq, w_uk, w_uv, w_o."""
    keys = ("g1", "w_dkv", "g_c", "w_uq", "w_uk", "w_uv", "w_o")
    w = llatte_attn_sublayer_weights(*[_p(weights.get(k)) for k in keys])
    g = llatte_attn_sublayer_grads(*[_p(grads.get(k)) for k in keys])
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().llatte_attn_sublayer_backward(
        ctypes.byref(desc), ctypes.byref(w), _p(r_kv), _p(r_cand), _p(kv_offsets), _p(hq_offsets),
        B, Mtot, Ktot, max_len, _p(d_out), _p(d_r_kv), _p(d_r_cand), ctypes.byref(g),
        _p(workspace), nbytes, _stream(stream))
    _check(st, "llatte_attn_sublayer_backward")


def llatte_mla_backward_workspace_size(desc, B, total_rows, max_len):
    return lib().llatte_mla_backward_workspace_size(ctypes.byref(desc), B, total_rows, max_len)


def llatte_mla_backward(desc, weights, hist_values, hist_offsets, hist_offsets_host, B,
                        total_rows, max_len, cand_x, ctx, d_out_cand, d_out_hist, d_out_emb,
                        grads, d_hist, d_cand_x, d_ctx, workspace, stream=None):
    """grads: an llatte_grads struct; hist_offsets_host: host sequence of B+1 ints."""
    off = (_c_int * (B + 1))(*[int(x) for x in hist_offsets_host])
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().llatte_mla_backward(
        ctypes.byref(desc), ctypes.byref(weights), _p(hist_values), _p(hist_offsets), off, B,
        total_rows, max_len, _p(cand_x), _p(ctx), _p(d_out_cand), _p(d_out_hist), _p(d_out_emb),
        ctypes.byref(grads), _p(d_hist), _p(d_cand_x), _p(d_ctx), _p(workspace), nbytes,
        _stream(stream))
    _check(st, "llatte_mla_backward")


def llatte_last_error():
    return lib().llatte_last_error().decode(errors="replace")


def llatte_version():
    return lib().llatte_version()


def llatte_kernel_timing_enable(on):
    lib().llatte_kernel_timing_enable(1 if on else 0)


def llatte_kernel_timing_reset():
    lib().llatte_kernel_timing_reset()


def llatte_kernel_timing_read(cap=64):
    """{kernel name: (launches, total ms)} of the timed launches so far."""
    stride = 64
    names = ctypes.create_string_buffer(stride * cap)
    counts = (_c_int * cap)()
    ms = (ctypes.c_double * cap)()
    n = lib().llatte_kernel_timing_read(names, stride, counts, ms, cap)
    out = {}
    for i in range(n):
        nm = names.raw[i * stride:(i + 1) * stride].split(b"\0", 1)[0].decode()
        out[nm] = (counts[i], ms[i])
    return out


LLATTE_ATTN_PHASE_FIELDS = 6
ATTN_PHASE_KEYS = ("workgroups", "prologue_us", "loop_us", "epilogue_us", "span_us", "longest_us")


def llatte_attention_phases_enable(max_workgroups):
    _check(lib().llatte_attention_phases_enable(int(max_workgroups)),
           "llatte_attention_phases_enable")


def llatte_attention_phases_read():
    """One dict per instrumented attention launch, in launch order."""
    n = lib().llatte_attention_phases_read(None, 0)
    buf = (ctypes.c_double * (max(n, 1) * LLATTE_ATTN_PHASE_FIELDS))()
    n = lib().llatte_attention_phases_read(buf, n)
    f = LLATTE_ATTN_PHASE_FIELDS
    return [dict(zip(ATTN_PHASE_KEYS, buf[i * f:(i + 1) * f])) for i in range(n)]


LLATTE_GEMM_PHASE_FIELDS = 9
GEMM_PHASE_KEYS = ("workgroups", "M", "N", "K", "first_us", "loop_us", "epilogue_us", "span_us",
                   "longest_us")


def llatte_gemm_phases_enable(max_workgroups):
    _check(lib().llatte_gemm_phases_enable(int(max_workgroups)), "llatte_gemm_phases_enable")


def llatte_gemm_phases_read():
    """One dict per instrumented matrix-product launch, in launch order."""
    n = lib().llatte_gemm_phases_read(None, 0)
    buf = (ctypes.c_double * (max(n, 1) * LLATTE_GEMM_PHASE_FIELDS))()
    n = lib().llatte_gemm_phases_read(buf, n)
    f = LLATTE_GEMM_PHASE_FIELDS
    return [dict(zip(GEMM_PHASE_KEYS, buf[i * f:(i + 1) * f])) for i in range(n)]
