"""Marshalling helpers around llatte_mla_forward: descriptor, device weights,
buffers. No arithmetic of the method happens here; it all runs in the HIP
library behind the C ABI."""
import ctypes

import numpy as np
import torch

from . import llatte as C


def make_desc(cfg, raw_readout=False):
    """llatte_model_desc from a workload description with the attributes
    d, h, dk, r, N, n_q, d_c, dtype ('f32'/'bf16'), norm_mode ('pre'/'post'),
    latent_norm, eps, pyramid (kind/values/floor/start/end), n_seeds, d_out
    and (optional) r_q. raw_readout: the readout returns Flatten(Z_raw)
    ([B, n_seeds*d]) instead of its W_p projection."""
    d = C.llatte_model_desc()
    d.d, d.n_heads, d.head_dim, d.rank = cfg.d, cfg.h, cfg.dk, cfg.r
    d.d_ff = 4 * cfg.d
    d.n_layers = cfg.N
    d.n_q, d.d_ctx = cfg.n_q, cfg.d_c
    d.dtype = C.LLATTE_BF16 if cfg.dtype == "bf16" else C.LLATTE_F32
    d.norm_mode = C.LLATTE_NORM_PRE if cfg.norm_mode == "pre" else C.LLATTE_NORM_POST
    d.latent_norm = 1 if cfg.latent_norm else 0
    d.eps = cfg.eps
    rule = cfg.pyramid
    if rule.kind == "fixed":
        d.pyramid.kind = C.LLATTE_PYR_FIXED
        for i, v in enumerate(rule.values):
            d.pyramid.values[i] = int(v)
    elif rule.kind == "halving":
        d.pyramid.kind = C.LLATTE_PYR_HALVING
        d.pyramid.floor = int(rule.floor)
    elif rule.kind == "geometric":
        d.pyramid.kind = C.LLATTE_PYR_GEOMETRIC
        d.pyramid.start, d.pyramid.end = int(rule.start), int(rule.end)
    else:
        raise ValueError(rule.kind)
    d.n_seeds, d.d_out = cfg.n_seeds, cfg.d_out
    d.flags = 0
    if raw_readout and cfg.n_seeds > 0:
        d.flags = C.LLATTE_FLAG_RAW_READOUT
        d.d_out = cfg.n_seeds * cfg.d
    d.q_rank = getattr(cfg, "r_q", 0)
    return d


def torch_dtype(cfg):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


class DeviceModel:
    """Weights of one model resident on the GPU plus the ctypes structs that
    point at them (kept alive together)."""

    _LAYER_KEYS = ("g1", "W_dkv", "g_c", "W_uq", "W_uk", "W_uv", "W_o", "g2",
                   "W1", "W2", "W_dq", "g_q")

    def __init__(self, cfg, W, device="cuda", raw_readout=False):
        self.cfg = cfg
        self.desc = make_desc(cfg, raw_readout)
        self.raw_readout = raw_readout
        self.device = device
        self._keep = []
        dt = torch_dtype(cfg)

        def mat(a):
            t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
            t = t.to(device=device).to(dt).contiguous()
            self._keep.append(t)
            return t

        def vec(a):
            t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
            self._keep.append(t)
            return t

        def layer(Wl):
            s = C.llatte_layer_weights()
            for k in self._LAYER_KEYS:
                if k not in Wl:   # W_dq / g_q of the low-rank query path
                    continue
                t = vec(Wl[k]) if k.startswith("g") else mat(Wl[k])
                setattr(s, k, t.data_ptr())
            return s

        self._layers = (C.llatte_layer_weights * cfg.N)(
            *[layer(Wl) for Wl in W["layers"]])
        w = C.llatte_weights()
        w.layers = ctypes.cast(self._layers, ctypes.POINTER(C.llatte_layer_weights))
        if cfg.n_q > 0:
            w.W_q = mat(W["W_q"]).data_ptr()
        if cfg.n_seeds > 0:
            w.seeds = vec(W["seeds"]).data_ptr()
            w.readout = layer(W["readout"])
            if not raw_readout:
                w.W_p = mat(W["W_p"]).data_ptr()
        self.weights = w
        self._ws = None
        self._bws = None
        self.packed = None

    def pack(self, stream=None):
        """Write the packed-weight blob once; later forwards reuse it."""
        n = C.llatte_packed_weights_size(self.desc)
        if n == 0:
            raise C.LlatteError(-1, "llatte_packed_weights_size")
        self.packed = torch.empty(n, dtype=torch.uint8, device=self.device)
        C.llatte_pack_weights(self.desc, self.weights, self.packed, stream)
        return self.packed

    def workspace(self, B, total, max_len):
        n = C.llatte_mla_forward_workspace_size(self.desc, B, total, max_len)
        if n == 0:
            raise C.LlatteError(-1, "llatte_mla_forward_workspace_size")
        if self._ws is None or self._ws.numel() < n:
            self._ws = torch.empty(n, dtype=torch.uint8, device=self.device)
        return self._ws

    def out_hist_rows(self, lengths):
        keep = C.llatte_pyramid_counts_host(self.desc.pyramid, self.cfg.N,
                                            list(lengths))
        return int(sum(keep[-1]))

    def alloc_outputs(self, lengths):
        cfg, dev = self.cfg, self.device
        B = len(lengths)
        out = {
            "cand": (torch.empty(B * cfg.n_q, cfg.d, device=dev)
                     if cfg.n_q else None),
            "hist": torch.empty(max(self.out_hist_rows(lengths), 1), cfg.d, device=dev),
            "hist_offsets": torch.empty(B + 1, dtype=torch.int32, device=dev),
            "emb": (torch.empty(B, self.desc.d_out, device=dev) if cfg.n_seeds else None),
        }
        return out

    def forward(self, hist, offsets, lengths, cand=None, ctx=None, out=None,
                stream=None):
        """hist [total, d] float32 and offsets [B+1] int32 on the device;
        lengths: host list of the per-user lengths (sizes only)."""
        B = len(lengths)
        total = int(sum(lengths))
        max_len = int(max(lengths))
        if out is None:
            out = self.alloc_outputs(lengths)
        ws = self.workspace(B, total, max_len)
        C.llatte_mla_forward(self.desc, self.weights, self.packed, hist,
                             offsets, B, total, max_len, cand, ctx,
                             out["cand"], out["hist"], out["hist_offsets"],
                             out["emb"], ws, stream)
        return out

    _GRAD_KEYS = ("g1", "W_dkv", "g_c", "W_uq", "W_uk", "W_uv", "W_o", "g2", "W1", "W2")

    def alloc_grads(self, lengths):
        """float32 gradient tensors laid out as the weights ({'layers': [dict
        per layer], 'readout', 'seeds', 'W_q', 'W_p'}) and the inputs ('hist',
        'cand', 'ctx'), plus the llatte_grads struct that points at them."""
        cfg, dev = self.cfg, self.device
        B, total = len(lengths), int(sum(lengths))
        d, hd, r, F = cfg.d, cfg.h * cfg.dk, cfg.r, 4 * cfg.d
        shapes = {"g1": (d,), "W_dkv": (d, r), "g_c": (r,), "W_uq": (d, hd), "W_uk": (r, hd),
                  "W_uv": (r, hd), "W_o": (hd, d), "g2": (d,), "W1": (d, F), "W2": (F, d)}
        buf = lambda *shape: torch.empty(*shape, device=dev)

        def layer():
            g = {k: buf(*shapes[k]) for k in self._GRAD_KEYS}
            return g, C.llatte_layer_grads(*[g[k].data_ptr() for k in self._GRAD_KEYS])

        out = {"layers": []}
        structs = []
        for _ in range(cfg.N):
            g, st = layer()
            out["layers"].append(g)
            structs.append(st)
        arr = (C.llatte_layer_grads * cfg.N)(*structs)
        G = C.llatte_grads()
        G.layers = ctypes.cast(arr, ctypes.POINTER(C.llatte_layer_grads))
        if cfg.n_q > 0:
            out["W_q"] = buf(d + cfg.d_c, d)
            G.W_q = out["W_q"].data_ptr()
        if cfg.n_seeds > 0:
            out["seeds"] = buf(cfg.n_seeds, d)
            G.seeds = out["seeds"].data_ptr()
            out["readout"], G.readout = layer()
            if not self.raw_readout:
                out["W_p"] = buf(cfg.n_seeds * d, self.desc.d_out)
                G.W_p = out["W_p"].data_ptr()
        out["hist"] = buf(total, d)
        out["cand"] = buf(B * cfg.n_q, d) if cfg.n_q else None
        out["ctx"] = buf(B, cfg.d_c) if cfg.n_q and cfg.d_c else None
        out["_struct"] = (G, arr)   # the struct and the array it points into
        return out

    def backward(self, hist, offsets, lengths, cand=None, ctx=None, d_out_cand=None,
                 d_out_hist=None, d_out_emb=None, grads=None, stream=None):
        """llatte_mla_backward into ``grads`` (from alloc_grads; allocated
        when None); returns the gradients."""
        B = len(lengths)
        total = int(sum(lengths))
        max_len = int(max(lengths))
        if grads is None:
            grads = self.alloc_grads(lengths)
        n = C.llatte_mla_backward_workspace_size(self.desc, B, total, max_len)
        if n == 0:
            raise C.LlatteError(-1, "llatte_mla_backward_workspace_size")
        if self._bws is None or self._bws.numel() < n:
            self._bws = torch.empty(n, dtype=torch.uint8, device=self.device)
        offs = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
        C.llatte_mla_backward(self.desc, self.weights, hist, offsets, offs, B, total, max_len,
                              cand, ctx, d_out_cand, d_out_hist, d_out_emb, grads["_struct"][0],
                              grads["hist"], grads["cand"], grads["ctx"], self._bws, stream)
        return grads
