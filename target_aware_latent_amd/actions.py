"""Device-resident action tokenizer: the tables and weights of one action
workload on the GPU plus the ctypes structs pointing at them (argument
marshalling only; the work runs in llatte_action_tokenize)."""
import numpy as np
import torch

from . import llatte as C


def make_action_desc(cfg):
    d = C.llatte_action_desc()
    for k in ("d", "d_hidden", "d_enc", "d_type", "d_item", "d_surf", "d_time",
              "d_meta", "d_meta_emb", "V_type", "V_item", "V_surf", "n_buckets"):
        setattr(d, k, getattr(cfg, k))
    d.dtype = C.LLATTE_BF16 if cfg.dtype == "bf16" else C.LLATTE_F32
    return d


class DeviceActions:
    _KEYS = ("E_type", "E_item", "E_surf", "E_time", "W_meta", "W_a", "W_b")

    def __init__(self, cfg, W, device="cuda"):
        self.cfg = cfg
        self.desc = make_action_desc(cfg)
        self.dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        self.device = device
        self._keep = []
        self.w = C.llatte_action_weights()
        for k in self._KEYS:
            t = torch.from_numpy(np.ascontiguousarray(W[k], dtype=np.float32))
            t = t.to(device=device).to(self.dt).contiguous()
            self._keep.append(t)
            setattr(self.w, k, t.data_ptr())
        self._ws = None

    def inputs(self, I):
        """The int32 / dtype input tensors of one batch, on the device."""
        dev = lambda a, dt=None: torch.from_numpy(np.ascontiguousarray(a)).to(self.device) \
            if dt is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(
                self.device).to(dt).contiguous()
        return {
            "offsets": dev(I["offsets"].astype(np.int32)),
            "t_req": dev(I["t_req"].astype(np.int32)),
            "tau": dev(I["tau"].astype(np.int32)),
            "type_id": dev(I["type_id"].astype(np.int32)),
            "item_id": dev(I["item_id"].astype(np.int32)),
            "surf_id": dev(I["surf_id"].astype(np.int32)),
            "meta": dev(I["meta"], self.dt),
        }

    def workspace(self, n):
        nbytes = C.llatte_action_tokenize_workspace_size(self.desc, n)
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self._ws

    def tokenize(self, X, out=None, stream=None):
        B = X["offsets"].numel() - 1
        n = X["tau"].numel()
        if out is None:
            out = torch.empty((n, self.cfg.d), dtype=torch.float32, device=self.device)
        C.llatte_action_tokenize(self.desc, self.w, X["offsets"], B, n, X["t_req"],
                                 X["tau"], X["type_id"], X["item_id"], X["surf_id"],
                                 X["meta"], out, self.workspace(n), stream)
        return out
