"""Device-resident sequence summaries: base weights and adapters of one
summary workload on the GPU, merged once into the packed layout
(argument marshalling only; the work runs in llatte_summary_pack and
llatte_summaries)."""
import numpy as np
import torch

from . import llatte as C


def make_summary_desc(cfg):
    d = C.llatte_summary_desc()
    d.d_z, d.d_hidden, d.d_seq = cfg.d_z, cfg.d_hidden, cfg.d_seq
    d.rank, d.n_summaries = cfg.rank, cfg.K
    d.dtype = C.LLATTE_BF16 if cfg.dtype == "bf16" else C.LLATTE_F32
    return d


class DeviceSummaries:
    _KEYS = ("W1", "W2", "A1", "B1", "A2", "B2")

    def __init__(self, cfg, L, device="cuda", stream=None):
        self.cfg = cfg
        self.desc = make_summary_desc(cfg)
        self.device = device
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        self._keep = []
        w = C.llatte_summary_weights()
        for k in self._KEYS:
            t = torch.from_numpy(np.ascontiguousarray(L[k], dtype=np.float32))
            t = t.to(device=device).to(dt).contiguous()
            self._keep.append(t)
            setattr(w, k, t.data_ptr())
        self.w = w
        n = C.llatte_summary_packed_size(self.desc)
        self.packed = torch.empty(n, dtype=torch.uint8, device=device)
        C.llatte_summary_pack(self.desc, w, self.packed, stream)
        self._ws = None

    def __call__(self, z, out=None, stream=None):
        """z: float32 [B, d_z] on the device -> float32 [K, B, d_seq]."""
        B = z.shape[0]
        if out is None:
            out = torch.empty((self.cfg.K, B, self.cfg.d_seq), dtype=torch.float32,
                              device=self.device)
        n = C.llatte_summaries_workspace_size(self.desc, B)
        if self._ws is None or self._ws.numel() < n:
            self._ws = torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)
        C.llatte_summaries(self.desc, self.packed, z, B, out, self._ws, stream)
        return out
