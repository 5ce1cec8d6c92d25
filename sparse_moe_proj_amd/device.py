"""Device-memory plumbing around the C ABI: upload host weight arrays into torch tensors on
the GPU, size and hold the workspace, and call lmoe_forward on the current stream.

Host arrays follow the storage layout of include/lmoe.h (bf16 as uint16 bit patterns,
MXFP4 records as bytes).  No arithmetic of the block happens here.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (LMOE_OK, check, lmoe_expert_record_bytes, lmoe_fold_router, lmoe_fold_router_bytes,  # noqa: F401
               lmoe_forward, lmoe_pack_experts, lmoe_workspace_bytes, make_config, make_opts, make_weights)


def to_device(a, device="cuda"):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16))
    else:
        t = torch.from_numpy(a)
    return t.to(device)


def pack_records(cfg, records, shared: bool):
    """Device copy of row-major expert records in the packed layout lmoe_forward reads."""
    n = 1 if shared else records.shape[0]
    need = n * lmoe_expert_record_bytes(cfg, int(shared))
    have = records.numel() * records.element_size()
    if have != need:
        raise ValueError(f"expert records hold {have} bytes, {n} records of this configuration need {need}")
    out = torch.empty_like(records)
    check(lmoe_pack_experts(cfg, int(shared), records, out, n))
    return out


def fold_router(cfg, D, Wr):
    """Device copy of the folded router [E][2][hidden] (bf16 hi/lo halves of Wr . D)."""
    n = lmoe_fold_router_bytes(cfg)
    out = torch.empty(n // 2, dtype=torch.int16, device=D.device)
    check(lmoe_fold_router(cfg, D, Wr, out))
    return out


class DeviceLayer:
    """One layer's weights resident in HBM (tensors kept alive by this object).  Expert records
    are uploaded row-major and packed on the device (fp32 records stay row-major).  pack=False
    keeps them as given: only for callers that use the routing entry points alone.  With bf16
    dense weights the folded router is computed too unless fold=False.  mx_mfma_min_t goes to
    lmoe_config (MXFP4 layers: 0 = default threshold of the block-scaled MFMA path, -1 = off)."""

    def __init__(self, lw=None, act="bf16", device="cuda", _copy_of=None, pack=True, fold=True, mx_mfma_min_t=0):
        self.Gr = None
        if _copy_of is not None:
            src = _copy_of
            self.shape, self.act, self.dense, self.expert = src.shape, src.act, src.dense, src.expert
            for n in ("D", "U", "Wr", "br", "shared", "experts", "Gr"):
                t = getattr(src, n)
                setattr(self, n, None if t is None else t.clone())
        else:
            self.shape, self.act, self.dense, self.expert = lw.shape, act, lw.dense, lw.expert
            self.D = to_device(lw.D, device)
            self.U = to_device(lw.U, device)
            self.Wr = to_device(lw.Wr, device)
            self.br = to_device(np.asarray(lw.br, dtype=np.float32), device)
            self.shared = to_device(lw.shared, device)
            self.experts = to_device(lw.experts, device)
        s = self.shape
        mx_min = src.cfg.mx_mfma_min_t if _copy_of is not None else mx_mfma_min_t
        self.cfg = make_config(s.hidden, s.latent, s.n_experts, s.top_k, s.ffn, s.shared_ffn, self.act, self.dense,
                               self.expert, getattr(s, "groups", 1), mx_min)
        if _copy_of is None and pack and self.expert != "f32":
            self.experts = pack_records(self.cfg, self.experts, False)
            if self.shared is not None:
                self.shared = pack_records(self.cfg, self.shared, True)
        if _copy_of is None and fold and self.dense == "bf16":
            self.Gr = fold_router(self.cfg, self.D, self.Wr)
        self.weights = make_weights(self.D, self.U, self.Wr, self.br, self.shared, self.experts, self.Gr)

    def clone(self) -> "DeviceLayer":
        """A byte-identical copy at other HBM addresses."""
        return DeviceLayer(_copy_of=self)

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.D, self.U, self.Wr, self.br, self.shared, self.experts)
                   if t is not None)


class Workspace:
    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None

    def get(self, nbytes: int):
        nbytes = max(256, int(nbytes))
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return self.buf


def forward(layer: DeviceLayer, x, y=None, opts=None, ws: Workspace | None = None, stream=None):
    """y = block(x) on the current stream; returns y (allocated when not given)."""
    T = x.shape[0]
    if y is None:
        dt = torch.float32 if (layer.act == "f32" or (opts is not None and opts.residual)) else torch.int16
        y = torch.empty((T, layer.shape.hidden), dtype=dt, device=x.device)
    ws = ws or Workspace(x.device)
    nb = lmoe_workspace_bytes(layer.cfg, T)
    buf = ws.get(nb)
    check(lmoe_forward(layer.cfg, layer.weights, x, T, y, opts, buf, buf.numel(), stream))
    return y
