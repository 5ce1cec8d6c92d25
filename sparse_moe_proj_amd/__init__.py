"""Python binding of liblmoe, the MI355X latent-MoE block library (C ABI in include/lmoe.h).

Argument marshalling only: every step of the block runs in the library's HIP kernels.  The
functions carry the C names and return the C status code (an int, LMOE_OK == 0); `check`
turns a non-zero status into LmoeError with the library's message.  Tensor arguments may be
torch tensors (their data_ptr() is passed), raw device addresses (int) or None.

The library is loaded at import time; a missing build raises ImportError, so nothing can
silently run on another implementation.
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblmoe.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "lmoe.h")

LMOE_OK, LMOE_ERR_NULL, LMOE_ERR_SHAPE, LMOE_ERR_DTYPE, LMOE_ERR_ALIGN = 0, 1, 2, 3, 4
LMOE_ERR_WORKSPACE, LMOE_ERR_UNSUPPORTED, LMOE_ERR_HIP = 5, 6, 7
LMOE_F32, LMOE_BF16, LMOE_MXFP4, LMOE_NVFP4 = 0, 1, 2, 3
DTYPES = {"f32": LMOE_F32, "bf16": LMOE_BF16, "mxfp4": LMOE_MXFP4, "nvfp4": LMOE_NVFP4}


class LmoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"lmoe status {status}: {message}")
        self.status = status


class lmoe_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("hidden", "latent", "n_experts", "top_k", "ffn", "shared_ffn",
                                              "act_dtype", "dense_dtype", "expert_dtype", "groups", "mx_mfma_min_t")]


class lmoe_weights(ctypes.Structure):
    _fields_ = [("D", ctypes.c_void_p), ("U", ctypes.c_void_p), ("Wr", ctypes.c_void_p), ("br", ctypes.c_void_p),
                ("shared", ctypes.c_void_p), ("experts", ctypes.c_void_p), ("Gr", ctypes.c_void_p)]


class lmoe_forward_opts(ctypes.Structure):
    _fields_ = [("prenorm", ctypes.c_int32), ("residual", ctypes.c_int32), ("aux_z", ctypes.c_void_p),
                ("aux_ids", ctypes.c_void_p), ("aux_w", ctypes.c_void_p), ("aux_offsets", ctypes.c_void_p),
                ("aux_perm", ctypes.c_void_p), ("stage_events", ctypes.c_void_p)]


def _load():
    # torch is imported first so that its HIP runtime is the one in the process: liblmoe.so
    # then binds to it (same soname) instead of loading a second runtime that would not share
    # torch's device memory and streams.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python sparse_moe_proj_amd/build.py` "
                          "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfgp = ctypes.POINTER(lmoe_config)
    wp = ctypes.POINTER(lmoe_weights)
    sig = {
        "lmoe_expert_record_bytes": (SZ, [cfgp, I32]),
        "lmoe_workspace_bytes": (I32, [cfgp, I32, ctypes.POINTER(SZ)]),
        "lmoe_permute_workspace_bytes": (I32, [cfgp, I32, ctypes.POINTER(SZ)]),
        "lmoe_route": (I32, [cfgp, wp, P, I32, P, P, P, SZ, P]),
        "lmoe_permute": (I32, [cfgp, P, I32, P, P, P, P, SZ, P]),
        "lmoe_forward": (I32, [cfgp, wp, P, I32, P, ctypes.POINTER(lmoe_forward_opts), P, SZ, P]),
        "lmoe_forward_noalloc": (I32, [cfgp, wp, P, I32, P, ctypes.POINTER(lmoe_forward_opts), P]),
        "lmoe_pack_experts": (I32, [cfgp, I32, P, P, I32, P]),
        "lmoe_fold_router_bytes": (SZ, [cfgp]),
        "lmoe_fold_router": (I32, [cfgp, P, P, P, P]),
        "lmoe_status_str": (ctypes.c_char_p, [I32]),
        "lmoe_last_error": (ctypes.c_char_p, []),
        "lmoe_version": (I32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def header_symbols() -> list[str]:
    """Every function the C header declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(lmoe_[a-z_]+)\s*\(", text)))


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def make_config(hidden, latent, n_experts, top_k, ffn, shared_ffn, act="bf16", dense="bf16", expert="bf16", groups=1,
                mx_mfma_min_t=0):
    """lmoe_config; mx_mfma_min_t: 0 = the library's default (96), -1 = no block-scaled MFMA path."""
    return lmoe_config(hidden, latent, n_experts, top_k, ffn, shared_ffn, DTYPES[act], DTYPES[dense], DTYPES[expert],
                       int(groups), int(mx_mfma_min_t))


def make_weights(D, U, Wr, br, shared, experts, Gr=None):
    """The struct of device pointers; it also holds references to the tensors given, so that a
    temporary (make_weights(..., to_device(a), ...)) stays allocated while the struct is in use."""
    w = lmoe_weights(_p(D), _p(U), _p(Wr), _p(br), _p(shared), _p(experts), _p(Gr))
    w._keep = (D, U, Wr, br, shared, experts, Gr)
    return w


LMOE_N_STAGES = 9
STAGES = ("prenorm", "D", "router", "topk", "permute", "expert_up", "expert_down", "combine", "U")


def make_opts(prenorm=0, residual=0, aux_z=None, aux_ids=None, aux_w=None, aux_offsets=None, aux_perm=None,
              stage_events=None):
    """stage_events: None or a ctypes array of 2 * LMOE_N_STAGES hipEvent_t handles (keep it alive)."""
    ev = ctypes.cast(stage_events, ctypes.c_void_p).value if stage_events is not None else None
    o = lmoe_forward_opts(int(prenorm), int(residual), _p(aux_z), _p(aux_ids), _p(aux_w), _p(aux_offsets),
                          _p(aux_perm), ev)
    o._keep = (aux_z, aux_ids, aux_w, aux_offsets, aux_perm, stage_events)
    return o


def last_error() -> str:
    return lib.lmoe_last_error().decode()


def check(status: int) -> None:
    if status != LMOE_OK:
        raise LmoeError(status, last_error())


def lmoe_expert_record_bytes(cfg, shared=0) -> int:
    return lib.lmoe_expert_record_bytes(ctypes.byref(cfg), int(shared))


def lmoe_workspace_bytes(cfg, T) -> int:
    n = ctypes.c_size_t(0)
    check(lib.lmoe_workspace_bytes(ctypes.byref(cfg), int(T), ctypes.byref(n)))
    return n.value


def lmoe_permute_workspace_bytes(cfg, T) -> int:
    n = ctypes.c_size_t(0)
    check(lib.lmoe_permute_workspace_bytes(ctypes.byref(cfg), int(T), ctypes.byref(n)))
    return n.value


def lmoe_route(cfg, weights, z, T, ids, w, ws, ws_bytes, stream=None) -> int:
    return lib.lmoe_route(ctypes.byref(cfg), ctypes.byref(weights), _p(z), int(T), _p(ids), _p(w), _p(ws),
                          int(ws_bytes), _stream(stream))


def lmoe_permute(cfg, ids, T, offsets, perm, inv, ws, ws_bytes, stream=None) -> int:
    return lib.lmoe_permute(ctypes.byref(cfg), _p(ids), int(T), _p(offsets), _p(perm), _p(inv), _p(ws), int(ws_bytes),
                            _stream(stream))


def lmoe_forward(cfg, weights, x, T, y, opts, ws, ws_bytes, stream=None) -> int:
    return lib.lmoe_forward(ctypes.byref(cfg), ctypes.byref(weights), _p(x), int(T), _p(y),
                            ctypes.byref(opts) if opts is not None else None, _p(ws), int(ws_bytes), _stream(stream))


LMOE_NOALLOC_SCRATCH_BYTES = 32 << 20  # the library's static workspace per GPU (lmoe.h)


def lmoe_forward_noalloc(cfg, weights, x, T, y, opts, stream=None) -> int:
    return lib.lmoe_forward_noalloc(ctypes.byref(cfg), ctypes.byref(weights), _p(x), int(T), _p(y),
                                    ctypes.byref(opts) if opts is not None else None, _stream(stream))


def lmoe_pack_experts(cfg, shared, src, dst, n_records, stream=None) -> int:
    return lib.lmoe_pack_experts(ctypes.byref(cfg), int(shared), _p(src), _p(dst), int(n_records), _stream(stream))


def lmoe_fold_router_bytes(cfg) -> int:
    return int(lib.lmoe_fold_router_bytes(ctypes.byref(cfg)))


def lmoe_fold_router(cfg, D, Wr, Gr, stream=None) -> int:
    return lib.lmoe_fold_router(ctypes.byref(cfg), _p(D), _p(Wr), _p(Gr), _stream(stream))


def lmoe_status_str(status: int) -> str:
    return lib.lmoe_status_str(int(status)).decode()


def lmoe_version() -> int:
    return lib.lmoe_version()
