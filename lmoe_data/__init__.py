"""Seeded synthetic inputs for the latent-MoE feed-forward block.

This module is the only code shared by the HIP path's tests/bench and the CPU
oracle.  It draws tensors and encodes them in the storage dtypes (fp32, bf16
bits, MXFP4 and NVFP4 bytes); it contains none of the block's arithmetic (no
projection, routing, SwiGLU, combine, and no 4-bit *decoding*).

Shapes follow the Edge0-145B model-detail page ("模型架构" spec table and the
Fig. 3 caption): hidden 2560, latent width l = 1792, 512 experts per layer with
10 routed + 1 shared active, SwiGLU width 640, 48 layers.

Storage conventions (all row-major, innermost dimension contiguous, every
matrix stored output-major with its reduction dimension K contiguous):
  D  [latent][hidden]      z = x . D^T
  U  [hidden][latent]      y = m . U^T
  Wr [E][latent]           router logits = z . Wr^T + br
  expert record (f32/bf16 elements): gate [F][l], up [F][l], down [l][F]
  expert record (MXFP4 bytes): gate nibbles [F][l/2], up nibbles [F][l/2],
      down nibbles [l][F/2], then gate scales [F][l/32], up scales [F][l/32],
      down scales [l][F/32].  Low nibble = even K index.  One e8m0 scale byte
      per 32 consecutive K values.
  expert record (NVFP4 bytes): the three nibble arrays as for MXFP4, then gate
      scales [F][l/16], up scales [F][l/16], down scales [l][F/16] (one FP8 e4m3
      byte per 16 consecutive K values), then the three matrices' fp32 tensor
      scales (gate, up, down) and 4 zero bytes.

Seeds: SeedSequence([0x4C4D4F45, workload id, layer (or expert bank), tensor
code, index]) feeding PCG64; normals are drawn in float32 and scaled by
float32(1/sqrt(fan_in)), then rounded to the storage dtype (bf16 by
round-to-nearest-even on the fp32 bits).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

MAGIC = 0x4C4D4F45

# tensor codes in the seed key
T_X, T_D, T_U, T_WR, T_BIAS, T_SHARED, T_EXPERT, T_H0 = 1, 2, 3, 4, 5, 6, 7, 8


@dataclass(frozen=True)
class Shape:
    hidden: int
    latent: int
    n_experts: int
    top_k: int
    ffn: int
    shared_ffn: int  # 0 = no shared expert
    # Expert groups with their own D/U pair: experts g*E/G .. (g+1)*E/G - 1 form group g, D is
    # [G*latent][hidden] (group g's rows g*latent ..), U is [hidden][G*latent] (its columns).
    groups: int = 1

    def record_elems(self, ffn: Optional[int] = None) -> int:
        f = self.ffn if ffn is None else ffn
        return 3 * f * self.latent

    def mxfp4_record_bytes(self) -> int:
        f, l = self.ffn, self.latent
        return 3 * (f * l // 2) + 3 * (f * l // 32)

    def nvfp4_record_bytes(self) -> int:
        f, l = self.ffn, self.latent
        return 3 * (f * l // 2) + 3 * (f * l // 16) + 16


TINY = Shape(hidden=256, latent=128, n_experts=16, top_k=2, ffn=64, shared_ffn=64)
EDGE0_145B = Shape(hidden=2560, latent=1792, n_experts=512, top_k=10, ffn=640, shared_ffn=640)
# The 120B model: the pages give only its latent width (1280); the other dimensions are read as
# the 145B's (same family, same expert pool layout).
EDGE0_120B = Shape(hidden=2560, latent=1280, n_experts=512, top_k=10, ffn=640, shared_ffn=640)
# The release report's description of the sharing (section "Edge0 的内部机制"): every 64 experts
# form a group that shares one pair of large matrices, so 512 experts have 8 D/U pairs.
EDGE0_145B_G64 = Shape(hidden=2560, latent=1792, n_experts=512, top_k=10, ffn=640, shared_ffn=640, groups=8)


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    shape: Shape
    T: int
    act: str       # 'f32' | 'bf16'   (x and y)
    dense: str     # 'f32' | 'bf16'   (D, U, Wr, shared expert)
    expert: str    # 'f32' | 'bf16' | 'mxfp4' | 'nvfp4'
    bias: str      # 'zero' | 'zipf'
    zipf_s: float = 1.1
    layers: int = 1
    expert_banks: int = 0  # >0: layer l's routed experts are drawn from bank l % expert_banks; 0: its own


WORKLOADS = {
    "tiny_f32": Workload(1, "tiny_f32", TINY, 32, "f32", "f32", "f32", "zero"),
    "decode_t8": Workload(2, "decode_t8", EDGE0_145B, 8, "bf16", "bf16", "bf16", "zipf"),
    "prefill_t4096": Workload(3, "prefill_t4096", EDGE0_145B, 4096, "bf16", "bf16", "bf16", "zero"),
    "prefill_t16384": Workload(4, "prefill_t16384", EDGE0_145B, 16384, "bf16", "bf16", "bf16", "zipf"),
    "stack48_mxfp4_t8": Workload(5, "stack48_mxfp4_t8", EDGE0_145B, 8, "bf16", "bf16", "mxfp4", "zipf",
                                 layers=48),
    "decode120_t8": Workload(6, "decode120_t8", EDGE0_120B, 8, "bf16", "bf16", "bf16", "zipf"),
    "decode_nvfp4_t8": Workload(7, "decode_nvfp4_t8", EDGE0_145B, 8, "bf16", "bf16", "nvfp4", "zipf"),
    "decode_group64_t8": Workload(8, "decode_group64_t8", EDGE0_145B_G64, 8, "bf16", "bf16", "bf16", "zipf"),
    "prefill_mxfp4_t16384": Workload(9, "prefill_mxfp4_t16384", EDGE0_145B, 16384, "bf16", "bf16", "mxfp4", "zipf"),
}


def n_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def rng_for(wid: int, layer: int, tensor: int, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([MAGIC, wid, layer, tensor, index])))


def normal_f32(rng: np.random.Generator, n: int, std: float) -> np.ndarray:
    a = rng.standard_normal(n, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even) and return the 16-bit patterns.

    Inputs are finite by construction.  The array passed in is consumed (modified in place).
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    t = u >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    u += t
    u >>= np.uint32(16)
    return u.astype(np.uint16)


# ---------------------------------------------------------------------------------------------
# MXFP4 encoder (OCP Microscaling Formats v1.0: MXFP4 = FP4 E2M1 elements, E8M0 shared scale per
# block of 32).  The shared exponent is floor(log2(amax)) - 2 (2 = emax of E2M1), elements are
# rounded to nearest-even on the E2M1 grid and saturate at +-6.  An all-zero block gets scale byte 0.
# ---------------------------------------------------------------------------------------------
# E2M1 rounding midpoints (between consecutive grid values 0, .5, 1, 1.5, 2, 3, 4, 6) and, for each,
# whether a value exactly on it rounds up: a tie goes to the even code, i.e. up at odd indices.
_E2M1_MIDS = ((0.25, False), (0.75, True), (1.25, False), (1.75, True), (2.5, False), (3.5, True), (5.0, False))


def _e2m1_codes(a: np.ndarray) -> np.ndarray:
    """|values| (already divided by their scale, float32 or float64) -> E2M1 magnitude codes,
    nearest-even, saturating at 6: the number of midpoints the value lies above (or on, for the
    midpoints whose tie rounds up).  Every midpoint is exact in both float types."""
    code = np.zeros(a.shape, dtype=np.uint8)
    for m, up in _E2M1_MIDS:
        code += (a >= m) if up else (a > m)
    return code


def mxfp4_encode(w: np.ndarray):
    """float32 [rows][K] (K % 32 == 0) -> (nibbles uint8 [rows][K/2], scales uint8 [rows][K/32]).

    Works in float32: the rescale by 2^-shared is a power-of-two product, exact unless the result
    falls below the float32 normal range, where it is far below the first midpoint either way."""
    w = np.asarray(w, dtype=np.float32)
    rows, K = w.shape
    assert K % 32 == 0
    blk = w.reshape(rows, K // 32, 32)
    mag = np.abs(blk)
    amax = mag.max(axis=2)
    _, ex = np.frexp(amax)                      # amax = m * 2^ex, m in [0.5, 1)
    shared = np.where(amax > 0, ex - 1 - 2, -127)
    shared = np.clip(shared, -127, 127)
    scales = (shared + 127).astype(np.uint8)
    mag *= np.ldexp(np.float32(1.0), -shared).astype(np.float32)[..., None]
    code = _e2m1_codes(mag)
    code |= (np.signbit(blk) & (code != 0)).view(np.uint8) << 3   # -0 is stored as +0
    nib = code.reshape(rows, K)
    packed = nib[:, 0::2] | (nib[:, 1::2] << 4)
    return packed, scales


# ---------------------------------------------------------------------------------------------
# NVFP4 encoder (the pages name the format only).  Elements are FP4 E2M1 as above; every 16
# consecutive K values share an FP8 E4M3 scale (1 sign, 4 exponent bits with bias 7, 3 mantissa
# bits, largest finite value 448, no infinities); every matrix has one fp32 tensor scale:
#     value = E2M1(element) * E4M3(block scale) * tensor_scale.
# The tensor scale is amax(matrix) / (6 * 448), so the largest block scale lands on 448; a
# block's scale is E4M3(amax(block) / 6 / tensor_scale) rounded to nearest-even (saturating at
# 448); elements are w / (block scale * tensor scale) rounded to nearest-even on the E2M1 grid
# (saturating at +-6).  A block whose scale rounds to 0 stores zeros.
# ---------------------------------------------------------------------------------------------
def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Non-negative float64 -> the nearest E4M3 value (ties to even), saturating at 448."""
    x = np.asarray(x, dtype=np.float64)
    _, ex = np.frexp(np.where(x > 0, x, 1.0))
    e = np.maximum(ex - 1, -6)                       # exponent of the binade (subnormals: -6)
    step = np.ldexp(1.0, e - 3)                      # 3 mantissa bits
    q = np.round(x / step) * step                    # numpy rounds half to even
    return np.minimum(np.where(x > 0, q, 0.0), 448.0)


def e4m3_bits(v: np.ndarray) -> np.ndarray:
    """E4M3 values (non-negative, exactly representable) -> their bytes."""
    v = np.asarray(v, dtype=np.float64)
    _, ex = np.frexp(np.where(v > 0, v, 1.0))
    e = ex - 1
    normal = (v >= 2.0 ** -6)
    mant = np.where(normal, np.round((v / np.ldexp(1.0, e) - 1.0) * 8), np.round(v / 2.0 ** -9))
    expf = np.where(normal, e + 7, 0)
    b = (expf.astype(np.int64) << 3) | mant.astype(np.int64)
    return np.where(v > 0, b, 0).astype(np.uint8)


def nvfp4_encode(w: np.ndarray):
    """float32 [rows][K] (K % 16 == 0) -> (nibbles uint8 [rows][K/2], scales uint8 [rows][K/16],
    tensor scale float32)."""
    w = np.asarray(w, dtype=np.float32)
    rows, K = w.shape
    assert K % 16 == 0
    amax_t = float(np.abs(w).max())
    ts = np.float32(amax_t / (6.0 * 448.0)) if amax_t > 0 else np.float32(1.0)
    blk = w.reshape(rows, K // 16, 16).astype(np.float64)
    sb = e4m3_round(np.abs(blk).max(axis=2) / 6.0 / float(ts))
    denom = sb[..., None] * float(ts)
    a = np.where(denom > 0, np.abs(blk) / np.where(denom > 0, denom, 1.0), 0.0)
    code = _e2m1_codes(a)
    sign = (blk < 0).astype(np.uint8) << 3
    sign[code == 0] = 0
    nib = (code | sign).reshape(rows, K)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return packed, e4m3_bits(sb).reshape(rows, K // 16), ts


# ---------------------------------------------------------------------------------------------
@dataclass
class LayerWeights:
    shape: Shape
    dense: str
    expert: str
    D: np.ndarray
    U: np.ndarray
    Wr: np.ndarray
    br: np.ndarray
    shared: Optional[np.ndarray]
    experts: np.ndarray           # [E][record] (float32 | uint16 bf16 bits | uint8 MXFP4 bytes)
    meta: dict = field(default_factory=dict)


def _encode(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return a
    if dtype == "bf16":
        return bf16_bits(a)
    raise ValueError(dtype)


def expert_record(shape: Shape, rng: np.random.Generator, dtype: str, ffn: Optional[int] = None) -> np.ndarray:
    """One expert's record: gate [F][l], up [F][l] ~ N(0, 1/l); down [l][F] ~ N(0, 1/F)."""
    f = shape.ffn if ffn is None else ffn
    l = shape.latent
    a = rng.standard_normal(3 * f * l, dtype=np.float32)
    a[: 2 * f * l] *= np.float32(1.0 / np.sqrt(l))
    a[2 * f * l:] *= np.float32(1.0 / np.sqrt(f))
    if dtype in ("f32", "bf16"):
        return _encode(a, dtype)
    g, u, d = a[: f * l].reshape(f, l), a[f * l: 2 * f * l].reshape(f, l), a[2 * f * l:].reshape(l, f)
    if dtype == "mxfp4":
        parts = [mxfp4_encode(m) for m in (g, u, d)]
        return np.concatenate([p[0].ravel() for p in parts] + [p[1].ravel() for p in parts])
    if dtype == "nvfp4":
        parts = [nvfp4_encode(m) for m in (g, u, d)]
        tail = np.array([p[2] for p in parts] + [0.0], dtype=np.float32).view(np.uint8)
        return np.concatenate([p[0].ravel() for p in parts] + [p[1].ravel() for p in parts] + [tail])
    raise ValueError(dtype)


def router_bias(wl: Workload, layer: int) -> np.ndarray:
    """Zipf(s) prior over expert ids as a log-prior bias: b_e = -s * ln(1 + pi(e)), pi a seeded
    permutation of 0..E-1, so that softmax weight ~ rank^-s.  'zero' gives b = 0."""
    E = wl.shape.n_experts
    if wl.bias == "zero":
        return np.zeros(E, dtype=np.float32)
    rng = rng_for(wl.wid, layer, T_BIAS)
    pi = rng.permutation(E)
    return (-wl.zipf_s * np.log1p(pi.astype(np.float64))).astype(np.float32)


def make_experts(wl: Workload, bank: int, threads: Optional[int] = None) -> np.ndarray:
    """All routed expert records of one layer (or expert bank): [E][record]."""
    s = wl.shape
    rec0 = expert_record(s, rng_for(wl.wid, bank, T_EXPERT, 0), wl.expert)
    experts = np.empty((s.n_experts, rec0.size), dtype=rec0.dtype)
    experts[0] = rec0

    def fill(e):
        experts[e] = expert_record(s, rng_for(wl.wid, bank, T_EXPERT, e), wl.expert)

    with ThreadPoolExecutor(threads or n_threads()) as ex:
        list(ex.map(fill, range(1, s.n_experts)))
    return experts


def expert_bank(wl: Workload, layer: int) -> int:
    return layer % wl.expert_banks if wl.expert_banks else layer


def make_layer(wl: Workload, layer: int = 0, threads: Optional[int] = None,
               experts: Optional[np.ndarray] = None) -> LayerWeights:
    """One layer's weights.  `experts` may pass in the already drawn records of this layer's
    expert bank (expert_bank(wl, layer)) so that banks shared by several layers are drawn once."""
    s = wl.shape
    H, L, E, G = s.hidden, s.latent, s.n_experts, s.groups
    # with expert groups: G stacked D matrices [G*L][H]; U [H][G*L], each group's U ~ N(0, 1/L)
    D = _encode(normal_f32(rng_for(wl.wid, layer, T_D), G * L * H, 1.0 / np.sqrt(H)), wl.dense).reshape(G * L, H)
    U = _encode(normal_f32(rng_for(wl.wid, layer, T_U), H * G * L, 1.0 / np.sqrt(L)), wl.dense).reshape(H, G * L)
    Wr = _encode(normal_f32(rng_for(wl.wid, layer, T_WR), E * L, 1.0 / np.sqrt(L)), wl.dense).reshape(E, L)
    br = router_bias(wl, layer)
    shared = None
    if s.shared_ffn > 0:
        shared = expert_record(s, rng_for(wl.wid, layer, T_SHARED), wl.dense, ffn=s.shared_ffn)
    bank = expert_bank(wl, layer)
    if experts is None:
        experts = make_experts(wl, bank, threads)
    return LayerWeights(s, wl.dense, wl.expert, D, U, Wr, br, shared, experts,
                        meta={"workload": wl.name, "layer": layer, "bank": bank})


def make_tokens(wl: Workload, T: Optional[int] = None, salt: int = 0) -> np.ndarray:
    """Block input x [T][hidden]: N(0,1) in the activation dtype (bf16 bits or float32)."""
    T = wl.T if T is None else T
    a = normal_f32(rng_for(wl.wid, salt, T_X), T * wl.shape.hidden, 1.0)
    return _encode(a, wl.act).reshape(T, wl.shape.hidden)


def make_residual(wl: Workload, T: Optional[int] = None) -> np.ndarray:
    """Stack input h_0 [T][hidden] fp32 ~ N(0,1) (the 48-layer stack carries h in fp32)."""
    T = wl.T if T is None else T
    return normal_f32(rng_for(wl.wid, 0, T_H0), T * wl.shape.hidden, 1.0).reshape(T, wl.shape.hidden)


def random_ids(T: int, E: int, k: int, seed: int = 0, skew: float = 0.0) -> np.ndarray:
    """Valid routing ids for permutation tests: per token k distinct experts in ascending order.
    skew > 0 biases the choice toward low ids (hot experts)."""
    rng = rng_for(99, seed, 0)
    out = np.empty((T, k), dtype=np.int32)
    p = None
    if skew > 0:
        p = 1.0 / np.arange(1, E + 1) ** skew
        p /= p.sum()
    for t in range(T):
        out[t] = np.sort(rng.choice(E, size=k, replace=False, p=p))
    return out
