"""CPU oracle for the Edge0-145B latent-MoE feed-forward block (numpy, float64).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module: only the
tests, the package smoke check and the benchmark's CPU-baseline leg use it.  It shares no
code with the HIP library (it imports numpy and nothing else); its inputs come from the
seeded generator in ``lmoe_data`` and are promoted to float64 here by its own decoders.

What it computes follows the Edge0-145B model-detail page, section "模型架构" (Fig. 3 caption
and the spec table after it):
  * attention works in the full 2560-d space; D then projects each token to the latent width
    l = 1792, one D per layer shared by all experts;
  * a router picks 10 of the 512 experts;
  * each chosen expert is a SwiGLU l -> 640 -> l; one shared expert runs alongside;
  * the merged result is projected back to 2560-d by U, one U per layer.
The page leaves the router's normalisation, tie order and the merge weights open; the
readings taken here (softmax over the selected logits, lower id wins exact ties, slots in
ascending expert id, shared expert weight 1, bias-free projections except the router) are
the plainest ones consistent with the caption and are listed with the design notes.

The release report "1450 亿参数端侧模型 Edge0-145B 开源" (section "Edge0 的内部机制", paragraph
"架构：在稀疏专家之间共享大型矩阵") describes the sharing per group instead: every 64 experts form a group sharing one pair of large
matrices.  With G groups (shape.groups; 1 is the model-detail page's form) group g owns D_g
and U_g; expert e is in group e // (E / G); its router row and its SwiGLU read that group's
latent z_g = x D_g^T, its weighted output joins that group's merged row m_g, and
y = sum_g m_g U_g^T.  The pages do not place the shared expert; it is read here as a member
of group 0 (z_0 in, m_0 out), which for G = 1 is the form above.

Every function below is written in the order the caption describes, with no blocking or
fusion: one numpy matmul per projection, explicit loops over tokens and chosen experts.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------------------------
# storage decoders (the oracle's own; exact)
# ---------------------------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (a bf16 value is the top half of a float32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


# Largest finite bf16 value, (2 - 2^-7) * 2^127 (bf16 keeps float32's 8 exponent bits and 7 of
# its 23 stored significand bits).
BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """float64 -> the nearest bf16 value (ties to even), returned as float64; one rounding of the
    exact value, with no float32 step in between.

    Used only where the method itself rounds to bf16 (the stack's block input).  bf16 has 8
    significant bits, so the spacing of the values around v in [2^(e-1), 2^e) is 2^(e-8); below
    the smallest normal 2^-126 the spacing stays 2^-133 (subnormals).  Values beyond the largest
    finite bf16 by half a spacing or more become infinities."""
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)                                   # |v| in [2^(e-1), 2^e)
    q = np.ldexp(1.0, np.maximum(e - 8, -133))           # spacing of bf16 values there
    r = np.rint(v / q) * q                               # v / q is exact; rint: ties to even
    return np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, v), r)


# E2M1 magnitudes by 3-bit code (OCP Microscaling Formats v1.0, FP4 E2M1): exponent bias 1,
# one mantissa bit, code 0b001 is the subnormal 0.5.
E2M1_VALUES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def mxfp4_decode(nibbles: np.ndarray, scales: np.ndarray, rows: int, K: int) -> np.ndarray:
    """MXFP4 -> float64 [rows][K]: value = (-1)^s * E2M1(code) * 2^(scale_byte - 127),
    one E8M0 scale byte per 32 consecutive K values, low nibble = even K index."""
    nib = np.asarray(nibbles, dtype=np.uint8).reshape(rows, K // 2)
    codes = np.empty((rows, K), dtype=np.uint8)
    codes[:, 0::2] = nib & 0x0F
    codes[:, 1::2] = nib >> 4
    table = np.array(E2M1_VALUES, dtype=np.float64)
    mag = table[codes & 0x7]
    val = np.where(codes & 0x8, -mag, mag)
    sc = np.asarray(scales, dtype=np.uint8).reshape(rows, K // 32).astype(np.int64) - 127
    return val * np.repeat(np.ldexp(1.0, sc), 32, axis=1)


def e4m3_decode(b: np.ndarray) -> np.ndarray:
    """FP8 E4M3 bytes -> float64: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is
    subnormal (m/8 * 2^-6); S.1111.111 is NaN; there are no infinities."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    e, m = (b >> 3) & 0xF, b & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.ldexp(1.0, e - 10))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(b & 0x80, -mag, mag)


def nvfp4_decode(nibbles: np.ndarray, scales: np.ndarray, tensor_scale: float, rows: int, K: int) -> np.ndarray:
    """NVFP4 -> float64 [rows][K]: value = (-1)^s * E2M1(code) * E4M3(scale byte) * tensor_scale,
    one E4M3 scale byte per 16 consecutive K values, low nibble = even K index."""
    nib = np.asarray(nibbles, dtype=np.uint8).reshape(rows, K // 2)
    codes = np.empty((rows, K), dtype=np.uint8)
    codes[:, 0::2] = nib & 0x0F
    codes[:, 1::2] = nib >> 4
    table = np.array(E2M1_VALUES, dtype=np.float64)
    mag = table[codes & 0x7]
    val = np.where(codes & 0x8, -mag, mag)
    sc = e4m3_decode(np.asarray(scales, dtype=np.uint8).reshape(rows, K // 16))
    return val * np.repeat(sc, 16, axis=1) * float(tensor_scale)


def decode(arr: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_to_f64(arr)
    raise ValueError(dtype)


def expert_matrices(record: np.ndarray, dtype: str, latent: int, ffn: int):
    """Split one expert record into (gate [F][l], up [F][l], down [l][F]) in float64."""
    l, f = latent, ffn
    if dtype in ("f32", "bf16"):
        r = decode(record, dtype)
        return (r[: f * l].reshape(f, l), r[f * l: 2 * f * l].reshape(f, l), r[2 * f * l: 3 * f * l].reshape(l, f))
    if dtype == "mxfp4":
        nb = f * l // 2
        sb = f * l // 32
        rec = np.asarray(record, dtype=np.uint8)
        g = mxfp4_decode(rec[0:nb], rec[3 * nb: 3 * nb + sb], f, l)
        u = mxfp4_decode(rec[nb: 2 * nb], rec[3 * nb + sb: 3 * nb + 2 * sb], f, l)
        d = mxfp4_decode(rec[2 * nb: 3 * nb], rec[3 * nb + 2 * sb: 3 * nb + 3 * sb], l, f)
        return g, u, d
    if dtype == "nvfp4":
        nb = f * l // 2
        sb = f * l // 16
        rec = np.asarray(record, dtype=np.uint8)
        ts = rec[3 * nb + 3 * sb: 3 * nb + 3 * sb + 12].view(np.float32).astype(np.float64)
        g = nvfp4_decode(rec[0:nb], rec[3 * nb: 3 * nb + sb], ts[0], f, l)
        u = nvfp4_decode(rec[nb: 2 * nb], rec[3 * nb + sb: 3 * nb + 2 * sb], ts[1], f, l)
        d = nvfp4_decode(rec[2 * nb: 3 * nb], rec[3 * nb + 2 * sb: 3 * nb + 3 * sb], ts[2], l, f)
        return g, u, d
    raise ValueError(dtype)


# ---------------------------------------------------------------------------------------------
# the block, step by step
# ---------------------------------------------------------------------------------------------

def silu(v: np.ndarray) -> np.ndarray:
    """SiLU(v) = v / (1 + e^-v), the gate nonlinearity of SwiGLU."""
    return v / (1.0 + np.exp(-v))


def swiglu(z: np.ndarray, gate: np.ndarray, up: np.ndarray, down: np.ndarray) -> np.ndarray:
    """One expert l -> F -> l: (SiLU(z gate^T) * (z up^T)) down^T, rows of z are tokens."""
    return (silu(z @ gate.T) * (z @ up.T)) @ down.T


def router_logits(z: np.ndarray, Wr: np.ndarray, br: np.ndarray, groups: int = 1) -> np.ndarray:
    """logits[t][e] = z_{g(e)}[t] . Wr[e] + br[e]; z is [T][groups * latent] (group g's latent
    in columns g*latent ..), expert e in group e // (E / groups)."""
    E, L = Wr.shape
    Eg = E // groups
    logits = np.empty((z.shape[0], E))
    for g in range(groups):
        logits[:, g * Eg:(g + 1) * Eg] = z[:, g * L:(g + 1) * L] @ Wr[g * Eg:(g + 1) * Eg].T
    return logits + br[None, :]


def route(z: np.ndarray, Wr: np.ndarray, br: np.ndarray, k: int, groups: int = 1):
    """Router: logits = z Wr^T + br (per expert group, see router_logits); keep the k largest
    (a lower expert id wins an exact tie); weights = softmax over the k kept logits (equal to a
    softmax over all E renormalised over the kept ones).  Returns ids [T][k] in ascending expert
    id, weights [T][k] in the same order, the 10th/11th gap lambda_(k) - lambda_(k+1) per token
    (inf when E == k), and logits."""
    logits = router_logits(z, Wr, br, groups)
    T, E = logits.shape
    order = np.argsort(-logits, axis=1, kind="stable")   # stable: equal values keep id order
    chosen = np.sort(order[:, :k], axis=1)
    srt = np.take_along_axis(logits, order, axis=1)
    gap = srt[:, k - 1] - srt[:, k] if E > k else np.full(T, np.inf)
    lam = np.take_along_axis(logits, chosen, axis=1)
    e = np.exp(lam - lam.max(axis=1, keepdims=True))
    w = e / e.sum(axis=1, keepdims=True)
    return chosen.astype(np.int32), w, gap, logits


def permute(ids: np.ndarray, n_experts: int):
    """Token->expert permutation.  Flat slot index f = t*k + s; perm lists the f's grouped by
    expert in ascending expert id and, inside an expert, in ascending f (a stable sort);
    offsets[e] is where expert e's segment starts (exclusive prefix sum of the counts,
    offsets[E] = T*k); inv is the inverse of perm."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=n_experts)
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(flat, kind="stable")
    inv = np.empty_like(perm)
    inv[perm] = np.arange(flat.size)
    return offsets.astype(np.int32), perm.astype(np.int32), inv.astype(np.int32)


class Layer:
    """float64 view of one layer's weights, decoding experts on first use."""

    def __init__(self, lw):
        s = lw.shape
        self.shape = s
        self.D = decode(lw.D, lw.dense)
        self.U = decode(lw.U, lw.dense)
        self.Wr = decode(lw.Wr, lw.dense)
        self.br = np.asarray(lw.br, dtype=np.float32).astype(np.float64)
        self.shared = None
        if lw.shared is not None and s.shared_ffn > 0:
            self.shared = expert_matrices(lw.shared, lw.dense, s.latent, s.shared_ffn)
        self._lw = lw
        self._cache = {}

    def expert(self, e: int):
        if e not in self._cache:
            s = self.shape
            self._cache[e] = expert_matrices(self._lw.experts[e], self._lw.expert, s.latent, s.ffn)
        return self._cache[e]

    def prefetch(self, experts, threads: int = 8):
        """Decode the given experts up front, several at a time (decoding only; no arithmetic
        of the block)."""
        from concurrent.futures import ThreadPoolExecutor
        todo = sorted(set(int(e) for e in np.asarray(experts).ravel()) - set(self._cache))
        s = self.shape
        with ThreadPoolExecutor(threads) as ex:
            mats = list(ex.map(lambda e: expert_matrices(self._lw.experts[e], self._lw.expert, s.latent, s.ffn), todo))
        self._cache.update(zip(todo, mats))


def block_forward(layer: Layer, x: np.ndarray, forced_ids: dict | None = None):
    """The latent-MoE block for the tokens in x (float64 [T][hidden]).

    forced_ids optionally maps a token row to an id set to use instead of the router's
    choice (the weights are then the softmax over those experts' logits).
    Returns dict(y, z, ids, w, gap, logits, m)."""
    s = layer.shape
    G, L = s.groups, s.latent
    Eg = s.n_experts // G
    z = x @ layer.D.T                                   # D: hidden -> latent (each group's D_g)
    ids, w, gap, logits = route(z, layer.Wr, layer.br, s.top_k, G)
    if forced_ids:
        ids = ids.copy()
        w = w.copy()
        for t, fid in forced_ids.items():
            fid = np.sort(np.asarray(fid, dtype=np.int64))
            lam = logits[t, fid]
            ee = np.exp(lam - lam.max())
            ids[t] = fid
            w[t] = ee / ee.sum()
    T = x.shape[0]
    m = np.zeros((T, G * L))                            # m_g in columns g*L ..
    if layer.shared is not None:
        m[:, :L] += swiglu(z[:, :L], *layer.shared)     # shared expert, weight 1 (group 0)
    for t in range(T):
        for slot in range(s.top_k):                     # slots in ascending expert id
            e = int(ids[t, slot])
            c = (e // Eg) * L                           # the expert's group
            g, u, d = layer.expert(e)
            m[t, c:c + L] += w[t, slot] * swiglu(z[t:t + 1, c:c + L], g, u, d)[0]
    y = m @ layer.U.T                                   # U: latent -> hidden (sum over groups)
    return dict(y=y, z=z, ids=ids, w=w, gap=gap, logits=logits, m=m)


def rmsnorm(h: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """Unit-gain RMSNorm over the hidden dimension."""
    return h / np.sqrt(np.mean(h * h, axis=1, keepdims=True) + eps)


def stack_step(layer: Layer, h: np.ndarray):
    """One residual layer of the FFN-only stack, h carried in float32:
    h_next = fp32(h + block(bf16(RMSNorm(h))))."""
    x = round_to_bf16(rmsnorm(h))
    out = block_forward(layer, x)
    out["h_next"] = (h + out["y"]).astype(np.float32).astype(np.float64)
    out["x"] = x
    return out
