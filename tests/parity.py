"""Helpers for the GPU parity tests: run the HIP block through the C ABI with every export
switched on, and compare with the CPU oracle.

Acceptance (numbers fixed in one place):
  * routing: the GPU's ids equal the oracle's for every token whose 10th/11th logit gap
    (k-th/(k+1)-th, on the oracle's float64 logits) is at least GAP; a token under the gap may
    pick either side of the near-tie, and then each of its picks must be within GAP of the
    oracle's k-th logit and its output is checked against the oracle run on those picks;
  * permutation: offsets/perm equal the oracle's stable sort of the GPU's ids, bit for bit;
  * outputs: per token, max|y_gpu - y_oracle| / max|y_oracle| <= TOL[dtype];
  * routing weights within WTOL of the oracle's.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import lmoe_data as gen
import oracle
import sparse_moe_proj_amd as lm
from sparse_moe_proj_amd.device import DeviceLayer, Workspace, to_device

GAP = 1e-3
TOL = {"f32": 1e-4, "bf16": 2e-2, "mxfp4": 6e-2, "nvfp4": 6e-2}
WTOL = 2e-4


def log(*a):
    print(*a, flush=True, file=sys.stderr)


def host(t: torch.Tensor) -> np.ndarray:
    a = t.detach().cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def act_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    return oracle.decode(a, dtype)


def normwise_rel(y: np.ndarray, ref: np.ndarray) -> np.ndarray:
    return np.abs(y - ref).max(axis=1) / np.maximum(np.abs(ref).max(axis=1), 1e-30)


def run_forward(dl: DeviceLayer, x: torch.Tensor, ws: Workspace | None = None, prenorm=0, residual=0, y=None):
    """One lmoe_forward with all exports; returns device tensors."""
    s = dl.shape
    T = x.shape[0]
    dev = x.device
    out = dict(
        z=torch.empty((T, s.groups * s.latent), dtype=torch.float32, device=dev),
        ids=torch.empty((T, s.top_k), dtype=torch.int32, device=dev),
        w=torch.empty((T, s.top_k), dtype=torch.float32, device=dev),
        offsets=torch.empty((s.n_experts + 1,), dtype=torch.int32, device=dev),
        perm=torch.empty((max(1, T * s.top_k),), dtype=torch.int32, device=dev),
    )
    if y is None:
        dt = torch.float32 if (dl.act == "f32" or residual) else torch.int16
        y = torch.empty((T, s.hidden), dtype=dt, device=dev)
    opts = lm.make_opts(prenorm, residual, out["z"], out["ids"], out["w"], out["offsets"], out["perm"])
    ws = ws or Workspace(dev)
    buf = ws.get(lm.lmoe_workspace_bytes(dl.cfg, T))
    lm.check(lm.lmoe_forward(dl.cfg, dl.weights, x, T, y, opts, buf, buf.numel()))
    out["y"] = y
    return out


def check_routing(ids_gpu, ids_o, gap_o, logits_o, k):
    """Returns (same mask, excluded mask); asserts the rule above."""
    same = np.all(ids_gpu == ids_o, axis=1)
    excluded = gap_o < GAP
    bad = np.where(~same & ~excluded)[0]
    assert bad.size == 0, f"routing differs on {bad.size} tokens with gap >= {GAP}: first {bad[:5]}"
    for t in np.where(~same)[0]:
        kth = np.sort(logits_o[t])[::-1][k - 1]
        assert len(set(ids_gpu[t].tolist())) == k
        assert np.all(logits_o[t, ids_gpu[t]] >= kth - GAP), f"token {t}: a pick is not a near-tie"
    return same, excluded


def check_block(lw, x_host, act, out, sample=None, tol=None, label=""):
    """Compare one GPU forward (`out` from run_forward) with the oracle.  Routing and the
    permutation are checked on every token, outputs on `sample` (default: all tokens)."""
    s = lw.shape
    k = s.top_k
    tol = TOL[lw.expert if lw.expert in ("mxfp4", "nvfp4") else act] if tol is None else tol
    L = oracle.Layer(lw)
    xo = act_to_f64(x_host, act)
    T = xo.shape[0]
    z = xo @ L.D.T
    ids_o, w_o, gap_o, logits_o = oracle.route(z, L.Wr, L.br, k, s.groups)
    ids_g = host(out["ids"])
    same, excluded = check_routing(ids_g, ids_o, gap_o, logits_o, k)

    off_o, perm_o, _ = oracle.permute(ids_g, s.n_experts)
    assert np.array_equal(host(out["offsets"]), off_o), "offsets differ"
    assert np.array_equal(host(out["perm"])[: T * k], perm_o), "perm differs"

    w_g = host(out["w"])
    assert np.all(np.abs(w_g.sum(axis=1) - 1) < 1e-5)
    dw = np.abs(w_g[same] - w_o[same]).max() if same.any() else 0.0
    assert dw <= WTOL, f"routing weights differ by {dw}"
    zg = host(out["z"]).astype(np.float64)
    zrel = np.abs(zg - z).max() / np.abs(z).max()
    assert zrel < 1e-5, f"latent z rel err {zrel}"

    if sample is None:
        sample = np.arange(T)
    elif isinstance(sample, str) and sample.startswith("tiles:"):
        # every expert tile of the GPU's own work list, plus first, last, ragged and random tokens
        rows, n_extra = (int(v) for v in sample[len("tiles:"):].split(","))
        perm_g = host(out["perm"])[: T * k]
        toks, tiles = tile_cover_tokens(host(out["offsets"]), perm_g, T, k, s.n_experts, rows, s.shared_ffn > 0)
        sample = np.array(sorted(toks | set(sample_tokens(T, n_extra).tolist())))
        assert_tiles_covered(tiles, sample, perm_g, k, s.n_experts)
        log(f"[{label}] output sample covers all {len(tiles)} tiles of {rows} rows "
            f"({sum(1 for t in tiles if t[0] == s.n_experts)} shared) with {sample.size} tokens")
    sample = np.asarray(sample)
    forced = {i: ids_g[t] for i, t in enumerate(sample) if not same[t]}
    L.prefetch(np.concatenate([ids_o[sample].ravel(), ids_g[sample].ravel()]))
    ob = oracle.block_forward(L, xo[sample], forced_ids=forced)
    yg = host(out["y"])
    yg = act_to_f64(yg, act) if yg.dtype == np.uint16 or act == "f32" else yg.astype(np.float64)
    err = normwise_rel(yg[sample], ob["y"])
    log(f"[{label}] T={T} tokens checked={len(sample)} max_rel={err.max():.3e} mean_rel={err.mean():.3e} "
        f"excluded={int(excluded.sum())} differing={int((~same).sum())} dw={dw:.2e} zrel={zrel:.2e}")
    assert err.max() <= tol, f"output rel err {err.max()} > {tol} (token {sample[err.argmax()]})"
    return dict(max_rel=float(err.max()), excluded=int(excluded.sum()), differing=int((~same).sum()))


def tile_cover_tokens(offsets, perm, T, k, E, rows, has_shared=True):
    """Tokens whose outputs cover every `rows`-row tile of the expert work: for each expert
    segment [offsets[e], offsets[e+1]) cut into tiles of `rows` positions, the token of the tile's
    last position (so each segment's ragged last tile is included), and for the shared segment
    (all T tokens, in tiles of `rows` tokens) the last token of each tile.  Returns (tokens,
    tiles) with tiles = [(segment, first position, end position)] for the coverage check."""
    toks, tiles = set(), []
    offsets = np.asarray(offsets)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        for p0 in range(a, b, rows):
            p1 = min(p0 + rows, b)
            toks.add(int(perm[p1 - 1]) // k)
            tiles.append((e, p0, p1))
    if has_shared:
        for t0 in range(0, T, rows):
            t1 = min(t0 + rows, T)
            toks.add(t1 - 1)
            tiles.append((E, t0, t1))
    return toks, tiles


def assert_tiles_covered(tiles, sample, perm, k, E):
    """Every tile holds at least one position whose token is in the sample."""
    chosen = set(int(t) for t in sample)
    for seg, p0, p1 in tiles:
        rows = range(p0, p1) if seg == E else (int(perm[p]) // k for p in range(p0, p1))
        assert any(t in chosen for t in rows), f"tile of segment {seg} at {p0}..{p1} has no checked token"


def sample_tokens(T, n, seed=0):
    """First, last, a ragged run at the end and random interior tokens."""
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    fixed = np.array(sorted({0, 1, T - 1, T - 2, T // 2}))
    rest = rng.choice(np.setdiff1d(np.arange(T), fixed), size=n - fixed.size, replace=False)
    return np.sort(np.concatenate([fixed, rest]))


def upload_tokens(x_host, device="cuda"):
    return to_device(x_host, device)


def small_layer(shape, act, dense, expert, bias="zipf", wid=77, layer=0):
    wl = gen.Workload(wid, "small", shape, 0, act, dense, expert, bias)
    return wl, gen.make_layer(wl, layer)
