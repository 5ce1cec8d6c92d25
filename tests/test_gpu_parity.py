"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Covers the workloads at full size (routing and permutation on every token; outputs on every
token up to T=8, for the prefill workloads on tokens that cover every 128-row expert tile of the
GPU's own work list and every shared-expert tile), plus small shapes that exercise ragged
tiles, both kernel paths, MXFP4 and NVFP4 records, no shared expert, E == k and E == k == 1.
"""
import numpy as np
import pytest
import torch

import lmoe_data as gen
import oracle
import sparse_moe_proj_amd as lm
from parity import (check_block, host, log, run_forward, sample_tokens, small_layer, upload_tokens, TOL,
                    check_routing, normwise_rel, act_to_f64)
from sparse_moe_proj_amd.device import DeviceLayer, Workspace, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ws():
    return Workspace("cuda")


# rows of the large-batch expert tiles (the pipelined and the block-scaled GEMMs' 128-row tiles)
TILE_ROWS = 128


def _workload_case(name, n_sample, ws, tiles=False):
    """One workload's layer at full size.  tiles: the outputs are checked on tokens that cover every
    expert tile of the GPU's own work list (and every shared-expert tile) plus n_sample first,
    last, ragged and random tokens; otherwise on n_sample such tokens (all when T <= n_sample)."""
    wl = gen.WORKLOADS[name]
    log(f"[{name}] generating layer")
    lw = gen.make_layer(wl, 0)
    dl = DeviceLayer(lw, act=wl.act)
    x = gen.make_tokens(wl)
    out = run_forward(dl, upload_tokens(x), ws)
    torch.cuda.synchronize()
    sample = f"tiles:{TILE_ROWS},{n_sample}" if tiles else sample_tokens(wl.T, n_sample)
    return check_block(lw, x, wl.act, out, sample=sample, label=name)


def test_tiny_f32_full(ws):
    _workload_case("tiny_f32", 32, ws)


def test_decode_t8_full(ws):
    _workload_case("decode_t8", 8, ws)


@pytest.fixture(scope="module")
def layer120():
    wl = gen.WORKLOADS["decode120_t8"]
    log("[decode120_t8] generating layer")
    lw = gen.make_layer(wl, 0)
    return wl, lw, DeviceLayer(lw, act=wl.act)


@pytest.mark.parametrize("T", [8, 1, 3, 16, 33, 64])
def test_120b_verify_batches(T, ws, layer120):
    """The 120B latent width (1280) over a sweep of verify-batch sizes (both small-batch paths and
    the tile path); T = 8 is the workload's own batch."""
    wl, lw, dl = layer120
    x = gen.make_tokens(wl) if T == wl.T else gen.make_tokens(wl, T=T, salt=T)
    out = run_forward(dl, upload_tokens(x), ws)
    torch.cuda.synchronize()
    check_block(lw, x, wl.act, out, label=f"decode120 T={T}")


@pytest.mark.timeout(600)
def test_prefill_t4096_every_tile(ws):
    _workload_case("prefill_t4096", 96, ws, tiles=True)


@pytest.mark.timeout(900)
def test_prefill_t16384_every_tile(ws):
    _workload_case("prefill_t16384", 96, ws, tiles=True)


@pytest.mark.timeout(900)
def test_prefill_mxfp4_t16384_every_tile(ws):
    # MXFP4 records on the block-scaled MFMA (z and H each as MXFP8 plus an MXFP4 residual), the default
    # path for MXFP4 batches from 96 tokens
    _workload_case("prefill_mxfp4_t16384", 64, ws, tiles=True)


SMALL = gen.Shape(hidden=256, latent=192, n_experts=24, top_k=3, ffn=128, shared_ffn=64)


@pytest.mark.parametrize("T", [1, 5, 16, 17, 100, 300, 700, 1500, 2100, 3001])
def test_small_bf16_ragged(T, ws):
    """Both small-batch paths, the 16-row streaming tiles and the pipelined GEMMs on 128-row
    tiles and (from T k >= 256 E: T = 2100, 3001) on 256-row tiles, with ragged last tiles."""
    wl, lw = small_layer(SMALL, "bf16", "bf16", "bf16")
    dl = DeviceLayer(lw, act="bf16")
    x = gen.make_tokens(wl, T=T, salt=T)
    out = run_forward(dl, upload_tokens(x), ws)
    torch.cuda.synchronize()
    check_block(lw, x, "bf16", out, label=f"small_bf16 T={T}")


ROUTE_512 = gen.Shape(hidden=256, latent=128, n_experts=512, top_k=10, ffn=128, shared_ffn=128)


@pytest.mark.parametrize("expert", ["bf16", "mxfp4"])
@pytest.mark.parametrize("T", [8, 40])
def test_many_winners_in_one_lane_whole_block(T, expert, ws):
    """The routing inside the small-batch gate/up launch when one lane of the top-k wave holds 8
    of the 10 kept experts (ids 5 + 64 j), which takes the top-k's exact fallback: the router
    weights are zero, so every token's logits are the bias, built with those 8 experts and two
    others far above the rest (ties among the kept ones only)."""
    wl, lw = small_layer(ROUTE_512, "bf16", "bf16", expert)
    E = ROUTE_512.n_experts
    lw.Wr = np.zeros_like(lw.Wr)
    br = np.random.default_rng(5).uniform(-3.0, 0.0, E).astype(np.float32)
    br[[5 + 64 * j for j in range(8)]] = [14, 14, 13, 12, 12, 11, 10, 10]
    br[[6, 200]] = [9.5, 9.0]
    lw.br = br
    dl = DeviceLayer(lw, act="bf16")
    x = gen.make_tokens(wl, T=T, salt=T)
    out = run_forward(dl, upload_tokens(x), ws)
    torch.cuda.synchronize()
    want = sorted([5 + 64 * j for j in range(8)] + [6, 200])
    assert (host(out["ids"]) == np.array(want)[None, :]).all()
    check_block(lw, x, "bf16", out, label=f"one-lane winners {expert} T={T}")


@pytest.mark.parametrize("T", [1, 5, 16])
def test_small_bf16_router_unfolded(T, ws):
    """Small batches without the folded router take the z-based router launch."""
    wl, lw = small_layer(SMALL, "bf16", "bf16", "bf16")
    dl = DeviceLayer(lw, act="bf16", fold=False)
    assert dl.Gr is None
    x = gen.make_tokens(wl, T=T, salt=T)
    out = run_forward(dl, upload_tokens(x), ws)
    torch.cuda.synchronize()
    check_block(lw, x, "bf16", out, label=f"small_bf16 unfolded T={T}")


@pytest.mark.parametrize("fold", [True, False])
@pytest.mark.parametrize("T", [5, 40, 100])
def test_small_prenorm_residual(T, fold, ws):
    """Pre-RMSNorm input and fp32 residual update (the stack's layer form) on each D path: the
    normalisation formed while staging the D launch (T <= 16, or with the folded router up to
    64 tokens) or by its own launch (otherwise)."""
    wl, lw = small_layer(SMALL, "bf16", "bf16", "bf16")
    dl = DeviceLayer(lw, act="bf16", fold=fold)
    k = lw.shape.top_k
    h = gen.make_residual(wl, T=T).astype(np.float32)
    hbuf = to_device(h)
    out = run_forward(dl, hbuf, ws, prenorm=1, residual=1, y=hbuf)
    torch.cuda.synchronize()
    L = oracle.Layer(lw)
    xo = oracle.round_to_bf16(oracle.rmsnorm(h.astype(np.float64)))
    ids_o, _, gap_o, logits_o = oracle.route(xo @ L.D.T, L.Wr, L.br, k)
    ids_g = host(out["ids"])
    same, _ = check_routing(ids_g, ids_o, gap_o, logits_o, k)
    forced = {t: ids_g[t] for t in range(T) if not same[t]}
    o = oracle.block_forward(L, xo, forced_ids=forced)
    y_gpu = host(hbuf).astype(np.float64) - h.astype(np.float64)
    err = normwise_rel(y_gpu, o["y"]).max()
    log(f"[prenorm T={T} fold={fold}] rel={err:.3e} differing={int((~same).sum())}")
    assert err <= TOL["bf16"]


SMALL_G = gen.Shape(hidden=256, latent=192, n_experts=24, top_k=3, ffn=128, shared_ffn=64, groups=4)
SMALL_G_MX = gen.Shape(hidden=256, latent=256, n_experts=24, top_k=3, ffn=128, shared_ffn=128, groups=3)


@pytest.mark.parametrize("T", [1, 5, 16, 17, 64, 100, 300])
def test_small_expert_groups(T, ws):
    """Expert groups with their own D/U pair (small batches and every larger-batch path)."""
    wl, lw = small_layer(SMALL_G, "bf16", "bf16", "bf16")
    dl = DeviceLayer(lw, act="bf16")
    x = gen.make_tokens(wl, T=T, salt=T)
    out = run_forward(dl, upload_tokens(x), ws)
    torch.cuda.synchronize()
    check_block(lw, x, "bf16", out, label=f"small_groups T={T}")


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("T", [3, 40, 100])
def test_small_expert_groups_4bit(fmt, T, ws):
    wl, lw = small_layer(SMALL_G_MX, "bf16", "bf16", fmt)
    dl = DeviceLayer(lw, act="bf16")
    x = gen.make_tokens(wl, T=T, salt=T)
    out = run_forward(dl, upload_tokens(x), ws)
    torch.cuda.synchronize()
    check_block(lw, x, "bf16", out, label=f"small_groups_{fmt} T={T}")


def test_expert_groups_need_the_folded_router(ws):
    wl, lw = small_layer(SMALL_G, "bf16", "bf16", "bf16")
    dl = DeviceLayer(lw, act="bf16", fold=False)
    x = upload_tokens(gen.make_tokens(wl, T=4))
    buf = ws.get(lm.lmoe_workspace_bytes(dl.cfg, 4))
    y = torch.empty((4, wl.shape.hidden), dtype=torch.int16, device="cuda")
    assert lm.lmoe_forward(dl.cfg, dl.weights, x, 4, y, None, buf, buf.numel()) == lm.LMOE_ERR_UNSUPPORTED


def test_decode_group64_t8_full(ws):
    _workload_case("decode_group64_t8", 8, ws)


def test_fold_router_halves():
    """hi + lo of the folded router carries G = Wr . D to the precision the halves allow."""
    wl, lw = small_layer(SMALL, "bf16", "bf16", "bf16")
    dl = DeviceLayer(lw, act="bf16")
    E, H = SMALL.n_experts, SMALL.hidden
    gr = dl.Gr.cpu().numpy().view(np.uint16).reshape(E, 2, H)
    hi, lo = act_to_f64(gr[:, 0], "bf16"), act_to_f64(gr[:, 1], "bf16")
    Wr, D = act_to_f64(lw.Wr, "bf16"), act_to_f64(lw.D, "bf16")
    G = Wr @ D                                  # [E][H], exact in fp64 for these sizes
    bound = np.abs(Wr) @ np.abs(D)              # fp32 accumulation error scale
    err = np.abs(hi + lo - G)
    assert np.all(err <= 2.0 ** -16 * np.abs(G) + SMALL.latent * 2.0 ** -24 * bound + 1e-30), err.max()
    # hi is the bf16 rounding of the fp32 sum: never further than one bf16 half-ulp plus that error
    assert np.all(np.abs(hi - G) <= 2.0 ** -8 * np.abs(G) + SMALL.latent * 2.0 ** -24 * bound + 1e-30)


SMALL_MX = gen.Shape(hidden=256, latent=256, n_experts=24, top_k=3, ffn=128, shared_ffn=128)


@pytest.mark.parametrize("T", [3, 16, 40, 80, 100, 383, 400, 1100])
def test_small_mxfp4(T, ws):
    wl, lw = small_layer(SMALL_MX, "bf16", "bf16", "mxfp4")
    dl = DeviceLayer(lw, act="bf16")
    x = gen.make_tokens(wl, T=T, salt=T)
    out = run_forward(dl, upload_tokens(x), ws)
    torch.cuda.synchronize()
    check_block(lw, x, "bf16", out, label=f"small_mxfp4 T={T}")


SMALL_MX_NOSH = gen.Shape(hidden=256, latent=384, n_experts=24, top_k=3, ffn=256, shared_ffn=0)


@pytest.mark.parametrize("path", ["mx_mfma", "decode_bf16"])
@pytest.mark.parametrize("shape,T", [("mx", 96), ("mx", 300), ("mx", 384), ("mx", 700), ("mx_nosh", 200),
                                     ("mx_nosh", 512), ("mx_nosh", 1500), ("groups", 150), ("groups", 400),
                                     ("groups", 900)])
def test_large_mxfp4_paths(path, shape, T, ws):
    """MXFP4 batches past the small-batch kernels: the block-scaled MFMA kernels (MXFP8
    activations, from 96 tokens) and, with them switched off (lmoe_config.mx_mfma_min_t = -1), the
    weight-streaming kernels below 384 tokens and the decode of the records to bf16 from 384; with
    and without a shared expert, and with expert groups."""
    sh = {"mx": SMALL_MX, "mx_nosh": SMALL_MX_NOSH, "groups": SMALL_G_MX}[shape]
    wl, lw = small_layer(sh, "bf16", "bf16", "mxfp4")
    dl = DeviceLayer(lw, act="bf16", mx_mfma_min_t=0 if path == "mx_mfma" else -1)
    x = gen.make_tokens(wl, T=T, salt=T + 7)
    out = run_forward(dl, upload_tokens(x), ws)
    torch.cuda.synchronize()
    check_block(lw, x, "bf16", out, label=f"large_mxfp4 {path} {shape} T={T}")


MX_NOSH_4K = gen.Shape(hidden=1024, latent=1024, n_experts=64, top_k=8, ffn=512, shared_ffn=0)


@pytest.mark.timeout(600)
def test_mxfp4_no_shared_every_token_t4096(ws):
    """The default MXFP4 path for large batches (block-scaled MFMA, z and H each as MXFP8 plus an
    MXFP4 residual) on a shape without a shared expert, where no exact bf16 term dilutes the
    activation rounding: every one of 4096 tokens against the oracle."""
    wl = gen.Workload(93, "mx_nosh_t4096", MX_NOSH_4K, 4096, "bf16", "bf16", "mxfp4", "zipf")
    lw = gen.make_layer(wl, 0)
    dl = DeviceLayer(lw, act="bf16")
    x = gen.make_tokens(wl)
    out = run_forward(dl, upload_tokens(x), ws)
    torch.cuda.synchronize()
    check_block(lw, x, "bf16", out, label="mxfp4 no shared expert T=4096")


@pytest.mark.parametrize("T", [3, 16, 40, 100, 383, 400, 1100])
def test_small_nvfp4(T, ws):
    wl, lw = small_layer(SMALL_MX, "bf16", "bf16", "nvfp4")
    dl = DeviceLayer(lw, act="bf16")
    x = gen.make_tokens(wl, T=T, salt=T)
    out = run_forward(dl, upload_tokens(x), ws)
    torch.cuda.synchronize()
    check_block(lw, x, "bf16", out, label=f"small_nvfp4 T={T}")


def test_decode_nvfp4_t8_full(ws):
    _workload_case("decode_nvfp4_t8", 8, ws)


def _scale_bf16(x, s):
    """bf16 bits x times the power of two s (exact: only the exponents change)."""
    f = (x.astype(np.uint32) << 16).view(np.float32) * np.float32(s)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def _routed_swiglu_max(lw, x):
    """Largest |SiLU(z G_e) * (z V_e)| over every token's routed experts (oracle, float64): the
    magnitudes the 4-bit small-batch path holds in fp16."""
    L = oracle.Layer(lw)
    z = oracle.decode(x, "bf16") @ L.D.T
    ids = oracle.route(z, L.Wr, L.br, lw.shape.top_k, lw.shape.groups)[0]
    m = 0.0
    for t in range(z.shape[0]):
        for e in ids[t]:
            g, u, _ = L.expert(int(e))
            with np.errstate(over="ignore"):  # exp(-v) of a large negative gate: SiLU is -0 there
                m = max(m, float(np.abs(oracle.silu(z[t] @ g.T) * (z[t] @ u.T)).max()))
    return m


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_small_4bit_large_activations(fmt, ws):
    """Tokens 32 times larger: z and SiLU(g) * u run to thousands, still inside fp16, which the
    4-bit small-batch path carries them in; outputs within the 4-bit tolerance."""
    wl, lw = small_layer(SMALL_MX, "bf16", "bf16", fmt)
    x = _scale_bf16(gen.make_tokens(wl, T=8, salt=5), 32.0)
    m = _routed_swiglu_max(lw, x)
    assert 1e3 < m < 65504, m
    out = run_forward(DeviceLayer(lw, act="bf16"), upload_tokens(x), ws)
    torch.cuda.synchronize()
    check_block(lw, x, "bf16", out, label=f"small_{fmt} tokens x32 (max |SiLU(g) u| {m:.0f})")


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_small_4bit_fp16_saturation_stays_finite(fmt, ws):
    """Tokens 8192 times larger: SiLU(g) * u of the routed experts exceeds fp16's 65504, and the
    4-bit small-batch path saturates it instead of overflowing, so every output stays finite (the
    values lose their size there and are not compared)."""
    wl, lw = small_layer(SMALL_MX, "bf16", "bf16", fmt)
    x = _scale_bf16(gen.make_tokens(wl, T=8, salt=5), 8192.0)
    m = _routed_swiglu_max(lw, x)
    assert m > 65504, m
    out = run_forward(DeviceLayer(lw, act="bf16"), upload_tokens(x), ws)
    torch.cuda.synchronize()
    y = oracle.decode(host(out["y"]), "bf16")
    log(f"[small_{fmt} tokens x8192] max |SiLU(g) u| {m:.3e}, max |y| {np.abs(y).max():.3e}")
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("T", [7, 70])
def test_small_f32(T, ws):
    wl, lw = small_layer(SMALL, "f32", "f32", "f32")
    dl = DeviceLayer(lw, act="f32")
    x = gen.make_tokens(wl, T=T, salt=T)
    out = run_forward(dl, upload_tokens(x), ws)
    torch.cuda.synchronize()
    check_block(lw, x, "f32", out, label=f"small_f32 T={T}")


@pytest.mark.parametrize("shape_kw,T", [
    (dict(shared_ffn=0), 9),                       # no shared expert
    (dict(shared_ffn=0), 130),
    (dict(n_experts=4, top_k=4), 11),              # every expert used
    (dict(n_experts=4, top_k=4), 70),
    (dict(n_experts=1, top_k=1, shared_ffn=0), 5),  # dense SwiGLU
    (dict(n_experts=1, top_k=1, shared_ffn=0), 200),
    (dict(top_k=16, n_experts=20), 33),            # largest k
    (dict(ffn=64, shared_ffn=128), 24),            # shared wider than routed
])
def test_degenerate_shapes(shape_kw, T, ws):
    base = dict(hidden=128, latent=128, n_experts=12, top_k=2, ffn=128, shared_ffn=64)
    base.update(shape_kw)
    shape = gen.Shape(**base)
    wl, lw = small_layer(shape, "bf16", "bf16", "bf16", wid=78)
    dl = DeviceLayer(lw, act="bf16")
    x = gen.make_tokens(wl, T=T, salt=T)
    out = run_forward(dl, upload_tokens(x), ws)
    torch.cuda.synchronize()
    check_block(lw, x, "bf16", out, label=f"degenerate {shape_kw} T={T}")


def test_identical_experts_output_independent_of_routing(ws):
    shape = gen.Shape(hidden=128, latent=128, n_experts=16, top_k=4, ffn=64, shared_ffn=64)
    wl, lw = small_layer(shape, "bf16", "bf16", "bf16", wid=79)
    lw.experts[:] = lw.experts[0]
    x = gen.make_tokens(wl, T=12)
    xt = upload_tokens(x)
    dl = DeviceLayer(lw, act="bf16")
    a = run_forward(dl, xt, ws)
    lw.br = np.linspace(4, -4, 16).astype(np.float32)
    dl2 = DeviceLayer(lw, act="bf16")
    b = run_forward(dl2, xt, ws)
    torch.cuda.synchronize()
    assert not np.array_equal(host(a["ids"]), host(b["ids"]))
    ya = act_to_f64(host(a["y"]), "bf16")
    yb = act_to_f64(host(b["y"]), "bf16")
    assert normwise_rel(yb, ya).max() < 1e-2


def test_determinism_and_batch_invariance(ws):
    wl = gen.WORKLOADS["decode_t8"]
    for T, sub in ((8, 3), (300, 120)):
        wl2, lw = small_layer(SMALL, "bf16", "bf16", "bf16", wid=80)
        dl = DeviceLayer(lw, act="bf16")
        x = gen.make_tokens(wl2, T=T, salt=1)
        xt = upload_tokens(x)
        a = run_forward(dl, xt, ws)
        b = run_forward(dl, xt, ws)
        torch.cuda.synchronize()
        for key in ("y", "z", "ids", "w", "offsets", "perm"):
            assert torch.equal(a[key], b[key]), f"run-to-run difference in {key} (T={T})"
        # the first `sub` tokens alone (same kernel path) give bitwise the same rows
        if sub > 16 or T <= 16:
            c = run_forward(dl, xt[:sub].contiguous(), ws)
            torch.cuda.synchronize()
            assert torch.equal(c["y"], a["y"][:sub]), f"batch invariance (T={T}, sub={sub})"
        # permuting tokens permutes outputs bitwise
        p = torch.randperm(T, generator=torch.Generator().manual_seed(0)).cuda()
        d = run_forward(dl, xt[p].contiguous(), ws)
        torch.cuda.synchronize()
        assert torch.equal(d["y"], a["y"][p]), f"token permutation (T={T})"


@pytest.mark.parametrize("case", ["groups_t8", "groups_t300", "mxfp4_t1100", "nvfp4_t500"])
def test_determinism_other_paths(case, ws):
    """Run-to-run bitwise equality and token-permutation equivariance on the expert-group paths
    and the large 4-bit batch path (records decoded once to bf16)."""
    shape, fmt, T = {"groups_t8": (SMALL_G, "bf16", 8), "groups_t300": (SMALL_G, "bf16", 300),
                     "mxfp4_t1100": (SMALL_MX, "mxfp4", 1100), "nvfp4_t500": (SMALL_MX, "nvfp4", 500)}[case]
    wl, lw = small_layer(shape, "bf16", "bf16", fmt, wid=81)
    dl = DeviceLayer(lw, act="bf16")
    xt = upload_tokens(gen.make_tokens(wl, T=T, salt=2))
    a = run_forward(dl, xt, ws)
    b = run_forward(dl, xt, ws)
    torch.cuda.synchronize()
    for key in ("y", "z", "ids", "w", "offsets", "perm"):
        assert torch.equal(a[key], b[key]), f"run-to-run difference in {key} ({case})"
    p = torch.randperm(T, generator=torch.Generator().manual_seed(1)).cuda()
    d = run_forward(dl, xt[p].contiguous(), ws)
    torch.cuda.synchronize()
    assert torch.equal(d["y"], a["y"][p]), f"token permutation ({case})"


def test_zero_tokens_noop(ws):
    wl, lw = small_layer(SMALL, "bf16", "bf16", "bf16")
    dl = DeviceLayer(lw, act="bf16")
    y = torch.full((4, SMALL.hidden), 7, dtype=torch.int16, device="cuda")
    x = torch.zeros((4, SMALL.hidden), dtype=torch.int16, device="cuda")
    buf = ws.get(1 << 20)
    assert lm.lmoe_forward(dl.cfg, dl.weights, x, 0, y, None, buf, buf.numel()) == lm.LMOE_OK
    torch.cuda.synchronize()
    assert torch.all(y == 7)
