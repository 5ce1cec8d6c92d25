"""lmoe_route and lmoe_permute on their own, through the C ABI, against the oracle."""
import numpy as np
import pytest
import torch

import lmoe_data as gen
import oracle
import sparse_moe_proj_amd as lm
from parity import GAP, WTOL, check_routing, host, log
from sparse_moe_proj_amd.device import DeviceLayer, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T", [1, 8, 16, 17, 333, 4096])
def test_route_isolated(T):
    """z comes from the oracle (float64 -> float32); the router must reproduce the oracle's
    top-k on the float32 values exactly (up to near-ties) and its weights."""
    wl = gen.WORKLOADS["decode_t8"]
    # routing reads only D (to form z here), Wr and br: the expert records are placeholders
    lw = gen.make_layer(wl, 0, experts=np.zeros((wl.shape.n_experts, 8), dtype=np.uint16))
    L = oracle.Layer(lw)
    x = oracle.decode(gen.make_tokens(wl, T=T, salt=T), "bf16")
    z32 = (x @ L.D.T).astype(np.float32)
    ids_o, w_o, gap_o, logits_o = oracle.route(z32.astype(np.float64), L.Wr, L.br, lw.shape.top_k)
    dl = DeviceLayer(lw, act="bf16", pack=False)
    k = lw.shape.top_k
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ws = torch.empty(T * lw.shape.n_experts * 4, dtype=torch.uint8, device="cuda")
    lm.check(lm.lmoe_route(dl.cfg, dl.weights, to_device(z32), T, ids, w, ws, ws.numel()))
    torch.cuda.synchronize()
    ids_g, w_g = host(ids), host(w)
    same, excl = check_routing(ids_g, ids_o, gap_o, logits_o, k)
    assert np.all(np.diff(ids_g, axis=1) > 0)
    assert np.abs(w_g[same] - w_o[same]).max() <= WTOL
    assert np.all(np.abs(w_g.sum(axis=1) - 1) < 1e-5)
    log(f"[route T={T}] excluded={int(excl.sum())} differing={int((~same).sum())}")


def test_route_exact_ties_pick_lower_id():
    """Logits with exact ties: Wr = identity block so logits equal z exactly in fp32."""
    E, k, L = 64, 4, 64
    shape = gen.Shape(hidden=64, latent=L, n_experts=E, top_k=k, ffn=64, shared_ffn=0)
    cfg = lm.make_config(shape.hidden, L, E, k, 64, 0, "bf16", "bf16", "bf16")
    Wr = np.eye(E, L, dtype=np.float32)
    Wr_bits = gen.bf16_bits(Wr.copy())
    rng = np.random.default_rng(3)
    T = 50
    z = rng.integers(-2, 3, size=(T, L)).astype(np.float32)
    Wr_d = to_device(Wr_bits)
    weights = lm.make_weights(None, None, Wr_d, None, None, None)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ws = torch.empty(T * E * 4, dtype=torch.uint8, device="cuda")
    lm.check(lm.lmoe_route(cfg, weights, to_device(z), T, ids, w, ws, ws.numel()))
    torch.cuda.synchronize()
    for t in range(T):
        want = sorted(sorted(range(E), key=lambda e: (-z[t, e], e))[:k])
        assert host(ids)[t].tolist() == want


@pytest.mark.parametrize("T", [50, 100])
@pytest.mark.parametrize("k", [10, 16])
def test_route_many_winners_in_one_lane(T, k):
    """The wave top-k races each lane's leading keys and falls back to the whole sorted run when
    one lane (ids e = c mod 64 share lane c) holds several of the winners: tokens whose top k put
    3, 4, 5 or 8 of the kept experts in one lane, with exact ties inside that lane and across
    lanes (Wr = identity, so the logits equal the integer-valued z exactly)."""
    E = L = 512
    shape = gen.Shape(hidden=64, latent=L, n_experts=E, top_k=k, ffn=64, shared_ffn=0)
    cfg = lm.make_config(shape.hidden, L, E, k, 64, 0, "bf16", "bf16", "bf16")
    Wr_bits = gen.bf16_bits(np.eye(E, L, dtype=np.float32))
    rng = np.random.default_rng(11 + T + k)
    z = rng.integers(-4, 4, size=(T, L)).astype(np.float32)
    for t in range(T):
        c, n_lane = t % 64, (3, 4, 5, 8)[t % 4]
        for j in range(n_lane):                   # n_lane high values in lane c, some equal
            z[t, c + 64 * j] = 20 + (j // 2)
        z[t, (c + 1) % 64] = 20                   # ties with the lane's lowest high values
        z[t, (c + 7) % 64 + 64] = 21
    Wr_d, z_d = to_device(Wr_bits), to_device(z)
    weights = lm.make_weights(None, None, Wr_d, None, None, None)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ws = torch.empty(T * E * 4, dtype=torch.uint8, device="cuda")
    lm.check(lm.lmoe_route(cfg, weights, z_d, T, ids, w, ws, ws.numel()))
    torch.cuda.synchronize()
    got = host(ids)
    for t in range(T):
        want = sorted(sorted(range(E), key=lambda e: (-z[t, e], e))[:k])
        assert got[t].tolist() == want, (t, got[t].tolist(), want)


@pytest.mark.parametrize("T,E,k,skew", [(1, 512, 10, 0.0), (8, 512, 10, 1.1), (64, 512, 10, 0.0), (65, 512, 10, 1.1),
                                        (1000, 16, 2, 0.0), (4096, 512, 10, 1.1), (16384, 512, 10, 1.1),
                                        (300, 1024, 16, 0.5), (77, 5, 5, 0.0)])
def test_permute_matches_stable_sort(T, E, k, skew):
    ids = gen.random_ids(T, E, k, seed=T + E, skew=skew)
    cfg = lm.make_config(256, 128, E, k, 64, 0, "bf16", "bf16", "bf16")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
    nb = lm.lmoe_permute_workspace_bytes(cfg, T)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
    lm.check(lm.lmoe_permute(cfg, to_device(ids), T, off, perm, inv, ws, nb))
    torch.cuda.synchronize()
    o, p, i = oracle.permute(ids, E)
    assert np.array_equal(host(off), o)
    assert np.array_equal(host(perm), p)
    assert np.array_equal(host(inv), i)


def test_permute_drops_invalid_ids():
    T, E, k = 100, 32, 3
    ids = gen.random_ids(T, E, k, seed=5)
    ids[3, 1] = -1
    ids[50, 0] = E
    ids[99, 2] = 10 ** 6
    cfg = lm.make_config(256, 128, E, k, 64, 0, "bf16", "bf16", "bf16")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
    nb = lm.lmoe_permute_workspace_bytes(cfg, T)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
    lm.check(lm.lmoe_permute(cfg, to_device(ids), T, off, perm, inv, ws, nb))
    torch.cuda.synchronize()
    flat = ids.ravel()
    valid = (flat >= 0) & (flat < E)
    want = sorted(np.where(valid)[0].tolist(), key=lambda f: (flat[f], f))
    n = len(want)
    assert host(off)[E] == n
    assert host(perm)[:n].tolist() == want
    assert np.all(host(perm)[n:] == -1)
    inv_h = host(inv)
    assert np.all(inv_h[~valid] == -1)
    assert [inv_h[f] for f in want] == list(range(n))
