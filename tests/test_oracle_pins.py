"""Pins for the CPU oracle, independent of the oracle's own code paths.

Each check pins the oracle to something other than itself: brute force on tiny inputs in
pure Python (math.exp, sorted), closed forms, invariants the block's definition fixes, special
cases that reduce to a textbook dense SwiGLU or a standard MoE, and library routines (torch)
for the element formats.  Together they are chosen so that a dropped term, a wrong sign or
index, or a transposed operand anywhere in the oracle fails at least one of them.
"""
import bisect
import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import lmoe_data as gen
import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def make_f32_layer(shape, seed, shared=True, same_experts=False, br=None):
    rng = np.random.default_rng(seed)
    H, L, E, F, G = shape.hidden, shape.latent, shape.n_experts, shape.ffn, shape.groups

    def mat(r, c, fan):
        return (rng.standard_normal((r, c)) / math.sqrt(fan)).astype(np.float32)

    D, U, Wr = mat(G * L, H, H), mat(H, G * L, L), mat(E, L, L)
    if br is None:
        br = (0.3 * rng.standard_normal(E)).astype(np.float32)

    def rec(f):
        return np.concatenate([mat(f, L, L).ravel(), mat(f, L, L).ravel(), mat(L, f, f).ravel()])

    sh = rec(shape.shared_ffn) if (shared and shape.shared_ffn) else None
    if same_experts:
        r0 = rec(F)
        ex = np.stack([r0] * E)
    else:
        ex = np.stack([rec(F) for _ in range(E)])
    return gen.LayerWeights(shape, "f32", "f32", D, U, Wr, np.asarray(br, np.float32), sh, ex)


def py_silu(v):
    return v / (1.0 + math.exp(-v))


def brute_forward(lw, x, forced=None, details=False):
    """Scalar-loop latent-MoE block in pure Python floats.  With expert groups, expert e is in
    group e // (E / G), which owns D rows and U columns g*L .. g*L + L - 1; the shared expert
    is in group 0.  forced maps a token row to the experts it must use instead of its top k (in
    any order; the weights are then the full softmax renormalised over those experts).  With
    details, returns (y, ids, w) with each token's experts in ascending id."""
    s = lw.shape
    H, L, E, k, F, G = s.hidden, s.latent, s.n_experts, s.top_k, s.ffn, s.groups
    Eg = E // G
    D = lw.D.astype(float).tolist()
    U = lw.U.astype(float).tolist()
    Wr = lw.Wr.astype(float).tolist()
    br = lw.br.astype(float).tolist()

    def split(rec, f):
        rec = rec.astype(float)
        g = rec[: f * L].reshape(f, L).tolist()
        u = rec[f * L: 2 * f * L].reshape(f, L).tolist()
        d = rec[2 * f * L:].reshape(L, f).tolist()
        return g, u, d

    def expert_out(zt, gud, f):
        g, u, d = gud
        h = []
        for j in range(f):
            a = sum(zt[i] * g[j][i] for i in range(L))
            b = sum(zt[i] * u[j][i] for i in range(L))
            h.append(py_silu(a) * b)
        return [sum(h[j] * d[r][j] for j in range(f)) for r in range(L)]

    out, all_ids, all_w = [], [], []
    for t, xt in enumerate(x.astype(float).tolist()):
        zg = [[sum(xt[i] * D[g * L + j][i] for i in range(H)) for j in range(L)] for g in range(G)]
        lam = [sum(zg[e // Eg][i] * Wr[e][i] for i in range(L)) + br[e] for e in range(E)]
        top = sorted(range(E), key=lambda e: (-lam[e], e))[:k]
        if forced and t in forced:
            top = [int(e) for e in forced[t]]
        # full softmax over all experts, then renormalise over the kept ones
        mx = max(lam)
        p = [math.exp(v - mx) for v in lam]
        z_all = sum(p)
        p = [v / z_all for v in p]
        norm = sum(p[e] for e in top)
        m = [[0.0] * L for _ in range(G)]
        if lw.shared is not None:
            so = expert_out(zg[0], split(lw.shared, s.shared_ffn), s.shared_ffn)
            m[0] = [a + b for a, b in zip(m[0], so)]
        for e in sorted(top):
            g = e // Eg
            yo = expert_out(zg[g], split(lw.experts[e], F), F)
            wgt = p[e] / norm
            m[g] = [a + wgt * b for a, b in zip(m[g], yo)]
        out.append([sum(m[g][i] * U[r][g * L + i] for g in range(G) for i in range(L)) for r in range(H)])
        all_ids.append(sorted(top))
        all_w.append([p[e] / norm for e in sorted(top)])
    if details:
        return np.array(out), np.array(all_ids), np.array(all_w)
    return np.array(out)


SMALL = gen.Shape(hidden=6, latent=4, n_experts=5, top_k=2, ffn=3, shared_ffn=3)


def test_forward_matches_scalar_brute_force():
    lw = make_f32_layer(SMALL, 1)
    x = np.random.default_rng(2).standard_normal((3, SMALL.hidden)).astype(np.float32)
    got = oracle.block_forward(oracle.Layer(lw), x.astype(np.float64))["y"]
    want = brute_forward(lw, x)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_forward_brute_force_no_shared_rect_shapes():
    s = gen.Shape(hidden=5, latent=7, n_experts=6, top_k=3, ffn=2, shared_ffn=0)
    lw = make_f32_layer(s, 3, shared=False)
    x = np.random.default_rng(4).standard_normal((4, s.hidden)).astype(np.float32)
    got = oracle.block_forward(oracle.Layer(lw), x.astype(np.float64))["y"]
    np.testing.assert_allclose(got, brute_forward(lw, x), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("G", [2, 3])
def test_grouped_forward_matches_scalar_brute_force(G):
    # the launch blog's form: every group of experts owns its own D/U pair
    s = gen.Shape(hidden=6, latent=4, n_experts=3 * G, top_k=3, ffn=3, shared_ffn=2, groups=G)
    lw = make_f32_layer(s, 11 + G)
    x = np.random.default_rng(12).standard_normal((4, s.hidden)).astype(np.float32)
    got = oracle.block_forward(oracle.Layer(lw), x.astype(np.float64))["y"]
    np.testing.assert_allclose(got, brute_forward(lw, x), rtol=1e-12, atol=1e-13)


def test_grouped_with_tied_pairs_equals_one_pair():
    # every group holding the same D and U: y = sum_g U m_g = U sum_g m_g, the one-pair block
    G = 4
    s1 = gen.Shape(hidden=8, latent=6, n_experts=8, top_k=3, ffn=4, shared_ffn=4)
    lw1 = make_f32_layer(s1, 21)
    sg = gen.Shape(hidden=8, latent=6, n_experts=8, top_k=3, ffn=4, shared_ffn=4, groups=G)
    lwg = gen.LayerWeights(sg, "f32", "f32", np.concatenate([lw1.D] * G, axis=0), np.concatenate([lw1.U] * G, axis=1),
                           lw1.Wr, lw1.br, lw1.shared, lw1.experts)
    x = np.random.default_rng(22).standard_normal((5, 8))
    a = oracle.block_forward(oracle.Layer(lw1), x)
    b = oracle.block_forward(oracle.Layer(lwg), x)
    assert np.array_equal(a["ids"], b["ids"])
    np.testing.assert_allclose(b["y"], a["y"], rtol=1e-12, atol=1e-13)


def test_group_locality():
    # tokens routed only inside group 1 (no shared expert) depend on U's group-1 columns alone
    G, L = 3, 5
    s = gen.Shape(hidden=7, latent=L, n_experts=6, top_k=2, ffn=3, shared_ffn=0, groups=G)
    br = np.zeros(6, np.float32)
    br[2:4] = 50.0  # experts 2, 3 = group 1
    lw = make_f32_layer(s, 31, shared=False, br=br)
    x = np.random.default_rng(32).standard_normal((4, 7))
    y = oracle.block_forward(oracle.Layer(lw), x)
    assert np.all(y["ids"] == [2, 3])
    U2 = lw.U.copy()
    U2[:, :L] = 0
    U2[:, 2 * L:] = 0
    y2 = oracle.block_forward(oracle.Layer(gen.LayerWeights(s, "f32", "f32", lw.D, U2, lw.Wr, lw.br, None, lw.experts)), x)
    np.testing.assert_array_equal(y2["y"], y["y"])
    U3 = lw.U.copy()
    U3[:, L:2 * L] = 0
    y3 = oracle.block_forward(oracle.Layer(gen.LayerWeights(s, "f32", "f32", lw.D, U3, lw.Wr, lw.br, None, lw.experts)), x)
    assert np.all(y3["y"] == 0)


def test_topk_bruteforce_with_exact_ties():
    # Wr = I and br = 0 make the logits equal z, so the selection can be driven directly.
    E, k, T = 12, 4, 40
    rng = np.random.default_rng(5)
    z = rng.integers(-3, 4, size=(T, E)).astype(np.float64)  # many exact ties
    ids, w, gap, _ = oracle.route(z, np.eye(E), np.zeros(E), k)
    for t in range(T):
        lam = z[t].tolist()
        order = sorted(range(E), key=lambda e: (-lam[e], e))
        assert ids[t].tolist() == sorted(order[:k])
        assert gap[t] == lam[order[k - 1]] - lam[order[k]]
        mx = max(lam[e] for e in order[:k])
        den = sum(math.exp(lam[e] - mx) for e in order[:k])
        for j, e in enumerate(ids[t]):
            assert abs(w[t, j] - math.exp(lam[e] - mx) / den) < 1e-15


def test_weights_equal_full_softmax_renormalised_and_sum_to_one():
    rng = np.random.default_rng(6)
    E, k = 64, 10
    lam = rng.standard_normal((20, E)) * 3
    ids, w, _, _ = oracle.route(lam, np.eye(E), np.zeros(E), k)
    p = torch.softmax(torch.tensor(lam), dim=1).numpy()
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-13)
    assert np.all(np.abs(w.sum(axis=1) - 1) < 1e-12)
    assert np.all(np.diff(ids, axis=1) > 0)  # ascending expert id


def test_bias_enters_selection_and_weights():
    E, k = 8, 2
    z = np.zeros((1, E))
    br = np.array([0, 0, 0, 5.0, 0, 4.0, 0, 0])
    ids, w, _, _ = oracle.route(z, np.eye(E), br, k)
    assert ids[0].tolist() == [3, 5]
    np.testing.assert_allclose(w[0], [math.exp(1) / (1 + math.exp(1)), 1 / (1 + math.exp(1))], rtol=1e-14)


def test_permutation_matches_python_stable_sort():
    T, E, k = 50, 9, 3
    ids = gen.random_ids(T, E, k, seed=3, skew=1.0)
    offsets, perm, inv = oracle.permute(ids, E)
    flat = ids.reshape(-1).tolist()
    want = sorted(range(T * k), key=lambda f: (flat[f], f))
    assert perm.tolist() == want
    assert [inv[f] for f in want] == list(range(T * k))
    counts = [flat.count(e) for e in range(E)]
    acc = [0]
    for c in counts:
        acc.append(acc[-1] + c)
    assert offsets.tolist() == acc
    for e in range(E):  # every segment holds only expert e
        assert all(flat[f] == e for f in perm[offsets[e]:offsets[e + 1]])


def test_identical_experts_make_output_independent_of_routing():
    s = gen.Shape(hidden=16, latent=12, n_experts=8, top_k=3, ffn=5, shared_ffn=5)
    x = np.random.default_rng(7).standard_normal((6, s.hidden))
    lw1 = make_f32_layer(s, 8, same_experts=True, br=np.zeros(8))
    lw2 = make_f32_layer(s, 8, same_experts=True, br=np.linspace(3, -3, 8))
    a = oracle.block_forward(oracle.Layer(lw1), x)
    b = oracle.block_forward(oracle.Layer(lw2), x)
    assert not np.array_equal(a["ids"], b["ids"])  # the bias really changed the routing
    np.testing.assert_allclose(a["y"], b["y"], rtol=1e-12, atol=1e-12)


def test_top1_of_one_expert_is_dense_swiglu():
    s = gen.Shape(hidden=10, latent=6, n_experts=1, top_k=1, ffn=4, shared_ffn=0)
    lw = make_f32_layer(s, 9, shared=False)
    x = np.random.default_rng(10).standard_normal((5, s.hidden))
    got = oracle.block_forward(oracle.Layer(lw), x)["y"]
    X = torch.tensor(x)
    D, U = torch.tensor(lw.D, dtype=torch.float64), torch.tensor(lw.U, dtype=torch.float64)
    r = torch.tensor(lw.experts[0], dtype=torch.float64)
    F, L = 4, 6
    G, V, O = r[:F * L].view(F, L), r[F * L:2 * F * L].view(F, L), r[2 * F * L:].view(L, F)
    z = torch.nn.functional.linear(X, D)
    h = torch.nn.functional.silu(torch.nn.functional.linear(z, G)) * torch.nn.functional.linear(z, V)
    want = torch.nn.functional.linear(torch.nn.functional.linear(h, O), U).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_identity_projections_reduce_to_standard_moe():
    s = gen.Shape(hidden=8, latent=8, n_experts=6, top_k=2, ffn=5, shared_ffn=0)
    lw = make_f32_layer(s, 11, shared=False)
    lw.D = np.eye(8, dtype=np.float32)
    lw.U = np.eye(8, dtype=np.float32)
    x = np.random.default_rng(12).standard_normal((7, 8))
    got = oracle.block_forward(oracle.Layer(lw), x)["y"]
    # standard (non-latent) top-k MoE on x directly, written with torch
    X = torch.tensor(x)
    logits = X @ torch.tensor(lw.Wr, dtype=torch.float64).T + torch.tensor(lw.br, dtype=torch.float64)
    val, idx = torch.topk(logits, 2, dim=1)
    gates = torch.softmax(val, dim=1)
    want = torch.zeros_like(X)
    for t in range(7):
        for j in range(2):
            r = torch.tensor(lw.experts[int(idx[t, j])], dtype=torch.float64)
            G, V, O = r[:40].view(5, 8), r[40:80].view(5, 8), r[80:].view(8, 5)
            hh = torch.nn.functional.silu(X[t] @ G.T) * (X[t] @ V.T)
            want[t] += gates[t, j] * (hh @ O.T)
    np.testing.assert_allclose(got, want.numpy(), rtol=1e-12, atol=1e-13)


def test_all_experts_selected_uses_full_softmax():
    s = gen.Shape(hidden=9, latent=7, n_experts=4, top_k=4, ffn=3, shared_ffn=3)
    lw = make_f32_layer(s, 13)
    x = np.random.default_rng(14).standard_normal((3, 9))
    L = oracle.Layer(lw)
    out = L and oracle.block_forward(L, x)
    assert np.all(out["ids"] == np.arange(4))
    assert np.all(np.isinf(out["gap"]))
    z = x @ lw.D.astype(np.float64).T
    p = torch.softmax(torch.tensor(z @ lw.Wr.astype(np.float64).T + lw.br), dim=1).numpy()
    m = oracle.swiglu(z, *L.shared)
    for e in range(4):
        m = m + p[:, e:e + 1] * oracle.swiglu(z, *L.expert(e))
    np.testing.assert_allclose(out["y"], m @ lw.U.astype(np.float64).T, rtol=1e-12, atol=1e-13)


def test_zero_shared_weights_equal_no_shared_expert():
    lw = make_f32_layer(SMALL, 15)
    x = np.random.default_rng(16).standard_normal((4, SMALL.hidden))
    a = oracle.block_forward(oracle.Layer(lw), x)["y"]
    lw0 = make_f32_layer(SMALL, 15)
    lw0.shared = np.zeros_like(lw0.shared)
    lwn = make_f32_layer(SMALL, 15)
    lwn.shared = None
    b = oracle.block_forward(oracle.Layer(lw0), x)["y"]
    c = oracle.block_forward(oracle.Layer(lwn), x)["y"]
    np.testing.assert_array_equal(b, c)
    assert np.max(np.abs(a - b)) > 1e-3  # the shared expert does contribute when present


def test_token_permutation_and_batch_invariance():
    s = gen.Shape(hidden=12, latent=8, n_experts=7, top_k=2, ffn=4, shared_ffn=4)
    lw = make_f32_layer(s, 17)
    L = oracle.Layer(lw)
    x = np.random.default_rng(18).standard_normal((9, 12))
    y = oracle.block_forward(L, x)["y"]
    p = np.random.default_rng(19).permutation(9)
    np.testing.assert_allclose(oracle.block_forward(L, x[p])["y"], y[p], rtol=1e-13, atol=1e-14)
    for t in (0, 4, 8):
        np.testing.assert_allclose(oracle.block_forward(L, x[t:t + 1])["y"][0], y[t], rtol=1e-13, atol=1e-14)


def test_scaling_u_by_two_doubles_output_exactly():
    lw = make_f32_layer(SMALL, 20)
    x = np.random.default_rng(21).standard_normal((3, SMALL.hidden))
    a = oracle.block_forward(oracle.Layer(lw), x)["y"]
    lw.U = lw.U * np.float32(2)
    b = oracle.block_forward(oracle.Layer(lw), x)["y"]
    np.testing.assert_array_equal(b, 2 * a)


def test_silu_against_torch_and_limits():
    v = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(oracle.silu(v), torch.nn.functional.silu(torch.tensor(v)).numpy(), rtol=1e-14, atol=1e-300)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert abs(oracle.silu(np.array([40.0]))[0] - 40.0) < 1e-12


def test_bf16_decode_and_round_against_torch():
    rng = np.random.default_rng(22)
    v = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    # ties: values exactly half-way between two bf16 values
    base = torch.tensor(v[:1000]).to(torch.bfloat16).to(torch.float32).numpy()
    ties = (base.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    v = np.concatenate([v, ties])
    want = torch.tensor(v).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_to_bf16(v.astype(np.float64)), want)
    bits = torch.tensor(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.bf16_to_f64(bits), want)
    # the generator's encoder agrees with torch's rounding too
    np.testing.assert_array_equal(gen.bf16_bits(v.copy()), bits)


def test_mxfp4_decode_hand_built_bytes():
    # one row, K = 64: two scale blocks
    codes = list(range(16)) * 4                     # every nibble value, twice per block
    nib = np.array([codes[i] | (codes[i + 1] << 4) for i in range(0, 64, 2)], dtype=np.uint8)
    scales = np.array([127, 129], dtype=np.uint8)   # 2^0 and 2^2
    got = oracle.mxfp4_decode(nib, scales, 1, 64)[0]
    mags = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    want = [(-1 if c & 8 else 1) * mags[c & 7] for c in codes]
    want = np.array(want[:32] + [4 * v for v in want[32:]])
    np.testing.assert_array_equal(got, want)
    # extreme scale bytes
    one = np.array([0x22] * 16, dtype=np.uint8)     # every element code 2 (= 1.0)
    assert oracle.mxfp4_decode(one, np.array([0], np.uint8), 1, 32)[0, 0] == 2.0 ** -127
    assert oracle.mxfp4_decode(one, np.array([254], np.uint8), 1, 32)[0, 5] == 2.0 ** 127


def test_mxfp4_encoder_decoder_round_trip():
    rng = np.random.default_rng(23)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    # values on the grid times a per-block power of two (with 6 present so amax fixes the scale)
    vals = rng.choice(grid, size=(8, 64)) * rng.choice([-1, 1], size=(8, 64))
    vals[:, 0] = 6.0
    vals[:, 32] = -6.0
    vals = vals * np.repeat(np.ldexp(1.0, rng.integers(-10, 10, size=(8, 2))), 32, axis=1)
    nib, sc = gen.mxfp4_encode(vals.astype(np.float32))
    np.testing.assert_array_equal(oracle.mxfp4_decode(nib, sc, 8, 64), vals)
    # random normals: error at most half a grid step of the block's scale (or saturation)
    w = rng.standard_normal((16, 128)).astype(np.float32)
    nib, sc = gen.mxfp4_encode(w)
    d = oracle.mxfp4_decode(nib, sc, 16, 128)
    scale = np.repeat(np.ldexp(1.0, sc.astype(np.int64) - 127), 32, axis=1)
    a = np.abs(w) / scale
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    assert np.all(np.abs(d - w) <= np.maximum(step / 2 * scale, np.maximum(np.abs(w) - 6 * scale, 0)) + 1e-12)


def test_mxfp4_encoder_ties_go_to_even():
    """Values exactly between two E2M1 grid points take the even code (OCP MX v1.0 rounding):
    0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4, at any block scale;
    just off a midpoint they go to the nearer point."""
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    to = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for s in (-20, -3, 0, 7):
        row = np.zeros(64)
        row[0] = 6.0                                   # amax = 6 * 2^s fixes the shared exponent at s
        row[1:8] = mids
        row[8:15] = [-m for m in mids]
        row[15:22] = np.nextafter(np.array(mids, dtype=np.float32), np.float32(0))
        row[22:29] = np.nextafter(np.array(mids, dtype=np.float32), np.float32(9))
        row[32] = -6.0
        row[33:40] = mids
        w = (row * 2.0 ** s).astype(np.float32)[None, :]
        nib, sc = gen.mxfp4_encode(w)
        assert list(sc[0]) == [127 + s, 127 + s]
        d = oracle.mxfp4_decode(nib, sc, 1, 64)[0] / 2.0 ** s
        np.testing.assert_array_equal(d[1:8], to)
        np.testing.assert_array_equal(d[8:15], [-v for v in to])
        below = [max(g for g in grid if g < m) for m in mids]
        above = [min(g for g in grid if g > m) for m in mids]
        np.testing.assert_array_equal(d[15:22], below)
        np.testing.assert_array_equal(d[22:29], above)
        np.testing.assert_array_equal(d[33:40], to)


def test_e4m3_decode_closed_forms():
    # FP8 E4M3 (sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 subnormal)
    b = np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x3C, 0x3F, 0x7E, 0xB8, 0x80], dtype=np.uint8)
    want = [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.5, 1.875, 448.0, -1.0, -0.0]
    np.testing.assert_array_equal(oracle.e4m3_decode(b), want)
    assert np.isnan(oracle.e4m3_decode(np.array([0x7F], np.uint8))[0])
    # every finite positive code: strictly increasing, each binade 8 evenly spaced values
    v = oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0) and v[-1] == 448.0
    for e in range(1, 16):
        seg = v[8 * e: 8 * e + 8]
        np.testing.assert_allclose(np.diff(seg), 2.0 ** (e - 10))


def test_e4m3_encoder_against_the_decoder():
    v = oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    # every value rounds to itself and encodes to its own byte
    np.testing.assert_array_equal(gen.e4m3_round(v), v)
    np.testing.assert_array_equal(gen.e4m3_bits(v), np.arange(0, 0x7F, dtype=np.uint8))
    # midpoints go to the even mantissa; above 448 saturates
    mid = (v[1:] + v[:-1]) / 2
    r = gen.e4m3_round(mid)
    codes = gen.e4m3_bits(r)
    assert np.all(codes % 2 == 0)
    assert gen.e4m3_round(np.array([500.0, 1e9]))[0] == 448.0


def test_nvfp4_decode_hand_built_bytes():
    codes = list(range(16)) * 2                     # one row, K = 32: two scale blocks
    nib = np.array([codes[i] | (codes[i + 1] << 4) for i in range(0, 32, 2)], dtype=np.uint8)
    scales = np.array([0x40, 0x30], dtype=np.uint8)  # 2.0 and 0.5
    got = oracle.nvfp4_decode(nib, scales, 0.25, 1, 32)[0]
    mags = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    base = [(-1 if c & 8 else 1) * mags[c & 7] for c in codes]
    want = np.array([v * 2.0 * 0.25 for v in base[:16]] + [v * 0.5 * 0.25 for v in base[16:]])
    np.testing.assert_array_equal(got, want)


def test_nvfp4_encoder_decoder_round_trip():
    rng = np.random.default_rng(29)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    ts = 2.0 ** -7
    # on-grid values: E2M1 * (an E4M3 block scale) * tensor scale, every block holding 6 * its
    # scale, and one block at the largest scale so that the tensor scale is amax / (6 * 448)
    bscale = oracle.e4m3_decode(rng.integers(0x20, 0x70, size=(4, 8)).astype(np.uint8))
    bscale[0, 0] = 448.0
    vals = rng.choice(grid, size=(4, 128)) * rng.choice([-1, 1], size=(4, 128))
    vals[:, ::16] = 6.0
    vals = vals * np.repeat(bscale, 16, axis=1) * ts
    nib, sc, t = gen.nvfp4_encode(vals.astype(np.float32))
    assert t == np.float32(np.abs(vals).max() / (6 * 448))
    np.testing.assert_array_equal(oracle.nvfp4_decode(nib, sc, t, 4, 128), vals)
    # random normals: within half an E2M1 step of the block scale, plus the scale's own rounding
    w = rng.standard_normal((16, 256)).astype(np.float32)
    nib, sc, t = gen.nvfp4_encode(w)
    d = oracle.nvfp4_decode(nib, sc, t, 16, 256)
    amax = np.repeat(np.abs(w.reshape(16, 16, 16)).max(axis=2), 16, axis=1)
    assert np.all(np.abs(d - w) <= amax * (1 / 6 + 1 / 16) + 1e-12)
    assert np.mean(np.abs(d - w)) / np.mean(np.abs(w)) < 0.12


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_four_bit_record_layout(fmt):
    """A generated 4-bit record decodes (by the oracle) to the normals it was drawn from, matrix by
    matrix, within the format's rounding: a misplaced nibble, scale or tensor-scale field would not."""
    s = gen.Shape(hidden=64, latent=128, n_experts=2, top_k=1, ffn=64, shared_ffn=0)
    rec = gen.expert_record(s, gen.rng_for(99, 0, gen.T_EXPERT, 0), fmt)
    ref = gen.expert_record(s, gen.rng_for(99, 0, gen.T_EXPERT, 0), "f32").astype(np.float64)
    f, l = s.ffn, s.latent
    want = (ref[: f * l].reshape(f, l), ref[f * l: 2 * f * l].reshape(f, l), ref[2 * f * l:].reshape(l, f))
    got = oracle.expert_matrices(rec, fmt, l, f)
    assert rec.size == (s.mxfp4_record_bytes() if fmt == "mxfp4" else s.nvfp4_record_bytes())
    for g_, w_ in zip(got, want):
        assert g_.shape == w_.shape
        rel = np.linalg.norm(g_ - w_) / np.linalg.norm(w_)
        assert rel < 0.15, rel


def test_rmsnorm_closed_form():
    h = np.full((2, 10), 3.0)
    h[1] = -0.5
    r = oracle.rmsnorm(h)
    np.testing.assert_allclose(r[0], 3 / math.sqrt(9 + 1e-6), rtol=1e-15)
    np.testing.assert_allclose(r[1], -0.5 / math.sqrt(0.25 + 1e-6), rtol=1e-15)


def test_stack_step_with_zero_block_is_identity():
    s = gen.Shape(hidden=8, latent=4, n_experts=3, top_k=1, ffn=2, shared_ffn=2)
    lw = make_f32_layer(s, 24)
    lw.U = np.zeros_like(lw.U)
    h = np.random.default_rng(25).standard_normal((3, 8)).astype(np.float32).astype(np.float64)
    out = oracle.stack_step(oracle.Layer(lw), h)
    np.testing.assert_array_equal(out["h_next"], h)
    np.testing.assert_array_equal(out["x"], oracle.round_to_bf16(oracle.rmsnorm(h)))


def test_forced_ids_match_scalar_brute_force():
    """block_forward(forced_ids=...) on tokens whose forced sets differ from their top k, given
    out of order: ids come back ascending, weights are the softmax over the forced experts'
    logits (the full softmax renormalised over them), the output uses exactly those experts."""
    s = gen.Shape(hidden=6, latent=5, n_experts=7, top_k=3, ffn=3, shared_ffn=2)
    lw = make_f32_layer(s, 41)
    x = np.random.default_rng(42).standard_normal((4, s.hidden)).astype(np.float32)
    L = oracle.Layer(lw)
    free = oracle.block_forward(L, x.astype(np.float64))
    forced = {}
    for t in (0, 2, 3):
        rest = [e for e in range(7) if e not in free["ids"][t]]
        # keep one routed expert, swap in two others, listed in descending id
        forced[t] = sorted([int(free["ids"][t][1]), rest[0], rest[-1]], reverse=True)
    got = oracle.block_forward(L, x.astype(np.float64), forced_ids=forced)
    y, ids, w = brute_forward(lw, x, forced=forced, details=True)
    np.testing.assert_array_equal(got["ids"], ids)
    np.testing.assert_allclose(got["w"], w, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(got["y"], y, rtol=1e-12, atol=1e-13)
    # the token left to the router is untouched by the others' forcing
    np.testing.assert_array_equal(got["ids"][1], free["ids"][1])
    np.testing.assert_array_equal(got["y"][1], free["y"][1])
    assert all(not np.array_equal(got["ids"][t], free["ids"][t]) for t in forced)


# Every finite non-negative bf16 value (bit patterns 0x0000 .. 0x7F7F), exactly, for the
# enumeration below.
_BF16_POS = None


def _bf16_values():
    global _BF16_POS
    if _BF16_POS is None:
        bits = np.arange(0, 0x7F80, dtype=np.uint32) << np.uint32(16)
        _BF16_POS = [Fraction(float(v)) for v in bits.view(np.float32)]
    return _BF16_POS


def py_bf16_nearest(v: float) -> float:
    """Nearest bf16 value of the exact double v by enumeration: locate v among all finite bf16
    values, compare the exact distances to its two neighbours, ties to the even bit pattern, and
    overflow to infinity from half a step above the largest finite value."""
    if v != v or v == 0.0:
        return v
    vals = _bf16_values()
    a = Fraction(abs(v))
    top = vals[-1] + (vals[-1] - vals[-2]) / 2
    if a >= top:
        return math.copysign(math.inf, v)
    i = bisect.bisect_left(vals, a)
    if i < len(vals) and vals[i] == a:
        r = i
    else:
        lo, hi = i - 1, min(i, len(vals) - 1)
        dl, dh = a - vals[lo], vals[hi] - a
        r = lo if dl < dh or (dl == dh and lo % 2 == 0) else hi
    return math.copysign(float(vals[r]), v)


def test_round_to_bf16_is_one_rounding_of_the_exact_value():
    u = 2.0 ** -8  # half a bf16 step at 1
    cases = [
        (1 + u + 2.0 ** -30, 1 + 2 * u),   # just above the midpoint; via float32 it would tie and fall to 1
        (1 + u, 1.0),                       # exact midpoint: to the even significand
        (1 + 3 * u, 1 + 4 * u),             # midpoint between odd 1 + 2u and even 1 + 4u
        (1 + u - 2.0 ** -40, 1.0),
        (-(1 + u + 2.0 ** -30), -(1 + 2 * u)),
        (2.0 ** -134, 0.0),                 # half the smallest subnormal: to even (zero)
        (3 * 2.0 ** -134, 2.0 ** -132),     # between subnormals 1 and 2 (units of 2^-133)
        (oracle.BF16_MAX + 2.0 ** 119, math.inf),
        (oracle.BF16_MAX + 2.0 ** 119 - 2.0 ** 100, oracle.BF16_MAX),
    ]
    for v, want in cases:
        assert oracle.round_to_bf16(np.array([v]))[0] == want, v
        assert py_bf16_nearest(v) == want, v
    # random doubles over a wide range of exponents with low bits below float32's precision
    rng = np.random.default_rng(44)
    v = rng.standard_normal(3000) * np.ldexp(1.0, rng.integers(-140, 120, 3000))
    v[:1000] = (v[:1000].astype(np.float32).astype(np.float64) * (1 + 2.0 ** -30))
    got = oracle.round_to_bf16(v)
    want = np.array([py_bf16_nearest(float(a)) for a in v])
    np.testing.assert_array_equal(got, want)


def _f32(v: float) -> float:
    return struct.unpack("f", struct.pack("f", v))[0]


def test_stack_step_matches_scalar_brute_force():
    """One residual layer: h_next = fp32(h + block(bf16(RMSNorm(h)))), every piece in scalar
    Python (the block by brute_forward, the bf16 rounding by enumeration)."""
    s = gen.Shape(hidden=8, latent=5, n_experts=6, top_k=2, ffn=3, shared_ffn=3)
    lw = make_f32_layer(s, 45)
    lw.U = lw.U * np.float32(4)  # a block output comparable to h
    rng = np.random.default_rng(46)
    h = (rng.standard_normal((3, 8)) * np.array([[1.0], [30.0], [0.01]])).astype(np.float32).astype(np.float64)
    out = oracle.stack_step(oracle.Layer(lw), h)
    x = []
    for row in h.tolist():
        rms = math.sqrt(sum(a * a for a in row) / len(row) + 1e-6)
        x.append([py_bf16_nearest(a / rms) for a in row])
    x = np.array(x)
    np.testing.assert_array_equal(out["x"], x)
    y = brute_forward(lw, x)
    want = np.array([[_f32(a + b) for a, b in zip(hr, yr)] for hr, yr in zip(h.tolist(), y.tolist())])
    assert np.abs(y).max() > 0.1 * np.abs(h).min()
    np.testing.assert_allclose(out["h_next"], want, rtol=1e-12, atol=0)


def test_page_shapes_pin_the_edge0_block():
    with open(os.path.join(HERE, "golden", "page_shapes.json")) as f:
        g = json.load(f)
    s = gen.EDGE0_145B
    assert s.hidden == g["hidden"]["value"]
    assert s.latent == g["latent_width"]["value"]
    assert s.n_experts == g["experts_per_layer"]["value"]
    assert s.top_k == g["routed_active"]["value"]
    assert s.ffn == g["swiglu_width"]["value"]
    assert (s.shared_ffn > 0) == (g["shared_active"]["value"] == 1)
    pool = g["layers"]["value"] * s.n_experts * s.record_elems()
    assert round(pool / 1e9, 1) == g["expert_pool_params_billions"]["value"]


def test_page_shapes_pin_the_120b_latent_width():
    with open(os.path.join(HERE, "golden", "page_shapes.json")) as f:
        g = json.load(f)
    assert gen.EDGE0_120B.latent == g["latent_width_120b"]["value"]
    assert gen.EDGE0_145B.latent == g["latent_width_145b_article"]["value"]
    # the other dimensions are read as the 145B's (the pages give none for the 120B)
    a, b = gen.EDGE0_120B, gen.EDGE0_145B
    assert (a.hidden, a.n_experts, a.top_k, a.ffn, a.shared_ffn) == (b.hidden, b.n_experts, b.top_k, b.ffn, b.shared_ffn)


def test_page_shapes_pin_the_expert_groups():
    with open(os.path.join(HERE, "golden", "page_shapes.json")) as f:
        g = json.load(f)
    s = gen.EDGE0_145B_G64
    assert s.n_experts // s.groups == g["experts_per_group"]["value"]
    assert s.n_experts == g["experts_per_layer"]["value"]
    assert (s.hidden, s.latent, s.top_k, s.ffn) == (gen.EDGE0_145B.hidden, gen.EDGE0_145B.latent, gen.EDGE0_145B.top_k,
                                                    gen.EDGE0_145B.ffn)


@pytest.mark.parametrize("wid", ["tiny_f32", "decode_t8"])
def test_generator_is_seed_stable(wid):
    wl = gen.WORKLOADS[wid]
    a = gen.make_tokens(wl, T=4)
    b = gen.make_tokens(wl, T=4)
    np.testing.assert_array_equal(a, b)
    if wid == "tiny_f32":
        l1, l2 = gen.make_layer(wl), gen.make_layer(wl)
        np.testing.assert_array_equal(l1.experts, l2.experts)
        np.testing.assert_array_equal(l1.D, l2.D)


def test_zipf_bias_is_a_log_prior_over_a_permutation():
    wl = gen.WORKLOADS["decode_t8"]
    b = gen.router_bias(wl, 0).astype(np.float64)
    ranks = np.rint(np.exp(-b / 1.1) - 1).astype(int)
    assert sorted(ranks.tolist()) == list(range(512))
    assert b.max() == 0.0
