"""lmoe_forward_noalloc (the allocation-free entry point) against lmoe_forward with a caller
workspace, through the C ABI.

Both run the same kernels on the same inputs, so the outputs and every export must agree bit for
bit (stricter than the block's tolerance).  Each case makes two calls in a row on the library's
one scratch array, the second with fewer tokens, so the second call runs on the first call's
leftovers.  A batch whose workspace exceeds the array is refused before anything is enqueued.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import lmoe_data as gen
import sparse_moe_proj_amd as lm
from sparse_moe_proj_amd.device import DeviceLayer, Workspace, to_device

pytestmark = pytest.mark.gpu


def _outputs(dl, T, fill):
    s = dl.shape
    return dict(
        y=torch.full((T, s.hidden), fill, dtype=torch.int16, device="cuda"),
        z=torch.full((T, s.groups * s.latent), float(fill), dtype=torch.float32, device="cuda"),
        ids=torch.full((T, s.top_k), fill, dtype=torch.int32, device="cuda"),
        w=torch.full((T, s.top_k), float(fill), dtype=torch.float32, device="cuda"),
        offsets=torch.full((s.n_experts + 1,), fill, dtype=torch.int32, device="cuda"),
        perm=torch.full((max(1, T * s.top_k),), fill, dtype=torch.int32, device="cuda"),
    )


def _call(dl, x, T, noalloc, fill):
    out = _outputs(dl, T, fill)
    opts = lm.make_opts(0, 0, out["z"], out["ids"], out["w"], out["offsets"], out["perm"])
    if noalloc:
        lm.check(lm.lmoe_forward_noalloc(dl.cfg, dl.weights, x, T, out["y"], opts))
    else:
        ws = Workspace("cuda").get(lm.lmoe_workspace_bytes(dl.cfg, T))
        lm.check(lm.lmoe_forward(dl.cfg, dl.weights, x, T, out["y"], opts, ws, ws.numel()))
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def _same(a, b, label):
    for key in a:
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), f"{label}: {key} differs"


CASES = [
    # (label, shape, expert format, first T, second T)
    ("edge0_145b_bf16", gen.EDGE0_145B, "bf16", 64, 8),
    ("edge0_145b_bf16_t8", gen.EDGE0_145B, "bf16", 8, 3),
    ("small_mxfp4", gen.Shape(hidden=256, latent=256, n_experts=24, top_k=3, ffn=128, shared_ffn=128), "mxfp4", 40, 7),
    ("small_nvfp4_groups", gen.Shape(hidden=256, latent=256, n_experts=24, top_k=3, ffn=128, shared_ffn=128, groups=2),
     "nvfp4", 17, 1),
]


@pytest.mark.parametrize("label,shape,expert,T1,T2", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_forward_on_two_calls(label, shape, expert, T1, T2):
    wl = gen.Workload(91, label, shape, T1, "bf16", "bf16", expert, "zipf")
    dl = DeviceLayer(gen.make_layer(wl, 0), act="bf16")
    for i, T in enumerate((T1, T2)):
        assert lm.lmoe_workspace_bytes(dl.cfg, T) <= lm.LMOE_NOALLOC_SCRATCH_BYTES
        x = to_device(gen.make_tokens(wl, T=T, salt=i))
        want = _call(dl, x, T, noalloc=False, fill=7)
        got = _call(dl, x, T, noalloc=True, fill=-3)
        _same(want, got, f"{label} call {i + 1} (T={T})")
        print(f"[{label}] call {i + 1}: T={T} bitwise equal to lmoe_forward", flush=True)


def test_noalloc_refuses_a_batch_beyond_its_array():
    shape = gen.EDGE0_145B
    cfg = lm.make_config(shape.hidden, shape.latent, shape.n_experts, shape.top_k, shape.ffn, shape.shared_ffn)
    T = 4096
    assert lm.lmoe_workspace_bytes(cfg, T) > lm.LMOE_NOALLOC_SCRATCH_BYTES
    y = torch.full((T, shape.hidden), 5, dtype=torch.int16, device="cuda")
    x = torch.zeros((T, shape.hidden), dtype=torch.int16, device="cuda")
    w = lm.make_weights(x, x, x, None, x, x)  # never read: the size check comes first
    st = lm.lmoe_forward_noalloc(cfg, w, x, T, y, None)
    assert st == lm.LMOE_ERR_WORKSPACE and "allocation-free" in lm.last_error()
    torch.cuda.synchronize()
    assert bool((y == 5).all()), "nothing may be written after a refused call"
