"""lmoe_forward captured into a HIP graph (via torch.cuda.graph) and replayed: every replay,
with eager work and synchronisations in between, must equal the eager result bit for bit."""
import pytest
import torch

import lmoe_data as gen
from parity import run_forward, small_layer, upload_tokens
from sparse_moe_proj_amd.device import DeviceLayer, Workspace

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T", [8, 200])
def test_graph_replays_match_eager(T):
    shape = gen.Shape(hidden=256, latent=192, n_experts=24, top_k=3, ffn=128, shared_ffn=64)
    wl, lw = small_layer(shape, "bf16", "bf16", "bf16", wid=81)
    dl = DeviceLayer(lw, act="bf16")
    x = upload_tokens(gen.make_tokens(wl, T=T, salt=2))
    ws = Workspace("cuda")
    eager = run_forward(dl, x, ws)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in eager.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        warm = run_forward(dl, x, ws)  # allocations happen outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = run_forward(dl, x, ws)
    for i in range(4):
        for v in cap.values():
            v.fill_(-1)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key in ("y", "z", "ids", "w", "offsets", "perm"):
            assert torch.equal(cap[key], ref[key]), f"replay {i}: {key} differs"
    del warm
