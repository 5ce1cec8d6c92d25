"""lmoe_pack_experts against an independent numpy statement of the packed layout (the header's
description: 1 KB tiles of 16 rows; inside a tile the unit of row j and column group q sits at
position 16 q + j; tiles ordered by row block, then column step), byte for byte."""
import numpy as np
import pytest
import torch

import lmoe_data as gen
import sparse_moe_proj_amd as lm
from sparse_moe_proj_amd.device import to_device

pytestmark = pytest.mark.gpu


def tiles(units: np.ndarray) -> np.ndarray:
    """units [N][C][u] (C units per row, u bytes each) -> packed order."""
    N, C, u = units.shape
    return units.reshape(N // 16, 16, C // 4, 4, u).transpose(0, 2, 3, 1, 4).reshape(-1)


def pack_bf16(rec: np.ndarray, F: int, L: int) -> np.ndarray:
    b = rec.view(np.uint8)
    fl = F * L * 2
    mats = [(b[:fl], F, L), (b[fl:2 * fl], F, L), (b[2 * fl:3 * fl], L, F)]
    return np.concatenate([tiles(m.reshape(N, K // 8, 16)) for m, N, K in mats])


def pack_mx(rec: np.ndarray, F: int, L: int) -> np.ndarray:
    nb, sb = F * L // 2, F * L // 32
    out = []
    for i, (N, K) in enumerate([(F, L), (F, L), (L, F)]):
        out.append(tiles(rec[i * nb:(i + 1) * nb].reshape(N, K // 32, 16)))
    for i, (N, K) in enumerate([(F, L), (F, L), (L, F)]):
        out.append(tiles(rec[3 * nb + i * sb:3 * nb + (i + 1) * sb].reshape(N, K // 32, 1)))
    return np.concatenate(out)


def pack_nv(rec: np.ndarray, F: int, L: int) -> np.ndarray:
    """NVFP4: nibble tiles as MXFP4; scale tiles hold the two E4M3 bytes of each 32-value unit;
    the 16-byte tail (three fp32 tensor scales and padding) is unchanged."""
    nb, sb = F * L // 2, F * L // 16
    out = []
    for i, (N, K) in enumerate([(F, L), (F, L), (L, F)]):
        out.append(tiles(rec[i * nb:(i + 1) * nb].reshape(N, K // 32, 16)))
    for i, (N, K) in enumerate([(F, L), (F, L), (L, F)]):
        out.append(tiles(rec[3 * nb + i * sb:3 * nb + (i + 1) * sb].reshape(N, K // 32, 2)))
    out.append(rec[3 * nb + 3 * sb:])
    return np.concatenate(out)


@pytest.mark.parametrize("expert", ["bf16", "mxfp4", "nvfp4"])
def test_pack_matches_layout(expert):
    shape = gen.Shape(256, 256, 5, 2, 128, 384)
    wl = gen.Workload(78, "pack", shape, 0, "bf16", "bf16", expert, "zero")
    lw = gen.make_layer(wl, 0)
    cfg = lm.make_config(256, 256, 5, 2, 128, 384, "bf16", "bf16", expert)
    src = to_device(lw.experts)
    dst = torch.zeros_like(src)
    lm.check(lm.lmoe_pack_experts(cfg, 0, src, dst, 5))
    ssrc = to_device(lw.shared)
    sdst = torch.zeros_like(ssrc)
    lm.check(lm.lmoe_pack_experts(cfg, 1, ssrc, sdst, 1))
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np.uint8).reshape(5, -1)
    for e in range(5):
        rec = np.ascontiguousarray(lw.experts[e])
        if expert == "mxfp4":
            want = pack_mx(rec.view(np.uint8), 128, 256)
        elif expert == "nvfp4":
            want = pack_nv(rec.view(np.uint8), 128, 256)
        else:
            want = pack_bf16(rec, 128, 256)
        assert np.array_equal(got[e], want), f"record {e}"
    want_sh = pack_bf16(np.ascontiguousarray(lw.shared), 384, 256)
    assert np.array_equal(sdst.cpu().numpy().view(np.uint8).reshape(-1), want_sh)
