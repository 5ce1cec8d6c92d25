"""C-ABI checks that need no GPU: the library loads, exports every function include/lmoe.h
declares, answers size queries, and rejects bad arguments on the host before enqueuing
anything (fake device addresses are never dereferenced because validation fails first)."""
import ctypes

import pytest

import lmoe_data as gen
import sparse_moe_proj_amd as lm

S = gen.EDGE0_145B
FAKE = 1 << 40  # a 16-byte aligned address that is never dereferenced


def cfg(**kw):
    base = dict(hidden=S.hidden, latent=S.latent, n_experts=S.n_experts, top_k=S.top_k, ffn=S.ffn,
                shared_ffn=S.shared_ffn, act="bf16", dense="bf16", expert="bf16")
    base.update(kw)
    return lm.make_config(**base)


def full_weights():
    return lm.make_weights(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)


def test_every_header_symbol_is_exported():
    syms = lm.header_symbols()
    assert {"lmoe_route", "lmoe_permute", "lmoe_forward"} <= set(syms)
    for name in syms:
        assert hasattr(lm.lib, name), name
        assert ctypes.cast(getattr(lm.lib, name), ctypes.c_void_p).value


def test_version_and_status_strings():
    assert lm.lmoe_version() >= 100
    for st in range(8):
        assert lm.lmoe_status_str(st)
    assert lm.lmoe_status_str(99) == "unknown status"


def test_record_sizes():
    assert lm.lmoe_expert_record_bytes(cfg(), 0) == 3 * 640 * 1792 * 2
    assert lm.lmoe_expert_record_bytes(cfg(expert="mxfp4"), 0) == S.mxfp4_record_bytes() == 1827840
    assert lm.lmoe_expert_record_bytes(cfg(expert="mxfp4"), 1) == 3 * 640 * 1792 * 2  # shared stays bf16
    assert lm.lmoe_expert_record_bytes(cfg(expert="nvfp4"), 0) == S.nvfp4_record_bytes() == 1935376
    assert lm.lmoe_expert_record_bytes(cfg(expert="nvfp4"), 1) == 3 * 640 * 1792 * 2
    t = gen.TINY
    c = lm.make_config(t.hidden, t.latent, t.n_experts, t.top_k, t.ffn, t.shared_ffn, "f32", "f32", "f32")
    assert lm.lmoe_expert_record_bytes(c, 0) == 3 * 64 * 128 * 4
    assert lm.lmoe_expert_record_bytes(cfg(shared_ffn=0), 1) == 0


def test_workspace_sizes_monotone():
    c = cfg()
    prev = 0
    for T in (0, 1, 8, 16, 17, 64, 65, 4096, 16384):
        n = lm.lmoe_workspace_bytes(c, T)
        assert n >= prev
        prev = n
    assert lm.lmoe_permute_workspace_bytes(c, 64) == 0
    assert lm.lmoe_permute_workspace_bytes(c, 65) > 0


@pytest.mark.parametrize("expert", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("mx_mfma", ["1", "0"])
def test_workspace_monotone_4bit_paths(expert, mx_mfma):
    """4-bit layers change kernels at 65 (small-batch -> weight streaming), at 96 (MXFP4: the
    block-scaled MFMA path, whose MXFP8 activations need workspace) and at 384 (the decode of the
    records to bf16: n_experts decoded records); the size query stays monotone in T across all.
    mx_mfma 0 switches the block-scaled path off through lmoe_config.mx_mfma_min_t = -1."""
    c = lm.make_config(2560, 1792, 512, 10, 640, 640, "bf16", "bf16", expert, 1, 0 if mx_mfma == "1" else -1)
    prev = 0
    for T in list(range(60, 100)) + [383, 384, 385, 4096, 16384]:
        n = lm.lmoe_workspace_bytes(c, T)
        assert n >= prev, (T, prev, n)
        prev = n
    decoded = 512 * 3 * 640 * 1792 * 2
    big = lm.lmoe_workspace_bytes(c, 384) - lm.lmoe_workspace_bytes(c, 383)
    if expert == "mxfp4" and mx_mfma == "1":
        assert big < decoded  # no decoded records on the block-scaled MFMA path
        assert lm.lmoe_workspace_bytes(c, 96) > lm.lmoe_workspace_bytes(c, 95)  # MXFP8 activations from 96
    else:
        assert big >= decoded


@pytest.mark.parametrize("kw,code", [
    (dict(hidden=100), lm.LMOE_ERR_SHAPE),
    (dict(latent=0), lm.LMOE_ERR_SHAPE),
    (dict(top_k=0), lm.LMOE_ERR_SHAPE),
    (dict(top_k=17, n_experts=64), lm.LMOE_ERR_SHAPE),
    (dict(n_experts=5, top_k=10), lm.LMOE_ERR_SHAPE),
    (dict(n_experts=2048), lm.LMOE_ERR_SHAPE),
    (dict(shared_ffn=32), lm.LMOE_ERR_SHAPE),
    (dict(expert="mxfp4", latent=192), lm.LMOE_ERR_SHAPE),
    (dict(expert="mxfp4", shared_ffn=64), lm.LMOE_ERR_SHAPE),
    (dict(act="f32"), lm.LMOE_ERR_UNSUPPORTED),
    (dict(expert="f32"), lm.LMOE_ERR_UNSUPPORTED),
    (dict(groups=3), lm.LMOE_ERR_SHAPE),
    (dict(groups=-1), lm.LMOE_ERR_SHAPE),
    (dict(groups=128, n_experts=1024), lm.LMOE_ERR_SHAPE),
])
def test_bad_config_rejected(kw, code):
    n = ctypes.c_size_t(0)
    assert lm.lib.lmoe_workspace_bytes(ctypes.byref(cfg(**kw)), 8, ctypes.byref(n)) == code
    assert lm.lmoe_forward(cfg(**kw), full_weights(), FAKE, 8, FAKE + 4096, None, FAKE, 1 << 40, 0) == code
    assert lm.last_error()


def test_bad_dtype_code():
    c = cfg()
    c.expert_dtype = 7
    assert lm.lmoe_forward(c, full_weights(), FAKE, 8, FAKE, None, FAKE, 1 << 40, 0) == lm.LMOE_ERR_DTYPE


def test_null_config_and_pointers():
    assert lm.lib.lmoe_forward(None, None, None, 8, None, None, None, 0, None) == lm.LMOE_ERR_NULL
    w = full_weights()
    w.Wr = None
    assert lm.lmoe_forward(cfg(), w, FAKE, 8, FAKE + (1 << 30), None, FAKE, 1 << 40, 0) == lm.LMOE_ERR_NULL
    w = full_weights()
    w.shared = None
    assert lm.lmoe_forward(cfg(), w, FAKE, 8, FAKE + (1 << 30), None, FAKE, 1 << 40, 0) == lm.LMOE_ERR_NULL
    assert lm.lmoe_route(cfg(), full_weights(), None, 8, FAKE, FAKE, FAKE, 1 << 30, 0) == lm.LMOE_ERR_NULL
    assert lm.lmoe_permute(cfg(), None, 8, FAKE, FAKE, FAKE, None, 0, 0) == lm.LMOE_ERR_NULL


def test_misaligned_pointers():
    assert lm.lmoe_forward(cfg(), full_weights(), FAKE + 2, 8, FAKE + (1 << 30), None, FAKE, 1 << 40, 0) == lm.LMOE_ERR_ALIGN
    w = full_weights()
    w.experts = FAKE + 8
    assert lm.lmoe_forward(cfg(), w, FAKE, 8, FAKE + (1 << 30), None, FAKE, 1 << 40, 0) == lm.LMOE_ERR_ALIGN
    assert lm.lmoe_permute(cfg(), FAKE + 4, 8, FAKE, FAKE, FAKE, None, 0, 0) == lm.LMOE_ERR_ALIGN


def test_workspace_too_small():
    need = lm.lmoe_workspace_bytes(cfg(), 8)
    assert lm.lmoe_forward(cfg(), full_weights(), FAKE, 8, FAKE + (1 << 30), None, FAKE, need - 1, 0) == lm.LMOE_ERR_WORKSPACE
    assert lm.lmoe_forward(cfg(), full_weights(), FAKE, 8, FAKE + (1 << 30), None, None, need, 0) == lm.LMOE_ERR_WORKSPACE
    assert lm.lmoe_route(cfg(), full_weights(), FAKE, 8, FAKE, FAKE, FAKE, 8 * 512 * 4 - 1, 0) == lm.LMOE_ERR_WORKSPACE
    assert lm.lmoe_permute(cfg(), FAKE, 65, FAKE, FAKE, FAKE, None, 0, 0) == lm.LMOE_ERR_WORKSPACE


def test_overlapping_x_y_rejected_and_options_checked():
    assert lm.lmoe_forward(cfg(), full_weights(), FAKE, 8, FAKE + 64, None, FAKE, 1 << 40, 0) == lm.LMOE_ERR_UNSUPPORTED
    t = gen.TINY
    c = lm.make_config(t.hidden, t.latent, t.n_experts, t.top_k, t.ffn, t.shared_ffn, "f32", "f32", "f32")
    o = lm.make_opts(prenorm=1)
    assert lm.lmoe_forward(c, full_weights(), FAKE, 8, FAKE + (1 << 30), o, FAKE, 1 << 40, 0) == lm.LMOE_ERR_UNSUPPORTED


def test_bad_T():
    assert lm.lmoe_forward(cfg(), full_weights(), FAKE, -1, FAKE, None, FAKE, 1 << 40, 0) == lm.LMOE_ERR_SHAPE
    assert lm.lmoe_forward(cfg(), full_weights(), FAKE, (1 << 20) + 1, FAKE, None, FAKE, 1 << 40, 0) == lm.LMOE_ERR_SHAPE


def test_zero_tokens_is_a_noop_without_device_access():
    # T = 0 returns OK before any pointer is used (all NULL here)
    nothing = lm.make_weights(None, None, None, None, None, None)
    assert lm.lmoe_forward(cfg(), nothing, None, 0, None, None, None, 0, 0) == lm.LMOE_OK
    assert lm.lmoe_route(cfg(), nothing, None, 0, None, None, None, 0, 0) == lm.LMOE_OK


def test_single_hip_runtime_in_process():
    """The library must share torch's HIP runtime: one libamdhip64 mapped in the process."""
    with open("/proc/self/maps") as f:
        libs = {line.split()[-1] for line in f if "libamdhip64" in line}
    assert len(libs) == 1, libs


def test_expert_groups_checked():
    t = gen.TINY
    g8 = cfg(groups=8)
    n1, n8 = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lm.lib.lmoe_workspace_bytes(ctypes.byref(cfg()), 64, ctypes.byref(n1)) == lm.LMOE_OK
    assert lm.lib.lmoe_workspace_bytes(ctypes.byref(g8), 64, ctypes.byref(n8)) == lm.LMOE_OK
    assert n8.value > n1.value  # z and the merged partials are eight latents wide
    # no folded router: unsupported; lmoe_route takes one latent only
    assert lm.lmoe_forward(g8, full_weights(), FAKE, 8, FAKE + (1 << 30), None, FAKE, 1 << 40, 0) == lm.LMOE_ERR_UNSUPPORTED
    assert lm.lmoe_route(g8, full_weights(), FAKE, 8, FAKE, FAKE, FAKE, 1 << 30, 0) == lm.LMOE_ERR_UNSUPPORTED
    f32 = lm.make_config(t.hidden, t.latent, t.n_experts, t.top_k, t.ffn, t.shared_ffn, "f32", "f32", "f32", groups=2)
    assert lm.lmoe_forward(f32, full_weights(), FAKE, 8, FAKE + (1 << 30), None, FAKE, 1 << 40, 0) == lm.LMOE_ERR_UNSUPPORTED
    # the fold reads all eight D matrices: Gr placed inside them overlaps
    far = FAKE + (1 << 36)
    d_bytes = 8 * S.latent * S.hidden * 2
    assert lm.lmoe_fold_router(g8, FAKE, far, FAKE + d_bytes - 4096, 0) == lm.LMOE_ERR_UNSUPPORTED


def test_fold_router_arguments_checked():
    c = cfg()
    t = gen.TINY
    f32 = lm.make_config(t.hidden, t.latent, t.n_experts, t.top_k, t.ffn, t.shared_ffn, "f32", "f32", "f32")
    assert lm.lmoe_fold_router_bytes(c) == c.n_experts * 2 * c.hidden * 2
    assert lm.lmoe_fold_router_bytes(f32) == 0
    far = FAKE + (1 << 34)
    assert lm.lmoe_fold_router(f32, FAKE, FAKE + (1 << 30), far, 0) == lm.LMOE_ERR_UNSUPPORTED
    assert lm.lmoe_fold_router(c, None, FAKE + (1 << 30), far, 0) == lm.LMOE_ERR_NULL
    assert lm.lmoe_fold_router(c, FAKE, FAKE + (1 << 30), None, 0) == lm.LMOE_ERR_NULL
    assert lm.lmoe_fold_router(c, FAKE + 8, FAKE + (1 << 30), far, 0) == lm.LMOE_ERR_ALIGN
    assert lm.lmoe_fold_router(c, FAKE, FAKE + (1 << 30), FAKE + 256, 0) == lm.LMOE_ERR_UNSUPPORTED  # Gr overlaps D


def test_pack_arguments_checked():
    c = cfg()
    rec = lm.lmoe_expert_record_bytes(c, 0)
    t = gen.TINY
    f32 = lm.make_config(t.hidden, t.latent, t.n_experts, t.top_k, t.ffn, t.shared_ffn, "f32", "f32", "f32")
    assert lm.lmoe_pack_experts(f32, 0, FAKE, FAKE + (1 << 30), 4, 0) == lm.LMOE_ERR_UNSUPPORTED
    assert lm.lmoe_pack_experts(cfg(shared_ffn=0), 1, FAKE, FAKE + (1 << 30), 1, 0) == lm.LMOE_ERR_SHAPE
    assert lm.lmoe_pack_experts(c, 1, FAKE, FAKE + (1 << 30), 2, 0) == lm.LMOE_ERR_SHAPE
    assert lm.lmoe_pack_experts(c, 0, FAKE, FAKE + (1 << 30), -1, 0) == lm.LMOE_ERR_SHAPE
    assert lm.lmoe_pack_experts(c, 0, None, FAKE, 4, 0) == lm.LMOE_ERR_NULL
    assert lm.lmoe_pack_experts(c, 0, FAKE + 4, FAKE + (1 << 34), 4, 0) == lm.LMOE_ERR_ALIGN
    assert lm.lmoe_pack_experts(c, 0, FAKE, FAKE + rec, 4, 0) == lm.LMOE_ERR_UNSUPPORTED  # overlap
    assert lm.lmoe_pack_experts(c, 0, None, None, 0, 0) == lm.LMOE_OK  # nothing to do


def test_noalloc_checks_arguments_on_the_host():
    """The allocation-free entry point refuses a batch whose workspace exceeds its static array
    (and bad shapes) before it looks for a device; T = 0 is a no-op."""
    too_big = 4096
    assert lm.lmoe_workspace_bytes(cfg(), too_big) > lm.LMOE_NOALLOC_SCRATCH_BYTES
    assert lm.lmoe_workspace_bytes(cfg(), 64) <= lm.LMOE_NOALLOC_SCRATCH_BYTES
    assert lm.lmoe_workspace_bytes(cfg(groups=8), 64) <= lm.LMOE_NOALLOC_SCRATCH_BYTES
    st = lm.lmoe_forward_noalloc(cfg(), full_weights(), FAKE, too_big, FAKE + (1 << 36), None, 0)
    assert st == lm.LMOE_ERR_WORKSPACE and "allocation-free" in lm.last_error()
    assert lm.lmoe_forward_noalloc(cfg(), full_weights(), FAKE, -1, FAKE, None, 0) == lm.LMOE_ERR_SHAPE
    nothing = lm.make_weights(None, None, None, None, None, None)
    assert lm.lmoe_forward_noalloc(cfg(), nothing, None, 0, None, None, 0) == lm.LMOE_OK


def test_mx_threshold_is_a_config_field():
    """The block-scaled MXFP4 path's threshold comes from lmoe_config (never the environment): the
    workspace grows where the MXFP8 activations appear, at the configured batch size."""
    for t0 in (0, 200):
        c = lm.make_config(2560, 1792, 512, 10, 640, 640, "bf16", "bf16", "mxfp4", 1, t0)
        at = 96 if t0 == 0 else 200
        jump = lm.lmoe_workspace_bytes(c, at) - lm.lmoe_workspace_bytes(c, at - 1)
        step = lm.lmoe_workspace_bytes(c, at + 1) - lm.lmoe_workspace_bytes(c, at)
        assert jump > 5 * step, (t0, jump, step)
    bad = lm.make_config(2560, 1792, 512, 10, 640, 640, "bf16", "bf16", "mxfp4", 1, -2)
    n = ctypes.c_size_t(0)
    assert lm.lib.lmoe_workspace_bytes(ctypes.byref(bad), 8, ctypes.byref(n)) == lm.LMOE_ERR_SHAPE
