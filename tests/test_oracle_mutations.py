"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a copy of the oracle's source (a dropped term, a
wrong sign or index, a transposed operand, a wrong constant, a missing rounding), loads the
copy as a module of its own, and runs every pin in test_oracle_pins against it.  The pins
pass on the real oracle (that file's own tests); here each planted mistake must make at least
one of them fail.  Nothing is changed in the real oracle module: the copy is a separate module
object that the pins see in place of it for the duration of one case.
"""
from __future__ import annotations

import importlib.util
import itertools
import os
import types

import pytest

import test_oracle_pins as pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "lmoe_oracle.py")

# (name, function whose body is edited or None for the whole file, text, replacement)
MUTANTS = [
    ("router bias dropped", "router_logits", "return logits + br[None, :]", "return logits"),
    ("router reads group 0's latent", "router_logits", "z[:, g * L:(g + 1) * L] @", "z[:, 0:L] @"),
    ("exact ties go to the higher id", "route", 'order = np.argsort(-logits, axis=1, kind="stable")',
     'order = logits.shape[1] - 1 - np.argsort(-logits[:, ::-1], axis=1, kind="stable")'),
    ("slots in score order, not ascending id", "route", "chosen = np.sort(order[:, :k], axis=1)",
     "chosen = order[:, :k]"),
    ("largest logit skipped", "route", "chosen = np.sort(order[:, :k], axis=1)",
     "chosen = np.sort(order[:, 1:k + 1], axis=1)"),
    ("gap taken one place early", "route", "gap = srt[:, k - 1] - srt[:, k]", "gap = srt[:, k - 2] - srt[:, k - 1]"),
    ("softmax over all experts, not renormalised", "route", "w = e / e.sum(axis=1, keepdims=True)",
     "w = e / np.exp(logits - lam.max(axis=1, keepdims=True)).sum(axis=1, keepdims=True)"),
    ("permutation not stable inside a segment", "permute", 'perm = np.argsort(flat, kind="stable")',
     'perm = flat.size - 1 - np.argsort(flat[::-1], kind="stable")'),
    ("offsets are the inclusive sum", "permute", "offsets[1:] = np.cumsum(counts)", "offsets[:-1] = np.cumsum(counts)"),
    ("inverse permutation is the permutation", "permute", "inv[perm] = np.arange(flat.size)", "inv[:] = perm"),
    ("SiLU with the wrong sign", "silu", "return v / (1.0 + np.exp(-v))", "return v / (1.0 + np.exp(v))"),
    ("SiLU on the up branch", "swiglu", "return (silu(z @ gate.T) * (z @ up.T)) @ down.T",
     "return ((z @ gate.T) * silu(z @ up.T)) @ down.T"),
    ("down read as stored [ffn][latent]", "swiglu", "return (silu(z @ gate.T) * (z @ up.T)) @ down.T",
     "return (silu(z @ gate.T) * (z @ up.T)) @ down.reshape(gate.shape[0], -1)"),
    ("D read as stored [hidden][latent]", "block_forward", "z = x @ layer.D.T", "z = x @ layer.D.reshape(x.shape[1], -1)"),
    ("shared expert missing", "block_forward", "m[:, :L] += swiglu(z[:, :L], *layer.shared)", "m[:, :L] += 0.0"),
    ("shared expert in the last group", "block_forward", "m[:, :L] += swiglu(z[:, :L], *layer.shared)",
     "m[:, (G - 1) * L:] += swiglu(z[:, (G - 1) * L:], *layer.shared)"),
    ("routing weight squared", "block_forward", "m[t, c:c + L] += w[t, slot] * swiglu(",
     "m[t, c:c + L] += w[t, slot] ** 2 * swiglu("),
    ("wrong expert group", "block_forward", "c = (e // Eg) * L", "c = (e % G) * L"),
    ("U read as stored [latent][hidden]", "block_forward", "y = m @ layer.U.T", "y = m @ layer.U.reshape(m.shape[1], -1)"),
    ("forced ids left in the given order", "block_forward", "fid = np.sort(np.asarray(fid, dtype=np.int64))",
     "fid = np.asarray(fid, dtype=np.int64)"),
    ("forced tokens keep the router's weights", "block_forward", "w[t] = ee / ee.sum()", "w[t] = w[t]"),
    ("forced weights from the first token's logits", "block_forward", "lam = logits[t, fid]", "lam = logits[0, fid]"),
    ("RMSNorm without epsilon", "rmsnorm", "np.mean(h * h, axis=1, keepdims=True) + eps",
     "np.mean(h * h, axis=1, keepdims=True)"),
    ("RMSNorm over the sum of squares", "rmsnorm", "np.mean(h * h", "np.sum(h * h"),
    ("stack residual subtracted", "stack_step", 'out["h_next"] = (h + out["y"])', 'out["h_next"] = (h - out["y"])'),
    ("stack residual not rounded to fp32", "stack_step",
     'out["h_next"] = (h + out["y"]).astype(np.float32).astype(np.float64)', 'out["h_next"] = (h + out["y"])'),
    ("stack block input not normalised", "stack_step", "x = round_to_bf16(rmsnorm(h))", "x = round_to_bf16(h)"),
    ("bf16 rounding through float32 first", "round_to_bf16", "v = np.asarray(v, dtype=np.float64)",
     "v = np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)"),
    ("bf16 rounding to 7 significant bits", "round_to_bf16", "np.maximum(e - 8, -133)", "np.maximum(e - 7, -133)"),
    ("bf16 decode shifted by 15", "bf16_to_f64", "<< np.uint32(16)", "<< np.uint32(15)"),
    ("E2M1 largest magnitude 5", None, "E2M1_VALUES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)",
     "E2M1_VALUES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 5.0)"),
    ("MXFP4 nibbles high first", "mxfp4_decode", "codes[:, 0::2] = nib & 0x0F\n    codes[:, 1::2] = nib >> 4",
     "codes[:, 1::2] = nib & 0x0F\n    codes[:, 0::2] = nib >> 4"),
    ("E8M0 bias 126", "mxfp4_decode", ".astype(np.int64) - 127", ".astype(np.int64) - 126"),
    ("E4M3 exponent bias 8", "e4m3_decode", "np.ldexp(1.0, e - 10)", "np.ldexp(1.0, e - 11)"),
    ("NVFP4 tensor scale ignored", "nvfp4_decode", "* float(tensor_scale)", "* 1.0"),
    ("NVFP4 scale per 32 values", "nvfp4_decode", "np.repeat(sc, 16, axis=1)", "np.repeat(sc[:, ::2], 32, axis=1)"),
]


def _function_span(src: str, name: str) -> tuple[int, int]:
    start = src.index(f"\ndef {name}(") + 1
    nxt = [i for i in (src.find("\ndef ", start), src.find("\nclass ", start)) if i >= 0]
    return start, (min(nxt) + 1 if nxt else len(src))


def mutant_module(func: str | None, old: str, new: str) -> types.ModuleType:
    with open(ORACLE_SRC) as f:
        src = f.read()
    a, b = _function_span(src, func) if func else (0, len(src))
    body = src[a:b]
    assert body.count(old) == 1, f"the planted text must occur once in {func or 'the oracle'}: {old!r}"
    src = src[:a] + body.replace(old, new) + src[b:]
    spec = importlib.util.spec_from_loader("oracle_mutant", loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


def pin_cases():
    """(name, callable) for every pin in test_oracle_pins, parametrized ones expanded."""
    out = []
    for name in sorted(dir(pins)):
        fn = getattr(pins, name)
        if not (name.startswith("test_") and callable(fn)):
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not marks:
            out.append((name, fn, {}))
            continue
        grids = []
        for m in marks:
            argnames = [a.strip() for a in m.args[0].split(",")] if isinstance(m.args[0], str) else list(m.args[0])
            vals = [v if len(argnames) > 1 else (v,) for v in m.args[1]]
            grids.append([dict(zip(argnames, v)) for v in vals])
        for combo in itertools.product(*grids):
            kw = {}
            for d in combo:
                kw.update(d)
            out.append((f"{name}{kw}", fn, kw))
    return out


def test_every_pin_passes_on_the_real_oracle_module():
    # the harness itself: with the unmodified source loaded the same way, every pin passes
    real = mutant_module(None, "def silu(", "def silu(")
    saved = pins.oracle
    try:
        pins.oracle = real
        for name, fn, kw in pin_cases():
            fn(**kw)
    finally:
        pins.oracle = saved


@pytest.mark.parametrize("name,func,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(name, func, old, new):
    mod = mutant_module(func, old, new)
    saved = pins.oracle
    caught = None
    try:
        pins.oracle = mod
        for pin, fn, kw in pin_cases():
            try:
                fn(**kw)
            except Exception as e:  # an assertion or an error raised by the planted mistake
                caught = (pin, type(e).__name__)
                break
    finally:
        pins.oracle = saved
    assert caught is not None, f"no pin fails with the planted mistake '{name}'"
    print(f"'{name}' fails {caught[0]} ({caught[1]})")
