"""Seeded synthetic inputs for one decode-step MoE layer.

Every tensor is drawn from its own NumPy PCG64 stream keyed by
``SeedSequence([seed, tag, tensor_id, index])`` so that a tensor (or one
expert of it, or one token of the activations) can be regenerated on its own
and in parallel.

Distributions (the standard deviation is the second parameter of N):
  hidden, residual  N(0, 1)            -> bf16 (round to nearest even)
  router weight     N(0, 1/sqrt(H))    -> bf16
  w13, shared w13   N(0, 1/sqrt(H))    -> fp8 e4m3fn with 128x128 block scales
  w2,  shared w2    N(0, 1/sqrt(I))    -> fp8 e4m3fn with 128x128 block scales
  gamma             1 + N(0, 0.1)      -> bf16
  router bias       N(0, bias_std) f32 (only when asked for)

Block quantisation (encoding of the inputs, not part of the layer):
  fp32 scales : s = fp32(amax / 448), 1 where amax == 0
  e8m0 scales : s = 2**ceil(log2(amax / 448)), stored as the byte e + 127
  codes       : q = e4m3fn(round-to-nearest-even(w / s)), saturated to +-448

bf16 values are carried as uint16 bit patterns, fp8 values as uint8 codes and
e8m0 scales as uint8 exponent bytes, the same bytes the device receives.
"""

from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np
import torch

# Tensor ids for the seed key.
_HIDDEN, _RESIDUAL, _ROUTER, _W13, _W2, _SW13, _SW2, _GAMMA, _BIAS = range(1, 10)

FP8_MAX = 448.0
BLOCK = 128


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """Sizes and constants of one MoE layer step."""

    T: int  # tokens in the step
    H: int  # hidden size
    E: int  # routed experts
    k: int  # experts per token
    I: int  # routed expert intermediate size
    Is: int  # shared expert intermediate size (0: no shared expert)
    scale_fmt: str = "fp32"  # "fp32" or "e8m0"
    limit: float = 7.0  # swiglu_limit
    rsf: float = 2.5  # routed_scaling_factor
    eps: float = 1e-5  # RMSNorm epsilon
    tag: int = 100  # seed key of the workload

    def replace(self, **kw) -> "LayerShape":
        return dataclasses.replace(self, **kw)


# The five workloads: a tiny correctness layer, the decode layer at 1 and 16
# tokens, the wide layer at 64 tokens with power-of-two scales and the
# speculative-verify batch of 128 tokens (32 requests x 4) with fp32 scales.
WORKLOADS = {
    "tiny_t1": LayerShape(T=1, H=256, E=8, k=2, I=128, Is=128, scale_fmt="fp32", tag=0),
    "decode_t1": LayerShape(T=1, H=4096, E=128, k=8, I=1536, Is=1536, scale_fmt="fp32", tag=1),
    "decode_t16": LayerShape(T=16, H=4096, E=128, k=8, I=1536, Is=1536, scale_fmt="fp32", tag=2),
    "wide_t64_e8m0": LayerShape(T=64, H=6144, E=256, k=8, I=2048, Is=2048, scale_fmt="e8m0", tag=3),
    "verify_t128": LayerShape(T=128, H=6144, E=256, k=8, I=2048, Is=2048, scale_fmt="fp32", tag=4),
    # a dense layer's MLP (no routed experts; the MLP in the shared-expert
    # slot) at the decode hidden size, intermediate 2 x hidden (the library's
    # largest): a synthetic choice, the pages give no dense-layer sizes
    "dense_t1": LayerShape(T=1, H=4096, E=0, k=0, I=0, Is=8192, scale_fmt="fp32", tag=5),
    "dense_t16": LayerShape(T=16, H=4096, E=0, k=0, I=0, Is=8192, scale_fmt="fp32", tag=6),
}
WORKLOAD_ORDER = ["tiny_t1", "decode_t1", "decode_t16", "wide_t64_e8m0", "verify_t128"]


@dataclasses.dataclass
class LayerInputs:
    """Host copies of every input of one layer step, as device bytes."""

    shape: LayerShape
    hidden: np.ndarray  # [T,H] uint16 (bf16 bits)
    residual: np.ndarray  # [T,H] uint16
    router_w: np.ndarray  # [E,H] uint16
    router_bias: Optional[np.ndarray]  # [E] float32 or None
    w13: np.ndarray  # [E,2I,H] uint8 (e4m3fn codes); rows [0,I) gate, [I,2I) up
    w13_scale: np.ndarray  # [E,2I/128,H/128] float32 or uint8 (e8m0)
    w2: np.ndarray  # [E,H,I] uint8
    w2_scale: np.ndarray  # [E,H/128,I/128]
    sw13: Optional[np.ndarray]  # [2Is,H] uint8
    sw13_scale: Optional[np.ndarray]  # [2Is/128,H/128]
    sw2: Optional[np.ndarray]  # [H,Is] uint8
    sw2_scale: Optional[np.ndarray]  # [H/128,Is/128]
    gamma: np.ndarray  # [H] uint16


def _rng(seed: int, tag: int, tensor: int, index: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, tensor, index])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of float32 values, rounded to nearest even (torch's cast)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _f32_to_e4m3_codes(a: np.ndarray) -> np.ndarray:
    """e4m3fn codes of float32 values already inside [-448, 448] (torch's RNE cast)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def quantize_blocks(w: np.ndarray, scale_fmt: str):
    """128x128 block quantisation of a float32 matrix [R, C] into e4m3fn codes.

    Returns (codes uint8 [R, C], scales [R/128, C/128]) with float32 scales
    (amax/448) or uint8 e8m0 exponent bytes (2**ceil(log2(amax/448))).
    """
    R, C = w.shape
    assert R % BLOCK == 0 and C % BLOCK == 0, (R, C)
    b = w.reshape(R // BLOCK, BLOCK, C // BLOCK, BLOCK)
    amax = np.abs(b).max(axis=(1, 3))
    if scale_fmt == "fp32":
        s = (amax / np.float32(FP8_MAX)).astype(np.float32)
        s[amax == 0] = 1.0
        stored = s
    elif scale_fmt == "e8m0":
        ratio = amax.astype(np.float64) / FP8_MAX
        mant, ex = np.frexp(ratio)  # ratio = mant * 2**ex, mant in [0.5, 1)
        e = np.where(mant == 0.5, ex - 1, ex)  # ceil(log2(ratio))
        e = np.where(amax == 0, 0, e)
        e = np.clip(e, -127, 127)
        stored = (e + 127).astype(np.uint8)
        s = np.ldexp(np.float32(1.0), e).astype(np.float32)
    else:
        raise ValueError(scale_fmt)
    q = b / s[:, None, :, None]
    np.clip(q, -FP8_MAX, FP8_MAX, out=q)
    return _f32_to_e4m3_codes(q.reshape(R, C)), stored


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    a *= np.float32(std)
    return a


def _threads() -> int:
    env = os.environ.get("SYNTH_THREADS")
    if env:
        return max(1, int(env))
    return max(1, min(16, os.cpu_count() or 1))


def make_layer(shape: LayerShape, seed: int = 0, with_bias: bool = False,
               bias_std: float = 0.05, threads: Optional[int] = None) -> LayerInputs:
    """Draw every input of one layer step (see the module docstring)."""
    T, H, E, I, Is = shape.T, shape.H, shape.E, shape.I, shape.Is
    for n in (H, I) + ((Is,) if Is else ()):
        assert n % BLOCK == 0, "H, I and Is must be multiples of 128"
    tag, fmt = shape.tag, shape.scale_fmt
    sdt = np.float32 if fmt == "fp32" else np.uint8

    hidden = np.empty((T, H), np.uint16)
    residual = np.empty((T, H), np.uint16)
    for t in range(T):
        hidden[t] = f32_to_bf16_bits(_normal(_rng(seed, tag, _HIDDEN, t), H, 1.0))
        residual[t] = f32_to_bf16_bits(_normal(_rng(seed, tag, _RESIDUAL, t), H, 1.0))
    router_w = f32_to_bf16_bits(_normal(_rng(seed, tag, _ROUTER, 0), (E, H), 1.0 / np.sqrt(H)))
    gamma = f32_to_bf16_bits(1.0 + _normal(_rng(seed, tag, _GAMMA, 0), H, 0.1))
    bias = None
    if with_bias:
        bias = _normal(_rng(seed, tag, _BIAS, 0), E, bias_std).astype(np.float32)

    w13 = np.empty((E, 2 * I, H), np.uint8)
    w13_scale = np.empty((E, 2 * I // BLOCK, H // BLOCK), sdt)
    w2 = np.empty((E, H, I), np.uint8)
    w2_scale = np.empty((E, H // BLOCK, I // BLOCK), sdt)

    def expert(e):
        w = _normal(_rng(seed, tag, _W13, e), (2 * I, H), 1.0 / np.sqrt(H))
        w13[e], w13_scale[e] = quantize_blocks(w, fmt)
        del w
        w = _normal(_rng(seed, tag, _W2, e), (H, I), 1.0 / np.sqrt(I))
        w2[e], w2_scale[e] = quantize_blocks(w, fmt)

    with ThreadPoolExecutor(threads or _threads()) as ex:
        list(ex.map(expert, range(E)))

    sw13 = sw13_scale = sw2 = sw2_scale = None
    if Is:
        sw13, sw13_scale = quantize_blocks(
            _normal(_rng(seed, tag, _SW13, 0), (2 * Is, H), 1.0 / np.sqrt(H)), fmt)
        sw2, sw2_scale = quantize_blocks(
            _normal(_rng(seed, tag, _SW2, 0), (H, Is), 1.0 / np.sqrt(Is)), fmt)
    return LayerInputs(shape, hidden, residual, router_w, bias, w13, w13_scale, w2,
                       w2_scale, sw13, sw13_scale, sw2, sw2_scale, gamma)


def make_layer_from_arrays(shape: LayerShape, **arrays) -> LayerInputs:
    """A LayerInputs from explicit arrays (hand-built examples); missing
    optional tensors default to None."""
    fields = {f.name: None for f in dataclasses.fields(LayerInputs)}
    fields.update(arrays)
    fields["shape"] = shape
    return LayerInputs(**fields)


def tokens_subset(inp: LayerInputs, rows) -> LayerInputs:
    """The same layer with only the listed token rows of the activations."""
    rows = np.asarray(rows)
    return dataclasses.replace(inp, shape=inp.shape.replace(T=len(rows)),
                               hidden=np.ascontiguousarray(inp.hidden[rows]),
                               residual=np.ascontiguousarray(inp.residual[rows]))
