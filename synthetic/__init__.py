"""Seeded synthetic inputs shared by the oracle side and the device side.

This module only draws numbers and packs them; it contains none of the
attention or bank arithmetic.  Both the CPU oracle (through the tests) and the
HIP path consume exactly the bytes produced here, so a parity comparison is
always on identical inputs.

Recipe (one stream per tensor, no stream is ever reused):

    numpy.random.Generator(PCG64(SeedSequence([seed, kind, layer, idx, stage, tensor])))
    -> standard_normal in float64 -> float32 -> (bf16 configs) bf16 by
       round-to-nearest-even of the float32 bit pattern.

kind   : 0 = renderer chunk input, 1 = anchor (planner cache-extraction output),
         2 = planner block input during its denoising steps
idx    : chunk id for kind 0, anchor id for kind 1, planner block for kind 2
stage  : denoising stage for kind 0, always 0 for kind 1, step for kind 2
tensor : 0 = Q, 1 = K, 2 = V, 3 = dO (output gradient of a backward pass)

Every tensor is token-major ``[tokens, n_heads, head_dim]``.
bf16 tensors are returned as ``uint16`` bit patterns; ``bf16_bits_to_f32``
widens them exactly.
"""
from __future__ import annotations

import numpy as np

KIND_RENDER = 0
KIND_ANCHOR = 1
KIND_PLANNER = 2
TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_DO = 0, 1, 2, 3


def _stream(seed: int, kind: int, layer: int, idx: int, stage: int, tensor: int) -> np.random.Generator:
    ss = np.random.SeedSequence([int(seed), int(kind), int(layer), int(idx), int(stage), int(tensor)])
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return uint16 bits.

    Inputs here are finite normal draws, so no NaN/Inf special-casing is needed.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_tensor(shape, *, seed: int, kind: int, layer: int, idx: int, stage: int, tensor: int,
                  dtype: str = "bf16", scale: float = 1.0) -> np.ndarray:
    """One seeded N(0, scale^2) tensor.  bf16 -> uint16 bits, f32 -> float32."""
    x = _stream(seed, kind, layer, idx, stage, tensor).standard_normal(size=tuple(shape))
    x = (x * scale).astype(np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of a generated tensor (bf16 bits or float32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def chunk_qkv(*, T: int, n_heads: int, head_dim: int, chunk: int, stage: int, seed: int = 0,
              layer: int = 0, chunk_latents: int = 3, dtype: str = "bf16", q_scale: float = 1.0):
    """Q, K, V of renderer chunk ``chunk`` at stage ``stage``: each [chunk_latents*T, nh, d]."""
    shape = (chunk_latents * T, n_heads, head_dim)
    kw = dict(seed=seed, kind=KIND_RENDER, layer=layer, idx=chunk, stage=stage, dtype=dtype)
    q = normal_tensor(shape, tensor=TENSOR_Q, scale=q_scale, **kw)
    k = normal_tensor(shape, tensor=TENSOR_K, **kw)
    v = normal_tensor(shape, tensor=TENSOR_V, **kw)
    return q, k, v


def anchor_kv(*, T: int, n_heads: int, head_dim: int, anchors, seed: int = 0, layer: int = 0,
              dtype: str = "bf16"):
    """K, V for a run of anchors, concatenated along tokens: each [len(anchors)*T, nh, d]."""
    ks, vs = [], []
    for a in anchors:
        kw = dict(seed=seed, kind=KIND_ANCHOR, layer=layer, idx=int(a), stage=0, dtype=dtype)
        ks.append(normal_tensor((T, n_heads, head_dim), tensor=TENSOR_K, **kw))
        vs.append(normal_tensor((T, n_heads, head_dim), tensor=TENSOR_V, **kw))
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)


def planner_qkv(*, T: int, n_heads: int, head_dim: int, block: int, step: int, n_latents: int, seed: int = 0,
                layer: int = 0, dtype: str = "bf16", q_scale: float = 1.0):
    """Q, K, V of planner block ``block`` at denoising step ``step``: each [n_latents*T, nh, d]."""
    shape = (n_latents * T, n_heads, head_dim)
    kw = dict(seed=seed, kind=KIND_PLANNER, layer=layer, idx=block, stage=step, dtype=dtype)
    q = normal_tensor(shape, tensor=TENSOR_Q, scale=q_scale, **kw)
    k = normal_tensor(shape, tensor=TENSOR_K, **kw)
    v = normal_tensor(shape, tensor=TENSOR_V, **kw)
    return q, k, v


def clip_tensors(*, T: int, n_heads: int, head_dim: int, n_chunks: int, stage: int = 0, seed: int = 0,
                 layer: int = 0, chunk_latents: int = 3, dtype: str = "bf16", q_scale: float = 1.0,
                 chunks=None):
    """Q, K, V, dO of a whole clip at one stage, chunk after chunk: each [n_chunks*chunk_latents*T, nh, d].

    Chunk i's Q, K, V are the renderer inputs of (chunk i, stage) (kind 0), so
    the clip equals the per-chunk inputs laid end to end; dO is tensor 3 of
    the same stream family.  ``chunks`` limits generation to those chunks (the
    other rows are zero).
    """
    L = chunk_latents * T
    shape = (L, n_heads, head_dim)
    out_dtype = np.uint16 if dtype == "bf16" else np.float32
    out = [np.zeros((n_chunks * L, n_heads, head_dim), dtype=out_dtype) for _ in range(4)]
    for i in (range(n_chunks) if chunks is None else chunks):
        kw = dict(seed=seed, kind=KIND_RENDER, layer=layer, idx=int(i), stage=stage, dtype=dtype)
        for t, (dst, scale) in enumerate(zip(out, (q_scale, 1.0, 1.0, 1.0))):
            dst[i * L:(i + 1) * L] = normal_tensor(shape, tensor=t, scale=scale, **kw)
    return tuple(out)
