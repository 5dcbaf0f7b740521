"""Seeded synthetic weights for the codec's workloads.

This module only draws inputs: it holds none of the codec's arithmetic, and
both the product path and the CPU oracle are fed from it by the callers
(tests, benchmark).  No dataset or trained checkpoint is used; the shapes
and distributions stand in for real LLM weights:

* a 1,048,576-element BF16 tensor drawn from N(0, 0.02^2);
* one Llama-3-8B-shaped transformer block (q, k, v, o, gate, up, down), with
  entries N(0, s^2), s ~ U[0.01, 0.04] per matrix -- the unit that
  the DFloat11 digest decompresses as one batch (section "Descompressao por
  bloco de transformer");
* the same block quantised per layer to uint8, either unsigned or asymmetric
  with a shifted zero point (the EntroLLM summary, "Metodologia": mixed
  tensor-level quantisation), the choice drawn from the seed;
* 32 such BF16 blocks (the whole 8B weight set);
* one Llama-3.1-405B-shaped block with Student-t (nu = 3) entries scaled to
  std 0.02, a heavy-tailed stress case.

Random streams: ``numpy.random.Generator(PCG64(SeedSequence(key)))``.  The
per-matrix parameters come first from key (seed, config, block); entries are
drawn in chunks of 2^24 elements, chunk c of matrix m from key
(seed, config, block, m, c), so the values do not depend on memory limits or
on how many threads draw them.  float32 draws are rounded to BF16 by
round-to-nearest-even on the float32 bit pattern.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 24

# (name, rows, cols) in the order the block is concatenated
LLAMA3_8B_BLOCK = (
    ("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
    ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336),
)
LLAMA31_405B_BLOCK = (
    ("q", 16384, 16384), ("k", 1024, 16384), ("v", 1024, 16384), ("o", 16384, 16384),
    ("gate", 53248, 16384), ("up", 53248, 16384), ("down", 16384, 53248),
)

# one large matrix on its own: the Llama-3-8B LM head (vocabulary x hidden)
LLAMA3_8B_LM_HEAD = (("lm_head", 128256, 4096),)

CONFIG_C1, CONFIG_8B_BF16, CONFIG_8B_U8, CONFIG_8B_FULL, CONFIG_405B, CONFIG_LM_HEAD, CONFIG_FORWARD, \
    CONFIG_8B_U4 = 1, 2, 3, 4, 5, 6, 7, 8


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _gen(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bit patterns (uint16), round to nearest even.  The
    inputs here are finite, so no NaN handling is needed."""
    b = np.ascontiguousarray(x, np.float32).view(np.uint32)
    return ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def scaled_shapes(shapes, div: int):
    """The same block with every dimension divided by div (for small tests)."""
    return tuple((n, max(1, r // div), max(1, c // div)) for n, r, c in shapes)


def _fill(out: np.ndarray, key, dist: str, scale: float, to_bf16: bool):
    n = out.size
    chunks = [(c, c * CHUNK, min(n, (c + 1) * CHUNK)) for c in range((n + CHUNK - 1) // CHUNK)]

    def work(ch):
        c, lo, hi = ch
        g = _gen(*key, c)
        if dist == "normal":
            x = g.standard_normal(hi - lo, dtype=np.float32) * np.float32(scale)
        elif dist == "t3":
            x = (g.standard_t(3, hi - lo) * scale).astype(np.float32)
        else:
            raise ValueError(dist)
        out[lo:hi] = bf16_rne(x) if to_bf16 else x

    if len(chunks) == 1:
        work(chunks[0])
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(work, chunks))


def c1_tensor(seed: int = 0, n: int = 1 << 20) -> np.ndarray:
    """One BF16 tensor, N(0, 0.02^2)."""
    out = np.empty(n, np.uint16)
    _fill(out, (seed, CONFIG_C1, 0, 0), "normal", 0.02, True)
    return out


def bf16_block(seed: int = 0, config: int = CONFIG_8B_BF16, block: int = 0,
               shapes=LLAMA3_8B_BLOCK, dist: str = "normal", out: np.ndarray | None = None):
    """A transformer block of BF16 weights, matrices flattened row-major and
    concatenated in q, k, v, o, gate, up, down order.

    dist "normal": N(0, s^2), s ~ U[0.01, 0.04] per matrix.
    dist "t3": Student-t(3) * 0.02 / sqrt(3) (std 0.02) for every matrix.
    Returns (uint16 array, [(name, offset, rows, cols), ...])."""
    g = _gen(seed, config, block)
    scales = [float(g.uniform(0.01, 0.04)) if dist == "normal" else 0.02 / np.sqrt(3.0)
              for _ in shapes]
    total = sum(r * c for _, r, c in shapes)
    if out is None:
        out = np.empty(total, np.uint16)
    assert out.size >= total and out.dtype == np.uint16
    index, off = [], 0
    for m, ((name, r, c), s) in enumerate(zip(shapes, scales)):
        _fill(out[off: off + r * c], (seed, config, block, m), dist, s, True)
        index.append((name, off, r, c))
        off += r * c
    return out[:total], index


def quantize_u8(x: np.ndarray, asymmetric: bool) -> np.ndarray:
    """Per-tensor uint8 quantisation of one layer (the EntroLLM summary,
    "Metodologia", names unsigned and asymmetric quantisation; the formulas are
    this repository's plain reading):
      unsigned:   s = max|x| / 127,          q = clamp(rint(x / s) + 128, 0, 255)
      asymmetric: s = (max - min) / 255,     zp = clamp(rint(-min / s), 0, 255),
                  q = clamp(rint(x / s) + zp, 0, 255)
    rint rounds half to even; arithmetic in float32."""
    x = np.asarray(x, np.float32)
    if x.size == 0:
        return np.zeros(0, np.uint8)
    if asymmetric:
        lo, hi = np.float32(x.min()), np.float32(x.max())
        s = np.float32((hi - lo) / np.float32(255))
        s = s if s > 0 else np.float32(1)       # a constant layer
        zp = np.clip(np.rint(-lo / s), 0, 255)
        q = np.rint(x / s) + zp
    else:
        s = np.float32(np.abs(x).max() / np.float32(127))
        s = s if s > 0 else np.float32(1)
        q = np.rint(x / s) + np.float32(128)
    return np.clip(q, 0, 255).astype(np.uint8)


def u8_block(seed: int = 0, config: int = CONFIG_8B_U8, block: int = 0, shapes=LLAMA3_8B_BLOCK):
    """The EntroLLM-style block: per layer, kind ~ Bernoulli(1/2) (0 unsigned,
    1 asymmetric) and s ~ U[0.01, 0.04], then N(0, s^2) weights quantised to
    uint8.  Returns [(name, uint8 array, asymmetric), ...]."""
    g = _gen(seed, config, block)
    params = [(int(g.integers(0, 2)), float(g.uniform(0.01, 0.04))) for _ in shapes]
    layers = []
    for m, ((name, r, c), (asym, s)) in enumerate(zip(shapes, params)):
        x = np.empty(r * c, np.float32)
        _fill(x, (seed, config, block, m), "normal", s, False)
        layers.append((name, quantize_u8(x, bool(asym)), bool(asym)))
    return layers


def quantize_u4(x: np.ndarray, asymmetric: bool) -> np.ndarray:
    """Per-tensor uint4 quantisation of one layer, the 4-bit counterpart of
    quantize_u8 (same reading, 16 levels), one value 0..15 per byte:
      unsigned:   s = max|x| / 7,            q = clamp(rint(x / s) + 8, 0, 15)
      asymmetric: s = (max - min) / 15,      zp = clamp(rint(-min / s), 0, 15),
                  q = clamp(rint(x / s) + zp, 0, 15)"""
    x = np.asarray(x, np.float32)
    if x.size == 0:
        return np.zeros(0, np.uint8)
    if asymmetric:
        lo, hi = np.float32(x.min()), np.float32(x.max())
        s = np.float32((hi - lo) / np.float32(15))
        s = s if s > 0 else np.float32(1)
        zp = np.clip(np.rint(-lo / s), 0, 15)
        q = np.rint(x / s) + zp
    else:
        s = np.float32(np.abs(x).max() / np.float32(7))
        s = s if s > 0 else np.float32(1)
        q = np.rint(x / s) + np.float32(8)
    return np.clip(q, 0, 15).astype(np.uint8)


def pack_u4(q: np.ndarray) -> np.ndarray:
    """Values 0..15 -> packed bytes, element 2j in the low nibble of byte j
    (input layout of the uint4 kind)."""
    q = np.asarray(q, np.uint8).reshape(-1)
    if q.size % 2:
        q = np.concatenate([q, np.zeros(1, np.uint8)])
    return (q[0::2] | (q[1::2] << 4)).astype(np.uint8)


def unpack_u4(packed: np.ndarray, n: int) -> np.ndarray:
    """Packed bytes -> n values 0..15."""
    b = np.asarray(packed, np.uint8).reshape(-1)
    out = np.empty(2 * b.size, np.uint8)
    out[0::2] = b & 0x0F
    out[1::2] = b >> 4
    return out[:n]


def u4_block(seed: int = 0, config: int = CONFIG_8B_U4, block: int = 0, shapes=LLAMA3_8B_BLOCK):
    """The EntroLLM-style 4-bit block: as u8_block, quantised to uint4 and
    packed two per byte.  Returns [(name, packed uint8 array, n, asymmetric), ...]."""
    g = _gen(seed, config, block)
    params = [(int(g.integers(0, 2)), float(g.uniform(0.01, 0.04))) for _ in shapes]
    layers = []
    for m, ((name, r, c), (asym, s)) in enumerate(zip(shapes, params)):
        x = np.empty(r * c, np.float32)
        _fill(x, (seed, config, block, m), "normal", s, False)
        layers.append((name, pack_u4(quantize_u4(x, bool(asym))), r * c, bool(asym)))
    return layers


def block_elems(shapes=LLAMA3_8B_BLOCK) -> int:
    return sum(r * c for _, r, c in shapes)
