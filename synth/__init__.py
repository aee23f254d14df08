"""Seeded synthetic inputs for the Q4_0 matmul: the only code shared by the CPU
oracle's tests and the GPU path's tests and benchmark.

This module holds none of the method's arithmetic.  It draws raw inputs and
lays them out as bytes; it never decodes a weight, never multiplies, never
sums.  A GGUF Q4_0 block is written as 18 bytes: the scale d as an IEEE
binary16 value in little-endian order, then 16 bytes of packed 4-bit codes.
The 16 code bytes are drawn as uniform random bytes, so every 4-bit code is
an independent draw from U{0..15} whichever nibble the decoder assigns to
which weight: the generator does not need, and does not encode, the nibble
order.  Which nibble is which weight is fixed by the decoders (the oracle and
the kernels) and pinned by a hand-built worked example in the tests.

Workloads follow the sizes that the pages' models run (a 4B-class decoder
block, its FFN-up projection, its 151936-entry logit head, 512-position
prefill passes).  The pages measure on real GGUF checkpoints; none is here,
and these seeded draws stand in for them:
  d ~ U[0.001, 0.01] drawn in float64 and rounded to binary16 (round to
      nearest even, numpy's conversion); the rounded value is the truth,
  codes ~ U{0..15} i.i.d. (uniform random bytes),
  x ~ N(0, 1), float32, or rounded to binary16 for the prefill passes.
Each matrix draws from its own child of ``numpy.random.SeedSequence(seed)``
in a fixed order (scales, codes, activations).
"""
from __future__ import annotations

import dataclasses

import numpy as np

BLOCK_WEIGHTS = 32          # weights per Q4_0 block
BLOCK_BYTES = 18            # 2-byte binary16 scale + 16 code bytes
D_RANGE = (0.001, 0.01)


def blocks_bytes(out: int, in_: int) -> int:
    """Size in bytes of an [out x in] matrix stored as GGUF Q4_0 blocks."""
    return out * (in_ // BLOCK_WEIGHTS) * BLOCK_BYTES


def _children(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(n)]


def assemble_blocks(d_f16: np.ndarray, qs: np.ndarray) -> np.ndarray:
    """Lay out scales and code bytes as GGUF Q4_0 blocks.

    d_f16: float16 [out, nb] scales.  qs: uint8 [out, nb, 16] code bytes, used
    as given.  Returns uint8 [out, nb, 18]: bytes 0-1 are the scale's binary16
    bit pattern, little-endian; bytes 2-17 are the code bytes.
    """
    d_f16 = np.ascontiguousarray(d_f16, dtype=np.float16)
    out, nb = d_f16.shape
    assert qs.shape == (out, nb, 16) and qs.dtype == np.uint8
    blk = np.empty((out, nb, BLOCK_BYTES), dtype=np.uint8)
    bits = d_f16.view(np.uint16)
    blk[..., 0] = (bits & 0xFF).astype(np.uint8)
    blk[..., 1] = (bits >> 8).astype(np.uint8)
    blk[..., 2:] = qs
    return blk


def make_blocks(out: int, in_: int, seed: int = 0,
                d_range=D_RANGE) -> np.ndarray:
    """Random [out x in] Q4_0 matrix as uint8 [out, in/32, 18] blocks."""
    if in_ % BLOCK_WEIGHTS:
        raise ValueError(f"in={in_} is not a multiple of 32")
    nb = in_ // BLOCK_WEIGHTS
    g_d, g_q = _children(seed, 2)
    d = g_d.uniform(d_range[0], d_range[1], size=(out, nb)).astype(np.float16)
    qs = g_q.integers(0, 256, size=(out, nb, 16), dtype=np.uint8)
    return assemble_blocks(d, qs)


def make_x(n: int, in_: int, seed: int = 0, dtype=np.float32) -> np.ndarray:
    """Activations x [n x in] ~ N(0,1), float32 or rounded to float16."""
    g = _children(seed, 3)[2]
    x = g.standard_normal(size=(n, in_), dtype=np.float64)
    return x.astype(np.float32).astype(dtype)


def constant_blocks(out: int, in_: int, d_bits: int, code_byte: int) -> np.ndarray:
    """Every block holds the scale bit pattern ``d_bits`` and every code byte
    equals ``code_byte`` (so both nibbles of a byte hold the same code when
    the byte is 0x88, 0x99, ...)."""
    nb = in_ // BLOCK_WEIGHTS
    d = np.full((out, nb), d_bits, dtype=np.uint16).view(np.float16)
    qs = np.full((out, nb, 16), code_byte, dtype=np.uint8)
    return assemble_blocks(d, qs)


@dataclasses.dataclass(frozen=True)
class Linear:
    name: str
    out: int
    in_: int


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    linears: tuple
    ns: tuple
    x_dtype: str           # "f32" or "f16"
    description: str


# The workloads: one small GEMV, a 4B-class block's FFN-up projection, the
# whole block's seven projections batched over n tokens, two 512-position
# prefill passes (FFN-up, then FFN-down on an independent activation), and a
# 151936-row logit head.
WORKLOADS = {
    "gemv_1024": Workload(
        "gemv_1024", (Linear("w", 1024, 1024),), (1,), "f32",
        "single Q4_0 GEMV, 1024x1024, n=1"),
    "ffn_up_decode": Workload(
        "ffn_up_decode", (Linear("up", 9728, 2560),), (1,), "f32",
        "decode GEMV, FFN-up 9728x2560, n=1"),
    "block_decode": Workload(
        "block_decode",
        (Linear("q", 4096, 2560), Linear("k", 1024, 2560),
         Linear("v", 1024, 2560), Linear("o", 2560, 4096),
         Linear("gate", 9728, 2560), Linear("up", 9728, 2560),
         Linear("down", 2560, 9728)),
        (1, 2, 4, 8), "f32",
        "batched decode over the 7 projections of a 4B-class block"),
    "prefill": Workload(
        "prefill", (Linear("up", 9728, 2560), Linear("down", 2560, 9728)),
        (512,), "f16",
        "prefill GEMM, 512 positions, fp16 x: FFN-up then FFN-down"),
    "logit_head": Workload(
        "logit_head", (Linear("head", 151936, 2560),), (1, 4), "f32",
        "logit head 151936x2560, n in {1,4}"),
}


def seed_for(workload: str, linear_index: int, base: int = 0) -> int:
    """Seed of one matrix of a workload: ``base`` for the first matrix, then
    consecutive integers, so every matrix of a workload draws independently."""
    return base + linear_index
