"""Seeded synthetic inputs shared by the CPU oracle side and the HIP side.

This module only draws numbers. It holds none of the all-reduce arithmetic
(no sums, no rounding to bfloat16, no packing), so neither side can borrow
the other's implementation through it.

Value recipes (workload shapes follow the tensor-parallel messages discussed
on "集合通信：NCCL 的算法、协议与推理框架的定制 all-reduce" (anrans.github.io,
serving/comm/nccl) and the hidden-8192 exercise on "多 GPU 与 NCCL"
(anrans.github.io, cuda/tools/multi-gpu, 练习 1)):

* ``normal_f32``  : ``Generator(PCG64(seed)).standard_normal(N, float32)``.
* ``integers_f32``: ``Generator(PCG64(seed)).integers(lo, hi, endpoint=True)``
  cast to float32 (exactly representable, so sums are exact in fp32).
* ``normal_bf16_bits``: the upper 16 bits of each ``normal_f32`` draw, i.e.
  the draw truncated toward zero to a bfloat16 pattern.  Truncation is used
  on purpose: it is a plain bit selection, not the round-to-nearest-even the
  method itself performs, so the generator shares no step with either side.
* ``fill_pattern_f32``: ``x[i] = g + i % 7`` for rank ``g`` -- the fill used
  by the single-process NCCL program on "多 GPU 与 NCCL" (NCCL 编程 section).

Seeds: ``seed = 1000 * config + rank`` unless a caller passes its own.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "rank_seed",
    "normal_f32",
    "integers_f32",
    "normal_bf16_bits",
    "fill_pattern_f32",
    "rank_inputs",
    "WORKLOADS",
]


def rank_seed(config: int, rank: int) -> int:
    """Seed of emulated rank ``rank`` in workload ``config``."""
    return 1000 * int(config) + int(rank)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(int(seed)))


def normal_f32(numel: int, seed: int) -> np.ndarray:
    """N(0,1) float32 draws."""
    return _rng(seed).standard_normal(int(numel), dtype=np.float32)


def integers_f32(numel: int, seed: int, lo: int = -8, hi: int = 8) -> np.ndarray:
    """Uniform integers in [lo, hi] (both ends included) stored as float32."""
    return _rng(seed).integers(lo, hi, size=int(numel), endpoint=True).astype(np.float32)


def normal_bf16_bits(numel: int, seed: int) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of N(0,1) draws truncated toward zero."""
    f = normal_f32(numel, seed)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def fill_pattern_f32(numel: int, g: int) -> np.ndarray:
    """``x[i] = g + i % 7`` as float32 (rank g's fill on the NCCL program page)."""
    i = np.arange(int(numel), dtype=np.int64)
    return (g + (i % 7)).astype(np.float32)


def rank_inputs(n: int, numel: int, dtype: str, kind: str, config: int) -> list:
    """Host arrays for ``n`` emulated ranks.

    ``dtype`` is ``"f32"`` (float32 arrays) or ``"bf16"`` (uint16 bit arrays).
    ``kind`` is ``"normal"``, ``"int"`` (U{-8..8}) or ``"fill"``.
    """
    out = []
    for r in range(n):
        seed = rank_seed(config, r)
        if kind == "normal":
            a = normal_f32(numel, seed) if dtype == "f32" else normal_bf16_bits(numel, seed)
        elif kind == "int":
            a = integers_f32(numel, seed)
            if dtype == "bf16":
                # small integers are exact in bfloat16: the pattern is the top half
                a = (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
        elif kind == "fill":
            a = fill_pattern_f32(numel, r)
            if dtype == "bf16":
                a = (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
        else:
            raise ValueError(f"unknown input kind {kind!r}")
        out.append(a)
    return out


# The five workloads, by what they are.  ``numel`` is per rank.
WORKLOADS = {
    "oneshot_n2_f32_int_4096": dict(config=0, algo="oneshot", n=2, dtype="f32", numel=4096, kind="int"),
    "oneshot_decode_n8_bf16_8x8192": dict(config=1, algo="oneshot", n=8, dtype="bf16", numel=8 * 8192, kind="normal"),
    "twoshot_prefill_n8_bf16_512x8192": dict(config=2, algo="twoshot", n=8, dtype="bf16", numel=512 * 8192, kind="normal"),
    "ll_n8_f32_64KiB": dict(config=3, algo="ll", n=8, dtype="f32", numel=16384, kind="normal"),
    "ll_n8_f32_1MiB": dict(config=3, algo="ll", n=8, dtype="f32", numel=262144, kind="normal"),
}
