"""Seeded synthetic inputs shared by the fp64 oracle, the tests and the bench.

This module is the only code that both the CPU oracle and the HIP path's
tests use.  It draws random numbers and rounds them to the storage types the
kernels read; it contains none of the method's arithmetic (no RoPE, no
attention, no cache logic, no flow update).

Recipe (stands in for the pages' GenBench evaluation videos, which need a
trained 14B model and are not available): every tensor is i.i.d. N(0, 1),
drawn in float64 from ``numpy.random.SeedSequence([1234, cfg, layer, entry,
tid])`` and rounded to the kernel's storage type with round-to-nearest-even.
Both sides receive exactly these bits.  Long streams (hundreds of blocks at
full size) cycle through a pool of seeded block entries so that host-side
generation stays bounded; block ``b`` uses entry ``(b - 1) % pool``.
"""

from __future__ import annotations

import dataclasses
import functools
from typing import Optional, Tuple

import numpy as np

ROOT_SEED = 1234

# tensor ids used as the last SeedSequence word
TID_Q, TID_K, TID_V, TID_SINK_K, TID_SINK_V, TID_X, TID_VEL = range(7)


def gaussian(key: Tuple[int, ...], shape) -> np.ndarray:
    """i.i.d. N(0,1) float64 array for a seed key (a tuple of non-negative ints)."""
    ss = np.random.SeedSequence([ROOT_SEED, *[int(k) for k in key]])
    return np.random.Generator(np.random.PCG64(ss)).standard_normal(shape)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 with round-to-nearest-even (single rounding).

    bfloat16 keeps 8 significant bits.  With x = m * 2**e, 0.5 <= |m| < 1,
    the value m * 2**8 lies in [128, 256) and ``np.rint`` rounds it half to
    even; the rounded value times 2**(e-8) is exact in float64 and in float32,
    so its float32 bit pattern shifted right by 16 is the bfloat16 pattern.
    Intended for the normal range of the synthetic data (no NaN/inf inputs);
    values that round to 2**128 or more saturate to inf.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    r = np.rint(m * 256.0)
    y = np.ldexp(r, e - 8)
    with np.errstate(over="ignore"):
        y32 = y.astype(np.float32)
    return (y32.view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of bfloat16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


@dataclasses.dataclass(frozen=True)
class Stored:
    """A synthetic tensor as the kernels store it and as the oracle reads it."""

    storage: np.ndarray  # uint16 bf16 bit patterns, or float32 (read-only)
    dtype: str           # "bf16" or "f32"

    @property
    def values(self) -> np.ndarray:
        """float64, exactly the stored values."""
        if self.dtype == "bf16":
            return bf16_bits_to_f64(self.storage)
        return self.storage.astype(np.float64)


def make_stored(x64: np.ndarray, dtype: str) -> Stored:
    if dtype == "bf16":
        s = f64_to_bf16_bits(x64)
    elif dtype == "f32":
        s = np.asarray(x64, dtype=np.float64).astype(np.float32)
    else:
        raise ValueError(f"unknown dtype {dtype!r}")
    s.flags.writeable = False
    return Stored(s, dtype)


@functools.lru_cache(maxsize=96)
def _tensor_cached(cfg_id, layer, entry, tid, shape, dtype, scale) -> Stored:
    x = gaussian((cfg_id, layer, entry, tid), shape)
    if scale != 1.0:
        x = x * scale
    return make_stored(x, dtype)


def tensor(cfg_id: int, layer: int, entry: int, tid: int, shape, dtype: str,
           scale: float = 1.0) -> Stored:
    """One seeded tensor, N(0,1) times ``scale``, rounded to ``dtype`` (memoised)."""
    return _tensor_cached(int(cfg_id), int(layer), int(entry), int(tid),
                          tuple(int(s) for s in shape), dtype, float(scale))


def clear_cache() -> None:
    _tensor_cached.cache_clear()


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """Shape of one streamed attention layer (tokens are frame-major, then h, then w)."""

    cfg_id: int
    dtype: str          # storage/compute type of Q/K/V: "bf16" or "f32"
    heads: int
    head_dim: int
    Hl: int             # latent frame height after patchify
    Wl: int             # latent frame width after patchify
    W: int              # ring window in blocks
    frames_per_block: int = 3
    layers: int = 1
    input_scale: float = 1.0
    pool: Optional[int] = None  # cycle block inputs through this many seeded entries

    @property
    def frame_tokens(self) -> int:
        return self.Hl * self.Wl

    @property
    def block_tokens(self) -> int:
        return self.frames_per_block * self.frame_tokens

    @property
    def sink_tokens(self) -> int:
        return self.frame_tokens

    def nk(self, block: int) -> int:
        """Keys seen by block ``block`` (1-based): sink + cached blocks + itself."""
        cached = min(block - 1, self.W)
        return self.sink_tokens + cached * self.block_tokens + self.block_tokens

    def entry(self, block: int) -> int:
        return (block - 1) % self.pool if self.pool else block

    def block_inputs(self, layer: int, block: int):
        """Raw (unrotated) Q, K, V of a block: each [block_tokens, heads, head_dim]."""
        shp = (self.block_tokens, self.heads, self.head_dim)
        e = self.entry(block)
        return tuple(tensor(self.cfg_id, layer, e, tid, shp, self.dtype, self.input_scale)
                     for tid in (TID_Q, TID_K, TID_V))

    def initial_sink(self, layer: int):
        """Raw sink K and V before the one-time replacement: [sink_tokens, heads, head_dim]."""
        shp = (self.sink_tokens, self.heads, self.head_dim)
        return tuple(tensor(self.cfg_id, layer, 0, tid, shp, self.dtype, self.input_scale)
                     for tid in (TID_SINK_K, TID_SINK_V))


# The five workloads.  Latent frames are 480x832 video -> 30x52 tokens and a
# 720p-shaped 44x80 token frame; blocks are three latent frames.
C1 = LayerShape(1, "f32", heads=2, head_dim=64, Hl=4, Wl=4, W=2)
C2 = LayerShape(2, "bf16", heads=40, head_dim=128, Hl=30, Wl=52, W=4)
C2_PRESCALED = dataclasses.replace(C2, cfg_id=12, input_scale=1.0 / np.sqrt(128.0))
C3 = LayerShape(3, "bf16", heads=40, head_dim=128, Hl=30, Wl=52, W=8, pool=16)
C4 = LayerShape(4, "bf16", heads=40, head_dim=128, Hl=30, Wl=52, W=4, layers=40, pool=4)
C5 = LayerShape(5, "bf16", heads=40, head_dim=128, Hl=44, Wl=80, W=4, pool=8)

# C4's latent: [channels, frames, height, width] fp32
C4_LATENT_SHAPE = (16, 3, 60, 104)

# Small layers for element-by-element parity: several tiles and ragged tails.
SMALL_BF16 = LayerShape(101, "bf16", heads=3, head_dim=128, Hl=5, Wl=7, W=2)
MID_BF16 = LayerShape(102, "bf16", heads=4, head_dim=128, Hl=12, Wl=13, W=3)
SMALL_F32 = LayerShape(103, "f32", heads=3, head_dim=64, Hl=5, Wl=7, W=3)
SMALL_F32_D128 = LayerShape(104, "f32", heads=2, head_dim=128, Hl=3, Wl=9, W=2)


def latent(cfg_id: int, block: int, tid: int, shape) -> Stored:
    """A seeded fp32 latent (TID_X) or velocity (TID_VEL)."""
    return tensor(cfg_id, 0, block, tid, shape, "f32")
