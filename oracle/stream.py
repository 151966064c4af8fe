"""One layer of the streaming timestep-forcing stage, block after block (oracle).

Pages cited:
  NOTES = papernotes.org, "Live Avatar: Streaming Real-time Audio-Driven Avatar
          Generation with Infinite Length"
  NEWS  = 10100.com, "连续直播上万秒不崩脸！阿里开源Live Avatar …"
  POP   = admirer.cn popular article on Live Avatar
  BLOG  = gitcode.csdn.net, "Live Avatar 深度解析：首个 14B 参数实时流式无限时长数字人"

Per block b (1-based) on one stage t_i -> t_{i-1}, for one attention layer:
  1. rotate the block's Q and K at temporal positions f0(b) + j, j = 0, 1, 2
     (NOTES 整体框架: a block is 3 latent frames), and the raw sink K at
     f0(b) + delta (NOTES 关键设计 3, POP RSFM section: sink position = current
     position + fixed offset);
  2. attend over [rotated sink | cached blocks | the block itself]
     (NOTES 整体框架 and 关键设计 2);
  3. append the block's rotated K and V, computed from this stage's own noisy
     input, to the window (BLOG 疑问 4; NEWS 方法概述; no clean refresh);
  4. after block 1 only: replace the sink once (NOTES 关键设计 3; BLOG 疑问 5).

Variants for the pages' ablations (NOTES, Table 4 and the Table 6 finding):
  rolling=False : the sink K keeps one fixed position, frame 0 (where the
                  reference frame sits), instead of following the block;
  aas=False     : the sink is never replaced (the input image stays the sink);
  cache_layer=c : the window's K/V and the sink belong to another stream c that
                  writes the cache (a clean-refresh pass, or the one stage of a
                  fixed-noise cache); this stream only attends to it.

Readings taken where the pages are silent: f0(b) = 3 (b - 1); delta = -1 (the
sink sits one latent frame before the block's first frame, where the
reference frame sits at block 1 if it is frame 0 of the video, and it stays
there relative to every later block); with no trained model, the
replacement sink is the first latent frame (first Hl*Wl tokens) of block 1's
raw K and V of the same layer.
"""

from __future__ import annotations

from typing import Iterable, Optional, Sequence

import numpy as np

from .attention import attention_lse
from .cache import Ring, Sink
from .rope import DEFAULT_THETA, rope3d

SINK_DELTA = -1
SINK_FIXED_POSITION = 0  # the sink's own frame when Rolling RoPE is off


def block_f0(block: int, frames_per_block: int = 3) -> int:
    """Temporal position of block ``block``'s first latent frame (1-based blocks)."""
    return frames_per_block * (block - 1)


class StreamOracle:
    """Float64 reference for one streamed layer.

    ``shape`` is a ``seeded_inputs.LayerShape`` (only its sizes and its input
    generators are used); ``heads`` restricts every computation to a subset
    of heads (attention is independent per head).
    """

    def __init__(self, shape, layer: int = 0, heads: Optional[Sequence[int]] = None,
                 theta: float = DEFAULT_THETA, delta: int = SINK_DELTA,
                 noise_level: float = 0.75, rolling: bool = True, aas: bool = True,
                 cache_layer: Optional[int] = None):
        self.shape = shape
        self.layer = layer
        self.rolling = rolling
        self.aas = aas
        self.cache_layer = layer if cache_layer is None else cache_layer
        self.heads = list(range(shape.heads)) if heads is None else list(heads)
        self.theta = theta
        self.delta = delta
        self.noise_level = noise_level
        self.scale = 1.0 / np.sqrt(shape.head_dim)

    # ---- inputs (float64 values of the stored bits), restricted to self.heads
    def raw_block(self, block: int, layer: Optional[int] = None):
        q, k, v = self.shape.block_inputs(self.layer if layer is None else layer, block)
        hs = self.heads
        return q.values[:, hs, :], k.values[:, hs, :], v.values[:, hs, :]

    def initial_sink(self):
        """The sink of the stream that owns the cache."""
        sk, sv = self.shape.initial_sink(self.cache_layer)
        return sk.values[:, self.heads, :], sv.values[:, self.heads, :]

    def replacement_sink(self):
        """Block 1's first latent frame of raw K and V of the cache owner (the AAS stand-in)."""
        _, k, v = self.raw_block(1, self.cache_layer)
        n = self.shape.sink_tokens
        return k[:n].copy(), v[:n].copy()

    # ---- step 1
    def rot_block(self, x: np.ndarray, block: int) -> np.ndarray:
        s = self.shape
        return rope3d(x, s.frames_per_block, s.Hl, s.Wl, block_f0(block, s.frames_per_block),
                      self.theta)

    def sink_position(self, block: int) -> int:
        if not self.rolling:
            return SINK_FIXED_POSITION
        return block_f0(block, self.shape.frames_per_block) + self.delta

    def rot_sink(self, k_raw: np.ndarray, block: int) -> np.ndarray:
        s = self.shape
        return rope3d(k_raw, 1, s.Hl, s.Wl, self.sink_position(block), self.theta)

    # ---- the window a block sees, straight from its definition
    def window_ids(self, block: int):
        """Blocks cached when block ``block`` attends: the last min(b-1, W)."""
        return list(range(max(1, block - self.shape.W), block))

    def sink_for(self, block: int):
        if block == 1 or not self.aas:
            return self.initial_sink()
        return self.replacement_sink()

    def block_output(self, block: int, rows: Optional[np.ndarray] = None, with_lse=False):
        """Attention output of block ``block`` (optionally only some query rows)."""
        q_raw, k_raw, v = self.raw_block(block)
        q_rot = self.rot_block(q_raw, block)
        k_rot = self.rot_block(k_raw, block)
        sk_raw, sv = self.sink_for(block)
        keys = [self.rot_sink(sk_raw, block)]
        vals = [sv]
        for b2 in self.window_ids(block):
            _, k2, v2 = self.raw_block(b2, self.cache_layer)
            keys.append(self.rot_block(k2, b2))
            vals.append(v2)
        keys.append(k_rot)
        vals.append(v)
        qq = q_rot if rows is None else q_rot[rows]
        out, lse = attention_lse(qq, np.concatenate(keys), np.concatenate(vals), self.scale)
        return (out, lse) if with_lse else out

    # ---- the same stream run step by step with the Ring and Sink models
    def run(self, n_blocks: int, record: Iterable[int] = ()):
        """Process blocks 1..n_blocks in order; returns ({block: output}, ring, sink).
        Only for a stream that writes its own cache."""
        if self.cache_layer != self.layer:
            raise ValueError("run() models a stream that writes its own cache")
        record = set(record)
        ring = Ring(self.shape.W, self.noise_level)
        sink = Sink(*self.initial_sink())
        outs = {}
        for b in range(1, n_blocks + 1):
            q_raw, k_raw, v = self.raw_block(b)
            q_rot = self.rot_block(q_raw, b)
            k_rot = self.rot_block(k_raw, b)
            ck, cv = ring.keys_values()
            keys = np.concatenate([self.rot_sink(sink.k_raw, b), *ck, k_rot])
            vals = np.concatenate([sink.v, *cv, v])
            if b in record:
                outs[b] = attention_lse(q_rot, keys, vals, self.scale)[0]
            ring.append(b, k_rot, v, self.noise_level)
            if b == 1 and self.aas:
                n = self.shape.sink_tokens
                sink.replace(k_raw[:n], v[:n])
        return outs, ring, sink
