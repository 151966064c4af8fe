"""Rolling noisy KV cache and the once-replaced attention sink (oracle models).

Pages cited:
  NOTES = papernotes.org, "Live Avatar: Streaming Real-time Audio-Driven Avatar
          Generation with Infinite Length"
  NEWS  = 10100.com, "连续直播上万秒不崩脸！阿里开源Live Avatar …", 方法概述
  BLOG  = gitcode.csdn.net, "Live Avatar 深度解析：首个 14B 参数实时流式无限时长数字人"

Ring: BLOG, 疑问 1 (history context lives in a rolling KV cache over the most
recent frames) and 疑问 4 (Live Avatar drops the clean-cache refresh and
stores the K/V of the step's own noisy x_t; the cache's noise level is forced
to equal the current latent's).  NEWS, 方法概述 (Stage 2 keeps the KV cache and
the noisy latents at one noise level).  NOTES, 关键设计 2 (History Corrupt: no
clean refresh; the cache keeps noisy representations) and 关键设计 4 (each TPP
GPU keeps its own local noisy sliding cache for its fixed step).
Reading taken: a FIFO window of the last W blocks; block b (1-based) is
appended after its own attention into physical slot (b - 1) mod W, evicting
block b - W when b > W; every entry carries the stage's noise level t_i and
an append at any other level is refused.

Sink: NOTES, 关键设计 3 (AAS: after the first block is generated, the model's
own first latent replaces the input reference as the permanent sink) and
BLOG, 疑问 5 (the anchor is updated exactly once, after the first block;
afterwards only its position encoding changes).
"""

from __future__ import annotations

import collections
from typing import Optional

import numpy as np


class RingStateError(RuntimeError):
    """An append or replacement that the cache rules refuse."""


class Ring:
    """Last-W-blocks window of (block_id, noise level, K_rot, V)."""

    def __init__(self, W: int, noise_level: float):
        if W < 1:
            raise ValueError("window must hold at least one block")
        self.W = W
        self.noise_level = float(noise_level)
        self._entries = collections.deque(maxlen=W)
        self.last_block = 0

    @staticmethod
    def slot_of(block_id: int, W: int) -> int:
        return (block_id - 1) % W

    def append(self, block_id: int, k: np.ndarray, v: np.ndarray,
               noise_level: float) -> Optional[int]:
        """Append block ``block_id``; returns the evicted block id or None."""
        if block_id != self.last_block + 1:
            raise RingStateError(f"block {block_id} out of order (last {self.last_block})")
        if float(noise_level) != self.noise_level:
            raise RingStateError("noise level differs from the cache's (timestep forcing)")
        evicted = self._entries[0][0] if len(self._entries) == self.W else None
        self._entries.append((block_id, self.noise_level, np.array(k), np.array(v)))
        self.last_block = block_id
        return evicted

    def ids(self):
        """Cached block ids, oldest first."""
        return [e[0] for e in self._entries]

    def noise_levels(self):
        return [e[1] for e in self._entries]

    def slots(self):
        """Physical slot -> block id for the cached blocks."""
        return {self.slot_of(b, self.W): b for b in self.ids()}

    def entry(self, block_id: int):
        for e in self._entries:
            if e[0] == block_id:
                return e[2], e[3]
        raise KeyError(block_id)

    def keys_values(self):
        """Cached K and V, oldest first, as lists of arrays."""
        return [e[2] for e in self._entries], [e[3] for e in self._entries]

    def __len__(self):
        return len(self._entries)


class Sink:
    """Raw (unrotated) sink K and V, replaceable exactly once."""

    def __init__(self, k_raw: np.ndarray, v: np.ndarray):
        self.k_raw = np.array(k_raw)
        self.v = np.array(v)
        self.replaced = False

    def replace(self, k_new_raw: np.ndarray, v_new: np.ndarray) -> None:
        if self.replaced:
            raise RingStateError("the sink has already been replaced once")
        if k_new_raw.shape != self.k_raw.shape or v_new.shape != self.v.shape:
            raise ValueError("replacement sink has a different shape")
        self.k_raw = np.array(k_new_raw)
        self.v = np.array(v_new)
        self.replaced = True
