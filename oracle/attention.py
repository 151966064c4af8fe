"""Block attention over {sink, rolling noisy cache, the block itself} (float64 oracle).

Pages cited:
  NOTES = papernotes.org, "Live Avatar: Streaming Real-time Audio-Driven Avatar
          Generation with Infinite Length"
  POP   = admirer.cn popular article on Live Avatar, two-stage training section
  BLOG  = gitcode.csdn.net, "Live Avatar 深度解析：首个 14B 参数实时流式无限时长数字人"

NOTES, 整体框架: the model advances one block of 3 latent frames at a time
under causal attention, with a static reference (sink) frame and a sliding
KV cache.  POP: a block may look at earlier blocks, never at later ones.
Reading taken: at inference one block is denoised at a time, so causality
is already given by which keys exist; inside the block attention is
bidirectional (the block is denoised jointly), so no mask is applied.  The
output is plain softmax attention, O = softmax(s * Q K^T) V with
s = 1/sqrt(head_dim), over the concatenated keys, per head.
"""

from __future__ import annotations

import numpy as np


def attention_lse(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                  row_chunk: int = 512):
    """Softmax attention per head in float64; returns (out, lse).

    q: [Nq, H, d]; k, v: [Nk, H, d] (keys in any order).
    out: [Nq, H, d]; lse: [H, Nq], natural-log sum of exp(scale * q.k) per row.
    Scores are materialised ``row_chunk`` query rows at a time.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Nq, H, d = q.shape
    Nk = k.shape[0]
    if k.shape != (Nk, H, d) or v.shape != (Nk, H, d):
        raise ValueError("q, k, v shapes disagree")
    if Nk == 0:
        raise ValueError("attention needs at least one key")
    out = np.empty((Nq, H, d), dtype=np.float64)
    lse = np.empty((H, Nq), dtype=np.float64)
    for h in range(H):
        kh = k[:, h, :]
        vh = v[:, h, :]
        for r0 in range(0, Nq, row_chunk):
            s = scale * (q[r0:r0 + row_chunk, h, :] @ kh.T)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            denom = p.sum(axis=1, keepdims=True)
            out[r0:r0 + row_chunk, h, :] = (p @ vh) / denom
            lse[h, r0:r0 + row_chunk] = (m + np.log(denom))[:, 0]
    return out, lse


def attention(q, k, v, scale: float, row_chunk: int = 512) -> np.ndarray:
    """Softmax attention output only; see attention_lse."""
    return attention_lse(q, k, v, scale, row_chunk)[0]
