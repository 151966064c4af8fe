"""3D rotary position embedding with a rolling sink position (float64 oracle).

Pages cited:
  NOTES = papernotes.org, "Live Avatar: Streaming Real-time Audio-Driven Avatar
          Generation with Infinite Length"
  POP   = admirer.cn popular article on Live Avatar, section on the rolling
          sink frame mechanism (RSFM)
  BLOG  = gitcode.csdn.net, "Live Avatar 深度解析：首个 14B 参数实时流式无限时长数字人"

NOTES, 关键设计 3 (Rolling RoPE): the sink frame's temporal RoPE offset is
adjusted so that its relative distance to the active block stays constant.
POP (RSFM section, second design): the sink's position is always the current
position plus a fixed offset.  BLOG, 疑问 5: after the one-time replacement
only the sink's position encoding changes.

The pages say "RoPE" without its axes, bands or base.  Reading taken here
(the conventional 3D factorisation of a video DiT's RoPE): head_dim d is cut
into three contiguous bands for the (frame, height, width) axes of widths
(d - 4*floor(d/6), 2*floor(d/6), 2*floor(d/6)); inside a band of width d_a,
dims (2k, 2k+1) form pair k, rotated by the angle p_a * theta**(-2k/d_a)
with theta = 10000 and p_a the token's coordinate on that axis:
(x, y) -> (x cos a - y sin a, x sin a + y cos a).
"""

from __future__ import annotations

import numpy as np

DEFAULT_THETA = 10000.0


def band_split(head_dim: int):
    """Widths of the (frame, height, width) bands of head_dim."""
    if head_dim <= 0 or head_dim % 2:
        raise ValueError("head_dim must be a positive even number")
    s = head_dim // 6
    t = head_dim - 4 * s
    if t <= 0 or t % 2:
        raise ValueError("head_dim gives an empty or odd frame band")
    return (t, 2 * s, 2 * s)


def band_frequencies(head_dim: int, theta: float = DEFAULT_THETA):
    """Per-band arrays of rotation frequencies theta**(-2k/d_a), k = 0..d_a/2-1."""
    return tuple(theta ** (-2.0 * np.arange(w // 2, dtype=np.float64) / w)
                 for w in band_split(head_dim))


def token_positions(n_frames: int, Hl: int, Wl: int, f0: int):
    """(frame, h, w) coordinates of the tokens of n_frames latent frames.

    Tokens are ordered frame-major, then h, then w: token (j*Hl + h)*Wl + w is
    at temporal position f0 + j and spatial position (h, w).
    """
    j, h, w = np.meshgrid(np.arange(n_frames), np.arange(Hl), np.arange(Wl), indexing="ij")
    return (f0 + j.reshape(-1)).astype(np.float64), h.reshape(-1).astype(np.float64), \
        w.reshape(-1).astype(np.float64)


def _rotate_pairs(x: np.ndarray, angles: np.ndarray) -> np.ndarray:
    """Rotate adjacent pairs of the last axis of x ([T, H, 2P]) by angles ([T, P])."""
    xe = x[..., 0::2]
    xo = x[..., 1::2]
    c = np.cos(angles)[:, None, :]
    s = np.sin(angles)[:, None, :]
    out = np.empty_like(x)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


def rope3d(x: np.ndarray, n_frames: int, Hl: int, Wl: int, f0: int,
           theta: float = DEFAULT_THETA) -> np.ndarray:
    """Rotate x ([n_frames*Hl*Wl, heads, head_dim]) at positions (f0+j, h, w), float64.

    Used for a block's Q and K at f0 = f0(b) and for the raw sink K (one
    frame) at f0 = f0(b) + delta.  V is never rotated.
    """
    x = np.asarray(x, dtype=np.float64)
    T, H, d = x.shape
    if T != n_frames * Hl * Wl:
        raise ValueError("token count does not match n_frames*Hl*Wl")
    pf, ph, pw = token_positions(n_frames, Hl, Wl, f0)
    out = np.empty_like(x)
    start = 0
    for pos, freqs, width in zip((pf, ph, pw), band_frequencies(d, theta), band_split(d)):
        angles = pos[:, None] * freqs[None, :]
        out[..., start:start + width] = _rotate_pairs(x[..., start:start + width], angles)
        start += width
    return out
