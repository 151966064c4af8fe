"""FP8 (e4m3) quantisation and the attention it feeds (TEST INFRASTRUCTURE).

The pages name FP8 quantisation, together with FlashAttention-3 and fused
kernels, as the operator-level step that took the pipeline from 20.88 to 45.20
FPS (papernotes.org "Live Avatar: Streaming Real-time Audio-Driven Avatar
Generation with Infinite Length", Table 3 / 推理效率与系统流水线消融).  They give
no format or scale convention; the reading here is the plainest one:

* the 8-bit format is E4M3 as in the OCP 8-bit floating point specification:
  1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; subnormals below
  2^-6 with quantum 2^-9; no infinities; the largest finite magnitude is
  1.75 * 2^8 = 448 and codes 0x7F / 0xFF are NaN;
* encoding rounds to the nearest representable value, ties to an even
  mantissa, and saturates: magnitudes beyond 448 become 448; the sign is kept,
  also when the value rounds to zero (-0 is code 0x80); a NaN becomes the NaN
  code of its sign (0x7F, or 0xFF with the sign bit set), the only codes the
  format reserves for NaN;
* a tensor is quantised with one per-tensor scale s: code = E4M3(x / s), and
  its value is decode(code) * s.

The attention of quantised tensors is then defined exactly: the ordinary
softmax attention of the decoded-and-rescaled Q, K and V.
"""

from __future__ import annotations

import numpy as np

from .attention import attention_lse

E4M3_MAX = 448.0
_BIAS = 7


def e4m3_decode(codes) -> np.ndarray:
    """float64 value of each e4m3 code (NaN for 0x7F and 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - _BIAS)
    sub = (m / 8.0) * 2.0 ** (1 - _BIAS)
    val = np.where(e == 0, sub, normal)
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return sign * val


def e4m3_encode(x) -> np.ndarray:
    """Nearest e4m3 code of each float64 value (ties to even mantissa), saturating
    at +-448; NaN gives the NaN code of its sign (0x7F / 0xFF)."""
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    a = np.minimum(np.abs(np.where(nan, 0.0, x)), E4M3_MAX)
    # exponent of the binade holding a, clamped to the subnormal binade at the bottom
    _, ex = np.frexp(a)  # a = f * 2^ex with 0.5 <= f < 1  (ex = 0 for a = 0)
    e = np.clip(ex - 1, 1 - _BIAS, 8)  # unbiased exponent, >= -6
    quantum = np.exp2(e - 3.0)  # spacing of representable values in that binade
    q = np.rint(a / quantum)  # exact division by a power of two; rint = ties to even
    # q in [8, 16] for normal binades (16 carries into the next binade), [0, 8] below 2^-6
    carry = q >= 16
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 8, q)
    normal = q >= 8
    code = np.where(normal, ((e + _BIAS).astype(np.int64) << 3) | (q.astype(np.int64) - 8),
                    q.astype(np.int64))
    code = np.where(nan, 0x7F, code)
    code = np.where(np.signbit(x), code | 0x80, code)  # the sign survives rounding to zero
    return code.astype(np.uint8)


def quantize(x, scale: float) -> np.ndarray:
    """Per-tensor quantisation: codes of x / scale, with the division done in float32
    (as the device does: it multiplies by the float32 reciprocal 1/scale, so the
    float32 product x * inv_scale is what gets rounded to e4m3)."""
    inv = np.float32(1.0) / np.float32(scale)
    prod = np.asarray(x, dtype=np.float32) * inv  # one float32 rounding
    return e4m3_encode(prod.astype(np.float64))


def dequantize(codes, scale: float) -> np.ndarray:
    return e4m3_decode(codes) * float(scale)


def attention_fp8(q8, k8, v8, sq: float, sk: float, sv: float, scale: float):
    """(out, lse) of softmax attention over the decoded, rescaled e4m3 tensors
    q8 [Nq, H, d], k8 / v8 [Nk, H, d] (exact float64)."""
    return attention_lse(dequantize(q8, sq), dequantize(k8, sk), dequantize(v8, sv), scale)
