// e4m3 encoding shared by the quantisation kernel and the RoPE kernel's e4m3
// output (device code only; included inside namespace la's anonymous namespace).
#pragma once

// e4m3 code of each float, round to nearest even (v_cvt_pk_fp8_f32) after
// clamping to +-448: the conversion instruction maps magnitudes that round past
// 448 to NaN, the quantisation saturates them.  A NaN becomes the NaN code of its
// sign, 0x7F / 0xFF (the clamp alone would turn it into -448).
__device__ __forceinline__ float clamp448(float x) { return fminf(fmaxf(x, -448.f), 448.f); }

__device__ __forceinline__ uint32_t nan_fix(uint32_t code, float x, int byte) {
  if (x == x) return code;
  const uint32_t nanc = 0x7Fu | ((__float_as_uint(x) >> 31) << 7);
  return (code & ~(0xFFu << (8 * byte))) | (nanc << (8 * byte));
}

__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(c), clamp448(d), w, true);
  uint32_t u = (uint32_t)w;
  u = nan_fix(u, a, 0);
  u = nan_fix(u, b, 1);
  u = nan_fix(u, c, 2);
  return nan_fix(u, d, 3);
}
