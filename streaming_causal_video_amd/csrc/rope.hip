// 3D RoPE with a rolling sink position, for gfx950.
//
// Rolling RoPE (papernotes.org "Live Avatar: Streaming Real-time Audio-Driven
// Avatar Generation with Infinite Length", 关键设计 3; admirer.cn article, RSFM
// section): the block's Q and K are rotated at (f0 + j, h, w) and the raw sink K
// at (f0 + delta, h, w), so the sink keeps a constant temporal distance to the
// active block.  head_dim is cut into (frame, h, w) bands; pair k of a band of
// width w_a turns by p * theta^(-2k/w_a).
//
// The kernel is HBM-bound (16 B read + 16 B written per 16 B chunk).  One
// workgroup walks a few tokens of one tensor; each thread owns one 16-byte
// chunk position inside a head row, looks up the cos/sin of the pairs in that
// chunk once per token (frame rows come by value from the host, spatial rows
// from a small float32 table that stays in cache), and then rotates that chunk
// for every head it is assigned.  No per-element integer division.
#include "la_internal.h"

namespace la {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to bf16 (round-to-nearest-even, v_cvt_pk_bf16_f32) and pack.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2_t f = {lo, hi};
  bf16x2_t b = __builtin_convertvector(f, bf16x2_t);
  return __builtin_bit_cast(uint32_t, b);
}

constexpr int kThreads = 256;

template <bool kBF16>
__global__ __launch_bounds__(kThreads) void rope3d_kernel(RopeTensor t0, RopeTensor t1,
                                                          RopeTensor t2, RopeGeom g,
                                                          RopeTemporal tc,
                                                          const float* __restrict__ table,
                                                          int tok_per_wg) {
  constexpr int kPPC = kBF16 ? 4 : 2;  // pairs per 16-byte chunk
  const RopeTensor T = blockIdx.y == 0 ? t0 : (blockIdx.y == 1 ? t1 : t2);
  if (T.in == nullptr) return;
  const int tok_begin = blockIdx.x * tok_per_wg;
  if (tok_begin >= T.tokens) return;
  const int cpr = g.head_dim / (2 * kPPC);  // chunks per head row
  const int hpb = kThreads / cpr;           // heads covered per pass
  const int ch = threadIdx.x % cpr;
  const int hoff = threadIdx.x / cpr;
  if (hoff >= hpb) return;
  const int tok_end = min(tok_begin + tok_per_wg, T.tokens);
  const int hw_pairs = g.tpairs + g.hpairs;
  const float* wtab = table + 2 * g.Hl * g.hpairs;

  for (int tok = tok_begin; tok < tok_end; ++tok) {
    const int frame = tok / g.HW;
    const int rem = tok - frame * g.HW;
    const int h = rem / g.Wl;
    const int w = rem - h * g.Wl;
    float cs[kPPC], sn[kPPC];
#pragma unroll
    for (int i = 0; i < kPPC; ++i) {
      const int gp = ch * kPPC + i;
      if (gp < g.tpairs) {
        cs[i] = tc.cs[T.trow0 + frame][gp][0];
        sn[i] = tc.cs[T.trow0 + frame][gp][1];
      } else if (gp < hw_pairs) {
        const float* e = table + 2 * (h * g.hpairs + (gp - g.tpairs));
        cs[i] = e[0];
        sn[i] = e[1];
      } else {
        const float* e = wtab + 2 * (w * g.wpairs + (gp - hw_pairs));
        cs[i] = e[0];
        sn[i] = e[1];
      }
    }
    const size_t row0 = (size_t)tok * g.heads;
    for (int head = hoff; head < g.heads; head += hpb) {
      const size_t off = (row0 + head) * (size_t)g.head_dim + (size_t)ch * 2 * kPPC;
      if constexpr (kBF16) {
        const uint4 x = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(T.in) + off);
        const uint32_t xin[4] = {x.x, x.y, x.z, x.w};
        uint32_t yout[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = bf_lo(xin[i]), b = bf_hi(xin[i]);
          yout[i] = pack_bf16(fmaf(a, cs[i], -b * sn[i]), fmaf(a, sn[i], b * cs[i]));
        }
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(T.out) + off) =
            make_uint4(yout[0], yout[1], yout[2], yout[3]);
      } else {
        const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(T.in) + off);
        float4 y;
        y.x = fmaf(x.x, cs[0], -x.y * sn[0]);
        y.y = fmaf(x.x, sn[0], x.y * cs[0]);
        y.z = fmaf(x.z, cs[1], -x.w * sn[1]);
        y.w = fmaf(x.z, sn[1], x.w * cs[1]);
        *reinterpret_cast<float4*>(static_cast<float*>(T.out) + off) = y;
      }
    }
  }
}

// Spatial cos/sin: [Hl][hpairs][2] then [Wl][wpairs][2]; float64 math, float32 store.
__global__ void rope_table_kernel(float* __restrict__ table, int Hl, int Wl, int hpairs,
                                  int wpairs, int hw, double theta) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int nh = Hl * hpairs, n = nh + Wl * wpairs;
  if (i >= n) return;
  int pos, k;
  if (i < nh) {
    pos = i / hpairs;
    k = i - pos * hpairs;
  } else {
    pos = (i - nh) / wpairs;
    k = (i - nh) - pos * wpairs;
  }
  const double freq = pow(theta, -2.0 * (double)k / (double)hw);
  const double a = (double)pos * freq;
  table[2 * i] = (float)cos(a);
  table[2 * i + 1] = (float)sin(a);
}

}  // namespace

hipError_t launch_rope(const RopeTensor* t, int nt, const RopeGeom& g, const RopeTemporal& tc,
                       const float* table, la_dtype dt, hipStream_t s) {
  RopeTensor tt[3] = {};
  int max_tokens = 0;
  for (int i = 0; i < nt && i < 3; ++i) {
    tt[i] = t[i];
    if (t[i].in && t[i].tokens > max_tokens) max_tokens = t[i].tokens;
  }
  if (max_tokens == 0) return hipSuccess;
  const int tok_per_wg = 4;
  dim3 grid((max_tokens + tok_per_wg - 1) / tok_per_wg, 3);
  if (dt == LA_BF16)
    hipLaunchKernelGGL(rope3d_kernel<true>, grid, dim3(kThreads), 0, s, tt[0], tt[1], tt[2], g,
                       tc, table, tok_per_wg);
  else
    hipLaunchKernelGGL(rope3d_kernel<false>, grid, dim3(kThreads), 0, s, tt[0], tt[1], tt[2], g,
                       tc, table, tok_per_wg);
  return hipGetLastError();
}

hipError_t launch_rope_table(float* table, int Hl, int Wl, int hpairs, int wpairs, int hw,
                             double theta, hipStream_t s) {
  const int n = Hl * hpairs + Wl * wpairs;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, s, table, Hl, Wl,
                     hpairs, wpairs, hw, theta);
  return hipGetLastError();
}

}  // namespace la
