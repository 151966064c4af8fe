// 3D RoPE with a rolling sink position, for gfx950.
//
// Rolling RoPE (papernotes.org "Live Avatar: Streaming Real-time Audio-Driven
// Avatar Generation with Infinite Length", 关键设计 3; admirer.cn article, RSFM
// section): the block's Q and K are rotated at (f0 + j, h, w) and the raw sink K
// at (f0 + delta, h, w), so the sink keeps a constant temporal distance to the
// active block.  head_dim is cut into (frame, h, w) bands; pair k of a band of
// width w_a turns by p * theta^(-2k/w_a).
//
// The kernel is HBM-bound (16 B read + 16 B written per 16 B chunk).  Each
// thread owns one 16-byte chunk position inside a head row, looks up the
// cos/sin of the pairs in that chunk once (frame rows come by value from the
// host, spatial rows from a small float32 table that stays in cache), and then
// rotates that chunk for every head it is assigned.  No per-element integer
// division.
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

#include "e4m3_dev.h"

constexpr int kThreads = 128;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// One workgroup rotates one token row (all heads) of one tensor.  Thread
// (hg, ch) owns 16-byte chunk ch of a head row and heads hg, hg + HG, ...
// (HG = head groups in the workgroup, kNH heads per pass).  Every load of the
// pass is issued, unpredicated (head indexes are clamped), before the first
// rotation, so a thread keeps kNH 16-byte loads in flight; only the stores are
// predicated.  The token is uniform, so addresses are a scalar row base plus a
// 32-bit lane offset.  Loads and stores are non-temporal: at a block's 224 MB the
// rotated tensors do not stay in the caches for the attention anyway (measured per
// C2-shaped call over buffers beyond the caches: 39.8 us against 42.6 us with
// ordinary stores, and no change inside the step).  Neither one workgroup per
// several rows nor more threads per row was faster (measured).  In-place calls are
// safe: a thread writes exactly the chunks it read.
//
// A tensor marked copy_only is copied as it is (the step stages the block's V in
// the ring's next slot within the same launch).  A tensor marked e4m3_out (bf16) is
// stored as e4m3 codes of its bf16 result times inv8, the arithmetic of the
// quantisation kernel (the e4m3 step rotates and quantises in one pass).
template <bool kBF16, int kNH>
__global__ __launch_bounds__(kThreads) void rope3d_kernel(RopeTensor t0, RopeTensor t1,
                                                          RopeTensor t2, RopeTensor t3,
                                                          RopeTensor t4, RopeGeom g,
                                                          RopeTemporal tc,
                                                          const float* __restrict__ table,
                                                          int wg0, int wg1, int wg2, int wg3) {
  constexpr int kPPC = kBF16 ? 4 : 2;  // pairs per 16-byte chunk
  constexpr int kEB = kBF16 ? 2 : 4;   // element bytes
  const int bid = __builtin_amdgcn_workgroup_id_x();
  const int tid = __builtin_amdgcn_workitem_id_x();
  const int e1 = wg0 + wg1, e2 = e1 + wg2, e3 = e2 + wg3;
  const int which = bid < wg0 ? 0 : (bid < e1 ? 1 : (bid < e2 ? 2 : (bid < e3 ? 3 : 4)));
  const RopeTensor T =
      which == 0 ? t0 : (which == 1 ? t1 : (which == 2 ? t2 : (which == 3 ? t3 : t4)));
  const int tok =
      bid - (which == 0 ? 0 : (which == 1 ? wg0 : (which == 2 ? e1 : (which == 3 ? e2 : e3))));
  const int cpr = g.head_dim / (2 * kPPC);  // chunks per head row
  const int hg_n = kThreads / cpr;          // head groups
  const int ch = tid % cpr;
  const int hg = tid / cpr;
  if (hg >= hg_n) return;

  const size_t row_bytes = (size_t)g.heads * g.head_dim * kEB;
  const char* src = static_cast<const char*>(T.in) + (size_t)tok * row_bytes;
  char* dst = static_cast<char*>(T.out) + (size_t)tok * row_bytes;
  // e4m3 output: one byte per element, 8 bytes per 16-byte input chunk
  char* dst8 = static_cast<char*>(T.out) + (size_t)tok * g.heads * g.head_dim;
  const bool to8 = kBF16 && T.e4m3_out;
  auto store8 = [&](int head, const u32x4_t& v) __attribute__((always_inline)) {
    const float inv = T.inv8;
    const uint32_t lo = e4m3x4(bf_lo(v[0]) * inv, bf_hi(v[0]) * inv, bf_lo(v[1]) * inv,
                               bf_hi(v[1]) * inv);
    const uint32_t hi = e4m3x4(bf_lo(v[2]) * inv, bf_hi(v[2]) * inv, bf_lo(v[3]) * inv,
                               bf_hi(v[3]) * inv);
    const uint32_t off = (uint32_t)(head * g.head_dim + ch * 2 * kPPC);
    typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
    __builtin_nontemporal_store(u32x2_t{lo, hi}, reinterpret_cast<u32x2_t*>(dst8 + off));
  };

  u32x4_t x[kNH];
  auto load_pass = [&](int h0) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kNH; ++k) {
      const int head = min(h0 + hg + k * hg_n, g.heads - 1);
      const uint32_t off = (uint32_t)(head * g.head_dim + ch * 2 * kPPC) * kEB;
      x[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + off));
    }
  };
  // The first pass's loads go out before the cos/sin lookups, so that one memory
  // latency covers both (the lookups' wait would otherwise come first).
  load_pass(0);
  if (T.copy_only) {
    for (int h0 = 0; h0 < g.heads; h0 += hg_n * kNH) {
      if (h0 > 0) load_pass(h0);
#pragma unroll
      for (int k = 0; k < kNH; ++k) {
        const int head = h0 + hg + k * hg_n;
        if (head < g.heads) {
          if (to8) {
            store8(head, x[k]);
          } else {
            const uint32_t off = (uint32_t)(head * g.head_dim + ch * 2 * kPPC) * kEB;
            __builtin_nontemporal_store(x[k], reinterpret_cast<u32x4_t*>(dst + off));
          }
        }
      }
    }
    return;
  }

  // cos/sin of this thread's kPPC pairs at (frame, h, w) of the token: the frame
  // band from the by-value rows, the h and w bands from the table (one load per
  // pair, index clamped so that every load is in bounds)
  const int frame = tok / g.HW;
  const int rem = tok - frame * g.HW;
  const int h = rem / g.Wl;
  const int w = rem - h * g.Wl;
  const int trow = T.trow0 + frame;
  const int hw_pairs = g.tpairs + g.hpairs;
  float cs[kPPC], sn[kPPC];
#pragma unroll
  for (int i = 0; i < kPPC; ++i) {
    const int gp = ch * kPPC + i;
    const int ti = min(gp, g.tpairs - 1);
    const int si = gp < hw_pairs ? h * g.hpairs + max(gp - g.tpairs, 0)
                                 : g.Hl * g.hpairs + w * g.wpairs + (gp - hw_pairs);
    const float2 e = *reinterpret_cast<const float2*>(table + 2 * si);
    const bool temporal = gp < g.tpairs;
    cs[i] = temporal ? tc.cs[trow][ti][0] : e.x;
    sn[i] = temporal ? tc.cs[trow][ti][1] : e.y;
  }
  // The token's cos/sin for a Q at the same positions (the step's bf16 attention
  // rotates its raw Q with them): times cs_scale, as the scaled rotation below
  // multiplies them (the product is exact for a scale of 1).
  if (T.cs_out != nullptr && hg == 0) {
    float e[2 * kPPC];
#pragma unroll
    for (int i = 0; i < kPPC; ++i) {
      e[2 * i] = cs[i] * T.cs_scale;
      e[2 * i + 1] = sn[i] * T.cs_scale;
    }
    float* dst_cs = T.cs_out + (size_t)tok * g.head_dim + ch * 2 * kPPC;
#pragma unroll
    for (int i = 0; i < 2 * kPPC; i += 4)
      *reinterpret_cast<f32x4_t*>(dst_cs + i) = f32x4_t{e[i], e[i + 1], e[i + 2], e[i + 3]};
  }
  // An output scale (the attention's score scale folded into Q) multiplies the
  // pair's cos/sin once per thread; with scale 1 the products are exact.
  if (T.scale != 1.0f) {
#pragma unroll
    for (int i = 0; i < kPPC; ++i) {
      cs[i] *= T.scale;
      sn[i] *= T.scale;
    }
  }

  for (int h0 = 0; h0 < g.heads; h0 += hg_n * kNH) {
    if (h0 > 0) load_pass(h0);
    // keep the loads together (the compiler would otherwise sink some of them,
    // and the rotations, into the predicated store blocks)
#pragma unroll
    for (int k = 0; k < kNH; ++k) asm volatile("" : "+v"(x[k]));
    u32x4_t y[kNH];
#pragma unroll
    for (int k = 0; k < kNH; ++k) {
      if constexpr (kBF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = bf_lo(x[k][i]), b = bf_hi(x[k][i]);
          y[k][i] = pack_bf16(fmaf(a, cs[i], -b * sn[i]), fmaf(a, sn[i], b * cs[i]));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const float a = __uint_as_float(x[k][2 * i]), b = __uint_as_float(x[k][2 * i + 1]);
          y[k][2 * i] = __float_as_uint(fmaf(a, cs[i], -b * sn[i]));
          y[k][2 * i + 1] = __float_as_uint(fmaf(a, sn[i], b * cs[i]));
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kNH; ++k) asm volatile("" : "+v"(y[k]));
    // stores after every rotation: a store between two waits on loads would make
    // the second wait cover the store as well (one in-order vector memory counter)
#pragma unroll
    for (int k = 0; k < kNH; ++k) {
      const int head = h0 + hg + k * hg_n;
      if (head < g.heads) {
        if (to8) {
          store8(head, y[k]);
        } else {
          const uint32_t off = (uint32_t)(head * g.head_dim + ch * 2 * kPPC) * kEB;
          __builtin_nontemporal_store(y[k], reinterpret_cast<u32x4_t*>(dst + off));
        }
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

template <bool kBF16>
static void launch_rope_nh(int nh, dim3 grid, hipStream_t s, const RopeTensor* tt,
                           const RopeGeom& g, const RopeTemporal& tc, const float* table,
                           const int* wg, const KernelTiming* tm) {
#define LA_ROPE_NH(N)                                                                        \
  case N:                                                                                    \
    launch_kernel(tm, rope3d_kernel<kBF16, N>, grid, dim3(kThreads), 0, s, tt[0], tt[1],     \
                  tt[2], tt[3], tt[4], g, tc, table, wg[0], wg[1], wg[2], wg[3]);            \
    break;
  switch (nh) {
    LA_ROPE_NH(1) LA_ROPE_NH(2) LA_ROPE_NH(3) LA_ROPE_NH(4)
    LA_ROPE_NH(5) LA_ROPE_NH(6) LA_ROPE_NH(7) default: LA_ROPE_NH(8)
  }
#undef LA_ROPE_NH
}

hipError_t launch_rope(const RopeTensor* t, int nt, const RopeGeom& g, const RopeTemporal& tc,
                       const float* table, la_dtype dt, hipStream_t s, const KernelTiming* tm) {
  RopeTensor tt[kMaxRopeTensors] = {};
  int wg[kMaxRopeTensors] = {};
  for (int i = 0; i < nt && i < kMaxRopeTensors; ++i) {
    tt[i] = t[i];
    if (t[i].in) wg[i] = t[i].tokens;
  }
  int total = 0;
  for (int i = 0; i < kMaxRopeTensors; ++i) total += wg[i];
  if (total == 0) return timing_without_kernel(tm, s);
  const int cpr = g.head_dim / (dt == LA_BF16 ? 8 : 4);
  const int hg_n = kThreads / cpr;
  const int nh = (g.heads + hg_n - 1) / hg_n;
  if (dt == LA_BF16)
    launch_rope_nh<true>(nh, dim3(total), s, tt, g, tc, table, wg, tm);
  else
    launch_rope_nh<false>(nh, dim3(total), s, tt, g, tc, table, wg, tm);
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
