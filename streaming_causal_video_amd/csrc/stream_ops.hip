// HBM-bound streaming kernels: cache append / sink replacement copies and the
// flow-matching Euler update, for gfx950.
//
// Cache append (gitcode.csdn.net "Live Avatar 深度解析…", 疑问 4: the cache
// stores the K/V of the step's own noisy x_t with no refresh pass) and the
// one-time sink replacement (papernotes.org "Live Avatar: Streaming Real-time
// Audio-Driven Avatar Generation with Infinite Length", 关键设计 3) are plain
// byte copies of two tensors (K and V) in one launch.  The Euler update follows
// the flow-matching velocity of the same notes' 损失函数 section:
// x <- x + dt * v, one fused multiply-add per element.
//
// Both kernels move 16-byte vectors, several per thread with all loads issued
// before the first store, so each wave keeps 4 KiB in flight.
//
// FP8 quantisation (papernotes.org notes, Table 3: FP8 quantisation among the
// operator-level optimisations): one per-tensor scale, e4m3 codes rounded to
// nearest even and saturated at +-448.
#include "la_internal.h"

namespace la {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Copies n16 16-byte vectors, then the last `tail` (< 16) bytes one by one.  A
// bounded grid loops over the vectors (kUnroll per thread and trip, all loads before
// the stores): at a block's 96 MB per tensor, 4096 workgroups per tensor looping run
// 6 % faster than one workgroup per 16 KB (measured, buffers beyond the caches).
__global__ __launch_bounds__(kThreads) void copy2_kernel(u32x4_t* __restrict__ d0,
                                                         const u32x4_t* __restrict__ s0,
                                                         u32x4_t* __restrict__ d1,
                                                         const u32x4_t* __restrict__ s1,
                                                         int64_t n16, int tail) {
  const u32x4_t* src = blockIdx.y ? s1 : s0;
  u32x4_t* dst = blockIdx.y ? d1 : d0;
  const int64_t step = (int64_t)gridDim.x * (kThreads * kUnroll);
  for (int64_t base = (int64_t)blockIdx.x * (kThreads * kUnroll) + threadIdx.x; base < n16;
       base += step) {
    u32x4_t r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + (int64_t)u * kThreads;
      if (i < n16) r[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + (int64_t)u * kThreads;
      if (i < n16) __builtin_nontemporal_store(r[u], dst + i);
    }
  }
  if (blockIdx.x == 0 && (int)threadIdx.x < tail) {
    const uint8_t* sb = reinterpret_cast<const uint8_t*>(src + n16);
    uint8_t* db = reinterpret_cast<uint8_t*>(dst + n16);
    db[threadIdx.x] = sb[threadIdx.x];
  }
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// kNT: non-temporal loads and stores, for latents far larger than the caches (a
// one-block latent of a few MB stays in the cache for the next stage instead).
template <bool kNT>
__global__ __launch_bounds__(kThreads) void euler_vec_kernel(float4* __restrict__ x,
                                                             const float4* __restrict__ v,
                                                             int64_t n4, float* __restrict__ xt,
                                                             const float* __restrict__ vt,
                                                             int tail, float dt) {
  const int64_t base = (int64_t)blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
  float4 a[kUnroll], b[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t i = base + (int64_t)u * kThreads;
    if (i < n4) {
      if constexpr (kNT) {
        const f32x4_t xa = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(x + i));
        const f32x4_t vb = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(v + i));
        a[u] = make_float4(xa[0], xa[1], xa[2], xa[3]);
        b[u] = make_float4(vb[0], vb[1], vb[2], vb[3]);
      } else {
        a[u] = x[i];
        b[u] = v[i];
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t i = base + (int64_t)u * kThreads;
    if (i < n4) {
      float4 y;
      y.x = fmaf(dt, b[u].x, a[u].x);
      y.y = fmaf(dt, b[u].y, a[u].y);
      y.z = fmaf(dt, b[u].z, a[u].z);
      y.w = fmaf(dt, b[u].w, a[u].w);
      if constexpr (kNT) {
        const f32x4_t yv = {y.x, y.y, y.z, y.w};
        __builtin_nontemporal_store(yv, reinterpret_cast<f32x4_t*>(x + i));
      } else
        x[i] = y;
    }
  }
  if (blockIdx.x == 0 && (int)threadIdx.x < tail) {
    xt[threadIdx.x] = fmaf(dt, vt[threadIdx.x], xt[threadIdx.x]);
  }
}

__global__ __launch_bounds__(kThreads) void euler_scalar_kernel(float* __restrict__ x,
                                                                const float* __restrict__ v,
                                                                int64_t n, float dt) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads)
    x[i] = fmaf(dt, v[i], x[i]);
}

#include "e4m3_dev.h"

// out[i] = e4m3(in[i] * inv): 16 elements per thread (two or four 16-byte loads,
// one 16-byte store); the last n % 16 elements by the thread after the last chunk.
template <bool kBF16>
__global__ __launch_bounds__(kThreads) void quant_fp8_kernel(const void* __restrict__ in,
                                                             uint8_t* __restrict__ out,
                                                             int64_t n16, int64_t n, float inv) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  float x[16];
  if (i < n16) {
    if constexpr (kBF16) {
      const uint4* p = static_cast<const uint4*>(in) + 2 * i;
      const uint4 a = p[0], b = p[1];
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        x[2 * k] = __uint_as_float(w[k] << 16) * inv;
        x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u) * inv;
      }
    } else {
      const float4* p = static_cast<const float4*>(in) + 4 * i;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 v = p[k];
        x[4 * k] = v.x * inv;
        x[4 * k + 1] = v.y * inv;
        x[4 * k + 2] = v.z * inv;
        x[4 * k + 3] = v.w * inv;
      }
    }
    reinterpret_cast<uint4*>(out)[i] = make_uint4(e4m3x4(x[0], x[1], x[2], x[3]),
                                                  e4m3x4(x[4], x[5], x[6], x[7]),
                                                  e4m3x4(x[8], x[9], x[10], x[11]),
                                                  e4m3x4(x[12], x[13], x[14], x[15]));
  } else if (i == n16) {
    for (int64_t e = 16 * n16; e < n; ++e) {
      const float v = kBF16 ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(in)[e] << 16)
                            : static_cast<const float*>(in)[e];
      out[e] = (uint8_t)(e4m3x4(v * inv, 0.f, 0.f, 0.f) & 0xffu);
    }
  }
}

__global__ __launch_bounds__(kThreads) void zero_u32_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads)
    p[i] = 0u;
}

}  // namespace

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 4);
  if (n == 0) return hipSuccess;
  int64_t wgs = (n + kThreads - 1) / kThreads;
  if (wgs > 1024) wgs = 1024;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)wgs), dim3(kThreads), 0, s,
                     static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

hipError_t launch_copy2(void* d0, const void* s0, void* d1, const void* s1, size_t bytes,
                        hipStream_t s, const KernelTiming* tm) {
  const int64_t n16 = (int64_t)(bytes / 16);
  const int tail = (int)(bytes - 16 * (size_t)n16);
  if (bytes == 0) return timing_without_kernel(tm, s);
  const int64_t per_wg = kThreads * kUnroll;
  int64_t wgs = n16 > 0 ? (n16 + per_wg - 1) / per_wg : 1;
  if (wgs > 4096) wgs = 4096;
  dim3 grid((unsigned)wgs, d1 ? 2 : 1);
  launch_kernel(tm, copy2_kernel, grid, dim3(kThreads), 0, s, static_cast<u32x4_t*>(d0),
                     static_cast<const u32x4_t*>(s0), static_cast<u32x4_t*>(d1),
                     static_cast<const u32x4_t*>(s1), n16, tail);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8(const void* in, int in_dtype, void* out, int64_t n, float inv,
                               hipStream_t s) {
  const int64_t n16 = n / 16;
  const int64_t threads = n16 + 1;  // one more thread for the tail
  const dim3 grid((unsigned)((threads + kThreads - 1) / kThreads));
  if (in_dtype == LA_BF16)
    hipLaunchKernelGGL(quant_fp8_kernel<true>, grid, dim3(kThreads), 0, s, in,
                       static_cast<uint8_t*>(out), n16, n, inv);
  else
    hipLaunchKernelGGL(quant_fp8_kernel<false>, grid, dim3(kThreads), 0, s, in,
                       static_cast<uint8_t*>(out), n16, n, inv);
  return hipGetLastError();
}

hipError_t launch_euler(float* x, const float* v, int64_t n, float dt, hipStream_t s,
                        const KernelTiming* tm) {
  if (n == 0) return timing_without_kernel(tm, s);
  const bool aligned = ((uintptr_t)x % 16 == 0) && ((uintptr_t)v % 16 == 0);
  if (aligned) {
    const int64_t n4 = n / 4;
    const int tail = (int)(n - 4 * n4);
    const int64_t per_wg = kThreads * kUnroll;
    const int64_t wgs = n4 > 0 ? (n4 + per_wg - 1) / per_wg : 1;
    if (wgs > 0x7fffffff) return hipErrorInvalidValue;
    // beyond 64 M elements (x and v 512 MB together, twice the 256 MB last-level cache)
    // the update streams through HBM: non-temporal accesses
    if (n >= ((int64_t)1 << 26))
      launch_kernel(tm, euler_vec_kernel<true>, dim3((unsigned)wgs), dim3(kThreads), 0, s,
                    reinterpret_cast<float4*>(x), reinterpret_cast<const float4*>(v), n4,
                    x + 4 * n4, v + 4 * n4, tail, dt);
    else
      launch_kernel(tm, euler_vec_kernel<false>, dim3((unsigned)wgs), dim3(kThreads), 0, s,
                    reinterpret_cast<float4*>(x), reinterpret_cast<const float4*>(v), n4,
                    x + 4 * n4, v + 4 * n4, tail, dt);
  } else {
    int64_t wgs = (n + kThreads - 1) / kThreads;
    if (wgs > 65536) wgs = 65536;
    launch_kernel(tm, euler_scalar_kernel, dim3((unsigned)wgs), dim3(kThreads), 0, s, x, v, n, dt);
  }
  return hipGetLastError();
}

}  // namespace la
