// Block attention in float32 (head_dim 64 or 128), for gfx950.
//
// Same operation as the bf16 MFMA kernel (papernotes.org "Live Avatar:
// Streaming Real-time Audio-Driven Avatar Generation with Infinite Length",
// 整体框架: the block attends to the sink frame, the sliding cache and itself,
// no mask), for the small float32 configurations whose results must hold to
// 1e-5.  This path is for exactness, not throughput: one wave per 64 query rows
// of one head, one query row per lane held in registers, 32-key K/V tiles in
// LDS read by broadcast, float32 online softmax.
#include "la_internal.h"

namespace la {
namespace {

constexpr int TK = 32;  // keys per tile

template <int DH>
__global__ __attribute__((amdgpu_flat_work_group_size(64, 64), amdgpu_waves_per_eu(1, 1))) void
attn_f32_kernel(const float* __restrict__ q, float* __restrict__ out, float* __restrict__ lse,
                const AttnSegs segs, int nq, int nk, int heads, float c2, int qtiles) {
  __shared__ __attribute__((aligned(16))) float ks[TK][DH];
  __shared__ __attribute__((aligned(16))) float vs[TK][DH];
  const int head = blockIdx.x / qtiles;
  const int qt = blockIdx.x - head * qtiles;
  const int tid = threadIdx.x;
  const int qrow = qt * 64 + tid;
  const int64_t rs = (int64_t)heads * DH;

  float qv[DH], ov[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d) {
    qv[d] = qrow < nq ? q[qrow * rs + head * DH + d] : 0.f;
    ov[d] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;

  for (int t0 = 0; t0 < nk; t0 += TK) {
    __syncthreads();
    for (int idx = tid; idx < TK * DH / 4; idx += 64) {
      const int row = idx / (DH / 4);
      const int c4 = idx - row * (DH / 4);
      const int key = t0 + row;
      float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
      if (key < nk) {
        int s = 0;
        while (key >= segs.end[s]) ++s;
        const int start = s ? segs.end[s - 1] : 0;
        const int64_t off = (int64_t)(key - start) * rs + head * DH + 4 * c4;
        kx = *reinterpret_cast<const float4*>(static_cast<const float*>(segs.k[s]) + off);
        vx = *reinterpret_cast<const float4*>(static_cast<const float*>(segs.v[s]) + off);
      }
      *reinterpret_cast<float4*>(&ks[row][4 * c4]) = kx;
      *reinterpret_cast<float4*>(&vs[row][4 * c4]) = vx;
    }
    __syncthreads();
    const int nvalid = min(TK, nk - t0);
    float sc[TK];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      float a = 0.f;
#pragma unroll
      for (int d = 0; d < DH; ++d) a = fmaf(qv[d], ks[j][d], a);
      sc[j] = j < nvalid ? a * c2 : -INFINITY;
      mx = fmaxf(mx, sc[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < DH; ++d) ov[d] *= alpha;
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      const float p = __builtin_amdgcn_exp2f(sc[j] - m_new);
      l_run += p;
#pragma unroll
      for (int d = 0; d < DH; ++d) ov[d] = fmaf(p, vs[j][d], ov[d]);
    }
    m_run = m_new;
  }
  if (qrow < nq) {
    const float inv = 1.f / l_run;
#pragma unroll
    for (int d = 0; d < DH; ++d) out[qrow * rs + head * DH + d] = ov[d] * inv;
    if (lse != nullptr) lse[(int64_t)head * nq + qrow] = (m_run + __log2f(l_run)) * 0.69314718055994531f;
  }
}

}  // namespace

hipError_t launch_attn_f32(const void* q, void* out, float* lse, const AttnSegs& segs, int nq,
                           int nk, int heads, int head_dim, float scale, hipStream_t s,
                           const KernelTiming* tm) {
  const int qtiles = (nq + 63) / 64;
  const float c2 = scale * 1.4426950408889634f;
  if (head_dim == 64)
    launch_kernel(tm, attn_f32_kernel<64>, dim3(qtiles * heads), dim3(64), 0, s,
                  static_cast<const float*>(q), static_cast<float*>(out), lse, segs, nq, nk, heads,
                  c2, qtiles);
  else
    launch_kernel(tm, attn_f32_kernel<128>, dim3(qtiles * heads), dim3(64), 0, s,
                  static_cast<const float*>(q), static_cast<float*>(out), lse, segs, nq, nk, heads,
                  c2, qtiles);
  return hipGetLastError();
}

}  // namespace la
