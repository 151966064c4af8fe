// Internal declarations shared by the host library and the kernel launchers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la.h"

namespace la {

// Events that take the begin (start) and end (stop) timestamps of a kernel itself,
// through the launch (hipExtLaunchKernelGGL), not as separate stream packets around
// it; either may be null.  A launcher given one passes it to its (only) kernel.
struct KernelTiming {
  hipEvent_t start;
  hipEvent_t stop;
};

// A timed operation that launches nothing still completes its events (an empty span).
inline hipError_t timing_without_kernel(const KernelTiming* tm, hipStream_t s) {
  if (!tm) return hipSuccess;
  if (tm->start) {
    const hipError_t e = hipEventRecord(tm->start, s);
    if (e != hipSuccess) return e;
  }
  return tm->stop ? hipEventRecord(tm->stop, s) : hipSuccess;
}

template <typename F, typename... Args>
inline void launch_kernel(const KernelTiming* tm, F kernel, const dim3& grid, const dim3& block,
                          uint32_t lds, hipStream_t s, Args... args) {
  if (tm && (tm->start || tm->stop))
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, tm->start, tm->stop, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
}

// Segment table of one attention call: keys [end[s-1], end[s]) come from
// segment s, whose rows start at k[s] / v[s] with a row stride of
// heads*head_dim elements.  Order: sink, cached blocks, current block.
// tend[s]: 64-key tiles of segments 0..s when each segment is tiled on its own
// (the bf16 kernel's tiling).
constexpr int kMaxSegs = LA_MAX_WINDOW + 2;
struct AttnSegs {
  const void* k[kMaxSegs];
  const void* v[kMaxSegs];
  int32_t end[kMaxSegs];
  int32_t tend[kMaxSegs];
  int32_t nseg;
};

// Temporal cos/sin rows passed by value: rows 0..n_frames-1 are the block's
// frames, row n_frames the sink's position.
constexpr int kMaxTPairs = 48;
constexpr int kMaxTRows = LA_MAX_BLOCK_FRAMES + 1;
struct RopeTemporal {
  float cs[kMaxTRows][kMaxTPairs][2];
};

struct RopeTensor {
  const void* in;
  void* out;
  int32_t tokens;
  int32_t trow0;  // temporal row of this tensor's frame 0
  float scale;    // factor applied to the rotated values before the store
  // optional: cs_out[tok][pair][2] receives each token's cos and sin times cs_scale
  // (the values a Q at the same positions, with scale cs_scale, is rotated with)
  float* cs_out;
  float cs_scale;
  int32_t copy_only;  // 1: copy the rows unrotated (no cos/sin use)
  // 1 (bf16 only): out receives e4m3 codes [tokens][heads][head_dim] bytes of the bf16
  // result times inv8, rounded as la_quantize_fp8 rounds them
  int32_t e4m3_out;
  float inv8;
};
// One launch serves up to this many tensors (rows of each in order).
constexpr int kMaxRopeTensors = 5;

struct RopeGeom {
  int32_t HW, Wl, Hl, heads, head_dim, tpairs, hpairs, wpairs;
};

hipError_t launch_rope(const RopeTensor* t, int nt, const RopeGeom& g, const RopeTemporal& tc,
                       const float* table, la_dtype dt, hipStream_t s,
                       const KernelTiming* tm = nullptr);
hipError_t launch_rope_table(float* table, int Hl, int Wl, int hpairs, int wpairs, int hw,
                             double theta, hipStream_t s);
hipError_t launch_copy2(void* d0, const void* s0, void* d1, const void* s1, size_t bytes,
                        hipStream_t s, const KernelTiming* tm = nullptr);
hipError_t launch_euler(float* x, const float* v, int64_t n, float dt, hipStream_t s,
                        const KernelTiming* tm = nullptr);
// Workspace of the bf16 attention's persistent schedule: an arrival counter per unit
// (zero between calls) and one partial record of kAttnRecFloats floats per slot.
constexpr int kAttnRecFloats = 4 * (8 * 3 * 64 * 4 + 2 * 3 * 64);
struct AttnWorkspace {
  int32_t* counters;  // nullptr: no workspace, one workgroup per unit
  float* partials;
  int32_t slots;      // persistent workgroups (two per CU)
};
struct AttnWork {  // as passed to the kernel
  int32_t* counters;
  float* partials;
  int32_t cuts;  // key ranges per unit of the last round (1: no unit is cut)
};
int attn_bf16_units(int nq, int heads);
// qmul: factor applied to Q (then rounded to bf16) so that the kernel's base-2 scores
// are Q K^T; 1.0f when the caller's Q is already scaled.
// qcs: nullptr when q is already rotated; else q is the raw Q and qcs[tok][pair][2]
// holds the cos and sin of each token's head_dim pairs, already multiplied by the
// factor RoPE applies to Q (rope3d_kernel writes it, see RopeTensor::cs_out): the kernel
// rotates each pair with them exactly as rope3d_kernel rotates Q.
hipError_t launch_attn_bf16(const void* q, void* out, float* lse, const AttnSegs& segs, int nq,
                            int nk, int heads, float qmul, const AttnWorkspace& ws,
                            hipStream_t s, const KernelTiming* tm = nullptr,
                            const float* qcs = nullptr);
// The e4m3 attention's logit factor in the exponent's units, scale dq dk log2(e): in
// float32 (the multiply-add path) and in float64 (the power-of-two test below).
inline float fp8_logit_factor(float scale, float dq, float dk) {
  return scale * dq * dk * 1.4426950408889634f;
}
inline double fp8_logit_factor64(float scale, float dq, float dk) {
  return (double)scale * (double)dq * (double)dk * 1.4426950408889634;
}
// The E8M0 code 127 + e (0..254) of the power of two 2^e, -127 <= e <= 127, that lies
// within a relative 2^-24 of the factor f (the float32 product above may be off by three
// times that), else -1.
inline int fp8_pow2_scale_code(double f) {
  if (!(f > 0.0) || !__builtin_isfinite(f)) return -1;
  int k = 0;
  const double m = __builtin_frexp(f, &k);  // f = m 2^k, 0.5 <= m < 1
  int e;
  if (m - 0.5 <= 0x1p-25) e = k - 1;
  else if (1.0 - m <= 0x1p-24) e = k;
  else return -1;
  return (e >= -127 && e <= 127) ? 127 + e : -1;
}
// When the logit factor is a power of two in that sense (fp8_pow2_scale_code >= 0) the
// kernel applies it with the score MFMA's operand scale and takes the reference through
// the MFMA's accumulator input, else with one multiply-add per score.
hipError_t launch_attn_fp8(const void* q, void* out, float* lse, const AttnSegs& segs, int nq,
                           int nk, int heads, float scale, float dq, float dk, float dv,
                           hipStream_t s, const KernelTiming* tm = nullptr);
hipError_t launch_quantize_fp8(const void* in, int in_dtype, void* out, int64_t n, float inv_scale,
                               hipStream_t s);
// la_block_attn_fwd with its workspace given explicitly: slot_cap > 0 limits the
// persistent grid to that many workgroups; clear_counters zeroes the arrival counters
// (with a small fill kernel) before the launch.
la_status attn_fwd(const la_kvring* r, const void* q_rot, const void* sink_k_rot,
                   const void* k_cur_rot, const void* v_cur, int32_t n_q, void* out,
                   float* lse_or_null, float scale, float q_scale, void* workspace,
                   size_t workspace_bytes, int slot_cap, bool clear_counters,
                   la_stream_t stream, const KernelTiming* tm = nullptr,
                   const float* qcs = nullptr);
// Bytes of an attention workspace for `slots` persistent workgroups.
size_t attn_workspace_bytes(int n_q, int heads, int slots);
// Status of a HIP error (records its text as the thread's last HIP error).
la_status status_of(hipError_t e);
// Zero `bytes` (a multiple of 4) of device memory on stream s.
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_attn_f32(const void* q, void* out, float* lse, const AttnSegs& segs, int nq,
                           int nk, int heads, int head_dim, float scale, hipStream_t s,
                           const KernelTiming* tm = nullptr);

}  // namespace la
