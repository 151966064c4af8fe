// Internal declarations shared by the host library and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la.h"

namespace la {

// Segment table of one attention call: keys [end[s-1], end[s]) come from
// segment s, whose rows start at k[s] / v[s] with a row stride of
// heads*head_dim elements.  Order: sink, cached blocks, current block.
constexpr int kMaxSegs = LA_MAX_WINDOW + 2;
struct AttnSegs {
  const void* k[kMaxSegs];
  const void* v[kMaxSegs];
  int32_t end[kMaxSegs];
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
};

struct RopeGeom {
  int32_t HW, Wl, Hl, heads, head_dim, tpairs, hpairs, wpairs;
};

hipError_t launch_rope(const RopeTensor* t, int nt, const RopeGeom& g, const RopeTemporal& tc,
                       const float* table, la_dtype dt, hipStream_t s);
hipError_t launch_rope_table(float* table, int Hl, int Wl, int hpairs, int wpairs, int hw,
                             double theta, hipStream_t s);
hipError_t launch_copy2(void* d0, const void* s0, void* d1, const void* s1, size_t bytes,
                        hipStream_t s);
hipError_t launch_euler(float* x, const float* v, int64_t n, float dt, hipStream_t s);
hipError_t launch_attn_bf16(const void* q, void* out, float* lse, const AttnSegs& segs, int nq,
                            int nk, int heads, float scale, hipStream_t s);
hipError_t launch_attn_fp8(const void* q, void* out, float* lse, const AttnSegs& segs, int nq,
                           int nk, int heads, float scale, float dq, float dk, float dv,
                           hipStream_t s);
hipError_t launch_quantize_fp8(const void* in, int in_dtype, void* out, int64_t n, float inv_scale,
                               hipStream_t s);
hipError_t launch_attn_f32(const void* q, void* out, float* lse, const AttnSegs& segs, int nq,
                           int nk, int heads, int head_dim, float scale, hipStream_t s);

}  // namespace la
