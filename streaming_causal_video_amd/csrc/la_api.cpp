// extern "C" entry points of liblahip: argument validation, the rolling-cache
// index state and the launches.  All device work goes to the caller's stream.
//
// Ring rules: gitcode.csdn.net "Live Avatar 深度解析…", 疑问 4 (the cache keeps the
// K/V of the step's own noisy x_t, no refresh, same noise level as the latent)
// and papernotes.org "Live Avatar: Streaming Real-time Audio-Driven Avatar
// Generation with Infinite Length", 关键设计 2 and 4 (local sliding noisy cache
// per timestep stage).  Sink rule: the same notes, 关键设计 3, and the blog's
// 疑问 5 (replaced exactly once, after the first block).
#include <math.h>
#include <string.h>

#include <string>

#include "la_internal.h"

namespace {

thread_local std::string g_last_hip_error;

la_status hip_status(hipError_t e) {
  if (e == hipSuccess) return LA_OK;
  g_last_hip_error = std::string(hipGetErrorName(e)) + ": " + hipGetErrorString(e);
  return LA_ERR_HIP;
}

// bytes per element of a ring's K/V slots, and of its sink (bf16 for e4m3 rings)
size_t elem_size(int dt) { return dt == LA_FP8_E4M3 ? 1 : (dt == LA_BF16 ? 2 : 4); }
size_t sink_elem_size(int dt) { return dt == LA_FP8_E4M3 ? 2 : elem_size(dt); }

// compute dtypes of the RoPE / bf16-f32 attention calls
bool valid_dtype(int dt) { return dt == LA_BF16 || dt == LA_F32; }
bool valid_ring_dtype(int dt) { return valid_dtype(dt) || dt == LA_FP8_E4M3; }

// Frame band width d - 4*floor(d/6); spatial bands 2*floor(d/6) each.
void bands(int d, int* t, int* hw) {
  const int s = d / 6;
  *t = d - 4 * s;
  *hw = 2 * s;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" {

const char* la_version(void) { return "liblahip 0.4 (gfx950) attn-v9 fp8-v6"; }

const char* la_status_string(int st) {
  switch (st) {
    case LA_OK: return "ok";
    case LA_ERR_INVALID_ARG: return "invalid argument";
    case LA_ERR_SHAPE: return "shape mismatch or unsupported size";
    case LA_ERR_DTYPE: return "unsupported dtype";
    case LA_ERR_STATE: return "invalid cache state for this call";
    case LA_ERR_NOISE_LEVEL: return "noise level differs from the cache's";
    case LA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* la_last_hip_error(void) { return g_last_hip_error.c_str(); }

la_status la_kvring_init(la_kvring* r, void* k_slots, void* v_slots, void* sink_k_raw,
                         void* sink_v, int32_t W, int32_t block_tokens, int32_t sink_tokens,
                         int32_t heads, int32_t head_dim, la_dtype dtype, float noise_level) {
  if (!r || !k_slots || !v_slots || !sink_k_raw || !sink_v) return LA_ERR_INVALID_ARG;
  if (!valid_ring_dtype(dtype)) return LA_ERR_DTYPE;
  if (W < 1 || W > LA_MAX_WINDOW || block_tokens < 1 || sink_tokens < 1 || heads < 1 ||
      head_dim < 8 || head_dim % 8 != 0 || head_dim > 256)
    return LA_ERR_SHAPE;
  if (!isfinite(noise_level)) return LA_ERR_INVALID_ARG;
  if (!aligned16(k_slots) || !aligned16(v_slots) || !aligned16(sink_k_raw) || !aligned16(sink_v))
    return LA_ERR_INVALID_ARG;
  memset(r, 0, sizeof(*r));
  r->k_slots = k_slots;
  r->v_slots = v_slots;
  r->sink_k_raw = sink_k_raw;
  r->sink_v = sink_v;
  r->W = W;
  r->block_tokens = block_tokens;
  r->sink_tokens = sink_tokens;
  r->heads = heads;
  r->head_dim = head_dim;
  r->dtype = dtype;
  r->noise_level = noise_level;
  return LA_OK;
}

la_status la_kvring_advance(const la_kvring* r, int64_t block_id, int32_t* slot,
                            int64_t* evicted) {
  if (!r || !slot || !evicted) return LA_ERR_INVALID_ARG;
  if (r->W < 1 || r->W > LA_MAX_WINDOW) return LA_ERR_STATE;
  if (block_id != r->last_block + 1 || block_id < 1) return LA_ERR_STATE;
  *slot = (int32_t)((block_id - 1) % r->W);
  *evicted = block_id > r->W ? block_id - r->W : 0;
  return LA_OK;
}

int32_t la_kvring_count(const la_kvring* r) {
  if (!r) return 0;
  return r->last_block < r->W ? (int32_t)r->last_block : r->W;
}

size_t la_rope_table_bytes(int32_t Hl, int32_t Wl, int32_t head_dim) {
  if (Hl < 1 || Wl < 1 || head_dim < 8) return 0;
  int t, hw;
  bands(head_dim, &t, &hw);
  return (size_t)(Hl + Wl) * (size_t)(hw / 2) * 2 * sizeof(float);
}

la_status la_rope_table_fill(void* dev_table, int32_t Hl, int32_t Wl, int32_t head_dim,
                             double theta, la_stream_t stream) {
  if (!dev_table || Hl < 1 || Wl < 1 || !(theta > 1.0)) return LA_ERR_INVALID_ARG;
  if (head_dim < 8 || head_dim % 8 != 0 || head_dim > 256) return LA_ERR_SHAPE;
  if ((uintptr_t)dev_table % 4) return LA_ERR_INVALID_ARG;
  int t, hw;
  bands(head_dim, &t, &hw);
  return hip_status(la::launch_rope_table(static_cast<float*>(dev_table), Hl, Wl, hw / 2, hw / 2,
                                          hw, theta, static_cast<hipStream_t>(stream)));
}

la_status la_rope3d_rolling(const void* q_in, void* q_out, const void* k_in, void* k_out,
                            int32_t n_frames, int64_t f0, const void* sink_k_in,
                            void* sink_k_out, int64_t sink_delta, const void* dev_table,
                            int32_t Hl, int32_t Wl, int32_t heads, int32_t head_dim,
                            la_dtype dtype, double theta, la_stream_t stream) {
  if (!valid_dtype(dtype)) return LA_ERR_DTYPE;
  if (!dev_table || !(theta > 1.0)) return LA_ERR_INVALID_ARG;
  if ((!q_in) != (!q_out) || (!k_in) != (!k_out) || (!sink_k_in) != (!sink_k_out))
    return LA_ERR_INVALID_ARG;
  if (n_frames < 1 || n_frames > LA_MAX_BLOCK_FRAMES || Hl < 1 || Wl < 1 || heads < 1 ||
      head_dim < 8 || head_dim % 8 != 0 || head_dim > 256)
    return LA_ERR_SHAPE;
  const void* ptrs[6] = {q_in, q_out, k_in, k_out, sink_k_in, sink_k_out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return LA_ERR_INVALID_ARG;
  int tband, hw;
  bands(head_dim, &tband, &hw);
  const int tpairs = tband / 2;
  if (tpairs > la::kMaxTPairs || hw < 2) return LA_ERR_SHAPE;
  const int64_t hwtok = (int64_t)Hl * Wl;
  if (hwtok * n_frames > INT32_MAX / 2) return LA_ERR_SHAPE;

  // Frame-axis cos/sin for the block's frames and the sink's position, float64 on the host.
  la::RopeTemporal tc;
  memset(&tc, 0, sizeof(tc));
  for (int row = 0; row <= n_frames; ++row) {
    const int64_t pos = row < n_frames ? f0 + row : f0 + sink_delta;
    for (int k = 0; k < tpairs; ++k) {
      const double a = (double)pos * pow(theta, -2.0 * (double)k / (double)tband);
      tc.cs[row][k][0] = (float)cos(a);
      tc.cs[row][k][1] = (float)sin(a);
    }
  }
  la::RopeGeom g;
  g.HW = (int32_t)hwtok;
  g.Wl = Wl;
  g.Hl = Hl;
  g.heads = heads;
  g.head_dim = head_dim;
  g.tpairs = tpairs;
  g.hpairs = hw / 2;
  g.wpairs = hw / 2;
  la::RopeTensor t[3] = {
      {q_in, q_out, (int32_t)(hwtok * n_frames), 0},
      {k_in, k_out, (int32_t)(hwtok * n_frames), 0},
      {sink_k_in, sink_k_out, (int32_t)hwtok, n_frames},
  };
  return hip_status(la::launch_rope(t, 3, g, tc, static_cast<const float*>(dev_table), dtype,
                                    static_cast<hipStream_t>(stream)));
}

la_status la_block_attn_fwd(const la_kvring* r, const void* q_rot, const void* sink_k_rot,
                            const void* k_cur_rot, const void* v_cur, int32_t n_q, void* out,
                            float* lse_or_null, float scale, la_stream_t stream) {
  if (!r || !q_rot || !sink_k_rot || !k_cur_rot || !v_cur || !out) return LA_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return LA_ERR_INVALID_ARG;
  if (!valid_dtype(r->dtype)) return LA_ERR_DTYPE;
  if (n_q != r->block_tokens || n_q < 1) return LA_ERR_SHAPE;
  if (r->dtype == LA_BF16 && r->head_dim != 128) return LA_ERR_SHAPE;
  if (r->dtype == LA_F32 && r->head_dim != 64 && r->head_dim != 128) return LA_ERR_SHAPE;
  const void* ptrs[5] = {q_rot, sink_k_rot, k_cur_rot, v_cur, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return LA_ERR_INVALID_ARG;
  if (lse_or_null && ((uintptr_t)lse_or_null % 4)) return LA_ERR_INVALID_ARG;
  if (out == q_rot || out == k_cur_rot || out == v_cur) return LA_ERR_INVALID_ARG;
  const int count = la_kvring_count(r);
  const int64_t nk64 = (int64_t)r->sink_tokens + (int64_t)(count + 1) * r->block_tokens;
  if (nk64 > INT32_MAX / 2 || (int64_t)n_q * r->heads * r->head_dim > ((int64_t)1 << 40))
    return LA_ERR_SHAPE;
  // the bf16 kernel addresses a segment with 32-bit byte offsets
  const int64_t seg_rows = (r->sink_tokens > r->block_tokens ? r->sink_tokens : r->block_tokens) + 64;
  if (r->dtype == LA_BF16 && seg_rows * r->heads * r->head_dim * 2 >= ((int64_t)1 << 32))
    return LA_ERR_SHAPE;

  la::AttnSegs segs;
  memset(&segs, 0, sizeof(segs));
  const size_t slot_bytes =
      (size_t)r->block_tokens * r->heads * r->head_dim * elem_size(r->dtype);
  int n = 0, end = 0;
  segs.k[n] = sink_k_rot;
  segs.v[n] = r->sink_v;
  end += r->sink_tokens;
  segs.end[n++] = end;
  // cached blocks, oldest first
  for (int64_t b = r->last_block - count + 1; b <= r->last_block; ++b) {
    const int slot = (int)((b - 1) % r->W);
    segs.k[n] = static_cast<const char*>(r->k_slots) + slot * slot_bytes;
    segs.v[n] = static_cast<const char*>(r->v_slots) + slot * slot_bytes;
    end += r->block_tokens;
    segs.end[n++] = end;
  }
  segs.k[n] = k_cur_rot;
  segs.v[n] = v_cur;
  end += r->block_tokens;
  segs.end[n++] = end;
  segs.nseg = n;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (r->dtype == LA_BF16)
    e = la::launch_attn_bf16(q_rot, out, lse_or_null, segs, n_q, end, r->heads, scale, s);
  else
    e = la::launch_attn_f32(q_rot, out, lse_or_null, segs, n_q, end, r->heads, r->head_dim,
                            scale, s);
  return hip_status(e);
}

la_status la_quantize_fp8(const void* in, la_dtype in_dtype, void* out, int64_t n,
                          float inv_scale, la_stream_t stream) {
  if (n < 0) return LA_ERR_INVALID_ARG;
  if (n == 0) return LA_OK;
  if (!in || !out) return LA_ERR_INVALID_ARG;
  if (!valid_dtype(in_dtype)) return LA_ERR_DTYPE;
  if (!(inv_scale > 0.f) || !isfinite(inv_scale)) return LA_ERR_INVALID_ARG;
  if (!aligned16(in) || !aligned16(out)) return LA_ERR_INVALID_ARG;
  const uintptr_t ia = (uintptr_t)in, oa = (uintptr_t)out;
  const uintptr_t ib = (uintptr_t)n * elem_size(in_dtype), ob = (uintptr_t)n;
  if (ia < oa + ob && oa < ia + ib) return LA_ERR_INVALID_ARG;
  return hip_status(la::launch_quantize_fp8(in, in_dtype, out, n, inv_scale,
                                            static_cast<hipStream_t>(stream)));
}

la_status la_block_attn_fwd_fp8(const la_kvring* r, const void* q8, const void* sink_k8,
                                const void* sink_v8, const void* k8_cur, const void* v8_cur,
                                int32_t n_q, void* out, float* lse_or_null, float scale,
                                float dq, float dk, float dv, la_stream_t stream) {
  if (!r || !q8 || !sink_k8 || !sink_v8 || !k8_cur || !v8_cur || !out) return LA_ERR_INVALID_ARG;
  const float f[4] = {scale, dq, dk, dv};
  for (float x : f)
    if (!(x > 0.f) || !isfinite(x)) return LA_ERR_INVALID_ARG;
  if (r->dtype != LA_FP8_E4M3) return LA_ERR_DTYPE;
  if (n_q != r->block_tokens || n_q < 1 || r->head_dim != 128) return LA_ERR_SHAPE;
  const void* ptrs[6] = {q8, sink_k8, sink_v8, k8_cur, v8_cur, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return LA_ERR_INVALID_ARG;
  if (lse_or_null && ((uintptr_t)lse_or_null % 4)) return LA_ERR_INVALID_ARG;
  if (out == q8 || out == k8_cur || out == v8_cur || out == sink_k8 || out == sink_v8)
    return LA_ERR_INVALID_ARG;
  const int count = la_kvring_count(r);
  const int64_t nk64 = (int64_t)r->sink_tokens + (int64_t)(count + 1) * r->block_tokens;
  if (nk64 > INT32_MAX / 2 || (int64_t)n_q * r->heads * r->head_dim > ((int64_t)1 << 40))
    return LA_ERR_SHAPE;
  // the kernel addresses a segment with 32-bit byte offsets
  const int64_t seg_rows = (r->sink_tokens > r->block_tokens ? r->sink_tokens : r->block_tokens) + 64;
  if (seg_rows * r->heads * r->head_dim >= ((int64_t)1 << 32)) return LA_ERR_SHAPE;

  la::AttnSegs segs;
  memset(&segs, 0, sizeof(segs));
  const size_t slot_bytes = (size_t)r->block_tokens * r->heads * r->head_dim;
  int n = 0, end = 0;
  segs.k[n] = sink_k8;
  segs.v[n] = sink_v8;
  end += r->sink_tokens;
  segs.end[n++] = end;
  for (int64_t b = r->last_block - count + 1; b <= r->last_block; ++b) {
    const int slot = (int)((b - 1) % r->W);
    segs.k[n] = static_cast<const char*>(r->k_slots) + slot * slot_bytes;
    segs.v[n] = static_cast<const char*>(r->v_slots) + slot * slot_bytes;
    end += r->block_tokens;
    segs.end[n++] = end;
  }
  segs.k[n] = k8_cur;
  segs.v[n] = v8_cur;
  end += r->block_tokens;
  segs.end[n++] = end;
  segs.nseg = n;
  return hip_status(la::launch_attn_fp8(q8, out, lse_or_null, segs, n_q, end, r->heads, scale,
                                        dq, dk, dv, static_cast<hipStream_t>(stream)));
}

la_status la_kvcache_append_evict(la_kvring* r, const void* k_rot, const void* v,
                                  int64_t block_id, float noise_level,
                                  int64_t* evicted_or_null, la_stream_t stream) {
  if (!r || !k_rot || !v) return LA_ERR_INVALID_ARG;
  if (!aligned16(k_rot) || !aligned16(v)) return LA_ERR_INVALID_ARG;
  int32_t slot;
  int64_t evicted;
  const la_status st = la_kvring_advance(r, block_id, &slot, &evicted);
  if (st != LA_OK) return st;
  if (noise_level != r->noise_level) return LA_ERR_NOISE_LEVEL;
  const size_t slot_bytes =
      (size_t)r->block_tokens * r->heads * r->head_dim * elem_size(r->dtype);
  const hipError_t e =
      la::launch_copy2(static_cast<char*>(r->k_slots) + slot * slot_bytes, k_rot,
                       static_cast<char*>(r->v_slots) + slot * slot_bytes, v, slot_bytes,
                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_status(e);
  r->slot_block[slot] = block_id;
  r->last_block = block_id;
  if (evicted_or_null) *evicted_or_null = evicted;
  return LA_OK;
}

la_status la_sink_replace(la_kvring* r, const void* k_new_raw, const void* v_new,
                          la_stream_t stream) {
  if (!r || !k_new_raw || !v_new) return LA_ERR_INVALID_ARG;
  if (!aligned16(k_new_raw) || !aligned16(v_new)) return LA_ERR_INVALID_ARG;
  if (r->sink_replaced || r->last_block < 1) return LA_ERR_STATE;
  const size_t bytes =
      (size_t)r->sink_tokens * r->heads * r->head_dim * sink_elem_size(r->dtype);
  const hipError_t e = la::launch_copy2(r->sink_k_raw, k_new_raw, r->sink_v, v_new, bytes,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_status(e);
  r->sink_replaced = 1;
  return LA_OK;
}

la_status la_fm_euler_step(float* x, const float* v, int64_t n, float dt, la_stream_t stream) {
  if (n < 0) return LA_ERR_INVALID_ARG;
  if (n == 0) return LA_OK;
  if (!x || !v || !isfinite(dt)) return LA_ERR_INVALID_ARG;
  if (x != v) {
    const uintptr_t xa = (uintptr_t)x, va = (uintptr_t)v, nb = (uintptr_t)n * 4;
    if (xa < va + nb && va < xa + nb) return LA_ERR_INVALID_ARG;  // partial overlap
  }
  return hip_status(la::launch_euler(x, v, n, dt, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Checks of one stage's arguments, shared by la_denoise_step and la_denoise_chain.
la_status validate_stage(const la_kvring* rings, int32_t n_layers, int64_t block_id,
                         const void* const* q_raw, const void* const* k_raw,
                         const void* const* v_raw, void* const* attn_out,
                         const void* const* sink_k_new, const void* const* sink_v_new,
                         int32_t Hl, int32_t Wl, int32_t frames_per_block, uint32_t flags) {
  if (!rings || n_layers < 1 || !q_raw || !k_raw || !v_raw || !attn_out)
    return LA_ERR_INVALID_ARG;
  if ((!sink_k_new) != (!sink_v_new)) return LA_ERR_INVALID_ARG;
  if (flags & ~LA_STEP_ATTEND_ONLY) return LA_ERR_INVALID_ARG;
  if ((flags & LA_STEP_ATTEND_ONLY) && sink_k_new) return LA_ERR_INVALID_ARG;
  if (frames_per_block < 1 || frames_per_block > LA_MAX_BLOCK_FRAMES || Hl < 1 || Wl < 1)
    return LA_ERR_SHAPE;
  const la_kvring& r0 = rings[0];
  if (!valid_dtype(r0.dtype)) return LA_ERR_DTYPE;  // the step runs bf16 / f32 rings
  if ((int64_t)r0.block_tokens != (int64_t)frames_per_block * Hl * Wl ||
      (int64_t)r0.sink_tokens != (int64_t)Hl * Wl)
    return LA_ERR_SHAPE;
  for (int l = 0; l < n_layers; ++l) {
    const la_kvring& r = rings[l];
    if (r.W != r0.W || r.block_tokens != r0.block_tokens || r.sink_tokens != r0.sink_tokens ||
        r.heads != r0.heads || r.head_dim != r0.head_dim || r.dtype != r0.dtype)
      return LA_ERR_SHAPE;
    if (r.noise_level != r0.noise_level) return LA_ERR_NOISE_LEVEL;
    if (r.last_block != block_id - 1 || block_id < 1) return LA_ERR_STATE;
    if (block_id == 1 && sink_k_new && r.sink_replaced) return LA_ERR_STATE;
    if (!q_raw[l] || !k_raw[l] || !v_raw[l] || !attn_out[l]) return LA_ERR_INVALID_ARG;
    if (sink_k_new && block_id == 1 && (!sink_k_new[l] || !sink_v_new[l]))
      return LA_ERR_INVALID_ARG;
  }
  return LA_OK;
}

// Enqueue one validated stage (per layer: RoPE, attention, append, sink
// replacement at block 1; then the Euler update).
la_status enqueue_stage(la_kvring* rings, int32_t n_layers, int64_t block_id,
                        const void* const* q_raw, const void* const* k_raw,
                        const void* const* v_raw, void* const* attn_out, void* q_rot_ws,
                        void* k_rot_ws, void* sink_k_rot_ws, const void* const* sink_k_new,
                        const void* const* sink_v_new, const void* rope_table, int32_t Hl,
                        int32_t Wl, int32_t frames_per_block, int64_t sink_delta, double theta,
                        float scale, float* x, const float* vel, int64_t n_latent, float dt,
                        uint32_t flags, void* const* timing_events, la_stream_t stream) {
  const bool append = !(flags & LA_STEP_ATTEND_ONLY);
  const int64_t f0 = (int64_t)frames_per_block * (block_id - 1);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  auto mark = [&](int i) -> la_status {
    if (!timing_events) return LA_OK;
    return hip_status(hipEventRecord(static_cast<hipEvent_t>(timing_events[i]), hs));
  };
#define LA_TRY(expr)                 \
  do {                               \
    const la_status st_ = (expr);    \
    if (st_ != LA_OK) return st_;    \
  } while (0)
  for (int l = 0; l < n_layers; ++l) {
    la_kvring* r = &rings[l];
    LA_TRY(mark(6 * l));
    LA_TRY(la_rope3d_rolling(q_raw[l], q_rot_ws, k_raw[l], k_rot_ws, frames_per_block, f0,
                             r->sink_k_raw, sink_k_rot_ws, sink_delta, rope_table, Hl, Wl,
                             r->heads, r->head_dim, (la_dtype)r->dtype, theta, stream));
    LA_TRY(mark(6 * l + 1));
    LA_TRY(mark(6 * l + 2));
    LA_TRY(la_block_attn_fwd(r, q_rot_ws, sink_k_rot_ws, k_rot_ws, v_raw[l], r->block_tokens,
                             attn_out[l], nullptr, scale, stream));
    LA_TRY(mark(6 * l + 3));
    LA_TRY(mark(6 * l + 4));
    if (append)
      LA_TRY(la_kvcache_append_evict(r, k_rot_ws, v_raw[l], block_id, r->noise_level, nullptr,
                                     stream));
    if (append && block_id == 1 && sink_k_new)
      LA_TRY(la_sink_replace(r, sink_k_new[l], sink_v_new[l], stream));
    LA_TRY(mark(6 * l + 5));
  }
  LA_TRY(mark(6 * n_layers));
  if (x && n_latent > 0) LA_TRY(la_fm_euler_step(x, vel, n_latent, dt, stream));
  LA_TRY(mark(6 * n_layers + 1));
#undef LA_TRY
  return LA_OK;
}

}  // namespace

extern "C" {

la_status la_denoise_step(la_kvring* rings, int32_t n_layers, int64_t block_id,
                          const void* const* q_raw, const void* const* k_raw,
                          const void* const* v_raw, void* const* attn_out, void* q_rot_ws,
                          void* k_rot_ws, void* sink_k_rot_ws, const void* const* sink_k_new,
                          const void* const* sink_v_new, const void* rope_table, int32_t Hl,
                          int32_t Wl, int32_t frames_per_block, int64_t sink_delta,
                          double theta, float scale, float* x, const float* vel,
                          int64_t n_latent, float dt, uint32_t flags,
                          void* const* timing_events, la_stream_t stream) {
  // ---- validate the whole step before enqueuing anything
  if (!q_rot_ws || !k_rot_ws || !sink_k_rot_ws || !rope_table) return LA_ERR_INVALID_ARG;
  const la_status v = validate_stage(rings, n_layers, block_id, q_raw, k_raw, v_raw, attn_out,
                                     sink_k_new, sink_v_new, Hl, Wl, frames_per_block, flags);
  if (v != LA_OK) return v;
  if (x && (!vel || n_latent < 0 || !isfinite(dt))) return LA_ERR_INVALID_ARG;
  if (timing_events)
    for (int i = 0; i < 6 * n_layers + 2; ++i)
      if (!timing_events[i]) return LA_ERR_INVALID_ARG;
  return enqueue_stage(rings, n_layers, block_id, q_raw, k_raw, v_raw, attn_out, q_rot_ws,
                       k_rot_ws, sink_k_rot_ws, sink_k_new, sink_v_new, rope_table, Hl, Wl,
                       frames_per_block, sink_delta, theta, scale, x, vel, n_latent, dt,
                       flags, timing_events, stream);
}

la_status la_denoise_chain(la_stage* stages, int32_t n_stages, int32_t n_layers,
                           int64_t block_id, void* q_rot_ws, void* k_rot_ws,
                           void* sink_k_rot_ws, const void* rope_table, int32_t Hl, int32_t Wl,
                           int32_t frames_per_block, int64_t sink_delta, double theta,
                           float scale, float* x, int64_t n_latent, la_stream_t stream) {
  // ---- validate every stage, and the noise-level chain, before enqueuing anything
  if (!stages || n_stages < 1 || !q_rot_ws || !k_rot_ws || !sink_k_rot_ws || !rope_table)
    return LA_ERR_INVALID_ARG;
  if (n_latent < 0 || (n_latent > 0 && !x)) return LA_ERR_INVALID_ARG;
  for (int s = 0; s < n_stages; ++s) {
    const la_stage& g = stages[s];
    const la_status v = validate_stage(g.rings, n_layers, block_id, g.q_raw, g.k_raw, g.v_raw,
                                       g.attn_out, g.sink_k_new, g.sink_v_new, Hl, Wl,
                                       frames_per_block, 0u);
    if (v != LA_OK) return v;
    if (!isfinite(g.dt) || (n_latent > 0 && !g.vel)) return LA_ERR_INVALID_ARG;
    if (g.rings[0].head_dim != stages[0].rings[0].head_dim ||
        g.rings[0].heads != stages[0].rings[0].heads ||
        g.rings[0].dtype != stages[0].rings[0].dtype ||
        g.rings[0].block_tokens != stages[0].rings[0].block_tokens)
      return LA_ERR_SHAPE;
    for (int t = 0; t < s; ++t)  // one ring belongs to one stage
      for (int l = 0; l < n_layers; ++l)
        for (int m = 0; m < n_layers; ++m)
          if (&stages[t].rings[l] == &g.rings[m]) return LA_ERR_INVALID_ARG;
    if (s > 0) {
      const double expect = (double)stages[s - 1].rings[0].noise_level + stages[s - 1].dt;
      if (fabs((double)g.rings[0].noise_level - expect) > 1e-6) return LA_ERR_NOISE_LEVEL;
    }
  }
  for (int s = 0; s < n_stages; ++s) {
    const la_stage& g = stages[s];
    const la_status st = enqueue_stage(g.rings, n_layers, block_id, g.q_raw, g.k_raw, g.v_raw,
                                       g.attn_out, q_rot_ws, k_rot_ws, sink_k_rot_ws,
                                       g.sink_k_new, g.sink_v_new, rope_table, Hl, Wl,
                                       frames_per_block, sink_delta, theta, scale,
                                       n_latent > 0 ? x : nullptr, g.vel, n_latent, g.dt,
                                       0u, nullptr, stream);
    if (st != LA_OK) return st;
  }
  return LA_OK;
}

}  // extern "C"
