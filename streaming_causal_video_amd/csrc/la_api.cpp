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

// Kernel timing of the operation the step driver is enqueuing on this thread (null
// otherwise): the entry points pass it to their kernel launch, so that the driver's
// timing events take the kernel's own begin and end timestamps.  Set only through
// TimedOp, for the duration of one entry-point call.
thread_local const la::KernelTiming* t_timing = nullptr;

struct TimedOp {
  explicit TimedOp(const la::KernelTiming* tm) { t_timing = tm; }
  ~TimedOp() { t_timing = nullptr; }
  TimedOp(const TimedOp&) = delete;
  TimedOp& operator=(const TimedOp&) = delete;
};

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

// Frame-axis cos/sin of pair k at position pos: float64 on the host, rounded to float32
// (positions are unbounded over a long stream).
void frame_cs(int64_t pos, int k, int tband, double theta, float* c, float* s) {
  const double ang = (double)pos * pow(theta, -2.0 * (double)k / (double)tband);
  *c = (float)cos(ang);
  *s = (float)sin(ang);
}

// Compute units of the current device (cached per device); 0 if it cannot be read.
int device_cus() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev] = n;
  return n;
}

// Workspace layout of the bf16 attention: counters (one int32 per unit, padded to
// 256 bytes), then one partial record per slot; slots = two per CU.
size_t attn_counter_bytes(int n_q, int heads) {
  return ((size_t)la::attn_bf16_units(n_q, heads) * 4 + 255) / 256 * 256;
}
size_t attn_ws_bytes(int n_q, int heads, int slots) {
  return attn_counter_bytes(n_q, heads) + (size_t)slots * la::kAttnRecFloats * sizeof(float);
}

}  // namespace

extern "C" {

const char* la_version(void) { return "liblahip 0.8 (gfx950) attn-v17 fp8-v10"; }

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

}  // extern "C"

namespace {

// Slots of a ring: W, or W + 1 for a staged ring; 0 if the struct is not a valid ring.
int ring_slots(const la_kvring* r) {
  if (r->W < 1 || r->W > LA_MAX_WINDOW) return 0;
  if (r->nslots != r->W && r->nslots != r->W + 1) return 0;
  if (r->nslots > LA_MAX_WINDOW) return 0;
  return r->nslots;
}

la_status ring_init(la_kvring* r, void* k_slots, void* v_slots, void* sink_k_raw, void* sink_v,
                    int32_t W, int32_t nslots, int32_t block_tokens, int32_t sink_tokens,
                    int32_t heads, int32_t head_dim, la_dtype dtype, float noise_level) {
  if (!r || !k_slots || !v_slots || !sink_k_raw || !sink_v) return LA_ERR_INVALID_ARG;
  if (!valid_ring_dtype(dtype)) return LA_ERR_DTYPE;
  if (W < 1 || nslots > LA_MAX_WINDOW || block_tokens < 1 || sink_tokens < 1 || heads < 1 ||
      head_dim < 8 || head_dim % 8 != 0 || head_dim > 256)
    return LA_ERR_SHAPE;
  if (!isfinite(noise_level)) return LA_ERR_INVALID_ARG;
  if (!aligned16(k_slots) || !aligned16(v_slots) || !aligned16(sink_k_raw) || !aligned16(sink_v))
    return LA_ERR_INVALID_ARG;
  // every slot and the sink must be whole 16-byte vectors, so that each slot starts
  // 16-byte aligned (an e4m3 ring with heads * head_dim * block_tokens not a multiple
  // of 16 would not)
  const int64_t row = (int64_t)heads * head_dim;
  if ((row * block_tokens * (int64_t)elem_size(dtype)) % 16 != 0 ||
      (row * sink_tokens * (int64_t)sink_elem_size(dtype)) % 16 != 0)
    return LA_ERR_SHAPE;
  memset(r, 0, sizeof(*r));
  r->k_slots = k_slots;
  r->v_slots = v_slots;
  r->sink_k_raw = sink_k_raw;
  r->sink_v = sink_v;
  r->W = W;
  r->nslots = nslots;
  r->block_tokens = block_tokens;
  r->sink_tokens = sink_tokens;
  r->heads = heads;
  r->head_dim = head_dim;
  r->dtype = dtype;
  r->noise_level = noise_level;
  return LA_OK;
}

}  // namespace

extern "C" {

la_status la_kvring_init(la_kvring* r, void* k_slots, void* v_slots, void* sink_k_raw,
                         void* sink_v, int32_t W, int32_t block_tokens, int32_t sink_tokens,
                         int32_t heads, int32_t head_dim, la_dtype dtype, float noise_level) {
  return ring_init(r, k_slots, v_slots, sink_k_raw, sink_v, W, W, block_tokens, sink_tokens,
                   heads, head_dim, dtype, noise_level);
}

la_status la_kvring_init_staged(la_kvring* r, void* k_slots, void* v_slots, void* sink_k_raw,
                                void* sink_v, int32_t W, int32_t block_tokens,
                                int32_t sink_tokens, int32_t heads, int32_t head_dim,
                                la_dtype dtype, float noise_level) {
  return ring_init(r, k_slots, v_slots, sink_k_raw, sink_v, W, W + 1, block_tokens, sink_tokens,
                   heads, head_dim, dtype, noise_level);
}

la_status la_kvring_advance(const la_kvring* r, int64_t block_id, int32_t* slot,
                            int64_t* evicted) {
  if (!r || !slot || !evicted) return LA_ERR_INVALID_ARG;
  const int ns = ring_slots(r);
  if (ns == 0) return LA_ERR_STATE;
  if (block_id != r->last_block + 1 || block_id < 1) return LA_ERR_STATE;
  *slot = (int32_t)((block_id - 1) % ns);
  *evicted = block_id > r->W ? block_id - r->W : 0;
  return LA_OK;
}

la_status la_kvring_next_slot(const la_kvring* r, void** k_slot, void** v_slot) {
  if (!r || !k_slot || !v_slot) return LA_ERR_INVALID_ARG;
  int32_t slot;
  int64_t evicted;
  const la_status st = la_kvring_advance(r, r->last_block + 1, &slot, &evicted);
  if (st != LA_OK) return st;
  // a ring of W slots reuses the slot of the block that leaves the window, which
  // the next block's attention still reads
  if (r->nslots == r->W && evicted != 0) return LA_ERR_STATE;
  const size_t slot_bytes =
      (size_t)r->block_tokens * r->heads * r->head_dim * elem_size(r->dtype);
  *k_slot = static_cast<char*>(r->k_slots) + slot * slot_bytes;
  *v_slot = static_cast<char*>(r->v_slots) + slot * slot_bytes;
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

}  // extern "C"

namespace {

// la_rope3d_rolling, and optionally in the same launch:
//  * q_cs_out != NULL (with k_in): the cos/sin of every block token's pairs times
//    q_scale into q_cs_out[token][head_dim / 2][2], what the rotation of a Q at those
//    positions multiplies by (the step hands it to the bf16 attention, which then
//    rotates its raw Q itself);
//  * v_in, v_out != NULL: a plain copy of the block's V (the step stages it in a ring
//    slot).
// The geometry and the frame-axis cos/sin (float64 on the host) of one block's RoPE
// launch: the block's frames f0 .. f0 + n_frames - 1 in rows 0 .. n_frames - 1, the
// sink's position f0 + sink_delta in row n_frames.
la_status rope_setup(int32_t n_frames, int64_t f0, int64_t sink_delta, int32_t Hl, int32_t Wl,
                     int32_t heads, int32_t head_dim, double theta, la::RopeGeom* g,
                     la::RopeTemporal* tc) {
  if (!(theta > 1.0)) return LA_ERR_INVALID_ARG;
  if (n_frames < 1 || n_frames > LA_MAX_BLOCK_FRAMES || Hl < 1 || Wl < 1 || heads < 1 ||
      head_dim < 8 || head_dim % 8 != 0 || head_dim > 256)
    return LA_ERR_SHAPE;
  int tband, hw;
  bands(head_dim, &tband, &hw);
  const int tpairs = tband / 2;
  if (tpairs > la::kMaxTPairs || hw < 2) return LA_ERR_SHAPE;
  const int64_t hwtok = (int64_t)Hl * Wl;
  if (hwtok * n_frames > INT32_MAX / 2) return LA_ERR_SHAPE;
  memset(tc, 0, sizeof(*tc));
  for (int row = 0; row <= n_frames; ++row) {
    const int64_t pos = row < n_frames ? f0 + row : f0 + sink_delta;
    for (int k = 0; k < tpairs; ++k)
      frame_cs(pos, k, tband, theta, &tc->cs[row][k][0], &tc->cs[row][k][1]);
  }
  g->HW = (int32_t)hwtok;
  g->Wl = Wl;
  g->Hl = Hl;
  g->heads = heads;
  g->head_dim = head_dim;
  g->tpairs = tpairs;
  g->hpairs = hw / 2;
  g->wpairs = hw / 2;
  return LA_OK;
}

la_status rope_rolling(const void* q_in, void* q_out, const void* k_in, void* k_out,
                       int32_t n_frames, int64_t f0, const void* sink_k_in, void* sink_k_out,
                       int64_t sink_delta, const void* dev_table, int32_t Hl, int32_t Wl,
                       int32_t heads, int32_t head_dim, la_dtype dtype, double theta,
                       float q_scale, float* q_cs_out, const void* v_in, void* v_out,
                       la_stream_t stream) {
  if (!valid_dtype(dtype)) return LA_ERR_DTYPE;
  if (!dev_table || !(theta > 1.0)) return LA_ERR_INVALID_ARG;
  if (!(q_scale > 0.f) || !isfinite(q_scale)) return LA_ERR_INVALID_ARG;
  if ((!q_in) != (!q_out) || (!k_in) != (!k_out) || (!sink_k_in) != (!sink_k_out))
    return LA_ERR_INVALID_ARG;
  la::RopeGeom g;
  la::RopeTemporal tc;
  const la_status st = rope_setup(n_frames, f0, sink_delta, Hl, Wl, heads, head_dim, theta, &g, &tc);
  if (st != LA_OK) return st;
  const void* ptrs[6] = {q_in, q_out, k_in, k_out, sink_k_in, sink_k_out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return LA_ERR_INVALID_ARG;
  const int64_t hwtok = (int64_t)Hl * Wl;
  if (q_cs_out && (!k_in || !aligned16(q_cs_out))) return LA_ERR_INVALID_ARG;
  if ((!v_in) != (!v_out) || (v_in && (!aligned16(v_in) || !aligned16(v_out))))
    return LA_ERR_INVALID_ARG;
  la::RopeTensor t[4] = {
      {q_in, q_out, (int32_t)(hwtok * n_frames), 0, q_scale, nullptr, 1.0f, 0},
      {k_in, k_out, (int32_t)(hwtok * n_frames), 0, 1.0f, q_cs_out, q_scale, 0},
      {sink_k_in, sink_k_out, (int32_t)hwtok, n_frames, 1.0f, nullptr, 1.0f, 0},
      {v_in, v_out, (int32_t)(hwtok * n_frames), 0, 1.0f, nullptr, 1.0f, 1},
  };
  return hip_status(la::launch_rope(t, 4, g, tc, static_cast<const float*>(dev_table), dtype,
                                    static_cast<hipStream_t>(stream), t_timing));
}

}  // namespace

extern "C" {

la_status la_rope3d_rolling(const void* q_in, void* q_out, const void* k_in, void* k_out,
                            int32_t n_frames, int64_t f0, const void* sink_k_in,
                            void* sink_k_out, int64_t sink_delta, const void* dev_table,
                            int32_t Hl, int32_t Wl, int32_t heads, int32_t head_dim,
                            la_dtype dtype, double theta, float q_scale, la_stream_t stream) {
  return rope_rolling(q_in, q_out, k_in, k_out, n_frames, f0, sink_k_in, sink_k_out, sink_delta,
                      dev_table, Hl, Wl, heads, head_dim, dtype, theta, q_scale, nullptr, nullptr,
                      nullptr, stream);
}

size_t la_attn_workspace_bytes(int32_t n_q, int32_t heads) {
  if (n_q < 1 || heads < 1) return 0;
  const int cus = device_cus();
  if (cus < 1) return 0;
  return attn_ws_bytes(n_q, heads, 2 * cus);
}

}  // extern "C"

namespace {

// Segment table of an attention call for the kernels that tile each segment on its
// own (bf16, e4m3), whose last tile is then partial (at 4680 rows, 8 of its 64 keys
// valid): the sink, then the cached blocks in slot (address) order -- softmax
// attention does not depend on the order of the keys -- then the current block.
// Segments whose K and V both continue where the previous one ends (neighbouring
// slots; the current block when the caller staged it in the ring's next slot, where
// it takes its place among the slots) are joined, as long as the kernels' 32-bit byte
// offsets still reach past the joined segment's end.  Fills segs (with the tile ends
// tend) and returns the number of keys.
int joined_segments(const la_kvring* r, int count, const void* sink_k, const void* sink_v,
                    const void* k_cur, const void* v_cur, la::AttnSegs& segs) {
  memset(&segs, 0, sizeof(segs));
  const size_t row_bytes = (size_t)r->heads * r->head_dim * elem_size(r->dtype);
  const size_t slot_bytes = (size_t)r->block_tokens * row_bytes;
  int n = 0, end = 0;
  int64_t rows = 0;  // rows of segment n - 1 while it may still grow
  auto add = [&](const void* k, const void* v, int len, bool may_join) {
    const bool joins =
        may_join && n > 0 && static_cast<const char*>(segs.k[n - 1]) + rows * row_bytes == k &&
        static_cast<const char*>(segs.v[n - 1]) + rows * row_bytes == v &&
        (rows + len + 64) * (int64_t)row_bytes < ((int64_t)1 << 32);
    end += len;
    if (joins) {
      rows += len;
      segs.end[n - 1] = end;
    } else {
      rows = len;
      segs.k[n] = k;
      segs.v[n] = v;
      segs.end[n++] = end;
    }
  };
  add(sink_k, sink_v, r->sink_tokens, false);
  const int ns = ring_slots(r);
  bool in_window[LA_MAX_WINDOW + 1] = {};
  for (int64_t b = r->last_block - count + 1; b <= r->last_block; ++b)
    in_window[(b - 1) % ns] = true;
  const int next = (int)(r->last_block % ns);
  const bool cur_in_slot = !in_window[next] &&
                           k_cur == static_cast<const char*>(r->k_slots) + next * slot_bytes &&
                           v_cur == static_cast<const char*>(r->v_slots) + next * slot_bytes;
  if (cur_in_slot) in_window[next] = true;
  bool first = true;  // the first cached run never joins the sink
  for (int slot = 0; slot < ns; ++slot)
    if (in_window[slot]) {
      add(static_cast<const char*>(r->k_slots) + slot * slot_bytes,
          static_cast<const char*>(r->v_slots) + slot * slot_bytes, r->block_tokens, !first);
      first = false;
    }
  if (!cur_in_slot) add(k_cur, v_cur, r->block_tokens, !first);
  segs.nseg = n;
  for (int i = 0, t = 0; i < n; ++i) {
    t += (segs.end[i] - (i ? segs.end[i - 1] : 0) + 63) / 64;
    segs.tend[i] = t;
  }
  return end;
}

}  // namespace

namespace la {

la_status status_of(hipError_t e) { return hip_status(e); }

la_status attn_fwd(const la_kvring* r, const void* q_rot, const void* sink_k_rot,
                   const void* k_cur_rot, const void* v_cur, int32_t n_q, void* out,
                   float* lse_or_null, float scale, float q_scale, void* workspace,
                   size_t workspace_bytes, int slot_cap, bool clear_counters,
                   la_stream_t stream, const KernelTiming* tm, const float* qcs) {
  if (!r || !q_rot || !sink_k_rot || !k_cur_rot || !v_cur || !out) return LA_ERR_INVALID_ARG;
  if (qcs && (r->dtype != LA_BF16 || !aligned16(qcs))) return LA_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return LA_ERR_INVALID_ARG;
  if (ring_slots(r) == 0) return LA_ERR_STATE;
  if (!(q_scale > 0.f) || !isfinite(q_scale)) return LA_ERR_INVALID_ARG;
  if (workspace && ((uintptr_t)workspace % 256)) return LA_ERR_INVALID_ARG;
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
  int end;
  if (r->dtype == LA_BF16) {
    end = joined_segments(r, count, sink_k_rot, r->sink_v, k_cur_rot, v_cur, segs);
  } else {
    // the float32 kernel: the sink, the cached blocks oldest first, the current block
    memset(&segs, 0, sizeof(segs));
    const size_t slot_bytes =
        (size_t)r->block_tokens * r->heads * r->head_dim * elem_size(r->dtype);
    int n = 0;
    end = 0;
    segs.k[n] = sink_k_rot;
    segs.v[n] = r->sink_v;
    end += r->sink_tokens;
    segs.end[n++] = end;
    const int ns = ring_slots(r);
    for (int64_t b = r->last_block - count + 1; b <= r->last_block; ++b) {
      const int slot = (int)((b - 1) % ns);
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
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (r->dtype == LA_BF16) {
    // base-2 scores: Q times scale * log2(e) / q_scale, rounded to bf16 in the kernel
    // unless that factor is 1 in float32 (Q already scaled by the caller)
    const float qmul = (float)((double)scale * 1.4426950408889634 / (double)q_scale);
    la::AttnWorkspace ws = {nullptr, nullptr, 0};
    if (workspace) {
      const int cus = device_cus();
      if (cus < 1) return LA_ERR_HIP;
      int slots = 2 * cus;
      if (slot_cap > 0 && slots > slot_cap) slots = slot_cap;
      if (workspace_bytes < attn_ws_bytes(n_q, r->heads, slots)) return LA_ERR_SHAPE;
      ws.counters = static_cast<int32_t*>(workspace);
      ws.partials = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             attn_counter_bytes(n_q, r->heads));
      ws.slots = slots;
      if (clear_counters) {
        e = la::launch_zero(workspace, attn_counter_bytes(n_q, r->heads), s);
        if (e != hipSuccess) return hip_status(e);
      }
    }
    e = la::launch_attn_bf16(q_rot, out, lse_or_null, segs, n_q, end, r->heads, qmul, ws, s, tm,
                             qcs);
  } else {
    e = la::launch_attn_f32(q_rot, out, lse_or_null, segs, n_q, end, r->heads, r->head_dim,
                            scale / q_scale, s, tm);
  }
  return hip_status(e);
}

size_t attn_workspace_bytes(int n_q, int heads, int slots) {
  return attn_ws_bytes(n_q, heads, slots);
}

}  // namespace la

extern "C" {

la_status la_block_attn_fwd(const la_kvring* r, const void* q_rot, const void* sink_k_rot,
                            const void* k_cur_rot, const void* v_cur, int32_t n_q, void* out,
                            float* lse_or_null, float scale, float q_scale, void* workspace,
                            size_t workspace_bytes, la_stream_t stream) {
  return la::attn_fwd(r, q_rot, sink_k_rot, k_cur_rot, v_cur, n_q, out, lse_or_null, scale,
                      q_scale, workspace, workspace_bytes, 0, false, stream, t_timing);
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
  if (ring_slots(r) == 0) return LA_ERR_STATE;
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
  const int end = joined_segments(r, count, sink_k8, sink_v8, k8_cur, v8_cur, segs);
  return hip_status(la::launch_attn_fp8(q8, out, lse_or_null, segs, n_q, end, r->heads, scale,
                                        dq, dk, dv, static_cast<hipStream_t>(stream), t_timing));
}

la_status la_fp8_q_factor_pow2(float scale, float dk, float dq_min, float* dq_out) {
  if (!dq_out) return LA_ERR_INVALID_ARG;
  const float f[3] = {scale, dk, dq_min};
  for (float x : f)
    if (!(x > 0.f) || !isfinite(x)) return LA_ERR_INVALID_ARG;
  // The factor is dq times K = scale dk log2(e); for the least power of two 2^e at or
  // above the factor of dq_min, dq = 2^e / K rounded to float32 has a factor within a
  // relative 2^-24 of 2^e, and so may the float below it (the window holds up to two
  // floats): the least of the two, or the next float up when the rounding fell below
  // dq_min, else the next power of two.
  if (la::fp8_pow2_scale_code(la::fp8_logit_factor64(scale, dq_min, dk)) >= 0) {
    *dq_out = dq_min;
    return LA_OK;
  }
  const double K = la::fp8_logit_factor64(scale, 1.f, dk);
  int k = 0;
  const double m = frexp(la::fp8_logit_factor64(scale, dq_min, dk), &k);
  int e = m == 0.5 ? k - 1 : k;
  for (int attempt = 0; attempt < 4; ++attempt, ++e) {
    const float dq = (float)ldexp(1.0 / K, e);
    for (float c : {nextafterf(dq, 0.f), dq, nextafterf(dq, INFINITY)}) {  // least first
      if (!(c >= dq_min) || !isfinite(c)) continue;
      if (la::fp8_pow2_scale_code(la::fp8_logit_factor64(scale, c, dk)) >= 0) {
        *dq_out = c;
        return LA_OK;
      }
    }
  }
  return LA_ERR_INVALID_ARG;
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
  char* kd = static_cast<char*>(r->k_slots) + slot * slot_bytes;
  char* vd = static_cast<char*>(r->v_slots) + slot * slot_bytes;
  // a half that is already in its slot (written there by the caller) is not copied
  const void* ks = k_rot == kd ? nullptr : k_rot;
  const void* vs = v == vd ? nullptr : v;
  if (!ks) {
    kd = vd;
    ks = vs;
    vd = nullptr;
    vs = nullptr;
  } else if (!vs) {
    vd = nullptr;
  }
  const hipError_t e =
      ks ? la::launch_copy2(kd, ks, vd, vs, slot_bytes, static_cast<hipStream_t>(stream), t_timing)
         : la::timing_without_kernel(t_timing, static_cast<hipStream_t>(stream));
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
  return hip_status(la::launch_euler(x, v, n, dt, static_cast<hipStream_t>(stream), t_timing));
}

}  // extern "C"

namespace {

// The step's scale and attention workspace (NULL, or 256-byte aligned and at least
// la_attn_workspace_bytes for the ring's geometry).
la_status validate_attn_ws(const la_kvring& r0, float scale, const void* ws, size_t bytes) {
  if (!(scale > 0.f) || !isfinite(scale)) return LA_ERR_INVALID_ARG;
  if (!ws) return LA_OK;
  if ((uintptr_t)ws % 256) return LA_ERR_INVALID_ARG;
  if (r0.dtype == LA_BF16 && bytes < la_attn_workspace_bytes(r0.block_tokens, r0.heads))
    return LA_ERR_SHAPE;
  return LA_OK;
}

// Checks of one stage's arguments, shared by la_denoise_step and la_denoise_chain.
la_status validate_stage(const la_kvring* rings, int32_t n_layers, int64_t block_id,
                         const void* const* q_raw, const void* const* k_raw,
                         const void* const* v_raw, void* const* attn_out,
                         const void* const* sink_k_new, const void* const* sink_v_new,
                         int32_t Hl, int32_t Wl, int32_t frames_per_block, uint32_t flags,
                         bool fp8 = false) {
  if (!rings || n_layers < 1 || !q_raw || !k_raw || !v_raw || !attn_out)
    return LA_ERR_INVALID_ARG;
  if ((!sink_k_new) != (!sink_v_new)) return LA_ERR_INVALID_ARG;
  if (flags & ~LA_STEP_ATTEND_ONLY) return LA_ERR_INVALID_ARG;
  if ((flags & LA_STEP_ATTEND_ONLY) && sink_k_new) return LA_ERR_INVALID_ARG;
  if (frames_per_block < 1 || frames_per_block > LA_MAX_BLOCK_FRAMES || Hl < 1 || Wl < 1)
    return LA_ERR_SHAPE;
  const la_kvring& r0 = rings[0];
  if (fp8) {
    if (r0.dtype != LA_FP8_E4M3) return LA_ERR_DTYPE;
    if (r0.head_dim != 128) return LA_ERR_SHAPE;
  } else if (!valid_dtype(r0.dtype)) {
    return LA_ERR_DTYPE;  // la_denoise_step runs bf16 / f32 rings
  }
  if ((int64_t)r0.block_tokens != (int64_t)frames_per_block * Hl * Wl ||
      (int64_t)r0.sink_tokens != (int64_t)Hl * Wl)
    return LA_ERR_SHAPE;
  for (int l = 0; l < n_layers; ++l) {
    const la_kvring& r = rings[l];
    if (ring_slots(&r) == 0) return LA_ERR_STATE;
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
                        float scale, void* attn_ws, size_t attn_ws_bytes, float* x,
                        const float* vel, int64_t n_latent, float dt, uint32_t flags,
                        void* const* timing_events, la_stream_t stream) {
  const bool append = !(flags & LA_STEP_ATTEND_ONLY);
  // bf16 rings: RoPE emits Q already multiplied by the attention's base-2 score scale
  // (one rounding), and the attention takes it as given
  const float q_scale =
      rings[0].dtype == LA_BF16 ? (float)((double)scale * 1.4426950408889634) : 1.0f;
  const int64_t f0 = (int64_t)frames_per_block * (block_id - 1);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  // timing events i, i + 1 as the begin and end of the kernel of one operation
  auto span = [&](int i) -> la::KernelTiming {
    return timing_events ? la::KernelTiming{static_cast<hipEvent_t>(timing_events[i]),
                                            static_cast<hipEvent_t>(timing_events[i + 1])}
                         : la::KernelTiming{nullptr, nullptr};
  };
#define LA_TRY(expr)                 \
  do {                               \
    const la_status st_ = (expr);    \
    if (st_ != LA_OK) return st_;    \
  } while (0)
  // bf16 rings with at least two heads: RoPE writes the block tokens' cos/sin (times
  // q_scale, 512 bytes a token) into q_rot_ws instead of rotating Q, and the attention
  // rotates the raw Q with them as it loads it (the same bits as rotating Q first)
  const bool fuse_q = rings[0].dtype == LA_BF16 && rings[0].heads >= 2;
  float* q_cs = fuse_q ? static_cast<float*>(q_rot_ws) : nullptr;
  for (int l = 0; l < n_layers; ++l) {
    la_kvring* r = &rings[l];
    // fused append: a staged ring takes the rotated K in its next slot directly, and
    // the same launch copies the block's V into the slot (no window block uses that
    // slot); the attention reads both there, and the append only records the block
    void* k_rot = k_rot_ws;
    void* v_stage = nullptr;
    if (append && r->nslots == r->W + 1) LA_TRY(la_kvring_next_slot(r, &k_rot, &v_stage));
    const la::KernelTiming t_rope = span(6 * l), t_attn = span(6 * l + 2),
                           t_app = span(6 * l + 4);
    {
      TimedOp op(&t_rope);
      LA_TRY(rope_rolling(fuse_q ? nullptr : q_raw[l], fuse_q ? nullptr : q_rot_ws, k_raw[l],
                          k_rot, frames_per_block, f0, r->sink_k_raw, sink_k_rot_ws, sink_delta,
                          rope_table, Hl, Wl, r->heads, r->head_dim, (la_dtype)r->dtype, theta,
                          q_scale, q_cs, v_stage ? v_raw[l] : nullptr, v_stage, stream));
    }
    {
      TimedOp op(&t_attn);
      // a staged block is read from its slot (its K and V then continue the
      // neighbouring slots, which the attention joins into one segment)
      const void* v_cur = v_stage ? v_stage : v_raw[l];
      if (fuse_q)
        LA_TRY(la::attn_fwd(r, q_raw[l], sink_k_rot_ws, k_rot, v_cur, r->block_tokens,
                            attn_out[l], nullptr, scale, q_scale, attn_ws, attn_ws_bytes, 0,
                            false, stream, t_timing, q_cs));
      else
        LA_TRY(la_block_attn_fwd(r, q_rot_ws, sink_k_rot_ws, k_rot, v_cur, r->block_tokens,
                                 attn_out[l], nullptr, scale, q_scale, attn_ws, attn_ws_bytes,
                                 stream));
    }
    if (append) {
      TimedOp op(&t_app);
      LA_TRY(la_kvcache_append_evict(r, k_rot, v_stage ? v_stage : v_raw[l], block_id,
                                     r->noise_level, nullptr, stream));
    } else {
      LA_TRY(hip_status(la::timing_without_kernel(&t_app, hs)));
    }
    if (append && block_id == 1 && sink_k_new)
      LA_TRY(la_sink_replace(r, sink_k_new[l], sink_v_new[l], stream));
  }
  const la::KernelTiming t_euler = span(6 * n_layers);
  if (x && n_latent > 0) {
    TimedOp op(&t_euler);
    LA_TRY(la_fm_euler_step(x, vel, n_latent, dt, stream));
  } else {
    LA_TRY(hip_status(la::timing_without_kernel(&t_euler, hs)));
  }
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
                          double theta, float scale, void* attn_ws, size_t attn_ws_bytes,
                          float* x, const float* vel, int64_t n_latent, float dt, uint32_t flags,
                          void* const* timing_events, la_stream_t stream) {
  // ---- validate the whole step before enqueuing anything
  if (!q_rot_ws || !k_rot_ws || !sink_k_rot_ws || !rope_table) return LA_ERR_INVALID_ARG;
  const la_status v = validate_stage(rings, n_layers, block_id, q_raw, k_raw, v_raw, attn_out,
                                     sink_k_new, sink_v_new, Hl, Wl, frames_per_block, flags);
  if (v != LA_OK) return v;
  if (x && (!vel || n_latent < 0 || !isfinite(dt))) return LA_ERR_INVALID_ARG;
  {
    const la_status w = validate_attn_ws(rings[0], scale, attn_ws, attn_ws_bytes);
    if (w != LA_OK) return w;
  }
  return enqueue_stage(rings, n_layers, block_id, q_raw, k_raw, v_raw, attn_out, q_rot_ws,
                       k_rot_ws, sink_k_rot_ws, sink_k_new, sink_v_new, rope_table, Hl, Wl,
                       frames_per_block, sink_delta, theta, scale, attn_ws, attn_ws_bytes, x, vel,
                       n_latent, dt, flags, timing_events, stream);
}

la_status la_denoise_step_fp8(la_kvring* rings, int32_t n_layers, int64_t block_id,
                              const void* const* q_raw, const void* const* k_raw,
                              const void* const* v_raw, void* const* attn_out, void* q_rot_ws,
                              void* k_rot_ws, void* sink_k_rot_ws, void* q8_ws, void* k8_ws,
                              void* v8_ws, void* sink_k8_ws, void* sink_v8_ws,
                              const void* const* sink_k_new, const void* const* sink_v_new,
                              const void* rope_table, int32_t Hl, int32_t Wl,
                              int32_t frames_per_block, int64_t sink_delta, double theta,
                              float scale, float dq, float dk, float dv, float* x,
                              const float* vel, int64_t n_latent, float dt, uint32_t flags,
                              void* const* timing_events, la_stream_t stream) {
  // ---- validate the whole step before enqueuing anything
  (void)q_rot_ws;  // unused: RoPE and the quantisation run as one launch
  (void)k_rot_ws;
  (void)sink_k_rot_ws;
  if (!rope_table || !q8_ws || !sink_k8_ws || !sink_v8_ws) return LA_ERR_INVALID_ARG;
  const la_status v = validate_stage(rings, n_layers, block_id, q_raw, k_raw, v_raw, attn_out,
                                     sink_k_new, sink_v_new, Hl, Wl, frames_per_block, flags,
                                     true);
  if (v != LA_OK) return v;
  const bool append = !(flags & LA_STEP_ATTEND_ONLY);
  for (int l = 0; l < n_layers; ++l)
    if (!(append && rings[l].nslots == rings[l].W + 1) && (!k8_ws || !v8_ws))
      return LA_ERR_INVALID_ARG;  // a plain ring (or no append) needs the K/V code workspaces
  const float f[4] = {scale, dq, dk, dv};
  for (float z : f)
    if (!(z > 0.f) || !isfinite(z)) return LA_ERR_INVALID_ARG;
  const void* ws[5] = {q8_ws, k8_ws, v8_ws, sink_k8_ws, sink_v8_ws};
  for (const void* p : ws)
    if (p && !aligned16(p)) return LA_ERR_INVALID_ARG;
  if (x && (!vel || n_latent < 0 || !isfinite(dt))) return LA_ERR_INVALID_ARG;
  for (int l = 0; l < n_layers; ++l)
    if (!aligned16(q_raw[l]) || !aligned16(k_raw[l]) || !aligned16(v_raw[l]))
      return LA_ERR_INVALID_ARG;

  const int64_t f0 = (int64_t)frames_per_block * (block_id - 1);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  auto ev = [&](int i) -> hipEvent_t {
    return timing_events ? static_cast<hipEvent_t>(timing_events[i]) : nullptr;
  };
  // the reciprocals the quantisation multiplies by, as la_quantize_fp8 takes them
  const float iq = 1.0f / dq, ik = 1.0f / dk, iv = 1.0f / dv;
#define LA_TRY(expr)                 \
  do {                               \
    const la_status st_ = (expr);    \
    if (st_ != LA_OK) return st_;    \
  } while (0)
  for (int l = 0; l < n_layers; ++l) {
    la_kvring* r = &rings[l];
    void* k8 = k8_ws;
    void* v8 = v8_ws;
    if (append && r->nslots == r->W + 1) LA_TRY(la_kvring_next_slot(r, &k8, &v8));
    const la::KernelTiming t_rope = {ev(6 * l), ev(6 * l + 1)},
                           t_attn = {ev(6 * l + 2), ev(6 * l + 3)},
                           t_app = {ev(6 * l + 4), ev(6 * l + 5)};
    // One launch: Q, K and the sink K rotated (no Q pre-scale), each rounded to bf16 and
    // quantised; the block's V and the ring's sink V quantised as they are.
    la::RopeGeom g;
    la::RopeTemporal tc;
    LA_TRY(rope_setup(frames_per_block, f0, sink_delta, Hl, Wl, r->heads, r->head_dim, theta,
                      &g, &tc));
    const int32_t bt = r->block_tokens, stk = r->sink_tokens;
    const la::RopeTensor t[5] = {
        {q_raw[l], q8_ws, bt, 0, 1.0f, nullptr, 1.0f, 0, 1, iq},
        {k_raw[l], k8, bt, 0, 1.0f, nullptr, 1.0f, 0, 1, ik},
        {r->sink_k_raw, sink_k8_ws, stk, frames_per_block, 1.0f, nullptr, 1.0f, 0, 1, ik},
        {v_raw[l], v8, bt, 0, 1.0f, nullptr, 1.0f, 1, 1, iv},
        {r->sink_v, sink_v8_ws, stk, 0, 1.0f, nullptr, 1.0f, 1, 1, iv},
    };
    LA_TRY(hip_status(la::launch_rope(t, 5, g, tc, static_cast<const float*>(rope_table),
                                      LA_BF16, hs, &t_rope)));
    {
      TimedOp op(&t_attn);
      LA_TRY(la_block_attn_fwd_fp8(r, q8_ws, sink_k8_ws, sink_v8_ws, k8, v8, r->block_tokens,
                                   attn_out[l], nullptr, scale, dq, dk, dv, stream));
    }
    if (append) {
      TimedOp op(&t_app);
      LA_TRY(la_kvcache_append_evict(r, k8, v8, block_id, r->noise_level, nullptr, stream));
    } else {
      LA_TRY(hip_status(la::timing_without_kernel(&t_app, hs)));
    }
    if (append && block_id == 1 && sink_k_new)
      LA_TRY(la_sink_replace(r, sink_k_new[l], sink_v_new[l], stream));
  }
  const la::KernelTiming t_euler = {ev(6 * n_layers), ev(6 * n_layers + 1)};
  if (x && n_latent > 0) {
    TimedOp op(&t_euler);
    LA_TRY(la_fm_euler_step(x, vel, n_latent, dt, stream));
  } else {
    LA_TRY(hip_status(la::timing_without_kernel(&t_euler, hs)));
  }
#undef LA_TRY
  return LA_OK;
}

la_status la_denoise_chain(la_stage* stages, int32_t n_stages, int32_t n_layers,
                           int64_t block_id, void* q_rot_ws, void* k_rot_ws,
                           void* sink_k_rot_ws, const void* rope_table, int32_t Hl, int32_t Wl,
                           int32_t frames_per_block, int64_t sink_delta, double theta,
                           float scale, void* attn_ws, size_t attn_ws_bytes, float* x,
                           int64_t n_latent, la_stream_t stream) {
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
  {
    const la_status w = validate_attn_ws(stages[0].rings[0], scale, attn_ws, attn_ws_bytes);
    if (w != LA_OK) return w;
  }
  for (int s = 0; s < n_stages; ++s) {
    const la_stage& g = stages[s];
    const la_status st = enqueue_stage(g.rings, n_layers, block_id, g.q_raw, g.k_raw, g.v_raw,
                                       g.attn_out, q_rot_ws, k_rot_ws, sink_k_rot_ws,
                                       g.sink_k_new, g.sink_v_new, rope_table, Hl, Wl,
                                       frames_per_block, sink_delta, theta, scale, attn_ws,
                                       attn_ws_bytes, n_latent > 0 ? x : nullptr, g.vel,
                                       n_latent, g.dt, 0u, nullptr, stream);
    if (st != LA_OK) return st;
  }
  return LA_OK;
}

}  // extern "C"
