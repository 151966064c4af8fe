/*
 * la.h - C ABI of the streaming timestep-forcing denoise step (Live Avatar hot path)
 *        for AMD Instinct MI355X (gfx950).
 *
 * Pages cited below:
 *   NOTES = papernotes.org, "Live Avatar: Streaming Real-time Audio-Driven Avatar
 *           Generation with Infinite Length"
 *   NEWS  = 10100.com, "连续直播上万秒不崩脸！阿里开源Live Avatar …"
 *   POP   = admirer.cn popular article on Live Avatar
 *   BLOG  = gitcode.csdn.net, "Live Avatar 深度解析：首个 14B 参数实时流式无限时长数字人"
 *
 * One stage of the timestep-forcing pipeline owns one fixed denoise step
 * t_i -> t_{i-1} and a local noisy KV cache per layer (NOTES, 关键设计 4; NEWS,
 * TPP figure caption).  Per block and layer the step rotates Q/K with 3D RoPE
 * and the sink K with the rolling offset (la_rope3d_rolling), attends over
 * {sink, cached blocks, the block} (la_block_attn_fwd), appends the block's
 * K/V to the window (la_kvcache_append_evict), replaces the sink once after
 * block 1 (la_sink_replace), and finally moves the latent one Euler step
 * (la_fm_euler_step).
 *
 * Conventions shared by every call
 *   - Device buffers are allocated, owned and freed by the caller.  The library
 *     never allocates or frees device memory and keeps no global state apart
 *     from a thread-local copy of the last HIP error text.
 *   - Activations are contiguous and token-major: [tokens][heads][head_dim].
 *     Tokens are ordered frame-major, then latent row h, then column w.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     device work is enqueued on it; nothing synchronises.  Host-side state
 *     (la_kvring) changes at call time, so the order of calls is the order of
 *     state changes.
 *   - Argument, shape, dtype and state errors are detected before any launch
 *     and change nothing.  A failed launch returns LA_ERR_HIP (see
 *     la_last_hip_error).  A fault inside a kernel surfaces at the caller's
 *     next synchronisation.
 *   - No handle is thread-safe.
 */
#ifndef LA_H_
#define LA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum la_status {
  LA_OK = 0,
  LA_ERR_INVALID_ARG = -1,  /* NULL pointer, non-positive size, bad enum value      */
  LA_ERR_SHAPE = -2,        /* sizes disagree with the ring or a kernel's limits    */
  LA_ERR_DTYPE = -3,        /* dtype not supported by this call                     */
  LA_ERR_STATE = -4,        /* block out of order, second sink replacement, ...     */
  LA_ERR_NOISE_LEVEL = -5,  /* append at another noise level than the cache's      */
  LA_ERR_HIP = -6           /* a HIP runtime call or launch failed                  */
} la_status;

/*
 * Element types.  LA_FP8_E4M3 is an 8-bit float (OCP E4M3: bias 7, 3 mantissa
 * bits, largest finite 448, no infinities) used for quantised attention
 * operands (NOTES, Table 3: FP8 quantisation); a la_kvring of this dtype keeps
 * its K/V slots in e4m3 and its sink (raw K and V) in bf16, because the sink
 * is re-rotated at every block from its raw values.
 */
/* C++ gives the enum a fixed underlying type, so that any int a C caller passes is a
 * value of the type (validated by every call) rather than undefined behaviour. */
#ifdef __cplusplus
typedef enum la_dtype : int { LA_BF16 = 0, LA_F32 = 1, LA_FP8_E4M3 = 2 } la_dtype;
#else
typedef enum la_dtype { LA_BF16 = 0, LA_F32 = 1, LA_FP8_E4M3 = 2 } la_dtype;
#endif

typedef void* la_stream_t; /* hipStream_t */

#define LA_MAX_WINDOW 64
#define LA_MAX_BLOCK_FRAMES 4

/*
 * la_kvring - one layer's rolling noisy KV cache plus its attention sink.
 * A plain host struct owned by the caller; it only points at device memory.
 *
 *   k_slots, v_slots : device, [nslots][block_tokens][heads][head_dim] of dtype.
 *                      (dtype LA_FP8_E4M3: e4m3 codes; the sink stays bf16.)
 *                      Slot s holds block b with (b - 1) mod nslots == s.
 *   nslots           : W (la_kvring_init), or W + 1 (la_kvring_init_staged: one
 *                      slot beyond the window, where the next block's K and V can
 *                      be written before the block's attention has read the
 *                      window; the fused step below uses it).
 *   sink_k_raw       : device, [sink_tokens][heads][head_dim], the sink's
 *                      unrotated K (it is re-rotated at every block).
 *   sink_v           : device, same shape, the sink's V.
 *   slot_block[s]    : block id held by slot s (0 = empty).
 *   last_block       : id of the last appended block (0 = none yet).
 *   noise_level      : the stage's t_i; every cached entry is at this level.
 *   sink_replaced    : 1 after the one-time replacement.
 *
 * Ring rules (BLOG, 疑问 4; NOTES, 关键设计 2): the cache holds the K/V that
 * this stage computed from its own noisy input x_{t_i} for the last W blocks,
 * oldest evicted first, with no clean refresh.  The index fields are part of
 * the bit-exact contract and may be saved and restored together with the
 * device buffers to checkpoint a stage.
 */
typedef struct la_kvring {
  void* k_slots;
  void* v_slots;
  void* sink_k_raw;
  void* sink_v;
  int32_t W;
  int32_t nslots;
  int32_t block_tokens;
  int32_t sink_tokens;
  int32_t heads;
  int32_t head_dim;
  int32_t dtype;          /* la_dtype */
  float noise_level;
  int32_t sink_replaced;
  int64_t last_block;
  int64_t slot_block[LA_MAX_WINDOW];
} la_kvring;

/* Text for a status code (static storage). */
const char* la_status_string(int status);

/* Text of the last HIP error seen on this thread ("" if none). */
const char* la_last_hip_error(void);

/* Library version string (static storage). */
const char* la_version(void);

/*
 * la_kvring_init - fill *r for an empty window.  Pure host; touches no device
 * memory (the slot contents are unspecified until blocks are appended).
 * 1 <= W <= LA_MAX_WINDOW; all sizes > 0; pointers non-NULL and 16-byte aligned;
 * 8 <= head_dim <= 256, head_dim % 8 == 0; a slot (block_tokens * heads *
 * head_dim elements) and the sink must each be a multiple of 16 bytes, else
 * LA_ERR_SHAPE (this only restricts e4m3 rings).
 */
la_status la_kvring_init(la_kvring* r, void* k_slots, void* v_slots, void* sink_k_raw,
                         void* sink_v, int32_t W, int32_t block_tokens, int32_t sink_tokens,
                         int32_t heads, int32_t head_dim, la_dtype dtype, float noise_level);

/*
 * la_kvring_init_staged - la_kvring_init for a ring with one slot more than its
 * window: k_slots and v_slots hold W + 1 slots (W + 1 <= LA_MAX_WINDOW, else
 * LA_ERR_SHAPE).  The window and its rules are unchanged (the last W blocks
 * are attended to; block b - W leaves the window when block b is appended);
 * only the placement differs: block b goes to slot (b - 1) mod (W + 1), which
 * holds no block of the window while block b is being computed.  That lets a
 * step write the block's rotated K straight into its slot (la_kvring_next_slot)
 * instead of into a workspace that the append then copies: the pages' fused
 * kernels (NOTES, Table 3, FP8 + FlashAttention-3 + fused kernels).
 */
la_status la_kvring_init_staged(la_kvring* r, void* k_slots, void* v_slots, void* sink_k_raw,
                                void* sink_v, int32_t W, int32_t block_tokens,
                                int32_t sink_tokens, int32_t heads, int32_t head_dim,
                                la_dtype dtype, float noise_level);

/*
 * la_kvring_next_slot - device addresses of the K and V slot that block
 * r->last_block + 1 will occupy.  Pure host.  LA_ERR_STATE if that slot still
 * holds a block of the window (a ring of W slots with W blocks cached), since
 * writing it before the block's attention would change what the attention
 * reads; a staged ring's next slot is always free.
 */
la_status la_kvring_next_slot(const la_kvring* r, void** k_slot, void** v_slot);

/*
 * la_kvring_advance - where appending block `block_id` would go, without
 * changing anything.  Pure host.  *slot = (block_id - 1) mod nslots; *evicted =
 * the block that leaves the window (block_id - W) or 0 if none.  Returns
 * LA_ERR_STATE unless block_id == r->last_block + 1.
 */
la_status la_kvring_advance(const la_kvring* r, int64_t block_id, int32_t* slot,
                            int64_t* evicted);

/* Number of cached blocks, min(last_block, W).  Pure host. */
int32_t la_kvring_count(const la_kvring* r);

/*
 * 3D RoPE tables.  head_dim d is split into bands (d - 4*floor(d/6),
 * 2*floor(d/6), 2*floor(d/6)) for the (frame, h, w) axes; pair k of a band of
 * width w_a (dims 2k, 2k+1 of the band) turns by p * theta^(-2k/w_a), where
 * p is the token's coordinate on that axis: (x, y) -> (x cos - y sin,
 * x sin + y cos).  (The pages name RoPE over the video's positions without
 * its axes or base; this is the conventional 3D factorisation.)
 *
 * la_rope_table_bytes: size of the spatial (h, w) cos/sin table.
 * la_rope_table_fill:  compute it on the device in float64 and store float32
 *                      into dev_table (caller-owned, >= la_rope_table_bytes,
 *                      4-byte aligned).  Asynchronous on `stream`.
 */
size_t la_rope_table_bytes(int32_t Hl, int32_t Wl, int32_t head_dim);
la_status la_rope_table_fill(void* dev_table, int32_t Hl, int32_t Wl, int32_t head_dim,
                             double theta, la_stream_t stream);

/*
 * la_rope3d_rolling - Rolling RoPE for one block (NOTES, 关键设计 3: the sink's
 * temporal offset follows the active block so their relative distance stays
 * constant; POP, RSFM section: sink position = current position + a fixed
 * offset; BLOG, 疑问 5: after the one-time replacement only the sink's
 * position encoding changes).
 *
 *   q_in/q_out, k_in/k_out : [n_frames*Hl*Wl][heads][head_dim]; token
 *       (j*Hl + h)*Wl + w is rotated at (f0 + j, h, w).  Either pair may be
 *       NULL (skipped).  Out-of-place or in place (out == in).
 *   sink_k_in/sink_k_out   : [Hl*Wl][heads][head_dim], the raw sink K rotated
 *       at (f0 + sink_delta, h, w).  May be NULL (skipped).
 *   dev_table              : filled by la_rope_table_fill for (Hl, Wl, head_dim, theta).
 *   The temporal cos/sin are computed on the host in float64 for these
 *   positions at every call, so positions can grow without bound (10,000 s
 *   streams) without float32 angle error.
 *   dtype LA_BF16: bf16 in/out, float32 arithmetic, round-to-nearest-even
 *   store.  LA_F32: float32 throughout.  1 <= n_frames <= LA_MAX_BLOCK_FRAMES;
 *   head_dim % 8 == 0, 8 <= head_dim <= 256, and the frame band holds at most
 *   48 pairs.
 *   q_scale (> 0, finite): q_out = q_scale * (rotated q), multiplied in float32
 *   before the one rounding of the store (k_out and the sink are not scaled).
 *   1 gives the plain rotation; la_denoise_step passes scale * log2(e) so that
 *   the attention that follows takes its base-2 scores straight from Q K^T.
 *   Pointers must be 16-byte aligned.
 */
la_status la_rope3d_rolling(const void* q_in, void* q_out, const void* k_in, void* k_out,
                            int32_t n_frames, int64_t f0, const void* sink_k_in,
                            void* sink_k_out, int64_t sink_delta, const void* dev_table,
                            int32_t Hl, int32_t Wl, int32_t heads, int32_t head_dim,
                            la_dtype dtype, double theta, float q_scale, la_stream_t stream);

/*
 * la_block_attn_fwd - block attention of the current block (NOTES, 整体框架:
 * a block of 3 latent frames attends causally, at block granularity, to the
 * static sink frame and the sliding KV cache; 关键设计 2: the cache holds noisy
 * K/V at the block's own noise level).  For every head:
 *
 *     out = softmax(scale * Q K_all^T) V_all,
 *     K_all = [sink_k_rot ; cached blocks of r ; k_cur_rot]
 *     V_all = [r->sink_v  ; cached blocks of r ; v_cur]
 *
 * with no mask (the block sees itself bidirectionally; later blocks do not
 * exist yet; the order of the keys does not change the attention).  Reads
 * la_kvring_count(r) cached blocks; call it before appending the current block.
 *
 *   q_rot, k_cur_rot, v_cur, out : [n_q][heads][head_dim]; n_q = r->block_tokens.
 *       q_rot holds q_scale times the rotated query (q_scale as given to
 *       la_rope3d_rolling; 1 for the plain rotation): the scores are
 *       scale / q_scale * q_rot . k.
 *   sink_k_rot : [r->sink_tokens][heads][head_dim] (output of la_rope3d_rolling).
 *   lse_or_null: if non-NULL, float32 [heads][n_q] natural-log
 *                log(sum exp(scale q.k)) per row.
 *   scale, q_scale : > 0 and finite.
 *   workspace  : NULL, or device memory of at least la_attn_workspace_bytes(n_q,
 *                r->heads) bytes, 256-byte aligned, zero-filled before its first
 *                use (each call leaves it zero-filled again).  Without a workspace
 *                the bf16 kernel runs one workgroup per (head, 192-query tile).
 *                With one it runs a persistent grid of two workgroups per compute
 *                unit: whole rounds of query tiles, then, when the last round would
 *                leave more than half of the workgroups idle, the query tiles of
 *                that round are cut into equal key ranges whose partial results
 *                are merged (in a fixed order) by the last piece to finish.
 *                Results are deterministic either way (not bit-identical between
 *                the two when a round is cut).  Calls that share a workspace must
 *                not run concurrently.  Ignored for LA_F32.
 *   LA_BF16: bf16 MFMA products with float32 accumulation and a float32 online
 *            softmax in base 2, bf16 output (round-to-nearest-even); head_dim ==
 *            128.  The products take Q times scale * log2(e) / q_scale rounded to
 *            bf16, or q_rot unchanged when that factor is 1 in float32 (q_scale ==
 *            scale * log2(e) rounded to float32).  The keys are visited as the
 *            sink, then the cached blocks in slot (address) order, then the
 *            current block, with blocks whose K and V both continue in memory
 *            where the previous one ends (neighbouring slots; k_cur_rot and
 *            v_cur staged in the ring's next slot) taken as one run: the result
 *            is the same attention, rounded along that order.
 *   LA_F32 : float32 throughout; head_dim 64 or 128.
 *   Pointers 16-byte aligned; `out` must not alias an input.
 */
la_status la_block_attn_fwd(const la_kvring* r, const void* q_rot, const void* sink_k_rot,
                            const void* k_cur_rot, const void* v_cur, int32_t n_q, void* out,
                            float* lse_or_null, float scale, float q_scale, void* workspace,
                            size_t workspace_bytes, la_stream_t stream);

/*
 * la_block_attn_fwd_noalloc - la_block_attn_fwd with a workspace that is a
 * static device array of the library instead of caller memory.  For callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It calls no allocating routine.
 *   The array holds the arrival counters of at most 16,384 (head, 192-query
 *   tile) units and the partial records of 512 persistent workgroups (53.5 MB on
 *   each device the library runs on, held until the process ends); more units
 *   (n_q / 192 rounded up, times heads) return LA_ERR_SHAPE.  On a device with
 *   more than 256 compute units the persistent grid is limited to 512
 *   workgroups.  Each call clears the counters first (a fill kernel on `stream`).
 *   All calls on one device share the array: calls that overlap on a device
 *   race.  Arguments and results otherwise as la_block_attn_fwd with a workspace.
 */
la_status la_block_attn_fwd_noalloc(const la_kvring* r, const void* q_rot,
                                    const void* sink_k_rot, const void* k_cur_rot,
                                    const void* v_cur, int32_t n_q, void* out,
                                    float* lse_or_null, float scale, float q_scale,
                                    la_stream_t stream);

/*
 * la_attn_workspace_bytes - size of the la_block_attn_fwd workspace for n_q
 * queries and `heads` heads on the current device (an arrival counter per
 * 192-query tile and head, and one partial record of 104,448 bytes per
 * workgroup of the persistent grid, two workgroups per compute unit: 53.5 MB on
 * a 256-CU MI355X).  0 if an argument is invalid or the device cannot be queried.
 */
size_t la_attn_workspace_bytes(int32_t n_q, int32_t heads);

/*
 * la_kvcache_append_evict - put block `block_id`'s rotated K and its V
 * (both [block_tokens][heads][head_dim], computed by this stage from its own
 * noisy input, BLOG 疑问 4) into slot (block_id - 1) mod nslots, evicting block
 * block_id - W.  Requires block_id == r->last_block + 1 (else LA_ERR_STATE)
 * and noise_level == r->noise_level (else LA_ERR_NOISE_LEVEL: the timestep-
 * forcing rule of NEWS 方法概述, the cache and the latent share one noise
 * level).  *evicted_or_null receives the evicted id or 0.  The copy is
 * enqueued on `stream`; the index update happens at call time.  A k_rot (v)
 * that is the destination slot's own K (V) buffer, as la_kvring_next_slot
 * returns it, is already in place and is not copied; any other k_rot or v must
 * not overlap the destination slot.
 */
la_status la_kvcache_append_evict(la_kvring* r, const void* k_rot, const void* v,
                                  int64_t block_id, float noise_level,
                                  int64_t* evicted_or_null, la_stream_t stream);

/*
 * la_sink_replace - Adaptive Attention Sink (NOTES, 关键设计 3; BLOG, 疑问 5):
 * once, after the first block, copy the new raw sink K and V (each
 * [sink_tokens][heads][head_dim]) into r->sink_k_raw / r->sink_v.  A second
 * call returns LA_ERR_STATE and changes nothing; so does a call before block
 * 1 has been appended.
 */
la_status la_sink_replace(la_kvring* r, const void* k_new_raw, const void* v_new,
                          la_stream_t stream);

/*
 * la_fm_euler_step - flow-matching Euler update in place (NOTES, 损失函数:
 * the model predicts the velocity v of the path, v = x_1 - x_0):
 * x[i] = x[i] + dt * v[i] for 0 <= i < n, float32, one rounding per element
 * (fused multiply-add).  n == 0 is a no-op.  x and v must not overlap
 * partially (x == v is allowed).
 */
la_status la_fm_euler_step(float* x, const float* v, int64_t n, float dt, la_stream_t stream);

/*
 * la_denoise_step - one block through one timestep-forcing stage t_i -> t_{i-1}
 * (NOTES, 关键设计 4: each pipeline GPU runs one fixed denoise step with its
 * local noisy caches and hands only the latent on; BLOG, 疑问 6).  For every
 * layer l, in order, on `stream`:
 *   1. la_rope3d_rolling of q_raw[l], k_raw[l] at f0 = frames_per_block *
 *      (block_id - 1) into q_rot_ws / k_rot_ws, and of rings[l].sink_k_raw at
 *      f0 + sink_delta into sink_k_rot_ws;
 *   2. la_block_attn_fwd into attn_out[l];
 *   3. la_kvcache_append_evict of (k_rot_ws, v_raw[l]) as block block_id;
 *   4. if block_id == 1 and sink_k_new != NULL: la_sink_replace with
 *      (sink_k_new[l], sink_v_new[l]) (Adaptive Attention Sink, NOTES 关键设计 3);
 * then la_fm_euler_step(x, vel, n_latent, dt) if x != NULL.
 * Fused append (NOTES, Table 3, fused kernels): for a staged ring
 * (la_kvring_init_staged) and without LA_STEP_ATTEND_ONLY, step 1's launch writes
 * the rotated K straight into the ring's next slot (la_kvring_next_slot) instead
 * of k_rot_ws and copies v_raw[l] into the same slot (no block of the window uses
 * that slot); step 2 reads the block's K and V there, and step 3 only records the
 * block (nothing is left to copy).  The window's contents are the same bits as
 * with k_rot_ws; the outputs are the same bits as la_block_attn_fwd given the
 * slot's K and V.
 * Fused Q rotation (NOTES, Table 3, fused kernels; RoPE as in la_rope3d_rolling):
 * for bf16 rings with heads >= 2, step 1 rotates only K and the sink K and writes
 * the cos/sin of every block token's head_dim pairs, times q_scale (float32,
 * head_dim * 4 bytes a token), into q_rot_ws instead of the rotated Q; step 2's
 * attention kernel rotates the raw q_raw[l] with them as it loads its Q fragments,
 * with la_rope3d_rolling's arithmetic (one fma per output, bf16 round to nearest
 * even), so the results are the same bits as with the rotated Q.
 *
 * flags (bitwise or):
 *   LA_STEP_ATTEND_ONLY : skip steps 3 and 4 (no append, no sink replacement);
 *       the rings are read, not written.  For the pages' cache ablations (NOTES,
 *       Table 4: a clean cache instead of the step's own noisy one; NOTES,
 *       关键发现 on Table 6: a fixed-noise cache): the denoise stages attend to a
 *       shared cache that one other pass writes (a clean refresh pass at noise
 *       level 0, NFE 5, or the stage at the fixed level).  sink_k_new must be NULL.
 * The other ablations need no flag: Rolling RoPE off = pass sink_delta =
 * p_sink - f0 (the sink stays at p_sink, e.g. frame 0); AAS off = never pass a
 * replacement sink.
 *
 *   rings[n_layers]        : one la_kvring per layer, identical geometry and
 *                            noise level, all at last_block == block_id - 1.
 *   q_raw/k_raw/v_raw/attn_out : arrays of n_layers device pointers, each
 *                            [block_tokens][heads][head_dim].
 *   q_rot_ws, k_rot_ws     : device workspaces [block_tokens][heads][head_dim],
 *                            reused by every layer (stream order keeps them safe).
 *   sink_k_rot_ws          : device workspace [sink_tokens][heads][head_dim].
 *   rope_table             : la_rope_table_fill output for (Hl, Wl, head_dim, theta);
 *                            block_tokens must equal frames_per_block*Hl*Wl and
 *                            sink_tokens Hl*Wl.
 *   scale                  : softmax scale (1/sqrt(head_dim) for the model).  For
 *                            bf16 rings the rotated Q is multiplied by
 *                            scale * log2(e) (la_rope3d_rolling's q_scale) and the
 *                            attention takes it as given.
 *   attn_ws, attn_ws_bytes : the la_block_attn_fwd workspace shared by every
 *                            layer (NULL for none).
 *   timing_events          : NULL, or 6*n_layers + 2 caller-created hipEvent_t
 *                            (as void*) that take the begin and end timestamps of
 *                            each layer's RoPE kernel [6l, 6l+1], attention kernel
 *                            [6l+2, 6l+3] and append copy [6l+4, 6l+5] (the sink
 *                            replacement is not included), and of the Euler kernel
 *                            [6n, 6n+1]; they are given to the kernel launches
 *                            themselves, so a span is the kernel's own duration (an
 *                            operation that launches nothing records an empty span,
 *                            two event packets on the stream).  An entry may be
 *                            NULL: that timestamp is not taken (e.g. the append of
 *                            a staged ring, which launches nothing).
 * The whole step is validated before the first launch; on an error nothing is
 * enqueued and no ring changes.  Pointer arrays are host memory read at call
 * time.
 */
la_status la_denoise_step(la_kvring* rings, int32_t n_layers, int64_t block_id,
                          const void* const* q_raw, const void* const* k_raw,
                          const void* const* v_raw, void* const* attn_out, void* q_rot_ws,
                          void* k_rot_ws, void* sink_k_rot_ws, const void* const* sink_k_new,
                          const void* const* sink_v_new, const void* rope_table, int32_t Hl,
                          int32_t Wl, int32_t frames_per_block, int64_t sink_delta,
                          double theta, float scale, void* attn_ws, size_t attn_ws_bytes,
                          float* x, const float* vel, int64_t n_latent, float dt,
                          uint32_t flags, void* const* timing_events, la_stream_t stream);

#define LA_STEP_ATTEND_ONLY 1u

/*
 * la_denoise_step_fp8 - la_denoise_step with the attention on e4m3 operands, for
 * rings of dtype LA_FP8_E4M3 (NOTES, Table 3: FP8 quantisation together with
 * FlashAttention-3 and fused kernels).  For every layer l, in order, on `stream`:
 *   1. one launch: the rotations of la_rope3d_rolling (Q, K at the block's
 *      positions, the ring's raw sink K at the sink's; no Q pre-scale), each
 *      result rounded to bf16 and then quantised with its per-tensor scale as
 *      la_quantize_fp8 does (code = E4M3(x * fl32(1 / d))), together with the
 *      quantisation of v_raw[l] and of the ring's sink V: Q into q8_ws (dq), K (dk)
 *      and V (dv) into the ring's next slot when the ring is staged and the step
 *      appends (else into k8_ws and v8_ws), the sink K into sink_k8_ws (dk) and the
 *      sink V into sink_v8_ws (dv) - the same codes as la_rope3d_rolling to bf16
 *      followed by la_quantize_fp8, with no bf16 intermediate in memory;
 *   2. la_block_attn_fwd_fp8 of these codes with (dq, dk, dv) and `scale` into
 *      attn_out[l] (bf16);
 *   3. la_kvcache_append_evict of the block's K and V codes as block block_id
 *      (nothing is copied when they are already in the slot), and at block 1 the
 *      sink replacement, as in la_denoise_step;
 * then la_fm_euler_step(x, vel, n_latent, dt) if x != NULL.
 * Every ring is LA_FP8_E4M3 with head_dim 128 (else LA_ERR_DTYPE / LA_ERR_SHAPE);
 * dq, dk, dv finite and > 0 (else LA_ERR_INVALID_ARG).  Workspaces, 16-byte
 * aligned, caller-owned: q8_ws, k8_ws, v8_ws [block_tokens][heads][head_dim]
 * bytes (k8_ws and v8_ws may be NULL when every ring is staged and flags lacks
 * LA_STEP_ATTEND_ONLY), sink_k8_ws and sink_v8_ws [sink_tokens][heads][head_dim]
 * bytes; q_rot_ws, k_rot_ws and sink_k_rot_ws are not used (may be NULL).  q_raw,
 * k_raw, v_raw 16-byte aligned.  The other arguments, flags, timing events (the
 * first pair of a layer spans the RoPE and quantisation launch) and errors are
 * those of la_denoise_step (it takes no attention workspace).
 */
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
                              void* const* timing_events, la_stream_t stream);

/*
 * la_quantize_fp8 - per-tensor FP8 quantisation (NOTES, Table 3: FP8
 * quantisation).  out[i] = E4M3(in[i] * inv_scale) for 0 <= i < n, where the
 * product is one float32 multiplication and E4M3 rounds to the nearest
 * representable value (ties to even mantissa), keeps the sign of zero and
 * saturates magnitudes beyond 448 to 448.  The dequantised value of a code c is
 * decode(c) / inv_scale.
 *   in        : device, n elements of in_dtype (LA_BF16 or LA_F32), 16-byte aligned.
 *   out       : device, n bytes, 16-byte aligned, not overlapping in.
 *   inv_scale : > 0 and finite.
 * n == 0 is a no-op.  A NaN input gives the NaN code of its sign (0x7F, 0xFF).
 */
la_status la_quantize_fp8(const void* in, la_dtype in_dtype, void* out, int64_t n,
                          float inv_scale, la_stream_t stream);

/*
 * la_block_attn_fwd_fp8 - la_block_attn_fwd on e4m3 operands: out =
 * softmax(scale * (dq Q)(dk K_all)^T) (dv V_all) with Q, K, V given as e4m3
 * codes and one dequantisation factor per tensor (dq, dk, dv; a code's value
 * is decode(code) * factor).  Key set and order as in la_block_attn_fwd:
 * [sink ; cached slots oldest first ; the block itself], no mask.
 *   r            : ring of dtype LA_FP8_E4M3, head_dim 128; its slots hold e4m3
 *                  K (rotated) and V quantised with the same dk, dv.
 *   q8           : [n_q][heads][128] e4m3, n_q == r->block_tokens.
 *   sink_k8/_v8  : [sink_tokens][heads][128] e4m3, the rotated sink K and the
 *                  sink V for this block (the ring's bf16 sink, rotated and
 *                  quantised by the caller with la_rope3d_rolling and
 *                  la_quantize_fp8).
 *   k8_cur/v8_cur: [n_q][heads][128] e4m3, this block's rotated K and its V.
 *   out          : [n_q][heads][128] bf16 (not aliasing an input).
 *   lse_or_null  : NULL or [heads][n_q] float32: the natural log of the sum of
 *                  the rounded probabilities (see below) times exp(max logit),
 *                  i.e. the exact log-sum-exp of the dequantised logits to
 *                  within log(1 + 2^-4).
 * The probabilities are rounded to e4m3 for the P V product (relative error
 * <= 2^-4 per probability); the row sum that normalises the output is taken
 * from the same rounded probabilities.
 * Pointers 16-byte aligned (lse 4-byte); factors and scale > 0 and finite.
 * When the logit factor scale * dq * dk * log2(e) (float64 from the float32
 * arguments) lies within a relative 2^-24 of a power of two 2^e (-127 <= e <= 127),
 * the kernel applies 2^e through the score MFMA's operand scale and forms each
 * score's exponent inside the MFMA (no multiply-add per score; la_fp8_q_factor_pow2
 * picks such a dq).  The factor then differs from the exact one by no more than
 * the float32 product of the other path does (up to 3 * 2^-24).
 */
la_status la_block_attn_fwd_fp8(const la_kvring* r, const void* q8, const void* sink_k8,
                                const void* sink_v8, const void* k8_cur, const void* v8_cur,
                                int32_t n_q, void* out, float* lse_or_null, float scale,
                                float dq, float dk, float dv, la_stream_t stream);

/*
 * la_fp8_q_factor_pow2 - the least float dq >= dq_min for which the e4m3
 * attention's logit factor scale * dq * dk * log2(e) (float64 from the float32
 * arguments) lies within a relative 2^-24 of a power of two 2^e with
 * -127 <= e <= 127, in *dq_out: quantising Q with that dq
 * (la_quantize_fp8 with inv_scale 1 / dq) lets la_block_attn_fwd_fp8 and
 * la_denoise_step_fp8 take their faster path.  The FP8 scaling recipe is the
 * caller's choice (NOTES, Table 3 names FP8 without one): a dq at most about twice
 * dq_min keeps Q's range (448 dq) at least that of dq_min.  Host-only: no GPU call.
 *   scale, dk, dq_min : > 0 and finite (else LA_ERR_INVALID_ARG).
 *   dq_out            : non-NULL; written only on LA_OK.
 * LA_ERR_INVALID_ARG also when no such float exists (the factor overflows).
 */
la_status la_fp8_q_factor_pow2(float scale, float dk, float dq_min, float* dq_out);

/*
 * One stage of a timestep-forcing chain (la_denoise_chain): the per-layer
 * caches and inputs of the stage that takes the latent from its noise level t
 * to t + dt.  Field meanings are those of the la_denoise_step arguments of the
 * same names; sink_k_new / sink_v_new are used at block 1 only (may be NULL).
 */
typedef struct la_stage {
  la_kvring* rings;              /* n_layers rings, all at noise level t */
  const void* const* q_raw;      /* n_layers device pointers each */
  const void* const* k_raw;
  const void* const* v_raw;
  void* const* attn_out;
  const void* const* sink_k_new;
  const void* const* sink_v_new;
  const float* vel;              /* velocity at this stage's input, n_latent floats */
  float dt;                      /* step of this stage: t_next - t (negative) */
} la_stage;

/*
 * la_denoise_chain - one block through n_stages timestep-forcing stages in
 * order, all on one GPU (NEWS, 论文阅读: the framework also runs on a single
 * 80 GB card; NOTES, Table 3: four denoise steps on one GPU before the steps are
 * spread over GPUs; NOTES, 关键设计 4 and BLOG, 疑问 6: each stage keeps caches
 * at its own noise level and hands only the latent on).  Stage s is la_denoise_step(stages[s].rings, ...,
 * x, stages[s].vel, n_latent, stages[s].dt) with the shared workspaces (attn_ws
 * included), RoPE table and geometry; the latent x is updated in place stage
 * after stage.
 *
 * Besides every la_denoise_step check for every stage, the noise levels must
 * chain: stages[s+1].rings[*].noise_level == stages[s].rings[*].noise_level +
 * stages[s].dt (to 1e-6), else LA_ERR_NOISE_LEVEL, since the latent handed to
 * stage s+1 is at that level.  All stages are validated before the first
 * launch; on an error nothing is enqueued and no ring changes.  x and every
 * vel are required when n_latent > 0.
 */
la_status la_denoise_chain(la_stage* stages, int32_t n_stages, int32_t n_layers,
                           int64_t block_id, void* q_rot_ws, void* k_rot_ws,
                           void* sink_k_rot_ws, const void* rope_table, int32_t Hl, int32_t Wl,
                           int32_t frames_per_block, int64_t sink_delta, double theta,
                           float scale, void* attn_ws, size_t attn_ws_bytes, float* x,
                           int64_t n_latent, la_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LA_H_ */
