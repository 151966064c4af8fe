// Block attention, bf16 MFMA, head_dim 128, for gfx950 (CDNA4).
//
// out = softmax(scale * Q K_all^T) V_all per head, over the keys of a segment
// table {rotated sink, cached blocks, the block itself} with no mask
// (papernotes.org "Live Avatar: Streaming Real-time Audio-Driven Avatar
// Generation with Infinite Length", 整体框架 and 关键设计 2: a 3-latent-frame
// block attends to the sink frame and to the sliding noisy KV cache).
//
// Design (MI355X-first, not a port of the pages' FlashAttention):
//  * One workgroup = 4 waves = 192 query rows of one head, two workgroups per
//    CU (two waves per SIMD, from different workgroups, so one workgroup's
//    barrier does not stall the other's waves).  Each wave owns 48 query rows
//    (three 16-row tiles) for the whole key range and keeps its Q fragments,
//    the running row max / row sum and the output accumulator in registers.
//  * Products on v_mfma_f32_16x16x32_bf16: every K or V^T fragment read from
//    LDS feeds three MFMAs (one per query tile), 48 flops per LDS byte; the
//    LDS operand traffic, not the matrix core, bounded the earlier 32-row
//    waves on 32x32x16 MFMAs.  At 4680 rows a head takes 25 workgroups
//    (2.5 % padding), and 40 heads fill 512 CU slots in two rounds.
//  * Scores are computed transposed, S^T = K Q^T: in each 16x16 result a lane
//    holds one query (lane % 16) and four keys; the row max needs two lane
//    swaps (v_permlane32_swap, v_permlane16_swap).
//  * K rows sit in LDS in an order that moves key bit 2 to row bit 4 and key
//    bits 3-4 to row bits 2-3 (within each 32-key half); then rows 4g .. 4g+3
//    of the row blocks 2h and 2h+1 hold keys 32h + 8g .. 32h + 8g + 7, so the
//    probabilities P^T come out of the score accumulators already in the
//    B-operand layout of O^T = V^T P^T, with no shuffle.
//  * Each 64-key tile is processed as two 32-key halves (scores, softmax,
//    P V): 24 score and 24 output registers per half instead of 48, which
//    keeps the kernel within the 256 registers of two waves per SIMD.
//  * Online softmax in float32 with the scale folded into a base-2 exponent
//    (one FMA and one v_exp_f32 per score).  Probabilities are taken against
//    the running reference max without a per-tile max; only when a query's
//    sum over the half leaves [0, 2^64] (always on the first tile, whose
//    reference starts at -1e30) is the reference raised to the half's max, O
//    and the row sum rescaled and the half's probabilities recomputed.  Exact:
//    numerator and denominator use the same reference, and P <= 2^64 keeps
//    the float32 accumulators far from overflow.  P is rounded to bf16 for
//    the second product (v_cvt_pk_bf16_f32) and the row sum is taken from
//    those same bf16 pairs with v_dot2c_f32_bf16.
//  * K tiles go global -> LDS by DMA (buffer_load ... lds): no staging
//    registers, issued one tile ahead right after the barrier, so a whole
//    tile of compute hides their latency.  A DMA writes each wave's 1 KB
//    contiguously, so K rows have no padding (256-byte pitch) and each
//    16-byte chunk c of row r sits at chunk c ^ (r & 15), which keeps the
//    fragment reads free of bank conflicts.  Tiles that straddle a segment
//    boundary or run past the last key take a synchronous per-row copy.
//  * V stays key-major in LDS (64 rows of 128 dims, 256-byte pitch) and the A
//    operand of the second product (V^T: 16 dims x 8 keys per lane) is read
//    with two ds_read_b64_tr_b16: in each 16-lane group lane i receives, as
//    element j, element i & 3 of the 8 bytes lane 4j + (i >> 2) addresses
//    (measured on gfx950), so a lane that addresses key j, dims 4m .. 4m+3
//    feeds exactly the operand layout; no v_perm transpose in the loader.
//    V tiles also arrive by DMA (issued after the first half's scores), with
//    16-byte chunk c of key k at chunk c ^ (2 (k & 3) + 8 (bit 3 of k)): the
//    8 keys and two chunks a half-wave reads then fill all 64 banks once, and
//    the d-tile of a read is an XOR of one per-lane address with 32 dt.
//  * Loader addressing: buffer loads from a scalar descriptor per tile with
//    per-thread 32-bit offsets computed once; the current segment's key range
//    and base pointers stay in scalar registers (the segment table in kernel
//    arguments is read only when a tile enters the next segment).
//  * Workgroups are renumbered so that all query tiles of a head run on the
//    same XCD (dispatch is round-robin over the 8 XCDs) and share its L2 while
//    they stream the head's K/V.
#include "la_internal.h"

namespace la {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int D = 128;
constexpr int NQT = 3;           // 16-query tiles per wave
constexpr int QW = 16 * NQT;     // query rows per wave
constexpr int NWAVES = 4;
constexpr int BM = QW * NWAVES;  // query rows per workgroup
constexpr int BN = 64;           // keys per tile
constexpr int NTHREADS = 64 * NWAVES;
constexpr int KP = 128;  // K row pitch in LDS (bf16): 256 B, chunks XOR-swizzled by row
constexpr int VP = 128;  // V row pitch in LDS (bf16): 256 B, key-major, chunks XOR-swizzled
constexpr int KBUF = BN * KP;
constexpr int VBUF = BN * VP;
constexpr int STAGE = KBUF + VBUF;
constexpr int kBufWord3 = 0x00020000;  // buffer descriptor word 3: raw 32-bit loads
constexpr uint32_t kSumLimitBits = 0x5f800000u;  // 2^64: a half's row sum above it
                                                 // raises the reference

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// max / sum over the four lanes c, c + 16, c + 32, c + 48 (one query's keys)
__device__ __forceinline__ float max4_lanes(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float sum4_lanes(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// Tile key held by LDS K row r (r = 0..63): row bits (5 | 4 | 3,2 | 1,0) are
// key bits (5 | 2 | 4,3 | 1,0).
__device__ __forceinline__ int key_of_krow(int r) {
  return (r & 32) | (((r >> 2) & 3) << 3) | (((r >> 4) & 1) << 2) | (r & 3);
}

__global__ __attribute__((amdgpu_flat_work_group_size(NTHREADS, NTHREADS),
                          amdgpu_waves_per_eu(2, 2))) void
attn_bf16_kernel(const uint16_t* __restrict__ q, uint16_t* __restrict__ out,
                 float* __restrict__ lse, const AttnSegs segs, int nq, int nk, int heads,
                 float c2, int qtiles, int nwg) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];

  // XCD-aware renumbering: consecutive logical ids on one XCD.
  const int pid = __builtin_amdgcn_workgroup_id_x();
  const int per = (nwg + 7) / 8;
  const int tall = (nwg % 8) == 0 ? 8 : (nwg % 8);
  const int xcd = pid % 8, loc = pid / 8;
  const int lin = xcd < tall ? xcd * per + loc : tall * per + (xcd - tall) * (per - 1) + loc;
  const int head = lin / qtiles;
  const int qt = lin - head * qtiles;

  const int tid = __builtin_amdgcn_workitem_id_x();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar
  const int c = lane & 15;  // query (scores) / row (operands) within a 16-tile
  const int g = lane >> 4;  // 8-element k-group of the operands
  const int64_t rs = (int64_t)heads * D;
  const int qbase = qt * BM + wave * QW;

  // Q^T B-operand fragments: lane holds Q[query qbase + 16 nt + c][32 s + 8 g .. +7].
  bf16x8_t qf[NQT][4];
#pragma unroll
  for (int nt = 0; nt < NQT; ++nt) {
    const int qrow = qbase + 16 * nt + c;
    if (qrow < nq) {
      const uint16_t* qp = q + qrow * rs + head * D + 8 * g;
#pragma unroll
      for (int s = 0; s < 4; ++s) qf[nt][s] = *reinterpret_cast<const bf16x8_t*>(qp + 32 * s);
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) qf[nt][s] = bf16x8_t{};
    }
  }

  f32x4_t o[8][NQT];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) o[dt][nt] = f32x4_t{};
  // Reference max (scale*log2(e) units) and this lane's row sum.  The reference
  // starts finite, so the first tile's probabilities overflow to +inf (never
  // NaN, even where masked keys hold -inf) and trigger the first raise.
  float m_run[NQT], l_run[NQT];
#pragma unroll
  for (int nt = 0; nt < NQT; ++nt) {
    m_run[nt] = -1e30f;
    l_run[nt] = 0.f;
  }

  // Loader geometry.  K DMA: wave w fills LDS rows 16 w + 4 i + t (t = lane
  // >> 4, i = 0..3), lane slot p = lane & 15 of a row receiving chunk
  // p ^ (row & 15) of key 32 (w >> 1) + 4 (w & 1) + 8 i + t.
  const int t4 = lane >> 4;
  const int ntiles = (nk + BN - 1) / BN;
  const uint32_t rs_bytes = (uint32_t)rs * 2u;
  const uint32_t hoff = (uint32_t)(head * D * 2);
  const uint32_t kkey0 = (uint32_t)(32 * (wave >> 1) + 4 * (wave & 1) + t4);
  uint32_t kdoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    kdoff[i] = kkey0 * rs_bytes + 16u * (uint32_t)((lane & 15) ^ (4 * i + t4));
  // V DMA: wave w fills key rows 16 w + 4 i + t, slot p receiving chunk
  // p ^ vswz(row), vswz(k) = 2 (k & 3) + 8 (bit 3 of k)
  const uint32_t vkey0 = (uint32_t)(16 * wave + t4);
  const uint32_t vdoff[2] = {vkey0 * rs_bytes + 16u * (uint32_t)((lane & 15) ^ (2 * t4)),
                             vkey0 * rs_bytes + 16u * (uint32_t)((lane & 15) ^ (2 * t4 + 8))};
  // V operand read: this lane's key 8 g + (c >> 2) (+ 4 B + 32 h), bytes 32 dt + 8 (c & 3)
  // of the row, i.e. chunk (2 dt + bit 1 of c) ^ vswz(key); XOR with 32 dt selects the d-tile
  const uint32_t vlane = (uint32_t)((8 * g + (c >> 2)) * 2 * VP + 16 * ((c >> 1) & 1) +
                                    16 * (2 * (c >> 2) + 8 * (g & 1)) + 8 * (c & 1));

  // Segment of the tile being loaded, kept in scalar registers: the segment
  // table is read only when a tile crosses into the next segment.
  int seg = 0, seg_start = 0, seg_end = segs.end[0];
  const char* seg_k = static_cast<const char*>(segs.k[0]);
  const char* seg_v = static_cast<const char*>(segs.v[0]);
  bool whole = true;             // tile inside one segment
  uint32_t sbase = 0, nbytes = 0;  // tile's byte offset in the segment, bytes left from there

  auto locate = [&](int tile) __attribute__((always_inline)) {
    const int t0 = tile * BN;
    while (t0 >= seg_end) {
      ++seg;
      seg_start = seg_end;
      seg_end = segs.end[seg];
      seg_k = static_cast<const char*>(segs.k[seg]);
      seg_v = static_cast<const char*>(segs.v[seg]);
    }
    whole = t0 + BN <= seg_end;
    sbase = (uint32_t)(t0 - seg_start) * rs_bytes + hoff;
    nbytes = (uint32_t)(seg_end - t0) * rs_bytes - hoff;
  };
  // one 16-byte chunk of tile row r; rows past the last key are clamped to it
  // (their scores are masked)
  auto row_load = [&](int t0, int r, int chunk, bool is_v) __attribute__((always_inline)) -> uint4 {
    const int key = min(t0 + r, nk - 1);
    int s = seg;
    while (key >= segs.end[s]) ++s;
    const int st = s ? segs.end[s - 1] : 0;
    const int64_t o = (int64_t)(key - st) * rs + head * D + chunk * 8;
    const uint16_t* base = static_cast<const uint16_t*>(is_v ? segs.v[s] : segs.k[s]);
    return *reinterpret_cast<const uint4*>(base + o);
  };
  auto kload = [&](int tile, int buf) __attribute__((always_inline)) {
    uint16_t* kb = lds + buf * STAGE;
    if (whole) {
      const __amdgpu_buffer_rsrc_t kr =
          __builtin_amdgcn_make_buffer_rsrc((void*)(seg_k + sbase), 0, nbytes, kBufWord3);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            kr, (__attribute__((address_space(3))) void*)(kb + (16 * wave + 4 * i) * KP), 16,
            kdoff[i], 8 * i * rs_bytes, 0, 0);
    } else {
      const int t0 = tile * BN;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * wave + 4 * i + t4;
        const uint4 x = row_load(t0, key_of_krow(r), (lane & 15) ^ (r & 15), false);
        *reinterpret_cast<uint4*>(kb + r * KP + (lane & 15) * 8) = x;
      }
    }
  };
  auto vload = [&](int tile, int buf) __attribute__((always_inline)) {
    uint16_t* vb = lds + buf * STAGE + KBUF;
    if (whole) {
      const __amdgpu_buffer_rsrc_t vr =
          __builtin_amdgcn_make_buffer_rsrc((void*)(seg_v + sbase), 0, nbytes, kBufWord3);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            vr, (__attribute__((address_space(3))) void*)(vb + (16 * wave + 4 * i) * VP), 16,
            vdoff[i >> 1], 4 * i * rs_bytes, 0, 0);
    } else {
      const int t0 = tile * BN;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * wave + 4 * i + t4;
        const int sw = 2 * (r & 3) + 8 * ((r >> 3) & 1);
        const uint4 x = row_load(t0, r, (lane & 15) ^ sw, true);
        *reinterpret_cast<uint4*>(vb + r * VP + (lane & 15) * 8) = x;
      }
    }
  };

  typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
  const bf16x2v_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  locate(0);
  kload(0, 0);
  vload(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): tile 0's K DMA has landed
  // One 64-key tile j computed from LDS buffer `cur` while tile j + 1 is staged
  // into buffer 1 - cur.  The loop below runs two tiles per trip so that both
  // buffers are compile-time constants (LDS addresses become immediates).
  auto tile = [&](const int j, const int cur) __attribute__((always_inline)) {
    __syncthreads();
    const bool more = j + 1 < ntiles;
    if (more) {
      locate(j + 1);
      kload(j + 1, 1 - cur);
    }
    const uint16_t* kb = lds + cur * STAGE;
    // K fragment: row 16 blk + c, chunk 4 s + g, stored at chunk (4 s + g) ^ c
    const uint16_t* kr = kb + c * KP;
    // V operand by transposing reads (B = 0, 1 for keys + 0..3, + 4..7): this lane
    // addresses key 32 h + 8 g + (c >> 2) + 4 B, dims 16 dt + 4 (c & 3) .. +3, which
    // sits in LDS row 32 h + 16 (g >> 1) + 8 B + 4 (g & 1) + (c >> 2)
    const char* vt = reinterpret_cast<const char*>(kb + KBUF);

#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // S^T[key][query] for keys 32 h .. 32 h + 31: row blocks 2 h and 2 h + 1.
      f32x4_t st[2][NQT];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int nt = 0; nt < NQT; ++nt) st[b][nt] = f32x4_t{};
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(
              kr + 16 * (2 * h + b) * KP + (((4 * s + g) ^ c) * 8));
#pragma unroll
          for (int nt = 0; nt < NQT; ++nt)
            st[b][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[nt][s], st[b][nt], 0, 0, 0);
        }
      if (h == 0 && more) vload(j + 1, 1 - cur);
      if ((j + 1) * BN > nk) {
        // last tile: row 4 g + i of block 2 h + b holds key 32 h + 8 g + 4 b + i
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (j * BN + 32 * h + 8 * g + 4 * b + i >= nk) {
#pragma unroll
              for (int nt = 0; nt < NQT; ++nt) st[b][nt][i] = -INFINITY;
            }
          }
      }

      // P^T fragment of query tile nt: keys 32 h + 8 g .. +7, i.e. rows
      // 4 g .. 4 g + 3 of both row blocks; tsum = this lane's sum of them.
      bf16x8_t pf[NQT];
      float tsum[NQT];
      auto probs = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int nt = 0; nt < NQT; ++nt) {
          const float nm = -m_run[nt];
          uint32_t w[4];
          float ts = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(st[e >> 1][nt][2 * (e & 1)], c2, nm));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(st[e >> 1][nt][2 * (e & 1) + 1], c2, nm));
            w[e] = pack_bf16(p0, p1);
            ts = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, w[e]), ones, ts,
                                                 false);
          }
          tsum[nt] = ts;
          pf[nt] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
        }
      };
      probs();
      bool over = false;
#pragma unroll
      for (int nt = 0; nt < NQT; ++nt)  // on the bits (sums are >= +0): also inf and any NaN,
        over |= __float_as_uint(tsum[nt]) > kSumLimitBits;  // whatever the NaN flags
      if (__builtin_amdgcn_ballot_w64(over) != 0) {
#pragma unroll
        for (int nt = 0; nt < NQT; ++nt) {
          const float a =
              fmaxf(fmaxf(fmaxf(st[0][nt][0], st[0][nt][1]), fmaxf(st[0][nt][2], st[0][nt][3])),
                    fmaxf(fmaxf(st[1][nt][0], st[1][nt][1]), fmaxf(st[1][nt][2], st[1][nt][3])));
          const float m_new = fmaxf(m_run[nt], max4_lanes(a) * c2);
          const float alpha = __builtin_amdgcn_exp2f(m_run[nt] - m_new);
          m_run[nt] = m_new;
          l_run[nt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) o[dt][nt] *= alpha;
        }
        probs();
      }
#pragma unroll
      for (int nt = 0; nt < NQT; ++nt) l_run[nt] += tsum[nt];

      // O^T[d][query] += V^T P^T: A operand = V^T[16 dt + c][32 h + 8 g .. +7]
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const char* va = vt + (vlane ^ (32 * dt)) + 64 * h * VP;
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(va));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(va + 4 * 2 * VP));
        const bf16x8_t a =
            __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int nt = 0; nt < NQT; ++nt)
          o[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[nt], o[dt][nt], 0, 0, 0);
      }
    }
    if (more) {
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the next tile's K DMA has landed
    }
  };
  for (int j = 0; j < ntiles; j += 2) {
    tile(j, 0);
    if (j + 1 < ntiles) tile(j + 1, 1);
  }

#pragma unroll
  for (int nt = 0; nt < NQT; ++nt) {
    const float lt = sum4_lanes(l_run[nt]);
    const int qrow = qbase + 16 * nt + c;
    if (qrow < nq) {
      const float inv = 1.f / lt;
      uint16_t* op = out + qrow * rs + head * D + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const uint32_t w0 = pack_bf16(o[dt][nt][0] * inv, o[dt][nt][1] * inv);
        const uint32_t w1 = pack_bf16(o[dt][nt][2] * inv, o[dt][nt][3] * inv);
        *reinterpret_cast<uint2*>(op + 16 * dt) = make_uint2(w0, w1);
      }
      if (lse != nullptr && g == 0)
        lse[(int64_t)head * nq + qrow] = (m_run[nt] + __log2f(lt)) * 0.69314718055994531f;
    }
  }
}

}  // namespace

hipError_t launch_attn_bf16(const void* q, void* out, float* lse, const AttnSegs& segs, int nq,
                            int nk, int heads, float scale, hipStream_t s) {
  const int qtiles = (nq + BM - 1) / BM;
  const float c2 = scale * 1.4426950408889634f;
  hipLaunchKernelGGL(attn_bf16_kernel, dim3(qtiles * heads), dim3(NTHREADS), 0, s,
                     static_cast<const uint16_t*>(q), static_cast<uint16_t*>(out), lse, segs, nq,
                     nk, heads, c2, qtiles, qtiles * heads);
  return hipGetLastError();
}

}  // namespace la
