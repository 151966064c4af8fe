// Block attention on FP8 (e4m3) Q, K and V, head_dim 128, for gfx950 (CDNA4).
//
// out = softmax(scale * (dq Q8)(dk K8)^T) (dv V8) per head over the keys of a
// segment table {sink, cached blocks, the block itself}, no mask: the block
// attention of papernotes.org "Live Avatar: Streaming Real-time Audio-Driven
// Avatar Generation with Infinite Length" (整体框架, 关键设计 2) on tensors
// quantised to 8 bits per element with one scale per tensor (the same notes,
// Table 3: FP8 quantisation is part of the operator-level optimisation).
//
// Design (gfx950-native):
//  * 4 waves x 32 query rows per workgroup, 64-key tiles double-buffered in LDS,
//    one barrier per tile, Q fragments and the output accumulator in registers.
//    Three waves per SIMD (<= 168 registers, 32 KB of LDS per workgroup, three
//    workgroups per CU): with the tiles arriving by DMA the kernel needs no
//    staging registers and fits 168 without spilling, and the third wave hides
//    more of the LDS latency (10 % faster than two waves per SIMD with the tiles
//    loaded through registers).
//  * K and V tiles go global -> LDS by DMA (buffer_load ... lds), issued for the
//    next tile right after the barrier: a DMA writes each wave's 1 KB
//    contiguously, so tile rows have no padding (128-byte pitch) and each
//    16-byte chunk c of a row sits at chunk c ^ swizzle(row), which keeps the
//    fragment reads free of bank conflicts.  One scalar buffer descriptor per
//    tile (segment base + tile row + head, record count = the segment's
//    remaining bytes): rows past a segment's end read as zeros.
//  * Each segment of the key table is tiled on its own (the last tile of a
//    segment partial, its missing keys masked), so no tile straddles two
//    segments.
//  * Both products run on v_mfma_f32_32x32x64_f8f6f4 (e4m3 x e4m3, float32
//    accumulate): S^T = K Q^T is 4 MFMAs per tile, O^T += V^T P^T another 4.
//  * The MFMA takes A[i][k] and B[k][j] from lane bytes under one fixed (lane,
//    byte) -> k assignment; any assignment shared by A and B gives the same
//    product, so the kernel picks its own: for S, lane l holds dims
//    64 ks + 32 (l / 32) + j of its row; for P V, keys 32 (l / 32) + j.
//  * K rows are fed to the score MFMA in the order that makes accumulator row
//    i of key block b hold key 32 ((i / 4) % 2) + 16 b + 4 (i / 8) + i % 4.
//    Then lane l's 32 scores are keys 32 (l / 32) .. +31 in byte order, so P
//    packs straight into the B operand of the second product.  The DMA places
//    each key in that order directly.
//  * V stays key-major in LDS and the A operand of the second product (32 dims
//    x 32 keys per lane) is read with four ds_read_b64_tr_b8: in each 16-lane
//    group lane i receives, as byte j, byte i & 7 of the 8 bytes lane
//    2j + (i >> 3) addresses (measured on gfx950), so lanes addressing 8 dims
//    of one key hand every lane the 8 keys of its dim.
//  * Softmax in float32 with scale * dq * dk * log2(e) folded into the exponent;
//    P = exp2(s - m + 6) rounded to e4m3 (the 2^6 lifts small probabilities out
//    of the subnormal range).  When that factor is a power of two to within a
//    relative 2^-24 (the caller picks dq for it), the score MFMA applies that
//    power as its E8M0 operand scale and takes 6 - m as its accumulator input,
//    so each score leaves the MFMA as its exponent and costs one v_exp_f32
//    instead of a multiply-add and the exp (1.7 % faster at the C2 shape; the
//    input is formed per tile, because keeping it live spilled a Q fragment).
//  * Issue priority (s_setprio) is raised while a wave computes its tile's
//    probabilities, as in the bf16 kernel.
//  * The row sum is one more MFMA per tile, of an all-ones A operand with the
//    same e4m3 P: it moves 32 additions per lane off the VALU, which bounds
//    this kernel, and numerator and denominator use the same rounded P.
//  * No per-tile max: P is computed against the current reference m, and a P
//    past the e4m3 range converts to a NaN code, which the row-sum MFMA
//    carries; only then (always on the first tile, whose reference starts at
//    -1e30, and whenever a tile's max exceeds m by about 2^2.8) is m raised to
//    the tile's max, O and the sum rescaled and the tile redone before its P V
//    product.  This saves the 24 max instructions of every other tile.
//    The output is multiplied by dv and divided by the sum.
#include "la_internal.h"

namespace la {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int D = 128;  // head_dim = bytes per row
constexpr int BM = 128;  // query rows per workgroup
// Third descriptor word of a raw buffer resource on gfx9 (32-bit data format,
// no swizzle): the same value the ROCm libraries use for gfx90a/gfx942/gfx950.
constexpr int kBufWord3 = 0x00020000;
constexpr int BN = 64;   // keys per tile
constexpr int NWAVES = 4;
constexpr int NTHREADS = 64 * NWAVES;
// K and V tiles in LDS: 64 rows of 128 bytes (no padding: a DMA writes each
// wave's 1 KB contiguously), 16-byte chunks XOR-swizzled per row.
constexpr int KBUF = BN * D;
constexpr int VBUF = BN * D;
constexpr float kPLift = 6.f;         // P is computed as exp2(s - m + 6)

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ float swap_halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Key held by LDS row R of a K tile (the rows are in the order that makes
// accumulator row i of key block b hold key 32 ((i / 4) % 2) + 16 b + 4 (i / 8) + i % 4).
__device__ __forceinline__ int k_row_key(int R) {
  return 32 * ((R >> 2) & 1) + 16 * (R >> 5) + 4 * ((R >> 3) & 3) + (R & 3);
}
// 16-byte chunk swizzles: chunk c of K row R sits at c ^ kswz(R); chunk c of V key
// row k at c ^ vswz(k).  16 lanes reading one chunk of 16 consecutive K rows, and
// 32 lanes reading two neighbouring chunks of 8 consecutive V keys, then cover the
// 64 banks once.
__device__ __forceinline__ int kswz(int R) { return (R >> 1) & 7; }
__device__ __forceinline__ int vswz(int k) { return ((k >> 1) & 3) << 1; }

__device__ __forceinline__ f32x16_t mma(const i32x8_t& a, const i32x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// The same product with A scaled by 2^(sc - 127) (the MFMA's E8M0 operand scale; B by
// 2^0): c + 2^(sc - 127) A B, measured exact on gfx950 for powers of two.
__device__ __forceinline__ f32x16_t mma_scaled(const i32x8_t& a, const i32x8_t& b,
                                               const f32x16_t& c, int sc) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sc, 0, 127);
}

// kFold: the logit factor is 2^(sc - 127) (to 2^-24), applied by the score MFMA's
// operand scale, and the MFMA's accumulator input carries the reference (6 - m): the
// scores come out in the exponent's units and P = exp2(S) needs no multiply-add.
template <bool kFold>
__global__ __attribute__((amdgpu_flat_work_group_size(NTHREADS, NTHREADS),
                          amdgpu_waves_per_eu(3, 3))) void
attn_fp8_kernel(const uint8_t* __restrict__ q, uint16_t* __restrict__ out,
                float* __restrict__ lse, const AttnSegs segs, int nq, int heads,
                float c2, int sc, float dv, float ln_scale, int qtiles, int nwg) {
  // The K and V buffers of the two stages are separate objects, so that the compiler
  // can tell a DMA into one stage from the fragment reads of the other.
  __shared__ __attribute__((aligned(16))) uint8_t lds_k0[KBUF], lds_v0[VBUF], lds_k1[KBUF],
      lds_v1[VBUF];
  auto kbuf = [&](int buf) __attribute__((always_inline)) -> uint8_t* {
    return buf ? lds_k1 : lds_k0;
  };
  auto vbuf = [&](int buf) __attribute__((always_inline)) -> uint8_t* {
    return buf ? lds_v1 : lds_v0;
  };

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
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int64_t rs = (int64_t)heads * D;  // row stride in bytes
  const uint32_t rs32 = (uint32_t)rs;
  const uint32_t hoff = (uint32_t)(head * D);
  const int ntiles = segs.tend[segs.nseg - 1];

  // Q^T B-operand fragments: lane holds bytes 64 ks + 32 hh .. +31 of its query row.
  const int qrow = qt * BM + wave * 32 + l32;
  i32x8_t qf[2];
  if (qrow < nq) {
    const uint8_t* qp = q + qrow * rs + hoff + 32 * hh;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint4 a = *reinterpret_cast<const uint4*>(qp + 64 * ks);
      const uint4 b = *reinterpret_cast<const uint4*>(qp + 64 * ks + 16);
      qf[ks] = i32x8_t{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z,
                       (int)b.w};
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) qf[ks] = i32x8_t{};
  }

  f32x16_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16_t{};
  // Reference max (exp2 units).  Without kFold it starts at -1e30 (finite: no
  // inf - inf), so that the first tile's probabilities overflow and set it.  With kFold
  // the scores carry 6 - m_run from the MFMA's accumulator input, which must not
  // swamp them: m_run starts at 6 (the input is 0) and the first tile always sets it.
  float m_run = kFold ? kPLift : -1e30f;
  float l_run = 0.f;  // running sum of the lifted, rounded P of this lane's query
  const i32x8_t ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                        0x38383838, 0x38383838, 0x38383838, 0x38383838};  // e4m3 1.0

  // DMA geometry.  Wave w fills LDS rows 16 w + 8 n + (lane >> 3) (n = 0, 1) of each
  // tile; lane slot p = lane & 7 of a row receives chunk p ^ swizzle(row) of its key.
  // K: LDS row R holds key k_row_key(R); V: row k holds key k.
  uint32_t kdoff[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int R = 16 * wave + 8 * n + (lane >> 3);
    kdoff[n] = (uint32_t)k_row_key(R) * rs32 + 16u * (uint32_t)((lane & 7) ^ kswz(R));
  }
  const int vk = 16 * wave + (lane >> 3);  // row of n = 0; n = 1 is 8 rows (same swizzle) on
  const uint32_t vdoff = (uint32_t)vk * rs32 + 16u * (uint32_t)((lane & 7) ^ vswz(vk));

  // Fragment reads.  K (A operand of S^T): row 32 b + l32, logical chunks 4 ks + 2 hh
  // and + 1 (bytes 64 ks + 32 hh .. +31), each at its swizzled place.
  const int ks_sw = kswz(l32);
  uint32_t kro[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int e = 0; e < 2; ++e)
      kro[ks][e] = (uint32_t)(l32 * D + 16 * ((4 * ks + 2 * hh + e) ^ ks_sw));
  // V^T (A operand of O^T): in each 16-lane group lane s addresses key
  // 32 hh + 8 r + (s >> 1), dims 32 db + 16 ((lane >> 4) & 1) + 8 (s & 1) .. +7, i.e.
  // chunk 2 db + ((lane >> 4) & 1) of that key at its swizzled place
  const int s16 = lane & 15;
  const int vsw = vswz(s16 >> 1);  // the key's swizzle (8 r and 32 hh leave it unchanged)
  uint32_t vro[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
    vro[db] = (uint32_t)((32 * hh + (s16 >> 1)) * D +
                         16 * ((2 * db + ((lane >> 4) & 1)) ^ vsw) + 8 * (s16 & 1));

  // Segment of the tile being loaded (scalar registers): each segment is tiled on
  // its own, its last tile partial.
  int seg = 0, seg_t1 = segs.tend[0], seg_len = segs.end[0], seg_t0 = 0;
  const uint8_t* seg_k = static_cast<const uint8_t*>(segs.k[0]);
  const uint8_t* seg_v = static_cast<const uint8_t*>(segs.v[0]);
  uint32_t sbase = 0, nbytes = 0;
  int valid = BN;
  auto locate = [&](int tile) __attribute__((always_inline)) {
    while (tile >= seg_t1) {
      seg_len = segs.end[seg + 1] - segs.end[seg];
      ++seg;
      seg_t0 = seg_t1;
      seg_t1 = segs.tend[seg];
      seg_k = static_cast<const uint8_t*>(segs.k[seg]);
      seg_v = static_cast<const uint8_t*>(segs.v[seg]);
    }
    const int r0 = (tile - seg_t0) * BN;
    valid = seg_len - r0 < BN ? seg_len - r0 : BN;
    sbase = (uint32_t)r0 * rs32 + hoff;
    nbytes = (uint32_t)(seg_len - r0) * rs32 - hoff;
  };
  auto kload = [&](int buf) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(seg_k + sbase), 0, nbytes, kBufWord3);
    uint8_t* kb = kbuf(buf);
#pragma unroll
    for (int n = 0; n < 2; ++n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          kr, (__attribute__((address_space(3))) void*)(kb + (16 * wave + 8 * n) * D), 16,
          kdoff[n], 0, 0, 0);
  };
  auto vload = [&](int buf) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(seg_v + sbase), 0, nbytes, kBufWord3);
    uint8_t* vb = vbuf(buf);
#pragma unroll
    for (int n = 0; n < 2; ++n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          vr, (__attribute__((address_space(3))) void*)(vb + (16 * wave + 8 * n) * D), 16,
          vdoff, 8 * n * rs32, 0, 0);
  };
  auto kvload = [&](int buf) __attribute__((always_inline)) {
    kload(buf);
    vload(buf);
  };

  // Zero both V buffers once: the rows of a segment's partial last tile past its end
  // are masked (P = 0 exactly) but still enter P V, so they must hold finite codes;
  // the DMA leaves either zeros there (rows outside the buffer descriptor) or the V
  // rows of an earlier tile.
#pragma unroll
  for (int i = 0; i < VBUF / (16 * NTHREADS); ++i) {
    reinterpret_cast<uint4*>(lds_v0)[i * NTHREADS + tid] = make_uint4(0, 0, 0, 0);
    reinterpret_cast<uint4*>(lds_v1)[i * NTHREADS + tid] = make_uint4(0, 0, 0, 0);
  }
  __syncthreads();
  locate(0);
  int valid_next = valid;
  kvload(0);
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the first tile's DMA has landed

  // One 64-key tile j from LDS buffer `cur` while tile j + 1 is staged into
  // 1 - cur.  The loop runs two tiles per trip so that both buffers are
  // compile-time constants (immediate LDS offsets).
  auto tile = [&](const int j, const int cur) __attribute__((always_inline)) {
    __syncthreads();
    const int nvalid = valid_next;
    const bool more = j + 1 < ntiles;
    if (more) {
      locate(j + 1);
      valid_next = valid;
      kvload(1 - cur);
    }
    const uint8_t* kb = kbuf(cur);
    const uint8_t* vb = vbuf(cur);

    // S^T for the two 32-row key blocks: A = LDS row 32 b + l32, bytes 64 ks + 32 hh ..
    auto kfrag = [&](int b, int ks) __attribute__((always_inline)) -> i32x8_t {
      const uint4 x0 = *reinterpret_cast<const uint4*>(kb + b * 32 * D + kro[ks][0]);
      const uint4 x1 = *reinterpret_cast<const uint4*>(kb + b * 32 * D + kro[ks][1]);
      return i32x8_t{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                     (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    };
    // the last tile of a segment: x[b][r] holds key 32 hh + 16 b + r of the tile
    auto mask = [&](f32x16_t (&x)[2]) __attribute__((always_inline)) {
      if (__builtin_expect(nvalid < BN, 0)) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * hh + 16 * b + r >= nvalid) x[b][r] = -INFINITY;
      }
    };
    f32x16_t st[2];
    if constexpr (kFold) {
      // S^T c2 + 6 - m: the exponents of the lifted probabilities (the accumulator
      // input formed here each tile: 16 registers fewer live across the loop)
      f32x16_t cref;
#pragma unroll
      for (int i = 0; i < 16; ++i) cref[i] = kPLift - m_run;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int b = 0; b < 2; ++b) st[b] = mma_scaled(kfrag(b, ks), qf[ks], ks ? st[b] : cref, sc);
    } else {
      st[0] = f32x16_t{};
      st[1] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int b = 0; b < 2; ++b) st[b] = mma(kfrag(b, ks), qf[ks], st[b]);
    }
    mask(st);

    // P^T fragment against the current reference max: byte 16 b + r = key
    // 32 hh + 16 b + r; tsum = the tile's row sum of the rounded, lifted P.
    i32x8_t pf;
    f32x16_t tsum;
    auto probs = [&]() __attribute__((always_inline)) {
      const float nm = kPLift - m_run;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float p[4];
#pragma unroll
          for (int t = 0; t < 4; ++t)
            p[t] = __builtin_amdgcn_exp2f(kFold ? st[b][4 * g + t]
                                                : fmaf(st[b][4 * g + t], c2, nm));
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
          pf[4 * b + g] = w;
        }
      tsum = mma(ones, pf, f32x16_t{});
    };
    // Issue priority raised for the probabilities only (the SIMD's three waves belong
    // to different workgroups): this wave's exp chain goes first while the others'
    // MFMAs fill the matrix core.  Measured 2.0-2.3 % faster at the C2 shape; raising
    // it through the overflow check as well gained less.
    __builtin_amdgcn_s_setprio(1);
    probs();
    __builtin_amdgcn_s_setprio(0);
    // A probability past the e4m3 range converts to a NaN code, which the row
    // sum carries: only then is the reference max raised to this tile's max
    // (always on the first tile: without kFold its reference starts at -1e30, with
    // kFold the first tile is taken here by its index), O and the row sum rescaled
    // and the tile's probabilities redone.
    const bool first = kFold && j == 0;
    if (__builtin_amdgcn_ballot_w64(first ||
                                    (__float_as_uint(tsum[0]) & 0x7fffffffu) > 0x7f800000u) != 0) {
      float mx = fmaxf(st[0][0], st[1][0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(st[0][r], st[1][r]));
      mx = swap_halves_max(mx);
      if constexpr (kFold) {
        // mx - 6 is the tile's excess over the reference: raise the reference by it
        // (on the first tile set it to the tile's max, whatever the sign)
        const float delta = first ? mx - kPLift : fmaxf(mx - kPLift, 0.f);
        const float alpha = first ? 0.f : __builtin_amdgcn_exp2f(-delta);
        m_run += delta;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] *= alpha;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i) st[b][i] -= delta;
        probs();
      } else {
        mx *= c2;
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] *= alpha;
        probs();
      }
    }
    l_run += tsum[0];

    // O^T[d][query] += V^T P^T: A = V^T row 32 db + lane % 32, keys 32 hh .. +31
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      i32x2_t part[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        part[r] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (lds_i32x2_t*)(vb + vro[db] + 8 * r * D));
      const i32x8_t a = {part[0][0], part[0][1], part[1][0], part[1][1],
                         part[2][0], part[2][1], part[3][0], part[3][1]};
      o[db] = mma(a, pf, o[db]);
    }
    if (more) __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the next tile has landed
  };
  for (int j = 0; j < ntiles; j += 2) {
    tile(j, 0);
    if (j + 1 < ntiles) tile(j + 1, 1);
  }

  const float lt = l_run;  // the full row sum (every row of the sum MFMA holds it)
  if (qrow < nq) {
    const float f = dv / lt;
    uint16_t* op = out + (qrow * (int64_t)heads + head) * D + 4 * hh;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t w0 = pack_bf16(o[db][4 * g] * f, o[db][4 * g + 1] * f);
        const uint32_t w1 = pack_bf16(o[db][4 * g + 2] * f, o[db][4 * g + 3] * f);
        *reinterpret_cast<uint2*>(op + 32 * db + 8 * g) = make_uint2(w0, w1);
      }
    if (lse != nullptr && hh == 0)
      lse[(int64_t)head * nq + qrow] = (m_run - kPLift + __log2f(lt)) * ln_scale;
  }
}

}  // namespace

hipError_t launch_attn_fp8(const void* q, void* out, float* lse, const AttnSegs& segs, int nq,
                           int nk, int heads, float scale, float dq, float dk, float dv,
                           hipStream_t s, const KernelTiming* tm) {
  (void)nk;
  const int qtiles = (nq + BM - 1) / BM;
  const float c2 = fp8_logit_factor(scale, dq, dk);
  const int sc = fp8_pow2_scale_code(fp8_logit_factor64(scale, dq, dk));
  if (sc >= 0)
    launch_kernel(tm, attn_fp8_kernel<true>, dim3(qtiles * heads), dim3(NTHREADS), 0, s,
                  static_cast<const uint8_t*>(q), static_cast<uint16_t*>(out), lse, segs, nq,
                  heads, c2, sc, dv, 0.69314718055994531f, qtiles, qtiles * heads);
  else
    launch_kernel(tm, attn_fp8_kernel<false>, dim3(qtiles * heads), dim3(NTHREADS), 0, s,
                  static_cast<const uint8_t*>(q), static_cast<uint16_t*>(out), lse, segs, nq,
                  heads, c2, 0, dv, 0.69314718055994531f, qtiles, qtiles * heads);
  return hipGetLastError();
}

}  // namespace la
