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
//    Two waves per SIMD (<= 256 registers, 39 KB of LDS per workgroup).  At
//    three per SIMD (168 registers) the loop-invariant addresses spilled to
//    scratch, and the reload after each barrier waited (one in-order counter)
//    for the next tile's prefetch as well (1.82 ms against 1.58 ms at two per SIMD).
//  * Tile loads are buffer loads from a scalar descriptor (segment base + tile
//    row + head, record count = the segment's remaining bytes) with one lane
//    offset for K and one for V; the other rows of a thread differ by uniform
//    multiples of the row stride, passed as the scalar offset.  No 64-bit
//    address registers, and a wrong offset reads zeros instead of faulting.
//  * Both products run on v_mfma_f32_32x32x64_f8f6f4 (e4m3 x e4m3, float32
//    accumulate): S^T = K Q^T is 4 MFMAs per tile, O^T += V^T P^T another 4.
//  * The MFMA takes A[i][k] and B[k][j] from lane bytes under one fixed (lane,
//    byte) -> k assignment; any assignment shared by A and B gives the same
//    product, so the kernel picks its own: for S, lane l holds dims
//    64 ks + 32 (l / 32) + j of its row; for P V, keys 32 (l / 32) + j.
//  * K rows are fed to the score MFMA in the order that makes accumulator row
//    i of key block b hold key 32 ((i / 4) % 2) + 16 b + 4 (i / 8) + i % 4.
//    Then lane l's 32 scores are keys 32 (l / 32) .. +31 in byte order, so P
//    packs straight into the B operand of the second product.
//  * V stays key-major in LDS (64 rows of 128 bytes, 160-byte pitch: the 8
//    consecutive keys one half-wave reads land on disjoint banks) and the A
//    operand of the second product (32 dims x 32 keys per lane) is read with
//    four ds_read_b64_tr_b8: in each 16-lane group lane i receives, as byte j,
//    byte i & 7 of the 8 bytes lane 2j + (i >> 3) addresses (measured on
//    gfx950), so lanes addressing 8 dims of one key hand every lane the 8 keys
//    of its dim.  The loader stores V rows as it loads them (no transpose).
//  * Softmax in float32 with scale * dq * dk * log2(e) folded into the exponent;
//    P = exp2(s - m + 6) rounded to e4m3 (the 2^6 lifts small probabilities out
//    of the subnormal range).
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
constexpr int KP = 144;  // K row pitch in LDS (bytes): 16 rows hit 16 disjoint bank quads
constexpr int VP = 160;  // V row pitch in LDS (bytes), key-major: 8 consecutive rows, disjoint banks
constexpr int KBUF = BN * KP;
constexpr int VBUF = BN * VP;
constexpr int STAGE = KBUF + VBUF;
constexpr float kPLift = 6.f;         // P is computed as exp2(s - m + 6)

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ float swap_halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// LDS row of the K tile that holds key kk (inverse of the feed order above).
__device__ __forceinline__ int k_lds_row(int kk) {
  const int h = (kk >> 5) & 1, b = (kk >> 4) & 1, g = (kk >> 2) & 3, t = kk & 3;
  return 32 * b + 8 * g + 4 * h + t;
}

// 32 bytes from a 16-byte aligned address (two 16-byte reads)
__device__ __forceinline__ i32x8_t ld32(const uint8_t* p) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint4 b = *reinterpret_cast<const uint4*>(p + 16);
  return i32x8_t{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

__device__ __forceinline__ f32x16_t mma(const i32x8_t& a, const i32x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__global__ __attribute__((amdgpu_flat_work_group_size(NTHREADS, NTHREADS),
                          amdgpu_waves_per_eu(2, 2))) void
attn_fp8_kernel(const uint8_t* __restrict__ q, uint16_t* __restrict__ out,
                float* __restrict__ lse, const AttnSegs segs, int nq, int nk, int heads,
                float c2, float dv, float ln_scale, int qtiles, int nwg) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];

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

  // Q^T B-operand fragments: lane holds bytes 64 ks + 32 hh .. +31 of its query row.
  const int qrow = qt * BM + wave * 32 + l32;
  i32x8_t qf[2];
  if (qrow < nq) {
    const uint8_t* qp = q + qrow * rs + head * D + 32 * hh;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) qf[ks] = ld32(qp + 64 * ks);
  } else {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) qf[ks] = i32x8_t{};
  }

  f32x16_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16_t{};
  float m_run = -1e30f;  // reference max (exp2 units; finite: no inf - inf)
  float l_run = 0.f;      // running sum of the lifted, rounded P of this lane's query
  const i32x8_t ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                        0x38383838, 0x38383838, 0x38383838, 0x38383838};  // e4m3 1.0

  // Loader.  K and V alike: thread covers 16-byte chunk kc of key rows kr0 and
  // kr0 + 32 (8 lanes read one 128-byte row).
  const int kc = tid & 7;
  const int kr0 = tid >> 3;
  const int ntiles = (nk + BN - 1) / BN;
  const uint32_t rs32 = (uint32_t)rs;
  // Lane offset of the tile loads (K and V) relative to the tile's first row of
  // this head; the other row of a thread is 32 row strides further (passed as the
  // buffer loads' scalar offset).
  const uint32_t koff = (uint32_t)kr0 * rs32 + (uint32_t)(kc * 16);
  uint4 kreg[2];
  uint4 vreg[2];
  // Segment holding the first key of the tile being loaded, with its key range
  // and base pointers kept in scalar registers: the segment table is read only
  // when a tile crosses into the next segment (a scalar load would also wait
  // for every LDS read in flight).
  int seg = 0, seg_start = 0, seg_end = segs.end[0];
  const uint8_t* seg_k = static_cast<const uint8_t*>(segs.k[0]);
  const uint8_t* seg_v = static_cast<const uint8_t*>(segs.v[0]);

  auto gload = [&](int tile) {
    const int t0 = tile * BN;
    while (t0 >= seg_end) {
      ++seg;
      seg_start = seg_end;
      seg_end = segs.end[seg];
      seg_k = static_cast<const uint8_t*>(segs.k[seg]);
      seg_v = static_cast<const uint8_t*>(segs.v[seg]);
    }
    if (t0 + BN <= seg_end) {
      // whole tile inside one segment: buffer loads from a scalar base with the
      // precomputed 32-bit offsets (no 64-bit address registers); the record
      // count ends the descriptor at the segment's end
      const uint32_t sbase = (uint32_t)(t0 - seg_start) * rs32 + (uint32_t)(head * D);
      const uint32_t nbytes = (uint32_t)(seg_end - t0) * rs32 - (uint32_t)(head * D);
      const __amdgpu_buffer_rsrc_t kr =
          __builtin_amdgcn_make_buffer_rsrc((void*)(seg_k + sbase), 0, nbytes, kBufWord3);
      const __amdgpu_buffer_rsrc_t vr =
          __builtin_amdgcn_make_buffer_rsrc((void*)(seg_v + sbase), 0, nbytes, kBufWord3);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b128(kr, koff, 32 * i * rs32, 0);
        kreg[i] = make_uint4(x[0], x[1], x[2], x[3]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b128(vr, koff, 32 * i * rs32, 0);
        vreg[i] = make_uint4(x[0], x[1], x[2], x[3]);
      }
    } else {
      // straddles a segment boundary or runs past the last key: per-row lookup,
      // rows past the last key are clamped to it (their scores are masked)
      auto row_base = [&](int r, bool is_v) -> const uint8_t* {
        const int key = min(t0 + r, nk - 1);
        int s = seg;
        while (key >= segs.end[s]) ++s;
        const int st = s ? segs.end[s - 1] : 0;
        return static_cast<const uint8_t*>(is_v ? segs.v[s] : segs.k[s]) +
               (int64_t)(key - st) * rs + head * D;
      };
      kreg[0] = *reinterpret_cast<const uint4*>(row_base(kr0, false) + kc * 16);
      kreg[1] = *reinterpret_cast<const uint4*>(row_base(kr0 + 32, false) + kc * 16);
      vreg[0] = *reinterpret_cast<const uint4*>(row_base(kr0, true) + kc * 16);
      vreg[1] = *reinterpret_cast<const uint4*>(row_base(kr0 + 32, true) + kc * 16);
    }
  };
  auto lstore = [&](int buf) {
    uint8_t* kb = lds + buf * STAGE;
    uint8_t* vt = kb + KBUF;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<uint4*>(kb + k_lds_row(kr0 + 32 * i) * KP + kc * 16) = kreg[i];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<uint4*>(vt + (kr0 + 32 * i) * VP + kc * 16) = vreg[i];
  };

  gload(0);
  // One 64-key tile j from LDS buffer `cur` (its K/V registers are stored there
  // first, then tile j + 1 is loaded into registers).  The loop runs two tiles per
  // trip so that both buffers are compile-time constants (immediate LDS offsets).
  auto tile = [&](const int j, const int cur) __attribute__((always_inline)) {
    lstore(cur);
    if (j + 1 < ntiles) gload(j + 1);
    __syncthreads();
    const uint8_t* kb = lds + cur * STAGE;
    // V operand by transposing reads: in each 16-lane group lane s addresses key
    // 32 hh + 8 r + (s >> 1), dims 32 db + 16 ((lane >> 4) & 1) + 8 (s & 1) .. +7
    const uint8_t* vt = kb + KBUF + (32 * hh + ((lane & 15) >> 1)) * VP + 16 * ((lane >> 4) & 1) +
                        8 * (lane & 1);

    // S^T for the two 32-row key blocks: A = LDS row 32 b + lane % 32, bytes 64 ks + 32 hh ..
    f32x16_t st[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const i32x8_t a = ld32(kb + (32 * b + l32) * KP + 64 * ks + 32 * hh);
        st[b] = mma(a, qf[ks], st[b]);
      }
    if ((j + 1) * BN > nk) {
      // last tile: mask keys past the end (st[b][r] holds key 32 hh + 16 b + r)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (j * BN + 32 * hh + 16 * b + r >= nk) st[b][r] = -INFINITY;
    }

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
            p[t] = __builtin_amdgcn_exp2f(fmaf(st[b][4 * g + t], c2, nm));
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
          pf[4 * b + g] = w;
        }
      tsum = mma(ones, pf, f32x16_t{});
    };
    probs();
    // A probability past the e4m3 range converts to a NaN code, which the row
    // sum carries: only then is the reference max raised to this tile's max
    // (always on the first tile, whose reference starts at -1e30), O and the
    // row sum rescaled and the tile's probabilities redone.
    if (__builtin_amdgcn_ballot_w64((__float_as_uint(tsum[0]) & 0x7fffffffu) > 0x7f800000u) != 0) {
      float mx = fmaxf(st[0][0], st[1][0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(st[0][r], st[1][r]));
      mx = swap_halves_max(mx) * c2;
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] *= alpha;
      probs();
    }
    l_run += tsum[0];

    // O^T[d][query] += V^T P^T: A = V^T row 32 db + lane % 32, keys 32 hh .. +31
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      i32x2_t part[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        part[r] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(vt + 8 * r * VP + 32 * db));
      const i32x8_t a = {part[0][0], part[0][1], part[1][0], part[1][1],
                         part[2][0], part[2][1], part[3][0], part[3][1]};
      o[db] = mma(a, pf, o[db]);
    }
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
  const int qtiles = (nq + BM - 1) / BM;
  const float c2 = scale * dq * dk * 1.4426950408889634f;
  launch_kernel(tm, attn_fp8_kernel, dim3(qtiles * heads), dim3(NTHREADS), 0, s,
                static_cast<const uint8_t*>(q), static_cast<uint16_t*>(out), lse, segs, nq, nk,
                heads, c2, dv, 0.69314718055994531f, qtiles, qtiles * heads);
  return hipGetLastError();
}

}  // namespace la
