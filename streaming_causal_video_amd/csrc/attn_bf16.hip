// Block attention, bf16 MFMA, head_dim 128, for gfx950 (CDNA4).
//
// out = softmax(scale * Q K_all^T) V_all per head, over the keys of a segment
// table {rotated sink, cached blocks, the block itself} with no mask
// (papernotes.org "Live Avatar: Streaming Real-time Audio-Driven Avatar
// Generation with Infinite Length", 整体框架 and 关键设计 2: a 3-latent-frame
// block attends to the sink frame and to the sliding noisy KV cache).
//
// Design (MI355X-first, not a port of the pages' FlashAttention):
//  * One workgroup = 8 waves (two per SIMD) = 256 query rows of one head; each
//    wave owns 32 query rows for the whole key range and keeps its Q fragments,
//    the running row max / row sum and the output accumulator in registers.
//    The K/V tile a workgroup stages in LDS serves 256 queries: the global
//    loads per query (measured to cost a quarter of the kernel's time at 128
//    queries per workgroup, whether they hit L2 or not) are halved.
//  * Keys are walked as one virtual range over the segment table, 64 keys per
//    tile, so tiles straddle segment boundaries and only the very last tile
//    can be partial.  K and V tiles are staged global -> registers -> LDS,
//    double buffered, one barrier per tile; the next tile's global loads are in
//    flight while the current tile is computed.  Waves 0-3 load V, waves 4-7 K
//    (four 16-byte loads per thread per tile).
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: in the 32x32 result each lane holds one query
//    (lane % 32) and half of the tile's keys, so the row max needs one
//    v_permlane32_swap per tile and the row sum none until the end.
//  * K rows are fed to the MFMA in an order that swaps bits 2 and 3 of the row
//    index; then the probabilities P^T come out of the score accumulator
//    already in the B-operand layout of the second product O^T = V^T P^T, with
//    no shuffle.
//  * V is stored transposed in LDS (V^T: 128 rows of 64 keys, 144-byte pitch):
//    each loader thread transposes a 4-key x 8-dim piece in registers with
//    v_perm_b32, so the V^T operand of the second product is read with plain
//    ds_read_b128 at immediate offsets (measured on gfx950: 16-byte LDS reads
//    deliver ~2.4x the bytes per clock of the transposing ds_read_b64_tr_b16).
//  * Online softmax in float32 with the scale folded into a base-2 exponent
//    (one FMA and one v_exp_f32 per score); P is rounded to bf16 for the second
//    product with v_cvt_pk_bf16_f32, and the row sum is taken from those same
//    bf16 pairs with v_dot2c_f32_bf16 (two scores per instruction, consistent
//    with the P V product it normalises).
//  * Lazy rescaling: the running max is only raised when a tile's max exceeds
//    it by more than 2^8 (in exp2 units), so O and the row sum are rescaled on
//    a handful of tiles instead of every tile.  Exact: numerator and
//    denominator use the same reference max; P stays <= 256.
//  * Loader: per-thread 32-bit row offsets are computed once; per tile only a
//    scalar segment base changes, and the current segment's key range and
//    base pointers stay in scalar registers (the segment table in kernel
//    arguments is read only when a tile enters the next segment: a scalar load
//    would also wait for all LDS reads in flight).  Tiles that straddle a
//    segment boundary or run past the last key take a slower per-row path.
//  * Workgroups are renumbered so that all query tiles of a head run on the
//    same XCD (dispatch is round-robin over the 8 XCDs) and share its L2 while
//    they stream the head's K/V.
#include "la_internal.h"

namespace la {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int D = 128;
constexpr int BM = 256;  // query rows per workgroup
constexpr int BN = 64;   // keys per tile
constexpr int NWAVES = 8;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int KP = 136;  // K row pitch in LDS (bf16): 272 B, 16 rows hit 16 disjoint bank quads
constexpr int VTP = 72;  // V^T row pitch in LDS (bf16): 144 B, 16 rows hit 16 disjoint bank quads
constexpr int KBUF = BN * KP;
constexpr int VBUF = D * VTP;
constexpr int STAGE = KBUF + VBUF;
constexpr float kRescaleSlack = 8.f;  // log2 units: P <= 2^8 between rescales

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ float swap_halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float swap_halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Row of the K tile that feeds MFMA row i: bits 2 and 3 of i swapped.
__device__ __forceinline__ int k_row_perm(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
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
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int64_t rs = (int64_t)heads * D;

  // Q^T B-operand fragments: lane holds Q[qrow][16 s + 8 hh .. +7].
  const int qrow = qt * BM + wave * 32 + l32;
  bf16x8_t qf[8];
  if (qrow < nq) {
    const uint16_t* qp = q + qrow * rs + head * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const bf16x8_t*>(qp + 16 * s);
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = bf16x8_t{};
  }

  f32x16_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16_t{};
  float m_run = -INFINITY;  // running max of scale*log2(e)*score
  float l_run = 0.f;        // this lane's half of the running row sum

  // Loader.  Waves 4-7 load K: thread covers 16-byte chunk lcc of tile rows
  // lr0 + 16 i (16 lanes read one 256-byte row).  Waves 0-3 load V: thread covers
  // 16-byte chunk vc (dims 8 vc .. +7) of tile rows 4 kq + i (a wave reads 64
  // contiguous bytes of every row) and writes it transposed.
  const bool kloader = __builtin_amdgcn_readfirstlane(wave) >= 4;
  const int ltid = tid & 255;
  const int lcc = ltid & 15;
  const int lr0 = ltid >> 4;
  const int kq = lane & 15;
  const int vc = 4 * (wave & 3) + (lane >> 4);
  const int ntiles = (nk + BN - 1) / BN;
  const uint32_t rs_bytes = (uint32_t)rs * 2u;
  uint32_t off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    off[i] = kloader ? (uint32_t)(lr0 + 16 * i) * rs_bytes + (uint32_t)(head * D * 2 + lcc * 16)
                     : (uint32_t)(4 * kq + i) * rs_bytes + (uint32_t)(head * D * 2 + vc * 16);
  uint4 reg[4];
  // Segment holding the first key of the tile being loaded, with its key range
  // and base pointers kept in scalar registers: the segment table is read only
  // when a tile crosses into the next segment (a scalar load would also wait
  // for every LDS read in flight).
  int seg = 0, seg_start = 0, seg_end = segs.end[0];
  const char* seg_k = static_cast<const char*>(segs.k[0]);
  const char* seg_v = static_cast<const char*>(segs.v[0]);

  auto gload = [&](int tile) __attribute__((always_inline)) {
    const int t0 = tile * BN;
    while (t0 >= seg_end) {
      ++seg;
      seg_start = seg_end;
      seg_end = segs.end[seg];
      seg_k = static_cast<const char*>(segs.k[seg]);
      seg_v = static_cast<const char*>(segs.v[seg]);
    }
    if (t0 + BN <= seg_end) {
      // whole tile inside one segment: scalar base + precomputed 32-bit offsets
      const uint32_t sbase = (uint32_t)(t0 - seg_start) * rs_bytes;
      const char* b = (kloader ? seg_k : seg_v) + sbase;
#pragma unroll
      for (int i = 0; i < 4; ++i) reg[i] = *reinterpret_cast<const uint4*>(b + off[i]);
    } else {
      // straddles a segment boundary or runs past the last key: per-row lookup,
      // rows past the last key are clamped to it (their scores are masked)
      auto row_load = [&](int r, int chunk, bool is_v) -> uint4 {
        const int key = min(t0 + r, nk - 1);
        int s = seg;
        while (key >= segs.end[s]) ++s;
        const int st = s ? segs.end[s - 1] : 0;
        const int64_t o = (int64_t)(key - st) * rs + head * D + chunk * 8;
        const uint16_t* base = static_cast<const uint16_t*>(is_v ? segs.v[s] : segs.k[s]);
        return *reinterpret_cast<const uint4*>(base + o);
      };
      if (kloader) {
        reg[0] = row_load(lr0, lcc, false);
        reg[1] = row_load(lr0 + 16, lcc, false);
        reg[2] = row_load(lr0 + 32, lcc, false);
        reg[3] = row_load(lr0 + 48, lcc, false);
      } else {
        reg[0] = row_load(4 * kq, vc, true);
        reg[1] = row_load(4 * kq + 1, vc, true);
        reg[2] = row_load(4 * kq + 2, vc, true);
        reg[3] = row_load(4 * kq + 3, vc, true);
      }
    }
  };
  auto lstore = [&](int buf) {
    uint16_t* kb = lds + buf * STAGE;
    uint16_t* vt = kb + KBUF;
    if (kloader) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint4*>(kb + (lr0 + 16 * i) * KP + lcc * 8) = reg[i];
    } else {
      // V^T[8 vc + j][4 kq .. 4 kq + 3]: pairs of keys packed per dword
      const uint32_t w[4][4] = {{reg[0].x, reg[0].y, reg[0].z, reg[0].w},
                                {reg[1].x, reg[1].y, reg[1].z, reg[1].w},
                                {reg[2].x, reg[2].y, reg[2].z, reg[2].w},
                                {reg[3].x, reg[3].y, reg[3].z, reg[3].w}};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint2 even = make_uint2(__builtin_amdgcn_perm(w[1][m], w[0][m], 0x05040100u),
                                      __builtin_amdgcn_perm(w[3][m], w[2][m], 0x05040100u));
        const uint2 odd = make_uint2(__builtin_amdgcn_perm(w[1][m], w[0][m], 0x07060302u),
                                     __builtin_amdgcn_perm(w[3][m], w[2][m], 0x07060302u));
        *reinterpret_cast<uint2*>(vt + (8 * vc + 2 * m) * VTP + 4 * kq) = even;
        *reinterpret_cast<uint2*>(vt + (8 * vc + 2 * m + 1) * VTP + 4 * kq) = odd;
      }
    }
  };

  const int krow_a = k_row_perm(l32);
  typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
  const bf16x2v_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  gload(0);
  for (int j = 0; j < ntiles; ++j) {
    lstore(j & 1);
    if (j + 1 < ntiles) gload(j + 1);
    __syncthreads();
    const uint16_t* kb = lds + (j & 1) * STAGE;
    const uint16_t* vt = kb + KBUF + l32 * VTP + 8 * hh;

    // S^T[key][query] for two 32-key blocks, chains interleaved.
    f32x16_t st[2];
    st[0] = f32x16_t{};
    st[1] = f32x16_t{};
    const uint16_t* kr0 = kb + krow_a * KP + 8 * hh;
    const uint16_t* kr1 = kr0 + 32 * KP;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8_t k0 = *reinterpret_cast<const bf16x8_t*>(kr0 + 16 * s);
      const bf16x8_t k1 = *reinterpret_cast<const bf16x8_t*>(kr1 + 16 * s);
      st[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[s], st[0], 0, 0, 0);
      st[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[s], st[1], 0, 0, 0);
    }
    if ((j + 1) * BN > nk) {
      // last tile: mask keys past the end (accumulator row i holds key 32 b + perm(i))
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = 8 * (r >> 2) + 4 * hh + (r & 3);
          if (j * BN + 32 * b + k_row_perm(i) >= nk) st[b][r] = -INFINITY;
        }
    }

    float mx = fmaxf(st[0][0], st[1][0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(st[0][r], st[1][r]));
    mx = swap_halves_max(mx) * c2;
    // raise the reference max only when this tile would push P above 2^8
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleSlack) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] *= alpha;
    }

    // P^T fragments: ks = 2 b + half, elements r = 8 half .. 8 half + 7.
    bf16x8_t pf[4];
    const float nm = -m_run;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(st[b][8 * half + 2 * e], c2, nm));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(st[b][8 * half + 2 * e + 1], c2, nm));
          w[e] = pack_bf16(p0, p1);
          l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, w[e]), ones,
                                                  l_run, false);
        }
        pf[2 * b + half] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
      }

    // O^T[d][query] += V^T P^T: A operand = V^T[32 db + lane % 32][16 ks + 8 hh .. +7]
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(vt + 32 * db * VTP + 16 * ks);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ks], o[db], 0, 0, 0);
      }
    }
  }

  const float lt = swap_halves_sum(l_run);
  if (qrow < nq) {
    const float inv = 1.f / lt;
    uint16_t* op = out + qrow * rs + head * D + 4 * hh;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t w0 = pack_bf16(o[db][4 * g] * inv, o[db][4 * g + 1] * inv);
        const uint32_t w1 = pack_bf16(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
        *reinterpret_cast<uint2*>(op + 32 * db + 8 * g) = make_uint2(w0, w1);
      }
    if (lse != nullptr && hh == 0)
      lse[(int64_t)head * nq + qrow] = (m_run + __log2f(lt)) * 0.69314718055994531f;
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
