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
//    waves on 32x32x16 MFMAs.  At 4680 rows a head takes 25 query tiles
//    (2.5 % padding); in the last one, waves left without rows only stage
//    their share of the K/V tiles and meet the barriers, leaving their SIMDs
//    to the other workgroup's waves (0.8 % faster at C2).
//  * Scores are computed transposed, S^T = K Q^T: in each 16x16 result a lane
//    holds one query (lane % 16) and four keys; the row max needs two lane
//    swaps (v_permlane32_swap, v_permlane16_swap).
//  * K rows sit in LDS in an order that moves key bit 2 to row bit 4 and key
//    bits 3-4 to row bits 2-3 (within each 32-key half); then rows 4g .. 4g+3
//    of the row blocks 2h and 2h+1 hold keys 32h + 8g .. 32h + 8g + 7, so the
//    probabilities P^T come out of the score accumulators already in the
//    B-operand layout of O^T = V^T P^T, with no shuffle.
//  * Each 64-key tile is processed as two 32-key halves: the scores of both
//    halves first, then the first half's softmax and P V, then the second's,
//    so that the first half's P V MFMAs share a block with the second half's
//    softmax.  Probabilities and the P V operands are held for one half at a
//    time, which keeps the kernel within the 256 registers of two waves per
//    SIMD.
//  * Issue priority (s_setprio) is raised while a wave runs the first half's
//    softmax, the one stretch with no MFMA of its own, and lowered again for
//    the scores and the P V blocks: the SIMD's other wave then fills the
//    matrix core while this wave's exp2 chain gets the issue slots first.
//  * Softmax in base 2 with the score scale folded into Q: the kernel takes Q
//    already multiplied by c = scale * log2(e), rounded to bf16 once (in the
//    step the kRotQ instantiation loads the raw Q and rotates it with per-token
//    cos/sin that already carry c, with the RoPE kernel's arithmetic; a caller's
//    rotated but plain Q is multiplied and rounded here when its Q fragments are
//    loaded), and the running
//    reference m of each query enters the first score MFMA of a half as its C
//    operand, so the accumulators leave the matrix core as c s - m and the
//    probability of each score is a single v_exp_f32.  Probabilities are taken
//    against the running reference without a per-tile max; only when a
//    query's sum over the half leaves [0, 2^64] (and always on the first half
//    of a piece) is the reference raised by the half's excess, the scores
//    moved down by it (after the first half, the second half's as well), O
//    and the row sum rescaled and the half's probabilities recomputed.  Exact: numerator and denominator use the same
//    reference, and P <= 2^64 keeps the float32 accumulators far from
//    overflow.  P is rounded to bf16 for the second product
//    (v_cvt_pk_bf16_f32) and the row sum is taken from those same bf16 pairs
//    with v_dot2c_f32_bf16.
//  * K tiles go global -> LDS by DMA (buffer_load ... lds): no staging
//    registers, issued one tile ahead right after the barrier, so a whole
//    tile of compute hides their latency.  A DMA writes each wave's 1 KB
//    contiguously, so K rows have no padding (256-byte pitch) and each
//    16-byte chunk c of row r sits at chunk c ^ (r & 15), which keeps the
//    fragment reads free of bank conflicts.
//  * Each segment of the key table is tiled on its own (segment s has
//    ceil(len_s / 64) tiles, the last one partial), so every tile lies in one
//    segment: its DMA uses one buffer descriptor whose record count ends at
//    the segment's last row (rows past it load as zeros) and its missing keys
//    are masked.  No per-row path for tiles that straddle two segments, and no
//    per-tile segment search beyond one compare.  The host joins segments that
//    continue in memory (neighbouring ring slots), so in the step the window
//    and the block are one segment: at 1560 + 5 x 4680 keys 0.3 % of the
//    computed keys are masked (1.3 % with six segments); at 3520 + 5 x 10560
//    none.
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
//  * Schedule.  A unit of work is (head, 192-query tile) over all ntiles
//    64-key tiles.  Without a workspace the grid has one workgroup per unit.
//    With one, the grid is persistent with P slots (two workgroups per CU):
//    slot s runs units s, P + s, ... for the R = U / P full rounds, and the
//    U' = U mod P units of the last round, when they would leave more than
//    half of the slots idle, are cut into m = P / U' equal key ranges run by
//    U' m slots (piece-major, so concurrent slots read the same key tiles of a
//    head, as whole rounds do).  Cutting units at arbitrary key offsets to
//    balance the slots exactly was measured 30 % slower at 1000 units: the
//    concurrent slices then stream a head's K/V at scattered offsets and L2
//    reuse is lost.  Each piece of a cut unit stores its unnormalised (O, m,
//    l) per row in the workspace; the piece that arrives last (a per-unit
//    counter) merges the pieces in piece order (so the result does not depend
//    on arrival order), writes the output and resets the counter to zero.
//    Nothing waits on another workgroup.
//  * Workgroups are renumbered so that consecutive slots (and so the query
//    tiles of one head) run on the same XCD (dispatch is round-robin over the
//    8 XCDs) and share its L2 while they stream the head's K/V.
#include "la_internal.h"

namespace la {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
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

// Rotate a wave's Q fragments in place (see the kRotQ path of the kernel): pair
// (a, b) with the token's scaled cos/sin (cs, sn) from qcs becomes
// (fma(a, cs, -b sn), fma(a, sn, b cs)), rounded to bf16 (nearest even).
__device__ __forceinline__ void rope_q(bf16x8_t (&qf)[NQT][4], const float* __restrict__ qcs,
                                       int qrow0, int nq, int c, int g) {
#pragma unroll
  for (int nt = 0; nt < NQT; ++nt) {
    // rows past nq hold zeros and stay zero; their lookup is clamped into the table
    const int tok = min(qrow0 + 16 * nt + c, nq - 1);
    const float* row = qcs + (int64_t)tok * D;  // D / 2 pairs x (cos, sin)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // pairs 16 s + 4 g .. +3: (cos, sin) x 4 = 32 contiguous bytes
      const f32x4_t e0 = *reinterpret_cast<const f32x4_t*>(row + 32 * s + 8 * g);
      const f32x4_t e1 = *reinterpret_cast<const f32x4_t*>(row + 32 * s + 8 * g + 4);
      const float cs[4] = {e0[0], e0[2], e1[0], e1[2]};
      const float sn[4] = {e0[1], e0[3], e1[1], e1[3]};
      const u32x4_t x = __builtin_bit_cast(u32x4_t, qf[nt][s]);
      u32x4_t y;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = __uint_as_float(x[i] << 16), b = __uint_as_float(x[i] & 0xffff0000u);
        y[i] = pack_bf16(fmaf(a, cs[i], -b * sn[i]), fmaf(a, sn[i], b * cs[i]));
      }
      qf[nt][s] = __builtin_bit_cast(bf16x8_t, y);
    }
  }
}

// Partial record of one piece (floats): per wave, O as f32x4 per (d-tile, query
// tile, lane), then m and the row sum l per (query tile, lane).
constexpr int kRecO = 8 * NQT * 64 * 4;
constexpr int kRecWave = kRecO + 2 * NQT * 64;
static_assert(NWAVES * kRecWave == kAttnRecFloats, "partial record size");

template <bool kRotQ>
__global__ __attribute__((amdgpu_flat_work_group_size(NTHREADS, NTHREADS),
                          amdgpu_waves_per_eu(2, 2))) void
attn_bf16_kernel(const uint16_t* __restrict__ q, uint16_t* __restrict__ out,
                 float* __restrict__ lse, const AttnSegs segs, int nq, int nk, int heads,
                 float qmul, int qtiles, int nwg, AttnWork wk,
                 const float* __restrict__ qcs) {
  // The K and V buffers of the two stages are separate objects, so that the compiler
  // can tell a DMA into one stage from the fragment reads of the other and does not
  // wait for the DMA before those reads.
  __shared__ __attribute__((aligned(16))) uint16_t lds_k0[KBUF], lds_v0[VBUF], lds_k1[KBUF],
      lds_v1[VBUF];
  __shared__ int s_arrival;
  auto kbuf = [&](int buf) __attribute__((always_inline)) -> uint16_t* {
    return buf ? lds_k1 : lds_k0;
  };
  auto vbuf = [&](int buf) __attribute__((always_inline)) -> uint16_t* {
    return buf ? lds_v1 : lds_v0;
  };

  // XCD-aware renumbering: consecutive logical ids on one XCD.
  const int pid = __builtin_amdgcn_workgroup_id_x();
  const int per = (nwg + 7) / 8;
  const int tall = (nwg % 8) == 0 ? 8 : (nwg % 8);
  const int xcd = pid % 8, loc = pid / 8;
  const int lin = xcd < tall ? xcd * per + loc : tall * per + (xcd - tall) * (per - 1) + loc;

  const int tid = __builtin_amdgcn_workitem_id_x();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar
  const int c = lane & 15;  // query (scores) / row (operands) within a 16-tile
  const int g = lane >> 4;  // 8-element k-group of the operands
  const int64_t rs = (int64_t)heads * D;
  const int ntiles = segs.tend[segs.nseg - 1];

  // Loader geometry (the same for every piece).  K DMA: wave w fills LDS rows
  // 16 w + 4 i + t (t = lane >> 4, i = 0..3), lane slot p = lane & 15 of a row
  // receiving chunk p ^ (row & 15) of key 32 (w >> 1) + 4 (w & 1) + 8 i + t.
  const int t4 = lane >> 4;
  const uint32_t rs_bytes = (uint32_t)rs * 2u;
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

  typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
  const bf16x2v_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  // This slot's pieces: whole units lin, lin + P, ... for the full rounds, then at
  // most one piece of a unit of the last round (cut into wk.cuts key ranges).
  const int units = qtiles * heads;
  const int P = nwg;
  const int rounds = units / P;
  const int urem = units - rounds * P;
  const int cuts = wk.cuts;
  const int npieces = rounds + (lin < urem * cuts ? 1 : 0);

  // Zero both V buffers once: the rows of a segment's partial last tile past its end
  // are masked (P = 0 exactly) but still enter P V, so they must hold finite values;
  // the DMA leaves either zeros there (rows outside the buffer descriptor) or the V
  // rows of an earlier tile.
#pragma unroll
  for (int i = 0; i < VBUF / (8 * NTHREADS); ++i) {
    const int e = (i * NTHREADS + tid) * 8;  // bf16 element index within a V buffer
    *reinterpret_cast<uint4*>(lds_v0 + e) = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(lds_v1 + e) = make_uint4(0, 0, 0, 0);
  }

  for (int it = 0; it < npieces; ++it) {
    int unit = it * P + lin, kt0 = 0, kt1 = ntiles, cut = 0;
    if (it == rounds) {
      cut = lin / urem;  // piece-major: concurrent slots share key ranges
      unit = rounds * P + (lin - cut * urem);
      const int len = ntiles / cuts;
      kt0 = cut * len;
      kt1 = cut == cuts - 1 ? ntiles : kt0 + len;
    }
    const int head = unit / qtiles;
    const int qt = unit - head * qtiles;
    const uint32_t hoff = (uint32_t)(head * D * 2);
    const int qbase = qt * BM + wave * QW;

    // Q^T B-operand fragments: lane holds Q[query qbase + 16 nt + c][32 s + 8 g .. +7],
    // multiplied by qmul (when it is not 1) and rounded to bf16.
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
    if constexpr (kRotQ) {
      // Rolling RoPE of the raw Q (the step's path): this lane's elements
      // 32 s + 8 g .. +7 are the head_dim pairs 16 s + 4 g + i (i = 0..3), rotated
      // with the row's cos/sin from qcs as the RoPE kernel rotates Q
      rope_q(qf, qcs, qbase, nq, c, g);
    }
    if (qmul != 1.0f) {
#pragma unroll
      for (int nt = 0; nt < NQT; ++nt)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          bf16x8_t v = qf[nt][s];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (__bf16)((float)v[e] * qmul);
          qf[nt][s] = v;
        }
    }

    f32x4_t o[8][NQT];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int nt = 0; nt < NQT; ++nt) o[dt][nt] = f32x4_t{};
    // cm[nt] = -m in all four elements, m = the query's reference (base-2 units): the
    // C operand of the first score MFMA of a half.  This lane's row sum in l_run.
    f32x4_t cm[NQT];
    float l_run[NQT];
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
      cm[nt] = f32x4_t{};
      l_run[nt] = 0.f;
    }

    // Segment of the tile being loaded, kept in scalar registers: the segment
    // table is read only when the tiles enter the next segment.
    int seg = 0, seg_t0 = 0, seg_t1 = segs.tend[0], seg_len = segs.end[0];
    const char* seg_k = static_cast<const char*>(segs.k[0]);
    const char* seg_v = static_cast<const char*>(segs.v[0]);
    uint32_t sbase = 0, nbytes = 0;  // tile's byte offset in the segment, bytes left from there
    int valid = BN;                  // keys of the tile inside its segment

    auto locate = [&](int tile) __attribute__((always_inline)) {
      while (tile >= seg_t1) {
        seg_len = segs.end[seg + 1] - segs.end[seg];
        ++seg;
        seg_t0 = seg_t1;
        seg_t1 = segs.tend[seg];
        seg_k = static_cast<const char*>(segs.k[seg]);
        seg_v = static_cast<const char*>(segs.v[seg]);
      }
      const int r0 = (tile - seg_t0) * BN;  // the tile's first row in the segment
      valid = seg_len - r0 < BN ? seg_len - r0 : BN;
      sbase = (uint32_t)r0 * rs_bytes + hoff;
      nbytes = (uint32_t)(seg_len - r0) * rs_bytes - hoff;
    };
    auto kload = [&](int buf) __attribute__((always_inline)) {
      uint16_t* kb = kbuf(buf);
      const __amdgpu_buffer_rsrc_t kr =
          __builtin_amdgcn_make_buffer_rsrc((void*)(seg_k + sbase), 0, nbytes, kBufWord3);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            kr, (__attribute__((address_space(3))) void*)(kb + (16 * wave + 4 * i) * KP), 16,
            kdoff[i], 8 * i * rs_bytes, 0, 0);
    };
    auto vload = [&](int buf) __attribute__((always_inline)) {
      uint16_t* vb = vbuf(buf);
      const __amdgpu_buffer_rsrc_t vr =
          __builtin_amdgcn_make_buffer_rsrc((void*)(seg_v + sbase), 0, nbytes, kBufWord3);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            vr, (__attribute__((address_space(3))) void*)(vb + (16 * wave + 4 * i) * VP), 16,
            vdoff[i >> 1], 4 * i * rs_bytes, 0, 0);
    };

    __syncthreads();  // the previous piece's last tile is done with both LDS buffers
    locate(kt0);
    int valid_next = valid;  // keys of the tile in flight
    kload(0);
    vload(0);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the first tile's K DMA has landed
    // One 64-key tile j computed from LDS buffer `cur` while tile j + 1 is staged
    // into buffer 1 - cur.  The loop below runs two tiles per trip so that both
    // buffers are compile-time constants (LDS addresses become immediates).
    auto tile = [&](const int j, const int cur) __attribute__((always_inline)) {
      __syncthreads();
      const int nvalid = valid_next;  // keys of this tile (the rest are masked)
      const bool more = j + 1 < kt1;
      if (more) {
        locate(j + 1);
        valid_next = valid;
        kload(1 - cur);
      }
      const uint16_t* kb = kbuf(cur);
      // K fragment: row 16 blk + c, chunk 4 s + g, stored at chunk (4 s + g) ^ c
      const uint16_t* kr = kb + c * KP;
      // V operand by transposing reads (B = 0, 1 for keys + 0..3, + 4..7): this lane
      // addresses key 32 h + 8 g + (c >> 2) + 4 B, dims 16 dt + 4 (c & 3) .. +3, which
      // sits in LDS row 32 h + 16 (g >> 1) + 8 B + 4 (g & 1) + (c >> 2)
      const char* vt = reinterpret_cast<const char*>(vbuf(cur));

      // Scores of both halves first (S^T[key][query] - m, keys 32 h .. 32 h + 31 in row
      // blocks 2 h and 2 h + 1): the first half's P V MFMAs then share a block with the
      // second half's softmax, which they can run beside (measured 1 % faster than
      // scores, softmax and P V half by half, and faster than the second half's scores
      // beside the first half's softmax).
      f32x4_t st[2][2][NQT];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int nt = 0; nt < NQT; ++nt) st[h][b][nt] = cm[nt];
      // Issue priority (the SIMD's two waves belong to different workgroups): raised
      // for the first half's softmax only, where the wave has no MFMA of its own to
      // overlap, so that its exp2 chain goes first while the other wave's MFMAs fill
      // the matrix core; normal for the scores and for the P V blocks (with the
      // second half's softmax, which runs beside its own first-half P V).  Measured:
      // C2 launch 3 % faster, C5 7 %; raising it also for the second half, or for the
      // scores instead, was slower.
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(
                kr + 16 * (2 * h + b) * KP + (((4 * s + g) ^ c) * 8));
#pragma unroll
            for (int nt = 0; nt < NQT; ++nt)
              st[h][b][nt] =
                  __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[nt][s], st[h][b][nt], 0, 0, 0);
          }
        if (h == 0 && more) vload(1 - cur);
      }
      __builtin_amdgcn_s_setprio(1);
      if (__builtin_expect(nvalid < BN, 0)) {
        // the last tile of a segment: row 4 g + i of block 2 h + b holds key
        // 32 h + 8 g + 4 b + i of the tile.  The lane's first key is formed here from
        // a copy of g that the compiler cannot see through, so that it does not keep
        // the sixteen key indexes live (in scratch) across the tile loop.
        int key0 = 8 * g;
        asm volatile("" : "+v"(key0));
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if (key0 + 32 * h + 4 * b + i >= nvalid) {
#pragma unroll
                for (int nt = 0; nt < NQT; ++nt) st[h][b][nt][i] = -INFINITY;
              }
            }
      }

#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // P^T fragment of query tile nt: keys 32 h + 8 g .. +7, i.e. rows
        // 4 g .. 4 g + 3 of both row blocks; tsum = this lane's sum of them.
        bf16x8_t pf[NQT];
        float tsum[NQT];
        auto probs = [&]() __attribute__((always_inline)) {
#pragma unroll
          for (int nt = 0; nt < NQT; ++nt) {
            uint32_t w[4];
            float ts = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float p0 = __builtin_amdgcn_exp2f(st[h][e >> 1][nt][2 * (e & 1)]);
              const float p1 = __builtin_amdgcn_exp2f(st[h][e >> 1][nt][2 * (e & 1) + 1]);
              w[e] = pack_bf16(p0, p1);
              ts = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, w[e]), ones, ts,
                                                   false);
            }
            tsum[nt] = ts;
            pf[nt] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
          }
        };
        probs();
        const bool first = h == 0 && j == kt0;
        bool over = first;
#pragma unroll
        for (int nt = 0; nt < NQT; ++nt)
          over |= __float_as_uint(tsum[nt]) > kSumLimitBits;
        if (__builtin_amdgcn_ballot_w64(over) != 0) {
#pragma unroll
          for (int nt = 0; nt < NQT; ++nt) {
            const float a = fmaxf(
                fmaxf(fmaxf(st[h][0][nt][0], st[h][0][nt][1]), fmaxf(st[h][0][nt][2], st[h][0][nt][3])),
                fmaxf(fmaxf(st[h][1][nt][0], st[h][1][nt][1]), fmaxf(st[h][1][nt][2], st[h][1][nt][3])));
            const float am = max4_lanes(a);
            const float delta = first ? am : fmaxf(am, 0.f);
            const float alpha = first ? 0.f : __builtin_amdgcn_exp2f(-delta);
            cm[nt] -= delta;
            // this half's scores and, when it is the first half, the second's as well
#pragma unroll
            for (int h2 = h; h2 < 2; ++h2) {
              st[h2][0][nt] -= delta;
              st[h2][1][nt] -= delta;
            }
            l_run[nt] *= alpha;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) o[dt][nt] *= alpha;
          }
          probs();
        }
#pragma unroll
        for (int nt = 0; nt < NQT; ++nt) l_run[nt] += tsum[nt];

        __builtin_amdgcn_s_setprio(0);
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
    if (qbase >= nq) {
      // A wave of the last query tile with no rows left: it takes part in the
      // workgroup's staging (its share of each K and V tile) and barriers only,
      // leaving its SIMD to the other workgroup's wave.
      for (int j = kt0; j < kt1; ++j) {
        __syncthreads();
        if (j + 1 < kt1) {
          locate(j + 1);
          kload((j + 1 - kt0) & 1);
          vload((j + 1 - kt0) & 1);
          __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
        }
      }
    } else {
      for (int j = kt0; j < kt1; j += 2) {
        tile(j, 0);
        if (j + 1 < kt1) tile(j + 1, 1);
      }
    }

    // Row totals; m of each row.
    float lt[NQT], mr[NQT];
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
      lt[nt] = sum4_lanes(l_run[nt]);
      mr[nt] = -cm[nt][0];
    }
    bool emit = true;
    if (kt0 != 0 || kt1 != ntiles) {
      // A piece of a cut unit: record (unit of the last round, piece) of the workspace.
      const int rec0 = (unit - rounds * P) * cuts;
      auto record = [&](int piece) -> float* {
        return wk.partials + (int64_t)(rec0 + piece) * kAttnRecFloats + wave * kRecWave;
      };
      {
        float* rec = record(cut);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
          for (int nt = 0; nt < NQT; ++nt)
            *reinterpret_cast<f32x4_t*>(rec + ((dt * NQT + nt) * 64 + lane) * 4) = o[dt][nt];
#pragma unroll
        for (int nt = 0; nt < NQT; ++nt) {
          rec[kRecO + nt * 64 + lane] = mr[nt];
          rec[kRecO + (NQT + nt) * 64 + lane] = lt[nt];
        }
      }
      __threadfence();  // this piece's record is visible before its arrival is counted
      __syncthreads();
      if (tid == 0) s_arrival = atomicAdd(&wk.counters[unit], 1);
      __syncthreads();
      emit = s_arrival == cuts - 1;
      if (emit) {
        // Last piece to arrive: merge every piece's record (this one's included) in
        // piece order, so the result is the same whichever piece arrives last.
        __threadfence();
        if (tid == 0) wk.counters[unit] = 0;
#pragma unroll
        for (int nt = 0; nt < NQT; ++nt) mr[nt] = -INFINITY;
        for (int i = 0; i < cuts; ++i) {
          const float* rec = record(i);
#pragma unroll
          for (int nt = 0; nt < NQT; ++nt) mr[nt] = fmaxf(mr[nt], rec[kRecO + nt * 64 + lane]);
        }
#pragma unroll
        for (int nt = 0; nt < NQT; ++nt) {
          lt[nt] = 0.f;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) o[dt][nt] = f32x4_t{};
        }
        for (int i = 0; i < cuts; ++i) {
          const float* rec = record(i);
#pragma unroll
          for (int nt = 0; nt < NQT; ++nt) {
            const float f = __builtin_amdgcn_exp2f(rec[kRecO + nt * 64 + lane] - mr[nt]);
            lt[nt] = fmaf(rec[kRecO + (NQT + nt) * 64 + lane], f, lt[nt]);
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
              const f32x4_t v =
                  *reinterpret_cast<const f32x4_t*>(rec + ((dt * NQT + nt) * 64 + lane) * 4);
#pragma unroll
              for (int e = 0; e < 4; ++e) o[dt][nt][e] = fmaf(v[e], f, o[dt][nt][e]);
            }
          }
        }
      }
    }
    if (emit) {
#pragma unroll
      for (int nt = 0; nt < NQT; ++nt) {
        const int qrow = qbase + 16 * nt + c;
        if (qrow < nq) {
          const float inv = 1.f / lt[nt];
          uint16_t* op = out + qrow * rs + head * D + 4 * g;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) {
            const uint32_t w0 = pack_bf16(o[dt][nt][0] * inv, o[dt][nt][1] * inv);
            const uint32_t w1 = pack_bf16(o[dt][nt][2] * inv, o[dt][nt][3] * inv);
            *reinterpret_cast<uint2*>(op + 16 * dt) = make_uint2(w0, w1);
          }
          if (lse != nullptr && g == 0)
            lse[(int64_t)head * nq + qrow] = (mr[nt] + __log2f(lt[nt])) * 0.69314718055994531f;
        }
      }
    }
  }
}

}  // namespace

int attn_bf16_units(int nq, int heads) { return (nq + BM - 1) / BM * heads; }

hipError_t launch_attn_bf16(const void* q, void* out, float* lse, const AttnSegs& segs, int nq,
                            int nk, int heads, float qmul, const AttnWorkspace& ws,
                            hipStream_t s, const KernelTiming* tm, const float* qcs) {
  const int qtiles = (nq + BM - 1) / BM;
  const int units = qtiles * heads;
  const int ntiles = segs.tend[segs.nseg - 1];
  AttnWork wk = {nullptr, nullptr, 1};
  int nwg = units;  // one workgroup per unit
  if (ws.counters != nullptr) {
    // persistent slots; the last round is cut when it would leave over half idle
    const int P = ws.slots;
    const int urem = units % P;
    int cuts = urem > 0 ? P / urem : 1;
    if (cuts > ntiles) cuts = ntiles;
    if (cuts >= 2) {
      wk.counters = ws.counters;
      wk.partials = ws.partials;
      wk.cuts = cuts;
      nwg = units < P ? urem * cuts : P;
    }
  }
  if (qcs != nullptr)
    launch_kernel(tm, attn_bf16_kernel<true>, dim3(nwg), dim3(NTHREADS), 0, s,
                  static_cast<const uint16_t*>(q), static_cast<uint16_t*>(out), lse, segs, nq,
                  nk, heads, qmul, qtiles, nwg, wk, qcs);
  else
    launch_kernel(tm, attn_bf16_kernel<false>, dim3(nwg), dim3(NTHREADS), 0, s,
                  static_cast<const uint16_t*>(q), static_cast<uint16_t*>(out), lse, segs, nq,
                  nk, heads, qmul, qtiles, nwg, wk, static_cast<const float*>(nullptr));
  return hipGetLastError();
}

}  // namespace la
