// Split-K multi-head attention over the selected blocks of the MXFP4 latent
// cache (gather + dequant + Q.K + online softmax + P.V in one pass).
//
// What is computed: one 512-d latent per entry is the key AND the value of
// every head (paper-digest.app page, Core Mechanics, "Compressed along three
// axes"); only the top-K selected blocks of 8 entries are attended
// (observer.broadside.tech card, Key ideas, "CSA2 with three static layer
// modes").  Per head: z_j = scale * q . V_j, o = softmax(z) V, lse = log sum
// exp z, over the selected, present, visible entries; splits of the selection
// are merged by log-sum-exp afterwards.
//
// Organisation: one workgroup = (row, split, group of 32 heads), 4 waves; wave
// dq owns latent dims [128dq, 128dq + 128) for all 32 heads.  Two workgroups
// fit on a CU (<= 256 registers per lane, ~48 KB LDS), so one wave's VALU work
// overlaps the other's MFMAs.  A tile is 32 entries (4 blocks).  Per tile:
//  * Q.K: lane (entry e = lane%32, half hh) loads 32 bytes of e's FP4 codes for
//    the wave's dims and feeds them unconverted to v_mfma_scale_f32_32x32x64_
//    f8f6f4 (A = E2M1 codes with their E8M0 scales, B = the query as three
//    FP6 E2M3 terms with one E8M0 scale per 32 dims; an FP4 x FP6 product runs
//    at twice the FP4 x FP8 rate): S^T[32 entries][32 heads] over 128 dims.
//    A wave whose query blocks spread too far for the scaled MFMA's sums (an
//    outlier channel over small values) runs Q.K on bf16 MFMAs instead, with
//    the codes dequantised to bf16 (exact) and the bf16 query itself.
//  * the 4 partial S^T tiles meet in LDS; wave dq sums the quarter of the tile
//    it owns (entries 8dq..8dq+7), runs the online softmax on it and writes its
//    quarter of P (fp16) back: every wave then reads the whole P^T tile as the
//    B operand of O^T += V^T P^T (v_mfma_f32_32x32x16_f16).
//  * V never touches LDS: the same codes, still in registers one tile later,
//    are the A operand of a scaled FP4 x FP4 MFMA against the identity, which
//    applies each entry's E8M0 scale (and a per-wave power-of-two base through
//    the B scale) and leaves V' fp32 with entries along the accumulator rows,
//    i.e. already transposed for the P.V A operand; v_cvt_pk_f16_f32 packs it.
//    Per 32 x 32 block that is one fast-rate MFMA and 8 conversions instead of
//    16 VALU dequantisation steps plus an LDS round trip.
//  * the running max moves lazily (only when a head's max grows by > 2^8); a
//    tile that needs a move takes a rare uniform slow path.
//  * workgroup order: each XCD takes a contiguous range of (row, split, head
//    group), so a row's query and (between its two head groups) its records
//    are read from HBM once and then hit that XCD's L2.
//  * row tiles: with 16 or fewer heads a row leaves columns of the tile idle,
//    so 2 or 4 rows of one sequence share them (see sparse_unit) and attend
//    the union of their selections, each block gathered and dequantised once
//    for all of them.
#include "device.h"
#include "launch.h"
#include "select.h"
#include "window_body.h"

namespace csa2 {

namespace {

constexpr int TILE = 32;                 // entries per tile
constexpr int PROW = 40;                 // fp16 slots per P row (32 entries + 8 pad)
constexpr int MAX_SPLIT_BLOCKS = 2048;   // selected block ids one workgroup stages in LDS
// row tiles stage twice as many (the union of up to R selections), so that a
// tile of two rows needs no second split for the K = 2048 of each
template <int R>
constexpr int stage_blocks() { return R > 1 ? 2 * MAX_SPLIT_BLOCKS : MAX_SPLIT_BLOCKS; }
constexpr float LAZY_LOG2 = 8.0f;        // move the running max only when it grows by > 2^8
constexpr float M_INIT = -1.0e30f;       // finite "no max yet": exp2(x - M_INIT) never NaN
constexpr int VBIAS = 140;               // V' = V * 2^(VBIAS - vbase): code 6 at vbase -> 6*2^13

typedef int int32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));

template <int R>
struct Lds {
  union {
    floatx4 sp[2][4][4][64];       // [buffer][wave][quarter][lane] partial S^T  32 KB
    uint32_t bm[8192];             // row tiles' prologue: each row's selected-block bitmap
  };
  uint16_t pb[2][32 * PROW];       // [buffer][head * PROW + slot] fp16 P        5 KB
  float qmax[2][4][32];            // [buffer][wave][head] quarter max of z*log2e
  int flag[2][4];                  // [buffer][wave] quarter needs a max move
  float lsum[4][32];               // epilogue: per-wave softmax denominators
  int emax[4][32];                 // epilogue: per-wave exponent of the largest |o|
  int32_t blk[stage_blocks<R>()];  // this split's selected block ids           8 KB (row tiles 16 KB)
  uint8_t memb[R > 1 ? stage_blocks<R>() : 4];   // row tiles: bit r = row r of the tile selected the item
  uint32_t scan[4];                // row tiles: per-wave sums of the union count
  int dup;                         // row tiles: some row lists a block twice
};

// A = 32 E2M1 codes, B = 32 E2M1 codes (byte 0 of each scale operand)
__device__ __forceinline__ floatx16 mfma_fp4_fp4(uint4 a, uint4 b, uint32_t sa, uint32_t sb) {
  const int32x8 av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const int32x8 bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, floatx16{}, 4, 4, 0, (int)sa, 0, (int)sb);
}

// A = 32 E2M1 codes, B = 32 E2M3 values (byte OPB of sb is B's scale)
template <int OPB>
__device__ __forceinline__ floatx16 mfma_fp4_fp6(uint4 a, const int32x8& b, floatx16 c, uint32_t sa, uint32_t sb) {
  const int32x8 av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, b, c, 4, 2, 0, (int)sa, OPB, (int)sb);
}

// A = 8 bf16 of 32 entries, B = 8 bf16 of 32 heads: S^T over 16 dims, fp32
__device__ __forceinline__ floatx16 mfma_bf16(uint4 a, uint4 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ floatx16 mfma_f16(uint4 a, uint4 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a),
                                                __builtin_bit_cast(halfx8, b), c, 0, 0, 0);
}

typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_f16(float a, float b) {    // v_cvt_pk_f16_f32, RNE
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{a, b}, halfx2));
}

typedef int int6v __attribute__((ext_vector_type(6)));
typedef float floatx32 __attribute__((ext_vector_type(32)));

// smallest e >= emin with mx * 2^-e <= 7.5 (the largest E2M3 value); 0 when mx
// is 0 or not finite
__device__ __forceinline__ int fp6_block_exp(float mx, int emin) {
  if (!(mx > 0.f && mx < __builtin_inff())) return max(0, emin);
  int e = ilogbf(mx) - 2;                      // mx * 2^-e in [4, 8)
  if (ldexpf(mx, -e) > 7.5f) ++e;
  return max(e, emin);
}

// (lane l, lane l^32) reductions: v_permlane32_swap gives {lane l%32, lane l%32 + 32}
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ int wave_max_int(int v) {
  v = (int)wave_allreduce((uint32_t)v, [](uint32_t a, uint32_t b) {
    return (uint32_t)max((int)a, (int)b);
  });
  return v;
}

struct Raw {
  uint4 c0, c1;    // 32 bytes of codes: this wave's dims 64s + 32hh + [0, 32), s = 0, 1
  uint32_t sc;     // scale bytes of groups 4dq .. 4dq + 3
  int valid;       // the entry is present and visible; row tiles: bit r = visible to row r of the tile
};

constexpr int BUF_DWORD3 = 0x00020000;   // gfx9 raw buffer descriptor word 3

}  // namespace

// One workgroup's share: split `split` of p.splits, head group hgi, of one
// tile of rows.  R == 1: the tile is row `row`, its 32 columns the heads 32 hgi
// + [0, 32).  R > 1 (few heads per row): the tile is group `row` of R
// consecutive rows of one sequence (the sequence's rows in groups of R, the
// last group possibly shorter), column e = row e / (32 / R) of the group and
// head (32 / R) hgi + e % (32 / R); the tile attends the union of its rows'
// selections, each block gathered and its V dequantised once for every row
// that selected it, and each column masked to its own row's blocks and causal
// limit.  Should a row list a block twice (or the cache be too large for the
// union's bitmap) the rows' lists are run one after the other instead, each
// block once per row that lists it, as a single row would count it.
// after_loop(oacc, m_run, l_lane, base_o) runs when the tile loop is done,
// before the epilogue, and may continue the softmax state (the fused launch
// runs its window share there, so both branches leave one partial).
template <int R, typename AfterLoop>
__device__ __forceinline__ void sparse_unit(const AttnParams& p, int row, int split, int hgi, Lds<R>& lds,
                                            AfterLoop after_loop) {
  constexpr int HP = 32 / R;      // heads per row among the tile's 32 columns
  const int tid = threadIdx.x;
  const int dq = tid >> 6;        // wave: latent dims [128dq, 128dq + 128)
  const int lane = tid & 63;
  const int e = lane & 31;        // Q.K: entry of the tile;  S^T, P^T, O^T: column of the tile
  const int hh = lane >> 5;
  int b, q0, nr;                  // the tile's sequence, first query and row count
  if (R == 1) {
    b = row / p.Q;
    q0 = row - b * p.Q;
    nr = 1;
  } else {
    const int ngq = (p.Q + R - 1) / R;
    b = row / ngq;
    q0 = (row - b * ngq) * R;
    nr = min(R, p.Q - q0);
  }
  const int row0 = b * p.Q + q0;
  const int rsub = e / HP;        // this lane's column: row row0 + rsub, head HP hgi + e % HP
  const int row_l = row0 + rsub;
  const int head = HP * hgi + e % HP;
  const bool head_ok = head < p.H && rsub < nr;

  const int n_ent = p.n_entries[b];
  const int nb_cap = p.cap / BLOCK;
  int n_items, t_begin, t_end, n_items_split, lim = n_ent;
  int lim_r[R];                   // row tiles: entries below lim_r[r] are present and visible to row r
  if (R == 1) {
    n_items = p.count[row];
    n_items = n_items < 0 ? 0 : (n_items > p.top_k ? p.top_k : n_items);
    const int t_pos = p.q_pos ? p.q_pos[row] : 0;
    const int n_tiles = (n_items + 3) / 4;
    // splits partition the row's top_k slots, not its count, so the first block
    // ids are requested before the count arrives; the count only ends the loop
    const int tps = ((p.top_k + 3) / 4 + p.splits - 1) / p.splits;
    t_begin = split * tps;
    t_end = min(n_tiles, t_begin + tps);
    // entries below lim are present and visible (entry j covers raw positions
    // 2j and 2j + 1; a causal query at raw position t sees 2j + 1 <= t)
    lim = p.q_pos ? min(n_ent, (t_pos + 1) >> 1) : n_ent;
    n_items_split = min(n_items, 4 * t_end);
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r)
      lim_r[r] = r < nr ? (p.q_pos ? min(n_ent, (p.q_pos[row0 + r] + 1) >> 1) : n_ent) : 0;
  }
  // this sequence's records as a raw buffer: ids outside [0, nb_cap) (the -1
  // padding included) fall outside it and load zeros
  const __amdgpu_buffer_rsrc_t rec_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.cache + (size_t)b * nb_cap * RECORD), (short)0, nb_cap * RECORD, BUF_DWORD3);
  const uint32_t code_off = (e & 7) * 256 + 64 * dq + 16 * hh;
  const uint32_t sc_off = SCALE_OFF + (e & 7) * 16 + 4 * dq;
  const float c_log2 = p.scale_log2;
  auto read_id = [&](int t) -> int {
    const int item = 4 * t + (e >> 3);
    return item < n_items_split ? lds.blk[min(item - 4 * t_begin, stage_blocks<R>() - 1)] : -1;
  };
  auto read_mb = [&](int t) -> int {
    const int item = 4 * t + (e >> 3);
    return R > 1 && item < n_items_split ? lds.memb[min(item - 4 * t_begin, stage_blocks<R>() - 1)] : 0;
  };
  auto fetch = [&](int blk, int mb, Raw& r) {
    const int ent = blk * BLOCK + (e & 7);
    r.valid = (uint32_t)blk < (uint32_t)nb_cap && ent < lim;
    if (R > 1) {
      int ok = 0;
#pragma unroll
      for (int k = 0; k < R; ++k) ok |= (r.valid && ((mb >> k) & 1) && ent < lim_r[k]) ? 1 << k : 0;
      r.valid = ok;
    }
    const uint32_t off = (uint32_t)blk * RECORD;
    r.c0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rec_rsrc, off + code_off, 0, 0));
    r.c1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rec_rsrc, off + code_off + 32, 0, 0));
    r.sc = __builtin_amdgcn_raw_buffer_load_b32(rec_rsrc, off + sc_off, 0, 0);
  };
  // the tile's entry mask for this lane's column: row tiles combine each
  // entry's presence with its row bits and the column row's causal limit
  auto tile_mask = [&](const Raw& r) -> uint32_t {
    if (R == 1) return (uint32_t)__ballot(r.valid);
    uint32_t vm = 0;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const uint32_t m = (uint32_t)__ballot((r.valid >> k) & 1);
      vm = rsub == k ? m : vm;
    }
    return vm;
  };

  // the query's bf16 values first (this lane's 64: dims 128dq + 64s + 32hh +
  // [0, 32)), so their latency overlaps the block ids' and the first records'
  const uint32_t qmask = head_ok ? 0xFFFFFFFFu : 0u;
  uint4 qraw[2][4];
  {
    const uint16_t* qrow = p.q + ((size_t)(head_ok ? row_l : row0) * p.H + (head_ok ? head : 0)) * D +
                           128 * dq + 32 * hh;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int u = 0; u < 4; ++u) qraw[s2][u] = reinterpret_cast<const uint4*>(qrow + 64 * s2)[u];
  }

  Raw r0, ra, rb, rx;     // raw tiles (see the tile loop)
  int id_next, mb_next = 0;   // this lane's block id (and row bits) for the next fetch (read a tile early)
  const int32_t* const idx_row = p.idx + (size_t)row0 * p.top_k;
  const int i_beg = 4 * (R == 1 ? t_begin : 0);
  int stage0 = 0;
  if (R == 1) {
    // block ids of the first three tiles straight from memory, so that the
    // first records are in flight while the query is converted; the whole
    // split's ids are staged in LDS meanwhile
    auto mem_id = [&](int t) -> int {
      const int item = 4 * t + (e >> 3);
      const int v = idx_row[min(item, p.top_k - 1)];   // unconditional: the loads overlap
      return item < n_items_split ? v : -1;
    };
    stage0 = idx_row[min(i_beg + tid, p.top_k - 1)];
    fetch(mem_id(t_begin), 0, r0);
    fetch(mem_id(t_begin + 1), 0, ra);
    id_next = mem_id(t_begin + 2);
  } else {
    // ---- row tile: the union of the rows' selections ----------------------
    // a bitmap of each row's blocks in LDS (over the S buffers, unused until
    // the first Q.K), then the union enumerated in ascending block order; the
    // split's share of it goes to blk, with each item's row bits in memb
    constexpr int BMW = 8192 / R;              // bitmap words per row
    const bool use_bm = nb_cap <= 32 * BMW;
    const int nw = (nb_cap + 31) >> 5;
    int nsel[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int c = r < nr ? p.count[row0 + r] : 0;
      nsel[r] = c < 0 ? 0 : (c > p.top_k ? p.top_k : c);
    }
    if (use_bm)
      for (int i = tid; i < R * nw; i += 256) lds.bm[(i / nw) * BMW + i % nw] = 0;
    if (tid == 0) lds.dup = 0;
    __syncthreads();
    if (use_bm) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        for (int i = tid; i < nsel[r]; i += 256) {
          const int id = idx_row[(size_t)r * p.top_k + i];
          if ((uint32_t)id < (uint32_t)nb_cap) {
            const uint32_t bit = 1u << (id & 31);
            if (atomicOr(&lds.bm[r * BMW + (id >> 5)], bit) & bit) lds.dup = 1;
          }
        }
    }
    __syncthreads();
    auto set_split = [&](int u) {
      n_items = u;
      const int nt = (u + 3) / 4;
      const int tps = (nt + p.splits - 1) / p.splits;
      t_begin = split * tps;
      t_end = min(nt, t_begin + tps);
      n_items_split = min(u, 4 * t_end);
    };
    if (use_bm && lds.dup == 0) {
      // thread t counts the union's blocks in words [wpt t, wpt t + wpt)
      const int wpt = (nw + 255) / 256;
      uint32_t cnt = 0;
      for (int k = 0; k < wpt; ++k) {
        const int w = wpt * tid + k;
        if (w < nw) {
          uint32_t u = 0;
#pragma unroll
          for (int r = 0; r < R; ++r) u |= lds.bm[r * BMW + w];
          cnt += __builtin_popcount(u);
        }
      }
      uint32_t total;
      uint32_t rank = sel::block_excl_scan<256>(cnt, lds.scan, &total);
      set_split((int)total);
      const uint32_t lo = 4 * t_begin, hi = n_items_split;
      for (int k = 0; k < wpt && rank < hi; ++k) {
        const int w = wpt * tid + k;
        if (w >= nw) break;
        uint32_t wr[R], u = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) wr[r] = lds.bm[r * BMW + w], u |= wr[r];
        for (; u != 0 && rank < hi; u &= u - 1, ++rank) {
          if (rank < lo) continue;
          const int bit = __builtin_ctz(u);
          int mb = 0;
#pragma unroll
          for (int r = 0; r < R; ++r) mb |= (int)((wr[r] >> bit) & 1u) << r;
          lds.blk[rank - lo] = 32 * w + bit;
          lds.memb[rank - lo] = (uint8_t)mb;
        }
      }
    } else {
      // the rows' own lists one after the other (item k of the concatenation:
      // row r's entry k - (the earlier rows' counts))
      int u = 0;
#pragma unroll
      for (int r = 0; r < R; ++r) u += nsel[r];
      set_split(u);
      for (int k = 4 * t_begin + tid; k < n_items_split; k += 256) {
        int r = 0, kk = k;
#pragma unroll
        for (int j = 0; j < R - 1; ++j)
          if (r == j && kk >= nsel[j]) kk -= nsel[j], r = j + 1;
        const int id = idx_row[(size_t)r * p.top_k + kk];
        lds.blk[k - 4 * t_begin] = (uint32_t)id < (uint32_t)nb_cap ? id : -1;
        lds.memb[k - 4 * t_begin] = (uint8_t)(1 << r);
      }
    }
    __syncthreads();      // the union's share staged; the bitmaps (over S) are free again
    fetch(read_id(t_begin), read_mb(t_begin), r0);
    fetch(read_id(t_begin + 1), read_mb(t_begin + 1), ra);
    id_next = read_id(t_begin + 2);
    mb_next = read_mb(t_begin + 2);
  }
  // ---- query -----------------------------------------------------------
  // FP6 form: three E2M3 terms per 32-dim block.  Lane (head, hh), k-step s:
  // FP6 value k = dim 128dq + 64s + 32hh + k.  Each lane's 32 values are one
  // block of the scaled MFMA with its own E8M0 scale: every term rounds (to
  // nearest even) what the earlier terms left, each at a scale 2^4 finer than
  // the last, which carries each value to within 2^-11.9 of the block's largest.
  // The scaled MFMA sums its 64 products to about 15 bits below the largest
  // one, so a query block whose values spread far below its largest (fewer than
  // half of them within 2^5 of it: an outlier channel over a bulk of small
  // values) would lose the bulk's share of q.K there, whatever the split.  A
  // wave holding such a block takes the bf16 form instead: K dequantised to
  // bf16 (exact) against the bf16 query itself on v_mfma_f32_32x32x16_bf16,
  // whose fp32 sums keep every bit the bulk needs.  Lane (head, hh) of bf16
  // MFMA m = 4s + u holds dims 128dq + 64s + 32hh + 8u + [0, 8), the same dims
  // its FP6 block covers, so both forms load the same query bytes and the same
  // codes.  The choice is wave-uniform (each wave's Q.K partial is its own sum),
  // and the bf16 query reuses the FP6 terms' registers.
  int32x8 qt[3][2];       // [term][k-step]; bf16 form: qt[T / 2][T % 2] holds MFMAs 2T, 2T + 1
  uint32_t qsb = 0;       // scale bytes: [0] term 0 s0, [1] term 0 s1, [2] term 1 s0, [3] term 1 s1
  uint32_t qsb2 = 0;      // FP6: [0] term 2 s0, [1] term 2 s1
  bool wide = false;
  {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float x[32];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint4 w = qraw[s][u];
        const uint32_t wv[4] = {w.x & qmask, w.y & qmask, w.z & qmask, w.w & qmask};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[8 * u + 2 * k] = __uint_as_float(wv[k] << 16);
          x[8 * u + 2 * k + 1] = __uint_as_float(wv[k] & 0xFFFF0000u);
        }
      }
      // y0[i], y1[i] = values 2i, 2i + 1 of the block
      floatx16 y0, y1;
#pragma unroll
      for (int i2 = 0; i2 < 16; ++i2) y0[i2] = x[2 * i2], y1[i2] = x[2 * i2 + 1];
      float mx = 0.f;
#pragma unroll
      for (int i2 = 0; i2 < 16; ++i2) mx = fmaxf(mx, fmaxf(fabsf(y0[i2]), fabsf(y1[i2])));
      {
        // values within 2^5 of the largest (same binade-or-above of 2^(e(mx) - 5))
        const uint32_t em = __float_as_uint(mx) >> 23;
        if (em > 5) {
          const float thr = __uint_as_float((em - 5) << 23);
          int near = 0;
#pragma unroll
          for (int k = 0; k < 32; ++k) near += fabsf(x[k]) >= thr ? 1 : 0;
          wide |= near < 16;
        }
      }
      // term scales 2^e0, 2^(e0 - 4), 2^(e0 - 8): the first puts the largest
      // |value| in (3.75, 7.5]; E2M3 rounding leaves at most 0.25 of a term's
      // scale, which the next term (2^4 finer) holds below 4, so no term
      // saturates and the last leaves at most 2^(e0 - 10) <= 2^-11.9 of the
      // largest.  The conversions take the scale (dividing, and multiplying back).
      const int e0 = max(fp6_block_exp(mx, -126), -126);
      const int ex[3] = {e0, max(e0 - 4, -126), max(e0 - 8, -126)};
#pragma unroll
      for (int term = 0; term < 3; ++term) {
        const float sc = __uint_as_float((uint32_t)(127 + ex[term]) << 23);
        const int6v c = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(y0, y1, sc);
        qt[term][s] = int32x8{c[0], c[1], c[2], c[3], c[4], c[5], 0, 0};
        const uint32_t sbyte = (uint32_t)(127 + ex[term]);
        if (term < 2) qsb |= sbyte << (8 * (2 * term + s));
        else qsb2 |= sbyte << (8 * s);
        if (term < 2) {
          const floatx32 d = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(c, sc);
#pragma unroll
          for (int i2 = 0; i2 < 16; ++i2) y0[i2] -= d[2 * i2], y1[i2] -= d[2 * i2 + 1];   // exact
        }
      }
    }
  }
  const bool qb = __any(wide) != 0;     // wave-uniform: the bf16 form
  if (qb) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const uint4 v = qraw[m >> 2][m & 3];
      const int T = m >> 1, o = 4 * (m & 1);
      qt[T >> 1][T & 1][o] = (int)(v.x & qmask);
      qt[T >> 1][T & 1][o + 1] = (int)(v.y & qmask);
      qt[T >> 1][T & 1][o + 2] = (int)(v.z & qmask);
      qt[T >> 1][T & 1][o + 3] = (int)(v.w & qmask);
    }
  }

  if (R == 1) {
    if (i_beg + tid < n_items_split) lds.blk[tid] = stage0;
    for (int i = i_beg + tid + 256; i < n_items_split; i += 256) lds.blk[i - i_beg] = idx_row[i];
    __syncthreads();
  }

  // ---- tile helpers -----------------------------------------------------
  // largest scale byte of the wave's groups in the tile (every fetched entry,
  // so no dequantised value can overflow fp16), folded into the running base
  auto raise_base = [&](const Raw& r, int cur) -> int {
    const uint32_t s = r.sc;
    const int smax = max(max((int)(s & 0xFF), (int)((s >> 8) & 0xFF)),
                         max((int)((s >> 16) & 0xFF), (int)(s >> 24)));
    if (__any(smax > cur)) return max(cur, wave_max_int(smax));
    return cur;
  };
  // Q.K partial S^T over the wave's 128 dims -> LDS
  auto qk_s = [&](int sbuf, const Raw& r) {
    // the MFMA reads the E8M0 scale from byte 0 of its scale operand
    const uint32_t s8 = r.sc >> (8 * hh);
    const uint32_t s8b = s8 >> 16;
    floatx16 sacc = floatx16{};
    if (qb) {
      const uint32_t cw[2][4] = {{r.c0.x, r.c0.y, r.c0.z, r.c0.w}, {r.c1.x, r.c1.y, r.c1.z, r.c1.w}};
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int ks = m >> 2, u = m & 3, T = m >> 1, o = 4 * (m & 1);
        const uint4 ka = dequant8(cw[ks][u], (r.sc >> (8 * (2 * ks + hh))) & 0xFFu);
        const int32x8& qv = qt[T >> 1][T & 1];
        sacc = mfma_bf16(ka, make_uint4((uint32_t)qv[o], (uint32_t)qv[o + 1], (uint32_t)qv[o + 2],
                                        (uint32_t)qv[o + 3]), sacc);
      }
    } else {
      sacc = mfma_fp4_fp6<0>(r.c0, qt[0][0], sacc, s8, qsb);
      sacc = mfma_fp4_fp6<2>(r.c0, qt[1][0], sacc, s8, qsb);
      sacc = mfma_fp4_fp6<0>(r.c0, qt[2][0], sacc, s8, qsb2);
      sacc = mfma_fp4_fp6<1>(r.c1, qt[0][1], sacc, s8b, qsb);
      sacc = mfma_fp4_fp6<3>(r.c1, qt[1][1], sacc, s8b, qsb);
      sacc = mfma_fp4_fp6<1>(r.c1, qt[2][1], sacc, s8b, qsb2);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      lds.sp[sbuf][dq][j][lane] = floatx4{sacc[4 * j], sacc[4 * j + 1], sacc[4 * j + 2], sacc[4 * j + 3]};
  };

  floatx16 oacc[4];       // O^T: [dims 128dq + 32mt + 8(i/4) + 4hh + i%4][head]
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) oacc[mt] = floatx16{};
  float m_run = M_INIT;   // running max of z * log2(e), per head (lane pair)
  float l_lane = 0.f;     // softmax denominator over this lane's quarter entries
  int base_o = 0;         // O^T is in units of 2^(base_o - VBIAS)
  int base_v = 0;         // base of the newest dequantised V tile
  floatx4 sq_prev = floatx4{};   // the previous tile's logits quarter (for a late max move)
  float pr_prev[4] = {0.f, 0.f, 0.f, 0.f};   // ... and its softmax weights
  uint4 pfr[2];           // P^T B fragments of the previous tile, [ks2]
  int base_prev = 0;      // base of those V^T fragments

  // V^T fragments come out of the dequantising MFMA with k = 8hh' + j of k-step
  // ks2 holding entry 16ks2 + 8(j/4) + 4hh' + j%4 (its output row order); P^T
  // uses the same order, so entry 8dq + 4hh + r sits at P slot pslot + r
  const int pslot = 16 * (dq >> 1) + 8 * hh + 4 * (dq & 1);
  // identity B operands of that MFMA (E2M1 1.0 = code 2): bid[h'] selects the
  // 32 dims 32h' + [0, 32) of a 64-dim k-step (lane (n, hb) holds k = 32hb + [0, 32))
  uint4 bid[2];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const uint32_t v = hh == h2 ? 2u << (4 * (e & 7)) : 0u;
    const int d = e >> 3;
    bid[h2] = make_uint4(d == 0 ? v : 0u, d == 1 ? v : 0u, d == 2 ? v : 0u, d == 3 ? v : 0u);
  }

  uint32_t vmask_cur = 0;
  if (t_begin < t_end) {
    base_v = raise_base(r0, 13);     // >= 13: the dequantising MFMA's B scale byte 267 - base fits
    base_o = base_v;
    qk_s(t_begin & 1, r0);
    vmask_cur = tile_mask(r0);
  }
  __syncthreads();

  // P(t-1).V(t-1): V^T of each 32-dim group straight from the tile's codes in
  // registers: a scaled FP4 x FP4 MFMA against the identity applies each
  // entry's E8M0 scale (A scale) and 2^(VBIAS - base) (B scale), giving fp32
  // V'[entry][dim] in the accumulator layout, whose rows are the A operand's k
  auto issue_pv = [&](const Raw& r) {
    if (base_prev != base_o) {        // that tile's V used a higher base: rescale O exactly
      const float f = ldexpf(1.f, base_o - base_prev);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) oacc[mt] *= f;
      base_o = base_prev;
    }
    const uint32_t bsb = (uint32_t)(127 + VBIAS - base_prev);
    const uint32_t s8 = r.sc >> (8 * hh);
    // two dequantising MFMAs in flight: mt + 1's runs while mt's result is packed
    floatx16 vn = mfma_fp4_fp4(r.c0, bid[0], s8, bsb);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const floatx16 v = vn;
      if (mt < 3) vn = mfma_fp4_fp4(mt + 1 < 2 ? r.c0 : r.c1, bid[(mt + 1) & 1], mt + 1 < 2 ? s8 : s8 >> 16, bsb);
      const uint4 a0 = make_uint4(pack_f16(v[0], v[1]), pack_f16(v[2], v[3]), pack_f16(v[4], v[5]),
                                  pack_f16(v[6], v[7]));
      const uint4 a1 = make_uint4(pack_f16(v[8], v[9]), pack_f16(v[10], v[11]), pack_f16(v[12], v[13]),
                                  pack_f16(v[14], v[15]));
      oacc[mt] = mfma_f16(a0, pfr[0], oacc[mt]);
      oacc[mt] = mfma_f16(a1, pfr[1], oacc[mt]);
    }
  };

  auto read_pfr = [&](int buf) {
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2)
      pfr[ks2] = *reinterpret_cast<const uint4*>(&lds.pb[buf][e * PROW + 16 * ks2 + 8 * hh]);
  };
  auto write_p = [&](int buf, const float (&pr)[4]) {
    uint16_t* pdst = &lds.pb[buf][e * PROW + pslot];
    *reinterpret_cast<uint2*>(pdst) = make_uint2(pack_f16(pr[0], pr[1]), pack_f16(pr[2], pr[3]));
  };
  // Tile t-1's P(t-1).V(t-1), after the rare max move it may need (decided from
  // every wave's quarter maxima of that tile, visible since the last barrier).
  auto finish_prev = [&](int pbuf, const Raw& rp) {
    const int4 fl = *reinterpret_cast<const int4*>(&lds.flag[pbuf][0]);
    read_pfr(pbuf);
    if (fl.x | fl.y | fl.z | fl.w) {          // rare (always after the first tile)
      const float tmax = fmaxf(fmaxf(lds.qmax[pbuf][0][e], lds.qmax[pbuf][1][e]),
                               fmaxf(lds.qmax[pbuf][2][e], lds.qmax[pbuf][3][e]));
      const float m_new = tmax > m_run + LAZY_LOG2 ? tmax : m_run;
      if (__any(m_new != m_run)) {
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) oacc[mt] *= alpha;
        l_lane *= alpha;
        m_run = m_new;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) pr_prev[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sq_prev[r], c_log2, -m_run));
      write_p(pbuf, pr_prev);
      __syncthreads();
      read_pfr(pbuf);
    }
    l_lane += (pr_prev[0] + pr_prev[1]) + (pr_prev[2] + pr_prev[3]);
    issue_pv(rp);
  };

  // Pipeline, one barrier per tile.  Tile t, between barriers B(t-1) and B(t)
  // (rc = tile t+1's records, loaded during tile t-1; rl receives tile t+2's,
  // requested first so that a whole tile of work hides their latency):
  //   reads: S(t) partials, P(t-1), flags(t-1) (all written before B(t-1))
  //   P(t-1).V(t-1), V dequantised from tile t-1's codes, still in registers
  //   (after a rare max move) | softmax(t): P(t), flags(t) written |
  //   Q.K(t+1), S(t+1) partial written
  // S, P and flags are double-buffered by tile parity; V never enters LDS.
  auto tile_step = [&](int t, const Raw& rp, Raw& rc, Raw& rl) {
    const int buf = t & 1;
    const bool more = t + 1 < t_end;
    fetch(id_next, mb_next, rl);
    id_next = read_id(t + 3);
    mb_next = read_mb(t + 3);
    floatx4 sw[4];
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) sw[w2] = lds.sp[buf][w2][dq][lane];
    if (t > t_begin) finish_prev(buf ^ 1, rp);
    int base_next = base_v;
    if (more) base_next = raise_base(rc, base_v);
    floatx4 sq;
#pragma unroll
    for (int r = 0; r < 4; ++r) sq[r] = (sw[0][r] + sw[1][r]) + (sw[2][r] + sw[3][r]);
    if (vmask_cur != 0xFFFFFFFFu) {
      const uint32_t vq = vmask_cur >> (8 * dq + 4 * hh);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (!((vq >> r) & 1u)) sq[r] = -__builtin_inff();
    }
    const float hmax = pair_max(fmaxf(fmaxf(sq[0], sq[1]), fmaxf(sq[2], sq[3]))) * c_log2;
    const bool bump = hmax > m_run + LAZY_LOG2;
#pragma unroll
    for (int r = 0; r < 4; ++r) pr_prev[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sq[r], c_log2, -m_run));
    write_p(buf, pr_prev);
    const int any_bump = __any(bump) ? 1 : 0;
    if (lane < 32) lds.qmax[buf][dq][lane] = hmax;
    if (lane == 0) lds.flag[buf][dq] = any_bump;
    sq_prev = sq;
    base_prev = base_v;           // the base tile t's V is dequantised with
    if (more) {
      qk_s(buf ^ 1, rc);
      vmask_cur = tile_mask(rc);
      base_v = base_next;
    }
    __syncthreads();
  };
  // raw tiles rotate through four register sets: tile t's codes serve Q.K(t)
  // at step t-1 and P.V(t) at step t+1; step k = t - t_begin: tile t in
  // R[k % 4], t+1 in R[(k+1) % 4], t+2 arriving in R[(k+2) % 4], t-1 in R[(k+3) % 4]
  for (int t = t_begin; t < t_end; t += 4) {
    tile_step(t, rx, ra, rb);
    if (t + 1 < t_end) tile_step(t + 1, r0, rb, rx);
    if (t + 2 < t_end) tile_step(t + 2, ra, rx, r0);
    if (t + 3 < t_end) tile_step(t + 3, rb, r0, ra);
  }
  if (t_begin < t_end) {
    const int k = (t_end - 1 - t_begin) & 3;
    finish_prev((t_end - 1) & 1, k == 0 ? r0 : k == 1 ? ra : k == 2 ? rb : rx);
  }
  after_loop(oacc, m_run, l_lane, base_o);

  // ---- finalize: denominators across the 4 quarter owners -----------------
  const float lq = pair_sum(l_lane);
  if (lane < 32) lds.lsum[dq][lane] = lq;
  __syncthreads();
  const float l = (lds.lsum[0][e] + lds.lsum[1][e]) + (lds.lsum[2][e] + lds.lsum[3][e]);
  const float il = l > 0.f ? 1.f / l : 0.f;
  if (head_ok && dq == 0 && hh == 0) {
    const float lse = l > 0.f ? (m_run + log2f(l)) * 0.69314718055994531f : -__builtin_inff();
    p.lse_out[((size_t)row_l * p.H + head) * p.out_splits + p.split_base + split] = lse;
  }
  const size_t orow = ((size_t)row_l * p.H + head) * p.out_splits + p.split_base + split;
  if (!p.o16_out) {                  // one split: the final fp32 o
    if (head_ok) {
      const float f = ldexpf(il, base_o - VBIAS);
      float* dst = p.o_out + orow * D + 128 * dq + 4 * hh;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          *reinterpret_cast<float4*>(dst + 32 * mt + 8 * jj) =
              make_float4(oacc[mt][4 * jj] * f, oacc[mt][4 * jj + 1] * f, oacc[mt][4 * jj + 2] * f,
                          oacc[mt][4 * jj + 3] * f);
    }
    return;
  }
  // split-K partial: fp16 o relative to a per-head power of two, so the largest
  // |o| of the head lands in [2^14, 2^15); the 4 waves (each with its own V base)
  // agree on it through LDS
  float am = 0.f;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(oacc[mt][i]));
  am = pair_max(am * il);
  constexpr int E_NONE = -100000;
  if (lane < 32) lds.emax[dq][lane] = am > 0.f ? ilogbf(am) + base_o - VBIAS : E_NONE;
  __syncthreads();
  int k = max(max(lds.emax[0][e], lds.emax[1][e]), max(lds.emax[2][e], lds.emax[3][e]));
  if (k == E_NONE) k = 0;
  if (head_ok) {
    if (dq == 0 && hh == 0) p.oexp_out[orow] = k - 14;
    store_o16_slice(oacc, il, base_o - VBIAS + 14 - k, hh, p.o16_out + orow * D + 128 * dq);
  }
}

// R rows per tile (1, 2, 4); a unit is (tile, split)
template <int R>
__global__ __launch_bounds__(256, 2) void sparse_fp4_kernel(AttnParams p, int n_units, int hgroups) {
  __shared__ Lds<R> lds;
  // every argument the prologue needs, in one round of scalar loads: left to
  // itself the compiler loads them in three dependent rounds, each waited on
  // where it is first used (the early return splits the prologue)
  asm volatile("" ::"s"(p.q), "s"(p.cache), "s"(p.idx), "s"(p.count), "s"(p.n_entries), "s"(p.q_pos),
               "s"(p.top_k), "s"(p.cap), "s"(p.Q), "s"(p.H), "s"(p.splits), "s"(p.scale_log2));
  int unit, hgi;
  map_unit(blockIdx.x, n_units, hgroups, p.splits > 1, unit, hgi);
  if (unit >= n_units) return;
  sparse_unit<R>(p, unit / p.splits, unit % p.splits, hgi, lds, [](floatx16(&)[4], float&, float&, int&) {});
}

// Both branches of one layer in one launch, in one of two arrangements:
//  * inline (pw.splits <= ps.splits): every sparse workgroup (row, split s,
//    head group) then runs the window's split s of the same row and head
//    group, when s < pw.splits, continuing its online softmax: the two
//    branches leave one partial per sparse split (pw's outputs are unused),
//    and a layer with one sparse split needs no combine.  The window work is
//    spread over all the sparse workgroups, so it adds a few tiles to each of
//    them instead of running as short workgroups after them.
//  * after: the grid is the sparse workgroups followed by the window's, so
//    the window runs in the slots the sparse workgroups free as they finish.
// Row tiles (R > 1) run the window inline on the same tile of rows (each
// column over its own row's window); after, on one row per workgroup.
template <int R>
__global__ __launch_bounds__(256, 2) void attend_kernel(AttnParams ps, int n_units, int hgroups,
                                                        int n_sparse_wg, AttnParams pw, int whgroups,
                                                        int inline_window) {
  __shared__ union {
    Lds<R> s;
    win::WinLds w;
  } lds;
  // every argument the sparse prologue needs, in one round of scalar loads (as
  // in sparse_fp4_kernel; decode attention calls 1-2 us faster)
  asm volatile("" ::"s"(ps.q), "s"(ps.cache), "s"(ps.idx), "s"(ps.count), "s"(ps.n_entries), "s"(ps.q_pos),
               "s"(ps.top_k), "s"(ps.cap), "s"(ps.Q), "s"(ps.H), "s"(ps.splits), "s"(ps.scale_log2));
  int unit, hgi;
  if ((int)blockIdx.x < n_sparse_wg) {
    map_unit(blockIdx.x, n_units, hgroups, ps.splits > 1, unit, hgi);
    if (unit >= n_units) return;
    const int row = unit / ps.splits, split = unit - row * ps.splits;
    if (inline_window && split < pw.splits) {
      // this workgroup's window split continues the softmax of its sparse
      // split: one partial for both.  The accumulator leaves its V base for
      // plain units first (an exact power of two), as the bf16 window rows
      // are not rescaled.
      sparse_unit<R>(ps, row, split, hgi, lds.s,
                  [&](floatx16 (&oacc)[4], float& m_run, float& l_lane, int& base_o) {
                    const float rs = ldexpf(1.f, base_o - VBIAS);
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) oacc[mt] *= rs;
                    base_o = VBIAS;
                    __syncthreads();          // the window reuses the LDS
                    win::window_tiles<R>(pw, row, split, hgi, lds.w, oacc, m_run, l_lane);
                    __syncthreads();          // the epilogue's LDS overlaps the window's
                  });
    } else {
      sparse_unit<R>(ps, row, split, hgi, lds.s, [](floatx16(&)[4], float&, float&, int&) {});
    }
  } else {
    const int wn = pw.rows * pw.splits;
    map_unit((int)blockIdx.x - n_sparse_wg, wn, whgroups, pw.splits > 1, unit, hgi);
    if (unit >= wn) return;
    win::window_unit(pw, unit / pw.splits, unit % pw.splits, hgi, lds.w);
  }
}

int sparse_fp4_splits(int rows, int H, int n_tiles, int stage) {
  const int hgroups = (H + 31) / 32;
  const int wgs = rows * hgroups;
  int s = (512 + wgs - 1) / wgs;                 // two workgroups per CU
  const int cap_by_tiles = n_tiles / 2 > 1 ? n_tiles / 2 : 1;
  if (s > cap_by_tiles) s = cap_by_tiles;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  const int min_s = (n_tiles + stage / 4 - 1) / (stage / 4);   // each split's share fits the staging
  if (s < min_s) s = min_s;
  return s;
}

// Rows per tile: a row fills the tile's 32 MFMA columns with its own heads when
// H > 16; with 16 or fewer heads (one GPU's share of 64 heads split 4 or 8
// ways) 2 or 4 consecutive rows of a sequence share the columns and every
// gathered block.
int sparse_rows_per_tile(int H, int Q) {
  int r = H <= 8 ? 4 : (H <= 16 ? 2 : 1);
  while (r > 1 && r > Q) r >>= 1;
  return r;
}

// Split count of a sparse launch over B sequences of Q rows: the rule above
// over its tiles (a row tile attends up to R selections, so its splits keep
// each split's share of the union within the LDS staging)
int sparse_attn_splits(int B, int Q, int H, int top_k) {
  const int r = sparse_rows_per_tile(H, Q);
  const int tiles = B * ((Q + r - 1) / r);
  const int hp = 32 / r;
  return sparse_fp4_splits(tiles * ((H + hp - 1) / hp), 32, (r * top_k + 3) / 4,
                           r > 1 ? stage_blocks<2>() : stage_blocks<1>());
}

namespace {
// grid of a sparse launch: (tile, split) units x head groups, the units a multiple of 8
struct SparseGrid {
  int r, n_units, hgroups;
  long long n_wg;
};
SparseGrid sparse_grid(const AttnParams& p) {
  SparseGrid g;
  g.r = sparse_rows_per_tile(p.H, p.Q);
  const int B = p.rows / p.Q;
  g.n_units = B * ((p.Q + g.r - 1) / g.r) * p.splits;
  const int hp = 32 / g.r;
  g.hgroups = (p.H + hp - 1) / hp;
  g.n_wg = (long long)((g.n_units + 7) / 8) * 8 * g.hgroups;
  return g;
}
}  // namespace

int launch_sparse_fp4(const AttnParams& p, hipStream_t stream) {
  const SparseGrid g = sparse_grid(p);
  if (g.n_wg > 0x7FFFFFFF) return -4;
  const dim3 grid((unsigned)g.n_wg);
  if (g.r == 4)
    sparse_fp4_kernel<4><<<grid, 256, 0, stream>>>(p, g.n_units, g.hgroups);
  else if (g.r == 2)
    sparse_fp4_kernel<2><<<grid, 256, 0, stream>>>(p, g.n_units, g.hgroups);
  else
    sparse_fp4_kernel<1><<<grid, 256, 0, stream>>>(p, g.n_units, g.hgroups);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_attend(const AttnParams& ps, const AttnParams& pw, bool inline_window, hipStream_t stream) {
  const SparseGrid g = sparse_grid(ps);
  const long long n_sparse = g.n_wg;   // a multiple of 8
  const int whgroups = (pw.H + 31) / 32;
  if (inline_window && (pw.splits > ps.splits || pw.H != ps.H || pw.Q != ps.Q || pw.rows != ps.rows)) return -4;
  const long long n_window = inline_window ? 0 : (long long)((pw.rows * pw.splits + 7) / 8) * 8 * whgroups;
  if (n_sparse + n_window > 0x7FFFFFFF) return -4;
  const dim3 grid((unsigned)(n_sparse + n_window));
  const int inl = inline_window ? 1 : 0;
  if (g.r == 4)
    attend_kernel<4><<<grid, 256, 0, stream>>>(ps, g.n_units, g.hgroups, (int)n_sparse, pw, whgroups, inl);
  else if (g.r == 2)
    attend_kernel<2><<<grid, 256, 0, stream>>>(ps, g.n_units, g.hgroups, (int)n_sparse, pw, whgroups, inl);
  else
    attend_kernel<1><<<grid, 256, 0, stream>>>(ps, g.n_units, g.hgroups, (int)n_sparse, pw, whgroups, inl);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace csa2
