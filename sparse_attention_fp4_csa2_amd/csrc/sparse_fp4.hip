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
//  * of the two workgroups on a CU the older one wins instruction arbitration
//    and finishes far ahead of the other; waves drop their priority on every
//    other tile, which evens out the two.
#include "device.h"
#include "launch.h"
#include "window_body.h"

namespace csa2 {

namespace {

constexpr int TILE = 32;                 // entries per tile
constexpr int PROW = 40;                 // fp16 slots per P row (32 entries + 8 pad)
constexpr int MAX_SPLIT_BLOCKS = 2048;   // selected block ids one workgroup stages in LDS
constexpr float LAZY_LOG2 = 8.0f;        // move the running max only when it grows by > 2^8
constexpr float M_INIT = -1.0e30f;       // finite "no max yet": exp2(x - M_INIT) never NaN
constexpr int VBIAS = 140;               // V' = V * 2^(VBIAS - vbase): code 6 at vbase -> 6*2^13

typedef int int32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));

struct Lds {
  floatx4 sp[2][4][4][64];         // [buffer][wave][quarter][lane] partial S^T  32 KB
  uint16_t pb[2][32 * PROW];       // [buffer][head * PROW + slot] fp16 P        5 KB
  float qmax[2][4][32];            // [buffer][wave][head] quarter max of z*log2e
  int flag[2][4];                  // [buffer][wave] quarter needs a max move
  float lsum[4][32];               // epilogue: per-wave softmax denominators
  int emax[4][32];                 // epilogue: per-wave exponent of the largest |o|
  int32_t blk[MAX_SPLIT_BLOCKS];   // this split's selected block ids           8 KB
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
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = max(v, __shfl_xor(v, m, 64));
  return v;
}

struct Raw {
  uint4 c0, c1;    // 32 bytes of codes: this wave's dims 64s + 32hh + [0, 32), s = 0, 1
  uint32_t sc;     // scale bytes of groups 4dq .. 4dq + 3
  int valid;
};

constexpr int BUF_DWORD3 = 0x00020000;   // gfx9 raw buffer descriptor word 3

}  // namespace

// One workgroup's share: rows `row`, split `split` of p.splits, head group hgi
__device__ __forceinline__ void sparse_unit(const AttnParams& p, int row, int split, int hgi, Lds& lds) {
  const int tid = threadIdx.x;
  const int dq = tid >> 6;        // wave: latent dims [128dq, 128dq + 128)
  const int lane = tid & 63;
  const int e = lane & 31;        // Q.K: entry of the tile;  S^T, P^T, O^T: head of the group
  const int hh = lane >> 5;
  const int b = row / p.Q;
  const int head = 32 * hgi + e;
  const bool head_ok = head < p.H;

  int n_items = p.count[row];
  n_items = n_items < 0 ? 0 : (n_items > p.top_k ? p.top_k : n_items);
  const int t_pos = p.q_pos ? p.q_pos[row] : 0;
  const int n_tiles = (n_items + 3) / 4;
  const int tps = (n_tiles + p.splits - 1) / p.splits;
  const int t_begin = split * tps;
  const int t_end = min(n_tiles, t_begin + tps);
  const int n_ent = p.n_entries[b];
  const int nb_cap = p.cap / BLOCK;
  // entries below lim are present and visible (entry j covers raw positions
  // 2j and 2j + 1; a causal query at raw position t sees 2j + 1 <= t)
  const int lim = p.q_pos ? min(n_ent, (t_pos + 1) >> 1) : n_ent;
  const int n_items_split = min(n_items, 4 * t_end);
  // this sequence's records as a raw buffer: ids outside [0, nb_cap) (the -1
  // padding included) fall outside it and load zeros
  const __amdgpu_buffer_rsrc_t rec_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.cache + (size_t)b * nb_cap * RECORD), (short)0, nb_cap * RECORD, BUF_DWORD3);
  const uint32_t code_off = (e & 7) * 256 + 64 * dq + 16 * hh;
  const uint32_t sc_off = SCALE_OFF + (e & 7) * 16 + 4 * dq;
  const float c_log2 = p.scale_log2;
  auto read_id = [&](int t) -> int {
    const int item = 4 * t + (e >> 3);
    return item < n_items_split ? lds.blk[min(item - 4 * t_begin, MAX_SPLIT_BLOCKS - 1)] : -1;
  };
  auto fetch = [&](int blk, Raw& r) {
    r.valid = (uint32_t)blk < (uint32_t)nb_cap && blk * BLOCK + (e & 7) < lim;
    const uint32_t off = (uint32_t)blk * RECORD;
    r.c0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rec_rsrc, off + code_off, 0, 0));
    r.c1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rec_rsrc, off + code_off + 32, 0, 0));
    r.sc = __builtin_amdgcn_raw_buffer_load_b32(rec_rsrc, off + sc_off, 0, 0);
  };

  // block ids of the first three tiles straight from memory, so that the first
  // records are in flight while the query is converted; the whole split's ids
  // are staged in LDS meanwhile
  const int32_t* const idx_row = p.idx + (size_t)row * p.top_k;
  auto mem_id = [&](int t) -> int {
    const int item = 4 * t + (e >> 3);
    const int v = idx_row[min(item, p.top_k - 1)];   // unconditional: the loads overlap
    return item < n_items_split ? v : -1;
  };
  const int i_beg = 4 * t_begin;
  const int stage0 = idx_row[min(i_beg + tid, p.top_k - 1)];
  Raw r0, ra, rb, rx;     // raw tiles (see the tile loop)
  fetch(mem_id(t_begin), r0);
  fetch(mem_id(t_begin + 1), ra);
  int id_next = mem_id(t_begin + 2);   // this lane's block id for the next fetch (read a tile early)

  // ---- query: three FP6 (E2M3) terms per 32-dim block -----------------
  // lane (head, hh), k-step s: FP6 value k = dim 128dq + 64s + 32hh + k.  Each
  // lane's 32 values are one block of the scaled MFMA with its own E8M0 scale:
  // every term rounds (to nearest even) what the earlier terms left, at the
  // scale of its own largest value.
  int32x8 qt[3][2];       // [term][k-step]
  uint32_t qsb = 0;       // scale bytes: [0] term 0 s0, [1] term 0 s1, [2] term 1 s0, [3] term 1 s1
  uint32_t qsb2 = 0;      // [0] term 2 s0, [1] term 2 s1
  {
    const uint16_t* qrow = p.q + ((size_t)row * p.H + (head_ok ? head : 0)) * D + 128 * dq + 32 * hh;
    const uint32_t m = head_ok ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float x[32];
      const uint4* src = reinterpret_cast<const uint4*>(qrow + 64 * s);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint4 w = src[u];
        const uint32_t wv[4] = {w.x & m, w.y & m, w.z & m, w.w & m};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[8 * u + 2 * k] = __uint_as_float(wv[k] << 16);
          x[8 * u + 2 * k + 1] = __uint_as_float(wv[k] & 0xFFFF0000u);
        }
      }
      // y0[i], y1[i] = values 2i, 2i + 1 of the block, relative to 2^etot
      floatx16 y0, y1;
#pragma unroll
      for (int i2 = 0; i2 < 16; ++i2) y0[i2] = x[2 * i2], y1[i2] = x[2 * i2 + 1];
      int etot = 0;
#pragma unroll
      for (int term = 0; term < 3; ++term) {
        float mx = 0.f;
#pragma unroll
        for (int i2 = 0; i2 < 16; ++i2) mx = fmaxf(mx, fmaxf(fabsf(y0[i2]), fabsf(y1[i2])));
        const int e = fp6_block_exp(mx, -127 - etot);
        const float f = ldexpf(1.f, -e);
#pragma unroll
        for (int i2 = 0; i2 < 16; ++i2) y0[i2] *= f, y1[i2] *= f;     // a power of two
        etot += e;
        const int6v c = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(y0, y1, 1.f);
        qt[term][s] = int32x8{c[0], c[1], c[2], c[3], c[4], c[5], 0, 0};
        const uint32_t sbyte = (uint32_t)(127 + etot);
        if (term < 2) qsb |= sbyte << (8 * (2 * term + s));
        else qsb2 |= sbyte << (8 * s);
        if (term < 2) {
          const floatx32 d = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(c, 1.f);
#pragma unroll
          for (int i2 = 0; i2 < 16; ++i2) y0[i2] -= d[2 * i2], y1[i2] -= d[2 * i2 + 1];   // exact
        }
      }
    }
  }

  if (i_beg + tid < n_items_split) lds.blk[tid] = stage0;
  for (int i = i_beg + tid + 256; i < n_items_split; i += 256) lds.blk[i - i_beg] = idx_row[i];
  __syncthreads();

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
    sacc = mfma_fp4_fp6<0>(r.c0, qt[0][0], sacc, s8, qsb);
    sacc = mfma_fp4_fp6<2>(r.c0, qt[1][0], sacc, s8, qsb);
    sacc = mfma_fp4_fp6<0>(r.c0, qt[2][0], sacc, s8, qsb2);
    sacc = mfma_fp4_fp6<1>(r.c1, qt[0][1], sacc, s8b, qsb);
    sacc = mfma_fp4_fp6<3>(r.c1, qt[1][1], sacc, s8b, qsb);
    sacc = mfma_fp4_fp6<1>(r.c1, qt[2][1], sacc, s8b, qsb2);
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
    vmask_cur = (uint32_t)__ballot(r0.valid);
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
  //   reads: S(t) partials, P(t-1), flags(t-1), V^T(t-1) (all written before B(t-1))
  //   P(t-1).V(t-1) (after a rare max move) | softmax(t): P(t), flags(t) written
  //   V(t+1) written, Q.K(t+1), S(t+1) partial written
  // S, P, flags and the V tile are double-buffered by tile parity.
  auto tile_step = [&](int t, const Raw& rp, Raw& rc, Raw& rl) {
    const int buf = t & 1;
    if (t & 1) __builtin_amdgcn_s_setprio(1);    // wave priority alternates by tile
    else __builtin_amdgcn_s_setprio(0);
    const bool more = t + 1 < t_end;
    fetch(id_next, rl);
    id_next = read_id(t + 3);
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
      vmask_cur = (uint32_t)__ballot(rc.valid);
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

  // ---- finalize: denominators across the 4 quarter owners -----------------
  const float lq = pair_sum(l_lane);
  if (lane < 32) lds.lsum[dq][lane] = lq;
  __syncthreads();
  const float l = (lds.lsum[0][e] + lds.lsum[1][e]) + (lds.lsum[2][e] + lds.lsum[3][e]);
  const float il = l > 0.f ? 1.f / l : 0.f;
  if (head_ok && dq == 0 && hh == 0) {
    const float lse = l > 0.f ? (m_run + log2f(l)) * 0.69314718055994531f : -__builtin_inff();
    p.lse_out[((size_t)row * p.out_splits + p.split_base + split) * p.H + head] = lse;
  }
  const size_t orow = ((size_t)row * p.out_splits + p.split_base + split) * p.H + head;
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

__global__ __launch_bounds__(256, 2) void sparse_fp4_kernel(AttnParams p, int n_units, int hgroups) {
  __shared__ Lds lds;
  int unit, hgi;
  map_unit(blockIdx.x, n_units, hgroups, p.splits > 1, unit, hgi);
  if (unit >= n_units) return;
  sparse_unit(p, unit / p.splits, unit % p.splits, hgi, lds);
}

// Both branches of one layer in one launch, in one of two arrangements:
//  * inline (pw.splits <= ps.splits): every sparse workgroup (row, split s,
//    head group) then runs the window's split s of the same row and head
//    group, when s < pw.splits.  The window work is spread over all the
//    sparse workgroups, so it adds a few tiles to each of them instead of
//    running as short workgroups after them.
//  * after: the grid is the sparse workgroups followed by the window's, so
//    the window runs in the slots the sparse workgroups free as they finish.
__global__ __launch_bounds__(256, 2) void attend_kernel(AttnParams ps, int n_units, int hgroups,
                                                        int n_sparse_wg, AttnParams pw, int whgroups,
                                                        int inline_window) {
  __shared__ union {
    Lds s;
    win::WinLds w;
  } lds;
  int unit, hgi;
  if ((int)blockIdx.x < n_sparse_wg) {
    map_unit(blockIdx.x, n_units, hgroups, ps.splits > 1, unit, hgi);
    if (unit >= n_units) return;
    const int row = unit / ps.splits, split = unit - row * ps.splits;
    sparse_unit(ps, row, split, hgi, lds.s);
    if (inline_window && split < pw.splits) {
      __syncthreads();                      // the window reuses the LDS
      win::window_unit(pw, row, split, hgi, lds.w);
    }
  } else {
    const int wn = pw.rows * pw.splits;
    map_unit((int)blockIdx.x - n_sparse_wg, wn, whgroups, pw.splits > 1, unit, hgi);
    if (unit >= wn) return;
    win::window_unit(pw, unit / pw.splits, unit % pw.splits, hgi, lds.w);
  }
}

int sparse_fp4_splits(int rows, int H, int n_tiles) {
  const int hgroups = (H + 31) / 32;
  const int wgs = rows * hgroups;
  int s = (512 + wgs - 1) / wgs;                 // two workgroups per CU
  const int cap_by_tiles = n_tiles / 2 > 1 ? n_tiles / 2 : 1;
  if (s > cap_by_tiles) s = cap_by_tiles;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  const int min_s = (n_tiles + MAX_SPLIT_BLOCKS / 4 - 1) / (MAX_SPLIT_BLOCKS / 4);
  if (s < min_s) s = min_s;
  return s;
}

int launch_sparse_fp4(const AttnParams& p, hipStream_t stream) {
  const int hgroups = (p.H + 31) / 32;
  const int n_units = p.rows * p.splits;
  const int groups = (n_units + 7) / 8;
  const long long n_wg = (long long)groups * 8 * hgroups;
  if (n_wg > 0x7FFFFFFF) return -4;
  sparse_fp4_kernel<<<dim3((unsigned)n_wg), 256, 0, stream>>>(p, n_units, hgroups);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_attend(const AttnParams& ps, const AttnParams& pw, bool inline_window, hipStream_t stream) {
  const int hgroups = (ps.H + 31) / 32;
  const int n_units = ps.rows * ps.splits;
  const long long n_sparse = (long long)((n_units + 7) / 8) * 8 * hgroups;   // a multiple of 8
  const int whgroups = (pw.H + 31) / 32;
  if (inline_window && (pw.splits > ps.splits || whgroups != hgroups || pw.rows != ps.rows)) return -4;
  const long long n_window = inline_window ? 0 : (long long)((pw.rows * pw.splits + 7) / 8) * 8 * whgroups;
  if (n_sparse + n_window > 0x7FFFFFFF) return -4;
  attend_kernel<<<dim3((unsigned)(n_sparse + n_window)), 256, 0, stream>>>(ps, n_units, hgroups, (int)n_sparse,
                                                                           pw, whgroups, inline_window ? 1 : 0);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace csa2
