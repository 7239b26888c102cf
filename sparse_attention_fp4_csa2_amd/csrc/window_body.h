// Window-attention workgroup body (bf16 rows of each sequence's sliding
// window), shared by the window kernel and the fused attention launch.
//
// The same organisation as the MXFP4 sparse kernel, on bf16 rows.  One
// workgroup = (row, split, group of 32 heads), 4 waves; wave dq owns latent
// dims [128dq, 128dq + 128) for all 32 heads; two workgroups share a CU.
// A tile is 32 window tokens.  Per tile:
//  * Q.K: lane (token e = lane%32, half hh) holds 64 contiguous dims of e's row
//    as the A operand of v_mfma_f32_32x32x16_bf16 (8 k-steps), the query the
//    B operand: S^T[32 tokens][32 heads] over the wave's 128 dims.
//  * the 4 partial S^T tiles meet in LDS; wave dq sums the quarter it owns
//    (tokens 8dq..8dq+7), runs the online softmax on it and writes its quarter
//    of P as bf16 hi + lo parts (16 significant bits: bf16 P alone leaves
//    errors near 1e-2 of the output RMS); every wave reads the whole P^T tile.
//  * V: the same registers go to the wave's own LDS tile (token-major) and come
//    back transposed with ds_read_b64_tr_b16 for O^T += V^T P^T (two MFMAs per
//    k-step, hi and lo).
//  * lazy running max (moves only when a head's max grows by > 2^8; a tile
//    that needs a move takes a rare uniform slow path); the rows of tile t+1
//    are requested at the start of tile t.
#pragma once
#include "device.h"
#include "launch.h"

namespace csa2 {
namespace win {

constexpr int TILE = 32;                 // tokens per tile
constexpr int VROWU = 20;                // 16-byte units per V row: 16 data + 4 pad
// unit u of V row r sits at u ^ ((r >> 1) & 3): with 20-unit rows both the
// row writes (b128) and the transposed reads are free of LDS bank conflicts
constexpr int PROW = 40;                 // bf16 slots per P row (32 tokens + 8 pad)
constexpr float LAZY_LOG2 = 8.0f;        // move the running max only when it grows by > 2^8
constexpr float M_INIT = -1.0e30f;       // finite "no max yet": exp2(x - M_INIT) never NaN
constexpr int WINDOW_TARGET_WGS = 256;   // workgroups the split count aims for
constexpr int WINDOW_MIN_TILES = 2;      // tiles per split, at least

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef float floatx2 __attribute__((ext_vector_type(2)));

struct WinLds {
  floatx4 sp[4][4][64];            // [wave][quarter][lane] partial S^T          16 KB
  uint4 v[4][TILE * VROWU];        // [wave][token * VROWU + unit] bf16 V tile   40 KB
  uint16_t ph[2][32 * PROW];       // [buffer][head * PROW + slot] bf16 P hi     5 KB
  uint16_t pl[2][32 * PROW];       // [buffer][head * PROW + slot] bf16 P lo     5 KB
  float qmax[2][4][32];            // [buffer][wave][head] quarter max of z*log2e
  int flag[2][4];                  // [buffer][wave] quarter needs a max move
  float lsum[4][32];               // epilogue: per-wave softmax denominators
  int emax[4][32];                 // epilogue: per-wave exponent of the largest |o|
};

__device__ __forceinline__ floatx16 mfma_bf16(uint4 a, uint4 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// (a, b) -> bf16 hi parts (v_cvt_pk_bf16_f32, round to nearest even) and the
// bf16 of the remainders, so that hi + lo carries 16 significant bits.
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{a, b}, bf16x2));
  const float ha = __uint_as_float(hi << 16), hb = __uint_as_float(hi & 0xFFFF0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{a - ha, b - hb}, bf16x2));
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

struct WinRaw {
  uint4 k[8];      // dims 128dq + 64hh + 8s + [0, 8) of token e, s < 8
};

// The window tiles of one workgroup's share (row `row`, split `split` of
// p.splits, head group hgi), continuing the online softmax state it is given:
// O^T in oacc (plain units), the running max and this lane's denominator.  The
// fused launch passes the state its sparse share left, so the two branches
// leave one partial; window_unit starts from an empty state.  R > 1: the
// sparse kernel's row tile (group `row` of R consecutive rows of a sequence,
// column e = row e / (32 / R), head (32 / R) hgi + e % (32 / R)); the tiles
// cover the union of the rows' windows and each column is masked to its own.
template <int R = 1>
__device__ __forceinline__ void window_tiles(const AttnParams& p, int row, int split, int hgi, WinLds& lds,
                                             floatx16 (&oacc)[4], float& m_run, float& l_lane) {
  constexpr int HP = 32 / R;      // heads per row among the 32 columns
  const int tid = threadIdx.x;
  const int dq = tid >> 6;        // wave: latent dims [128dq, 128dq + 128)
  const int lane = tid & 63;
  const int e = lane & 31;        // Q.K: token of the tile;  S^T, P^T, O^T: column of the tile
  const int hh = lane >> 5;
  int b, q0, nr;
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
  const int rsub = e / HP;
  const int head = HP * hgi + e % HP;
  const bool head_ok = head < p.H && rsub < nr;

  // ---- visible window slots [lo, lo + n_items) of this row (row tiles: the
  // union of the rows' visible slots, row r's own being [lo + zlo[r], lo + zhi[r]]) ----
  const int len = min(p.swa_len[b], p.Lw);
  const int pos0 = p.swa_pos0 ? p.swa_pos0[b] : 0;
  int za = 0x7FFFFFFF, zb = -0x7FFFFFFF;
  int zlo[R], zhi[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int tq = r < nr ? (p.q_pos ? p.q_pos[row0 + r] : pos0 + len - 1) : 0;
    zlo[r] = max(tq - p.W + 1, pos0);
    zhi[r] = r < nr ? min(tq, pos0 + len - 1) : zlo[r] - 1;
    if (zhi[r] >= zlo[r]) za = min(za, zlo[r]), zb = max(zb, zhi[r]);
  }
  const int n_items = zb >= za ? zb - za + 1 : 0;
  const int lo = n_items ? za - pos0 : 0;
  if (n_items)
#pragma unroll
    for (int r = 0; r < R; ++r) zlo[r] -= za, zhi[r] -= za;
  const int n_tiles = (n_items + TILE - 1) / TILE;
  const int tps = (n_tiles + p.splits - 1) / p.splits;
  const int t_begin = split * tps;
  const int t_end = min(n_tiles, t_begin + tps);
  const int dim0 = 128 * dq + 64 * hh;      // this lane's 64 contiguous dims
  const float c_log2 = p.scale_log2;

  // ---- query: B operand, lane (column, hh), k-step s: dims dim0 + 8s + [0, 8) ----
  uint4 qf[8];
  {
    const uint4* src = reinterpret_cast<const uint4*>(
        p.q + ((size_t)(head_ok ? row0 + rsub : row0) * p.H + (head_ok ? head : 0)) * D + dim0);
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) qf[s8] = head_ok ? src[s8] : make_uint4(0, 0, 0, 0);
  }
  // the tile's token mask for this lane's column
  auto tile_mask = [&](int t) -> uint32_t {
    const bool ok = t < t_end && TILE * t + e < n_items;
    if (R == 1) return (uint32_t)__ballot(ok);
    const int sl = TILE * t + e;
    uint32_t vm = 0;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const uint32_t m = (uint32_t)__ballot(ok && sl >= zlo[k] && sl <= zhi[k]);
      vm = rsub == k ? m : vm;
    }
    return vm;
  };

  // ---- tile helpers -----------------------------------------------------
  // token e of tile t; slots past the split or the window read the row's first
  // visible slot (in bounds whenever the split has tiles); their logits are
  // masked and their P is 0
  auto token_ok = [&](int t) { return t < t_end && TILE * t + e < n_items; };
  auto fetch = [&](int t, WinRaw& r) {
    const int slot = token_ok(t) ? TILE * t + e : 0;
    const uint4* src = reinterpret_cast<const uint4*>(
        p.swa + ((size_t)b * p.Lw + lo + slot) * D + dim0);
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) r.k[s8] = src[s8];
  };
  uint4* const vrow = &lds.v[dq][e * VROWU];
  const int vx = (e >> 1) & 3;
  auto write_v = [&](const WinRaw& r) {
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) vrow[(8 * hh + s8) ^ vx] = r.k[s8];
  };
  auto qk_s = [&](const WinRaw& r) {
    floatx16 sacc = floatx16{};
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) sacc = mfma_bf16(r.k[s8], qf[s8], sacc);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      lds.sp[dq][j][lane] = floatx4{sacc[4 * j], sacc[4 * j + 1], sacc[4 * j + 2], sacc[4 * j + 3]};
  };

  uint2 vt[2][4][2];      // V^T A fragments of the previous tile, [ks2][mt][half]
  uint4 phf[2], plf[2];   // P^T B fragments (hi, lo) of the previous tile, [ks2]
  bool have_pv = false;

  // P slot of token 8dq + 4hh + r within its 16-token k-step, matching the
  // k -> token order of the transposed V^T reads
  const int pslot = 16 * (dq >> 1) + 8 * hh + 4 * (dq & 1);

  WinRaw rn;              // rows of the next tile, requested at the start of a tile
  uint32_t vmask_cur = 0;
  if (t_begin < t_end) {
    fetch(t_begin, rn);
    write_v(rn);
    qk_s(rn);
    vmask_cur = tile_mask(t_begin);
  }
  __syncthreads();

  auto issue_pv = [&]() {
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const uint4 va = make_uint4(vt[ks2][mt][0].x, vt[ks2][mt][0].y, vt[ks2][mt][1].x, vt[ks2][mt][1].y);
        oacc[mt] = mfma_bf16(va, phf[ks2], oacc[mt]);
        oacc[mt] = mfma_bf16(va, plf[ks2], oacc[mt]);
      }
  };

  const int sl = lane & 15, blk16 = lane >> 4;
  const int u0 = 2 * (blk16 & 1) + ((sl & 3) >> 1);
  auto read_pfr = [&](int buf) {
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      phf[ks2] = *reinterpret_cast<const uint4*>(&lds.ph[buf][e * PROW + 16 * ks2 + 8 * hh]);
      plf[ks2] = *reinterpret_cast<const uint4*>(&lds.pl[buf][e * PROW + 16 * ks2 + 8 * hh]);
    }
  };
  auto write_p = [&](int buf, const float (&pr)[4]) {
    uint32_t h0, l0, h1, l1;
    split_bf16x2(pr[0], pr[1], h0, l0);
    split_bf16x2(pr[2], pr[3], h1, l1);
    *reinterpret_cast<uint2*>(&lds.ph[buf][e * PROW + pslot]) = make_uint2(h0, h1);
    *reinterpret_cast<uint2*>(&lds.pl[buf][e * PROW + pslot]) = make_uint2(l0, l1);
  };

  // Pipeline, two barriers per tile t (the rows of tile t+1 are requested at
  // its start and consumed at its end):
  //   X(t) = [B1(t), B2(t)): P.V(t-1) MFMAs | S(t) quarter reads, softmax,
  //          P(t) written
  //   Y(t) = [B2(t), B1(t+1)): P^T(t), V^T(t) reads | V(t+1) written, Q.K(t+1)
  //          MFMAs, S(t+1) partial written
  for (int t = t_begin; t < t_end; ++t) {
    const int buf = t & 1;
    const bool more = t + 1 < t_end;
    if (more) fetch(t + 1, rn);
    // ---- X(t) ---------------------------------------------------------------
    floatx4 sw[4];
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) sw[w2] = lds.sp[w2][dq][lane];
    if (have_pv) issue_pv();
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
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sq[r], c_log2, -m_run));
    write_p(buf, pr);
    const int any_bump = __any(bump) ? 1 : 0;
    if (lane < 32) lds.qmax[buf][dq][lane] = hmax;
    if (lane == 0) lds.flag[buf][dq] = any_bump;
    __syncthreads();

    // ---- Y(t): every LDS read of the tile at once: flags, P^T(t), V^T(t) ------
    const int4 fl = *reinterpret_cast<const int4*>(&lds.flag[buf][0]);
    read_pfr(buf);
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      const int r0 = 16 * ks2 + 4 * (blk16 >> 1) + (sl >> 2);
      const int x0 = (r0 >> 1) & 3, x1 = ((r0 + 8) >> 1) & 3;
      const uint16_t* vb0 = reinterpret_cast<const uint16_t*>(&lds.v[dq][r0 * VROWU + (u0 ^ x0)]) + 4 * (sl & 1);
      const uint16_t* vb1 = reinterpret_cast<const uint16_t*>(&lds.v[dq][(r0 + 8) * VROWU + (u0 ^ x1)]) + 4 * (sl & 1);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        vt[ks2][mt][0] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                                      (lds_bf16x4*)(vb0 + 32 * mt)));
        vt[ks2][mt][1] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                                      (lds_bf16x4*)(vb1 + 32 * mt)));
      }
    }
    have_pv = true;

    // rare: a head's max moved by more than 2^8 (always on the first tile)
    if (fl.x | fl.y | fl.z | fl.w) {
      const float tmax = fmaxf(fmaxf(lds.qmax[buf][0][e], lds.qmax[buf][1][e]),
                               fmaxf(lds.qmax[buf][2][e], lds.qmax[buf][3][e]));
      const float m_new = tmax > m_run + LAZY_LOG2 ? tmax : m_run;
      if (__any(m_new != m_run)) {
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) oacc[mt] *= alpha;
        l_lane *= alpha;
        m_run = m_new;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sq[r], c_log2, -m_run));
      write_p(buf, pr);
      __syncthreads();
      read_pfr(buf);
    }
    l_lane += (pr[0] + pr[1]) + (pr[2] + pr[3]);

    if (more) {
      write_v(rn);                // after this wave's V^T(t) reads: the LDS keeps their order
      qk_s(rn);
      vmask_cur = tile_mask(t + 1);
      __syncthreads();
    }
  }
  if (have_pv) issue_pv();
}

// One workgroup's share: row `row`, split `split` of p.splits, head group hgi
// (R > 1: the row tile `row`, its columns as in window_tiles)
template <int R = 1>
__device__ __forceinline__ void window_unit(const AttnParams& p, int row, int split, int hgi, WinLds& lds) {
  constexpr int HP = 32 / R;
  const int tid = threadIdx.x;
  const int dq = tid >> 6;
  const int lane = tid & 63;
  const int e = lane & 31;
  const int hh = lane >> 5;
  int row_l = row, nr = 1;
  if (R > 1) {
    const int ngq = (p.Q + R - 1) / R;
    const int b = row / ngq, q0 = (row - b * ngq) * R;
    nr = min(R, p.Q - q0);
    row_l = b * p.Q + q0 + e / HP;
  }
  const int head = HP * hgi + e % HP;
  const bool head_ok = head < p.H && e / HP < nr;
  floatx16 oacc[4];       // O^T: [dims 128dq + 32mt + 8(i/4) + 4hh + i%4][head]
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) oacc[mt] = floatx16{};
  float m_run = M_INIT;   // running max of z * log2(e), per head (lane pair)
  float l_lane = 0.f;     // softmax denominator over this lane's quarter tokens
  window_tiles<R>(p, row, split, hgi, lds, oacc, m_run, l_lane);

  // ---- finalize: denominators across the 4 quarter owners -----------------
  const float lq = pair_sum(l_lane);
  if (lane < 32) lds.lsum[dq][lane] = lq;
  __syncthreads();
  const float l = (lds.lsum[0][e] + lds.lsum[1][e]) + (lds.lsum[2][e] + lds.lsum[3][e]);
  const float il = l > 0.f ? 1.f / l : 0.f;
  const size_t orow = ((size_t)row_l * p.H + head) * p.out_splits + p.split_base + split;
  if (head_ok && dq == 0 && hh == 0) {
    const float lse = l > 0.f ? (m_run + log2f(l)) * 0.69314718055994531f : -__builtin_inff();
    p.lse_out[orow] = lse;
  }
  // fp16 partial relative to a per-head power of two: the head's largest |o|
  // lands in [2^14, 2^15); the 4 waves agree on it through LDS
  float am = 0.f;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(oacc[mt][i]));
  am = pair_max(am * il);
  constexpr int E_NONE = -100000;
  if (lane < 32) lds.emax[dq][lane] = am > 0.f ? ilogbf(am) : E_NONE;
  __syncthreads();
  int k = max(max(lds.emax[0][e], lds.emax[1][e]), max(lds.emax[2][e], lds.emax[3][e]));
  if (k == E_NONE) k = 0;
  if (head_ok) {
    if (dq == 0 && hh == 0) p.oexp_out[orow] = k - 14;
    store_o16_slice(oacc, il, 14 - k, hh, p.o16_out + orow * D + 128 * dq);
  }
}

}  // namespace win
}  // namespace csa2
