// Split-K multi-head attention over (a) the selected blocks of the MXFP4 latent
// cache and (b) the bf16 sliding window, plus the log-sum-exp combine.
//
// What is computed: one 512-d latent per entry is the key AND the value for
// every head (paper-digest.app page, Core Mechanics, "Compressed along three
// axes"); only the top-K selected blocks of 8 entries are attended, and each
// layer adds its own sliding-window branch (observer.broadside.tech card, Key
// ideas, "CSA2 with three static layer modes").  z = scale * q_h . V_j,
// o = softmax(z) V, lse = log sum exp z; branches and splits are merged by
// log-sum-exp.
//
// Kernel organisation (one workgroup = 4 waves = one (row, split, 64-head group)):
//  * wave w = (hg, dh): heads [32hg, 32hg+32) of the group and latent dims
//    [256dh, 256dh+256).  It keeps its heads' queries for its dims in
//    registers and the output slice O^T[256 dims][32 heads] in fp32 MFMA
//    accumulators.
//  * a tile is 32 entries (4 blocks).  Lane (e = lane%32, hh = lane/32) loads
//    64 bytes of codes + 4 scale bytes of entry e straight from the block
//    record and dequantises them once, with the hardware FP4 conversion, into
//    the A operand of v_mfma_f32_32x32x16: S^T[entries][heads] = K.Q^T over the
//    wave's 256 dims.  The two waves sharing a head half add their partials
//    through LDS, so every lane then holds one head's 16 logits of the tile in
//    registers: the row max is in-register plus one exchange with lane^32.
//  * those registers are already the B operand of O^T += V^T.P^T; V^T comes
//    from the tile written to LDS entry-major and read back with
//    ds_read_b64_tr_b16.  LDS is double-buffered: one barrier per tile.
//  * online softmax per head with lazy rescaling (the running max moves only
//    when it grows by more than 8 in log2 units).
//  * precision: MXFP4 source -- K and V are dequantised to fp16 with a
//    per-wave power-of-two base (V' = V * 2^(140 - vbase), vbase = the largest
//    scale byte the wave has seen, raised with an exact rescale of O), which
//    keeps every code * scale exact in fp16; queries are scaled into fp16 by a
//    per-head power of two; P is fp16 (fp16's 11 significant bits keep the P.V
//    error near 1e-3 of the output RMS, where bf16 P reached ~1e-2).  bf16
//    window source -- bf16 K/V/Q, and P split into bf16 hi + lo parts (two
//    MFMAs).
#include "device.h"
#include "launch.h"

namespace csa2 {

namespace {

constexpr int TILE = 32;              // entries per tile
constexpr int VROW = 288;             // 16-bit elements per V row (256 + 32 pad)
// 16-byte unit u of V row r is stored at unit u ^ ((r >> 2) & 3): with the
// 288-element stride both the entry-major row writes and the transposed reads
// are free of LDS bank conflicts.
constexpr int MAX_SPLIT_BLOCKS = 2048; // selected blocks one workgroup stages in LDS
constexpr float LAZY_LOG2 = 8.0f;     // rescale only when the max grows by > 2^8
constexpr int VBIAS = 140;            // V' = V * 2^(VBIAS - vbase): code 6 at vbase -> 6*2^13

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));

struct Lds {
  uint16_t vbuf[2][2][TILE * VROW];   // [buffer][dh][entry][dim]  (fp16 or bf16)
  floatx4 sred[2][4][4][64];          // [buffer][wave][i/4][lane]: partial S^T
  int32_t blk[MAX_SPLIT_BLOCKS];      // this split's selected block ids
};

__device__ __forceinline__ floatx16 mfma_bf16(uint4 a, uint4 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ floatx16 mfma_f16(uint4 a, uint4 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a),
                                                __builtin_bit_cast(halfx8, b), c, 0, 0, 0);
}

// 8 MXFP4 codes -> 8 fp16 values, scaled by the float whose bits are scale_bits.
__device__ __forceinline__ uint4 dequant8_f16(uint32_t codes, uint32_t scale_bits) {
  const float sc = __uint_as_float(scale_bits);
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, sc, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, sc, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, sc, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, sc, 3));
  return r;
}

__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}

__device__ __forceinline__ uint32_t pack_bf16(uint16_t a, uint16_t b) {
  return (uint32_t)a | ((uint32_t)b << 16);
}

__device__ __forceinline__ int floor_log2_mag(uint32_t mag) {   // bf16 magnitude bits, > 0
  const uint32_t ef = mag >> 7;
  return ef ? (int)ef - 127 : (31 - __builtin_clz(mag)) - 133;
}

__device__ __forceinline__ int wave_max_int(int v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = max(v, __shfl_xor(v, m, 64));
  return v;
}

struct Raw {
  uint4 c[4];     // 64 bytes of codes (128 dims)
  uint32_t sc;    // 4 scale bytes (one per 32 dims)
  int valid;
};

}  // namespace

// Pair (lane l, lane l^32) reductions on gfx950 without an LDS round trip:
// v_permlane32_swap returns {value of lane l%32, value of lane l%32 + 32}.
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <bool FP4>
__global__ __launch_bounds__(256, 1) void attn_kernel(AttnParams p) {
  __shared__ Lds lds;
  const int split = blockIdx.x;
  const int row = blockIdx.y;
  const int HG = blockIdx.z;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int e = lane & 31;        // entry of the tile (A rows) / head of the wave (B cols)
  const int hh = lane >> 5;       // lane half: which 8 of each 16 contraction slots
  const int hg = w & 1;           // head half of the 64-head group
  const int dh = w >> 1;          // latent half
  const int b = row / p.Q;
  const int head = HG * 64 + 32 * hg + e;
  const bool head_ok = head < p.H;

  // ---- work range -------------------------------------------------------
  int n_items;         // MXFP4: selected blocks; window: visible slots
  int lo = 0;          // window: first visible slot
  int t_pos = 0;
  if (FP4) {
    n_items = p.count[row];
    n_items = n_items < 0 ? 0 : (n_items > p.top_k ? p.top_k : n_items);
    if (p.q_pos) t_pos = p.q_pos[row];
  } else {
    const int len = min(p.swa_len[b], p.Lw);
    const int pos0 = p.swa_pos0 ? p.swa_pos0[b] : 0;
    const int t = p.q_pos ? p.q_pos[row] : pos0 + len - 1;
    const int a = max(t - p.W + 1, pos0), z = min(t, pos0 + len - 1);
    lo = a - pos0;
    n_items = z >= a ? z - a + 1 : 0;
  }
  const int per_tile = FP4 ? 4 : TILE;
  const int n_tiles = (n_items + per_tile - 1) / per_tile;
  const int tps = (n_tiles + p.splits - 1) / p.splits;
  const int t_begin = split * tps;
  const int t_end = min(n_tiles, t_begin + tps);
  const int n_ent = FP4 ? p.n_entries[b] : 0;
  const int nb_cap = p.cap / BLOCK;
  const int dim0 = 256 * dh + 128 * hh;     // this lane's 128 contraction dims

  // Contraction order: register k-step ks holds dims dim0 + 8 * ((ks + 8hg) % 16).
  // The rotation by hg makes each head-half wave's first 8 k-steps the 64 dims
  // it stores for the shared V tile, so register indices stay static.
  // ---- queries: B operand (column = head) ----
  uint4 qf[16];
  int cq = 0;                                // MXFP4: q' = q * 2^cq in fp16
  {
    const uint4* src = reinterpret_cast<const uint4*>(p.q + ((size_t)row * p.H + head) * D + dim0);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qf[ks] = head_ok ? src[(ks + 8 * hg) & 15] : make_uint4(0, 0, 0, 0);
    if (FP4) {
      uint32_t mx = 0;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const uint32_t wv[4] = {qf[ks].x, qf[ks].y, qf[ks].z, qf[ks].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) mx = max(mx, max(wv[k] & 0x7FFFu, (wv[k] >> 16) & 0x7FFFu));
      }
      mx = (uint32_t)pair_max(__uint_as_float(mx));     // non-negative ints order like floats
      if (mx != 0 && mx < 0x7F80u) cq = 13 - floor_log2_mag(mx);
      const float f = ldexpf(1.f, cq);
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const uint32_t wv[4] = {qf[ks].x, qf[ks].y, qf[ks].z, qf[ks].w};
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          o[k] = pack_f16(__uint_as_float(wv[k] << 16) * f, __uint_as_float(wv[k] & 0xFFFF0000u) * f);
        qf[ks] = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
  }

  // stage the split's block ids in LDS once: no dependent global load per tile
  if (FP4) {
    const int i0 = 4 * t_begin, i1 = min(4 * t_end, n_items);
    for (int i = i0 + tid; i < i1; i += 256) lds.blk[i - i0] = p.idx[(size_t)row * p.top_k + i];
  }
  __syncthreads();

  floatx16 oacc[8];       // O^T: [dims 32mt + 8(i/4) + 4hh + i%4][head]
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) oacc[mt] = floatx16{};
  float m_run = -__builtin_inff();
  float l_lane = 0.f;
  int vbase = 0;          // MXFP4: power-of-two base of O and of the tile being accumulated
  int vbase_next = 0;     // base the next tile is dequantised with (>= vbase)
  const float c_log2 = p.scale_log2;

  // Raw tile fetch, branch-free: absent/invisible entries read block 0 of the
  // sequence and are zeroed (zero values keep stale bytes out of P.V; their
  // logits are masked).  Window source: the bf16 rows themselves.
  auto fetch = [&](int t, Raw& r) {
    if (FP4) {
      const int item = 4 * t + (e >> 3);
      const bool have = t < t_end && item < n_items;
      const int blk = have ? lds.blk[item - 4 * t_begin] : 0;
      const int j = blk * BLOCK + (e & 7);
      r.valid = have && blk >= 0 && blk < nb_cap && j < n_ent && (!p.q_pos || 2 * j + 1 <= t_pos);
      const int sb = r.valid ? blk : 0;
      const uint8_t* rec = p.cache + ((size_t)b * nb_cap + sb) * RECORD;
      const uint4* cp = reinterpret_cast<const uint4*>(rec + (e & 7) * 256 + 128 * dh + 64 * hh);
      r.c[0] = cp[(0 + 2 * hg) & 3]; r.c[1] = cp[(1 + 2 * hg) & 3];
      r.c[2] = cp[(2 + 2 * hg) & 3]; r.c[3] = cp[(3 + 2 * hg) & 3];
      const uint32_t sc = *reinterpret_cast<const uint32_t*>(rec + SCALE_OFF + (e & 7) * 16 + 8 * dh + 4 * hh);
      r.sc = hg ? ((sc >> 16) | (sc << 16)) : sc;      // scale byte g <-> 32-dim group (g + 2hg) % 4
    } else {
      const int slot = TILE * t + e;
      r.valid = t < t_end && slot < n_items;
      r.sc = 0;
    }
  };
  auto zero_invalid = [&](Raw& r) {
    if (FP4) {
      const uint32_t m = r.valid ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int g = 0; g < 4; ++g) { r.c[g].x &= m; r.c[g].y &= m; r.c[g].z &= m; r.c[g].w &= m; }
      r.sc &= m;
    }
  };
  // K (= V) fragments of a tile: entry e, dims dim0 + 8ks.
  auto kfrags = [&](int t, const Raw& r, int base, uint4 (&kf)[16]) {
    if (FP4) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int sbv = (int)((r.sc >> (8 * g)) & 0xFF);
        const uint32_t bits = (uint32_t)max(sbv - base + VBIAS, 0) << 23;
        const uint4 cw = r.c[g];
        kf[4 * g + 0] = dequant8_f16(cw.x, bits);
        kf[4 * g + 1] = dequant8_f16(cw.y, bits);
        kf[4 * g + 2] = dequant8_f16(cw.z, bits);
        kf[4 * g + 3] = dequant8_f16(cw.w, bits);
      }
    } else {
      const int slot = r.valid ? TILE * t + e : 0;
      const uint4* src = reinterpret_cast<const uint4*>(
          p.swa + ((size_t)b * p.Lw + lo + slot) * D + dim0);
      const uint32_t m = r.valid ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const uint4 v = src[(ks + 8 * hg) & 15];
        kf[ks] = make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
      }
    }
  };
  // S^T partial over this wave's dims, at true scale (times c_log2), and this
  // wave's half of the tile's V rows (dims 128hh + 64hg + [0,64)) into LDS.
  auto qk_and_store = [&](const uint4 (&kf)[16], int base, int sbuf, floatx16& sacc) {
    sacc = floatx16{};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
      sacc = FP4 ? mfma_f16(kf[ks], qf[ks], sacc) : mfma_bf16(kf[ks], qf[ks], sacc);
    const float f = FP4 ? ldexpf(c_log2, base - VBIAS - cq) : c_log2;
    sacc *= f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      lds.sred[sbuf][w][j][lane] = floatx4{sacc[4 * j], sacc[4 * j + 1], sacc[4 * j + 2], sacc[4 * j + 3]};
    // kf[0..7] hold dims 128hh + 64hg + [0,64) (contraction order rotated by hg)
    uint16_t* vrow = &lds.vbuf[sbuf][dh][e * VROW + 128 * hh + 64 * hg];
    const int xw = (e >> 2) & 3;
#pragma unroll
    for (int k = 0; k < 8; ++k) *reinterpret_cast<uint4*>(vrow + 8 * (k ^ xw)) = kf[k];
  };
  auto raise_base = [&](const Raw& r, int cur) -> int {   // largest valid scale byte of the wave
    int smax = 0;
    if (r.valid) smax = max(max((int)(r.sc & 0xFF), (int)((r.sc >> 8) & 0xFF)),
                            max((int)((r.sc >> 16) & 0xFF), (int)(r.sc >> 24)));
    if (__any(smax > cur)) return max(cur, wave_max_int(smax));
    return cur;
  };

  // ---- prologue: tile t_begin through Q.K, tile t_begin+1 fetched ----------
  floatx16 scur = floatx16{};
  uint32_t vmask = 0;
  Raw rn;
  if (t_begin < t_end) {
    Raw r0;
    fetch(t_begin, r0);
    fetch(t_begin + 1, rn);
    zero_invalid(r0);
    if (FP4) { vbase = raise_base(r0, vbase); vbase_next = vbase; }
    uint4 kf[16];
    kfrags(t_begin, r0, vbase, kf);
    qk_and_store(kf, vbase, t_begin & 1, scur);
    vmask = (uint32_t)__ballot(r0.valid);
  }
  __syncthreads();

  for (int t = t_begin; t < t_end; ++t) {
    const int buf = t & 1;
    // ---- head of iteration: logits of tile t, rare rescales ----------------
    if (FP4 && vbase_next != vbase) {          // tile t was dequantised with a higher base
      const float f = ldexpf(1.f, vbase - vbase_next);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) oacc[mt] *= f;
      vbase = vbase_next;
    }
    float x[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const floatx4 o4 = lds.sred[buf][w ^ 2][j][lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) x[4 * j + r] = scur[4 * j + r] + o4[r];
    }
    if (vmask != 0xFFFFFFFFu) {
      const uint32_t mh = vmask >> (4 * hh);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (!((mh >> (8 * (i >> 2) + (i & 3))) & 1u)) x[i] = -__builtin_inff();
    }
    float tmax = x[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) tmax = fmaxf(tmax, x[i]);
    tmax = pair_max(tmax);
    const bool bump = tmax > m_run + LAZY_LOG2;
    if (__any(bump)) {
      const float alpha = bump ? (m_run == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m_run - tmax)) : 1.f;
      if (bump) m_run = tmax;
      l_lane *= alpha;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) oacc[mt] *= alpha;
    }
    const bool has_next = t + 1 < t_end;
    Raw rc = rn;
    zero_invalid(rc);
    if (FP4 && has_next) vbase_next = raise_base(rc, vbase);

    // ---- main block: P(t).V(t) interleaved with fetch(t+2), dequant + Q.K(t+1)
    fetch(t + 2, rn);
    const bool live = m_run != -__builtin_inff();
    float pr[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      pr[i] = live ? __builtin_amdgcn_exp2f(x[i] - m_run) : 0.f;
      l_lane += pr[i];
    }
    uint4 pb[2], pl[2];
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      if (FP4) {
        pb[ks2] = make_uint4(pack_f16(pr[8 * ks2 + 0], pr[8 * ks2 + 1]), pack_f16(pr[8 * ks2 + 2], pr[8 * ks2 + 3]),
                             pack_f16(pr[8 * ks2 + 4], pr[8 * ks2 + 5]), pack_f16(pr[8 * ks2 + 6], pr[8 * ks2 + 7]));
      } else {
        uint16_t hi[8], lw[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          hi[j] = f32_to_bf16_rne(pr[8 * ks2 + j]);
          lw[j] = f32_to_bf16_rne(pr[8 * ks2 + j] - bf16_to_f32(hi[j]));
        }
        pb[ks2] = make_uint4(pack_bf16(hi[0], hi[1]), pack_bf16(hi[2], hi[3]), pack_bf16(hi[4], hi[5]), pack_bf16(hi[6], hi[7]));
        pl[ks2] = make_uint4(pack_bf16(lw[0], lw[1]), pack_bf16(lw[2], lw[3]), pack_bf16(lw[4], lw[5]), pack_bf16(lw[6], lw[7]));
      }
    }
    // V^T(t) fragments for the P.V MFMAs, read early so their latency hides
    // under the next tile's dequant and Q.K work
    uint2 vr[2][8][2];
    {
      const int sl = lane & 15, blk16 = lane >> 4;
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        const int r0 = 16 * ks2 + 4 * (blk16 >> 1) + (sl >> 2);
        const int u0 = 2 * (blk16 & 1) + ((sl & 3) >> 1);            // unit within each 4-unit group
        const int x0 = (blk16 >> 1) & 3, x1 = ((blk16 >> 1) + 2) & 3;  // swizzle of rows r0, r0 + 8
        const uint16_t* vb0 = &lds.vbuf[buf][dh][r0 * VROW + 8 * (u0 ^ x0) + 4 * (sl & 1)];
        const uint16_t* vb1 = &lds.vbuf[buf][dh][(r0 + 8) * VROW + 8 * (u0 ^ x1) + 4 * (sl & 1)];
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
          vr[ks2][mt][0] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                                        (lds_bf16x4*)(vb0 + 32 * mt)));
          vr[ks2][mt][1] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                                        (lds_bf16x4*)(vb1 + 32 * mt)));
        }
      }
    }
    // next tile's K/V and Q.K (its buffer was last read before the previous barrier)
    floatx16 snext;
    {
      uint4 kf[16];
      kfrags(t + 1, rc, vbase_next, kf);
      qk_and_store(kf, vbase_next, buf ^ 1, snext);
    }
    // O^T += V^T(t) . P^T(t): A = V^T (transposed LDS reads above), B = this lane's P
    {
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
          const uint4 va = make_uint4(vr[ks2][mt][0].x, vr[ks2][mt][0].y, vr[ks2][mt][1].x, vr[ks2][mt][1].y);
          if (FP4) {
            oacc[mt] = mfma_f16(va, pb[ks2], oacc[mt]);
          } else {
            oacc[mt] = mfma_bf16(va, pb[ks2], oacc[mt]);
            oacc[mt] = mfma_bf16(va, pl[ks2], oacc[mt]);
          }
        }
      }
    }
    vmask = (uint32_t)__ballot(rc.valid);
    scur = snext;
    // Interleave the block: prefetch loads and the first transposed reads go
    // out first; the dequant and softmax VALU work fills the shadows of the
    // Q.K(t+1) MFMAs; the P.V(t) MFMAs each get the next transposed reads.
    __builtin_amdgcn_sched_group_barrier(0x100, 33, 0);    // DS reads (V^T(t), block ids)
    __builtin_amdgcn_sched_group_barrier(0x020, 5, 0);     // VMEM reads (tile t+2)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // VALU
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA  (Q.K t+1)
    }
    __builtin_amdgcn_sched_group_barrier(0x200, 12, 0);    // DS writes
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, FP4 ? 1 : 2, 0);  // MFMA (P.V t)
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);   // VALU
    }
    __syncthreads();
  }

  // ---- finalize ----------------------------------------------------------
  const float l = pair_sum(l_lane);
  const float il = l > 0.f ? 1.f / l : 0.f;
  if (head_ok) {
    if (dh == 0 && hh == 0) {
      const float lse = l > 0.f ? (m_run + log2f(l)) * 0.69314718055994531f : -__builtin_inff();
      p.lse_out[((size_t)row * p.out_splits + p.split_base + split) * p.H + head] = lse;
    }
    const float f = FP4 ? ldexpf(il, vbase - VBIAS) : il;
    float* dst = p.o_out + (((size_t)row * p.out_splits + p.split_base + split) * p.H + head) * D + 256 * dh + 4 * hh;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        *reinterpret_cast<float4*>(dst + 32 * mt + 8 * jj) =
            make_float4(oacc[mt][4 * jj] * f, oacc[mt][4 * jj + 1] * f, oacc[mt][4 * jj + 2] * f,
                        oacc[mt][4 * jj + 3] * f);
  }
}

int attn_splits(int rows, int H, int n_tiles) {
  const int hgroups = (H + 63) / 64;
  const int wgs = rows * hgroups;
  int s = (256 + wgs - 1) / wgs;
  const int cap_by_tiles = n_tiles / 2 > 1 ? n_tiles / 2 : 1;
  if (s > cap_by_tiles) s = cap_by_tiles;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  // a split stages at most MAX_SPLIT_BLOCKS block ids (4 per tile) in LDS
  const int min_s = (n_tiles + MAX_SPLIT_BLOCKS / 4 - 1) / (MAX_SPLIT_BLOCKS / 4);
  if (s < min_s) s = min_s;
  return s;
}

int window_splits(int rows, int H, int n_tiles) {
  const int hgroups = (H + 63) / 64;
  const int wgs = rows * hgroups;
  int s = (128 + wgs - 1) / wgs;
  const int cap_by_tiles = n_tiles / 4 > 1 ? n_tiles / 4 : 1;
  if (s > cap_by_tiles) s = cap_by_tiles;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  return s;
}

int launch_attention(const AttnParams& p, bool fp4_source, hipStream_t stream) {
  const int hgroups = (p.H + 63) / 64;
  dim3 grid(p.splits, p.rows, hgroups);
  if (fp4_source) attn_kernel<true><<<grid, 256, 0, stream>>>(p);
  else attn_kernel<false><<<grid, 256, 0, stream>>>(p);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// ---- combine -----------------------------------------------------------
// Log-sum-exp merge of the split-K partials (and an optional extra branch) of
// one (row, head): wave 0 turns the partials' lse into weights in LDS, then
// every thread streams its float4 of the 512 dims over all splits.
constexpr int MAX_COMBINE_SPLITS = 128;

__global__ __launch_bounds__(128) void combine_kernel(const float* __restrict__ o_part,
                                                      const float* __restrict__ lse_part,
                                                      int splits, int H,
                                                      const float* __restrict__ o_ext,
                                                      const float* __restrict__ lse_ext,
                                                      float* __restrict__ out,
                                                      float* __restrict__ lse_out) {
  __shared__ float wts[MAX_COMBINE_SPLITS + 1];
  __shared__ float L_sh;
  const int h = blockIdx.x, row = blockIdx.y, t = threadIdx.x;
  const size_t rh = (size_t)row * H + h;
  const float* lp = lse_part + (size_t)row * splits * H + h;     // split s at lp[s * H]
  if (t < 64) {
    const float le = (o_ext && t == 0) ? lse_ext[rh] : -__builtin_inff();
    float m = le;
    for (int s = t; s < splits; s += 64) m = fmaxf(m, lp[(size_t)s * H]);
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) m = fmaxf(m, __shfl_xor(m, k, 64));
    float sum = 0.f;
    if (m != -__builtin_inff()) {
      for (int s = t; s < splits; s += 64) sum += expf(lp[(size_t)s * H] - m);
      if (t == 0 && o_ext) sum += expf(le - m);
    }
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) sum += __shfl_xor(sum, k, 64);
    const float L = m == -__builtin_inff() ? -__builtin_inff() : m + logf(sum);
    for (int s = t; s < splits; s += 64)
      wts[s] = L == -__builtin_inff() ? 0.f : expf(lp[(size_t)s * H] - L);
    if (t == 0) {
      wts[splits] = (o_ext && L != -__builtin_inff()) ? expf(le - L) : 0.f;
      L_sh = L;
    }
  }
  __syncthreads();
  const float4* src = reinterpret_cast<const float4*>(o_part + ((size_t)row * splits * H + h) * D) + t;
  const size_t stride4 = (size_t)H * D / 4;                      // one split, in float4
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  int s = 0;
  for (; s + 4 <= splits; s += 4) {
    const float4 v0 = src[(s + 0) * stride4], v1 = src[(s + 1) * stride4];
    const float4 v2 = src[(s + 2) * stride4], v3 = src[(s + 3) * stride4];
    const float w0 = wts[s], w1 = wts[s + 1], w2 = wts[s + 2], w3 = wts[s + 3];
    acc.x += w0 * v0.x + w1 * v1.x + w2 * v2.x + w3 * v3.x;
    acc.y += w0 * v0.y + w1 * v1.y + w2 * v2.y + w3 * v3.y;
    acc.z += w0 * v0.z + w1 * v1.z + w2 * v2.z + w3 * v3.z;
    acc.w += w0 * v0.w + w1 * v1.w + w2 * v2.w + w3 * v3.w;
  }
  for (; s < splits; ++s) {
    const float4 v = src[s * stride4];
    const float wv = wts[s];
    acc.x += wv * v.x; acc.y += wv * v.y; acc.z += wv * v.z; acc.w += wv * v.w;
  }
  if (o_ext) {
    const float we = wts[splits];
    if (we != 0.f) {
      const float4 v = reinterpret_cast<const float4*>(o_ext + rh * D)[t];
      acc.x += we * v.x; acc.y += we * v.y; acc.z += we * v.z; acc.w += we * v.w;
    }
  }
  __syncthreads();   // o_ext may alias out: every read above precedes the writes below
  reinterpret_cast<float4*>(out + rh * D)[t] = acc;
  if (t == 0) lse_out[rh] = L_sh;
}

int launch_combine(const float* o_part, const float* lse_part, int rows, int splits, int H,
                   const float* o_ext, const float* lse_ext, float* out, float* lse_out,
                   hipStream_t stream) {
  dim3 grid(H, rows);
  combine_kernel<<<grid, 128, 0, stream>>>(o_part, lse_part, splits, H, o_ext, lse_ext, out,
                                           lse_out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace csa2
