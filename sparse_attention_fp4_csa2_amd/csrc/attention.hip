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
//  * wave w owns latent dims [128w, 128w+128): its slice of every head's query
//    (registers), of each tile's keys/values, and of the output accumulator
//    O[64 heads][128 dims] (fp32, MFMA accumulators).
//  * a tile is 32 entries (4 blocks).  Each lane (entry e = lane%32, half
//    hh = lane/32) loads 32 bytes of FP4 codes + 2 scale bytes straight from
//    the block record and dequantises them with the hardware FP4->bf16
//    conversion into the B operand of v_mfma_f32_32x32x16_bf16.
//  * QK^T: each wave forms a partial S[64 heads][32 entries] over its 128 dims;
//    partials meet in LDS, wave w reduces heads {32mt + 8w + 0..7} and runs the
//    online softmax for them (lazy rescaling: the running max only moves when
//    it grows by more than 8 in log2 units).
//  * P goes to LDS; the wave's own V slice goes to LDS entry-major and comes
//    back through ds_read_b64_tr_b16 as the transposed B operand of the P.V
//    MFMA.  Two barriers per tile.
//  * Precision of P.V.  bf16 softmax weights (8 significant bits) cost up to
//    ~1% of the output RMS when one entry dominates, so P.V runs in fp16:
//    MXFP4 source -- V is re-dequantised straight to fp16 with a per-wave
//    power-of-two base (V' = V * 2^(140 - vbase), vbase = the largest scale
//    byte seen by the wave, raised lazily with an exact rescale of O), which
//    keeps every code * scale exact in fp16; P is fp16 (< 2^8 by the lazy
//    softmax).  bf16 window source -- V stays bf16 and P is split into
//    bf16 hi + lo parts (two MFMAs), exact to ~2^-17.  Q.K stays bf16 (exact K).
#include "device.h"
#include "launch.h"

namespace csa2 {

namespace {

constexpr int NWAVE = 4;
constexpr int TILE = 32;              // entries per tile
constexpr int PSTRIDE = 40;           // bf16 per P row (32 + pad)
constexpr int VSTRIDE = 136;          // bf16 per V row (128 + pad)
constexpr float LAZY_LOG2 = 8.0f;     // rescale only when the max grows by > 2^8

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
constexpr int VBIAS = 140;            // fp16 V' = V * 2^(VBIAS - vbase): largest code 6 -> 6*2^13

struct Lds {
  floatx4 sred[NWAVE][2][4][64];      // partial S per wave: [mt][i/4][lane] (float4)
  uint16_t pbuf[64 * PSTRIDE];        // P[head][entry]: fp16 (MXFP4 source) or bf16 hi (window)
  uint16_t pbuf_lo[64 * PSTRIDE];     // window source: bf16 lo part of P
  uint16_t vbuf[NWAVE][TILE * VSTRIDE];  // per-wave V slice, entry-major (fp16 or bf16)
  float alpha[64];
  float inv_l[64];
  int flag[2];
};

__device__ __forceinline__ floatx16 mfma32(uint4 a, uint4 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ floatx16 mfma32_f16(uint4 a, uint4 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a),
                                                __builtin_bit_cast(halfx8, b), c, 0, 0, 0);
}

// 8 MXFP4 codes -> 8 fp16 values times 2^(sb - 127 + shift); scale given as float bits.
__device__ __forceinline__ uint4 dequant8_f16(uint32_t codes, uint32_t scale_bits) {
  const float sc = __uint_as_float(scale_bits);
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, sc, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, sc, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, sc, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, sc, 3));
  return r;
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ __forceinline__ int wave_max_int(int v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = max(v, __shfl_xor(v, m, 64));
  return v;
}

__device__ __forceinline__ float max_half32(float v) {
  // max over the 32 lanes of this lane's half of the wave
#pragma unroll
  for (int m = 1; m < 32; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

__device__ __forceinline__ float sum_half32(float v) {
#pragma unroll
  for (int m = 1; m < 32; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

struct Raw {
  uint4 c0, c1;   // 32 bytes of codes (64 dims)
  uint32_t sc;    // 2 scale bytes (low byte: first 32 dims)
  int valid;
};

}  // namespace

template <int MT, bool FP4>
__global__ __launch_bounds__(256, 1) void attn_kernel(AttnParams p) {
  __shared__ Lds lds;
  const int split = blockIdx.x;
  const int row = blockIdx.y;
  const int hg = blockIdx.z;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int e = lane & 31;        // entry within tile / row within M-tile
  const int hh = lane >> 5;       // lane half
  const int b = row / p.Q;

  // ---- work range -------------------------------------------------------
  int n_items;         // FP4: selected blocks; window: visible slots
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

  // ---- query fragments: heads 32mt + e, dims 128w + 64hh + 8ks ----------
  uint4 qf[MT][8];
  {
    const int dim0 = 128 * w + 64 * hh;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int h = hg * 64 + 32 * mt + e;
      const uint4* src = reinterpret_cast<const uint4*>(p.q + ((size_t)row * p.H + h) * D + dim0);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qf[mt][ks] = (h < p.H) ? src[ks] : make_uint4(0, 0, 0, 0);
    }
  }

  floatx16 oacc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) oacc[mt][nt] = floatx16{};
  float m_run[MT][4], l_lane[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) { m_run[mt][r] = -__builtin_inff(); l_lane[mt][r] = 0.f; }

  if (tid < 2) lds.flag[tid] = 0;
  int vbase = 0;    // MXFP4 source: power-of-two base of this wave's fp16 V slice

  // ---- raw tile loader --------------------------------------------------
  auto load_fp4 = [&](int t) -> Raw {
    Raw r;
    const int item = 4 * t + (e >> 3);
    const int blk = item < n_items ? p.idx[(size_t)row * p.top_k + item] : -1;
    const int j = blk * BLOCK + (e & 7);
    const bool inrange = blk >= 0 && blk < nb_cap;
    r.valid = inrange && j < n_ent && (!p.q_pos || 2 * j + 1 <= t_pos);
    // absent / invisible entries are read as zeros: their softmax weight is 0,
    // and zero values keep stale bytes (even NaN patterns) out of P.V
    if (r.valid) {
      const uint8_t* rec = p.cache + ((size_t)b * nb_cap + blk) * RECORD;
      const uint4* cp = reinterpret_cast<const uint4*>(rec + (e & 7) * 256 + 64 * w + 32 * hh);
      r.c0 = cp[0];
      r.c1 = cp[1];
      r.sc = *reinterpret_cast<const uint16_t*>(rec + SCALE_OFF + (e & 7) * 16 + 4 * w + 2 * hh);
    } else {
      r.c0 = make_uint4(0, 0, 0, 0);
      r.c1 = r.c0;
      r.sc = 0;
    }
    return r;
  };

  Raw nxt;
  if (FP4 && t_begin < t_end) nxt = load_fp4(t_begin);

  for (int t = t_begin; t < t_end; ++t) {
    // ---- K/V fragments for this tile: entry e, dims 128w + 64hh + 8ks ----
    uint4 kf[8];
    uint4 vf[8];     // MXFP4 source: fp16 V' for P.V
    int valid;
    if (FP4) {
      Raw cur = nxt;
      if (t + 1 < t_end) nxt = load_fp4(t + 1);
      valid = cur.valid;
      const uint32_t sa = cur.sc & 0xFFu, sbb = (cur.sc >> 8) & 0xFFu;
      kf[0] = dequant8(cur.c0.x, sa);
      kf[1] = dequant8(cur.c0.y, sa);
      kf[2] = dequant8(cur.c0.z, sa);
      kf[3] = dequant8(cur.c0.w, sa);
      kf[4] = dequant8(cur.c1.x, sbb);
      kf[5] = dequant8(cur.c1.y, sbb);
      kf[6] = dequant8(cur.c1.z, sbb);
      kf[7] = dequant8(cur.c1.w, sbb);
      // raise the wave's V base to the largest valid scale byte (exact O rescale)
      const int tmax = wave_max_int(valid ? (int)max(sa, sbb) : 0);
      if (tmax > vbase) {
        const float f = ldexpf(1.f, vbase - tmax);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) oacc[mt][nt] *= f;
        vbase = tmax;
      }
      const int ea = max((int)sa - vbase + VBIAS, 0), eb = max((int)sbb - vbase + VBIAS, 0);
      const uint32_t fa = (uint32_t)ea << 23, fb = (uint32_t)eb << 23;
      vf[0] = dequant8_f16(cur.c0.x, fa);
      vf[1] = dequant8_f16(cur.c0.y, fa);
      vf[2] = dequant8_f16(cur.c0.z, fa);
      vf[3] = dequant8_f16(cur.c0.w, fa);
      vf[4] = dequant8_f16(cur.c1.x, fb);
      vf[5] = dequant8_f16(cur.c1.y, fb);
      vf[6] = dequant8_f16(cur.c1.z, fb);
      vf[7] = dequant8_f16(cur.c1.w, fb);
    } else {
      const int slot = TILE * t + e;
      valid = slot < n_items;
      const int s = lo + (valid ? slot : 0);
      const uint4* src = reinterpret_cast<const uint4*>(
          p.swa + ((size_t)b * p.Lw + s) * D + 128 * w + 64 * hh);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) kf[ks] = valid ? src[ks] : make_uint4(0, 0, 0, 0);
    }

    // ---- partial S over this wave's 128 dims ----
    floatx16 sacc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      sacc[mt] = floatx16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) sacc[mt] = mfma32(qf[mt][ks], kf[ks], sacc[mt]);
    }
    // own V slice -> LDS, entry-major
    {
      uint4* vrow = reinterpret_cast<uint4*>(&lds.vbuf[w][e * VSTRIDE + 64 * hh]);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) vrow[ks] = FP4 ? vf[ks] : kf[ks];
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        lds.sred[w][mt][j][lane] =
            floatx4{sacc[mt][4 * j], sacc[mt][4 * j + 1], sacc[mt][4 * j + 2], sacc[mt][4 * j + 3]};
    __syncthreads();
    if (tid == 0) lds.flag[(t + 1) & 1] = 0;

    // ---- reduce own heads, online softmax ----
    bool rescaled = false;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      floatx4 s = lds.sred[0][mt][w][lane];
#pragma unroll
      for (int src = 1; src < NWAVE; ++src) s += lds.sred[src][mt][w][lane];
      float x[4], pv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = valid ? s[r] * p.scale_log2 : -__builtin_inff();
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float tmax = max_half32(x[r]);
        float alpha = 1.f;
        if (tmax > m_run[mt][r] + LAZY_LOG2 || (m_run[mt][r] == -__builtin_inff() && tmax != -__builtin_inff())) {
          alpha = (m_run[mt][r] == -__builtin_inff()) ? 0.f : exp2f(m_run[mt][r] - tmax);
          m_run[mt][r] = tmax;
          rescaled = true;
        }
        pv[r] = (m_run[mt][r] == -__builtin_inff()) ? 0.f : exp2f(x[r] - m_run[mt][r]);
        l_lane[mt][r] = l_lane[mt][r] * alpha + pv[r];
        const int hl = 32 * mt + 8 * w + 4 * hh + r;
        if (FP4) {
          lds.pbuf[hl * PSTRIDE + e] = f32_to_f16_bits(pv[r]);
        } else {
          const uint16_t hi = f32_to_bf16_rne(pv[r]);
          lds.pbuf[hl * PSTRIDE + e] = hi;
          lds.pbuf_lo[hl * PSTRIDE + e] = f32_to_bf16_rne(pv[r] - bf16_to_f32(hi));
        }
        if (e == 0) lds.alpha[hl] = alpha;
      }
    }
    if (rescaled) lds.flag[t & 1] = 1;
    __syncthreads();

    // ---- rescale O if any head moved its max ----
    if (lds.flag[t & 1]) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        float a[16];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const floatx4 a4 = *reinterpret_cast<const floatx4*>(&lds.alpha[32 * mt + 8 * jj + 4 * hh]);
          a[4 * jj] = a4[0]; a[4 * jj + 1] = a4[1]; a[4 * jj + 2] = a4[2]; a[4 * jj + 3] = a4[3];
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[mt][nt][i] *= a[i];
      }
    }

    // ---- O += P V ----
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      uint4 pa[MT], pl[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int off = (32 * mt + e) * PSTRIDE + 16 * ks2 + 8 * hh;
        pa[mt] = *reinterpret_cast<const uint4*>(&lds.pbuf[off]);
        if (!FP4) pl[mt] = *reinterpret_cast<const uint4*>(&lds.pbuf_lo[off]);
      }
      const int sl = lane & 15, blk16 = lane >> 4;
      const int krow = 16 * ks2 + 8 * (blk16 >> 1) + (sl >> 2);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int ncol = 32 * nt + 16 * (blk16 & 1) + 4 * (sl & 3);
        const uint16_t* base = &lds.vbuf[w][krow * VSTRIDE + ncol];
        const uint2 v0 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                                     (lds_bf16x4*)(base)));
        const uint2 v1 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                                     (lds_bf16x4*)(base + 4 * VSTRIDE)));
        const uint4 vb = make_uint4(v0.x, v0.y, v1.x, v1.y);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if (FP4) {
            oacc[mt][nt] = mfma32_f16(pa[mt], vb, oacc[mt][nt]);
          } else {
            oacc[mt][nt] = mfma32(pa[mt], vb, oacc[mt][nt]);
            oacc[mt][nt] = mfma32(pl[mt], vb, oacc[mt][nt]);
          }
        }
      }
    }
  }

  // ---- finalize: l per owned head, 1/l to LDS, write o and lse ----------
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float l = sum_half32(l_lane[mt][r]);
      const int hl = 32 * mt + 8 * w + 4 * hh + r;
      if (e == 0) {
        lds.inv_l[hl] = l > 0.f ? 1.f / l : 0.f;
        const int h = hg * 64 + hl;
        if (h < p.H) {
          const float lse = l > 0.f ? (m_run[mt][r] + log2f(l)) * 0.69314718055994531f
                                    : -__builtin_inff();
          p.lse_out[((size_t)row * p.splits + split) * p.H + h] = lse;
        }
      }
    }
  __syncthreads();
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int hl = 32 * mt + 8 * (i >> 2) + 4 * hh + (i & 3);
      const int h = hg * 64 + hl;
      if (h >= p.H) continue;
      const float il = lds.inv_l[hl];
      const int vshift = FP4 ? vbase - VBIAS : 0;
      float* dst = p.o_out + (((size_t)row * p.splits + split) * p.H + h) * D + 128 * w + e;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) dst[32 * nt] = ldexpf(oacc[mt][nt][i] * il, vshift);
    }
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
  return s;
}

int launch_attention(const AttnParams& p, bool fp4_source, hipStream_t stream) {
  const int hgroups = (p.H + 63) / 64;
  dim3 grid(p.splits, p.rows, hgroups);
  const bool one_tile = p.H <= 32;
  if (fp4_source) {
    if (one_tile) attn_kernel<1, true><<<grid, 256, 0, stream>>>(p);
    else attn_kernel<2, true><<<grid, 256, 0, stream>>>(p);
  } else {
    if (one_tile) attn_kernel<1, false><<<grid, 256, 0, stream>>>(p);
    else attn_kernel<2, false><<<grid, 256, 0, stream>>>(p);
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// ---- combine -----------------------------------------------------------
__global__ __launch_bounds__(128) void combine_kernel(const float* __restrict__ o_part,
                                                      const float* __restrict__ lse_part,
                                                      int splits, int H,
                                                      const float* __restrict__ o_ext,
                                                      const float* __restrict__ lse_ext,
                                                      float* __restrict__ out,
                                                      float* __restrict__ lse_out) {
  const int h = blockIdx.x, row = blockIdx.y, t = threadIdx.x;
  const size_t rh = (size_t)row * H + h;
  float m = -__builtin_inff();
  for (int s = 0; s < splits; ++s) m = fmaxf(m, lse_part[((size_t)row * splits + s) * H + h]);
  const float le = o_ext ? lse_ext[rh] : -__builtin_inff();
  m = fmaxf(m, le);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float L = -__builtin_inff();
  if (m != -__builtin_inff()) {
    float sum = 0.f;
    for (int s = 0; s < splits; ++s) sum += expf(lse_part[((size_t)row * splits + s) * H + h] - m);
    if (o_ext) sum += expf(le - m);
    L = m + logf(sum);
    for (int s = 0; s < splits; ++s) {
      const size_t ps = ((size_t)row * splits + s) * H + h;
      const float wgt = expf(lse_part[ps] - L);
      if (wgt == 0.f) continue;
      const float4 v = reinterpret_cast<const float4*>(o_part + ps * D)[t];
      acc.x += wgt * v.x; acc.y += wgt * v.y; acc.z += wgt * v.z; acc.w += wgt * v.w;
    }
    if (o_ext) {
      const float wgt = expf(le - L);
      if (wgt != 0.f) {
        const float4 v = reinterpret_cast<const float4*>(o_ext + rh * D)[t];
        acc.x += wgt * v.x; acc.y += wgt * v.y; acc.z += wgt * v.z; acc.w += wgt * v.w;
      }
    }
  }
  __syncthreads();   // o_ext may alias out: every read above precedes the writes below
  reinterpret_cast<float4*>(out + rh * D)[t] = acc;
  if (t == 0) lse_out[rh] = L;
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
