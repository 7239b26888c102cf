// Sliding-window attention over the bf16 window, and the log-sum-exp combine
// of split-K partials.
//
// What is computed: each layer attends its own window of recent uncompressed
// entries besides the selected compressed blocks (observer.broadside.tech
// card, Key ideas, "CSA2 with three static layer modes"), and one 512-d
// latent is the key and the value for every head (paper-digest.app page, Core
// Mechanics, "Compressed along three axes").  z = scale * q_h . V_j,
// o = softmax(z) V, lse = log sum exp z; splits and branches are merged by
// log-sum-exp.
//
// Window kernel (one workgroup = 4 waves = one (row, split, 64-head group)):
//  * wave w = (hg, dh): heads [32hg, 32hg+32) of the group and latent dims
//    [256dh, 256dh+256).  It keeps its heads' queries for its dims in
//    registers and the output slice O^T[256 dims][32 heads] in fp32 MFMA
//    accumulators.
//  * a tile is 32 entries.  Lane (e = lane%32, hh = lane/32) holds 128 dims of
//    entry e as the A operand of v_mfma_f32_32x32x16_bf16 for
//    S^T[entries][heads] = K.Q^T over the wave's 256 dims; the two waves of a
//    head half add their partials through LDS, so every lane then holds one
//    head's 16 logits of the tile in registers.  Tiles are loaded into
//    registers two ahead: tile t+2 is in flight during all of tile t's work.
//  * V^T for O^T += V^T.P^T is the same tile written to LDS entry-major and
//    read back with ds_read_b64_tr_b16; LDS is double-buffered, one barrier
//    per tile.
//  * online softmax per head with lazy rescaling (the running max moves only
//    when it grows by more than 8 in log2 units); P is split into bf16 hi + lo
//    parts (two MFMAs), as bf16 P alone leaves errors near 1e-2 of the output
//    RMS.
#include "device.h"
#include "launch.h"

namespace csa2 {

namespace {

constexpr int TILE = 32;              // entries per tile
constexpr int VROW = 288;             // 16-bit elements per V row (256 + 32 pad)
// 16-byte unit u of V row r is stored at unit u ^ ((r >> 2) & 3): with the
// 288-element stride both the entry-major row writes and the transposed reads
// are free of LDS bank conflicts.
constexpr float LAZY_LOG2 = 8.0f;     // rescale only when the max grows by > 2^8
constexpr int WINDOW_TARGET_WGS = 128;   // workgroups the split count aims for
constexpr int WINDOW_MIN_TILES = 4;      // tiles per split, at least

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

struct Lds {
  uint16_t vbuf[2][2][TILE * VROW];   // [buffer][dh][entry][dim]  (bf16)
  floatx4 sred[2][4][4][64];          // [buffer][wave][i/4][lane]: partial S^T
};

__device__ __forceinline__ floatx16 mfma_bf16(uint4 a, uint4 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

typedef float floatx2 __attribute__((ext_vector_type(2)));

// (a, b) -> bf16 hi parts (v_cvt_pk_bf16_f32, round to nearest even) and the
// bf16 of the remainders, so that hi + lo carries 16 significant bits.
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{a, b}, bf16x2));
  const float ha = __uint_as_float(hi << 16), hb = __uint_as_float(hi & 0xFFFF0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{a - ha, b - hb}, bf16x2));
}

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

__global__ __launch_bounds__(256, 1) void window_kernel(AttnParams p) {
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

  // ---- visible window slots [lo, lo + n_items) of this row ------------------
  const int len = min(p.swa_len[b], p.Lw);
  const int pos0 = p.swa_pos0 ? p.swa_pos0[b] : 0;
  const int tq = p.q_pos ? p.q_pos[row] : pos0 + len - 1;
  const int a = max(tq - p.W + 1, pos0), z = min(tq, pos0 + len - 1);
  const int lo = a - pos0;
  const int n_items = z >= a ? z - a + 1 : 0;
  const int n_tiles = (n_items + TILE - 1) / TILE;
  const int tps = (n_tiles + p.splits - 1) / p.splits;
  const int t_begin = split * tps;
  const int t_end = min(n_tiles, t_begin + tps);
  const int dim0 = 256 * dh + 128 * hh;     // this lane's 128 contraction dims

  // Contraction order: register k-step ks holds dims dim0 + 8 * ((ks + 8hg) % 16).
  // The rotation by hg makes each head-half wave's first 8 k-steps the 64 dims
  // it stores for the shared V tile, so register indices stay static.
  uint4 qf[16];
  {
    const uint4* src = reinterpret_cast<const uint4*>(p.q + ((size_t)row * p.H + head) * D + dim0);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qf[ks] = head_ok ? src[(ks + 8 * hg) & 15] : make_uint4(0, 0, 0, 0);
  }

  floatx16 oacc[8];       // O^T: [dims 32mt + 8(i/4) + 4hh + i%4][head]
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) oacc[mt] = floatx16{};
  float m_run = -__builtin_inff();
  float l_lane = 0.f;
  const float c_log2 = p.scale_log2;

  // Entry e of tile t, this lane's dims.  Slots past the split or the window
  // read the row's first visible slot (always in bounds when the split has
  // tiles); their logits are masked and their P is 0.
  auto load_tile = [&](int t, uint4 (&kr)[16]) -> bool {
    const int slot = TILE * t + e;
    const bool valid = t < t_end && slot < n_items;
    const uint4* src = reinterpret_cast<const uint4*>(
        p.swa + ((size_t)b * p.Lw + lo + (valid ? slot : 0)) * D + dim0);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) kr[ks] = src[(ks + 8 * hg) & 15];
    return valid;
  };
  // S^T partial over this wave's dims (times c_log2) into LDS, and this wave's
  // half of the tile's V rows (dims 128hh + 64hg + [0,64)) into LDS.
  auto qk_and_store = [&](const uint4 (&kf)[16], int sbuf, floatx16& sacc) {
    sacc = floatx16{};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) sacc = mfma_bf16(kf[ks], qf[ks], sacc);
    sacc *= c_log2;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      lds.sred[sbuf][w][j][lane] = floatx4{sacc[4 * j], sacc[4 * j + 1], sacc[4 * j + 2], sacc[4 * j + 3]};
    uint16_t* vrow = &lds.vbuf[sbuf][dh][e * VROW + 128 * hh + 64 * hg];
    const int xw = (e >> 2) & 3;
#pragma unroll
    for (int k = 0; k < 8; ++k) *reinterpret_cast<uint4*>(vrow + 8 * (k ^ xw)) = kf[k];
  };

  // ---- prologue: tile t_begin through Q.K, tile t_begin+1 loaded -----------
  floatx16 scur = floatx16{};
  uint32_t vmask = 0;
  uint4 ka[16], kb[16];   // register tiles, alternating: one feeds Q.K, one loads
  bool va = false, vb = false;
  if (t_begin < t_end) {
    uint4 k0[16];
    const bool v0 = load_tile(t_begin, k0);
    va = load_tile(t_begin + 1, ka);
    qk_and_store(k0, t_begin & 1, scur);
    vmask = (uint32_t)__ballot(v0);
  }
  __syncthreads();

  // One tile: kq holds tile t+1 (loaded during the previous tile), kl receives
  // tile t+2.
  auto tile_step = [&](int t, uint4 (&kq)[16], bool& vq, uint4 (&kl)[16], bool& vl) {
    const int buf = t & 1;
    // tile t+2 loads go out first; nothing below waits for them
    vl = load_tile(t + 2, kl);
    __builtin_amdgcn_sched_barrier(0);
    // ---- logits of tile t, rare rescales -----------------------------------
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

    // ---- P(t); V^T(t) reads; Q.K(t+1); P.V(t) --------------------------------
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
      const float* q8 = pr + 8 * ks2;
      split_bf16x2(q8[0], q8[1], pb[ks2].x, pl[ks2].x);
      split_bf16x2(q8[2], q8[3], pb[ks2].y, pl[ks2].y);
      split_bf16x2(q8[4], q8[5], pb[ks2].z, pl[ks2].z);
      split_bf16x2(q8[6], q8[7], pb[ks2].w, pl[ks2].w);
    }
    // V^T(t) fragments for the P.V MFMAs, read early so their latency hides
    // under the next tile's Q.K work
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
    // next tile's Q.K (its buffer was last read before the previous barrier)
    floatx16 snext;
    qk_and_store(kq, buf ^ 1, snext);
    // O^T += V^T(t) . P^T(t): A = V^T (transposed LDS reads above), B = this lane's P
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const uint4 v4 = make_uint4(vr[ks2][mt][0].x, vr[ks2][mt][0].y, vr[ks2][mt][1].x, vr[ks2][mt][1].y);
        oacc[mt] = mfma_bf16(v4, pb[ks2], oacc[mt]);
        oacc[mt] = mfma_bf16(v4, pl[ks2], oacc[mt]);
      }
    }
    vmask = (uint32_t)__ballot(vq);
    scur = snext;
    __syncthreads();
  };

  for (int t = t_begin; t < t_end; t += 2) {
    tile_step(t, ka, va, kb, vb);
    if (t + 1 < t_end) tile_step(t + 1, kb, vb, ka, va);
  }

  // ---- finalize ----------------------------------------------------------
  const float l = pair_sum(l_lane);
  const float il = l > 0.f ? 1.f / l : 0.f;
  if (head_ok) {
    if (dh == 0 && hh == 0) {
      const float lse = l > 0.f ? (m_run + log2f(l)) * 0.69314718055994531f : -__builtin_inff();
      p.lse_out[((size_t)row * p.out_splits + p.split_base + split) * p.H + head] = lse;
    }
    float* dst = p.o_out + (((size_t)row * p.out_splits + p.split_base + split) * p.H + head) * D + 256 * dh + 4 * hh;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        *reinterpret_cast<float4*>(dst + 32 * mt + 8 * jj) =
            make_float4(oacc[mt][4 * jj] * il, oacc[mt][4 * jj + 1] * il, oacc[mt][4 * jj + 2] * il,
                        oacc[mt][4 * jj + 3] * il);
  }
}

int window_splits(int rows, int H, int n_tiles) {
  const int hgroups = (H + 63) / 64;
  const int wgs = rows * hgroups;
  int s = (WINDOW_TARGET_WGS + wgs - 1) / wgs;
  const int cap_by_tiles = n_tiles / WINDOW_MIN_TILES > 1 ? n_tiles / WINDOW_MIN_TILES : 1;
  if (s > cap_by_tiles) s = cap_by_tiles;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  return s;
}

int launch_window(const AttnParams& p, hipStream_t stream) {
  const int hgroups = (p.H + 63) / 64;
  dim3 grid(p.splits, p.rows, hgroups);
  window_kernel<<<grid, 256, 0, stream>>>(p);
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
