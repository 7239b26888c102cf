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
// The window workgroup body is in window_body.h (the fused attention launch in
// sparse_fp4.hip runs it too).
#include "device.h"
#include "launch.h"
#include "window_body.h"

namespace csa2 {

__global__ __launch_bounds__(256, 2) void window_kernel(AttnParams p, int hgroups) {
  __shared__ win::WinLds lds;
  int unit, hgi;
  map_unit(blockIdx.x, p.rows * p.splits, hgroups, p.splits > 1, unit, hgi);
  if (unit >= p.rows * p.splits) return;
  win::window_unit(p, unit / p.splits, unit % p.splits, hgi, lds);
}

int window_splits(int rows, int H, int n_tiles) {
  const int hgroups = (H + 31) / 32;
  const int wgs = rows * hgroups;
  int s = (win::WINDOW_TARGET_WGS + wgs - 1) / wgs;
  const int cap_by_tiles = n_tiles / win::WINDOW_MIN_TILES > 1 ? n_tiles / win::WINDOW_MIN_TILES : 1;
  if (s > cap_by_tiles) s = cap_by_tiles;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  return s;
}

int launch_window(const AttnParams& p, hipStream_t stream) {
  const int hgroups = (p.H + 31) / 32;
  const int n_units = p.rows * p.splits;
  const long long n_wg = (long long)((n_units + 7) / 8) * 8 * hgroups;
  if (n_wg > 0x7FFFFFFF) return -4;
  window_kernel<<<dim3((unsigned)n_wg), 256, 0, stream>>>(p, hgroups);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// ---- combine -----------------------------------------------------------
// Log-sum-exp merge of the split-K partials (and an optional fp32 extra
// branch) of one (row, head): wave 0 turns the partials' lse and exponents into
// weights in LDS, then every thread streams 4 of the 512 dims over the splits,
// 16 splits in flight at a time.
constexpr int MAX_COMBINE_SPLITS = 128;

__global__ __launch_bounds__(128) void combine_kernel(const uint16_t* __restrict__ o16,
                                                      const int32_t* __restrict__ oexp,
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
  const size_t part0 = (size_t)row * splits * H + h;              // split s at part0 + s * H
  const float* lp = lse_part + part0;
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
      wts[s] = L == -__builtin_inff() ? 0.f : ldexpf(expf(lp[(size_t)s * H] - L), oexp[part0 + (size_t)s * H]);
    if (t == 0) {
      wts[splits] = (o_ext && L != -__builtin_inff()) ? expf(le - L) : 0.f;
      L_sh = L;
    }
  }
  typedef _Float16 halfx4 __attribute__((ext_vector_type(4)));
  const uint2* src = reinterpret_cast<const uint2*>(o16 + part0 * D) + t;
  const size_t stride = (size_t)H * D / 4;                       // one split, in uint2
  // 16 splits' loads in flight per thread, the first 16 requested before the
  // weights are ready (the partials do not depend on them)
  constexpr int PF = 16;
  uint2 buf[PF];
#pragma unroll
  for (int i = 0; i < PF; ++i) buf[i] = i < splits ? src[(size_t)i * stride] : make_uint2(0u, 0u);
  __syncthreads();
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < splits; s0 += PF) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      if (s0 + i < splits) {
        const floatx4 f = __builtin_convertvector(__builtin_bit_cast(halfx4, buf[i]), floatx4);
        const float wv = wts[s0 + i];
        acc.x += wv * f[0]; acc.y += wv * f[1]; acc.z += wv * f[2]; acc.w += wv * f[3];
      }
    }
#pragma unroll
    for (int i = 0; i < PF; ++i)
      if (s0 + PF + i < splits) buf[i] = src[(size_t)(s0 + PF + i) * stride];
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

int launch_combine(const uint16_t* o16, const int32_t* oexp, const float* lse_part, int rows,
                   int splits, int H, const float* o_ext, const float* lse_ext, float* out,
                   float* lse_out, hipStream_t stream) {
  dim3 grid(H, rows);
  combine_kernel<<<grid, 128, 0, stream>>>(o16, oexp, lse_part, splits, H, o_ext, lse_ext, out,
                                           lse_out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace csa2
