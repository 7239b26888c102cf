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

// R rows per tile (1, 2, 4: as the sparse kernel's row tiles); a unit is (tile, split)
template <int R>
__global__ __launch_bounds__(256, 2) void window_kernel(AttnParams p, int n_units, int hgroups) {
  __shared__ win::WinLds lds;
  int unit, hgi;
  map_unit(blockIdx.x, n_units, hgroups, p.splits > 1, unit, hgi);
  if (unit >= n_units) return;
  win::window_unit<R>(p, unit / p.splits, unit % p.splits, hgi, lds);
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

// the rule above over a launch's tiles: rows, or row tiles of 32 / R heads
int window_attn_splits(int B, int Q, int H, int W) {
  const int r = sparse_rows_per_tile(H, Q);
  const int hp = 32 / r;
  return window_splits(B * ((Q + r - 1) / r) * ((H + hp - 1) / hp), 32, (W + 31) / 32);
}

int launch_window(const AttnParams& p, hipStream_t stream) {
  const int r = sparse_rows_per_tile(p.H, p.Q);
  const int hp = 32 / r;
  const int hgroups = (p.H + hp - 1) / hp;
  const int n_units = (p.rows / p.Q) * ((p.Q + r - 1) / r) * p.splits;
  const long long n_wg = (long long)((n_units + 7) / 8) * 8 * hgroups;
  if (n_wg > 0x7FFFFFFF) return -4;
  const dim3 grid((unsigned)n_wg);
  if (r == 4)
    window_kernel<4><<<grid, 256, 0, stream>>>(p, n_units, hgroups);
  else if (r == 2)
    window_kernel<2><<<grid, 256, 0, stream>>>(p, n_units, hgroups);
  else
    window_kernel<1><<<grid, 256, 0, stream>>>(p, n_units, hgroups);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// ---- combine -----------------------------------------------------------
// Log-sum-exp merge of the split-K partials (and an optional fp32 extra
// branch) of one (row, head): wave 0 turns the partials' lse and exponents into
// weights in LDS while every wave already streams its share of the partials:
// wave g takes splits g, g + 4, ..., each lane 8 of the 512 dims (16-byte
// loads, 8 splits in flight); the four waves' sums meet in LDS and each thread
// writes 2 dims.  512 dims x 33 splits of fp16 at 64 heads x 8 rows is 17 MB:
// bandwidth-bound, so each CU needs many bytes in flight.
constexpr int MAX_COMBINE_SPLITS = 128;
constexpr int CMB_WAVES = 4;
constexpr int CMB_PF = 8;

__global__ __launch_bounds__(64 * CMB_WAVES) void combine_kernel(const uint16_t* __restrict__ o16,
                                                                 const int32_t* __restrict__ oexp,
                                                                 const float* __restrict__ lse_part,
                                                                 int splits, int H,
                                                                 const float* __restrict__ o_ext,
                                                                 const float* __restrict__ lse_ext,
                                                                 float* __restrict__ out,
                                                                 float* __restrict__ lse_out, int xcd_rows) {
  __shared__ float wts[MAX_COMBINE_SPLITS + 1];
  __shared__ float L_sh;
  __shared__ __align__(16) float red[CMB_WAVES][D];
  int h, row;
  if (xcd_rows) {
    // 1-D grid of rows x H: workgroup L runs on XCD L % 8, and takes a (row,
    // head) of rows [x R/8, (x + 1) R/8), the rows whose split partials the
    // attention launch wrote on that XCD; an XCD's workgroups then read the
    // partials of neighbouring heads of few rows
    const int L = blockIdx.x, x = L & 7, k = L >> 3;
    row = x * xcd_rows + k / H;
    h = k - (k / H) * H;
  } else {
    h = blockIdx.x;
    row = blockIdx.y;
  }
  const int t = threadIdx.x;
  const int g = t >> 6, l = t & 63;
  const size_t rh = (size_t)row * H + h;
  const size_t part0 = rh * splits;                               // split s at part0 + s
  const float* lp = lse_part + part0;

  // this wave's partials: splits g + 4i, lane dims [8l, 8l + 8); the first
  // CMB_PF requested before the weights exist (they do not depend on them)
  typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
  const uint4* src = reinterpret_cast<const uint4*>(o16 + part0 * D) + l;
  const size_t stride = (size_t)CMB_WAVES * D / 8;               // 4 splits, in uint4
  const int n_mine = g < splits ? (splits - g + CMB_WAVES - 1) / CMB_WAVES : 0;
  src += (size_t)g * D / 8;
  uint4 buf[CMB_PF];
#pragma unroll
  for (int i = 0; i < CMB_PF; ++i) buf[i] = i < n_mine ? src[(size_t)i * stride] : make_uint4(0u, 0u, 0u, 0u);

  if (g == 0) {
    // lane l holds splits l and l + 64 (splits <= 128): every load issued at once
    float lv[2];
    int ev[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int s = l + 64 * j;
      lv[j] = s < splits ? lp[s] : -__builtin_inff();
      ev[j] = s < splits ? oexp[part0 + s] : 0;
    }
    const float le = (o_ext && l == 0) ? lse_ext[rh] : -__builtin_inff();
    float m = fmaxf(le, fmaxf(lv[0], lv[1]));
    m = __uint_as_float(wave_allreduce(__float_as_uint(m), [](uint32_t a, uint32_t b) {
      return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
    }));
    float sum = 0.f;
    if (m != -__builtin_inff()) sum = expf(lv[0] - m) + expf(lv[1] - m) + expf(le - m);
    sum = __uint_as_float(wave_allreduce(__float_as_uint(sum), [](uint32_t a, uint32_t b) {
      return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
    }));
    const float L = m == -__builtin_inff() ? -__builtin_inff() : m + logf(sum);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int s = l + 64 * j;
      if (s < splits) wts[s] = L == -__builtin_inff() ? 0.f : ldexpf(expf(lv[j] - L), ev[j]);
    }
    if (l == 0) {
      wts[splits] = (o_ext && L != -__builtin_inff()) ? expf(le - L) : 0.f;
      L_sh = L;
    }
  }
  __syncthreads();

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int i0 = 0; i0 < n_mine; i0 += CMB_PF) {
#pragma unroll
    for (int i = 0; i < CMB_PF; ++i) {
      if (i0 + i < n_mine) {
        const float wv = wts[g + CMB_WAVES * (i0 + i)];
        const halfx8 hv = __builtin_bit_cast(halfx8, buf[i]);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] += wv * (float)hv[k];
      }
    }
#pragma unroll
    for (int i = 0; i < CMB_PF; ++i)
      if (i0 + CMB_PF + i < n_mine) buf[i] = src[(size_t)(i0 + CMB_PF + i) * stride];
  }
  reinterpret_cast<float4*>(&red[g][8 * l])[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  reinterpret_cast<float4*>(&red[g][8 * l])[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  __syncthreads();

  // thread t: dims 2t, 2t + 1
  float2 o = make_float2(0.f, 0.f);
#pragma unroll
  for (int w = 0; w < CMB_WAVES; ++w) {
    const float2 v = reinterpret_cast<const float2*>(red[w])[t];
    o.x += v.x; o.y += v.y;
  }
  if (o_ext) {
    // o_ext may alias out: this thread reads exactly the dims it then writes
    const float we = wts[splits];
    if (we != 0.f) {
      const float2 v = reinterpret_cast<const float2*>(o_ext + rh * D)[t];
      o.x += we * v.x; o.y += we * v.y;
    }
  }
  reinterpret_cast<float2*>(out + rh * D)[t] = o;
  if (t == 0) lse_out[rh] = L_sh;
}

int launch_combine(const uint16_t* o16, const int32_t* oexp, const float* lse_part, int rows,
                   int splits, int H, const float* o_ext, const float* lse_ext, float* out,
                   float* lse_out, hipStream_t stream) {
  if (splits > MAX_COMBINE_SPLITS) return -4;
  if (rows % 8 == 0) {
    // the attention launches place rows [x R/8, (x + 1) R/8) on XCD x when R is
    // a multiple of 8 (map_unit): the combine follows them there.  Decode
    // attention calls 1.5-2 us faster (decode1m 45.7-47.0 -> 43.7-44.4 us cold),
    // though the partials are still fetched from beyond L2 (5% less)
    combine_kernel<<<dim3((unsigned)(rows * H)), 64 * CMB_WAVES, 0, stream>>>(o16, oexp, lse_part, splits, H, o_ext,
                                                                              lse_ext, out, lse_out, rows / 8);
  } else {
    dim3 grid(H, rows);
    combine_kernel<<<grid, 64 * CMB_WAVES, 0, stream>>>(o16, oexp, lse_part, splits, H, o_ext, lse_ext, out,
                                                        lse_out, 0);
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace csa2
