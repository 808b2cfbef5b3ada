// Grouped expert projections for small batches (noticiai.com.br page on
// Lily, section "Prefill e decode: onde estao os ganhos": weights rebuilt to
// bf16 on chip, fp32 accumulation; at small batches the weight bytes, not
// the arithmetic, set the pace).
//
// With a few tokens the tiles of the block map hold a few rows each, and the
// matrix-core tiles (one wavefront rebuilding 64 weight rows over all of K)
// leave most SIMDs idle. Here every wavefront rebuilds only a handful of
// weight rows once, keeps them in registers as bf16, and reuses them for
// every row of its tile with v_dot2_f32_bf16:
//   gate_up_gemv  one wavefront per (tile, 2 units): the 4 weight rows gate
//                 n, n+1 and up n, n+1 (32 input columns per lane, d <= 2048),
//                 then per permuted row of the tile the dot products with
//                 that row's token, reduced over the wavefront, and
//                 h = bf16(silu(gate) * up);
//   down_gemv     one wavefront per (tile, 64 / L output rows), L = f / 32
//                 lanes per row, 32 units per lane; per permuted row the dot
//                 products with h, reduced over the L lanes, into o (bf16
//                 for routed rows, fp32 for the shared expert's).
// Same inputs and outputs as the matrix-core kernels (the block map's tiles,
// h [T*k+T][f], o_routed, o_shared), so the two are interchangeable.
#include "moe_launch.h"

namespace moe {

constexpr int kGvWaves = 4;                       // wavefronts per workgroup
constexpr int kGvUnits = 2;                       // gate/up units per wavefront
constexpr int kGvUnitsPerWg = kGvWaves * kGvUnits;
constexpr int kGvMaxD = kWave * 32;               // one pass of 32 columns per lane
// tokens up to which the layer takes these kernels (measured on the
// Qwen-shaped layer: 1.6x faster than the matrix-core tiles at T = 2, 1.3x
// at T = 4, 5% slower at T = 8)
constexpr int kGvMaxT = 6;

__device__ __forceinline__ float dot8(uint4 w, uint4 x, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x),
                                        __builtin_bit_cast(bf16x2_t, x.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y),
                                        __builtin_bit_cast(bf16x2_t, x.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z),
                                        __builtin_bit_cast(bf16x2_t, x.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w),
                                        __builtin_bit_cast(bf16x2_t, x.w), acc, false);
  return acc;
}

// 32 rebuilt weights (four words of bf16 pairs) dotted with 32 bf16 activations.
__device__ __forceinline__ float dot32(const uint4 (&w)[4], const uint4 (&x)[4]) {
  float a = dot8(w[0], x[0], 0.f);
  a = dot8(w[1], x[1], a);
  a = dot8(w[2], x[2], a);
  return dot8(w[3], x[3], a);
}

__device__ __forceinline__ uint32_t gv_scale_bias(const W4 &m, size_t gi) {
  return (uint32_t)m.scales[gi] | ((uint32_t)m.biases[gi] << 16);
}

__device__ __forceinline__ void load_row32(const uint16_t *p, uint4 (&v)[4]) {
  const uint4 *q = (const uint4 *)p;
  v[0] = q[0];
  v[1] = q[1];
  v[2] = q[2];
  v[3] = q[3];
}

__global__ __launch_bounds__(kGvWaves * kWave) void gate_up_gemv_kernel(
    const uint16_t *__restrict__ x, W4 wr, W4 ws, const int32_t *__restrict__ sorted_token,
    const int32_t *__restrict__ tile_map, const int32_t *__restrict__ num_tiles_p,
    uint16_t *__restrict__ h, int T, int d, int f, int E, int k) {
  const int ublocks = f / kGvUnitsPerWg;
  const int tile = blockIdx.x / ublocks;
  if (tile >= *num_tiles_p) return;
  const int4 tm = *(const int4 *)(tile_map + 4 * (size_t)tile);
  const int g = tm.x, rb = tm.y, re = tm.z;
  const bool shared = g >= E;
  const W4 W = shared ? ws : wr;
  const size_t ex = shared ? 0 : (size_t)g;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = (blockIdx.x % ublocks) * kGvUnitsPerWg + wave * kGvUnits;
  const int TK = T * k;
  // lanes past d (d < 2048) re-read column 0; their dots are dropped
  const bool col_ok = lane * 32 < d;
  const int col = col_ok ? lane * 32 : 0;
  const int ng = d / kGroup;

  // the 4 weight rows (gate n0, n0+1, up n0, n0+1), rebuilt once
  uint4 c[4];
  uint32_t sb[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const size_t row = ex * 2 * f + (r < 2 ? n0 + r : f + n0 + r - 2);
    c[r] = *(const uint4 *)(W.codes + row * (size_t)(d / 2) + col / 2);
    sb[r] = gv_scale_bias(W, row * ng + col / kGroup);
  }
  // the first row's activations, in flight with the weights
  auto token = [&](int p) {
    const int t = shared ? p - TK : sorted_token[p];
    return t < 0 ? 0 : (t >= T ? T - 1 : t);  // in range for any block map
  };
  uint4 xv[4];
  load_row32(x + (size_t)token(rb) * d + col, xv);
  uint4 w[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) dequant32(c[r], sb[r], w[r]);

  for (int p = rb; p < re; ++p) {
    // the next row's activations, loaded before this row's arithmetic
    uint4 xn[4];
    load_row32(x + (size_t)token(p + 1 < re ? p + 1 : p) * d + col, xn);
    float a[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = dot32(w[r], xv);
      a[r] = wave_sum_dpp(col_ok ? v : 0.f);
    }
    if (lane == 0)
      *(uint32_t *)(h + (size_t)p * f + n0) =
          pack_bf16x2(silu_mul_fast(a[0], a[2]), silu_mul_fast(a[1], a[3]));
#pragma unroll
    for (int q = 0; q < 4; ++q) xv[q] = xn[q];
  }
}

// L lanes per weight row of the down projection (f = 32 L), 64 / L rows per wavefront.
template <int L>
__global__ __launch_bounds__(kGvWaves * kWave) void down_gemv_kernel(
    const uint16_t *__restrict__ h, W4 wr, W4 ws, const int32_t *__restrict__ tile_map,
    const int32_t *__restrict__ num_tiles_p, uint16_t *__restrict__ o_routed,
    float *__restrict__ o_shared, int T, int d, int f, int E, int k) {
  constexpr int kRowsPerWave = kWave / L;
  constexpr int kRowsPerWg = kGvWaves * kRowsPerWave;
  const int mblocks = (d + kRowsPerWg - 1) / kRowsPerWg;
  const int tile = blockIdx.x / mblocks;
  if (tile >= *num_tiles_p) return;
  const int4 tm = *(const int4 *)(tile_map + 4 * (size_t)tile);
  const int g = tm.x, rb = tm.y, re = tm.z;
  const bool shared = g >= E;
  const W4 W = shared ? ws : wr;
  const size_t ex = shared ? 0 : (size_t)g;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = (blockIdx.x % mblocks) * kRowsPerWg + wave * kRowsPerWave + lane / L;
  const bool m_ok = m < d;  // rows past d compute on row 0 and are not stored
  const int c0 = (lane % L) * 32;
  const int TK = T * k;
  const size_t row = ex * d + (m_ok ? m : 0);
  const uint4 cc = *(const uint4 *)(W.codes + row * (size_t)(f / 2) + c0 / 2);
  const uint32_t sbv = gv_scale_bias(W, row * (f / kGroup) + c0 / kGroup);
  uint4 hv[4];
  load_row32(h + (size_t)rb * f + c0, hv);
  uint4 w[4];
  dequant32(cc, sbv, w);
  for (int p = rb; p < re; ++p) {
    uint4 hn[4];
    load_row32(h + (size_t)(p + 1 < re ? p + 1 : p) * f + c0, hn);
    float a;
    if constexpr (L <= 16)
      a = group_sum_dpp<L>(dot32(w, hv));
    else
      a = group_sum<L>(dot32(w, hv));
    if (m_ok && lane % L == 0) {
      if (shared)
        o_shared[(size_t)(p - TK) * d + m] = a;
      else
        o_routed[(size_t)p * d + m] = to_bf16(a);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) hv[q] = hn[q];
  }
}

bool gemv_supported(const Dims &dm) {
  const int L = dm.f / 32;
  return dm.T <= kGvMaxT && dm.d <= kGvMaxD && L >= 2 && L <= 64 && (L & (L - 1)) == 0;
}

hipError_t launch_gate_up_gemv(const Dims &dm, const uint16_t *x, const Weights &w,
                               const int32_t *sorted_token, const int32_t *tile_map,
                               const int32_t *num_tiles, uint16_t *h, hipStream_t s) {
  const int grid = tile_capacity(dm) * (dm.f / kGvUnitsPerWg);
  gate_up_gemv_kernel<<<grid, kGvWaves * kWave, 0, s>>>(x, w.w13, w.s13, sorted_token, tile_map,
                                                        num_tiles, h, dm.T, dm.d, dm.f, dm.E,
                                                        dm.k);
  return hipGetLastError();
}

template <int L>
static void launch_down_l(const Dims &dm, const uint16_t *h, const Weights &w,
                          const int32_t *tile_map, const int32_t *num_tiles, uint16_t *o_routed,
                          float *o_shared, hipStream_t s) {
  constexpr int kRowsPerWg = kGvWaves * (kWave / L);
  const int grid = tile_capacity(dm) * ((dm.d + kRowsPerWg - 1) / kRowsPerWg);
  down_gemv_kernel<L><<<grid, kGvWaves * kWave, 0, s>>>(h, w.w2, w.s2, tile_map, num_tiles,
                                                        o_routed, o_shared, dm.T, dm.d, dm.f,
                                                        dm.E, dm.k);
}

hipError_t launch_down_gemv(const Dims &dm, const uint16_t *h, const Weights &w,
                            const int32_t *tile_map, const int32_t *num_tiles,
                            uint16_t *o_routed, float *o_shared, hipStream_t s) {
  switch (dm.f / 32) {
    case 2: launch_down_l<2>(dm, h, w, tile_map, num_tiles, o_routed, o_shared, s); break;
    case 4: launch_down_l<4>(dm, h, w, tile_map, num_tiles, o_routed, o_shared, s); break;
    case 8: launch_down_l<8>(dm, h, w, tile_map, num_tiles, o_routed, o_shared, s); break;
    case 16: launch_down_l<16>(dm, h, w, tile_map, num_tiles, o_routed, o_shared, s); break;
    case 32: launch_down_l<32>(dm, h, w, tile_map, num_tiles, o_routed, o_shared, s); break;
    default: launch_down_l<64>(dm, h, w, tile_map, num_tiles, o_routed, o_shared, s); break;
  }
  return hipGetLastError();
}

}  // namespace moe
