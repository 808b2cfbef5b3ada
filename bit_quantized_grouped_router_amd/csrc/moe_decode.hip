// Batch-1 decode path of the layer (noticiai.com.br page on Lily, section
// "Prefill e decode: onde estao os ganhos": at batch 1 there is almost no
// weight reuse, so memory bandwidth sets the ceiling).
//
// Two kernels, no permutation and no GEMM tiles:
//   decode_gate_up  every workgroup recomputes the top-k of the token's
//                   logits on chip (one wavefront, 256 logits) and streams
//                   gate/up rows of the k routed experts and the shared one
//                   with 16-byte loads per lane (32 codes), dequantises
//                   them exactly like the GEMM tiles, and writes
//                   h = bf16(silu(gate) * up) for (k+1) x f units;
//   decode_down     stages h in LDS, streams the down rows of the same
//                   (k+1) experts (16 lanes x 16 bytes per row at f = 512)
//                   and writes y = shared + sum_j w_j * routed_j in fp32.
// Products of two bf16 values are exact in fp32; they are summed with
// v_dot2c_f32_bf16 in fp32.
#include "moe_launch.h"

namespace moe {

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

// 32 weights (16 bytes of codes, one group) dotted with 32 bf16 activations.
__device__ __forceinline__ float dot32(uint4 c, float s, float b, const uint4 *xv, float acc) {
  acc = dot8(dequant8(c.x, s, b), xv[0], acc);
  acc = dot8(dequant8(c.y, s, b), xv[1], acc);
  acc = dot8(dequant8(c.z, s, b), xv[2], acc);
  acc = dot8(dequant8(c.w, s, b), xv[3], acc);
  return acc;
}

constexpr int kDecUnitsPerWave = 2;

template <int kMaxPerLane>
__global__ __launch_bounds__(256) void decode_gate_up_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ logits, W4 w13, W4 s13, int d,
    int f, int E, int k, int32_t *__restrict__ ids_out, float *__restrict__ wts_out,
    uint16_t *__restrict__ h) {
  __shared__ int s_ids[32];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (wave == 0) {
    int id;
    float l;
    wave_topk<kMaxPerLane>(logits, E, k, &id, &l);
    if (lane < k) s_ids[lane] = id;
    if (blockIdx.x == 0) {
      const float m = __shfl(l, 0, kWave);
      const float e = lane < k ? expf(l - m) : 0.f;
      const float sum = wave_sum(e);
      if (lane < k) {
        ids_out[lane] = id;
        wts_out[lane] = e / sum;
      }
    }
  }
  __syncthreads();
  const int item = (blockIdx.x * 4 + wave) * kDecUnitsPerWave;
  if (item >= (k + 1) * f) return;
  const int slot = item / f, n = item % f;
  const bool shared = slot == k;
  const W4 W = shared ? s13 : w13;
  const size_t rb = (shared ? 0 : (size_t)s_ids[slot]) * 2 * f;
  const size_t rows[4] = {rb + n, rb + n + 1, rb + f + n, rb + f + n + 1};
  const int ngroups = d / kGroup;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = lane * 32; c0 < d; c0 += kWave * 32) {
    const uint4 *xp = (const uint4 *)(x + c0);
    const uint4 xv[4] = {xp[0], xp[1], xp[2], xp[3]};
    uint4 c[4];
    float s[4], b[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      c[r] = *(const uint4 *)(W.codes + rows[r] * (size_t)(d / 2) + c0 / 2);
      const size_t gi = rows[r] * (size_t)ngroups + c0 / kGroup;
      s[r] = bf16_to_f32(W.scales[gi]);
      b[r] = bf16_to_f32(W.biases[gi]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = dot32(c[r], s[r], b[r], xv, acc[r]);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] = wave_sum(acc[r]);
  if (lane == 0) {
    h[(size_t)slot * f + n] = to_bf16(silu_mul(acc[0], acc[2]));
    h[(size_t)slot * f + n + 1] = to_bf16(silu_mul(acc[1], acc[3]));
  }
}

template <int kLanesPerRow>
__global__ __launch_bounds__(128) void decode_down_kernel(
    const int32_t *__restrict__ ids, const float *__restrict__ wts,
    const uint16_t *__restrict__ h, W4 w2, W4 s2, int d, int f, int E, int k,
    float *__restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint16_t hs[];
  __shared__ int s_ids[32];
  __shared__ float s_w[32];
  const int tid = threadIdx.x;
  for (int i = tid * 8; i < (k + 1) * f; i += blockDim.x * 8)
    *(uint4 *)(hs + i) = *(const uint4 *)(h + i);
  if (tid < k) {
    s_ids[tid] = ids[tid];
    s_w[tid] = wts[tid];
  }
  __syncthreads();
  constexpr int kRowsPerWave = kWave / kLanesPerRow;
  const int wave = tid >> 6, lane = tid & 63;
  const int m = (blockIdx.x * (blockDim.x / kWave) + wave) * kRowsPerWave + lane / kLanesPerRow;
  if (m >= d) return;  // whole wavefronts leave together: d % 64 == 0
  const int c0 = (lane % kLanesPerRow) * 32;
  const int ngroups = f / kGroup;
  float acc = 0.f;
  for (int s = 0; s <= k; ++s) {
    const bool sh = s == k;
    const W4 W = sh ? s2 : w2;
    const size_t row = (sh ? 0 : (size_t)s_ids[s]) * d + m;
    const uint4 c = *(const uint4 *)(W.codes + row * (size_t)(f / 2) + c0 / 2);
    const size_t gi = row * (size_t)ngroups + c0 / kGroup;
    const float sc = bf16_to_f32(W.scales[gi]), bi = bf16_to_f32(W.biases[gi]);
    const uint4 *hp = (const uint4 *)(hs + (size_t)s * f + c0);
    const uint4 hv[4] = {hp[0], hp[1], hp[2], hp[3]};
    float part = group_sum<kLanesPerRow>(dot32(c, sc, bi, hv, 0.f));
    acc = sh ? acc + part : fmaf(s_w[s], part, acc);
  }
  if (lane % kLanesPerRow == 0) y[m] = acc;
}

bool decode_supported(const Dims &dm) {
  const int lpr = dm.f / 32;
  const bool pow2 = lpr >= 2 && lpr <= 64 && (lpr & (lpr - 1)) == 0;
  return dm.T == 1 && pow2 && (size_t)(dm.k + 1) * dm.f * 2 <= 48 * 1024;
}

template <int kLanesPerRow>
static void launch_down_t(const Dims &dm, const int32_t *ids, const float *wts, const uint16_t *h,
                          const Weights &w, float *y, hipStream_t s) {
  constexpr int kRowsPerWave = kWave / kLanesPerRow;
  const int waves = dm.d / kRowsPerWave;
  const int blocks = (waves + 1) / 2;
  const size_t lds = (size_t)(dm.k + 1) * dm.f * 2;
  decode_down_kernel<kLanesPerRow><<<blocks, 128, lds, s>>>(ids, wts, h, w.w2, w.s2, dm.d, dm.f,
                                                            dm.E, dm.k, y);
}

hipError_t launch_decode(const Dims &dm, const uint16_t *x, const float *logits, const Weights &w,
                         int32_t *ids, float *wts, uint16_t *h, float *y, hipStream_t s) {
  const int waves = (dm.k + 1) * dm.f / kDecUnitsPerWave;
  const int blocks = (waves + 3) / 4;
  if (dm.E <= 64)
    decode_gate_up_kernel<1><<<blocks, 256, 0, s>>>(x, logits, w.w13, w.s13, dm.d, dm.f, dm.E,
                                                    dm.k, ids, wts, h);
  else if (dm.E <= 256)
    decode_gate_up_kernel<4><<<blocks, 256, 0, s>>>(x, logits, w.w13, w.s13, dm.d, dm.f, dm.E,
                                                    dm.k, ids, wts, h);
  else
    decode_gate_up_kernel<16><<<blocks, 256, 0, s>>>(x, logits, w.w13, w.s13, dm.d, dm.f, dm.E,
                                                     dm.k, ids, wts, h);
  switch (dm.f / 32) {
    case 2: launch_down_t<2>(dm, ids, wts, h, w, y, s); break;
    case 4: launch_down_t<4>(dm, ids, wts, h, w, y, s); break;
    case 8: launch_down_t<8>(dm, ids, wts, h, w, y, s); break;
    case 16: launch_down_t<16>(dm, ids, wts, h, w, y, s); break;
    case 32: launch_down_t<32>(dm, ids, wts, h, w, y, s); break;
    default: launch_down_t<64>(dm, ids, wts, h, w, y, s); break;
  }
  return hipGetLastError();
}

}  // namespace moe
