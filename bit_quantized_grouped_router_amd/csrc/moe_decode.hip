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

constexpr int kDecUnitsPerWave = 2;

// uint4 chunks of h each of the 128 threads of decode_down stages through
// registers (0: copy in a plain loop instead), for up to kMaxK routed slots
// and expert width f. The LDS allocation covers the chunks staged.
constexpr int h_stage_chunks(int kMaxK, int f) {
  return ((kMaxK + 1) * f / 8 + 127) / 128 <= 12 ? ((kMaxK + 1) * f / 8 + 127) / 128 : 0;
}

// 32 weights of one group (16 bytes of codes) dotted with 32 bf16
// activations, using the GEMM tiles' dequantisation (fast path when exact).
__device__ __forceinline__ float dot32_any(uint4 c, uint32_t sb, const uint4 *xv, float acc) {
  uint4 w[4];
  dequant32(c, sb, w);
  acc = dot8(w[0], xv[0], acc);
  acc = dot8(w[1], xv[1], acc);
  acc = dot8(w[2], xv[2], acc);
  acc = dot8(w[3], xv[3], acc);
  return acc;
}

// One wavefront = one slot (routed slot j < k, or the shared expert at
// j == k) and two intermediate units (4 weight rows). Loads are issued as
// early as their addresses are known: x first, the shared expert's rows at
// once, a routed slot's rows right after the workgroup's on-chip top-k.
template <int kMaxPerLane>
__global__ __launch_bounds__(256) void decode_gate_up_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ logits, W4 w13, W4 s13, int d,
    int f, int E, int k, int32_t *__restrict__ ids_out, float *__restrict__ wts_out,
    uint16_t *__restrict__ h) {
  __shared__ int s_expert;
  // token blockIdx.y (a few tokens take the same kernels, one grid row each)
  {
    const int t = blockIdx.y;
    x += (size_t)t * d;
    logits += (size_t)t * E;
    ids_out += (size_t)t * k;
    wts_out += (size_t)t * k;
    h += (size_t)t * (k + 1) * f;
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gw = blockIdx.x * 4 + wave;
  // the launch has exactly (k + 1) * f / 2 wavefronts (f % 8 == 0), and the
  // 8 units of a workgroup belong to one slot
  const int item = gw * kDecUnitsPerWave;
  const int slot = item / f, n = item % f;
  const bool shared = slot == k;
  // this lane's first 32 columns of x, loaded before the routing (independent of it)
  uint4 xv0[4] = {};
  if (lane * 32 < d) {
    const uint4 *xp = (const uint4 *)(x + lane * 32);
    xv0[0] = xp[0];
    xv0[1] = xp[1];
    xv0[2] = xp[2];
    xv0[3] = xp[3];
  }
  // the top-k once per workgroup (wavefront 0; the other three wait at the
  // barrier instead of repeating it), shared through LDS
  if (wave == 0 && !shared) {
    int id;
    float l;
    wave_topk<kMaxPerLane>(logits, E, k, &id, &l);
    if (lane == slot) s_expert = id;
    if (gw == 0) {
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
  const int expert = shared ? 0 : __builtin_amdgcn_readfirstlane(s_expert);
  const W4 W = shared ? s13 : w13;
  const size_t rb = (size_t)expert * 2 * f;
  const size_t rows[4] = {rb + n, rb + n + 1, rb + f + n, rb + f + n + 1};
  const int ngroups = d / kGroup;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = lane * 32; c0 < d; c0 += kWave * 32) {
    uint4 c[4];
    uint16_t sr[4], br[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      c[r] = *(const uint4 *)(W.codes + rows[r] * (size_t)(d / 2) + c0 / 2);
      const size_t gi = rows[r] * (size_t)ngroups + c0 / kGroup;
      sr[r] = W.scales[gi];
      br[r] = W.biases[gi];
    }
    uint4 xv[4] = {xv0[0], xv0[1], xv0[2], xv0[3]};
    if (c0 != lane * 32) {
      const uint4 *xp = (const uint4 *)(x + c0);
      xv[0] = xp[0];
      xv[1] = xp[1];
      xv[2] = xp[2];
      xv[3] = xp[3];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      acc[r] = dot32_any(c[r], (uint32_t)sr[r] | ((uint32_t)br[r] << 16), xv, acc[r]);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] = wave_sum_dpp(acc[r]);
  if (lane == 0) {
    h[(size_t)slot * f + n] = to_bf16(silu_mul(acc[0], acc[2]));
    h[(size_t)slot * f + n + 1] = to_bf16(silu_mul(acc[1], acc[3]));
  }
}

// Rows of the down projection: kLanesPerRow lanes x 32 columns per row,
// (k + 1) experts per row. Every weight load is issued before any arithmetic:
// the shared expert's at once, the routed ones as soon as the chosen ids
// (written by decode_gate_up) arrive; h is staged in LDS meanwhile.
// Rows of the down projection: kLanesPerRow lanes x 32 columns per row,
// (k + 1) experts per row. The routed rows depend on the chosen ids written
// by decode_gate_up, so the critical path is two memory round trips: first
// the ids (scalar loads) together with h (staged in LDS), then every weight
// load of the row (the shared expert's and the k routed ones) at once.
template <int kLanesPerRow, int kMaxK>
__global__ __launch_bounds__(128) void decode_down_kernel(
    const int32_t *__restrict__ ids, const float *__restrict__ wts,
    const uint16_t *__restrict__ h, W4 w2, W4 s2, int d, int f, int E, int k,
    float *__restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint16_t hs[];
  {
    const int t = blockIdx.y;  // token
    ids += (size_t)t * k;
    wts += (size_t)t * k;
    h += (size_t)t * (k + 1) * f;
    y += (size_t)t * d;
  }
  const int tid = threadIdx.x;
  constexpr int kRowsPerWave = kWave / kLanesPerRow;
  const int wave = tid >> 6, lane = tid & 63;
  const int m = (blockIdx.x * (blockDim.x / kWave) + wave) * kRowsPerWave + lane / kLanesPerRow;
  const bool row_ok = m < d;  // whole wavefronts agree: d % 64 == 0
  const int mm = row_ok ? m : 0;
  const int c0 = (lane % kLanesPerRow) * 32;
  const int ngroups = f / kGroup;
  // round trip 1: the chosen ids and weights (scalar loads) and h into LDS.
  // The loads are unconditional (clamped) so they can be issued together.
  int eid[kMaxK];
  float wr[kMaxK];
#pragma unroll
  for (int s = 0; s < kMaxK; ++s) {
    eid[s] = ids[s < k ? s : k - 1];
    wr[s] = s < k ? wts[s < k ? s : k - 1] : 0.f;
  }
  // f = 32 * kLanesPerRow, so the chunk count per thread is known at compile
  // time; all loads go out before the stores (chunks past the end re-read
  // chunk 0 and land in the LDS padding)
  constexpr int kHChunks = h_stage_chunks(kMaxK, 32 * kLanesPerRow);
  const int hn = (k + 1) * f / 8;  // uint4 chunks of h
  if (kHChunks > 0) {
    uint4 hr[kHChunks > 0 ? kHChunks : 1];
#pragma unroll
    for (int i = 0; i < kHChunks; ++i) {
      const int ci = tid + i * 128;
      hr[i] = ((const uint4 *)h)[ci < hn ? ci : 0];
    }
#pragma unroll
    for (int i = 0; i < kHChunks; ++i) ((uint4 *)hs)[tid + i * 128] = hr[i];
  } else {
    for (int ci = tid; ci < hn; ci += 128) ((uint4 *)hs)[ci] = ((const uint4 *)h)[ci];
  }
  lds_barrier();
  if (!row_ok) return;
  // round trip 2: every weight of the row. Scales and biases stay 16-bit until
  // used, so no instruction waits on a load early.
  const size_t srow = (size_t)mm;
  const uint4 csh = *(const uint4 *)(s2.codes + srow * (size_t)(f / 2) + c0 / 2);
  const uint16_t ssh = s2.scales[srow * ngroups + c0 / kGroup];
  const uint16_t bsh = s2.biases[srow * ngroups + c0 / kGroup];
  uint4 cr[kMaxK];
  uint16_t sr[kMaxK], br[kMaxK];
#pragma unroll
  for (int s = 0; s < kMaxK; ++s) {
    const size_t row = (size_t)eid[s] * d + mm;
    cr[s] = *(const uint4 *)(w2.codes + row * (size_t)(f / 2) + c0 / 2);
    sr[s] = w2.scales[row * ngroups + c0 / kGroup];
    br[s] = w2.biases[row * ngroups + c0 / kGroup];
  }
  // per-lane partial dots first, one group reduction at the end
  float part = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxK; ++s) {
    if (s >= k) continue;
    const uint4 *hp = (const uint4 *)(hs + (size_t)s * f + c0);
    const uint4 hv[4] = {hp[0], hp[1], hp[2], hp[3]};
    part = fmaf(wr[s], dot32_any(cr[s], (uint32_t)sr[s] | ((uint32_t)br[s] << 16), hv, 0.f), part);
  }
  {
    const uint4 *hp = (const uint4 *)(hs + (size_t)k * f + c0);
    const uint4 hv[4] = {hp[0], hp[1], hp[2], hp[3]};
    part += dot32_any(csh, (uint32_t)ssh | ((uint32_t)bsh << 16), hv, 0.f);
  }
  float acc;
  if constexpr (kLanesPerRow <= 16)
    acc = group_sum_dpp<kLanesPerRow>(part);
  else
    acc = group_sum<kLanesPerRow>(part);
  if (lane % kLanesPerRow == 0) y[m] = acc;
}

// Tokens up to which the layer runs these kernels, one grid row per token
// (each token's experts are streamed for it alone; the weights two tokens
// share come from the caches the second time).
constexpr int kDecodeMaxT = 16;

bool decode_supported(const Dims &dm) {
  const int lpr = dm.f / 32;
  const bool pow2 = lpr >= 2 && lpr <= 64 && (lpr & (lpr - 1)) == 0;
  return dm.T >= 1 && dm.T <= kDecodeMaxT && pow2 && (size_t)(dm.k + 1) * dm.f * 2 <= 48 * 1024 &&
         (size_t)h_stage_chunks(dm.k <= 8 ? 8 : 32, dm.f) * 128 * 16 <= 48 * 1024;
}

template <int kLanesPerRow>
static void launch_down_t(const Dims &dm, const int32_t *ids, const float *wts, const uint16_t *h,
                          const Weights &w, float *y, hipStream_t s) {
  constexpr int kRowsPerWave = kWave / kLanesPerRow;
  const int waves = dm.d / kRowsPerWave;
  const int blocks = (waves + 1) / 2;
  // h, or every chunk the kernel stages (128 threads x 16 bytes each)
  auto lds_bytes = [&](int kmax) {
    const size_t need = (size_t)(dm.k + 1) * dm.f * 2;
    const size_t staged = (size_t)h_stage_chunks(kmax, 32 * kLanesPerRow) * 128 * 16;
    return need > staged ? need : staged;
  };
  if (dm.k <= 8)
    decode_down_kernel<kLanesPerRow, 8><<<dim3(blocks, dm.T), 128, lds_bytes(8), s>>>(
        ids, wts, h, w.w2, w.s2, dm.d, dm.f, dm.E, dm.k, y);
  else
    decode_down_kernel<kLanesPerRow, 32><<<dim3(blocks, dm.T), 128, lds_bytes(32), s>>>(
        ids, wts, h, w.w2, w.s2, dm.d, dm.f, dm.E, dm.k, y);
}

hipError_t launch_decode(const Dims &dm, const uint16_t *x, const float *logits, const Weights &w,
                         int32_t *ids, float *wts, uint16_t *h, float *y, hipStream_t s) {
  const int waves = (dm.k + 1) * dm.f / kDecUnitsPerWave;
  const int blocks = (waves + 3) / 4;
  if (dm.E <= 64)
    decode_gate_up_kernel<1><<<dim3(blocks, dm.T), 256, 0, s>>>(x, logits, w.w13, w.s13, dm.d, dm.f, dm.E,
                                                    dm.k, ids, wts, h);
  else if (dm.E <= 256)
    decode_gate_up_kernel<4><<<dim3(blocks, dm.T), 256, 0, s>>>(x, logits, w.w13, w.s13, dm.d, dm.f, dm.E,
                                                    dm.k, ids, wts, h);
  else
    decode_gate_up_kernel<16><<<dim3(blocks, dm.T), 256, 0, s>>>(x, logits, w.w13, w.s13, dm.d, dm.f, dm.E,
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
