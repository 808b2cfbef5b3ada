// Batch-1 decode path of the layer (noticiai.com.br page on Lily, section
// "Prefill e decode: onde estao os ganhos": at batch 1 there is almost no
// weight reuse, so memory bandwidth sets the ceiling).
//
// Two kernels, no permutation and no GEMM tiles:
//   decode_gate_up  every workgroup stages x in LDS, recomputes the top-k of
//                   the token's logits on chip (one wavefront, 256 logits)
//                   and streams gate/up rows of the k routed experts and the
//                   shared one with 16-byte loads per lane (32 codes),
//                   dequantises them exactly like the GEMM tiles, and writes
//                   h = bf16(silu(gate) * up) for (k+1) x f units;
//   decode_down     one wavefront per expert slot streams that slot's down
//                   rows (16 lanes x 16 bytes per row at f = 512) with its
//                   h columns read straight from memory, and the first
//                   wavefront writes y = shared + sum_j w_j * routed_j in
//                   fp32, adding the slots' partial rows in slot order.
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

// wavefronts per workgroup of decode_gate_up; the workgroup's units (4 or 8)
// belong to one slot (f % 64 == 0)
constexpr int kDecWaves = 4;
// columns of x a decode_gate_up workgroup stages in LDS: each lane's first
// 32 (64 lanes x 32)
constexpr int kDecXCols = kWave * 32;
static_assert(kDecWaves * kWave * 8 == kDecXCols, "the workgroup's lanes stage the columns, 8 each");
// tokens up to which decode_gate_up takes one unit per wavefront (two above)
constexpr int kDecOneUnitMaxT = 4;
// wavefronts of a decode_down_slots workgroup at most (one per expert slot)
constexpr int kDownSlotWaves = 16;

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
// j == k) and U intermediate units (a gate row and an up row each). The
// logits and x are loaded first, together; past the workgroup's barrier each
// wavefront loads its slot's weight rows (a routed slot's once the on-chip
// top-k has chosen the expert).
template <int kMaxPerLane, int U>
__global__ __launch_bounds__(kDecWaves * 64) void decode_gate_up_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ logits, W4 w13, W4 s13, int d,
    int f, int E, int k, int32_t *__restrict__ ids_out, float *__restrict__ wts_out,
    uint16_t *__restrict__ h) {
  __shared__ int s_expert;
  __shared__ __attribute__((aligned(16))) uint16_t s_x[kDecXCols];
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
  const int gw = blockIdx.x * kDecWaves + wave;
  // the launch has exactly (k + 1) * f / U wavefronts, and the U * kDecWaves
  // (<= 8) units of a workgroup belong to one slot
  const int item = gw * U;
  const int slot = item / f, n = item % f;
  const bool shared = slot == k;
  // the top-k runs once per workgroup (wavefront 0; the other three wait at
  // the barrier instead of repeating it); its logits are loaded first, so
  // that their round trip overlaps the staging of x below instead of
  // following it
  float lv[kMaxPerLane];
  if (wave == 0 && !shared) wave_load_logits<kMaxPerLane>(logits, E, lv);
  // x's first kDecXCols columns, staged in LDS once per workgroup before the
  // routing (independent of it): each wavefront loads a quarter, 16 bytes per
  // lane, instead of every wavefront loading all of them from the caches
  {
    const int c = (wave * kWave + lane) * 8;
    if (c < d && c < kDecXCols) *(uint4 *)(s_x + c) = *(const uint4 *)(x + c);
  }
  // the selection, shared through LDS. A workgroup of slot j needs only the
  // first j + 1 selection rounds; the first workgroup of the last routed slot
  // takes all k and writes the token's ids and weights, at its end, so that
  // no store is outstanding at the barrier below.
  const bool writer = wave == 0 && !shared && slot == k - 1 && n == 0;  // wave-uniform
  int wid = 0;
  float ww = 0.f;
  if (wave == 0 && !shared) {
    int id;
    float l;
    wave_topk_loaded<kMaxPerLane>(lv, E, writer ? k : slot + 1, &id, &l);
    if (lane == slot) s_expert = id;
    if (writer) {
      const float m = __shfl(l, 0, kWave);
      const float e = lane < k ? expf(l - m) : 0.f;
      const float sum = wave_sum(e);
      wid = id;
      ww = e / sum;
    }
  }
  // x and the chosen expert are in LDS; the barrier waits for LDS operations
  // only, not for the global loads the other wavefronts may have in flight
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  // this lane's first 32 columns of x (lane * 32 < kDecXCols always)
  uint4 xv0[4] = {};
  if (lane * 32 < d) {
    const uint4 *xp = (const uint4 *)(s_x + lane * 32);
    xv0[0] = xp[0];
    xv0[1] = xp[1];
    xv0[2] = xp[2];
    xv0[3] = xp[3];
  }
  const int expert = shared ? 0 : __builtin_amdgcn_readfirstlane(s_expert);
  const W4 W = shared ? s13 : w13;
  const size_t rb = (size_t)expert * 2 * f;
  // gate rows n .. n + U - 1, then the up rows f + n ..
  size_t rows[2 * U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    rows[u] = rb + n + u;
    rows[U + u] = rb + f + n + u;
  }
  const int ngroups = d / kGroup;
  float acc[2 * U] = {};
  for (int c0 = lane * 32; c0 < d; c0 += kWave * 32) {
    uint4 c[2 * U];
    uint16_t sr[2 * U], br[2 * U];
#pragma unroll
    for (int r = 0; r < 2 * U; ++r) {
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
    for (int r = 0; r < 2 * U; ++r)
      acc[r] = dot32_any(c[r], (uint32_t)sr[r] | ((uint32_t)br[r] << 16), xv, acc[r]);
  }
#pragma unroll
  for (int r = 0; r < 2 * U; ++r) acc[r] = wave_sum_dpp(acc[r]);
  if (lane == 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) h[(size_t)slot * f + n + u] = to_bf16(silu_mul(acc[u], acc[U + u]));
  }
  if (writer && lane < k) {
    ids_out[lane] = wid;
    wts_out[lane] = ww;
  }
}

// Down projection with one wavefront per expert slot: the workgroup covers
// R = 64 / kLanesPerRow output rows for every slot (routed slots 0..k-1 and
// the shared expert at slot k), wavefront w taking slots w, w + W, ... of the
// W wavefronts. Each lane holds 32 columns of one row. The dequantisation of
// the (k + 1) rows is spread over (k + 1) wavefronts instead of one, and a
// wavefront reads its slot's h columns straight from memory, so nothing
// waits on an LDS stage: the chosen id (a scalar load, issued with the h
// loads) is the only round trip before the weight loads. Each wavefront
// leaves its weighted partial rows in LDS, summed over its L lanes; the
// first wavefront adds them in slot order and writes y.
template <int kLanesPerRow>
__global__ __launch_bounds__(1024) void decode_down_slots_kernel(
    const int32_t *__restrict__ ids, const float *__restrict__ wts,
    const uint16_t *__restrict__ h, W4 w2, W4 s2, int d, int f, int E, int k,
    float *__restrict__ y) {
  constexpr int R = kWave / kLanesPerRow;
  __shared__ float part[kDownSlotWaves][R];
  {
    const int t = blockIdx.y;  // token
    ids += (size_t)t * k;
    wts += (size_t)t * k;
    h += (size_t)t * (k + 1) * f;
    y += (size_t)t * d;
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int r = lane / kLanesPerRow, c0 = (lane % kLanesPerRow) * 32;
  const int m = blockIdx.x * R + r;  // grid = d / R rows of workgroups: m < d
  const int ngroups = f / kGroup;
  float acc = 0.f;
  for (int j = wave; j <= k; j += W) {
    const bool sh = j == k;
    // the slot's h columns do not depend on the id: their loads go out first
    // and stay in flight while the id's scalar load returns (the scheduling
    // barrier keeps the compiler from sinking them below its wait)
    const uint4 *hp = (const uint4 *)(h + (size_t)j * f + c0);
    const uint4 hv[4] = {hp[0], hp[1], hp[2], hp[3]};
    __builtin_amdgcn_sched_barrier(0);
    const int e = sh ? 0 : min(max(ids[j], 0), E - 1);  // in range for any ids
    const float wj = sh ? 1.f : wts[j];
    const W4 M = sh ? s2 : w2;
    const size_t row = (size_t)e * d + m;
    const uint4 cv = *(const uint4 *)(M.codes + row * (size_t)(f / 2) + c0 / 2);
    const uint32_t sv = M.scales[row * ngroups + c0 / kGroup];
    const uint32_t bv = M.biases[row * ngroups + c0 / kGroup];
    acc = fmaf(wj, dot32_any(cv, sv | (bv << 16), hv, 0.f), acc);
  }
  if constexpr (kLanesPerRow <= 16)
    acc = group_sum_dpp<kLanesPerRow>(acc);
  else
    acc = group_sum<kLanesPerRow>(acc);
  if (lane % kLanesPerRow == 0) part[wave][r] = acc;
  lds_barrier();
  if (wave == 0 && lane < R) {
    float sum = part[0][lane];
    for (int w = 1; w < W; ++w) sum += part[w][lane];
    y[blockIdx.x * R + lane] = sum;
  }
}

// Tokens up to which the layer runs these kernels, one grid row per token
// (each token's experts are streamed for it alone; the weights two tokens
// share come from the caches the second time).
constexpr int kDecodeMaxT = 16;

bool decode_supported(const Dims &dm) {
  const int lpr = dm.f / 32;
  const bool pow2 = lpr >= 2 && lpr <= 64 && (lpr & (lpr - 1)) == 0;
  return dm.T >= 1 && dm.T <= kDecodeMaxT && pow2;
}

template <int kLanesPerRow>
static void launch_down_slots(const Dims &dm, const int32_t *ids, const float *wts,
                              const uint16_t *h, const Weights &w, float *y, hipStream_t s) {
  constexpr int R = kWave / kLanesPerRow;
  // every slot its own wavefront at one token; with more tokens (grid rows)
  // each wavefront takes several slots
  const int per = dm.T <= 1 ? 1 : (dm.T <= 2 ? 2 : (dm.T <= 4 ? 4 : (dm.T <= 8 ? 5 : 9)));
  int waves = (dm.k + per) / per;
  if (waves > kDownSlotWaves) waves = kDownSlotWaves;
  decode_down_slots_kernel<kLanesPerRow><<<dim3(dm.d / R, dm.T), waves * kWave, 0, s>>>(
      ids, wts, h, w.w2, w.s2, dm.d, dm.f, dm.E, dm.k, y);
}

template <int kMaxPerLane, int U>
static void launch_gate_up_t(const Dims &dm, const uint16_t *x, const float *logits,
                             const Weights &w, int32_t *ids, float *wts, uint16_t *h, hipStream_t s) {
  const int blocks = (dm.k + 1) * dm.f / U / kDecWaves;  // f % 64 == 0: whole workgroups
  decode_gate_up_kernel<kMaxPerLane, U><<<dim3(blocks, dm.T), kDecWaves * 64, 0, s>>>(
      x, logits, w.w13, w.s13, dm.d, dm.f, dm.E, dm.k, ids, wts, h);
}

hipError_t launch_decode(const Dims &dm, const uint16_t *x, const float *logits, const Weights &w,
                         int32_t *ids, float *wts, uint16_t *h, float *y, hipStream_t s) {
  if (dm.T <= kDecOneUnitMaxT) {
    if (dm.E <= 64)
      launch_gate_up_t<1, 1>(dm, x, logits, w, ids, wts, h, s);
    else if (dm.E <= 256)
      launch_gate_up_t<4, 1>(dm, x, logits, w, ids, wts, h, s);
    else
      launch_gate_up_t<16, 1>(dm, x, logits, w, ids, wts, h, s);
  } else {
    if (dm.E <= 64)
      launch_gate_up_t<1, 2>(dm, x, logits, w, ids, wts, h, s);
    else if (dm.E <= 256)
      launch_gate_up_t<4, 2>(dm, x, logits, w, ids, wts, h, s);
    else
      launch_gate_up_t<16, 2>(dm, x, logits, w, ids, wts, h, s);
  }
  switch (dm.f / 32) {
    case 2: launch_down_slots<2>(dm, ids, wts, h, w, y, s); break;
    case 4: launch_down_slots<4>(dm, ids, wts, h, w, y, s); break;
    case 8: launch_down_slots<8>(dm, ids, wts, h, w, y, s); break;
    case 16: launch_down_slots<16>(dm, ids, wts, h, w, y, s); break;
    case 32: launch_down_slots<32>(dm, ids, wts, h, w, y, s); break;
    default: launch_down_slots<64>(dm, ids, wts, h, w, y, s); break;
  }
  return hipGetLastError();
}

}  // namespace moe
