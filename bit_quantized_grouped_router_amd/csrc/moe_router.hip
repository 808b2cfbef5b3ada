// Router projection: every token's score for every expert, logits = x . Wr^T
// with bf16 operands and fp32 accumulation (noticiai.com.br page on Lily,
// section "O modelo em tres formatos de carga": the router scores the 256
// experts before eight are kept).
//
// gfx950 design
//   - a dense contraction (T x d times d x E), so it runs on the matrix
//     cores: v_mfma_f32_32x32x16_bf16, one 64-token x 64-expert tile per
//     workgroup, one 32 x 32 block per wavefront;
//   - eight wavefronts per workgroup, two per SIMD: wavefronts 0-3 sum the
//     first half of K and wavefronts 4-7 the second half at the same time,
//     each half with its own LDS ring, and the two partial tiles are added in
//     a fixed order (half 0 + half 1) at the end. The K chain each wavefront
//     walks is half as long, and each SIMD has a second wavefront to run
//     while the first waits;
//   - both operands go global -> LDS directly (global_load_lds_dwordx4, no
//     registers and no LDS stores), four K steps of 64 per half in flight;
//     each x row serves 64 experts and each router row 64 tokens; 16-byte
//     chunks are XOR-swizzled by row so that fragment reads of 16
//     consecutive rows hit distinct banks (each DMA lane fetches the chunk
//     that belongs at its contiguous LDS slot);
//   - rows past T or E re-read the last row (their results are never
//     stored), and steps past a half's end read through a buffer resource
//     with no records (zeros, no memory touched), so every step issues the
//     same loads and the wait counts stay exact;
//   - at T = 4096 the launch is 64 x 4 workgroups, one per CU, and the four
//     expert blocks of one token block land on one XCD (workgroup ids differ
//     by a multiple of 8), so they share that XCD's L2 copy of x.
#include "moe_launch.h"

namespace moe {

constexpr int kRtTile = 64;                    // tokens and experts per workgroup
constexpr int kRtKT = 64;                      // K per step: 128 bytes of a row
constexpr int kRtStages = 4;                   // ring depth per K half
constexpr int kRtOpBytes = kRtTile * 128;      // one operand's K step in LDS (8 KB)
constexpr int kRtStageBytes = 2 * kRtOpBytes;  // x and Wr of one step
constexpr int kRtLds = 2 * kRtStages * kRtStageBytes;  // both halves' rings: 128 KB

typedef __attribute__((address_space(3))) void rt_lds_void;

// byte offset of 16-byte chunk j (0..7) of tile row r in an operand's step
__device__ __forceinline__ uint32_t rt_swz(int r, int j) {
  return (uint32_t)(r * 128 + ((j ^ (r & 7) ^ ((r >> 3) & 1)) << 4));
}

#define RT_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (0x7 << 4) | (0xF << 8) | (((n) >> 4) << 14))

// Workgroup barrier after this wavefront's own LDS operations have completed
// (s_waitcnt lgkmcnt(0)). Unlike a release fence on LDS, it does not wait for
// the LDS DMA loads still in flight for later steps (those count in vmcnt,
// which the caller limits explicitly). The empty asm statements keep the
// compiler from moving memory accesses across it.
#define RT_BARRIER()                                                        \
  {                                                                         \
    asm volatile("" ::: "memory");                                          \
    __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14)); \
    __builtin_amdgcn_s_barrier();                                           \
    asm volatile("" ::: "memory");                                          \
  }

__global__ __launch_bounds__(512, 1) void router_logits_kernel(const uint16_t *__restrict__ x,
                                                            const uint16_t *__restrict__ wr,
                                                            int T, int d, int E,
                                                            float *__restrict__ logits) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = wave >> 2, wq = wave & 3;
  const int t0 = blockIdx.x * kRtTile, e0 = blockIdx.y * kRtTile;
  const int ksteps = d / kRtKT;
  const int kh0 = (ksteps + 1) / 2;                   // steps of half 0 (half 1 has the rest)
  const int kb = half ? kh0 : 0;                      // this half's first K step
  const int nsteps = half ? ksteps - kh0 : kh0;       // this half's steps (<= kh0)
  uint8_t *ring = lds + half * (kRtStages * kRtStageBytes);

  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc((void *)x, (short)0, (uint32_t)((size_t)T * d * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t wrr =
      __builtin_amdgcn_make_buffer_rsrc((void *)wr, (short)0, (uint32_t)((size_t)E * d * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc((void *)x, (short)0, 0, 0x00020000);

  // DMA: wavefront wq of a half fills tile rows 16 wq .. 16 wq + 15 of both
  // operands, 8 rows (1 KB) per instruction: lane l lands in row
  // r = 16 wq + 8 i + l / 8 at 16-byte slot l % 8, which holds logical chunk
  // (l % 8) ^ (r % 8) ^ ((r / 8) % 2) of the row
  uint32_t xo[2], wo[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 16 * wq + 8 * i + (lane >> 3);
    const uint32_t j = (uint32_t)((lane & 7) ^ (r & 7) ^ ((r >> 3) & 1));
    xo[i] = ((uint32_t)min(t0 + r, T - 1) * (uint32_t)d + (uint32_t)kb * kRtKT + j * 8u) * 2u;
    wo[i] = ((uint32_t)min(e0 + r, E - 1) * (uint32_t)d + (uint32_t)kb * kRtKT + j * 8u) * 2u;
  }
  // step s of this half (K step kb + s) into ring stage s % kRtStages
#define RT_DMA(s_)                                                                             \
  {                                                                                            \
    const bool ok_ = (s_) < nsteps;                                                            \
    const int so_ = ok_ ? (s_) * (kRtKT * 2) : 0;                                              \
    uint8_t *st_ = ring + ((s_) % kRtStages) * kRtStageBytes + 16 * wq * 128;                  \
    _Pragma("unroll") for (int i = 0; i < 2; ++i) {                                            \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ok_ ? xr : none, (rt_lds_void *)(st_ + i * 1024), \
                                               16, xo[i], so_, 0, 0);                          \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ok_ ? wrr : none,                               \
                                               (rt_lds_void *)(st_ + kRtOpBytes + i * 1024),   \
                                               16, wo[i], so_, 0, 0);                          \
    }                                                                                          \
  }

  // this wavefront's block: tokens am .. am+31 and experts bn .. bn+31 of the tile
  const int am = 32 * (wq & 1), bn = 32 * (wq >> 1);
  f32x16_t acc = f32x16_t{0};
  // K slice q of a step: lane half h supplies input columns 16 q + 8 h .. +7
  // of its row, for the x and the Wr fragment alike
#define RT_MMA(stage_)                                                                         \
  {                                                                                            \
    const uint8_t *sx_ = ring + (stage_) * kRtStageBytes;                                      \
    bf16x8_t a_[4], b_[4];                                                                     \
    _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                            \
      const int c_ = 2 * q + (lane >> 5);                                                      \
      a_[q] = *(const bf16x8_t *)(sx_ + rt_swz(am + (lane & 31), c_));                         \
      b_[q] = *(const bf16x8_t *)(sx_ + kRtOpBytes + rt_swz(bn + (lane & 31), c_));            \
    }                                                                                          \
    /* all eight reads in flight before the first MFMA waits on one */                        \
    asm volatile("" : "+v"(a_[0]), "+v"(a_[1]), "+v"(a_[2]), "+v"(a_[3]), "+v"(b_[0]),       \
                 "+v"(b_[1]), "+v"(b_[2]), "+v"(b_[3]));                                       \
    _Pragma("unroll") for (int q = 0; q < 4; ++q)                                              \
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_[q], b_[q], acc, 0, 0, 0);               \
  }

  // prologue: steps 0 .. kRtStages - 2 in flight
#pragma unroll
  for (int s = 0; s < kRtStages - 1; ++s) RT_DMA(s);
  // step s: wait for this wavefront's DMA of step s (the 4 instructions of
  // each of the kRtStages - 2 later steps may still be in flight), barrier
  // (every wavefront's share of step s is in LDS, and every wavefront's reads
  // of step s - 1 have completed: the barrier waits for its LDS reads), DMA
  // of step s + kRtStages - 1 into the stage step s - 1 used, then the step's
  // MFMAs. Both halves take kh0 steps, so they meet at every barrier; half 1
  // idles through its last step when K has an odd number of steps.
  for (int s = 0; s < kh0; ++s) {
    RT_WAIT_VMCNT(4 * (kRtStages - 2));
    RT_BARRIER();
    RT_DMA(s + kRtStages - 1);
    if (s < nsteps) RT_MMA(s % kRtStages);
  }
  RT_WAIT_VMCNT(0);
#undef RT_MMA
#undef RT_DMA

  // the two halves' partial tiles, added in a fixed order through LDS (no DMA
  // of any wavefront is in flight past this barrier)
  RT_BARRIER();
  float *red = (float *)lds + wq * (16 * 64);
  if (half == 1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) red[r * 64 + lane] = acc[r];
  }
  RT_BARRIER();
  if (half == 1) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] += red[r * 64 + lane];

  // C layout of the 32x32 MFMA: lane l holds column (expert) l % 32,
  // register r holds row (token) 8 (r / 4) + 4 (l / 32) + r % 4
  const int e = e0 + bn + (lane & 31);
  if (e >= E) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = t0 + am + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    if (t < T) logits[(size_t)t * E + e] = acc[r];
  }
}

// Up to kRtSmallT tokens the tiles above leave most of the chip idle (one
// workgroup per 64 tokens and 64 experts: 4 to 8 at E = 256) while each walks
// all of K, 8.4-8.7 us at any such T. There the scores are dot products on
// the VALU instead: one wavefront per expert and block of kRtTB tokens, each
// lane holding 8 columns of the router row and of each token's row per
// 16-byte chunk (4 chunks, 2048 columns, per pass), products summed in fp32
// with v_dot2_f32_bf16 and then over the wavefront with DPP, in a fixed
// order: 2.6 us at T = 1, 3.8 at 32, 7.9 at 128 (d = 2048, E = 256).
constexpr int kRtSmallT = 128;  // tokens up to which the dot-product kernel runs
constexpr int kRtTB = 4;        // tokens per wavefront
constexpr int kRtChunks = 4;    // 16-byte chunks per lane per pass

__device__ __forceinline__ float rt_dot8(uint4 a, uint4 b, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x),
                                        __builtin_bit_cast(bf16x2_t, b.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y),
                                        __builtin_bit_cast(bf16x2_t, b.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z),
                                        __builtin_bit_cast(bf16x2_t, b.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w),
                                        __builtin_bit_cast(bf16x2_t, b.w), acc, false);
  return acc;
}

__global__ __launch_bounds__(256) void router_logits_dot_kernel(const uint16_t *__restrict__ x,
                                                                const uint16_t *__restrict__ wr,
                                                                int T, int d, int E,
                                                                float *__restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ntb = (T + kRtTB - 1) / kRtTB;
  const int e = gw / ntb, t0 = (gw % ntb) * kRtTB;
  if (e >= E) return;  // wave-uniform: the launch rounds the wavefronts up to whole workgroups
  const uint16_t *wrow = wr + (size_t)e * d;
  float acc[kRtTB] = {};
  for (int c0 = 0; c0 < d; c0 += kWave * 8 * kRtChunks) {
    // the router row's chunks and every token's, all loads issued together;
    // chunks past d read nothing and add zero
    uint4 wv[kRtChunks], xv[kRtTB][kRtChunks];
#pragma unroll
    for (int i = 0; i < kRtChunks; ++i) {
      const int c = c0 + (lane + kWave * i) * 8;
      wv[i] = c < d ? *(const uint4 *)(wrow + c) : uint4{0, 0, 0, 0};
#pragma unroll
      for (int t = 0; t < kRtTB; ++t) {
        const int tt = min(t0 + t, T - 1);  // tokens past T re-read the last (never stored)
        xv[t][i] = c < d ? *(const uint4 *)(x + (size_t)tt * d + c) : uint4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int t = 0; t < kRtTB; ++t)
#pragma unroll
      for (int i = 0; i < kRtChunks; ++i) acc[t] = rt_dot8(wv[i], xv[t][i], acc[t]);
  }
#pragma unroll
  for (int t = 0; t < kRtTB; ++t) {
    const float v = wave_sum_dpp(acc[t]);
    if (lane == 0 && t0 + t < T) logits[(size_t)(t0 + t) * E + e] = v;
  }
}

// More than 64 KB of dynamic LDS needs a per-kernel opt-in (once per process).
static hipError_t router_setup() {
  static const hipError_t st = hipFuncSetAttribute(
      (const void *)router_logits_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kRtLds);
  return st;
}

hipError_t launch_router_logits(const uint16_t *x, const uint16_t *wr, int T, int d, int E,
                                float *logits, hipStream_t s) {
  if (T <= kRtSmallT) {
    const long long waves = (long long)E * ((T + kRtTB - 1) / kRtTB);
    router_logits_dot_kernel<<<(unsigned)((waves + 3) / 4), 256, 0, s>>>(x, wr, T, d, E, logits);
    return hipGetLastError();
  }
  if (const hipError_t e = router_setup()) return e;
  const dim3 grid((T + kRtTile - 1) / kRtTile, (E + kRtTile - 1) / kRtTile);
  router_logits_kernel<<<grid, 512, kRtLds, s>>>(x, wr, T, d, E, logits);
  return hipGetLastError();
}

}  // namespace moe
