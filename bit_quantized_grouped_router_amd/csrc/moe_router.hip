// Router projection: every token's score for every expert, logits = x . Wr^T
// with bf16 operands and fp32 accumulation (noticiai.com.br page on Lily,
// section "O modelo em tres formatos de carga": the router scores the 256
// experts before eight are kept).
//
// gfx950 design
//   - a dense contraction (T x d times d x E), so it runs on the matrix
//     cores: v_mfma_f32_32x32x16_bf16, one 32 x 32 block per wavefront, four
//     wavefronts per 64-token x 64-expert workgroup tile;
//   - both operands pass through LDS once per workgroup (each x row serves 64
//     experts, each router row 64 tokens), 16-byte chunks XOR-swizzled by row
//     so that fragment reads of 16 consecutive rows hit distinct banks;
//   - the loop is bound by global-load latency, not arithmetic (4 MFMAs per
//     64-wide K step per wavefront), so eight K steps (32 KB per workgroup)
//     are kept in flight in registers, loaded through buffer resources; steps
//     past the last one read through a resource with no records, which
//     returns zeros without touching memory, so every iteration issues the
//     same loads and the wait counts stay exact;
//   - with 64 tokens per tile the T = 4096 launch is 64 x 4 workgroups, and
//     the four expert blocks of one token block land on one XCD (workgroup
//     ids differ by a multiple of 8), so they share that XCD's L2 copy of x.
#include "moe_launch.h"

namespace moe {

constexpr int kRtTile = 64;              // tokens and experts per workgroup
constexpr int kRtKT = 64;                // K per step: 128 bytes of a row
constexpr int kRtDepth = 8;              // K steps in flight in registers
constexpr int kRtStage = kRtTile * 128;  // bytes of one operand's K step in LDS

typedef uint32_t rt_u32x4_t __attribute__((ext_vector_type(4)));

// byte offset of 16-byte chunk j (0..7) of tile row r in a stage
__device__ __forceinline__ uint32_t rt_swz(int r, int j) {
  return (uint32_t)(r * 128 + ((j ^ (r & 7) ^ ((r >> 3) & 1)) << 4));
}

__global__ __launch_bounds__(256, 1) void router_logits_kernel(const uint16_t *__restrict__ x,
                                                            const uint16_t *__restrict__ wr,
                                                            int T, int d, int E,
                                                            float *__restrict__ logits) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kRtStage];  // [buffer][x, Wr]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.x * kRtTile, e0 = blockIdx.y * kRtTile;
  const int ksteps = d / kRtKT;

  // loads: thread tid fetches 16-byte chunk tid % 8 of tile rows tid / 8 and
  // tid / 8 + 32, of x and of Wr; rows past T or E re-read the last row (their
  // results are never stored)
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc((void *)x, (short)0, (uint32_t)((size_t)T * d * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t wrr =
      __builtin_amdgcn_make_buffer_rsrc((void *)wr, (short)0, (uint32_t)((size_t)E * d * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc((void *)x, (short)0, 0, 0x00020000);
  const int lj = tid & 7, lr = tid >> 3;
  uint32_t xo[2], wo[2], so[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = lr + 32 * i;
    xo[i] = ((uint32_t)min(t0 + r, T - 1) * (uint32_t)d + (uint32_t)lj * 8u) * 2u;
    wo[i] = ((uint32_t)min(e0 + r, E - 1) * (uint32_t)d + (uint32_t)lj * 8u) * 2u;
    so[i] = rt_swz(r, lj);
  }
  rt_u32x4_t ra[kRtDepth][2], rb[kRtDepth][2];

#define RT_LOAD(slot_, kt_)                                                                   \
  {                                                                                           \
    const bool ok_ = (kt_) < ksteps;                                                          \
    const int so_ = ok_ ? (kt_) * (kRtKT * 2) : 0;                                            \
    _Pragma("unroll") for (int i = 0; i < 2; ++i) {                                           \
      ra[slot_][i] = __builtin_bit_cast(                                                      \
          rt_u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ok_ ? xr : none, xo[i], so_, 0));  \
      rb[slot_][i] = __builtin_bit_cast(                                                      \
          rt_u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ok_ ? wrr : none, wo[i], so_, 0)); \
    }                                                                                         \
  }
#define RT_STORE(slot_, buf_)                                               \
  {                                                                         \
    _Pragma("unroll") for (int i = 0; i < 2; ++i) {                         \
      *(rt_u32x4_t *)(&lds[buf_][0][0] + so[i]) = ra[slot_][i];             \
      *(rt_u32x4_t *)(&lds[buf_][1][0] + so[i]) = rb[slot_][i];             \
    }                                                                       \
  }

  // this wavefront's block: tokens am .. am+31 and experts bn .. bn+31 of the tile
  const int am = 32 * (wave & 1), bn = 32 * (wave >> 1);
  f32x16_t acc = f32x16_t{0};
  // K slice s of a step: lane half h supplies input columns 16 s + 8 h .. +7
  // of its row, for the x and the Wr fragment alike
#define RT_MMA(buf_)                                                                           \
  {                                                                                            \
    bf16x8_t a_[4], b_[4];                                                                     \
    _Pragma("unroll") for (int s = 0; s < 4; ++s) {                                            \
      const int c_ = 2 * s + (lane >> 5);                                                      \
      a_[s] = *(const bf16x8_t *)(&lds[buf_][0][0] + rt_swz(am + (lane & 31), c_));           \
      b_[s] = *(const bf16x8_t *)(&lds[buf_][1][0] + rt_swz(bn + (lane & 31), c_));           \
    }                                                                                          \
    /* all eight reads in flight before the first MFMA waits on one */                        \
    asm volatile("" : "+v"(a_[0]), "+v"(a_[1]), "+v"(a_[2]), "+v"(a_[3]), "+v"(b_[0]),       \
                 "+v"(b_[1]), "+v"(b_[2]), "+v"(b_[3]));                                       \
    _Pragma("unroll") for (int s = 0; s < 4; ++s)                                              \
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_[s], b_[s], acc, 0, 0, 0);               \
  }

  // step kt (slot kt % 8) is in LDS buffer kt % 2 when its MFMAs run; meanwhile
  // step kt + 1 goes from registers into the other buffer (read last in step
  // kt - 1, before the previous barrier) and step kt + 8 is loaded into the
  // registers step kt has vacated
#define RT_STEP(kt_, s_)                              \
  {                                                   \
    if ((kt_) < ksteps) RT_MMA((s_) & 1);             \
    RT_STORE(((s_) + 1) % kRtDepth, ((s_) + 1) & 1);  \
    RT_LOAD((s_), (kt_) + kRtDepth);                  \
    __syncthreads();                                  \
  }

#pragma unroll
  for (int s = 0; s < kRtDepth; ++s) RT_LOAD(s, s);
  RT_STORE(0, 0);
  __syncthreads();
  for (int kt = 0; kt < ksteps; kt += kRtDepth) {
    RT_STEP(kt, 0);
    RT_STEP(kt + 1, 1);
    RT_STEP(kt + 2, 2);
    RT_STEP(kt + 3, 3);
    RT_STEP(kt + 4, 4);
    RT_STEP(kt + 5, 5);
    RT_STEP(kt + 6, 6);
    RT_STEP(kt + 7, 7);
  }
#undef RT_STEP
#undef RT_MMA
#undef RT_STORE
#undef RT_LOAD

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

hipError_t launch_router_logits(const uint16_t *x, const uint16_t *wr, int T, int d, int E,
                                float *logits, hipStream_t s) {
  const dim3 grid((T + kRtTile - 1) / kRtTile, (E + kRtTile - 1) / kRtTile);
  router_logits_kernel<<<grid, 256, 0, s>>>(x, wr, T, d, E, logits);
  return hipGetLastError();
}

}  // namespace moe
