// Grouped expert GEMMs with the int4-g64 dequantisation fused into the tile
// (noticiai.com.br page on Lily, section "Prefill e decode: onde estao os
// ganhos": the tensor units take bf16, so the 4-bit weights are rebuilt to
// bf16 one tile at a time in on-chip memory, with fp32 accumulation).
//
// gfx950 design
//   - one workgroup = 4 wavefronts = one (tile of <= 128 permuted rows) x
//     (N block) of the output; the tile comes from the block map;
//   - per K step of 64 (exactly one quantisation group per weight row) the
//     activation rows are copied to LDS and the weight rows are loaded as
//     packed codes + one bf16 scale/bias, dequantised by the VALU and stored
//     to LDS as bf16; global loads of step k+1 are in flight while the
//     MFMAs of step k run;
//   - v_mfma_f32_32x32x16_bf16, fp32 accumulators; the 2x2 waves each own a
//     64-row slab; 32-row slabs past the tile's last row skip their MFMAs;
//   - LDS rows are padded to 144 bytes so that the 16-byte fragment reads of
//     32 consecutive rows fall on distinct banks;
//   - the grid is sized from the block map's capacity (a host-side bound);
//     workgroups past num_tiles (read on the device) exit at once, so no
//     host synchronisation is needed; block ids are remapped so that the
//     N blocks of one tile, and neighbouring tiles of one expert, run on the
//     same XCD and share its L2.
#include "moe_launch.h"

namespace moe {

constexpr int kKT = 64;             // K per step: one quantisation group
constexpr int kLdsStride = kKT + 8; // bf16 elements per LDS row (144 B)
constexpr int kGuUnits = 64;        // gate/up: intermediate units per workgroup (128 weight rows)
constexpr int kDnCols = 128;        // down: output columns per workgroup
constexpr int kXcds = 8;

__device__ __forceinline__ int xcd_remap(int bid, int grid) {
  // workgroups are dispatched round-robin over the XCDs; give XCD x the
  // contiguous logical range [x*grid/8, (x+1)*grid/8)
  const int per = grid / kXcds;
  return (bid % kXcds) * per + bid / kXcds;
}

__device__ __forceinline__ bf16x8_t lds_frag(const uint16_t *p) {
  return __builtin_bit_cast(bf16x8_t, *(const uint4 *)p);
}

// ------------------------------------------------------------------ gate/up

__global__ __launch_bounds__(256, 2) void gate_up_kernel(
    const uint16_t *__restrict__ x, W4 w13, W4 s13, const int32_t *__restrict__ sorted_token,
    const int32_t *__restrict__ tile_map, const int32_t *__restrict__ num_tiles_p,
    uint16_t *__restrict__ h, int T, int d, int f, int E, int k, int grid) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kBlockM * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2 * kGuUnits * kLdsStride];

  const int nblk = f / kGuUnits;
  const int logical = xcd_remap(blockIdx.x, grid);
  const int tile = logical / nblk;
  if (tile >= *num_tiles_p) return;
  const int n0 = (logical % nblk) * kGuUnits;
  const int4 tm = *(const int4 *)(tile_map + 4 * (size_t)tile);
  const int g = tm.x, row_begin = tm.y, row_end = tm.z;
  const bool shared = g >= E;
  const W4 W = shared ? s13 : w13;
  const size_t ex = shared ? 0 : (size_t)g;
  const int tid = threadIdx.x;
  const int TK = T * k;

  // activation rows: 4 chunks of 16 B per thread per K step
  const uint16_t *a_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (tid >> 3) + 32 * i;
    const int p = row_begin + row;
    a_src[i] = nullptr;
    if (p < row_end) {
      int tok = shared ? p - TK : sorted_token[p];
      tok = tok < 0 ? 0 : (tok >= T ? T - 1 : tok);  // in range even for malformed routing
      a_src[i] = x + (size_t)tok * d + (tid & 7) * 8;
    }
  }
  // weight rows: 2 threads per row, 32 columns (16 B of codes) each
  const int wr = tid >> 1, half = tid & 1;
  const int grow = wr < kGuUnits ? n0 + wr : f + n0 + (wr - kGuUnits);
  const uint8_t *c_src = W.codes + (ex * 2 * f + grow) * (size_t)(d / 2) + half * 16;
  const uint16_t *s_src = W.scales + (ex * 2 * f + grow) * (size_t)(d / kGroup);
  const uint16_t *b_src = W.biases + (ex * 2 * f + grow) * (size_t)(d / kGroup);

  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int rows = row_end - row_begin;
  const bool act0 = wm * 64 < rows, act1 = wm * 64 + 32 < rows;

  f32x16_t accg0 = {0}, accg1 = {0}, accu0 = {0}, accu1 = {0};
  uint4 ar[4], cr;
  uint32_t sb;

  auto load = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ar[i] = a_src[i] ? *(const uint4 *)(a_src[i] + kt * kKT) : make_uint4(0, 0, 0, 0);
    cr = *(const uint4 *)(c_src + kt * (kKT / 2));
    sb = (uint32_t)s_src[kt] | ((uint32_t)b_src[kt] << 16);
  };

  const int ksteps = d / kKT;
  load(0);
  for (int kt = 0; kt < ksteps; ++kt) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(uint4 *)(As + ((tid >> 3) + 32 * i) * kLdsStride + (tid & 7) * 8) = ar[i];
    {
      const float s = bf16_to_f32(sb & 0xFFFFu), b = bf16_to_f32(sb >> 16);
      uint16_t *dst = Bs + wr * kLdsStride + half * 32;
      *(uint4 *)(dst + 0) = dequant8(cr.x, s, b);
      *(uint4 *)(dst + 8) = dequant8(cr.y, s, b);
      *(uint4 *)(dst + 16) = dequant8(cr.z, s, b);
      *(uint4 *)(dst + 24) = dequant8(cr.w, s, b);
    }
    __syncthreads();
    if (kt + 1 < ksteps) load(kt + 1);
#pragma unroll
    for (int ks = 0; ks < kKT / 16; ++ks) {
      const int ko = ks * 16 + (lane >> 5) * 8;
      const bf16x8_t bg = lds_frag(Bs + (wn * 32 + (lane & 31)) * kLdsStride + ko);
      const bf16x8_t bu = lds_frag(Bs + (kGuUnits + wn * 32 + (lane & 31)) * kLdsStride + ko);
      if (act0) {
        const bf16x8_t a = lds_frag(As + (wm * 64 + (lane & 31)) * kLdsStride + ko);
        accg0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bg, accg0, 0, 0, 0);
        accu0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bu, accu0, 0, 0, 0);
      }
      if (act1) {
        const bf16x8_t a = lds_frag(As + (wm * 64 + 32 + (lane & 31)) * kLdsStride + ko);
        accg1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bg, accg1, 0, 0, 0);
        accu1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bu, accu1, 0, 0, 0);
      }
    }
  }

  // epilogue: h = bf16(silu(gate) * up); C layout of the 32x32 MFMA: lane l
  // holds column l%32, register r holds row 8*(r/4) + 4*(l/32) + r%4
  const int unit = n0 + wn * 32 + (lane & 31);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const f32x16_t &ag = mb ? accg1 : accg0;
    const f32x16_t &au = mb ? accu1 : accu0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int p = row_begin + wm * 64 + mb * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      if (p < row_end) h[(size_t)p * f + unit] = to_bf16(silu_mul(ag[r], au[r]));
    }
  }
}

// ------------------------------------------------------------------ down

__global__ __launch_bounds__(256, 2) void down_kernel(
    const uint16_t *__restrict__ h, W4 w2, W4 s2, const int32_t *__restrict__ tile_map,
    const int32_t *__restrict__ num_tiles_p, uint16_t *__restrict__ o_routed,
    float *__restrict__ o_shared, int T, int d, int f, int E, int k, int grid) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kBlockM * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kDnCols * kLdsStride];

  const int nblk = (d + kDnCols - 1) / kDnCols;
  const int logical = xcd_remap(blockIdx.x, grid);
  const int tile = logical / nblk;
  if (tile >= *num_tiles_p) return;
  const int n0 = (logical % nblk) * kDnCols;
  const int4 tm = *(const int4 *)(tile_map + 4 * (size_t)tile);
  const int g = tm.x, row_begin = tm.y, row_end = tm.z;
  const bool shared = g >= E;
  const W4 W = shared ? s2 : w2;
  const size_t ex = shared ? 0 : (size_t)g;
  const int tid = threadIdx.x;
  const int TK = T * k;

  const uint16_t *a_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = row_begin + (tid >> 3) + 32 * i;
    a_src[i] = p < row_end ? h + (size_t)p * f + (tid & 7) * 8 : nullptr;
  }
  const int wr = tid >> 1, half = tid & 1;
  const int grow = n0 + wr;
  const bool wvalid = grow < d;
  const size_t wrow = ex * (size_t)d + (wvalid ? grow : 0);
  const uint8_t *c_src = W.codes + wrow * (size_t)(f / 2) + half * 16;
  const uint16_t *s_src = W.scales + wrow * (size_t)(f / kGroup);
  const uint16_t *b_src = W.biases + wrow * (size_t)(f / kGroup);

  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int rows = row_end - row_begin;
  const bool act0 = wm * 64 < rows, act1 = wm * 64 + 32 < rows;

  f32x16_t acc00 = {0}, acc01 = {0}, acc10 = {0}, acc11 = {0};
  uint4 ar[4], cr;
  uint32_t sb;

  auto load = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ar[i] = a_src[i] ? *(const uint4 *)(a_src[i] + kt * kKT) : make_uint4(0, 0, 0, 0);
    if (wvalid) {
      cr = *(const uint4 *)(c_src + kt * (kKT / 2));
      sb = (uint32_t)s_src[kt] | ((uint32_t)b_src[kt] << 16);
    } else {
      cr = make_uint4(0, 0, 0, 0);
      sb = 0u;
    }
  };

  const int ksteps = f / kKT;
  load(0);
  for (int kt = 0; kt < ksteps; ++kt) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(uint4 *)(As + ((tid >> 3) + 32 * i) * kLdsStride + (tid & 7) * 8) = ar[i];
    {
      const float s = bf16_to_f32(sb & 0xFFFFu), b = bf16_to_f32(sb >> 16);
      uint16_t *dst = Bs + wr * kLdsStride + half * 32;
      *(uint4 *)(dst + 0) = dequant8(cr.x, s, b);
      *(uint4 *)(dst + 8) = dequant8(cr.y, s, b);
      *(uint4 *)(dst + 16) = dequant8(cr.z, s, b);
      *(uint4 *)(dst + 24) = dequant8(cr.w, s, b);
    }
    __syncthreads();
    if (kt + 1 < ksteps) load(kt + 1);
#pragma unroll
    for (int ks = 0; ks < kKT / 16; ++ks) {
      const int ko = ks * 16 + (lane >> 5) * 8;
      const bf16x8_t b0 = lds_frag(Bs + (wn * 64 + (lane & 31)) * kLdsStride + ko);
      const bf16x8_t b1 = lds_frag(Bs + (wn * 64 + 32 + (lane & 31)) * kLdsStride + ko);
      if (act0) {
        const bf16x8_t a = lds_frag(As + (wm * 64 + (lane & 31)) * kLdsStride + ko);
        acc00 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, acc00, 0, 0, 0);
        acc01 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, acc01, 0, 0, 0);
      }
      if (act1) {
        const bf16x8_t a = lds_frag(As + (wm * 64 + 32 + (lane & 31)) * kLdsStride + ko);
        acc10 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, acc10, 0, 0, 0);
        acc11 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, acc11, 0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const f32x16_t &acc = mb ? (nb ? acc11 : acc10) : (nb ? acc01 : acc00);
      const int col = n0 + wn * 64 + nb * 32 + (lane & 31);
      if (col >= d) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int p = row_begin + wm * 64 + mb * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (p >= row_end) continue;
        if (shared)
          o_shared[(size_t)(p - TK) * d + col] = acc[r];
        else
          o_routed[(size_t)p * d + col] = to_bf16(acc[r]);
      }
    }
  }
}

static int round_up8(long long n) { return (int)((n + kXcds - 1) / kXcds * kXcds); }

hipError_t launch_gate_up(const Dims &dm, const uint16_t *x, const Weights &w,
                          const int32_t *sorted_token, const int32_t *tile_map,
                          const int32_t *num_tiles, uint16_t *h, hipStream_t s) {
  const int grid = round_up8((long long)tile_capacity(dm) * (dm.f / kGuUnits));
  gate_up_kernel<<<grid, 256, 0, s>>>(x, w.w13, w.s13, sorted_token, tile_map, num_tiles, h,
                                      dm.T, dm.d, dm.f, dm.E, dm.k, grid);
  return hipGetLastError();
}

hipError_t launch_down(const Dims &dm, const uint16_t *h, const Weights &w,
                       const int32_t *tile_map, const int32_t *num_tiles, uint16_t *o_routed,
                       float *o_shared, hipStream_t s) {
  const int nblk = (dm.d + kDnCols - 1) / kDnCols;
  const int grid = round_up8((long long)tile_capacity(dm) * nblk);
  down_kernel<<<grid, 256, 0, s>>>(h, w.w2, w.s2, tile_map, num_tiles, o_routed, o_shared, dm.T,
                                   dm.d, dm.f, dm.E, dm.k, grid);
  return hipGetLastError();
}

// ------------------------------------------------------------------ dequant (inspection)

__global__ __launch_bounds__(256) void dequant_kernel(W4 m, int rows, int cols,
                                                      uint16_t *__restrict__ out) {
  const long long words = (long long)rows * cols / 8;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < words;
       i += (long long)gridDim.x * blockDim.x) {
    const long long col0 = (i * 8) % cols, row = (i * 8) / cols;
    const uint32_t c = ((const uint32_t *)m.codes)[i];
    const long long gi = row * (cols / kGroup) + col0 / kGroup;
    const uint4 r = dequant8(c, bf16_to_f32(m.scales[gi]), bf16_to_f32(m.biases[gi]));
    *(uint4 *)(out + i * 8) = r;
  }
}

hipError_t launch_dequant(const W4 &m, int rows, int cols, uint16_t *out, hipStream_t s) {
  const long long words = (long long)rows * cols / 8;
  long long blocks = (words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  dequant_kernel<<<(int)blocks, 256, 0, s>>>(m, rows, cols, out);
  return hipGetLastError();
}

}  // namespace moe
