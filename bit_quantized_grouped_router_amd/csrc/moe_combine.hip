// Weighted unpermute and combine with the shared expert (noticiai.com.br page
// on Lily, section "O modelo em tres formatos de carga": every token also
// goes through one shared expert; it is added with weight 1):
//   y[t] = o_shared[t] + sum_j w[t][j] * o_routed[row_of[t*k + j]]   (fp32)
// HBM bound: each workgroup owns one token row; each thread 8 columns, read
// as 16-byte bf16 vectors of the routed rows and 32-byte fp32 vectors of the
// shared row.
#include "moe_launch.h"

namespace moe {

template <int kMaxK>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t *__restrict__ o_routed,
                                                      const float *__restrict__ o_shared,
                                                      const float *__restrict__ wts,
                                                      const int32_t *__restrict__ row_of, int d,
                                                      int k, float *__restrict__ y) {
  const int t = blockIdx.x;
  // the token's rows and weights: unconditional (clamped) loads, issued together
  int row[kMaxK];
  float wj[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    const int jj = j < k ? j : k - 1;
    row[j] = row_of[(size_t)t * k + jj];
    wj[j] = j < k ? wts[(size_t)t * k + jj] : 0.f;
  }
  for (int c0 = threadIdx.x * 8; c0 < d; c0 += blockDim.x * 8) {
    const float4 s0 = *(const float4 *)(o_shared + (size_t)t * d + c0);
    const float4 s1 = *(const float4 *)(o_shared + (size_t)t * d + c0 + 4);
    uint4 v[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) v[j] = *(const uint4 *)(o_routed + (size_t)row[j] * d + c0);
    float acc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j >= k) continue;
      const uint32_t u[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(wj[j], bf16_to_f32(u[q] & 0xFFFFu), acc[2 * q]);
        acc[2 * q + 1] = fmaf(wj[j], bf16_to_f32(u[q] >> 16), acc[2 * q + 1]);
      }
    }
    *(float4 *)(y + (size_t)t * d + c0) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *(float4 *)(y + (size_t)t * d + c0 + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

hipError_t launch_combine(const Dims &dm, const uint16_t *o_routed, const float *o_shared,
                          const float *wts, const int32_t *row_of, float *y, hipStream_t s) {
  if (dm.k <= 8)
    combine_kernel<8><<<dm.T, 256, 0, s>>>(o_routed, o_shared, wts, row_of, dm.d, dm.k, y);
  else
    combine_kernel<32><<<dm.T, 256, 0, s>>>(o_routed, o_shared, wts, row_of, dm.d, dm.k, y);
  return hipGetLastError();
}

}  // namespace moe
