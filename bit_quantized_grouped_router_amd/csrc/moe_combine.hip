// Weighted unpermute and combine with the shared expert (noticiai.com.br page
// on Lily, section "O modelo em tres formatos de carga": every token also
// goes through one shared expert; it is added with weight 1):
//   y[t] = o_shared[t] + sum_j w[t][j] * o_routed[row_of[t*k + j]]   (fp32)
// HBM bound: each workgroup owns one token row; each thread 8 columns, read
// as 16-byte bf16 vectors of the routed rows and 32-byte fp32 vectors of the
// shared row.
#include "moe_launch.h"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t *__restrict__ o_routed,
                                                      const float *__restrict__ o_shared,
                                                      const float *__restrict__ wts,
                                                      const int32_t *__restrict__ row_of, int d,
                                                      int k, float *__restrict__ y) {
  const int t = blockIdx.x;
  __shared__ int s_row[32];
  __shared__ float s_w[32];
  if (threadIdx.x < k) {
    s_row[threadIdx.x] = row_of[(size_t)t * k + threadIdx.x];
    s_w[threadIdx.x] = wts[(size_t)t * k + threadIdx.x];
  }
  __syncthreads();
  for (int c0 = threadIdx.x * 8; c0 < d; c0 += blockDim.x * 8) {
    const float4 s0 = *(const float4 *)(o_shared + (size_t)t * d + c0);
    const float4 s1 = *(const float4 *)(o_shared + (size_t)t * d + c0 + 4);
    float acc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    for (int j = 0; j < k; ++j) {
      const uint4 v = *(const uint4 *)(o_routed + (size_t)s_row[j] * d + c0);
      const float wj = s_w[j];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(wj, bf16_to_f32(u[q] & 0xFFFFu), acc[2 * q]);
        acc[2 * q + 1] = fmaf(wj, bf16_to_f32(u[q] >> 16), acc[2 * q + 1]);
      }
    }
    *(float4 *)(y + (size_t)t * d + c0) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *(float4 *)(y + (size_t)t * d + c0 + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

hipError_t launch_combine(const Dims &dm, const uint16_t *o_routed, const float *o_shared,
                          const float *wts, const int32_t *row_of, float *y, hipStream_t s) {
  combine_kernel<<<dm.T, 256, 0, s>>>(o_routed, o_shared, wts, row_of, dm.d, dm.k, y);
  return hipGetLastError();
}

}  // namespace moe
