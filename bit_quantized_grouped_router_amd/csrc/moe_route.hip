// Router: top-k experts per token by one wavefront, and the softmax over the
// k chosen logits (noticiai.com.br page on Lily, section "O modelo em tres
// formatos de carga": score 256 experts, keep eight).
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

template <int kMaxPerLane>
__global__ __launch_bounds__(256) void route_kernel(const float *__restrict__ logits, int T, int E,
                                                    int k, int32_t *__restrict__ ids,
                                                    float *__restrict__ wts) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  int id;
  float l;
  wave_topk<kMaxPerLane>(logits + (size_t)t * E, E, k, &id, &l);
  const float m = __shfl(l, 0, kWave);
  const float e = lane < k ? expf(l - m) : 0.f;
  const float s = wave_sum(e);
  if (lane < k) {
    ids[(size_t)t * k + lane] = id;
    wts[(size_t)t * k + lane] = e / s;
  }
}

hipError_t launch_route(const float *logits, int T, int E, int k, int32_t *ids, float *wts,
                        hipStream_t s) {
  const dim3 grid((T + 3) / 4), block(256);
  if (E <= 64)
    route_kernel<1><<<grid, block, 0, s>>>(logits, T, E, k, ids, wts);
  else if (E <= 256)
    route_kernel<4><<<grid, block, 0, s>>>(logits, T, E, k, ids, wts);
  else
    route_kernel<16><<<grid, block, 0, s>>>(logits, T, E, k, ids, wts);
  return hipGetLastError();
}

}  // namespace moe
