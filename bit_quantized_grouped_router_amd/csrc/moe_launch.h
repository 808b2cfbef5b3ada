// Internal launchers of the gfx950 kernels; the C ABI layer (moe_api.hip)
// validates arguments and then calls these on the caller's stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_device.h"

namespace moe {

// Rows per tile of the block map, shared by both grouped GEMMs.
constexpr int kBlockM = 128;
// XCDs of the chip: the grouped GEMMs deal schedule position i to XCD i % 8
// (workgroups go to the XCDs round-robin), and the schedule is built for it.
constexpr int kXcds = 8;
// Largest input width of a grouped GEMM: a tile keeps the scales and biases
// of its 256 weight rows for all K/64 groups in LDS, next to 64 KB of
// activation buffers (1 KB per group, 160 KB of LDS per CU).
constexpr int kGemmMaxK = 6144;
// Tokens per block of the permutation pipeline.
constexpr int kPermTokens = 256;

struct Dims {
  int T, d, f, E, k;
};

struct Weights {
  W4 w13, w2, s13, s2;
};

inline int tile_capacity(const Dims &dm) {
  const long long tk = (long long)dm.T * dm.k;
  const long long nonempty = tk < dm.E ? tk : dm.E;
  long long routed = (tk + nonempty * (kBlockM - 1)) / kBlockM;
  if (routed > tk) routed = tk;
  return (int)(routed + (dm.T + kBlockM - 1) / kBlockM);
}

inline int perm_blocks(int T) { return (T + kPermTokens - 1) / kPermTokens; }

hipError_t launch_route(const float *logits, int T, int E, int k, int32_t *ids, float *wts,
                        hipStream_t s);

hipError_t launch_router_logits(const uint16_t *x, const uint16_t *wr, int T, int d, int E,
                                float *logits, hipStream_t s);

// block_counts: scratch int32 [perm_blocks(T)][E]
hipError_t launch_permute(const Dims &dm, const int32_t *ids, int32_t *counts, int32_t *offsets,
                          int32_t *sorted_token, int32_t *row_of, int32_t *tile_map,
                          int32_t *num_tiles, int32_t *block_counts, hipStream_t s);

// moe_route then moe_permute; up to 64 tokens in one single-workgroup launch.
hipError_t launch_route_permute(const Dims &dm, const float *logits, int32_t *ids, float *wts,
                                int32_t *counts, int32_t *offsets, int32_t *sorted_token,
                                int32_t *row_of, int32_t *tile_map, int32_t *num_tiles,
                                int32_t *block_counts, hipStream_t s);

// Small batches: the same projections with a few weight rows per wavefront
// and dot products on the VALU (launch_gate_up / launch_down call these when
// gemv_supported).
bool gemv_supported(const Dims &dm);
hipError_t launch_gate_up_gemv(const Dims &dm, const uint16_t *x, const Weights &w,
                               const int32_t *sorted_token, const int32_t *tile_map,
                               const int32_t *num_tiles, uint16_t *h, hipStream_t s);
hipError_t launch_down_gemv(const Dims &dm, const uint16_t *h, const Weights &w,
                            const int32_t *tile_map, const int32_t *num_tiles,
                            uint16_t *o_routed, float *o_shared, hipStream_t s);

hipError_t launch_gate_up(const Dims &dm, const uint16_t *x, const Weights &w,
                          const int32_t *sorted_token, const int32_t *tile_map,
                          const int32_t *num_tiles, uint16_t *h, hipStream_t s);

hipError_t launch_down(const Dims &dm, const uint16_t *h, const Weights &w,
                       const int32_t *tile_map, const int32_t *num_tiles, uint16_t *o_routed,
                       float *o_shared, hipStream_t s);

hipError_t launch_combine(const Dims &dm, const uint16_t *o_routed, const float *o_shared,
                          const float *wts, const int32_t *row_of, float *y, hipStream_t s);

// Batch-1 decode. ids/wts: int32/fp32 [k]; h: bf16 [(k+1)][f].
bool decode_supported(const Dims &dm);
hipError_t launch_decode(const Dims &dm, const uint16_t *x, const float *logits, const Weights &w,
                         int32_t *ids, float *wts, uint16_t *h, float *y, hipStream_t s);

hipError_t launch_dequant(const W4 &m, int rows, int cols, uint16_t *out, hipStream_t s);

}  // namespace moe
