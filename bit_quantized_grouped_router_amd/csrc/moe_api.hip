// C ABI of the int4-g64 grouped MoE layer: host-side validation, workspace
// carving and launch sequencing on the caller's stream. No allocation, no
// host synchronisation, no exceptions across the interface.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "../../include/moe_w4.h"
#include "moe_launch.h"

using namespace moe;

namespace {

thread_local int32_t g_last_hip_error = 0;

moe_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip_error = (int32_t)e;
  return MOE_E_HIP;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// MOE_OK, or the first failing check of a pointer that must be present.
moe_status check_ptr(const void *p) {
  if (p == nullptr) return MOE_E_INVALID;
  if (!aligned16(p)) return MOE_E_ALIGN;
  return MOE_OK;
}

#define MOE_TRY(expr)                   \
  do {                                  \
    const moe_status st_ = (expr);      \
    if (st_ != MOE_OK) return st_;      \
  } while (0)

moe_status check_dims(const moe_dims *dm) {
  if (dm == nullptr) return MOE_E_INVALID;
  if (dm->T < 0 || dm->d <= 0 || dm->f <= 0 || dm->E <= 0 || dm->k <= 0 || dm->f_shared <= 0)
    return MOE_E_INVALID;
  if (dm->k > dm->E) return MOE_E_INVALID;
  // a shared expert of another width is a valid layer these kernels do not run
  if (dm->f_shared != dm->f) return MOE_E_UNSUPPORTED;
  if (dm->d % kGroup != 0 || dm->f % kGroup != 0) return MOE_E_UNSUPPORTED;
  if (dm->E > 1024 || dm->k > 32) return MOE_E_UNSUPPORTED;
  if (dm->d > kGemmMaxK || dm->f > kGemmMaxK) return MOE_E_UNSUPPORTED;
  const long long rows = (long long)dm->T * (dm->k + 1);
  const long long big = dm->d > 2 * dm->f ? dm->d : 2 * dm->f;
  if (rows * big >= (1ll << 31) || (long long)dm->E * 2 * dm->f * dm->d >= (1ll << 34))
    return MOE_E_UNSUPPORTED;
  return MOE_OK;
}

moe_status check_matrix(const moe_w4_matrix &m) {
  MOE_TRY(check_ptr(m.codes));
  MOE_TRY(check_ptr(m.scales));
  MOE_TRY(check_ptr(m.biases));
  return MOE_OK;
}

moe_status check_weights(const moe_w4_weights *w, bool up, bool down) {
  if (w == nullptr) return MOE_E_INVALID;
  if (up) {
    MOE_TRY(check_matrix(w->w13));
    MOE_TRY(check_matrix(w->s13));
  }
  if (down) {
    MOE_TRY(check_matrix(w->w2));
    MOE_TRY(check_matrix(w->s2));
  }
  return MOE_OK;
}

// Shapes the router projection takes: d a multiple of 64 (one K step), E up to
// 1024, and x, Wr and the logits each under 2^31 elements.
moe_status check_router_dims(int32_t T, int32_t d, int32_t E) {
  if (T < 0 || d <= 0 || E <= 0) return MOE_E_INVALID;
  if (d % kGroup != 0 || E > 1024) return MOE_E_UNSUPPORTED;
  if ((long long)T * d >= (1ll << 31) || (long long)E * d >= (1ll << 31) ||
      (long long)T * E >= (1ll << 31))
    return MOE_E_UNSUPPORTED;
  return MOE_OK;
}

Dims to_dims(const moe_dims *dm) { return Dims{dm->T, dm->d, dm->f, dm->E, dm->k}; }

W4 to_w4(const moe_w4_matrix &m) { return W4{m.codes, m.scales, m.biases}; }

Weights to_weights(const moe_w4_weights *w) {
  return Weights{to_w4(w->w13), to_w4(w->w2), to_w4(w->s13), to_w4(w->s2)};
}

hipStream_t as_stream(void *s) { return (hipStream_t)s; }

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Carving of the layer workspace. With base == nullptr only sizes are computed.
struct LayerWs {
  int32_t *ids, *counts, *offsets, *sorted_token, *row_of, *tile_map, *num_tiles, *block_counts;
  float *wts, *o_shared, *logits;
  uint16_t *h, *o_routed;
  size_t bytes;
};

template <typename P>
P *take(char *base, size_t &off, size_t count) {
  P *p = base ? (P *)(base + off) : nullptr;
  off += align256(count * sizeof(P));
  return p;
}

LayerWs carve_layer(const Dims &dm, char *base) {
  LayerWs w{};
  size_t off = 0;
  const size_t tk = (size_t)dm.T * dm.k;
  w.ids = take<int32_t>(base, off, tk);
  w.wts = take<float>(base, off, tk);
  w.counts = take<int32_t>(base, off, dm.E);
  w.offsets = take<int32_t>(base, off, dm.E + 1);
  w.sorted_token = take<int32_t>(base, off, tk);
  w.row_of = take<int32_t>(base, off, tk);
  w.tile_map = take<int32_t>(base, off, (size_t)tile_capacity(dm) * 4);
  w.num_tiles = take<int32_t>(base, off, 4);
  w.block_counts = take<int32_t>(base, off, (size_t)perm_blocks(dm.T) * dm.E);
  w.h = take<uint16_t>(base, off, (tk + dm.T) * (size_t)dm.f);
  w.o_routed = take<uint16_t>(base, off, tk * (size_t)dm.d);
  w.o_shared = take<float>(base, off, (size_t)dm.T * dm.d);
  w.logits = take<float>(base, off, (size_t)dm.T * dm.E);  // router scores (hidden-state entry)
  w.bytes = off;
  return w;
}

// Scratch of moe_layer_forward_noalloc: one copy per GPU, loaded with the
// library's code object and held until the process ends. Host code never uses
// the array's name as an address (on the host it is a stand-in, not device
// memory): each device's address comes from hipGetSymbolAddress, taken once
// per device with that device current, and is kept below.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// This device's address of the scratch array (looked up on the first call).
moe_status scratch_address(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return MOE_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (p == nullptr || ((uintptr_t)p & 255u) != 0) return MOE_E_ALIGN;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char *moe_status_string(int32_t st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_E_INVALID: return "invalid argument";
    case MOE_E_UNSUPPORTED: return "unsupported shape";
    case MOE_E_ALIGN: return "pointer not 16-byte aligned";
    case MOE_E_WORKSPACE: return "workspace too small";
    case MOE_E_HIP: return "HIP error";
    default: return "unknown status";
  }
}

int32_t moe_last_hip_error(void) { return g_last_hip_error; }

int32_t moe_block_m(void) { return kBlockM; }

int32_t moe_tile_capacity(const moe_dims *dm) {
  if (check_dims(dm) != MOE_OK) return -1;
  return tile_capacity(to_dims(dm));
}

size_t moe_permute_workspace_bytes(const moe_dims *dm) {
  if (check_dims(dm) != MOE_OK) return 0;
  return (size_t)perm_blocks(dm->T) * dm->E * sizeof(int32_t);
}

size_t moe_layer_workspace_bytes(const moe_dims *dm) {
  if (check_dims(dm) != MOE_OK) return 0;
  return carve_layer(to_dims(dm), nullptr).bytes;
}

moe_status moe_route(const float *logits, int32_t T, int32_t E, int32_t k, int32_t *topk_ids,
                     float *topk_w, void *stream) {
  if (T < 0 || E <= 0 || k <= 0 || k > E) return MOE_E_INVALID;
  if (E > 1024 || k > 32) return MOE_E_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  MOE_TRY(check_ptr(logits));
  MOE_TRY(check_ptr(topk_ids));
  MOE_TRY(check_ptr(topk_w));
  return hip_status(launch_route(logits, T, E, k, topk_ids, topk_w, as_stream(stream)));
}

moe_status moe_permute(const moe_dims *dm, const int32_t *topk_ids, int32_t *counts,
                       int32_t *offsets, int32_t *sorted_token, int32_t *row_of,
                       int32_t *tile_map, int32_t *num_tiles, void *ws, size_t ws_bytes,
                       void *stream) {
  MOE_TRY(check_dims(dm));
  if (dm->T == 0) return MOE_OK;
  MOE_TRY(check_ptr(topk_ids));
  MOE_TRY(check_ptr(counts));
  MOE_TRY(check_ptr(offsets));
  MOE_TRY(check_ptr(sorted_token));
  MOE_TRY(check_ptr(row_of));
  MOE_TRY(check_ptr(tile_map));
  MOE_TRY(check_ptr(num_tiles));
  MOE_TRY(check_ptr(ws));
  if (ws_bytes < moe_permute_workspace_bytes(dm)) return MOE_E_WORKSPACE;
  return hip_status(launch_permute(to_dims(dm), topk_ids, counts, offsets, sorted_token, row_of,
                                   tile_map, num_tiles, (int32_t *)ws, as_stream(stream)));
}

moe_status moe_route_permute(const moe_dims *dm, const float *logits, int32_t *topk_ids,
                             float *topk_w, int32_t *counts, int32_t *offsets,
                             int32_t *sorted_token, int32_t *row_of, int32_t *tile_map,
                             int32_t *num_tiles, void *ws, size_t ws_bytes, void *stream) {
  MOE_TRY(check_dims(dm));
  if (dm->T == 0) return MOE_OK;
  MOE_TRY(check_ptr(logits));
  MOE_TRY(check_ptr(topk_ids));
  MOE_TRY(check_ptr(topk_w));
  MOE_TRY(check_ptr(counts));
  MOE_TRY(check_ptr(offsets));
  MOE_TRY(check_ptr(sorted_token));
  MOE_TRY(check_ptr(row_of));
  MOE_TRY(check_ptr(tile_map));
  MOE_TRY(check_ptr(num_tiles));
  MOE_TRY(check_ptr(ws));
  if (ws_bytes < moe_permute_workspace_bytes(dm)) return MOE_E_WORKSPACE;
  return hip_status(launch_route_permute(to_dims(dm), logits, topk_ids, topk_w, counts, offsets,
                                         sorted_token, row_of, tile_map, num_tiles,
                                         (int32_t *)ws, as_stream(stream)));
}

moe_status moe_expert_gate_up_w4(const moe_dims *dm, const uint16_t *x, const moe_w4_weights *w,
                                 const int32_t *sorted_token, const int32_t *tile_map,
                                 const int32_t *num_tiles, uint16_t *h, void *stream) {
  MOE_TRY(check_dims(dm));
  if (dm->T == 0) return MOE_OK;
  MOE_TRY(check_weights(w, true, false));
  MOE_TRY(check_ptr(x));
  MOE_TRY(check_ptr(sorted_token));
  MOE_TRY(check_ptr(tile_map));
  MOE_TRY(check_ptr(num_tiles));
  MOE_TRY(check_ptr(h));
  return hip_status(launch_gate_up(to_dims(dm), x, to_weights(w), sorted_token, tile_map,
                                   num_tiles, h, as_stream(stream)));
}

moe_status moe_expert_down_w4(const moe_dims *dm, const uint16_t *h, const moe_w4_weights *w,
                              const int32_t *tile_map, const int32_t *num_tiles,
                              uint16_t *o_routed, float *o_shared, void *stream) {
  MOE_TRY(check_dims(dm));
  if (dm->T == 0) return MOE_OK;
  MOE_TRY(check_weights(w, false, true));
  MOE_TRY(check_ptr(h));
  MOE_TRY(check_ptr(tile_map));
  MOE_TRY(check_ptr(num_tiles));
  MOE_TRY(check_ptr(o_routed));
  MOE_TRY(check_ptr(o_shared));
  return hip_status(launch_down(to_dims(dm), h, to_weights(w), tile_map, num_tiles, o_routed,
                                o_shared, as_stream(stream)));
}

moe_status moe_expert_ffn_w4(const moe_dims *dm, const uint16_t *x, const moe_w4_weights *w,
                             const int32_t *sorted_token, const int32_t *tile_map,
                             const int32_t *num_tiles, uint16_t *h, uint16_t *o_routed,
                             float *o_shared, void *stream) {
  MOE_TRY(check_dims(dm));
  if (dm->T == 0) return MOE_OK;
  MOE_TRY(check_weights(w, true, true));
  MOE_TRY(check_ptr(o_routed));
  MOE_TRY(check_ptr(o_shared));
  MOE_TRY(moe_expert_gate_up_w4(dm, x, w, sorted_token, tile_map, num_tiles, h, stream));
  return moe_expert_down_w4(dm, h, w, tile_map, num_tiles, o_routed, o_shared, stream);
}

moe_status moe_unpermute_combine(const moe_dims *dm, const uint16_t *o_routed,
                                 const float *o_shared, const float *topk_w,
                                 const int32_t *row_of, float *y, void *stream) {
  MOE_TRY(check_dims(dm));
  if (dm->T == 0) return MOE_OK;
  MOE_TRY(check_ptr(o_routed));
  MOE_TRY(check_ptr(o_shared));
  MOE_TRY(check_ptr(topk_w));
  MOE_TRY(check_ptr(row_of));
  MOE_TRY(check_ptr(y));
  return hip_status(
      launch_combine(to_dims(dm), o_routed, o_shared, topk_w, row_of, y, as_stream(stream)));
}

// The layer from logits on; arguments already validated.
static moe_status enqueue_layer(const Dims &d, const uint16_t *x, const float *logits, const Weights &W,
                         float *y, const LayerWs &L, hipStream_t s) {
  if (decode_supported(d))
    return hip_status(launch_decode(d, x, logits, W, L.ids, L.wts, L.h, y, s));
  MOE_TRY(hip_status(launch_route_permute(d, logits, L.ids, L.wts, L.counts, L.offsets,
                                          L.sorted_token, L.row_of, L.tile_map, L.num_tiles,
                                          L.block_counts, s)));
  MOE_TRY(hip_status(launch_gate_up(d, x, W, L.sorted_token, L.tile_map, L.num_tiles, L.h, s)));
  MOE_TRY(hip_status(launch_down(d, L.h, W, L.tile_map, L.num_tiles, L.o_routed, L.o_shared, s)));
  return hip_status(launch_combine(d, L.o_routed, L.o_shared, L.wts, L.row_of, y, s));
}

moe_status moe_layer_forward(const moe_dims *dm, const uint16_t *x, const float *logits,
                             const moe_w4_weights *w, float *y, void *ws, size_t ws_bytes,
                             void *stream) {
  MOE_TRY(check_dims(dm));
  if (dm->T == 0) return MOE_OK;
  MOE_TRY(check_weights(w, true, true));
  MOE_TRY(check_ptr(x));
  MOE_TRY(check_ptr(logits));
  MOE_TRY(check_ptr(y));
  MOE_TRY(check_ptr(ws));
  const Dims d = to_dims(dm);
  const LayerWs L = carve_layer(d, (char *)ws);
  if (ws_bytes < L.bytes) return MOE_E_WORKSPACE;
  return enqueue_layer(d, x, logits, to_weights(w), y, L, as_stream(stream));
}

moe_status moe_layer_forward_noalloc(const moe_dims *dm, const uint16_t *x, const float *logits,
                                     const moe_w4_weights *w, float *y, void *stream) {
  MOE_TRY(check_dims(dm));
  if (dm->T == 0) return MOE_OK;
  MOE_TRY(check_weights(w, true, true));
  MOE_TRY(check_ptr(x));
  MOE_TRY(check_ptr(logits));
  MOE_TRY(check_ptr(y));
  const Dims d = to_dims(dm);
  // the size check comes before any HIP call
  if (carve_layer(d, nullptr).bytes > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_E_WORKSPACE;
  void *base = nullptr;
  MOE_TRY(scratch_address(&base));
  const LayerWs L = carve_layer(d, (char *)base);
  return enqueue_layer(d, x, logits, to_weights(w), y, L, as_stream(stream));
}

moe_status moe_router_logits(const uint16_t *x, const uint16_t *w_router, int32_t T, int32_t d,
                             int32_t E, float *logits, void *stream) {
  MOE_TRY(check_router_dims(T, d, E));
  if (T == 0) return MOE_OK;
  MOE_TRY(check_ptr(x));
  MOE_TRY(check_ptr(w_router));
  MOE_TRY(check_ptr(logits));
  return hip_status(launch_router_logits(x, w_router, T, d, E, logits, as_stream(stream)));
}

moe_status moe_layer_forward_hidden(const moe_dims *dm, const uint16_t *x,
                                    const uint16_t *w_router, const moe_w4_weights *w, float *y,
                                    void *ws, size_t ws_bytes, void *stream) {
  MOE_TRY(check_dims(dm));
  if (dm->T == 0) return MOE_OK;
  MOE_TRY(check_router_dims(dm->T, dm->d, dm->E));
  MOE_TRY(check_weights(w, true, true));
  MOE_TRY(check_ptr(x));
  MOE_TRY(check_ptr(w_router));
  MOE_TRY(check_ptr(y));
  MOE_TRY(check_ptr(ws));
  const Dims d = to_dims(dm);
  const LayerWs L = carve_layer(d, (char *)ws);
  if (ws_bytes < L.bytes) return MOE_E_WORKSPACE;
  const hipStream_t s = as_stream(stream);
  MOE_TRY(hip_status(launch_router_logits(x, w_router, d.T, d.d, d.E, L.logits, s)));
  return enqueue_layer(d, x, L.logits, to_weights(w), y, L, s);
}

moe_status moe_dequant_w4(const moe_w4_matrix *m, int32_t rows, int32_t cols, uint16_t *out,
                          void *stream) {
  if (m == nullptr || rows < 0 || cols <= 0) return MOE_E_INVALID;
  if (cols % kGroup != 0) return MOE_E_UNSUPPORTED;
  if ((long long)rows * cols >= (1ll << 34)) return MOE_E_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  MOE_TRY(check_matrix(*m));
  MOE_TRY(check_ptr(out));
  return hip_status(launch_dequant(to_w4(*m), rows, cols, out, as_stream(stream)));
}

}  // extern "C"
