/*
 * moe_w4.h - C ABI of the MI355X (gfx950) int4-g64 grouped MoE expert layer.
 *
 * The layer is the one the noticiai.com.br page on Perplexity's Lily engine
 * describes for Qwen3.6-35B-A3B:
 *   - section "O modelo em tres formatos de carga": a router scores E = 256
 *     experts and keeps k = 8 per token; one shared expert sees every token;
 *   - section "Prefill e decode: onde estao os ganhos": expert weights are
 *     4-bit affine codes in groups of 64 that share one bf16 scale and one
 *     bf16 bias; they are rebuilt to bf16 one tile at a time inside the
 *     grouped GEMM and accumulated in fp32; the routing histogram, prefix
 *     scan, scatter and block map run on the GPU with no CPU synchronisation
 *     inside the layer; at batch-1 decode the layer is bandwidth bound.
 *
 * Conventions for every entry point
 *   - Every tensor pointer is a DEVICE pointer, allocated and owned by the
 *     caller. The library never allocates, frees, copies to the host or
 *     synchronises. Scratch space comes from a caller workspace.
 *   - `stream` is a hipStream_t (NULL = the default stream). All work is
 *     enqueued on it in order and the call returns without waiting.
 *   - Arguments are validated on the host before anything is enqueued. On a
 *     failed check a negative moe_status is returned and nothing is enqueued.
 *     A failed kernel launch returns MOE_E_HIP (moe_last_hip_error() has the
 *     hipError_t). Faults inside kernels surface at the caller's next sync.
 *   - T == 0 is valid: the call returns MOE_OK and enqueues nothing.
 *   - Every pointer must be 16-byte aligned (MOE_E_ALIGN otherwise).
 *   - Outputs must not alias inputs.
 *   - No C++ exception crosses this interface. Apart from a thread-local last
 *     error and the device scratch of moe_layer_forward_noalloc (with its
 *     per-device address table), the library holds no mutable state, so calls
 *     on different streams or threads are safe when their buffers do not
 *     overlap.
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *
 * Shapes (moe_dims)
 *   T tokens, d hidden size, f routed expert width, f_shared the shared
 *   expert's width, E routed experts, k experts chosen per token.
 *   Limits: T >= 0, d % 64 == 0, f % 64 == 0, d <= 6144, f <= 6144,
 *   1 <= k <= min(E, 32), 1 <= E <= 1024, T*(k+1) < 2^31 and every tensor
 *   under 2^31 elements. f_shared must equal f (a different shared width is
 *   a valid layer this version does not run: MOE_E_UNSUPPORTED; f_shared <= 0
 *   is MOE_E_INVALID).
 *
 * Weight layout (moe_w4_matrix), canonical and unshuffled
 *   codes  uint8 [n][rows][cols/2]: column c of a row is byte c>>1, in the
 *          low nibble when c is even and the high nibble when c is odd;
 *   scales bf16  [n][rows][cols/64]: group j covers columns 64j .. 64j+63;
 *   biases bf16  [n][rows][cols/64];
 *   weight w = bf16_rne( fp32( s * q + b ) ), q the unsigned code 0..15.
 *   Matrices are stored [out][in]: groups run along the input dimension.
 *
 * Permuted rows
 *   The T*k token-expert assignments are sorted by expert (stable in token
 *   order) into rows 0 .. T*k-1; the shared expert owns rows T*k .. T*k+T-1,
 *   row T*k+t holding token t. Intermediate tensors h and o are indexed by
 *   these rows.
 */
#ifndef MOE_W4_H
#define MOE_W4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_E_INVALID = -1,     /* null pointer, negative or inconsistent size */
  MOE_E_UNSUPPORTED = -2, /* a valid shape outside the limits above */
  MOE_E_ALIGN = -3,       /* a pointer is not 16-byte aligned */
  MOE_E_WORKSPACE = -4,   /* workspace smaller than the *_workspace_bytes figure */
  MOE_E_HIP = -5          /* a HIP call failed; see moe_last_hip_error() */
} moe_status;

typedef struct {
  int32_t T;        /* tokens */
  int32_t d;        /* hidden size (input of gate/up, output of down) */
  int32_t f;        /* routed expert intermediate width */
  int32_t E;        /* routed experts */
  int32_t k;        /* experts chosen per token */
  int32_t f_shared; /* shared expert intermediate width; must equal f */
} moe_dims;

typedef struct {
  const uint8_t *codes;   /* [n][rows][cols/2] packed 4-bit codes */
  const uint16_t *scales; /* [n][rows][cols/64] bf16 */
  const uint16_t *biases; /* [n][rows][cols/64] bf16 */
} moe_w4_matrix;

typedef struct {
  moe_w4_matrix w13; /* routed gate|up: n = E, rows = 2f (gate rows 0..f-1, up rows f..2f-1), cols = d */
  moe_w4_matrix w2;  /* routed down:    n = E, rows = d, cols = f */
  moe_w4_matrix s13; /* shared gate|up: n = 1, rows = 2 f_shared, cols = d */
  moe_w4_matrix s2;  /* shared down:    n = 1, rows = d, cols = f_shared */
} moe_w4_weights;

/*
 * moe_router_logits - the router's score of every expert for every token
 * (page section "O modelo em tres formatos de carga": the router scores the
 * E experts), as a bias-free projection of the hidden states:
 *   logits[t][e] = sum_c x[t][c] * w_router[e][c]
 * Products of two bf16 values are exact in fp32; they are summed in fp32, on
 * the matrix cores above 128 tokens and as dot products on the vector units
 * up to 128 (the summation order is unspecified but fixed, so results may
 * differ from another fp32 order by rounding, within d * 2^-24 * sum_c |x w|,
 * and repeat bit for bit).
 *   x         bf16 [T][d]   hidden states
 *   w_router  bf16 [E][d]   router matrix
 *   logits    fp32 [T][E]   out
 * Limits: T >= 0, d % 64 == 0, 1 <= E <= 1024, and T*d, E*d and T*E each
 * under 2^31 (MOE_E_INVALID for negative or zero sizes, MOE_E_UNSUPPORTED
 * past the limits).
 */
moe_status moe_router_logits(const uint16_t *x, const uint16_t *w_router, int32_t T, int32_t d,
                             int32_t E, float *logits, void *stream);

/*
 * moe_route - top-k selection and router weights
 * (page section "O modelo em tres formatos de carga": score E experts, keep k).
 *   logits   fp32  [T][E]  router logits
 *   topk_ids int32 [T][k]  out: chosen experts, by logit descending; equal
 *                          logits go to the lower expert index; -0 == +0
 *   topk_w   fp32  [T][k]  out: softmax over the k chosen logits
 * One wavefront per token. Preconditions (not checked on the device): no NaN
 * and at least k finite logits per token; if violated, the ids are still k
 * distinct values in [0, E) and the weights are unspecified.
 */
moe_status moe_route(const float *logits, int32_t T, int32_t E, int32_t k,
                     int32_t *topk_ids, float *topk_w, void *stream);

/* Rows per tile of the block map (the M tile height of the grouped GEMMs). */
int32_t moe_block_m(void);

/* Upper bound on the number of tiles of the block map; rows of tile_map to allocate. */
int32_t moe_tile_capacity(const moe_dims *dm);

/* Bytes of scratch workspace moe_permute needs (may be 0). */
size_t moe_permute_workspace_bytes(const moe_dims *dm);

/*
 * moe_permute - routing histogram, exclusive prefix scan, stable scatter and
 * tile block map, all on the device, no host synchronisation
 * (page section "Prefill e decode: onde estao os ganhos").
 *   topk_ids     int32 [T][k]         from moe_route
 *   counts       int32 [E]            out: rows per expert
 *   offsets      int32 [E+1]          out: exclusive scan, offsets[E] = T*k
 *   sorted_token int32 [T*k]          out: token of each permuted row
 *   row_of       int32 [T*k]          out: permuted row of assignment t*k+j
 *   tile_map     int32 [cap][4]       out: {group, row_begin, row_end, sched}
 *                                     per tile, cap = moe_tile_capacity(dm);
 *                                     groups 0..E-1 in order, then the shared
 *                                     group E (rows T*k .. T*k+T-1); each group
 *                                     split into ceil(count/BM) tiles of at most
 *                                     BM = moe_block_m() rows. sched of row i is
 *                                     the index of the i-th tile in the order
 *                                     the grouped GEMMs run them (position i
 *                                     on XCD i % 8), a permutation of
 *                                     0..num_tiles-1: first the F full tiles,
 *                                     in tile order cut into 8 runs whose
 *                                     lengths differ by at most one (longer
 *                                     runs first), the r-th tile of run x at
 *                                     position 8r + x; then the partial tiles,
 *                                     tallest first, equal heights in tile
 *                                     order. Entries past num_tiles are left
 *                                     untouched.
 *   num_tiles    int32 [1]            out: tiles written
 *   ws, ws_bytes                      scratch, >= moe_permute_workspace_bytes(dm)
 * Deterministic: the row order does not depend on scheduling.
 * Precondition: every id in [0, E) and distinct within a token (as
 * moe_route produces).
 */
moe_status moe_permute(const moe_dims *dm, const int32_t *topk_ids, int32_t *counts,
                       int32_t *offsets, int32_t *sorted_token, int32_t *row_of,
                       int32_t *tile_map, int32_t *num_tiles, void *ws, size_t ws_bytes,
                       void *stream);

/*
 * moe_route_permute - moe_route followed by moe_permute, with the same
 * outputs bit for bit. Up to 64 tokens the permutation is a single
 * one-workgroup launch (histogram, scan, block map and scatter together),
 * which removes most of the fixed cost of the routing at small batches; the
 * top-k runs in the same launch while it is short (at most 16 selection
 * rounds per wavefront, e.g. up to 32 tokens at k = 8 and E <= 256), and in
 * the moe_route kernel just before it otherwise.
 *   logits                      fp32 [T][E]
 *   topk_ids, topk_w            out, as moe_route
 *   counts .. num_tiles         out, as moe_permute
 *   ws, ws_bytes                as moe_permute
 */
moe_status moe_route_permute(const moe_dims *dm, const float *logits, int32_t *topk_ids,
                             float *topk_w, int32_t *counts, int32_t *offsets,
                             int32_t *sorted_token, int32_t *row_of, int32_t *tile_map,
                             int32_t *num_tiles, void *ws, size_t ws_bytes, void *stream);

/*
 * moe_expert_gate_up_w4 - grouped gate/up GEMM over the block map with the
 * int4-g64 dequantisation fused into the tile (the weights' bf16 MFMA
 * operands rebuilt in registers one K step at a time, fp32 accumulation; page
 * section "Prefill e decode: onde estao os ganhos"), and SiLU(gate)*up in the
 * epilogue. The block map may also be built by the caller: tiles of at most
 * moe_block_m() rows of one group, in moe_permute's layout, with a schedule
 * column that is a permutation of the tile indices.
 *   x            bf16  [T][d]
 *   sorted_token int32 [T*k], tile_map, num_tiles from moe_permute
 *   h            bf16  [T*k+T][f] out: h[p] = bf16(silu(gate_p) * up_p), with
 *                gate_p = W13_g[0:f] x_t and up_p = W13_g[f:2f] x_t for row p
 *                of group g carrying token t
 */
moe_status moe_expert_gate_up_w4(const moe_dims *dm, const uint16_t *x,
                                 const moe_w4_weights *w, const int32_t *sorted_token,
                                 const int32_t *tile_map, const int32_t *num_tiles,
                                 uint16_t *h, void *stream);

/*
 * moe_expert_down_w4 - grouped down GEMM, same fused dequantisation.
 *   h         bf16 [T*k+T][f] from moe_expert_gate_up_w4
 *   o_routed  bf16 [T*k][d]   out: W2_g h_p for the routed rows (rounded to bf16)
 *   o_shared  fp32 [T][d]     out: S2 h_p for the shared rows, row T*k+t -> t
 */
moe_status moe_expert_down_w4(const moe_dims *dm, const uint16_t *h, const moe_w4_weights *w,
                              const int32_t *tile_map, const int32_t *num_tiles,
                              uint16_t *o_routed, float *o_shared, void *stream);

/* moe_expert_ffn_w4 - moe_expert_gate_up_w4 followed by moe_expert_down_w4. */
moe_status moe_expert_ffn_w4(const moe_dims *dm, const uint16_t *x, const moe_w4_weights *w,
                             const int32_t *sorted_token, const int32_t *tile_map,
                             const int32_t *num_tiles, uint16_t *h, uint16_t *o_routed,
                             float *o_shared, void *stream);

/*
 * moe_unpermute_combine - weighted unpermute plus the shared expert
 * (page section "O modelo em tres formatos de carga": the shared expert sees
 * every token; it is added with weight 1).
 *   y[t] = o_shared[t] + sum_j topk_w[t][j] * o_routed[row_of[t*k+j]], fp32
 *   o_routed bf16 [T*k][d], o_shared fp32 [T][d], topk_w fp32 [T][k],
 *   row_of int32 [T*k], y fp32 [T][d] (out)
 */
moe_status moe_unpermute_combine(const moe_dims *dm, const uint16_t *o_routed,
                                 const float *o_shared, const float *topk_w,
                                 const int32_t *row_of, float *y, void *stream);

/* Bytes of workspace moe_layer_forward and moe_layer_forward_hidden need for
 * these dims. */
size_t moe_layer_workspace_bytes(const moe_dims *dm);

/*
 * moe_layer_forward - the whole layer on one stream with no host sync:
 * route, permute, gate/up, down, combine, or, for up to 16 tokens, the
 * decode path (two launches, one grid row per token: routing recomputed on
 * chip, each token's k + 1 experts' 4-bit weights streamed with 128-bit loads;
 * page section "Prefill e decode: onde estao os ganhos": at small batches
 * bandwidth sets the ceiling). The two paths agree within rounding; the
 * workspace's routing and permutation buffers are only written by the
 * first.
 *   x      bf16 [T][d]
 *   logits fp32 [T][E]
 *   y      fp32 [T][d] out
 *   ws     >= moe_layer_workspace_bytes(dm) bytes of device scratch
 */
moe_status moe_layer_forward(const moe_dims *dm, const uint16_t *x, const float *logits,
                             const moe_w4_weights *w, float *y, void *ws, size_t ws_bytes,
                             void *stream);

/* Bytes of the library's own device scratch array used by
 * moe_layer_forward_noalloc (one array per GPU the library runs on). */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * moe_layer_forward_noalloc - moe_layer_forward for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same kernels and results, with the
 * scratch taken from a device array the library owns instead of a caller
 * workspace. The call allocates nothing.
 *   x, logits, w, y  as moe_layer_forward (the caller still owns all of them)
 * Limits: the layer's scratch (moe_layer_workspace_bytes of the dims) must fit
 * in MOE_NOALLOC_SCRATCH_BYTES = 64 MiB, otherwise MOE_E_WORKSPACE is returned
 * before any HIP call. At d = 2048, f = 512, E = 256, k = 8 that is T <= 1307
 * (every T that takes the decode path fits).
 * The array: one per GPU, loaded with the library's code object and kept until
 * the process ends; its device address is looked up (hipGetSymbolAddress) on
 * the first call on each device, with that device current, so the stream must
 * belong to the current device. Every call on a GPU shares that GPU's array and
 * leaves its contents behind; nothing in it has to start at zero (every piece
 * is written before it is read within a call). Calls that may overlap on one
 * GPU (two streams, two threads, two captured graphs replayed concurrently)
 * race on the array: order them, or use moe_layer_forward with separate
 * workspaces.
 */
moe_status moe_layer_forward_noalloc(const moe_dims *dm, const uint16_t *x, const float *logits,
                                     const moe_w4_weights *w, float *y, void *stream);

/*
 * moe_layer_forward_hidden - moe_layer_forward starting from hidden states:
 * moe_router_logits into the workspace, then the layer on those logits (the
 * same kernels, small batches included). Every argument is validated before the
 * first launch.
 *   x         bf16 [T][d]
 *   w_router  bf16 [E][d]
 *   y         fp32 [T][d] out
 *   ws        >= moe_layer_workspace_bytes(dm) bytes of device scratch
 */
moe_status moe_layer_forward_hidden(const moe_dims *dm, const uint16_t *x,
                                    const uint16_t *w_router, const moe_w4_weights *w, float *y,
                                    void *ws, size_t ws_bytes, void *stream);

/*
 * moe_dequant_w4 - rebuild one int4-g64 matrix to bf16 with the same device
 * arithmetic the GEMM tiles use (for inspection and tests).
 *   m     one matrix (n = 1) of rows x cols, cols % 64 == 0
 *   out   bf16 [rows][cols]
 */
moe_status moe_dequant_w4(const moe_w4_matrix *m, int32_t rows, int32_t cols, uint16_t *out,
                          void *stream);

const char *moe_status_string(int32_t status);

/* hipError_t of the last MOE_E_HIP on this thread (0 if none). */
int32_t moe_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W4_H */
