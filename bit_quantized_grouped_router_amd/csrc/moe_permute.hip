// Routing histogram, exclusive prefix scan, stable scatter and tile block map,
// all on the device (noticiai.com.br page on Lily, section "Prefill e decode:
// onde estao os ganhos": these four steps stay in one GPU submission so that
// no CPU synchronisation happens inside an MoE layer).
//
// Two kernels on one stream, over blocks of 256 tokens:
//   perm_hist   one workgroup per block: per-expert count of the block's
//               assignments (LDS atomics), written to block_counts[b][E];
//   perm_place  one workgroup per block, plus one more. Every workgroup
//               redoes the small scan it needs from block_counts (per-expert
//               total and count over the earlier blocks, exclusive scan over
//               experts), so no third launch has to wait for a global scan.
//               A block workgroup then scatters its tokens: the rank of an
//               assignment among the block's assignments to the same expert
//               comes from a token bitmask per expert (popcount of the bits
//               below the token), so the row order is a stable counting sort
//               and does not depend on the order atomics happen in. The
//               extra workgroup writes counts, offsets, the tile map and the
//               order the grouped GEMMs take the tiles in (fourth column:
//               tallest first, so the longest work items start first and the
//               short ones fill the tail of the launch).
#include "moe_launch.h"

namespace moe {

constexpr int kMaxExperts = 1024;
constexpr int kMaskWords = kPermTokens / 32;
constexpr int kPlaceThreads = 1024;
// assignments of one token block per thread: kPermTokens * k / kPlaceThreads, k <= 32
constexpr int kPerThread = kPermTokens * 32 / kPlaceThreads;
// block counts each thread loads at once
constexpr int kChunk = 16;

__device__ __forceinline__ int clamp_id(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

__global__ __launch_bounds__(256) void perm_hist_kernel(const int32_t *__restrict__ ids, int T,
                                                        int E, int k,
                                                        int32_t *__restrict__ block_counts) {
  __shared__ int cnt[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int t0 = blockIdx.x * kPermTokens;
  const int na = min(kPermTokens, T - t0) * k;
  const int32_t *blk = ids + (size_t)t0 * k;
  // up to 32 ids per thread (k <= 32), all loaded before the atomics
  int v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int a = threadIdx.x + i * 256;
    v[i] = a < na ? blk[a] : -1;
  }
#pragma unroll
  for (int i = 0; i < 32; ++i)
    if (threadIdx.x + i * 256 < na) atomicAdd(&cnt[clamp_id(v[i], E)], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    block_counts[(size_t)blockIdx.x * E + e] = cnt[e];
}

// Inclusive scan of v over the 1024 threads of the block.
__device__ __forceinline__ int block_inclusive_scan(int v, int *wave_tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  if (lane == 63) wave_tot[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int w = lane < 16 ? wave_tot[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int o = __shfl_up(w, off, kWave);
      if (lane >= off) w += o;
    }
    if (lane < 16) wave_tot[lane] = w;
  }
  __syncthreads();
  const int add = wave > 0 ? wave_tot[wave - 1] : 0;
  __syncthreads();
  return v + add;
}

// Tiles are full (kBlockM rows) except the last of each group (c % kBlockM
// rows). The schedule (fourth column of the tile map: row i names the i-th
// tile to run) lists every full tile first, then the partial tiles by
// decreasing height, equal heights in tile order. Partial tiles are ranked
// with one LDS bitmask of groups per height, so the order is exact and
// independent of the order atomics happen in.
// The grouped GEMMs deal schedule position i to XCD i % kXcds. The full
// tiles, in tile order, are cut into kXcds runs of equal length (the first
// nfull % kXcds one tile longer), and run x goes to positions x, x + kXcds,
// x + 2 kXcds, ...: each XCD gets consecutive tiles, so a hot expert's full
// tiles share one XCD's L2 instead of every XCD fetching that expert's
// weights. Each XCD still receives the same positions, hence the same number
// of tiles of each height.
// Run x and place r in it of full tile p (0 <= p < nfull); the next tile is
// at r + 1 of the same run, or at 0 of run x + 1 once r reaches its length.
struct FullRuns {
  int q, rem;  // run length nfull / kXcds; the first rem runs are one longer
  __device__ explicit FullRuns(int nfull) : q(nfull / kXcds), rem(nfull % kXcds) {}
  __device__ int len(int x) const { return q + (x < rem ? 1 : 0); }
  __device__ void locate(int p, int &x, int &r) const {
    const int big = rem * (q + 1);  // tiles in the longer runs
    if (p < big) {
      x = p / (q + 1);
      r = p - x * (q + 1);
    } else {  // here q >= 1, since p < nfull
      x = rem + (p - big) / q;
      r = p - big - (x - rem) * q;
    }
  }
};
constexpr int kMaxGroups = kMaxExperts + 1;
constexpr int kGroupWords = (kMaxGroups + 31) / 32;

struct PlaceLds {
  int wave_tot[16];
  int routed_tiles, routed_full;
  union {
    struct {
      int off[kMaxExperts];                   // first row of the block's assignments per expert
      uint32_t mask[kMaxExperts * kMaskWords];  // per expert: tokens of the block
    } s;
    struct {
      uint32_t hmask[kBlockM][kGroupWords];  // groups whose partial tile has height r
      int hstart[kBlockM];                   // schedule position of height r's first tile
    } m;
  } u;
};

// Tile map, counts and offsets (the extra workgroup). Thread e owns expert e.
__device__ void write_tile_map(PlaceLds &L, int c, int c_incl, int T, int E, int k,
                               int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                               int32_t *__restrict__ tile_map, int32_t *__restrict__ num_tiles) {
  const int e = threadIdx.x;
  for (int i = e; i < kBlockM * kGroupWords; i += kPlaceThreads) (&L.u.m.hmask[0][0])[i] = 0u;
  const int nt = (c + kBlockM - 1) / kBlockM;
  const int nf = c / kBlockM;  // full tiles
  const int nt_incl = block_inclusive_scan(nt, L.wave_tot);
  const int nf_incl = block_inclusive_scan(nf, L.wave_tot);
  const int off = c_incl - c;
  const int tbase = nt_incl - nt;
  const int fbase = nf_incl - nf;
  if (e < E) {
    counts[e] = c;
    offsets[e] = off;
    for (int i = 0; i < nt; ++i) {
      const int rb = off + i * kBlockM;
      const int re = min(rb + kBlockM, off + c);
      int32_t *row = tile_map + 4 * (size_t)(tbase + i);
      row[0] = e;
      row[1] = rb;
      row[2] = re;
    }
    if (c % kBlockM) atomicOr(&L.u.m.hmask[c % kBlockM][e >> 5], 1u << (e & 31));
  }
  if (e == kPlaceThreads - 1) {
    offsets[E] = c_incl;  // == T*k
    L.routed_tiles = nt_incl;
    L.routed_full = nf_incl;
  }
  __syncthreads();
  // the shared group E: rows T*k .. T*k+T-1
  const int rbase = L.routed_tiles;
  const int ns = (T + kBlockM - 1) / kBlockM;
  const int sh0 = T * k;
  for (int i = e; i < ns; i += kPlaceThreads) {
    const int rb = sh0 + i * kBlockM;
    const int re = min(rb + kBlockM, sh0 + T);
    int32_t *row = tile_map + 4 * (size_t)(rbase + i);
    row[0] = E;
    row[1] = rb;
    row[2] = re;
  }
  if (e == 0) {
    *num_tiles = rbase + ns;
    if (T % kBlockM) atomicOr(&L.u.m.hmask[T % kBlockM][E >> 5], 1u << (E & 31));
  }
  __syncthreads();
  // tiles per height, then the first schedule position of each height
  // (heights kBlockM-1 .. 1 after all full tiles)
  const int nfull = L.routed_full + T / kBlockM;
  int hc = 0;
  const int hgt = kBlockM - 1 - e;  // thread e counts height kBlockM-1-e (e < kBlockM-1)
  if (e < kBlockM - 1)
    for (int w = 0; w < kGroupWords; ++w) hc += __popc(L.u.m.hmask[hgt][w]);
  const int hc_incl = block_inclusive_scan(e < kBlockM - 1 ? hc : 0, L.wave_tot);
  if (e < kBlockM - 1) L.u.m.hstart[hgt] = nfull + hc_incl - hc;
  __syncthreads();
  // schedule entries: full routed tiles, full shared tiles, partial tiles
  const FullRuns runs(nfull);
  if (e < E && nf > 0) {
    // this expert's full tiles fbase .. fbase + nf - 1: located once, then
    // stepped through the runs
    int x, r;
    runs.locate(fbase, x, r);
    for (int i = 0; i < nf; ++i) {
      tile_map[4 * (size_t)(kXcds * r + x) + 3] = tbase + i;
      if (++r == runs.len(x)) {
        ++x;
        r = 0;
      }
    }
  }
  if (e < E) {
    const int r = c % kBlockM;
    if (r) {
      int rank = __popc(L.u.m.hmask[r][e >> 5] & ((1u << (e & 31)) - 1u));
      for (int w = 0; w < (e >> 5); ++w) rank += __popc(L.u.m.hmask[r][w]);
      tile_map[4 * (size_t)(L.u.m.hstart[r] + rank) + 3] = tbase + nf;
    }
  }
  for (int i = e; i < T / kBlockM; i += kPlaceThreads) {
    int x, r;
    runs.locate(L.routed_full + i, x, r);
    tile_map[4 * (size_t)(kXcds * r + x) + 3] = rbase + i;
  }
  if (e == 0 && T % kBlockM) {
    const int r = T % kBlockM;
    int rank = 0;
    for (int w = 0; w <= (E >> 5); ++w)
      rank += __popc(w < (E >> 5) ? L.u.m.hmask[r][w]
                                  : (L.u.m.hmask[r][w] & ((1u << (E & 31)) - 1u)));
    tile_map[4 * (size_t)(L.u.m.hstart[r] + rank) + 3] = rbase + ns - 1;
  }
}

__global__ __launch_bounds__(kPlaceThreads) void perm_place_kernel(
    const int32_t *__restrict__ ids, const int32_t *__restrict__ block_counts, int nblocks, int T,
    int E, int k, int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ sorted_token, int32_t *__restrict__ row_of,
    int32_t *__restrict__ tile_map, int32_t *__restrict__ num_tiles) {
  __shared__ PlaceLds L;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;  // token block, or nblocks for the tile-map workgroup
  const bool mapper = b == nblocks;
  const int t0 = b * kPermTokens;
  const int na = mapper ? 0 : min(kPermTokens, T - t0) * k;  // assignments of this block
  // the block's ids, in flight while the counts are scanned
  int cur[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int a = tid + i * kPlaceThreads;
    cur[i] = a < na ? clamp_id(ids[(size_t)t0 * k + a], E) : 0;
  }
  if (!mapper)
    for (int i = tid; i < E * kMaskWords; i += kPlaceThreads) L.u.s.mask[i] = 0u;
  // thread e: total of expert e and its count over the blocks before b
  const int e = tid;
  int c = 0, before = 0;
  if (e < E) {
    for (int b0 = 0; b0 < nblocks; b0 += kChunk) {
      int v[kChunk];
#pragma unroll
      for (int i = 0; i < kChunk; ++i)
        v[i] = b0 + i < nblocks ? block_counts[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kChunk; ++i) {
        if (b0 + i == b) before = c;
        c += v[i];
      }
    }
  }
  const int c_incl = block_inclusive_scan(c, L.wave_tot);
  if (mapper) {
    write_tile_map(L, c, c_incl, T, E, k, counts, offsets, tile_map, num_tiles);
    return;
  }
  if (e < E) L.u.s.off[e] = c_incl - c + before;
  // the block's token bitmask per expert (the scan's barriers ordered the
  // clearing of mask before these)
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int a = tid + i * kPlaceThreads;
    if (a < na) {
      const int tl = a / k;
      atomicOr(&L.u.s.mask[cur[i] * kMaskWords + (tl >> 5)], 1u << (tl & 31));
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int a = tid + i * kPlaceThreads;
    if (a < na) {
      const int tl = a / k, ex = cur[i];
      const uint32_t *m = L.u.s.mask + ex * kMaskWords;
      int rank = __popc(m[tl >> 5] & ((1u << (tl & 31)) - 1u));
      for (int w = 0; w < (tl >> 5); ++w) rank += __popc(m[w]);
      const int p = L.u.s.off[ex] + rank;
      sorted_token[p] = t0 + tl;
      row_of[(size_t)t0 * k + a] = p;
    }
  }
}

// ------------------------------------------------------------------ small batches
// Up to kSmallT tokens the permutation takes one workgroup: the histogram is
// counted in LDS, then the scan, tile map and schedule and the stable scatter
// follow as in the two-kernel path (all tokens form a single token block).
// With little selection work the same workgroup also does the routing, so
// routing and permutation are one launch: wavefront w selects the top-k of
// tokens w, w + 16, w + 32 and w + 48 (all their logits loaded before the
// first selection). With more selection work (kMaxPerLane == 0) the route
// kernel selects first, one wavefront per token over many CUs, and this
// kernel reads its ids: the sixteen wavefronts of one workgroup would run
// their tokens' k selection rounds one after another. Same outputs, bit for bit,
// as moe_route then moe_permute, either way.
constexpr int kSmallT = 64;
constexpr int kSmallPerWave = kSmallT / (kPlaceThreads / kWave);  // 4

template <int kMaxPerLane>
__global__ __launch_bounds__(kPlaceThreads) void route_permute_small_kernel(
    const float *__restrict__ logits, int T, int E, int k, int32_t *__restrict__ ids_out,
    float *__restrict__ wts_out, int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ sorted_token, int32_t *__restrict__ row_of,
    int32_t *__restrict__ tile_map, int32_t *__restrict__ num_tiles) {
  __shared__ PlaceLds L;
  __shared__ int cnt[kMaxExperts];
  __shared__ int ids_s[kSmallT * 32];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int i = tid; i < E; i += kPlaceThreads) cnt[i] = 0;
  if constexpr (kMaxPerLane == 0) {
    // ---- the route kernel's ids (in range for any input), counted in LDS
    __syncthreads();
    for (int a = tid; a < T * k; a += kPlaceThreads) {
      const int id = clamp_id(ids_out[a], E);
      ids_s[a] = id;
      atomicAdd(&cnt[id], 1);
    }
  } else {
    constexpr int kM = kMaxPerLane > 0 ? kMaxPerLane : 1;
    float v[kSmallPerWave][kM];
#pragma unroll
    for (int i = 0; i < kSmallPerWave; ++i) {
      const int t = wave + 16 * i;
      wave_load_logits<kM>(logits + (size_t)(t < T ? t : T - 1) * E, E, v[i]);
    }
    __syncthreads();
    // ---- top-k and router weights (the same arithmetic as the route kernel)
#pragma unroll
    for (int i = 0; i < kSmallPerWave; ++i) {
      const int t = wave + 16 * i;
      if (t >= T) break;  // wave-uniform
      int id;
      float l;
      wave_topk_loaded<kM>(v[i], E, k, &id, &l);
      const float m = __shfl(l, 0, kWave);
      const float e = lane < k ? expf(l - m) : 0.f;
      const float sum = wave_sum(e);
      if (lane < k) {
        ids_out[(size_t)t * k + lane] = id;
        wts_out[(size_t)t * k + lane] = e / sum;
        ids_s[t * k + lane] = id;
        atomicAdd(&cnt[id], 1);
      }
    }
  }
  __syncthreads();
  // ---- counts, offsets, tile map and schedule (thread e owns expert e).
  // Fewer than kBlockM tokens: every non-empty group is a single partial
  // tile, so one scan of (rows, 1 << 16 per tile) gives both the offsets and
  // the tile indices, and the schedule only orders heights 1 .. T.
  static_assert(kSmallT < kBlockM, "one partial tile per group");
  for (int i = tid; i < (kSmallT + 1) * kGroupWords; i += kPlaceThreads) (&L.u.m.hmask[0][0])[i] = 0u;
  const int c = tid < E ? cnt[tid] : 0;
  const int packed = block_inclusive_scan(c + (c > 0 ? 1 << 16 : 0), L.wave_tot);
  const int c_incl = packed & 0xFFFF, tiles_incl = packed >> 16;
  const int tile_e = tiles_incl - (c > 0);
  if (tid < E) {
    counts[tid] = c;
    offsets[tid] = c_incl - c;
    if (c > 0) {
      int32_t *row = tile_map + 4 * (size_t)tile_e;
      row[0] = tid;
      row[1] = c_incl - c;
      row[2] = c_incl;
      atomicOr(&L.u.m.hmask[c][tid >> 5], 1u << (tid & 31));
    }
  }
  if (tid == kPlaceThreads - 1) {
    offsets[E] = c_incl;  // == T*k
    L.routed_tiles = tiles_incl;
  }
  if (tid == 0) atomicOr(&L.u.m.hmask[T][E >> 5], 1u << (E & 31));  // the shared group's tile
  __syncthreads();
  const int shared_tile = L.routed_tiles;
  if (tid == 0) {
    int32_t *row = tile_map + 4 * (size_t)shared_tile;
    row[0] = E;
    row[1] = T * k;
    row[2] = T * k + T;
    *num_tiles = shared_tile + 1;
  }
  // first schedule position of each height, tallest first: one wavefront,
  // lane l for height kSmallT - l
  if (tid < kWave) {
    const int hgt = kSmallT - tid;
    int hc = 0;
    if (hgt >= 1)
      for (int w = 0; w < kGroupWords; ++w) hc += __popc(L.u.m.hmask[hgt][w]);
    int incl = hc;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int o = __shfl_up(incl, off, kWave);
      if (tid >= off) incl += o;
    }
    if (hgt >= 1) L.u.m.hstart[hgt] = incl - hc;
  }
  __syncthreads();
  // schedule entries: equal heights in group (= tile) order; group g's rank
  // among its height's groups counts the bits below g
  auto rank_of = [&](int g, int h) {
    int rank = __popc(L.u.m.hmask[h][g >> 5] & ((1u << (g & 31)) - 1u));
    for (int w = 0; w < (g >> 5); ++w) rank += __popc(L.u.m.hmask[h][w]);
    return L.u.m.hstart[h] + rank;
  };
  if (tid < E && c > 0) tile_map[4 * (size_t)rank_of(tid, c) + 3] = tile_e;
  if (tid == 0) tile_map[4 * (size_t)rank_of(E, T) + 3] = shared_tile;
  __syncthreads();  // the LDS union passes from the tile map to the scatter
  // ---- stable scatter of the T*k assignments
  if (tid < E) L.u.s.off[tid] = c_incl - c;
  for (int i = tid; i < E * kMaskWords; i += kPlaceThreads) L.u.s.mask[i] = 0u;
  __syncthreads();
  const int TK = T * k;
  for (int a = tid; a < TK; a += kPlaceThreads) {
    const int t = a / k;
    atomicOr(&L.u.s.mask[ids_s[a] * kMaskWords + (t >> 5)], 1u << (t & 31));
  }
  __syncthreads();
  for (int a = tid; a < TK; a += kPlaceThreads) {
    const int t = a / k, ex = ids_s[a];
    const uint32_t *m = L.u.s.mask + ex * kMaskWords;
    int rank = __popc(m[t >> 5] & ((1u << (t & 31)) - 1u));
    for (int w = 0; w < (t >> 5); ++w) rank += __popc(m[w]);
    const int p = L.u.s.off[ex] + rank;
    sorted_token[p] = t;
    row_of[a] = p;
  }
}

hipError_t launch_route_permute(const Dims &dm, const float *logits, int32_t *ids, float *wts,
                                int32_t *counts, int32_t *offsets, int32_t *sorted_token,
                                int32_t *row_of, int32_t *tile_map, int32_t *num_tiles,
                                int32_t *block_counts, hipStream_t s) {
  if (dm.T > kSmallT) {
    if (const hipError_t e = launch_route(logits, dm.T, dm.E, dm.k, ids, wts, s)) return e;
    return launch_permute(dm, ids, counts, offsets, sorted_token, row_of, tile_map, num_tiles,
                          block_counts, s);
  }
  // selection rounds per wavefront in the one-launch kernel, weighted 4x for
  // the general selection (more than 256 experts); measured on gfx950, one
  // launch is faster up to about 16 (T = 32 at k = 8)
  const int rounds = (dm.T + 15) / 16 * dm.k * (dm.E > 256 ? 4 : 1);
  if (rounds > 16) {
    if (const hipError_t e = launch_route(logits, dm.T, dm.E, dm.k, ids, wts, s)) return e;
    route_permute_small_kernel<0><<<1, kPlaceThreads, 0, s>>>(
        logits, dm.T, dm.E, dm.k, ids, wts, counts, offsets, sorted_token, row_of, tile_map,
        num_tiles);
    return hipGetLastError();
  }
  if (dm.E <= 64)
    route_permute_small_kernel<1><<<1, kPlaceThreads, 0, s>>>(
        logits, dm.T, dm.E, dm.k, ids, wts, counts, offsets, sorted_token, row_of, tile_map,
        num_tiles);
  else if (dm.E <= 256)
    route_permute_small_kernel<4><<<1, kPlaceThreads, 0, s>>>(
        logits, dm.T, dm.E, dm.k, ids, wts, counts, offsets, sorted_token, row_of, tile_map,
        num_tiles);
  else
    route_permute_small_kernel<16><<<1, kPlaceThreads, 0, s>>>(
        logits, dm.T, dm.E, dm.k, ids, wts, counts, offsets, sorted_token, row_of, tile_map,
        num_tiles);
  return hipGetLastError();
}

hipError_t launch_permute(const Dims &dm, const int32_t *ids, int32_t *counts, int32_t *offsets,
                          int32_t *sorted_token, int32_t *row_of, int32_t *tile_map,
                          int32_t *num_tiles, int32_t *block_counts, hipStream_t s) {
  const int nb = perm_blocks(dm.T);
  perm_hist_kernel<<<nb, 256, 0, s>>>(ids, dm.T, dm.E, dm.k, block_counts);
  perm_place_kernel<<<nb + 1, kPlaceThreads, 0, s>>>(ids, block_counts, nb, dm.T, dm.E, dm.k,
                                                    counts, offsets, sorted_token, row_of,
                                                    tile_map, num_tiles);
  return hipGetLastError();
}

}  // namespace moe
