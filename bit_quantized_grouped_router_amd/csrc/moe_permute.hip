// Routing histogram, exclusive prefix scan, stable scatter and tile block map,
// all on the device (noticiai.com.br page on Lily, section "Prefill e decode:
// onde estao os ganhos": these four steps stay in one GPU submission so that
// no CPU synchronisation happens inside an MoE layer).
//
// Three kernels on one stream:
//   perm_hist    per block of 256 tokens, a per-expert count (LDS atomics);
//   perm_scan    one workgroup: per-expert running prefix over the blocks,
//                exclusive scan over experts (offsets), tiles per group and
//                their exclusive scan, then the tile map, and the order the
//                grouped GEMMs take the tiles in (fourth column: tallest
//                first, so the longest work items start first and the short
//                ones fill the tail of the launch);
//   perm_scatter per block, the rank of each assignment among the block's
//                assignments to the same expert, from a token bitmask per
//                expert (popcount of the bits below the token), so the row
//                order is a stable counting sort and does not depend on the
//                order atomics happen in.
#include "moe_launch.h"

namespace moe {

constexpr int kMaxExperts = 1024;
constexpr int kMaskWords = kPermTokens / 32;

__device__ __forceinline__ int clamp_id(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

__global__ __launch_bounds__(256) void perm_hist_kernel(const int32_t *__restrict__ ids, int T,
                                                        int E, int k,
                                                        int32_t *__restrict__ block_counts) {
  __shared__ int cnt[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int t0 = blockIdx.x * kPermTokens;
  const int nt = min(kPermTokens, T - t0);
  const int32_t *blk = ids + (size_t)t0 * k;
  for (int a = threadIdx.x; a < nt * k; a += blockDim.x) atomicAdd(&cnt[clamp_id(blk[a], E)], 1);
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
// tile to run) lists every full tile in tile order, then the partial tiles
// by decreasing height, equal heights in tile order. Partial tiles are
// ranked with one LDS bitmask of groups per height, so the order is exact
// and independent of the order atomics happen in.
constexpr int kMaxGroups = kMaxExperts + 1;
constexpr int kGroupWords = (kMaxGroups + 31) / 32;

__global__ __launch_bounds__(1024) void perm_scan_kernel(int32_t *__restrict__ block_counts,
                                                         int nblocks, int T, int E, int k,
                                                         int32_t *__restrict__ counts,
                                                         int32_t *__restrict__ offsets,
                                                         int32_t *__restrict__ tile_map,
                                                         int32_t *__restrict__ num_tiles) {
  __shared__ int wave_tot[16];
  __shared__ int s_routed_tiles, s_routed_full;
  __shared__ uint32_t hmask[kBlockM][kGroupWords];  // groups whose partial tile has height r
  __shared__ int hstart[kBlockM];                   // schedule position of height r's first tile
  const int e = threadIdx.x;
  for (int i = e; i < kBlockM * kGroupWords; i += blockDim.x) (&hmask[0][0])[i] = 0u;
  // per-expert running prefix over token blocks, in place; the counts of 16
  // blocks are loaded together before any is overwritten (a load after a
  // store to the same array would otherwise wait for a full round trip each)
  int c = 0;
  if (e < E) {
    constexpr int kChunk = 16;
    for (int b0 = 0; b0 < nblocks; b0 += kChunk) {
      int v[kChunk];
#pragma unroll
      for (int i = 0; i < kChunk; ++i)
        v[i] = b0 + i < nblocks ? block_counts[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kChunk; ++i) {
        if (b0 + i < nblocks) block_counts[(size_t)(b0 + i) * E + e] = c;
        c += v[i];
      }
    }
  }
  const int nt = (c + kBlockM - 1) / kBlockM;
  const int nf = c / kBlockM;  // full tiles
  const int c_incl = block_inclusive_scan(c, wave_tot);
  const int nt_incl = block_inclusive_scan(nt, wave_tot);
  const int nf_incl = block_inclusive_scan(nf, wave_tot);
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
    if (c % kBlockM) atomicOr(&hmask[c % kBlockM][e >> 5], 1u << (e & 31));
  }
  if (e == blockDim.x - 1) {
    offsets[E] = c_incl;  // == T*k
    s_routed_tiles = nt_incl;
    s_routed_full = nf_incl;
  }
  __syncthreads();
  // the shared group E: rows T*k .. T*k+T-1
  const int rbase = s_routed_tiles;
  const int ns = (T + kBlockM - 1) / kBlockM;
  const int sh0 = T * k;
  for (int i = e; i < ns; i += blockDim.x) {
    const int rb = sh0 + i * kBlockM;
    const int re = min(rb + kBlockM, sh0 + T);
    int32_t *row = tile_map + 4 * (size_t)(rbase + i);
    row[0] = E;
    row[1] = rb;
    row[2] = re;
  }
  if (e == 0) {
    *num_tiles = rbase + ns;
    if (T % kBlockM) atomicOr(&hmask[T % kBlockM][E >> 5], 1u << (E & 31));
  }
  __syncthreads();
  // tiles per height, then the first schedule position of each height
  // (heights kBlockM-1 .. 1 after all full tiles)
  const int nfull = s_routed_full + T / kBlockM;
  int hc = 0;
  const int hgt = kBlockM - 1 - e;  // thread e counts height kBlockM-1-e (e < kBlockM-1)
  if (e < kBlockM - 1)
    for (int w = 0; w < kGroupWords; ++w) hc += __popc(hmask[hgt][w]);
  const int hc_incl = block_inclusive_scan(e < kBlockM - 1 ? hc : 0, wave_tot);
  if (e < kBlockM - 1) hstart[hgt] = nfull + hc_incl - hc;
  __syncthreads();
  // schedule entries: full routed tiles, full shared tiles, partial tiles
  if (e < E) {
    for (int i = 0; i < nf; ++i) tile_map[4 * (size_t)(fbase + i) + 3] = tbase + i;
    const int r = c % kBlockM;
    if (r) {
      int rank = __popc(hmask[r][e >> 5] & ((1u << (e & 31)) - 1u));
      for (int w = 0; w < (e >> 5); ++w) rank += __popc(hmask[r][w]);
      tile_map[4 * (size_t)(hstart[r] + rank) + 3] = tbase + nf;
    }
  }
  for (int i = e; i < T / kBlockM; i += blockDim.x)
    tile_map[4 * (size_t)(s_routed_full + i) + 3] = rbase + i;
  if (e == 0 && T % kBlockM) {
    const int r = T % kBlockM;
    int rank = 0;
    for (int w = 0; w <= (E >> 5); ++w)
      rank += __popc(w < (E >> 5) ? hmask[r][w] : (hmask[r][w] & ((1u << (E & 31)) - 1u)));
    tile_map[4 * (size_t)(hstart[r] + rank) + 3] = rbase + ns - 1;
  }
}

__global__ __launch_bounds__(kPermTokens) void perm_scatter_kernel(
    const int32_t *__restrict__ ids, int T, int E, int k, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ block_prefix, int32_t *__restrict__ sorted_token,
    int32_t *__restrict__ row_of) {
  __shared__ uint32_t mask[kMaxExperts * kMaskWords];
  for (int i = threadIdx.x; i < E * kMaskWords; i += blockDim.x) mask[i] = 0u;
  __syncthreads();
  const int tl = threadIdx.x;
  const int t = blockIdx.x * kPermTokens + tl;
  const bool valid = t < T;
  const int word = tl >> 5;
  const uint32_t bit = 1u << (tl & 31);
  if (valid)
    for (int j = 0; j < k; ++j) atomicOr(&mask[clamp_id(ids[(size_t)t * k + j], E) * kMaskWords + word], bit);
  __syncthreads();
  if (!valid) return;
  const int32_t *pre = block_prefix + (size_t)blockIdx.x * E;
  for (int j = 0; j < k; ++j) {
    const int e = clamp_id(ids[(size_t)t * k + j], E);
    const uint32_t *m = mask + e * kMaskWords;
    int rank = __popc(m[word] & (bit - 1u));
    for (int w = 0; w < word; ++w) rank += __popc(m[w]);
    const int p = offsets[e] + pre[e] + rank;
    sorted_token[p] = t;
    row_of[(size_t)t * k + j] = p;
  }
}

hipError_t launch_permute(const Dims &dm, const int32_t *ids, int32_t *counts, int32_t *offsets,
                          int32_t *sorted_token, int32_t *row_of, int32_t *tile_map,
                          int32_t *num_tiles, int32_t *block_counts, hipStream_t s) {
  const int nb = perm_blocks(dm.T);
  perm_hist_kernel<<<nb, 256, 0, s>>>(ids, dm.T, dm.E, dm.k, block_counts);
  perm_scan_kernel<<<1, 1024, 0, s>>>(block_counts, nb, dm.T, dm.E, dm.k, counts, offsets,
                                      tile_map, num_tiles);
  perm_scatter_kernel<<<nb, kPermTokens, 0, s>>>(ids, dm.T, dm.E, dm.k, offsets, block_counts,
                                                 sorted_token, row_of);
  return hipGetLastError();
}

}  // namespace moe
