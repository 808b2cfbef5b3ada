// Grouped expert GEMMs with the int4-g64 dequantisation fused into the tile
// (noticiai.com.br page on Lily, section "Prefill e decode: onde estao os
// ganhos": the tensor units take bf16, so the 4-bit weights are rebuilt to
// bf16 one tile at a time on chip, with fp32 accumulation).
//
// gfx950 design
//   - one workgroup = 4 wavefronts = a tile of <= 128 permuted rows (from the
//     block map) x 256 weight rows; every wavefront covers all 128 rows and
//     its own 64 weight rows, so each weight is dequantised exactly once per
//     tile and 32-row slabs past the tile's last row skip their MFMAs;
//   - v_mfma_f32_32x32x16_bf16 with fp32 accumulators (4 x 2 blocks of 32x32
//     per wavefront);
//   - the weights never pass through LDS: each lane loads 16 bytes of codes
//     (32 consecutive input columns of one weight row, one quantisation
//     group), rebuilds them to bf16 with the VALU and uses them directly as
//     its MFMA B fragments. Within a K step of 64, lane half h feeds input
//     columns 32h + 8s .. 32h + 8s + 7 to K slice s; the A fragments are read
//     with the same column mapping, which only permutes the order of the sum;
//   - the activation rows go through an LDS double buffer (16 KB per K
//     step), 16-byte chunks XOR-swizzled by row so that the fragment reads of
//     8 consecutive rows hit distinct banks; one barrier per K step;
//   - global loads run two K steps ahead of the MFMAs (activations one step
//     in registers, codes two steps);
//   - the grid is sized from the block map's capacity (a host-side bound);
//     workgroups past num_tiles (read on the device) exit at once, so no
//     host synchronisation is needed; block ids are remapped so that the
//     N blocks of one tile, and neighbouring tiles of one expert, run on the
//     same XCD and share its L2.
#include <type_traits>

#include "moe_launch.h"

namespace moe {

constexpr int kKT = 64;        // K per step: one quantisation group
constexpr int kWgCols = 256;   // weight rows per workgroup (64 per wavefront)
constexpr int kXcds = 8;

enum { kGateUp = 0, kDown = 1 };

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup b runs on
// XCD b % 8). Of the `active` work items (known only on the device), XCD x
// takes the contiguous range [x*per, (x+1)*per), per = ceil(active / 8): the
// work is spread evenly over the XCDs and neighbouring items (the N blocks
// of one tile, the tiles of one expert) share an L2. Returns -1 for a
// workgroup with no work. Needs gridDim.x >= 8 * per (true for a grid of at
// least `active` workgroups, rounded up to a multiple of 8).
__device__ __forceinline__ int xcd_remap(int bid, int active) {
  const int per = (active + kXcds - 1) / kXcds;
  const int slot = bid / kXcds;
  const int logical = (bid % kXcds) * per + slot;
  return (slot < per && logical < active) ? logical : -1;
}

// Byte offset of 16-byte chunk j (0..7) of row r in a 128-byte-row LDS tile.
// The chunk is XOR-swizzled with (r % 8) ^ ((r / 8) % 2): any 8 consecutive
// rows put a given chunk in 8 different bank groups, and so do the even (and
// the odd) rows among any 16, so 16-byte accesses of 8 or 16 consecutive rows
// are conflict-free whether the LDS serves 8 or 16 lanes per cycle.
__device__ __forceinline__ int swz(int r, int j) {
  return r * 128 + ((j ^ (r & 7) ^ ((r >> 3) & 1)) << 4);
}

// Per-workgroup state of one tile, set up once before the K loop.
struct TileSetup {
  const uint16_t *act;       // activation matrix (x for gate/up, h for down)
  uint32_t a_off[4];         // element offsets of this thread's 4 activation chunks
  int a_dst0;                // LDS byte offset of chunk 0 (chunk i adds 4096 i)
  const uint8_t *cbase;      // the expert's codes
  const uint16_t *sbase, *bbase;
  uint32_t c_off[2], s_off[2];  // this lane's weight rows, per 32-row block
  int ksteps;
  int nrb;                   // active 32-row blocks of the tile (1..4), wave-uniform
  bool wave_on;              // wave-uniform: this wavefront has weight rows (both blocks:
                             // f and d are multiples of 64)
};

// K loop of one tile. FULL: all four row blocks active (no per-block branches
// inside the K step, so the scheduler can interleave dequantisation with MFMAs).
template <bool FULL>
__device__ __forceinline__ void gemm_k_loop(const TileSetup &st, uint8_t (*lds)[kBlockM * 128],
                                            f32x16_t (&acc)[4][2]) {
  const int lane = threadIdx.x & 63;
  const int klast = st.ksteps - 1;
  uint4 ar0, ar1, ar2, ar3;
  auto load_a = [&](int kt) __attribute__((always_inline)) {
    const uint16_t *a = st.act + kt * kKT;
    ar0 = *(const uint4 *)(a + st.a_off[0]);
    ar1 = *(const uint4 *)(a + st.a_off[1]);
    ar2 = *(const uint4 *)(a + st.a_off[2]);
    ar3 = *(const uint4 *)(a + st.a_off[3]);
  };
  auto store_a = [&](int buf) __attribute__((always_inline)) {
    *(uint4 *)(&lds[buf][st.a_dst0]) = ar0;
    *(uint4 *)(&lds[buf][st.a_dst0 + 4096]) = ar1;
    *(uint4 *)(&lds[buf][st.a_dst0 + 8192]) = ar2;
    *(uint4 *)(&lds[buf][st.a_dst0 + 12288]) = ar3;
  };
  // codes, scales and biases of two K steps (the one in use and the next, in
  // flight); the loop is unrolled by two so every slot index is a compile-time
  // constant (registers, not scratch). Scale and bias stay raw until used, so
  // no instruction waits on them early. Loads are unconditional: an idle
  // wavefront reads weight row 0 of its matrix and discards the result.
  uint4 cr[2][2];
  uint16_t sr[2][2], br[2][2];
  auto load_b = [&](int kt, auto SLOT) __attribute__((always_inline)) {
    constexpr int slot = decltype(SLOT)::value;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      cr[slot][cb] = *(const uint4 *)(st.cbase + st.c_off[cb] + kt * (kKT / 2));
      sr[slot][cb] = st.sbase[st.s_off[cb] + kt];
      br[slot][cb] = st.bbase[st.s_off[cb] + kt];
    }
  };
  // LDS byte address of this lane's A fragment for K slice 0 and row block 0:
  // slice ks xors its chunk index, row block rb adds rb * 4096 (the swizzle
  // depends on row % 16 only)
  const int lrow = (lane & 31) * 128, lx = (lane & 7) ^ ((lane >> 3) & 1), lh = 4 * (lane >> 5);
  auto step = [&](int kt, auto SLOT) __attribute__((always_inline)) {
    constexpr int slot = decltype(SLOT)::value;
    // A(kt+1) to the other LDS buffer (at the last step: a harmless rewrite of
    // a buffer no one reads any more), then the loads of A(kt+2) and of the
    // codes of step kt+1 (into the slot step kt-1 has finished with)
    store_a((kt + 1) & 1);
    load_a(min(kt + 2, klast));
    load_b(min(kt + 1, klast), std::integral_constant<int, slot ^ 1>{});
    const uint8_t *abuf = lds[kt & 1];
    const uint32_t sb0 = (uint32_t)sr[slot][0] | ((uint32_t)br[slot][0] << 16);
    const uint32_t sb1 = (uint32_t)sr[slot][1] | ((uint32_t)br[slot][1] << 16);
    const DqGroup q0 = dq_prepare(sb0), q1 = dq_prepare(sb1);
    // one wave-uniform choice per K step: the fast dequantisation when every
    // lane's groups allow it, else the plain one (exact for every input)
    const bool all_fast = __builtin_amdgcn_ballot_w64(!(q0.fast && q1.fast)) == 0;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint32_t w0 = ks == 0 ? cr[slot][0].x : ks == 1 ? cr[slot][0].y : ks == 2 ? cr[slot][0].z : cr[slot][0].w;
      const uint32_t w1 = ks == 0 ? cr[slot][1].x : ks == 1 ? cr[slot][1].y : ks == 2 ? cr[slot][1].z : cr[slot][1].w;
      uint4 d0, d1;
      if (all_fast) {
        d0 = dequant8_fast(w0, q0);
        d1 = dequant8_fast(w1, q1);
      } else {
        d0 = dequant8(w0, bf16_to_f32(sb0 & 0xFFFFu), bf16_to_f32(sb0 >> 16));
        d1 = dequant8(w1, bf16_to_f32(sb1 & 0xFFFFu), bf16_to_f32(sb1 >> 16));
      }
      const bf16x8_t b0 = __builtin_bit_cast(bf16x8_t, d0);
      const bf16x8_t b1 = __builtin_bit_cast(bf16x8_t, d1);
      const uint8_t *aks = abuf + lrow + (((lh + ks) ^ lx) << 4);
      if (FULL) {
        // all four A fragments first (one LDS wait), then eight MFMAs
        bf16x8_t a[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
          a[rb] = __builtin_bit_cast(bf16x8_t, *(const uint4 *)(aks + rb * 4096));
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          acc[rb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[rb], b0, acc[rb][0], 0, 0, 0);
          acc[rb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[rb], b1, acc[rb][1], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          if (rb >= st.nrb) continue;
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, *(const uint4 *)(aks + rb * 4096));
          acc[rb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, acc[rb][0], 0, 0, 0);
          acc[rb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, acc[rb][1], 0, 0, 0);
        }
      }
    }
    lds_barrier();
  };

  // prologue: A(0) in LDS, A(1) in registers, codes(0) in flight
  load_a(0);
  load_b(0, std::integral_constant<int, 0>{});
  store_a(0);
  load_a(min(1, klast));
  lds_barrier();
  // whole pairs of steps in the loop (every path through its body is the
  // same, so the memory wait counters carried around the loop are exact),
  // then the remaining step if ksteps is odd
  int kt = 0;
  for (; kt + 2 <= st.ksteps; kt += 2) {
    step(kt, std::integral_constant<int, 0>{});
    step(kt + 1, std::integral_constant<int, 1>{});
  }
  if (kt < st.ksteps) step(kt, std::integral_constant<int, 0>{});
}

template <int KIND>
__global__ __launch_bounds__(256, 2) void grouped_gemm_w4_kernel(
    const uint16_t *__restrict__ act, W4 wr, W4 ws, const int32_t *__restrict__ sorted_token,
    const int32_t *__restrict__ tile_map, const int32_t *__restrict__ num_tiles_p,
    uint16_t *__restrict__ out_bf16, float *__restrict__ out_f32, int T, int d, int f, int E,
    int k, int grid) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][kBlockM * 128];

  // K: input width of the GEMM
  const int K = KIND == kGateUp ? d : f;
  const int ncols = KIND == kGateUp ? f : d;          // gate/up: units; down: output columns
  const int wg_cols = KIND == kGateUp ? kWgCols / 2 : kWgCols;
  const int nblk = (ncols + wg_cols - 1) / wg_cols;
  const int logical = xcd_remap(blockIdx.x, *num_tiles_p * nblk);
  if (logical < 0) return;
  const int tile = logical / nblk;
  const int n0 = (logical % nblk) * wg_cols;
  const int4 tm = *(const int4 *)(tile_map + 4 * (size_t)tile);
  const int g = tm.x, row_begin = tm.y, row_end = tm.z;
  const bool shared = g >= E;
  const W4 W = shared ? ws : wr;
  const size_t ex = shared ? 0 : (size_t)g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in a scalar register
  const int TK = T * k;

  TileSetup st;
  st.act = act;
  st.ksteps = K / kKT;
  // ---- activation rows: 4 chunks of 16 B per thread per K step. Rows past
  // the tile's end re-read its last row (their results are never stored), so
  // every load is unconditional and the wait counters stay exact. Chunk i of
  // this thread is row (tid >> 3) + 32 i, whose swizzle equals that of row
  // tid >> 3 (it depends on row % 16 only).
  st.a_dst0 = swz(tid >> 3, tid & 7);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = min(row_begin + (tid >> 3) + 32 * i, row_end - 1);
    uint32_t row;
    if (KIND == kGateUp) {
      int tok = shared ? p - TK : sorted_token[p];
      tok = tok < 0 ? 0 : (tok >= T ? T - 1 : tok);  // in range even for malformed routing
      row = (uint32_t)tok;
    } else {
      row = (uint32_t)p;
    }
    st.a_off[i] = row * (uint32_t)K + (uint32_t)(tid & 7) * 8u;
  }
  // ---- this wavefront's two 32-row blocks of weight rows
  int wrow0, wrow1;
  if (KIND == kGateUp) {
    const int unit = n0 + wave * 32;
    st.wave_on = unit < f;
    wrow0 = unit + (lane & 31);          // gate rows
    wrow1 = f + unit + (lane & 31);      // up rows
  } else {
    const int col = n0 + wave * 64;
    st.wave_on = col < d;
    wrow0 = col + (lane & 31);
    wrow1 = col + 32 + (lane & 31);
  }
  const int nrows_w = KIND == kGateUp ? 2 * f : d;
  // 32-bit offsets from the expert's base pointers (every matrix set < 4 GiB)
  st.cbase = W.codes + ex * (size_t)nrows_w * (K / 2);
  st.sbase = W.scales + ex * (size_t)nrows_w * (K / kGroup);
  st.bbase = W.biases + ex * (size_t)nrows_w * (K / kGroup);
  const uint32_t R0 = st.wave_on ? (uint32_t)wrow0 : 0u, R1 = st.wave_on ? (uint32_t)wrow1 : 0u;
  st.c_off[0] = R0 * (uint32_t)(K / 2) + (uint32_t)(lane >> 5) * 16u;
  st.c_off[1] = R1 * (uint32_t)(K / 2) + (uint32_t)(lane >> 5) * 16u;
  st.s_off[0] = R0 * (uint32_t)(K / kGroup);
  st.s_off[1] = R1 * (uint32_t)(K / kGroup);
  const int rows = row_end - row_begin;
  st.nrb = st.wave_on ? (rows + 31) / 32 : 0;

  f32x16_t acc[4][2];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) acc[rb][0] = acc[rb][1] = f32x16_t{0};
  if (st.nrb == 4)
    gemm_k_loop<true>(st, lds, acc);
  else
    gemm_k_loop<false>(st, lds, acc);

  // epilogue; C layout of the 32x32 MFMA: lane l holds column l%32, register
  // r holds row 8*(r/4) + 4*(l/32) + r%4
  if (!st.wave_on) return;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    if (rb >= st.nrb) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int p = row_begin + rb * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      if (p >= row_end) continue;
      if (KIND == kGateUp) {
        out_bf16[(size_t)p * f + wrow0] = to_bf16(silu_mul(acc[rb][0][r], acc[rb][1][r]));
      } else if (shared) {
        out_f32[(size_t)(p - TK) * d + wrow0] = acc[rb][0][r];
        out_f32[(size_t)(p - TK) * d + wrow1] = acc[rb][1][r];
      } else {
        out_bf16[(size_t)p * d + wrow0] = to_bf16(acc[rb][0][r]);
        out_bf16[(size_t)p * d + wrow1] = to_bf16(acc[rb][1][r]);
      }
    }
  }
}

static int round_up8(long long n) { return (int)((n + kXcds - 1) / kXcds * kXcds); }

hipError_t launch_gate_up(const Dims &dm, const uint16_t *x, const Weights &w,
                          const int32_t *sorted_token, const int32_t *tile_map,
                          const int32_t *num_tiles, uint16_t *h, hipStream_t s) {
  const int nblk = (dm.f + kWgCols / 2 - 1) / (kWgCols / 2);
  const int grid = round_up8((long long)tile_capacity(dm) * nblk);
  grouped_gemm_w4_kernel<kGateUp><<<grid, 256, 0, s>>>(x, w.w13, w.s13, sorted_token, tile_map,
                                                       num_tiles, h, nullptr, dm.T, dm.d, dm.f,
                                                       dm.E, dm.k, grid);
  return hipGetLastError();
}

hipError_t launch_down(const Dims &dm, const uint16_t *h, const Weights &w,
                       const int32_t *tile_map, const int32_t *num_tiles, uint16_t *o_routed,
                       float *o_shared, hipStream_t s) {
  const int nblk = (dm.d + kWgCols - 1) / kWgCols;
  const int grid = round_up8((long long)tile_capacity(dm) * nblk);
  grouped_gemm_w4_kernel<kDown><<<grid, 256, 0, s>>>(h, w.w2, w.s2, nullptr, tile_map, num_tiles,
                                                     o_routed, o_shared, dm.T, dm.d, dm.f, dm.E,
                                                     dm.k, grid);
  return hipGetLastError();
}

// ------------------------------------------------------------------ dequant (inspection)

__global__ __launch_bounds__(256) void dequant_kernel(W4 m, int rows, int cols,
                                                      uint16_t *__restrict__ out) {
  // one thread per 32 columns (16 bytes of codes, one group half), the same
  // fast/plain choice the GEMM tiles make
  const long long chunks = (long long)rows * cols / 32;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < chunks;
       i += (long long)gridDim.x * blockDim.x) {
    const long long col0 = (i * 32) % cols, row = (i * 32) / cols;
    const uint4 c = ((const uint4 *)m.codes)[i];
    const long long gi = row * (cols / kGroup) + col0 / kGroup;
    uint4 r[4];
    dequant32(c, (uint32_t)m.scales[gi] | ((uint32_t)m.biases[gi] << 16), r);
#pragma unroll
    for (int q = 0; q < 4; ++q) *(uint4 *)(out + i * 32 + q * 8) = r[q];
  }
}

hipError_t launch_dequant(const W4 &m, int rows, int cols, uint16_t *out, hipStream_t s) {
  const long long chunks = (long long)rows * cols / 32;
  long long blocks = (chunks + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  dequant_kernel<<<(int)blocks, 256, 0, s>>>(m, rows, cols, out);
  return hipGetLastError();
}

}  // namespace moe
