// Grouped expert GEMMs with the int4-g64 dequantisation fused into the tile
// (noticiai.com.br page on Lily, section "Prefill e decode: onde estao os
// ganhos": the tensor units take bf16, so the 4-bit weights are rebuilt to
// bf16 one tile at a time on chip, with fp32 accumulation).
//
// gfx950 design
//   - one workgroup = 4 wavefronts = a tile of <= 128 permuted rows (from the
//     block map) x 256 weight rows; every wavefront covers all 128 rows and
//     its own 64 weight rows, so each weight is dequantised exactly once per
//     tile; 32-row blocks past the tile's last row are not moved, read or
//     multiplied (the K loop is compiled for 1..4 active blocks);
//   - v_mfma_f32_32x32x16_bf16 with fp32 accumulators (4 x 2 blocks of 32x32
//     per wavefront);
//   - the weights never pass through LDS: each lane loads 16 bytes of codes
//     (32 consecutive input columns of one weight row, one quantisation
//     group) with a buffer load whose K offset is a scalar, rebuilds them to
//     bf16 with the VALU and uses them directly as its MFMA B fragments.
//     Within a K step of 64, lane half h feeds input columns 32h + 8s ..
//     32h + 8s + 7 to K slice s; the A fragments are read with the same
//     column mapping, which only permutes the order of the sum;
//   - the activation rows go global -> LDS directly (global_load_lds_dwordx4,
//     no registers), into a ring of three 16 KB stages, two K steps ahead;
//     16-byte chunks are XOR-swizzled by row so that fragment reads of 8 or
//     16 consecutive rows hit distinct banks: each lane of a DMA instruction
//     fetches the chunk that belongs at its (contiguous) LDS slot;
//   - the scales and biases of the tile's 256 weight rows sit in an LDS
//     table filled once per tile; whether every group of a wavefront's rows
//     allows the fast dequantisation is decided there too, so the K loop is
//     specialised on it and carries no per-step test;
//   - the grid is sized from the block map's capacity (a host-side bound);
//     workgroups past the device-side tile count exit at once, so no host
//     synchronisation is needed; tiles are taken in the block map's schedule
//     order (tallest first) and dealt round-robin to the 8 XCDs, the N
//     blocks of one tile on the same XCD so they share its L2.
#include <type_traits>

#include "moe_launch.h"

namespace moe {

constexpr int kKT = 64;                      // K per step: one quantisation group
constexpr int kWaves = 4;                     // wavefronts per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kWgCols = 64 * kWaves;         // weight rows per workgroup (64 per wavefront)
constexpr int kRB = kBlockM / 32;            // 32-row blocks per tile
constexpr int kStages = 3;                   // activation ring depth
constexpr int kDmaRows = kThreads / 8;        // tile rows one DMA instruction of the workgroup fills
static_assert(kWaves % 2 == 0 && kBlockM % kDmaRows == 0 && kDmaRows == 32, "DMA row mapping");

// The kernel is compiled twice: for tiles of up to MRB = kRB row blocks (the
// block map's full tiles), and for MRB = 1, used when no tile of the launch
// can have more than 32 rows (small batches). The second needs a quarter of
// the accumulators and of the activation ring, so more workgroups share a CU
// and hide one another's latencies; per row block it runs the same
// instructions, so its results are the same bits.
constexpr int kShortOcc = 3;  // workgroups per CU of the MRB = 1 kernel
template <int MRB>
constexpr int stage_bytes() { return MRB * 32 * 128; }  // one K step of the tile's rows, bf16
// workgroups per CU the register budget is sized for (128-row tiles leave
// room for two; 256-row tiles need all 512 registers of a lane)
template <int MRB>
constexpr int gemm_occ() { return MRB == 1 ? kShortOcc : (MRB <= 4 && kWaves <= 4 ? 2 : 1); }

enum { kGateUp = 0, kDown = 1 };

// Work item of workgroup bid. Workgroups are dispatched in id order,
// round-robin over the 8 XCDs (workgroup b runs on XCD b % 8). XCD x takes
// the tiles at schedule positions x, x + 8, x + 16, ... (the block map's
// schedule lists the tallest tiles first), each with its nblk N blocks in
// consecutive slots: the long work items start first on every XCD, the short
// ones fill the tail, and the N blocks of one tile share that XCD's L2.
// Returns false for a workgroup with no work. Needs gridDim.x >= 8 * nblk *
// ceil(ntiles / 8).
__device__ __forceinline__ bool sched_item(int bid, int ntiles, int nblk, int &pos, int &nb) {
  const int x = bid % kXcds, slot = bid / kXcds;
  const int rank = slot / nblk;
  pos = x + kXcds * rank;
  nb = slot - rank * nblk;
  return pos < ntiles;
}

// s_waitcnt with only the vector-memory counter limited (expcnt and lgkmcnt
// left at their maxima, which means no wait on them).
#define MOE_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (0x7 << 4) | (0xF << 8) | (((n) >> 4) << 14))

typedef __attribute__((address_space(3))) void lds_void;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Activations of K step src into ring stage `stage`: this lane's 16-byte
// chunks (see the kernel for the lane -> row/chunk assignment), LDS DMA
// through a buffer resource (byte offsets: a_off, plus the step as a scalar).
// DMA instruction i fills 32-row block i of the tile, so a tile with NRB
// active row blocks issues the first NRB.
template <int NRB, int MRB>
__device__ __forceinline__ void dma_stage(__amdgpu_buffer_rsrc_t actr,
                                          const uint32_t *a_off, uint8_t *lds,
                                          uint32_t a_lds, int src, int stage) {
  uint8_t *s = lds + stage * stage_bytes<MRB>() + a_lds;
#pragma unroll
  for (int i = 0; i < NRB; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(actr, (lds_void *)(s + i * kDmaRows * 128), 16, a_off[i],
                                             src * (kKT * 2), 0, 0);
}

// Per-workgroup state of one tile, set up once before the K loop.
template <int MRB>
struct TileSetup {
  __amdgpu_buffer_rsrc_t actr;       // activation matrix (x for gate/up, h for down)
  __amdgpu_buffer_rsrc_t actr_none;  // the same with no records: every access out of range
  uint32_t a_off[MRB];    // byte offsets (K step 0) of this lane's DMA chunks (one per row block)
  uint32_t a_lds;         // LDS byte offset of this wavefront's first DMA slot in a stage
  __amdgpu_buffer_rsrc_t codes;       // the expert's codes
  __amdgpu_buffer_rsrc_t codes_none;  // the same with no records
  uint32_t c_off[2];      // byte offsets of this lane's two weight rows (plus its half)
  const uint32_t *sbl;    // LDS table [K/64][256] of (scale | bias << 16) per weight row
  int lr0;                // this lane's table column for block 0 (block 1 adds 32)
  int ksteps;
  int nrb;                // active 32-row blocks of the tile (1..MRB), wave-uniform
};

// Schedule check build (MOE_SCHED_CHECK=1, a separate library made by the
// build for a regression test): a scheduling barrier after each K step's
// loads pushes more of the step's A-fragment LDS reads towards its end, up to
// the next step's barrier. The results must stay bit-identical, which holds
// only while every barrier of the loop also waits for the wavefront's own LDS
// reads (the stage they read is refilled by the DMA issued right after it).
#if defined(MOE_SCHED_CHECK) && MOE_SCHED_CHECK
#define MOE_SCHED_CHECK_POINT() __builtin_amdgcn_sched_barrier(0)
#else
#define MOE_SCHED_CHECK_POINT() \
  do {                          \
  } while (0)
#endif

// K loop of one tile. NRB: the tile's active 32-row blocks (1..MRB), known
// at compile time, so a short tile moves, reads and multiplies only the rows
// it has (the activation DMA, the A-fragment reads and the MFMAs all scale
// with NRB; the dequantisation does not). FAST: every group of this
// wavefront's weight rows takes the fast dequantisation.
//
// Order of one K step kt: wait until this wavefront's DMA of stage kt has
// landed (at most the NRB DMA chunks of stage kt+1, issued one step later,
// may still be in flight; code loads issued after them only make the wait
// stricter), barrier (every wavefront's stage kt is in LDS, and every
// wavefront's reads of stage kt-1 have completed: the barrier also waits for
// the wavefront's own LDS operations, since the compiler may leave the last
// slice's fragment reads in flight past the end of a step), DMA of stage
// kt+2 into the slot of stage kt-1, code loads for step kt+2, then the four
// K slices.
template <int NRB, bool FAST, int MRB>
__device__ __forceinline__ void gemm_k_loop(const TileSetup<MRB> &st, uint8_t *lds,
                                            f32x16_t (&acc)[MRB][2], const u32x4_t (&cr0)[2],
                                            const u32x4_t (&cr1)[2]) {
  const int lane = threadIdx.x & 63;
  const int klast = st.ksteps - 1;
  const DqRegs dk = dq_regs();
  // codes of three K steps (in use, and the next two in flight); the loop is
  // unrolled by three so every slot index is a compile-time constant. Steps 0
  // and 1 (codes and activation stages) were issued by the caller; step kt
  // issues step kt + 2 (through the empty resources once past the last step).
  u32x4_t cr[3][2] = {{cr0[0], cr0[1]}, {cr1[0], cr1[1]}, {}};
  // LDS byte address of this lane's A fragment for K slice 0 and row block 0:
  // slice ks xors its chunk index, row block rb adds rb * 4096 (the swizzle
  // depends on row % 16 only)
  const int lrow = (lane & 31) * 128, lx = (lane & 7) ^ ((lane >> 3) & 1), lh = 4 * (lane >> 5);
  // scale/bias words of the next step (read one step ahead)
  uint32_t sb0, sb1;

  // activations of K step src_ into ring stage stage_
  // steps past the last one read through the empty resources: the loads
  // stay in the instruction stream (so every wait count holds) but touch no
  // memory and return zeros into a stage or code slot no one reads
#define MOE_DMA(src_, stage_)                                                                \
  {                                                                                          \
    const __amdgpu_buffer_rsrc_t r_ = (src_) <= klast ? st.actr : st.actr_none;             \
    dma_stage<NRB, MRB>(r_, st.a_off, lds, st.a_lds, (src_) <= klast ? (src_) : 0, (stage_)); \
  }
#define MOE_LOAD_B(kt_, slot_)                                                              \
  {                                                                                         \
    const __amdgpu_buffer_rsrc_t r_ = (kt_) <= klast ? st.codes : st.codes_none;             \
    const int so_ = (kt_) <= klast ? (kt_) * (kKT / 2) : 0;                                  \
    cr[slot_][0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(       \
                                                 r_, st.c_off[0], so_, 0));                  \
    cr[slot_][1] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(       \
                                                 r_, st.c_off[1], so_, 0));                  \
  }

  // B fragments (dequantised codes) of one K slice of this lane's two weight
  // rows; q*_ / p*_ are the group constants of the step the codes belong to
#define MOE_DQ(w0_, w1_, q0_, q1_, sb0_, sb1_, out0_, out1_)                                   \
  {                                                                                          \
    uint4 d0_, d1_;                                                                          \
    if (FAST) {                                                                              \
      d0_ = dequant8_fast(w0_, q0_, dk);                                                     \
      d1_ = dequant8_fast(w1_, q1_, dk);                                                     \
    } else {                                                                                 \
      d0_ = dequant8(w0_, bf16_to_f32((sb0_) & 0xFFFFu), bf16_to_f32((sb0_) >> 16));         \
      d1_ = dequant8(w1_, bf16_to_f32((sb1_) & 0xFFFFu), bf16_to_f32((sb1_) >> 16));         \
    }                                                                                        \
    out0_ = __builtin_bit_cast(bf16x8_t, d0_);                                               \
    out1_ = __builtin_bit_cast(bf16x8_t, d1_);                                               \
  }

  // one K step; slot_ is a literal (0..2) equal to kt_ % 3. The B fragments
  // are rebuilt one K slice ahead: while the MFMAs of slice ks run, the VALU
  // rebuilds slice ks + 1 (after slice 3: slice 0 of the next step, from the
  // codes and scales already in registers), so the dequantisation and the
  // matrix cores work on independent data.
#define MOE_STEP(kt_, slot_)                                                                 \
  {                                                                                          \
    const int ktv_ = (kt_);                                                                  \
    MOE_WAIT_VMCNT(NRB + 2);                                                                 \
    /* the barrier waits for this wavefront's LDS reads too: the DMA issued  */              \
    /* right after it refills the stage the previous step read from          */              \
    lds_barrier();                                                                           \
    /* no LDS access or use of this step's codes moves above the wait and barrier */        \
    asm volatile("" : "+v"(cr[slot_][0]), "+v"(cr[slot_][1])::"memory");                    \
    MOE_DMA(ktv_ + 2, (ktv_ + 2) % kStages);                                                 \
    MOE_LOAD_B(ktv_ + 2, ((slot_) + 2) % 3);                                                 \
    MOE_SCHED_CHECK_POINT();                                                                 \
    const uint32_t s0_ = sb0, s1_ = sb1;                                                     \
    {                                                                                        \
      const int kn_ = min(ktv_ + 1, klast) * kWgCols + st.lr0;                               \
      sb0 = st.sbl[kn_];                                                                     \
      sb1 = st.sbl[kn_ + 32];                                                                \
    }                                                                                        \
    const uint8_t *abuf_ = lds + (ktv_ % kStages) * stage_bytes<MRB>();                      \
    const DqGroup q0_ = dq_consts(s0_), q1_ = dq_consts(s1_);                                \
    _Pragma("unroll") for (int ks = 0; ks < 4; ++ks) {                                       \
      const uint8_t *aks_ = abuf_ + lrow + (((lh + ks) ^ lx) << 4);                          \
      bf16x8_t a_[NRB];                                                                      \
      _Pragma("unroll") for (int rb = 0; rb < NRB; ++rb)                                     \
        a_[rb] = __builtin_bit_cast(bf16x8_t, *(const uint4 *)(aks_ + rb * 4096));           \
      bf16x8_t n0_, n1_;                                                                     \
      if (ks < 3) {                                                                          \
        MOE_DQ(cr[slot_][0][ks + 1], cr[slot_][1][ks + 1], q0_, q1_, s0_, s1_, n0_, n1_);    \
      } else {                                                                               \
        const DqGroup r0_ = dq_consts(sb0), r1_ = dq_consts(sb1);                            \
        MOE_DQ(cr[((slot_) + 1) % 3][0][0], cr[((slot_) + 1) % 3][1][0], r0_, r1_, sb0, sb1, \
               n0_, n1_);                                                                    \
      }                                                                                      \
      _Pragma("unroll") for (int rb = 0; rb < NRB; ++rb) {                                   \
        acc[rb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_[rb], bq0, acc[rb][0], 0, 0, 0); \
        acc[rb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_[rb], bq1, acc[rb][1], 0, 0, 0); \
      }                                                                                      \
      bq0 = n0_;                                                                             \
      bq1 = n1_;                                                                             \
    }                                                                                        \
  }

  // the scales of step 0, slice 0 of step 0 rebuilt
  sb0 = st.sbl[st.lr0];
  sb1 = st.sbl[st.lr0 + 32];
  bf16x8_t bq0, bq1;
  {
    const DqGroup r0 = dq_consts(sb0), r1 = dq_consts(sb1);
    MOE_DQ(cr[0][0][0], cr[0][1][0], r0, r1, sb0, sb1, bq0, bq1);
  }
  // whole triples of steps in the loop (every path through its body is the
  // same, so the memory wait counters carried around the loop are exact),
  // then the one or two remaining steps
  int kt = 0;
  for (; kt + 3 <= st.ksteps; kt += 3) {
    MOE_STEP(kt, 0);
    MOE_STEP(kt + 1, 1);
    MOE_STEP(kt + 2, 2);
  }
  if (kt < st.ksteps) MOE_STEP(kt, 0);
  if (kt + 1 < st.ksteps) MOE_STEP(kt + 1, 1);
  // no DMA may still be writing LDS when the workgroup moves on
  MOE_WAIT_VMCNT(0);
#undef MOE_STEP
#undef MOE_DQ
#undef MOE_DMA
#undef MOE_LOAD_B
}

// DMA of ring stages 0 and 1 (K steps 0 and 1) for a tile of NRB row blocks.
template <int NRB, int MRB>
__device__ __forceinline__ void prologue_dma(const TileSetup<MRB> &st, uint8_t *lds, int klast) {
  dma_stage<NRB, MRB>(st.actr, st.a_off, lds, st.a_lds, 0, 0);
  dma_stage<NRB, MRB>(st.actr, st.a_off, lds, st.a_lds, min(1, klast), 1);
}

// The K loop for a tile of NRB row blocks, entered once stage 0 has landed
// (only the NRB chunks of stage 1 may still be in flight, so the loop's
// first wait holds at once).
template <int NRB, int MRB>
__device__ __forceinline__ void tile_k_loop(const TileSetup<MRB> &st, uint8_t *lds,
                                            f32x16_t (&acc)[MRB][2], const u32x4_t (&cr0)[2],
                                            const u32x4_t (&cr1)[2], bool fast) {
  MOE_WAIT_VMCNT(NRB);
  if (fast)
    gemm_k_loop<NRB, true>(st, lds, acc, cr0, cr1);
  else
    gemm_k_loop<NRB, false>(st, lds, acc, cr0, cr1);
}

// Stores one wavefront's block of results: acc[rb][0..1] for the tile's first
// nrb row blocks. colbase: gate/up, the first of 32 units (acc[.][0] holds
// their gate rows and acc[.][1] their up rows); down, the first of 64 output
// columns (acc[.][0] columns colbase .. +31, acc[.][1] the next 32). bf16
// outputs go through the LDS region ep as [row][col] tiles and leave as
// 16-byte row chunks; the shared expert's fp32 down outputs are stored
// directly.
template <int KIND, int MRB>
__device__ __forceinline__ void store_block(const f32x16_t (&acc)[MRB][2], int nrb, int colbase,
                                            bool shared, int row_begin, int row_end, int TK,
                                            int d, int f, uint8_t *ep, uint16_t *out_bf16,
                                            float *out_f32) {
  const int lane = threadIdx.x & 63;
  // C layout of the 32x32 MFMA: lane l holds column l%32, register r holds
  // row 8*(r/4) + 4*(l/32) + r%4
  const int c = lane & 31, hh = lane >> 5;
  if (KIND == kDown && shared) {
    // fp32 rows of the shared expert: 128 contiguous bytes per half-wavefront
    const int wrow0 = colbase + c, wrow1 = colbase + 32 + c;
#pragma unroll
    for (int rb = 0; rb < MRB; ++rb) {
      if (rb >= nrb) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int p = row_begin + rb * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);
        if (p >= row_end) continue;
        out_f32[(size_t)(p - TK) * d + wrow0] = acc[rb][0][r];
        out_f32[(size_t)(p - TK) * d + wrow1] = acc[rb][1][r];
      }
    }
    return;
  }
  // gate/up: 32 columns (64 bytes) per row, physical row r ^ (2 * ((r / 4) %
  // 2)); down: 64 columns (128 bytes) per row, 16-byte chunk j stored at j ^
  // (4 * ((r / 4) % 2)). Either way the two halves of the wavefront (rows r
  // and r + 4) write disjoint banks.
#pragma unroll
  for (int rb = 0; rb < MRB; ++rb) {
    if (rb >= nrb) continue;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const int row = rb * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);  // even; row + 1 is r + 1's
      if (KIND == kGateUp) {
        const uint32_t pk = pack_bf16x2(silu_mul_fast(acc[rb][0][r], acc[rb][1][r]),
                                        silu_mul_fast(acc[rb][0][r + 1], acc[rb][1][r + 1]));
        const int pr = row ^ (((row >> 2) & 1) << 1);
        *(uint16_t *)(ep + pr * 64 + c * 2) = (uint16_t)pk;
        *(uint16_t *)(ep + (pr + 1) * 64 + c * 2) = (uint16_t)(pk >> 16);
      } else {
        const int sw = ((row >> 2) & 1) * 4;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const uint32_t pk = pack_bf16x2(acc[rb][b][r], acc[rb][b][r + 1]);
          const int off = ((((b * 32 + c) >> 3) ^ sw) << 4) + (c & 7) * 2;
          *(uint16_t *)(ep + row * 128 + off) = (uint16_t)pk;
          *(uint16_t *)(ep + (row + 1) * 128 + off) = (uint16_t)(pk >> 16);
        }
      }
    }
  }
  if (KIND == kGateUp) {
    for (int it = 0; it < nrb * 2; ++it) {
      const int r = it * 16 + (lane >> 2), j = lane & 3;
      const int pr = r ^ (((r >> 2) & 1) << 1);
      const uint4 v = *(const uint4 *)(ep + pr * 64 + j * 16);
      const int p = row_begin + r;
      if (p < row_end) *(uint4 *)(out_bf16 + (size_t)p * f + colbase + j * 8) = v;
    }
  } else {
    for (int it = 0; it < nrb * 4; ++it) {
      const int r = it * 8 + (lane >> 3), j = lane & 7;
      const uint4 v = *(const uint4 *)(ep + r * 128 + ((j ^ (((r >> 2) & 1) * 4)) << 4));
      const int p = row_begin + r;
      if (p < row_end) *(uint4 *)(out_bf16 + (size_t)p * d + colbase + j * 8) = v;
    }
  }
}

template <int KIND, int MRB>
__global__ __launch_bounds__(kThreads, gemm_occ<MRB>()) void grouped_gemm_w4_kernel(
    const uint16_t *__restrict__ act, W4 wr, W4 ws, const int32_t *__restrict__ sorted_token,
    const int32_t *__restrict__ tile_map, const int32_t *__restrict__ num_tiles_p,
    uint16_t *__restrict__ out_bf16, float *__restrict__ out_f32, int T, int d, int f, int E,
    int k) {
  // LDS: the activation ring, then the scale/bias table of the tile's 256
  // weight rows for all K/64 groups (sized by the launch), then (MRB = 1
  // down only) the output staging
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint32_t *sbl = (uint32_t *)(smem + kStages * stage_bytes<MRB>());

  // K: input width of the GEMM
  const int K = KIND == kGateUp ? d : f;
  const int ncols = KIND == kGateUp ? f : d;          // gate/up: units; down: output columns
  const int wg_cols = KIND == kGateUp ? kWgCols / 2 : kWgCols;
  const int nblk = (ncols + wg_cols - 1) / wg_cols;
  int pos, nb;
  const int ntiles = *num_tiles_p;
  if (!sched_item(blockIdx.x, ntiles, nblk, pos, nb)) return;
  const int tile = min(max(tile_map[4 * (size_t)pos + 3], 0), ntiles - 1);  // in range for any map
  const int n0 = nb * wg_cols;
  const int4 tm = *(const int4 *)(tile_map + 4 * (size_t)tile);
  const int g = tm.x, row_begin = tm.y, row_end = tm.z;
  const bool shared = g >= E;
  const W4 W = shared ? ws : wr;
  const size_t ex = shared ? 0 : (size_t)g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in a scalar register
  const int TK = T * k;

  TileSetup<MRB> st;
  {
    // x: T rows of d; h: T*k routed + T shared rows of f (under 2^32 bytes)
    const uint32_t act_bytes =
        (uint32_t)((KIND == kGateUp ? (size_t)T : (size_t)TK + T) * (size_t)K * 2);
    st.actr = __builtin_amdgcn_make_buffer_rsrc((void *)act, (short)0, act_bytes, 0x00020000);
    st.actr_none = __builtin_amdgcn_make_buffer_rsrc((void *)act, (short)0, 0, 0x00020000);
  }
  st.ksteps = K / kKT;
  const int klast = st.ksteps - 1;
  // The tile's 32-row blocks (clamped to 1..kRB for any map), taken MRB at a
  // time: the full-tile kernel makes one pass, the MRB = 1 kernel one pass
  // per block (each rebuilding the weights; it is launched for small batches,
  // where nearly every tile has a single block). Passes after the first reuse
  // the scale table.
  const int rows = row_end - row_begin;
  const int tile_blocks = min(max((rows + 31) / 32, 1), kRB);
  const int npass = MRB == kRB ? 1 : tile_blocks;
  // ---- this wavefront's two 32-row blocks of weight rows
  bool wave_on;  // wave-uniform: this wavefront has weight rows (both blocks: f, d % 64 == 0)
  int wrow0, wrow1;
  if (KIND == kGateUp) {
    const int unit = n0 + wave * 32;
    wave_on = unit < f;
    wrow0 = unit + (lane & 31);          // gate rows
    wrow1 = f + unit + (lane & 31);      // up rows
  } else {
    const int col = n0 + wave * 64;
    wave_on = col < d;
    wrow0 = col + (lane & 31);
    wrow1 = col + 32 + (lane & 31);
  }
  const int nrows_w = KIND == kGateUp ? 2 * f : d;
  const uint32_t R0 = wave_on ? (uint32_t)wrow0 : 0u, R1 = wave_on ? (uint32_t)wrow1 : 0u;
  st.codes = __builtin_amdgcn_make_buffer_rsrc((void *)(W.codes + ex * (size_t)nrows_w * (K / 2)),
                                               (short)0, nrows_w * (K / 2), 0x00020000);
  st.codes_none = __builtin_amdgcn_make_buffer_rsrc((void *)W.codes, (short)0, 0, 0x00020000);
  st.c_off[0] = R0 * (uint32_t)(K / 2) + (uint32_t)(lane >> 5) * 16u;
  st.c_off[1] = R1 * (uint32_t)(K / 2) + (uint32_t)(lane >> 5) * 16u;
  st.sbl = sbl;
  st.lr0 = wave * 64 + (lane & 31);
  st.a_lds = (uint32_t)wave * 1024u;
  // output staging, per wavefront: inside the ring for the full-tile kernel
  // and for MRB = 1 gate/up (8 KB), after the scale table for MRB = 1 down,
  // whose 16 KB would reach into the table that later passes reuse
  static_assert(kWaves * 32 * 64 <= kStages * stage_bytes<1>(), "gate/up staging fits in the ring");
  uint8_t *const ep_base =
      smem + (MRB == 1 && KIND == kDown
                  ? kStages * stage_bytes<MRB>() + (K / kGroup) * kWgCols * 4 : 0);
  bool fast = true;

  // one pass over rows pr_begin .. pr_end - 1; FIRST: the pass that loads
  // the scale table
  auto run_pass = [&](auto first_tag, const int pr_begin, const int pr_end) {
    constexpr bool FIRST = decltype(first_tag)::value;
    // the pass's active 32-row blocks (the same for every wavefront: the DMA
    // fills each row block with all four)
    const int tile_rb = MRB == 1 ? 1 : tile_blocks;
    // ---- prologue. The loads go out in dependency order so that their
    // latencies overlap: token indices (they gate the activation DMA), codes
    // of steps 0 and 1 and (first pass) the tile's scales (they need only the
    // tile), then the DMA of stages 0 and 1; the scale table is written while
    // the DMA is in flight.
    //
    // Activation rows: DMA instruction i of wavefront w fills rows
    // R i + 8 w .. +7 of the pass, R = 8 x wavefronts (1 KB, 16 bytes per
    // lane in lane order); lane l lands in row r = R i + 8 w + l / 8 at
    // 16-byte slot l % 8, which holds logical chunk (l % 8) ^ (r % 8) ^
    // ((r / 8) % 2) of the row (the swizzle; (r / 8) % 2 == w % 2 as R / 8 is
    // even). Rows past the pass's end re-read its last row (their results
    // are never stored), so every load is unconditional.
    int tok[MRB];
#pragma unroll
    for (int i = 0; i < MRB; ++i) {
      const int p = min(pr_begin + kDmaRows * i + 8 * wave + (lane >> 3), pr_end - 1);
      tok[i] = KIND == kGateUp ? (shared ? p - TK : sorted_token[p]) : p;
    }
    u32x4_t cr0[2], cr1[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      cr0[b] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(st.codes, st.c_off[b], 0, 0));
      cr1[b] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                               st.codes, st.c_off[b], min(1, klast) * (kKT / 2), 0));
    }
    // the scale/bias table (first pass): lane l of wavefront w fills column
    // 64 w + l, which is weight row R0 (l < 32) or R1 (l >= 32) of lane l %
    // 32, for all groups; the wavefront reads back only its own columns. The
    // same pass decides whether all of them allow the fast dequantisation.
    // Groups are taken 32 at a time with all their loads issued together.
    const int ng = K / kGroup;
    const size_t srow = (ex * (size_t)nrows_w + ((lane >> 5) ? R1 : R0)) * (size_t)ng;
    const uint16_t *sp = W.scales + srow, *bp = W.biases + srow;
    uint32_t *col = sbl + wave * 64 + lane;
    const bool vec = ng % 8 == 0;  // rows start 16-byte aligned: 16-byte loads
    uint4 sv[4], bv[4];
    if (FIRST && vec) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int g0 = min(8 * q, ng - 8);
        sv[q] = *(const uint4 *)(sp + g0);
        bv[q] = *(const uint4 *)(bp + g0);
      }
    }
    // token rows -> activation offsets, then the DMA of stages 0 and 1
    {
      const uint32_t j = (uint32_t)((lane & 7) ^ (lane >> 3) ^ (wave & 1));
#pragma unroll
      for (int i = 0; i < MRB; ++i) {
        const int t = KIND == kGateUp ? (tok[i] < 0 ? 0 : (tok[i] >= T ? T - 1 : tok[i])) : tok[i];
        st.a_off[i] = ((uint32_t)t * (uint32_t)K + j * 8u) * 2u;  // token clamped: in range for any routing
      }
    }
    // a later pass's DMA refills LDS that the previous pass's epilogue read
    if (!FIRST) lds_barrier();
    if constexpr (MRB == 1) {
      prologue_dma<1>(st, smem, klast);
    } else {
      switch (tile_rb) {
        case 1: prologue_dma<1>(st, smem, klast); break;
        case 2: prologue_dma<2>(st, smem, klast); break;
        case 3: prologue_dma<3>(st, smem, klast); break;
        default: prologue_dma<MRB>(st, smem, klast); break;
      }
    }
    if (FIRST) {
      bool fast_ok = true;
      if (vec) {
        for (int g0 = 0; g0 < ng; g0 += 32) {
          if (g0 > 0) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int g1 = min(g0 + 8 * q, ng - 8);
              sv[q] = *(const uint4 *)(sp + g1);
              bv[q] = *(const uint4 *)(bp + g1);
            }
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (g0 + 8 * q >= ng) break;
            const uint32_t su[4] = {sv[q].x, sv[q].y, sv[q].z, sv[q].w};
            const uint32_t bu[4] = {bv[q].x, bv[q].y, bv[q].z, bv[q].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t w0 = (su[e] & 0xFFFFu) | (bu[e] << 16);
              const uint32_t w1 = (su[e] >> 16) | (bu[e] & 0xFFFF0000u);
              col[(g0 + 8 * q + 2 * e) * kWgCols] = w0;
              col[(g0 + 8 * q + 2 * e + 1) * kWgCols] = w1;
              fast_ok &= (int)dq_fast_ok(w0) & (int)dq_fast_ok(w1);
            }
          }
        }
      } else {
        for (int g0 = 0; g0 < ng; ++g0) {
          const uint32_t w0 = (uint32_t)sp[g0] | ((uint32_t)bp[g0] << 16);
          col[g0 * kWgCols] = w0;
          fast_ok &= dq_fast_ok(w0);
        }
      }
      fast = __builtin_amdgcn_ballot_w64(!fast_ok) == 0;  // wave-uniform
    }
    st.nrb = wave_on ? tile_rb : 0;

    f32x16_t acc[MRB][2];
#pragma unroll
    for (int rb = 0; rb < MRB; ++rb) acc[rb][0] = acc[rb][1] = f32x16_t{0};
    // a wavefront with no weight rows runs the same loop (its share of the
    // DMA and the barriers are needed) and stores nothing
    if constexpr (MRB == 1) {
      tile_k_loop<1>(st, smem, acc, cr0, cr1, fast);
    } else {
      switch (tile_rb) {
        case 1: tile_k_loop<1>(st, smem, acc, cr0, cr1, fast); break;
        case 2: tile_k_loop<2>(st, smem, acc, cr0, cr1, fast); break;
        case 3: tile_k_loop<3>(st, smem, acc, cr0, cr1, fast); break;
        default: tile_k_loop<MRB>(st, smem, acc, cr0, cr1, fast); break;
      }
    }

    // ---- epilogue. Every wavefront's LDS reads of the ring have completed
    // before any wavefront reuses the LDS.
    lds_barrier();
    asm volatile("" ::: "memory");
    if (wave_on) {
      uint8_t *ep = ep_base + wave * (KIND == kGateUp ? MRB * 32 * 64 : MRB * 32 * 128);
      store_block<KIND, MRB>(acc, st.nrb, KIND == kGateUp ? n0 + wave * 32 : n0 + wave * 64,
                             shared, pr_begin, pr_end, TK, d, f, ep, out_bf16, out_f32);
    }
  };

  run_pass(std::true_type{}, row_begin, min(row_end, row_begin + MRB * 32));
  if constexpr (MRB == 1) {
    for (int pass = 1; pass < npass; ++pass) {
      const int pr_begin = row_begin + pass * 32;
      run_pass(std::false_type{}, pr_begin, min(row_end, pr_begin + 32));
    }
  }
}

// Batches of up to 32 tokens take the MRB = 1 kernel. With distinct experts
// per token (the library's own routing) no group has more rows than tokens,
// so every tile is one pass; caller ids that repeat an expert make taller
// groups, which take several passes. (Up to 64 tokens it was no faster: the
// shared expert's two-block tile, run as two passes, became the launch's
// longest work item.)
constexpr int kShortTileMaxT = 32;

static long long round_up8(long long n) { return (n + kXcds - 1) / kXcds * kXcds; }

// LDS of one GEMM workgroup for input width K: the activation ring and the
// scale/bias table (K/64 groups x 256 weight rows x 4 bytes), and the output
// staging (per wavefront its rows x 128 bytes for down, x 64 for gate/up):
// over the ring and table in the full-tile kernel, after the table in the
// MRB = 1 down kernel.
template <int KIND, int MRB>
static size_t gemm_lds_bytes(int K) {
  const size_t loop = (size_t)kStages * stage_bytes<MRB>() + (size_t)(K / kGroup) * kWgCols * 4;
  const size_t epilogue = (size_t)kWaves * MRB * 32 * (KIND == kGateUp ? 64 : 128);
  if (MRB == 1 && KIND == kDown) return loop + epilogue;
  return loop > epilogue ? loop : epilogue;
}

// More than 64 KB of dynamic LDS needs a per-kernel opt-in (once per process).
static hipError_t gemm_setup() {
  static const hipError_t st = [] {
    const void *kernels[4] = {(const void *)grouped_gemm_w4_kernel<kGateUp, kRB>,
                              (const void *)grouped_gemm_w4_kernel<kDown, kRB>,
                              (const void *)grouped_gemm_w4_kernel<kGateUp, 1>,
                              (const void *)grouped_gemm_w4_kernel<kDown, 1>};
    const int max_lds[4] = {(int)gemm_lds_bytes<kGateUp, kRB>(kGemmMaxK),
                            (int)gemm_lds_bytes<kDown, kRB>(kGemmMaxK),
                            (int)gemm_lds_bytes<kGateUp, 1>(kGemmMaxK),
                            (int)gemm_lds_bytes<kDown, 1>(kGemmMaxK)};
    hipError_t e = hipSuccess;
    for (int i = 0; i < 4 && e == hipSuccess; ++i)
      e = hipFuncSetAttribute(kernels[i], hipFuncAttributeMaxDynamicSharedMemorySize, max_lds[i]);
    return e;
  }();
  return st;
}

hipError_t launch_gate_up(const Dims &dm, const uint16_t *x, const Weights &w,
                          const int32_t *sorted_token, const int32_t *tile_map,
                          const int32_t *num_tiles, uint16_t *h, hipStream_t s) {
  if (gemv_supported(dm)) return launch_gate_up_gemv(dm, x, w, sorted_token, tile_map, num_tiles, h, s);
  if (const hipError_t e = gemm_setup()) return e;
  const int nblk = (dm.f + kWgCols / 2 - 1) / (kWgCols / 2);
  const int grid = (int)(nblk * round_up8(tile_capacity(dm)));
  if (dm.T <= kShortTileMaxT)
    grouped_gemm_w4_kernel<kGateUp, 1><<<grid, kThreads, gemm_lds_bytes<kGateUp, 1>(dm.d), s>>>(
        x, w.w13, w.s13, sorted_token, tile_map, num_tiles, h, nullptr, dm.T, dm.d, dm.f, dm.E,
        dm.k);
  else
    grouped_gemm_w4_kernel<kGateUp, kRB><<<grid, kThreads, gemm_lds_bytes<kGateUp, kRB>(dm.d), s>>>(
        x, w.w13, w.s13, sorted_token, tile_map, num_tiles, h, nullptr, dm.T, dm.d, dm.f, dm.E,
        dm.k);
  return hipGetLastError();
}

hipError_t launch_down(const Dims &dm, const uint16_t *h, const Weights &w,
                       const int32_t *tile_map, const int32_t *num_tiles, uint16_t *o_routed,
                       float *o_shared, hipStream_t s) {
  if (gemv_supported(dm)) return launch_down_gemv(dm, h, w, tile_map, num_tiles, o_routed, o_shared, s);
  if (const hipError_t e = gemm_setup()) return e;
  const int nblk = (dm.d + kWgCols - 1) / kWgCols;
  const int grid = (int)(nblk * round_up8(tile_capacity(dm)));
  if (dm.T <= kShortTileMaxT)
    grouped_gemm_w4_kernel<kDown, 1><<<grid, kThreads, gemm_lds_bytes<kDown, 1>(dm.f), s>>>(
        h, w.w2, w.s2, nullptr, tile_map, num_tiles, o_routed, o_shared, dm.T, dm.d, dm.f, dm.E,
        dm.k);
  else
    grouped_gemm_w4_kernel<kDown, kRB><<<grid, kThreads, gemm_lds_bytes<kDown, kRB>(dm.f), s>>>(
        h, w.w2, w.s2, nullptr, tile_map, num_tiles, o_routed, o_shared, dm.T, dm.d, dm.f, dm.E,
        dm.k);
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
