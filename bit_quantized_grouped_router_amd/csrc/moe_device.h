// Device-side helpers shared by the gfx950 kernels of the int4-g64 MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kGroup = 64;  // weights per (scale, bias) pair along the input dimension
constexpr int kWave = 64;   // CDNA wavefront width

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct W4 {
  const uint8_t *codes;
  const uint16_t *scales;
  const uint16_t *biases;
};

// Workgroup barrier ordering LDS only. __syncthreads() also orders global
// memory, which on gfx9 means waiting for every outstanding global load
// (vmcnt(0)); this barrier waits for LDS operations only, so loads issued
// ahead for later K steps stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Two fp32 values rounded to nearest-even bf16 and packed (a in the low half).
// On gfx950 this is one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t to_bf16(float a) {
  return __builtin_bit_cast(uint16_t, (__bf16)a);
}

// Dequantise eight consecutive columns of one row (one 32-bit word of codes,
// all in the same 64-column group): w = bf16_rne(fp32(s*q + b)).
// s*q is exact in fp32, so fmaf rounds exactly once, like a multiply then add.
// Result: four words of packed bf16 pairs, columns (0,1) (2,3) (4,5) (6,7).
__device__ __forceinline__ uint4 dequant8(uint32_t c, float s, float b) {
  const uint32_t lo = c & 0x0F0F0F0Fu;         // even columns: bytes' low nibbles
  const uint32_t hi = (c >> 4) & 0x0F0F0F0Fu;  // odd columns: bytes' high nibbles
  uint4 r;
  r.x = pack_bf16x2(fmaf(s, (float)(lo & 0xFFu), b), fmaf(s, (float)(hi & 0xFFu), b));
  r.y = pack_bf16x2(fmaf(s, (float)((lo >> 8) & 0xFFu), b), fmaf(s, (float)((hi >> 8) & 0xFFu), b));
  r.z = pack_bf16x2(fmaf(s, (float)((lo >> 16) & 0xFFu), b), fmaf(s, (float)((hi >> 16) & 0xFFu), b));
  r.w = pack_bf16x2(fmaf(s, (float)(lo >> 24), b), fmaf(s, (float)(hi >> 24), b));
  return r;
}

// Per (row, group) constants of the fast dequantisation below.
struct DqGroup {
  float s, s16, c0, c1;
  bool fast;
};

// The fast path builds each code q as an fp16 1024 + q (or 1024 + 16q) by
// OR-ing the nibble into the mantissa of 1024.0, and lets one mixed-precision
// FMA form s*(1024 + q) + (b - 1024 s) = s*q + b. That equals fp32(s*q + b)
// exactly when b - 1024 s and b - 64 s are exact in fp32 (then the FMA rounds
// once, like the plain formula): both are sums of two 8-bit significands, so
// they are exact when the exponents of b and s differ by -5 .. 21. The test
// below asks for that, with both exponents away from the fp32 range ends
// (s exponent 20 .. 230, b exponent <= 230; b is then a nonzero normal
// number). Every other group, zeros and non-finite values included, takes the
// plain path, which is exact for all inputs.
__device__ __forceinline__ bool dq_fast_ok(uint32_t sb) {
  const uint32_t es = (sb >> 7) & 0xFFu, eb = (sb >> 23) & 0xFFu;
  return (es - 20u) <= 210u && eb <= 230u && (eb - es + 5u) <= 26u;
}

// The constants of the fast path (meaningful when dq_fast_ok holds).
__device__ __forceinline__ DqGroup dq_consts(uint32_t sb) {
  DqGroup q;
  q.s = __uint_as_float(sb << 16);
  const float b = __uint_as_float(sb & 0xFFFF0000u);
  q.s16 = q.s * 0.0625f;
  q.c0 = fmaf(-1024.0f, q.s, b);
  q.c1 = fmaf(-64.0f, q.s, b);
  q.fast = true;
  return q;
}

__device__ __forceinline__ DqGroup dq_prepare(uint32_t sb) {
  DqGroup q = dq_consts(sb);
  q.fast = dq_fast_ok(sb);
  return q;
}

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Constants of the fast dequantisation, held in registers: gfx9 VOP3
// encodings take no literal operand, so v_and_or_b32 needs its masks in
// registers. The asm makes the values opaque to the compiler, which would
// otherwise fold them back into two VOP2 operations with literals (it is not
// volatile, so repeated calls are merged into one).
struct DqRegs {
  uint32_t m_lo, m_hi;  // 0x000F000F, 0x00F000F0 (scalar registers)
  uint32_t magic;       // 0x64006400: fp16 1024.0 in both halves (vector register)
};

__device__ __forceinline__ DqRegs dq_regs() {
  DqRegs r;
  asm("s_mov_b32 %0, 0x000f000f" : "=s"(r.m_lo));
  asm("s_mov_b32 %0, 0x00f000f0" : "=s"(r.m_hi));
  asm("v_mov_b32 %0, 0x64006400" : "=v"(r.magic));
  return r;
}

// (a & m) | o in one VALU operation.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(o));
  return r;
}

// Fast path of dequant8 (see dq_fast_ok), bit-identical to it: each fp16
// operand 1024 + q (or 1024 + 16q) is built by one v_and_or_b32; 17 VALU
// operations for eight weights (one shift, four and-or, eight mixed FMAs,
// four packing conversions).
__device__ __forceinline__ uint4 dequant8_fast(uint32_t c, const DqGroup &q, const DqRegs &k) {
  const uint32_t y = c >> 8;
  const f16x2_t h0 = __builtin_bit_cast(f16x2_t, and_or(c, k.m_lo, k.magic));  // cols 0, 4
  const f16x2_t h1 = __builtin_bit_cast(f16x2_t, and_or(c, k.m_hi, k.magic));  // cols 1, 5
  const f16x2_t h2 = __builtin_bit_cast(f16x2_t, and_or(y, k.m_lo, k.magic));  // cols 2, 6
  const f16x2_t h3 = __builtin_bit_cast(f16x2_t, and_or(y, k.m_hi, k.magic));  // cols 3, 7
  uint4 r;
  r.x = pack_bf16x2(fmaf((float)h0[0], q.s, q.c0), fmaf((float)h1[0], q.s16, q.c1));
  r.y = pack_bf16x2(fmaf((float)h2[0], q.s, q.c0), fmaf((float)h3[0], q.s16, q.c1));
  r.z = pack_bf16x2(fmaf((float)h0[1], q.s, q.c0), fmaf((float)h1[1], q.s16, q.c1));
  r.w = pack_bf16x2(fmaf((float)h2[1], q.s, q.c0), fmaf((float)h3[1], q.s16, q.c1));
  return r;
}

// SiLU(g) * u with the hardware exp2 and reciprocal (about 1 ulp each): the
// product is rounded to bf16 afterwards, so a few fp32 ulps do not matter.
__device__ __forceinline__ float silu_mul_fast(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * g);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// 32 consecutive columns of one row (16 bytes of codes, one group), either path.
__device__ __forceinline__ void dequant32(uint4 c, uint32_t sb, uint4 out[4]) {
  const DqGroup q = dq_prepare(sb);
  if (q.fast) {
    const DqRegs k = dq_regs();
    out[0] = dequant8_fast(c.x, q, k);
    out[1] = dequant8_fast(c.y, q, k);
    out[2] = dequant8_fast(c.z, q, k);
    out[3] = dequant8_fast(c.w, q, k);
  } else {
    const float s = bf16_to_f32(sb & 0xFFFFu), b = bf16_to_f32(sb >> 16);
    out[0] = dequant8(c.x, s, b);
    out[1] = dequant8(c.y, s, b);
    out[2] = dequant8(c.z, s, b);
    out[3] = dequant8(c.w, s, b);
  }
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + expf(-g)) * u;
}

// Order-preserving 32-bit key of a router logit: larger logit -> larger key;
// -0 and +0 map to the same key; NaN maps below -inf (to 1). 0 is never a
// key, so it marks an empty or already chosen slot.
__device__ __forceinline__ uint32_t logit_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return v != v ? 1u : ord;
}

// The logit a key was made from (-0 comes back as +0, NaN as a NaN).
__device__ __forceinline__ float key_logit(uint32_t ord) {
  const uint32_t u = (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord;
  return __uint_as_float(u);
}

// Maximum of v over the wavefront, in a scalar register. Six DPP steps
// (lane swaps within quads, mirrors within 8 and 16 lanes, row broadcasts)
// leave the maximum in lane 63; no LDS traffic.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, false));   // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, false));   // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));  // row_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// v plus the value a DPP lane pattern brings in (lanes of rows outside
// row_mask add 0).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
  const int o = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, false);
  return v + __builtin_bit_cast(float, o);
}

// Sum over the wavefront with six DPP steps (no LDS traffic): pairs and
// quads, half-row and row mirrors, then the row broadcasts carry each row's
// total into the next; the sum ends in lane 63 and is returned to all lanes.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = dpp_add<0xb1, 0xf>(v);   // quad_perm 1,0,3,2
  v = dpp_add<0x4e, 0xf>(v);   // quad_perm 2,3,0,1
  v = dpp_add<0x141, 0xf>(v);  // row_half_mirror
  v = dpp_add<0x140, 0xf>(v);  // row_mirror
  v = dpp_add<0x142, 0xa>(v);  // row_bcast:15
  v = dpp_add<0x143, 0xc>(v);  // row_bcast:31
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Sum over aligned groups of L lanes, L = 2, 4, 8 or 16, with DPP: every lane
// of a group ends with the group's sum.
template <int L>
__device__ __forceinline__ float group_sum_dpp(float v) {
  static_assert(L == 2 || L == 4 || L == 8 || L == 16, "DPP groups of 2 to 16 lanes");
  v = dpp_add<0xb1, 0xf>(v);                   // pairs
  if constexpr (L >= 4) v = dpp_add<0x4e, 0xf>(v);   // quads
  if constexpr (L >= 8) v = dpp_add<0x141, 0xf>(v);  // half rows
  if constexpr (L >= 16) v = dpp_add<0x140, 0xf>(v); // rows
  return v;
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = width / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Top-k over E logits of one token by one wavefront (all 64 lanes active).
// Lane l holds experts l, l+64, l+128, ... Each of the k rounds takes the
// largest remaining key: a lane-local maximum, a DPP wavefront maximum, and,
// only when several lanes hold that same key, a second DPP pass for the
// lowest expert index among them. Returns, in lanes 0..k-1, the chosen
// expert (slot j in lane j, keys descending, equal keys by ascending index)
// and its logit. If fewer than k keys exist (k > E cannot happen), ids stay
// in [0, E).
// This lane's logits of one token: experts lane, lane + 64, ... All loads are
// unconditional (clamped index) so they are in flight together.
template <int kMaxPerLane>
__device__ __forceinline__ void wave_load_logits(const float *__restrict__ row, int E,
                                                 float (&v)[kMaxPerLane]) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + i * kWave;
    v[i] = row[e < E ? e : 0];
  }
}

// Selection for at most 4 logits per lane. Each lane first orders its keys
// descending with a stable odd-even transposition sort (adjacent swaps only
// on a strictly larger key, so equal keys keep ascending slots, i.e. the
// lower expert index first). A round then takes the wavefront maximum of the
// lanes' first keys; among lanes whose first key equals it, the lowest
// expert index (no lane holds an equal key further down with a lower index:
// its first key would equal the maximum too, with a lower slot). The winning
// lane shifts its list by one. Same result as the general selection below.
template <int kMaxPerLane>
__device__ __forceinline__ void wave_topk_sorted(const float (&v)[kMaxPerLane], int E, int k,
                                                 int *out_id, float *out_logit) {
  static_assert(kMaxPerLane >= 1 && kMaxPerLane <= 4, "sorted selection: up to 4 keys per lane");
  constexpr int M = kMaxPerLane;
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t key[4] = {0u, 0u, 0u, 0u};  // entries past M stay 0 (empty)
  int slot[4] = {0, 1, 2, 3};
#pragma unroll
  for (int i = 0; i < M; ++i) key[i] = lane + i * kWave < E ? logit_key(v[i]) : 0u;
#pragma unroll
  for (int pass = 0; pass < M; ++pass)
#pragma unroll
    for (int i = pass & 1; i + 1 < M; i += 2)
      if (key[i + 1] > key[i]) {
        const uint32_t tk = key[i];
        key[i] = key[i + 1];
        key[i + 1] = tk;
        const int ts = slot[i];
        slot[i] = slot[i + 1];
        slot[i + 1] = ts;
      }
  // the list's slots, one byte each (byte i: slot of key[i]), so that the
  // winning lane's shift below is one register shift
  uint32_t slots = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) slots |= (uint32_t)slot[i] << (8 * i);
  // the list as four named registers inside the loop
  uint32_t k0 = key[0], k1 = key[1], k2 = key[2], k3 = key[3];
  int my_id = 0;
  float my_logit = 0.f;
  for (int j = 0; j < k; ++j) {
    const uint32_t m = wave_max_u32(k0);
    const uint64_t tied = __builtin_amdgcn_ballot_w64(k0 == m);
    int wl = __builtin_ctzll(tied);
    if (__builtin_expect((tied & (tied - 1)) != 0, 0)) {
      // lowest expert index lane + 64 * slot among the lanes holding key m first
      const uint32_t idx = (uint32_t)(lane + kWave * (int)(slots & 0xffu));
      wl = (int)(~wave_max_u32(k0 == m ? ~idx : 0u) & (kWave - 1));
    }
    int id = wl + kWave * (int)(__builtin_amdgcn_readlane(slots, wl) & 0xffu);
    if (id >= E) id = 0;  // unreachable while k <= E; keeps ids in range
    // the winning lane drops its first key (selects, no branch)
    const bool win = lane == wl;
    k0 = win ? k1 : k0;
    k1 = win ? k2 : k1;
    k2 = win ? k3 : k2;
    k3 = win ? 0u : k3;
    slots = win ? slots >> 8 : slots;
    const bool mine = lane == j;
    my_id = mine ? id : my_id;
    my_logit = mine ? key_logit(m) : my_logit;
  }
  *out_id = my_id;
  *out_logit = my_logit;
}

// The selection on logits already in registers (as wave_load_logits leaves them).
template <int kMaxPerLane>
__device__ __forceinline__ void wave_topk_loaded(const float (&v)[kMaxPerLane], int E, int k,
                                                 int *out_id, float *out_logit) {
  if constexpr (kMaxPerLane <= 4) {
    wave_topk_sorted<kMaxPerLane>(v, E, k, out_id, out_logit);
    return;
  }
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t key[kMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) key[i] = lane + i * kWave < E ? logit_key(v[i]) : 0u;
  int my_id = 0;
  float my_logit = 0.f;
  for (int j = 0; j < k; ++j) {
    // lane-local best: the largest key, the lowest slot among equals
    uint32_t best = key[0];
    int bi = 0;
#pragma unroll
    for (int i = 1; i < kMaxPerLane; ++i)
      if (key[i] > best) {
        best = key[i];
        bi = i;
      }
    const uint32_t m = wave_max_u32(best);
    const uint64_t tied = __builtin_amdgcn_ballot_w64(best == m);
    int wl;
    if (__builtin_popcountll(tied) == 1) {
      wl = __builtin_ctzll(tied);
    } else {
      // lowest expert index lane + 64*slot among the lanes holding key m
      const uint32_t idx = (uint32_t)(lane + kWave * bi);
      wl = (int)(~wave_max_u32(best == m ? ~idx : 0u) & (kWave - 1));
    }
    const int wslot = __builtin_amdgcn_readlane(bi, wl);
    int id = wl + kWave * wslot;
    if (id >= E) id = 0;  // unreachable while k <= E; keeps ids in range
    if (lane == wl) {
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i)
        if (i == wslot) key[i] = 0u;
    }
    if (lane == j) {
      my_id = id;
      my_logit = key_logit(m);
    }
  }
  *out_id = my_id;
  *out_logit = my_logit;
}

template <int kMaxPerLane>
__device__ __forceinline__ void wave_topk(const float *__restrict__ row, int E, int k,
                                          int *out_id, float *out_logit) {
  float v[kMaxPerLane];
  wave_load_logits<kMaxPerLane>(row, E, v);
  wave_topk_loaded<kMaxPerLane>(v, E, k, out_id, out_logit);
}

}  // namespace moe
