// Device helpers shared by the gfx950 kernels: vector types for the matrix
// core builtins, bf16 rounding, wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tte {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr int WAVE = 64;

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Two floats to bf16 (round to nearest even) in one instruction
// (v_cvt_pk_bf16_f32): a in the low half, b in the high half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// Wave-wide sum / max, returned to every lane.  DPP lane moves (no LDS
// round trip): swaps within quads, the half-row and row mirrors give every
// lane its 16-lane row's result; row_bcast:15 and row_bcast:31 (gfx9) then
// fold rows 0..3 into lane 63, which readlane broadcasts.  The combining
// order is fixed, so results are deterministic.  `id` is the operation's
// identity, which lanes of rows a broadcast step leaves out receive.
#define TTE_DPP(x, ctrl, row_mask, id)                                                                          \
  __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(id), __float_as_int(x), (ctrl), (row_mask), 0xF, \
                                             false))

__device__ __forceinline__ float wave_sum(float v) {
  v += TTE_DPP(v, 0xB1, 0xF, 0.f);   // quad_perm [1, 0, 3, 2]
  v += TTE_DPP(v, 0x4E, 0xF, 0.f);   // quad_perm [2, 3, 0, 1]
  v += TTE_DPP(v, 0x141, 0xF, 0.f);  // row_half_mirror
  v += TTE_DPP(v, 0x140, 0xF, 0.f);  // row_mirror
  v += TTE_DPP(v, 0x142, 0xA, 0.f);  // row_bcast:15 into rows 1 and 3
  v += TTE_DPP(v, 0x143, 0xC, 0.f);  // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_max(float v) {
  const float id = -__builtin_huge_valf();
  v = fmaxf(v, TTE_DPP(v, 0xB1, 0xF, id));
  v = fmaxf(v, TTE_DPP(v, 0x4E, 0xF, id));
  v = fmaxf(v, TTE_DPP(v, 0x141, 0xF, id));
  v = fmaxf(v, TTE_DPP(v, 0x140, 0xF, id));
  v = fmaxf(v, TTE_DPP(v, 0x142, 0xA, id));
  v = fmaxf(v, TTE_DPP(v, 0x143, 0xC, id));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
#undef TTE_DPP

// The largest b with a[b] <= v in the strictly increasing a[0..n] (a[0] <=
// v), returned to every lane: the whole wave reads the n + 1 entries 64 at
// a time and counts those <= v, so a pack's texts cost one load round
// instead of a binary search's chain of dependent loads.  Every lane of the
// wave must call it, with the same v.
__device__ __forceinline__ int wave_find(const int* __restrict__ a, int n, int v) {
  const int lane = (int)__lane_id();
  int count = 0;
  for (int base = 0; base <= n; base += WAVE) {
    const int i = base + lane;
    const uint64_t m = __ballot(i <= n && a[i] <= v);
    count += __popcll(m);
    if (m != ~0ull) break;
  }
  return count - 1;
}

// 7-bit row code: clamp(rint(x * inv), -63, 63) with ties to even.
__device__ __forceinline__ int quant7(float x, float inv) {
  float q = __builtin_rintf(x * inv);
  q = fminf(fmaxf(q, -63.f), 63.f);
  return (int)q;
}

// Erf-form GELU in fp32: gelu(a) = a * Phi(a), Phi the standard normal CDF.
// Phi comes from erfc by the rational approximation of Abramowitz & Stegun,
// Handbook of Mathematical Functions, formula 7.1.26: for z >= 0,
// erfc(z) = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-z^2) with
// t = 1 / (1 + p z) and absolute error <= 1.5e-7.  With z = |a| / sqrt(2)
// and h = 1/2 - erfc(z)/2, Phi(a) = 1/2 + sign(a) h, so
// gelu(a) = a/2 + |a| h.  In fp32 the result is within 4.7e-7 of the exact
// GELU over |a| <= 12 (and exact to fp32 beyond), as close as
// 0.5 a (1 + erff(a / sqrt(2))) in fp32, in 13 instructions.
__device__ __forceinline__ float gelu_erf(float a) {
  constexpr float P = 0.3275911f * 0.70710678118654752f;  // p / sqrt(2): t from |a| directly
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(P, fabsf(a), 1.f));
  // erfc(z)/2 = t * poly(t) * exp(-z^2), the coefficients halved
  float p = __builtin_fmaf(t, 0.5f * 1.061405429f, 0.5f * -1.453152027f);
  p = __builtin_fmaf(t, p, 0.5f * 1.421413741f);
  p = __builtin_fmaf(t, p, 0.5f * -0.284496736f);
  p = __builtin_fmaf(t, p, 0.5f * 0.254829592f);
  // exp(-z^2) = 2^(-a^2 log2(e) / 2)
  const float e = __builtin_amdgcn_exp2f(a * a * (-0.5f * 1.4426950408889634f));
  const float h = __builtin_fmaf(-t * p, e, 0.5f);
  return __builtin_fmaf(fabsf(a), h, 0.5f * a);
}

// s_waitcnt vmcnt(n), expcnt and lgkmcnt left at their maxima (gfx9
// encoding: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14).
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
#define TTE_W(k) \
  case k: __builtin_amdgcn_s_waitcnt(0x0F70 | ((k) & 15) | ((((k) >> 4) & 3) << 14)); break;
    TTE_W(0) TTE_W(1) TTE_W(2) TTE_W(3) TTE_W(4) TTE_W(5) TTE_W(6) TTE_W(7) TTE_W(8) TTE_W(9) TTE_W(10)
    TTE_W(11) TTE_W(12) TTE_W(13) TTE_W(14) TTE_W(15) TTE_W(16) TTE_W(17) TTE_W(18) TTE_W(19) TTE_W(20)
#undef TTE_W
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
  }
}

typedef __attribute__((address_space(3))) void* lds_ptr;

// One direct-to-LDS load (global_load_lds_dwordx4): each lane's 16 bytes at
// g go to LDS l + 16 * lane (l must be the same for the whole wave).  Kept
// a plain (non-template) function: the builtin inside templated kernels
// loses the host-side kernel stub in this compiler.
__device__ __forceinline__ void dma16(const void* g, uint8_t* l) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr)l, 16, 0, 0);
}

}  // namespace tte
