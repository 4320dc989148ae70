// Device-side building blocks shared by the libbdg kernels (gfx950, wave64).
//
// The packed-weight arithmetic here is the on-chip dequantisation of the
// pages: MXFP4 (FP4 E2M1 codes, one E8M0 scale per 32 K-elements; OCP MX
// v1.0) for the gpt-oss experts ("Sovereign gpt-oss-20B (MXFP4) on Apple
// Silicon", section 1), and group-quantized int4 w = (q - z) * s for the
// 30B-class model ("Single-stream int4 decode of a 30B MoE on Apple
// Silicon", section 6).  A 16-byte load carries 32 codes: one MX block, or
// half an int4 group of 64 (the 16-byte row loads of tracker entry D110).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bdg {

typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kChunkElems = 32;     // elements per 16-byte code chunk
constexpr int kXStride = 36;        // LDS floats per staged x chunk (32 + 4 pad)

// ---------------------------------------------------------------- global loads

// Loads through explicit global (address space 1) pointers: pointers read
// from kernel-argument structs or tables are generic to the compiler, which would otherwise emit
// flat loads.  Callers pass in-bounds addresses and issue these loads
// unconditionally (no branch around a load), so the compiler waits for a
// load's data only at its first use.
#define BDG_GLOBAL __attribute__((address_space(1)))

typedef unsigned int bdg_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int bdg_u32x2 __attribute__((ext_vector_type(2)));
typedef float bdg_f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ldg_u128(const void* p) {
  const bdg_u32x4 v = *reinterpret_cast<const BDG_GLOBAL bdg_u32x4*>(reinterpret_cast<uintptr_t>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ldg_u8(const void* p) {
  return *reinterpret_cast<const BDG_GLOBAL uint8_t*>(reinterpret_cast<uintptr_t>(p));
}
__device__ __forceinline__ uint32_t ldg_u16(const void* p) {
  return *reinterpret_cast<const BDG_GLOBAL uint16_t*>(reinterpret_cast<uintptr_t>(p));
}
__device__ __forceinline__ float4 ldg_f4(const void* p) {
  const bdg_f32x4 v = *reinterpret_cast<const BDG_GLOBAL bdg_f32x4*>(reinterpret_cast<uintptr_t>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ldg_u64(const void* p) {
  const bdg_u32x2 v = *reinterpret_cast<const BDG_GLOBAL bdg_u32x2*>(reinterpret_cast<uintptr_t>(p));
  return make_uint2(v.x, v.y);
}

// ---------------------------------------------------------------- block barrier

// A barrier for LDS hand-offs between the waves of a block, issued while
// global loads are still in flight: each wave waits for its own LDS
// accesses only (lgkmcnt 0), then meets the others at s_barrier.
// __syncthreads() would also wait for every outstanding global load of the
// wave (its workgroup-scope release fence waits for vmcnt 0), so a block
// that stages x or h after issuing its weight loads could not start on the
// first rows before the last rows had arrived.  The wavefront-scope fences
// only keep the compiler from moving memory accesses across the barrier.
// Not for hand-offs through global memory.
__device__ __forceinline__ void block_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // gfx9 encoding: lgkmcnt(0), vmcnt and expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------- scalars

// E8M0 byte -> fp32 2^(e-127).  e = 0 is the fp32 subnormal 2^-127,
// e = 255 is NaN.  Built from bits, no arithmetic.
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  uint32_t bits = (e == 0u) ? 0x00400000u : (e == 255u ? 0x7FC00000u : (e << 23));
  return __uint_as_float(bits);
}

// FP4 E2M1 code -> fp32, exact, integer-only (sign bit 3, exponent bits 2..1
// with bias 1, mantissa bit 0; exponent field 0 is the subnormal 0.5*m).
// Magnitudes 2..7 are 1.0 + (mag-2)*0.5 steps in the fp32 exponent/mantissa
// field, i.e. 0x3F800000 + (mag-2) << 22.
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  uint32_t mag = c & 7u;
  uint32_t bits = mag < 2u ? (mag ? 0x3F000000u : 0u) : (0x3F800000u + ((mag - 2u) << 22));
  return __uint_as_float(bits | ((c & 8u) << 28));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);   // quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// ---------------------------------------------------------------- cross-lane sums

__device__ __forceinline__ float dpp_quad_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_quad_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}
// ds_swizzle in bit-mask mode: lane' = lane ^ M within each group of 32 lanes
template <int M>
__device__ __forceinline__ float swz_xor(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (M << 10) | 0x1F));
}

// A value plus its partner's at lane ^ 16 / lane ^ 32, by gfx950's permlane
// swaps of a register with itself (the two results hold the pair in either
// order, so every lane gets the same sum).
__device__ __forceinline__ float add_pair16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_pair32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over aligned groups of L lanes (L in {4, 8, 16, 32, 64}); every lane of
// a group receives the group's sum.  All steps stay in the VALU (quad DPP,
// row half-mirror and mirror, permlane swaps).  Fixed order: deterministic.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(L == 4 || L == 8 || L == 16 || L == 32 || L == 64, "group size");
  v += dpp_quad_xor1(v);
  v += dpp_quad_xor2(v);
  if constexpr (L > 4) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  if constexpr (L > 8) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  if constexpr (L > 16) v = add_pair16(v);
  if constexpr (L > 32) v = add_pair32(v);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }

// One DPP move of a 32-bit value (lanes with no source, or outside ROW_MASK,
// get 0).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xF, false));
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xF, false);
}

// Sum over aligned groups of L lanes, valid only in the LAST lane of each
// group (lane L-1, 2L-1, ...).  All steps are DPP moves inside the VALU (row
// shifts, then the GFX9 row broadcasts across rows), no LDS round trip:
// after row_shr 1, 2, 4, 8 lane 15 of each 16-lane row holds its row sum;
// row_bcast:15 adds row r-1's lane 15 into rows 1 and 3, row_bcast:31 adds
// lane 31 into rows 2 and 3.  Lanes with no source read the old value 0.
// Fixed order: deterministic.
template <int L>
__device__ __forceinline__ float group_sum_last(float v) {
  static_assert(L == 4 || L == 8 || L == 16 || L == 32 || L == 64, "group size");
  v += dpp_f32<0x111, 0xF>(v);                          // row_shr:1
  v += dpp_f32<0x112, 0xF>(v);                          // row_shr:2
  if constexpr (L > 4) v += dpp_f32<0x114, 0xF>(v);     // row_shr:4
  if constexpr (L > 8) v += dpp_f32<0x118, 0xF>(v);     // row_shr:8
  if constexpr (L > 16) v += dpp_f32<0x142, 0xA>(v);    // row_bcast:15 into rows 1, 3
  if constexpr (L > 32) v += dpp_f32<0x143, 0xC>(v);    // row_bcast:31 into rows 2, 3
  return v;
}

// ---------------------------------------------------------------- chunk dot products

// MXFP4: unscaled sum_i E2M1(code_i) * x_i over one 16-byte chunk (32 codes),
// x in registers.  v_cvt_scalef32_pk_f32_fp4 decodes the two nibbles of the
// selected byte (low nibble first) with a unit scale; the E8M0 block scale is
// applied once to the block sum by the caller.
template <int SEL>
__device__ __forceinline__ f32x2 fp4_pair(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// Two interleaved partial sums (even and odd elements): enough independent
// chains for back-to-back wave64 issue, one add to combine them.
__device__ __forceinline__ float fp4_chunk_dot(const uint4 q, const float* __restrict__ x) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    f32x2 p0 = fp4_pair<0>(w[d]);
    f32x2 p1 = fp4_pair<1>(w[d]);
    f32x2 p2 = fp4_pair<2>(w[d]);
    f32x2 p3 = fp4_pair<3>(w[d]);
    a0 = __builtin_fmaf(p0.x, x[8 * d + 0], a0);
    a1 = __builtin_fmaf(p0.y, x[8 * d + 1], a1);
    a0 = __builtin_fmaf(p1.x, x[8 * d + 2], a0);
    a1 = __builtin_fmaf(p1.y, x[8 * d + 3], a1);
    a0 = __builtin_fmaf(p2.x, x[8 * d + 4], a0);
    a1 = __builtin_fmaf(p2.y, x[8 * d + 5], a1);
    a0 = __builtin_fmaf(p3.x, x[8 * d + 6], a0);
    a1 = __builtin_fmaf(p3.y, x[8 * d + 7], a1);
  }
  return a0 + a1;
}

// int4: sum_i q_i * x_i over one 16-byte chunk (32 unsigned nibbles).
// A nibble q placed in a byte reads as the FP8 E4M3 value q * 2^-9 exactly
// (exponent field 0 is the subnormal m * 2^-9, exponent field 1 gives
// (8 + m) * 2^-9), so v_cvt_scalef32_pk_f32_fp8 with scale 2^9 turns two
// nibble bytes into two exact fp32 integers.  The even elements of a dword
// are its low-nibble plane, the odd ones its high-nibble plane.
// The zero point is folded by the caller: sum (q - z) x = sum q x - z sum x.
template <bool HI_WORD>
__device__ __forceinline__ f32x2 u4_pair(uint32_t plane) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(plane, 512.0f, HI_WORD);
}

__device__ __forceinline__ float u4_chunk_dot(const uint4 q, const float* __restrict__ x) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t lo = w[d] & 0x0F0F0F0Fu;          // elements 8d + 0, 2, 4, 6
    const uint32_t hi = (w[d] >> 4) & 0x0F0F0F0Fu;   // elements 8d + 1, 3, 5, 7
    const f32x2 e02 = u4_pair<false>(lo);
    const f32x2 e46 = u4_pair<true>(lo);
    const f32x2 e13 = u4_pair<false>(hi);
    const f32x2 e57 = u4_pair<true>(hi);
    a0 = __builtin_fmaf(e02.x, x[8 * d + 0], a0);
    a1 = __builtin_fmaf(e13.x, x[8 * d + 1], a1);
    a0 = __builtin_fmaf(e02.y, x[8 * d + 2], a0);
    a1 = __builtin_fmaf(e13.y, x[8 * d + 3], a1);
    a0 = __builtin_fmaf(e46.x, x[8 * d + 4], a0);
    a1 = __builtin_fmaf(e57.x, x[8 * d + 5], a1);
    a0 = __builtin_fmaf(e46.y, x[8 * d + 6], a0);
    a1 = __builtin_fmaf(e57.y, x[8 * d + 7], a1);
  }
  return a0 + a1;
}

// ---------------------------------------------------------------- packed-matrix view

enum Fmt : int { kMXFP4 = 0, kINT4G = 1 };

// One packed matrix (one expert) in the PLAIN layout.
struct QMat {
  const uint8_t* codes;    // [n][k/2]
  const uint8_t* scales;   // MXFP4: [n][k/32] bytes; INT4G: [n][k/group] fp16 (as bytes)
  const uint8_t* zeros;    // INT4G: [n][ceil(G/2)]
};

// Weighted contribution of chunk c of row r: scale * block partial.
// For int4, xsum is sum of the 32 x values of the chunk.
template <int FMT>
__device__ __forceinline__ float chunk_contrib(const uint4 q, uint32_t scale_raw, uint32_t zero_nib,
                                               const float* __restrict__ x, float xsum) {
  if constexpr (FMT == kMXFP4) {
    // block sum * 2^(e-127); e = 255 is NaN
    const float r = __builtin_amdgcn_ldexpf(fp4_chunk_dot(q, x), (int)scale_raw - 127);
    return scale_raw == 255u ? __uint_as_float(0x7FC00000u) : r;
  } else {
    const float s = f16_bits_to_f32((uint16_t)scale_raw);
    const float part = u4_chunk_dot(q, x) - (float)zero_nib * xsum;
    return part * s;
  }
}

}  // namespace bdg
