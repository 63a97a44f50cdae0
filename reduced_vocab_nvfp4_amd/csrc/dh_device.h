// Device-side helpers of the draft-head kernels (gfx950 / CDNA4, wave64).
//
// Number formats (page 3, "...MTP-NVFP4-h98k", "How it was built": e2m1
// values, E4M3 block scales per 16 elements, a float32 global scale):
//   e2m1   sign bit 3, magnitude index bits 0-2 into {0,.5,1,1.5,2,3,4,6}
//   E4M3   OCP e4m3fn: bias 7, 3 mantissa bits, subnormals m*2^-9, max 448
// Every encoder here is exact: it works on the binary32 bit pattern or on
// comparisons against exactly representable midpoints, so the result does
// not depend on instruction-level rounding modes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dh {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// E4M3 code of a non-negative binary32, rounded to nearest-even, saturating
// at 448 (code 0x7E); the NaN code 0x7F is never produced.
__device__ __forceinline__ uint32_t e4m3_encode_nonneg(float s) {
  if (!(s < 448.0f)) return 0x7Eu;
  if (s < 0.015625f) {
    // Below the smallest normal 2^-6 the grid step is 2^-9: scale by 2^9
    // (exact) and round to an integer, ties to even (v_rndne_f32).
    return (uint32_t)__builtin_rintf(s * 512.0f);
  }
  // Normal range: keep 3 of the 23 mantissa bits with round-to-nearest-even
  // on the bit pattern (a carry moves into the exponent), then rebias the
  // exponent from 127 to 7.
  uint32_t u = __float_as_uint(s);
  u += 0x7FFFFu + ((u >> 20) & 1u);
  return (u >> 20) - (120u << 3);
}

// Value of a non-negative E4M3 code (0x00..0x7E), exact.
__device__ __forceinline__ float e4m3_decode_nonneg(uint32_t c) {
  uint32_t e = c >> 3, m = c & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20))
           : (float)m * 0.001953125f;  // m * 2^-9
}

// e2m1 magnitude index of a non-negative binary32, round-to-nearest-even,
// saturating at 6: count the midpoints passed.  A value equal to a
// midpoint goes to the even index (0.25->0, 0.75->2, 1.25->2, 1.75->4,
// 2.5->4, 3.5->6, 5->6).
__device__ __forceinline__ uint32_t e2m1_encode_mag(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) +
         (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
         (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
}

// ------------------------------------------------------------ LDS copies

// global_load_lds_dwordx4: the 16 bytes at src of each lane land in LDS at
// lds_base + 16 * lane (lds_base wave-uniform).  The LDS address travels in
// M0, which the compiler loads itself for the asm's "{m0}" input operand.
// This is inline assembly rather than __builtin_amdgcn_global_load_lds
// because with the builtin the compiler waits for every outstanding vector
// load (vmcnt(0)) before the first LDS read that follows, which would also
// wait for the weight loads issued after the copy.  The compiler does not
// know that the copy writes LDS: the caller waits for it with an explicit
// s_waitcnt before reading the destination (vector memory loads retire in
// issue order).
__device__ __forceinline__ void lds_copy_x4(const void* src,
                                            uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "{m0}"(lds_base)
               : "memory");
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)p);
}

// Block barrier for LDS traffic only: waits for this wave's LDS operations
// (lgkmcnt), then s_barrier.  __syncthreads also waits for every
// outstanding vector memory operation (its workgroup release fence), which
// in the GEMV kernels means the ring's last, unused loads: a memory round
// trip for nothing.  The "memory" clobbers keep LDS accesses on their side.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------------ reductions

// DPP control words (GCN/CDNA encoding).
enum : int {
  DPP_QUAD_1032 = 0xB1,      // quad_perm [1,0,3,2]
  DPP_QUAD_2301 = 0x4E,      // quad_perm [2,3,0,1]
  DPP_ROW_HALF_MIRROR = 0x141,
  DPP_ROW_MIRROR = 0x140,
  DPP_ROW_BCAST15 = 0x142,   // lane 15 of each row to the next row
  DPP_ROW_BCAST31 = 0x143,   // lane 31 to rows 2 and 3
};

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(
      0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of G lanes (G in {1,2,4,8,16,32,64}); every lane
// of a group ends with the group's sum.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 2) v += dpp_f32<DPP_QUAD_1032>(v);
  if constexpr (G >= 4) v += dpp_f32<DPP_QUAD_2301>(v);
  if constexpr (G >= 8) v += dpp_f32<DPP_ROW_HALF_MIRROR>(v);
  if constexpr (G >= 16) v += dpp_f32<DPP_ROW_MIRROR>(v);
  if constexpr (G >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (G >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// Argmax order: a larger value wins; equal values go to the lower row.
// -0.0 == +0.0 under IEEE comparison, so signed zeros tie.
__device__ __forceinline__ bool better(float v, int r, float bv, int br) {
  return v > bv || (v == bv && r < br);
}

// (value, row) argmax over the whole wave with DPP moves (no LDS round
// trips): quad swaps and row mirrors give every lane its 16-lane row's best,
// row_bcast15 / row_bcast31 fold rows 0..3 into row 3, and lane 63's result
// is broadcast.  The order "larger value, then lower row" is a total order,
// so the combination order does not matter.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void argmax_step(float& v, int& r) {
  const float ov = __int_as_float(__builtin_amdgcn_update_dpp(
      __float_as_int(v), __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
  const int orow =
      __builtin_amdgcn_update_dpp(r, r, CTRL, ROW_MASK, 0xF, false);
  if (better(ov, orow, v, r)) {
    v = ov;
    r = orow;
  }
}

// (value, row) argmax within each 16-lane row: every lane ends with its
// row's best.
__device__ __forceinline__ void row_argmax(float& v, int& r) {
  argmax_step<DPP_QUAD_1032, 0xF>(v, r);
  argmax_step<DPP_QUAD_2301, 0xF>(v, r);
  argmax_step<DPP_ROW_HALF_MIRROR, 0xF>(v, r);
  argmax_step<DPP_ROW_MIRROR, 0xF>(v, r);
}

__device__ __forceinline__ void wave_argmax(float& v, int& r) {
  row_argmax(v, r);
  argmax_step<DPP_ROW_BCAST15, 0xA>(v, r);
  argmax_step<DPP_ROW_BCAST31, 0xC>(v, r);
  v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  r = __builtin_amdgcn_readlane(r, 63);
}

}  // namespace dh
