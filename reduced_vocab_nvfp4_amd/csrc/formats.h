// Weight formats of the draft-head GEMV kernels (device side).
//
// Three row-major weight layouts share the kernels; each is described by a
// policy struct used as a template argument:
//   Nvfp4  page 3 ("...MTP-NVFP4-h98k", "How it was built"): e2m1 codes, two
//          per byte (low nibble = even element), one E4M3 scale per 16
//          elements in a separate array, a float32 global scale;
//   E4m3   page 2 ("FP8 MTP draft stack for vLLM", _fp8_convert_draft_head):
//          one OCP e4m3fn byte per element and one float32 scale for the
//          whole tensor;
//   Bf16   the stock target head (page 4, the unmodified drafter reads the
//          full BF16 lm_head every draft step): raw BF16 elements.
// A "chunk" is 16 bytes of one row (EPC elements): the unit of the 128-bit
// loads.  A "unit" is 8 bytes (EPU elements): the unit of the generic kernel.
//
// Every decode below is exact: e2m1 and E4M3 values, and their products with
// an E4M3 scale (at most 6 significant bits, magnitudes 2^-10 .. 2688), are
// representable in BF16 and binary32.  Products with BF16 activations are
// accumulated in binary32 (v_dot2_f32_bf16 or the MFMA's fp32 accumulator).
#pragma once

#include "dh_device.h"

namespace dh {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

enum WeightFormat : int { FMT_NVFP4 = 0, FMT_E4M3 = 1, FMT_BF16 = 2 };

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) {
  return __builtin_bit_cast(bf16x2, u);
}

__device__ __forceinline__ float dot2(uint32_t w, uint32_t h, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w), as_bf16x2(h), acc,
                                         false);
}

__device__ __forceinline__ uint32_t bf16x2_bits(bf16x2 v) {
  return __builtin_bit_cast(uint32_t, v);
}

// ------------------------------------------------------------------ NVFP4

// Eight e2m1 weights (one dword of nibbles) against four BF16 pairs of h.
// v_cvt_scalef32_pk_bf16_fp4 with scale 1.0 turns byte SEL into a BF16 pair
// (low nibble in the low half), exactly.
__device__ __forceinline__ float fp4_dot8(uint32_t w, const uint32_t* hp,
                                          float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(
      __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0), as_bf16x2(hp[0]),
      acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(
      __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1), as_bf16x2(hp[1]),
      acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(
      __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2), as_bf16x2(hp[2]),
      acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(
      __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3), as_bf16x2(hp[3]),
      acc, false);
  return acc;
}

// Four e2m1 weights of byte SEL of w, times the block scale s, as BF16 pairs
// for an MFMA operand (the fp32 products are exact, so is the conversion).
template <int SEL>
__device__ __forceinline__ uint32_t fp4_scaled_pair(uint32_t w, float s) {
  const f32x2 x = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
  bf16x2 r;
  r.x = (__bf16)(x.x * s);
  r.y = (__bf16)(x.y * s);
  return bf16x2_bits(r);
}

struct Nvfp4 {
  static constexpr int kFmt = FMT_NVFP4;
  static constexpr int EPC = 32;  // elements per 16-byte chunk
  static constexpr int EPU = 16;  // elements per 8-byte unit (one block)
  static constexpr bool SCALED = true;
  static constexpr bool FP8_ACT = false;  // h is BF16

  // One chunk (two 16-element blocks; their E4M3 scales in bytes 0/1 of sb)
  // against EPC/2 = 16 BF16 pairs of h.
  __device__ static __forceinline__ float chunk_dot(const uint4& p,
                                                    uint32_t sb,
                                                    const uint32_t* hp,
                                                    float acc) {
    const float b0 = fp4_dot8(p.y, hp + 4, fp4_dot8(p.x, hp, 0.0f));
    const float b1 = fp4_dot8(p.w, hp + 12, fp4_dot8(p.z, hp + 8, 0.0f));
    acc = fmaf(__builtin_amdgcn_cvt_f32_fp8(sb, 0), b0, acc);
    acc = fmaf(__builtin_amdgcn_cvt_f32_fp8(sb, 1), b1, acc);
    return acc;
  }

  // One 8-byte unit = one block, scale byte in the low byte of sc.
  __device__ static __forceinline__ float unit_dot(const uint2& p,
                                                   uint32_t sc,
                                                   const uint32_t* hp,
                                                   float acc) {
    const float b = fp4_dot8(p.y, hp + 4, fp4_dot8(p.x, hp, 0.0f));
    return fmaf(__builtin_amdgcn_cvt_f32_fp8(sc, 0), b, acc);
  }

  // MFMA operand T (elements 8T .. 8T+7 of the chunk, all in block T/2):
  // the dequantized weights e2m1 * e4m3 as eight BF16.  The chunk's two
  // scale bytes are bytes SB and SB + 1 of sb.
  template <int T, int SB = 0>
  __device__ static __forceinline__ bf16x8 operand(const uint4& p,
                                                   uint32_t sb) {
    const uint32_t w = T == 0 ? p.x : T == 1 ? p.y : T == 2 ? p.z : p.w;
    const float s = __builtin_amdgcn_cvt_f32_fp8(sb, SB + T / 2);
    const uint4 r = make_uint4(fp4_scaled_pair<0>(w, s), fp4_scaled_pair<1>(w, s),
                               fp4_scaled_pair<2>(w, s), fp4_scaled_pair<3>(w, s));
    return __builtin_bit_cast(bf16x8, r);
  }
};

// ------------------------------------------------------------------- E4M3

// Two E4M3 bytes (word SEL of w, low byte first) as an exact BF16 pair.
template <bool HI>
__device__ __forceinline__ uint32_t fp8_pair(uint32_t w) {
  return bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

__device__ __forceinline__ float fp8_dot4(uint32_t w, const uint32_t* hp,
                                          float acc) {
  acc = dot2(fp8_pair<false>(w), hp[0], acc);
  return dot2(fp8_pair<true>(w), hp[1], acc);
}

struct E4m3 {
  static constexpr int kFmt = FMT_E4M3;
  static constexpr int EPC = 16;
  static constexpr int EPU = 8;
  static constexpr bool SCALED = false;
  static constexpr bool FP8_ACT = false;  // h is BF16

  __device__ static __forceinline__ float chunk_dot(const uint4& p, uint32_t,
                                                    const uint32_t* hp,
                                                    float acc) {
    acc = fp8_dot4(p.x, hp, acc);
    acc = fp8_dot4(p.y, hp + 2, acc);
    acc = fp8_dot4(p.z, hp + 4, acc);
    return fp8_dot4(p.w, hp + 6, acc);
  }

  __device__ static __forceinline__ float unit_dot(const uint2& p, uint32_t,
                                                   const uint32_t* hp,
                                                   float acc) {
    return fp8_dot4(p.y, hp + 2, fp8_dot4(p.x, hp, acc));
  }

  template <int T, int SB = 0>
  __device__ static __forceinline__ bf16x8 operand(const uint4& p, uint32_t) {
    const uint32_t w0 = T == 0 ? p.x : p.z, w1 = T == 0 ? p.y : p.w;
    const uint4 r = make_uint4(fp8_pair<false>(w0), fp8_pair<true>(w0),
                               fp8_pair<false>(w1), fp8_pair<true>(w1));
    return __builtin_bit_cast(bf16x8, r);
  }
};

// The same E4M3 head against E4M3 activation codes (the W8A8 step): both
// MFMA operands are raw E4M3 bytes (v_mfma_f32_16x16x32_fp8_fp8), so the
// weights need no decode at all; h is staged as the tokens' codes, one byte
// per element.  The products of two E4M3 values are exact in fp32.
struct E4m3Fp8 {
  static constexpr int kFmt = FMT_E4M3;
  static constexpr int EPC = 16;
  static constexpr int EPU = 8;
  static constexpr bool SCALED = false;
  static constexpr bool FP8_ACT = true;

  // MFMA operand T: bytes 8T .. 8T+7 of the chunk, as they are
  template <int T>
  __device__ static __forceinline__ uint64_t operand8(const uint4& p) {
    return T == 0 ? ((uint64_t)p.y << 32 | p.x) : ((uint64_t)p.w << 32 | p.z);
  }
};

// ------------------------------------------------------------------- BF16

struct Bf16 {
  static constexpr int kFmt = FMT_BF16;
  static constexpr int EPC = 8;
  static constexpr int EPU = 4;
  static constexpr bool SCALED = false;
  static constexpr bool FP8_ACT = false;  // h is BF16

  __device__ static __forceinline__ float chunk_dot(const uint4& p, uint32_t,
                                                    const uint32_t* hp,
                                                    float acc) {
    acc = dot2(p.x, hp[0], acc);
    acc = dot2(p.y, hp[1], acc);
    acc = dot2(p.z, hp[2], acc);
    return dot2(p.w, hp[3], acc);
  }

  __device__ static __forceinline__ float unit_dot(const uint2& p, uint32_t,
                                                   const uint32_t* hp,
                                                   float acc) {
    return dot2(p.y, hp[1], dot2(p.x, hp[0], acc));
  }

  template <int T, int SB = 0>
  __device__ static __forceinline__ bf16x8 operand(const uint4& p, uint32_t) {
    return __builtin_bit_cast(bf16x8, p);
  }
};

}  // namespace dh
