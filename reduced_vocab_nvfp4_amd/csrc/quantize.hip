// Gather + quantization of the kept head rows on the device: NVFP4 (the
// method's format) and per-tensor E4M3 (the FP8 head it is compared with).
//
// Recipe (page 3, "...MTP-NVFP4-h98k", "How it was built"): global scale
// amax / (6*448), E4M3 block scales per 16 elements, e2m1 codes rounded to
// nearest-even.  Page 1 ("q38_draft.py", load_draft_model) feeds the
// quantizer the gathered rows W[dh_idx], so amax is taken over those rows.
// The 1e-12 floor on amax is the guard of page 2's FP8 head conversion.
//
// Three launches on the caller's stream:
//   1. k_gather_amax   max |x| over the gathered rows as an atomicMax on the
//                      binary32 bit pattern (exact and order-independent for
//                      non-negative floats);
//   2. k_nvfp4_encode  two lanes per 16-element block: block max, E4M3
//                      scale, 8 e2m1 codes per lane packed into 4 bytes;
//   3. k_quant_finish  writes the global scale and returns the amax slot of
//                      the workspace to zero.
// Every float result is the single IEEE binary32 operation the recipe names,
// with round-to-nearest-even (no contraction), in the order
// gs = max(amax,1e-12)/2688, s = bmax/(6*gs), q = x/(e4m3(s)*gs); the
// per-element quotients are the correctly rounded divisions, computed with
// Markstein's correction (below).
//
// Per-tensor E4M3 (page 2, "FP8 MTP draft stack for vLLM",
// _fp8_convert_draft_head: one scale amax/448 for the whole head, elements
// divided by it, clamped to +-448 and cast to e4m3fn): the same amax pass,
// then k_e4m3_encode with one thread per 8 elements, scale =
// max(amax,1e-12)/448, code = E4M3 of clamp(x/scale), sign kept (a negative
// zero quotient gives 0x80).
#include "dh_device.h"
#include "dh_internal.h"

namespace dh {

namespace {

constexpr int QTHREADS = 256;
constexpr int QWAVES = QTHREADS / 64;

__device__ __forceinline__ uint32_t abs_bf16_pair_max(uint32_t v) {
  uint32_t lo = v & 0x7FFFu, hi = (v >> 16) & 0x7FFFu;
  return lo > hi ? lo : hi;
}

__device__ __forceinline__ uint32_t abs_bf16_max8(const uint4& v) {
  uint32_t a = abs_bf16_pair_max(v.x), b = abs_bf16_pair_max(v.y);
  uint32_t c = abs_bf16_pair_max(v.z), d = abs_bf16_pair_max(v.w);
  a = a > b ? a : b;
  c = c > d ? c : d;
  return a > c ? a : c;
}

// Value of a 16-bit element: BF16, or (F16) IEEE binary16, both exact in
// binary32.  For either, the magnitude bits (bits & 0x7FFF) order like the
// magnitudes.
template <bool F16>
__device__ __forceinline__ float elem_f32(uint32_t bits16) {
  if constexpr (F16)
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
  return bf16_to_f32(bits16);
}

__device__ __forceinline__ float global_scale_from(uint32_t amax_bits) {
  float amax = __uint_as_float(amax_bits);
  return fmaxf(amax, 1e-12f) / 2688.0f;
}

// Correctly rounded quotients without a division per element.  Given
// rd = RN(1/d) (one correctly rounded division per divisor),
// q0 = RN(ax * rd) is within an ulp of ax / d, the residual
// r = ax - q0 * d is exact in one fma, and RN(q0 + r * rd) is the correctly
// rounded quotient (Markstein's correction).  The kernels use it for d in
// [2^-60, 2^60] and ax <= 2^60 (no overflow) and divide otherwise.  Where
// ax is below about 2^-100 the residual underflows and the result can be an
// ulp off, but the quotient is then below 2^-40, and every e2m1 and E4M3
// code of a quotient below 2^-11 is 0 whatever its last bits.  Equality
// with the division for every quotient of at least 2^-24, over every bf16
// ax in range, is checked by brute force on the CPU (tests/native).
__device__ __forceinline__ bool divisor_in_range(float d) {
  return d >= 0x1p-60f && d <= 0x1p60f;
}

// e2m1 magnitude index of RN-to-nearest-even of q >= 0 (or NaN -> 0),
// saturating at 6.  Below 1 the two midpoints 0.25 and 0.75 are counted
// (0.25 -> 0 and 0.75 -> 2 by ties-to-even); from 1 up the code is the
// float's exponent and top mantissa bit after rounding the pattern at that
// bit (a carry moves into the exponent).  Checked against counting all
// seven midpoints for every non-negative float and NaN.
__device__ __forceinline__ uint32_t e2m1_code(float q) {
  const uint32_t lo = (uint32_t)(q > 0.25f) + (uint32_t)(q >= 0.75f);
  const uint32_t u = __float_as_uint(q);
  const uint32_t t = u + 0x1FFFFFu + ((u >> 22) & 1u);
  uint32_t c = (t >> 22) - 252u;  // 1.0 = exponent 127 -> code 2
  c = c < 7u ? c : 7u;
  return q >= 1.0f ? c : lo;
}

// The gathered rows in tiles of 64 16-byte units (512 elements) of one row:
// a wave takes a tile, lane i its unit i, so the row and its source id are
// wave-uniform and every load instruction reads 1 KB contiguous.
struct Tiles {
  int64_t per_row, count;
  __device__ Tiles(int64_t hidden, int64_t n_rows)
      : per_row((hidden / 8 + 63) / 64), count(n_rows * per_row) {}
};

template <bool F16>
__global__ __launch_bounds__(QTHREADS) void k_gather_amax(
    const uint16_t* __restrict__ w, int64_t hidden,
    const int32_t* __restrict__ ids, int64_t n_rows,
    uint32_t* __restrict__ amax_bits) {
  const Tiles tl(hidden, n_rows);
  const int lane = threadIdx.x & 63;
  const int64_t upr = hidden / 8;
  const int64_t wave = (int64_t)blockIdx.x * QWAVES +
                       __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * QWAVES;
  uint32_t m = 0;
  // four tiles per round, all loads issued before any is used
  for (int64_t t0 = wave; t0 < tl.count; t0 += 4 * nwaves) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t t = t0 + u * nwaves;
      const int64_t j = t / tl.per_row;
      const int64_t k = (t - j * tl.per_row) * 64 + lane;
      v[u] = make_uint4(0u, 0u, 0u, 0u);
      if (t < tl.count && k < upr)
        v[u] = *reinterpret_cast<const uint4*>(w + (int64_t)ids[j] * hidden +
                                               k * 8);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t a = abs_bf16_max8(v[u]);
      m = m > a ? m : a;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    uint32_t o = __shfl_xor(m, off, 64);
    m = m > o ? m : o;
  }
  __shared__ uint32_t wmax[QWAVES];
  if (lane == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = wmax[0];
    for (int i = 1; i < QWAVES; ++i) r = r > wmax[i] ? r : wmax[i];
    // the binary32 bits of the largest magnitude: for non-negative values
    // their unsigned order is the numeric order
    if (r) atomicMax(amax_bits, __float_as_uint(elem_f32<F16>(r)));
  }
}

// Tiles per round of the encoders: all loads of a round are issued before
// any is used, so a wave keeps 4 KB in flight.
constexpr int ROUND = 4;

// Tile t of a round (last tiles first, see below): its row, first unit and
// the load of this lane's 16 bytes (a lane past the row's end re-reads the
// row's last block pair).  Tiles past the end repeat tile 0.
struct TileLoad {
  int64_t j, k;
  bool live;
  uint4 v;
};

__device__ __forceinline__ TileLoad load_tile(const uint16_t* w,
                                              int64_t hidden,
                                              const int32_t* ids,
                                              const Tiles& tl, int64_t i,
                                              int lane) {
  TileLoad r;
  const int64_t upr = hidden / 8;
  const int64_t t = i < tl.count ? tl.count - 1 - i : 0;
  r.j = t / tl.per_row;
  const int64_t k0 = (t - r.j * tl.per_row) * 64;
  r.live = i < tl.count && k0 + lane < upr;
  r.k = k0 + lane < upr ? k0 + lane : upr - 2 + (lane & 1);
  r.v = *reinterpret_cast<const uint4*>(w + (int64_t)ids[r.j] * hidden +
                                        r.k * 8);
  return r;
}

// Hardware converts with scale 1.0.  A hardware probe over every float bit
// pattern found:
//   * v_cvt_scalef32_pk_fp4_f32 rounds to the nearest e2m1 value, ties to
//     even, saturates at 6 and keeps the sign (-0 gives 0x8): exactly the
//     element code of the recipe applied to the quotient;
//   * v_cvt_scalef32_pk_fp8_f32 rounds to the nearest E4M3 value, ties to
//     even, up to 464, and gives the NaN code beyond: exact for inputs
//     clamped to +-448.
// src0 goes to the low nibble (fp4) or the low byte (fp8).
__device__ __forceinline__ uint32_t fp4_pair(uint32_t old, float a, float b,
                                             int byte) {
  switch (byte) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, 3);
  }
}

typedef short short2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t fp8_pair(float a, float b) {
  const short2_t z = {0, 0};
  const short2_t r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, a, b, 1.0f,
                                                              false);
  return (uint32_t)(uint16_t)r[0];
}

// The largest bf16 magnitude (bits) of the Markstein quotient's range.
constexpr uint32_t BF16_2P60 = 0x5D80u;

// The element codes of a lane's 8 elements with divisions and the midpoint
// count, for a block whose scale code is sc (the slow path below).
template <bool F16>
__device__ __forceinline__ uint32_t encode_slow(const uint32_t (&x)[4],
                                                uint32_t sc, float gs) {
  const float d = e4m3_decode_nonneg(sc) * gs;
  uint32_t out = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t bits = (x[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
    const float ax = elem_f32<F16>(bits & 0x7FFFu);
    const uint32_t mag = sc == 0 ? 0u : e2m1_code(ax / d);
    out |= (((bits >> 15) << 3) | mag) << (4 * e);
  }
  return out;
}

// One lane per 8 elements, two lanes (i, i^1) per 16-element block.  The
// encode pass walks the tiles from the last to the first: the amax pass has
// just read the same bytes in the opposite order, so the first tiles read
// here are the ones most likely still in the device's last-level cache.
//
// Fast path, per block: s = bmax / (6 gs) as a Markstein quotient (the
// divisor is the same for the whole call, so its correctly rounded
// reciprocal is computed once), the E4M3 code of s with the hardware
// convert (exact: s stays below 449, and the convert rounds to nearest-even
// up to 464), and the divisor d = e4m3(s) * gs with its correctly rounded
// reciprocal from a table of the 127 codes that each block builds once.
// Per element: the Markstein quotient of the signed value (rounding to
// nearest is symmetric, so it is the signed correctly rounded quotient),
// the sign of x put back (a zero quotient of a negative x is -0), and half
// a hardware convert.  A zero scale gives d = 1, rd = 0, so every quotient
// is a zero of x's sign.  A wave with a block outside these ranges (a NaN or
// infinity, |x| > 2^60, a divisor outside the Markstein range) encodes its
// tiles with divisions, the software E4M3 encoder and the midpoint count.
template <bool F16>
__global__ __launch_bounds__(QTHREADS) void k_nvfp4_encode(
    const uint16_t* __restrict__ w, int64_t hidden,
    const int32_t* __restrict__ ids, int64_t n_rows,
    const uint32_t* __restrict__ amax_bits, uint8_t* __restrict__ packed,
    uint8_t* __restrict__ scales) {
  const Tiles tl(hidden, n_rows);
  const int lane = threadIdx.x & 63;
  const float gs = global_scale_from(*amax_bits);
  const float six_gs = 6.0f * gs;
  const float r_six_gs = 1.0f / six_gs;
  const bool six_in_range = divisor_in_range(six_gs);
  // (d, 1/d) of every non-negative E4M3 code; code 0 (a zero scale) as above
  __shared__ float2 dtab[128];
  if (threadIdx.x < 128) {
    const uint32_t c = threadIdx.x;
    const float d = e4m3_decode_nonneg(c < 0x7Fu ? c : 0x7Eu) * gs;
    dtab[c] = c == 0 ? make_float2(1.0f, 0.0f) : make_float2(d, 1.0f / d);
  }
  __syncthreads();
  const int64_t wave = (int64_t)blockIdx.x * QWAVES +
                       __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * QWAVES;
  for (int64_t i0 = wave; i0 < tl.count; i0 += ROUND * nwaves) {
    TileLoad ld[ROUND];
#pragma unroll
    for (int u = 0; u < ROUND; ++u)
      ld[u] = load_tile(w, hidden, ids, tl, i0 + u * nwaves, lane);
#pragma unroll
    for (int u = 0; u < ROUND; ++u) {
      const uint4 v = ld[u].v;
      uint32_t bm = abs_bf16_max8(v);
      const uint32_t other = (uint32_t)__builtin_amdgcn_update_dpp(
          0, (int)bm, DPP_QUAD_1032, 0xF, 0xF, false);
      bm = bm > other ? bm : other;
      const float bmax = elem_f32<F16>(bm);
      const uint32_t x[4] = {v.x, v.y, v.z, v.w};
      // finite and at most 2^60 (binary16 magnitudes never reach it)
      const bool x_ok = F16 ? bm < 0x7C00u : bm <= BF16_2P60;
      uint32_t sc, out = 0;
      if (__builtin_amdgcn_ballot_w64(!(six_in_range && x_ok)) == 0) {
        const float q0 = bmax * r_six_gs;
        const float rr = __builtin_fmaf(-q0, six_gs, bmax);
        const float s = __builtin_fmaf(rr, r_six_gs, q0);
        sc = fp8_pair(s, s) & 0xFFu;
        const float2 dd = dtab[sc & 0x7Fu];  // (s < 449: never the NaN code)
        const float d = dd.x, rd = dd.y;
        if (__builtin_amdgcn_ballot_w64(!(sc == 0 || divisor_in_range(d))) ==
            0) {
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const uint32_t xw = x[e >> 1];
            float q[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const float xs =
                  F16 ? elem_f32<true>(h ? xw >> 16 : xw & 0xFFFFu)
                      : __uint_as_float(h ? xw & 0xFFFF0000u : xw << 16);
              const float a0 = xs * rd;
              const float ra = __builtin_fmaf(-a0, d, xs);
              q[h] = __builtin_copysignf(__builtin_fmaf(ra, rd, a0), xs);
            }
            out = fp4_pair(out, q[0], q[1], e >> 1);
          }
        } else {
          out = encode_slow<F16>(x, sc, gs);
        }
      } else {
        const float s = bmax / six_gs;
        sc = e4m3_encode_nonneg(s);
        out = encode_slow<F16>(x, sc, gs);
      }
      if (ld[u].live) {
        const int64_t j = ld[u].j, k = ld[u].k;
        // element 2i in the low nibble of byte i
        *reinterpret_cast<uint32_t*>(packed + j * (hidden / 2) + k * 4) = out;
        if ((lane & 1) == 0) scales[j * (hidden / 16) + k / 2] = (uint8_t)sc;
      }
    }
  }
}

__device__ __forceinline__ float e4m3_scale_from(uint32_t amax_bits) {
  float amax = __uint_as_float(amax_bits);
  return fmaxf(amax, 1e-12f) / 448.0f;
}

// One lane per 8 elements, tiles from the last to the first (as above).
// Fast path: Markstein quotient, clamp, hardware convert; a wave with an
// element outside the Markstein range takes the division and the software
// encode instead.
__global__ __launch_bounds__(QTHREADS) void k_e4m3_encode(
    const uint16_t* __restrict__ w, int64_t hidden,
    const int32_t* __restrict__ ids, int64_t n_rows,
    const uint32_t* __restrict__ amax_bits, uint8_t* __restrict__ q) {
  const Tiles tl(hidden, n_rows);
  const int lane = threadIdx.x & 63;
  const float scale = e4m3_scale_from(*amax_bits);
  const float rs = 1.0f / scale;
  const bool scale_fast = divisor_in_range(scale);
  const int64_t wave = (int64_t)blockIdx.x * QWAVES +
                       __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * QWAVES;
  for (int64_t i0 = wave; i0 < tl.count; i0 += ROUND * nwaves) {
    TileLoad ld[ROUND];
#pragma unroll
    for (int u = 0; u < ROUND; ++u)
      ld[u] = load_tile(w, hidden, ids, tl, i0 + u * nwaves, lane);
#pragma unroll
    for (int u = 0; u < ROUND; ++u) {
      const uint32_t x[4] = {ld[u].v.x, ld[u].v.y, ld[u].v.z, ld[u].v.w};
      const bool fast = scale_fast && abs_bf16_max8(ld[u].v) <= BF16_2P60;
      uint32_t out[2] = {0u, 0u};
      if (__builtin_amdgcn_ballot_w64(!fast) == 0) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          float t[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t bits = (x[(e + h) >> 1] >> (((e + h) & 1) * 16)) &
                                  0xFFFFu;
            const float ax = bf16_to_f32(bits & 0x7FFFu);
            const float q0 = ax * rs;
            const float r = __builtin_fmaf(-q0, scale, ax);
            const float mag = fminf(__builtin_fmaf(r, rs, q0), 448.0f);
            t[h] = __uint_as_float(__float_as_uint(mag) |
                                   ((bits & 0x8000u) << 16));
          }
          out[e >> 2] |= fp8_pair(t[0], t[1]) << ((e & 2) * 8);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t bits = (x[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
          float t = bf16_to_f32(bits) / scale;
          t = fminf(fmaxf(t, -448.0f), 448.0f);
          const uint32_t code =
              e4m3_encode_nonneg(fabsf(t)) | ((__float_as_uint(t) >> 31) << 7);
          out[e >> 2] |= code << ((e & 3) * 8);
        }
      }
      if (ld[u].live)
        *reinterpret_cast<uint2*>(q + ld[u].j * hidden + ld[u].k * 8) =
            make_uint2(out[0], out[1]);
    }
  }
}

// Writes the tensor scale (NVFP4 global scale or E4M3 scale) and returns the
// amax slot to zero.
template <bool E4M3>
__global__ void k_quant_finish(uint32_t* __restrict__ amax_bits,
                               float* __restrict__ scale) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    *scale = E4M3 ? e4m3_scale_from(*amax_bits) : global_scale_from(*amax_bits);
    *amax_bits = 0u;
  }
}

// Per-token dynamic E4M3 activations: one block per row of h.  The row's
// scale is max(amax, 1e-12)/448, the head's recipe with one scale per token;
// each element is x / scale (an IEEE division: a row has at most 16 384),
// clamped to +-448 and converted in hardware, which is exact there.  The
// codes go to qx and, decoded back to BF16 (exact: every E4M3 value is a
// BF16 value), to hq, the activations the GEMV kernels read.  Either output
// may be null.
__global__ __launch_bounds__(QTHREADS) void k_fp8_tokens(
    const uint16_t* __restrict__ h, int64_t hidden, uint8_t* __restrict__ qx,
    uint16_t* __restrict__ hq, float* __restrict__ sx) {
  __shared__ uint32_t red[QWAVES];
  const int64_t b = blockIdx.x;
  const uint4* row = reinterpret_cast<const uint4*>(h + b * hidden);
  const int n8 = (int)(hidden / 8);
  // the row stays in registers between the two passes: at most 16 384
  // values, TOK_U pieces of 8 per thread, all loads issued at once
  constexpr int TOK_U = 16384 / 8 / QTHREADS;
  uint4 rv[TOK_U];
#pragma unroll
  for (int u = 0; u < TOK_U; ++u) {
    const int i = threadIdx.x + u * QTHREADS;
    rv[u] = i < n8 ? row[i] : make_uint4(0u, 0u, 0u, 0u);
  }
  uint32_t m = 0u;
#pragma unroll
  for (int u = 0; u < TOK_U; ++u) {
    const uint32_t v = abs_bf16_max8(rv[u]);
    m = v > m ? v : m;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)m, off, 64);
    m = o > m ? o : m;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int w = 1; w < QWAVES; ++w) m = red[w] > m ? red[w] : m;
  // magnitudes are compared as bf16 bit patterns (monotonic for |x|)
  const float scale = fmaxf(bf16_to_f32(m), 1e-12f) / 448.0f;
#pragma unroll
  for (int u = 0; u < TOK_U; ++u) {
    const int i = threadIdx.x + u * QTHREADS;
    if (i >= n8) break;
    const uint4 v = rv[u];
    const uint32_t x[4] = {v.x, v.y, v.z, v.w};
    uint32_t code[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      float t[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t bits = (x[(e + k) >> 1] >> (((e + k) & 1) * 16)) &
                              0xFFFFu;
        t[k] = fminf(fmaxf(bf16_to_f32(bits) / scale, -448.0f), 448.0f);
      }
      code[e >> 2] |= fp8_pair(t[0], t[1]) << ((e & 2) * 8);
    }
    if (qx)
      *reinterpret_cast<uint2*>(qx + b * hidden + 8 * i) =
          make_uint2(code[0], code[1]);
    if (hq) {
      // each call decodes the low (false) or high (true) pair of a word
      const uint32_t d0 = __builtin_bit_cast(
          uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(code[0], 1.0f, false));
      const uint32_t d1 = __builtin_bit_cast(
          uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(code[0], 1.0f, true));
      const uint32_t d2 = __builtin_bit_cast(
          uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(code[1], 1.0f, false));
      const uint32_t d3 = __builtin_bit_cast(
          uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(code[1], 1.0f, true));
      *reinterpret_cast<uint4*>(hq + b * hidden + 8 * i) =
          make_uint4(d0, d1, d2, d3);
    }
  }
  if (threadIdx.x == 0) sx[b] = scale;
}

// Blocks for n_rows gathered rows: one wave per tile, at most 8 blocks of
// 4 waves per CU (one resident round at the kernels' register use).
int grid_for(int64_t n_rows, int64_t hidden, int cus) {
  const int64_t tiles = n_rows * ((hidden / 8 + 63) / 64);
  int64_t want = (tiles + QWAVES - 1) / QWAVES;
  const int64_t cap = (int64_t)cus * 8;
  if (want > cap) want = cap;
  return (int)(want < 1 ? 1 : want);
}

}  // namespace

hipError_t launch_nvfp4_quantize(const QuantArgs& a, hipStream_t s) {
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  uint32_t* amax = reinterpret_cast<uint32_t*>(a.ws + WS_AMAX);
  const int grid = grid_for(a.n_rows, a.hidden, di.cus);
  if (a.f16) {
    k_gather_amax<true><<<grid, QTHREADS, 0, s>>>(a.w, a.hidden, a.ids,
                                                  a.n_rows, amax);
    k_nvfp4_encode<true><<<grid, QTHREADS, 0, s>>>(
        a.w, a.hidden, a.ids, a.n_rows, amax, a.packed, a.scales);
  } else {
    k_gather_amax<false><<<grid, QTHREADS, 0, s>>>(a.w, a.hidden, a.ids,
                                                   a.n_rows, amax);
    k_nvfp4_encode<false><<<grid, QTHREADS, 0, s>>>(
        a.w, a.hidden, a.ids, a.n_rows, amax, a.packed, a.scales);
  }
  k_quant_finish<false><<<1, 64, 0, s>>>(amax, a.global_scale);
  return hipGetLastError();
}

hipError_t launch_fp8_tokens(const uint16_t* h, int64_t batch, int64_t hidden,
                             uint8_t* qx, uint16_t* hq, float* sx,
                             hipStream_t s) {
  // the kernel holds a row of at most 16 384 values in registers
  if (batch < 1 || hidden < 8 || hidden > 16384 || hidden % 8 != 0)
    return hipErrorInvalidValue;
  k_fp8_tokens<<<(unsigned)batch, QTHREADS, 0, s>>>(h, hidden, qx, hq, sx);
  return hipGetLastError();
}

hipError_t launch_e4m3_quantize(const QuantE4m3Args& a, hipStream_t s) {
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  uint32_t* amax = reinterpret_cast<uint32_t*>(a.ws + WS_AMAX);
  const int grid = grid_for(a.n_rows, a.hidden, di.cus);
  k_gather_amax<false><<<grid, QTHREADS, 0, s>>>(a.w, a.hidden, a.ids,
                                                 a.n_rows, amax);
  k_e4m3_encode<<<grid, QTHREADS, 0, s>>>(a.w, a.hidden, a.ids, a.n_rows,
                                          amax, a.q);
  k_quant_finish<true><<<1, 64, 0, s>>>(amax, a.scale);
  return hipGetLastError();
}

}  // namespace dh
