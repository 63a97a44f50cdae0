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
//   2. k_nvfp4_encode  one thread per 16-element block: block max, E4M3
//                      scale, 16 e2m1 codes packed into 8 bytes;
//   3. k_quant_finish  writes the global scale and returns the amax slot of
//                      the workspace to zero.
// Every float operation is a single IEEE binary32 operation with
// round-to-nearest-even (no contraction, correctly rounded division), in the
// order gs = max(amax,1e-12)/2688, s = bmax/(6*gs), q = x/(e4m3(s)*gs).
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

__device__ __forceinline__ uint32_t abs_bf16_pair_max(uint32_t v) {
  uint32_t lo = v & 0x7FFFu, hi = (v >> 16) & 0x7FFFu;
  return lo > hi ? lo : hi;
}

__device__ __forceinline__ float global_scale_from(uint32_t amax_bits) {
  float amax = __uint_as_float(amax_bits);
  return fmaxf(amax, 1e-12f) / 2688.0f;
}

__global__ __launch_bounds__(QTHREADS) void k_gather_amax(
    const uint16_t* __restrict__ w, int64_t hidden,
    const int32_t* __restrict__ ids, int64_t n_rows,
    uint32_t* __restrict__ amax_bits) {
  const int64_t upr = hidden / 8;  // 16-byte units per row
  const int64_t total = n_rows * upr;
  uint32_t m = 0;
  for (int64_t u = (int64_t)blockIdx.x * QTHREADS + threadIdx.x; u < total;
       u += (int64_t)gridDim.x * QTHREADS) {
    int64_t j = u / upr, k = u - j * upr;
    const uint4 v =
        *reinterpret_cast<const uint4*>(w + (int64_t)ids[j] * hidden + k * 8);
    uint32_t a = abs_bf16_pair_max(v.x), b = abs_bf16_pair_max(v.y);
    uint32_t c = abs_bf16_pair_max(v.z), d = abs_bf16_pair_max(v.w);
    a = a > b ? a : b;
    c = c > d ? c : d;
    a = a > c ? a : c;
    m = m > a ? m : a;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    uint32_t o = __shfl_xor(m, off, 64);
    m = m > o ? m : o;
  }
  __shared__ uint32_t wmax[QTHREADS / 64];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = wmax[0];
    for (int i = 1; i < QTHREADS / 64; ++i) r = r > wmax[i] ? r : wmax[i];
    // |bf16| bits shifted into place are the binary32 bits of the same
    // non-negative value, whose unsigned order is the numeric order.
    if (r) atomicMax(amax_bits, r << 16);
  }
}

__global__ __launch_bounds__(QTHREADS) void k_nvfp4_encode(
    const uint16_t* __restrict__ w, int64_t hidden,
    const int32_t* __restrict__ ids, int64_t n_rows,
    const uint32_t* __restrict__ amax_bits, uint8_t* __restrict__ packed,
    uint8_t* __restrict__ scales) {
  const int64_t nblk = hidden / 16;
  const int64_t total = n_rows * nblk;
  const float gs = global_scale_from(*amax_bits);
  const float six_gs = 6.0f * gs;
  for (int64_t u = (int64_t)blockIdx.x * QTHREADS + threadIdx.x; u < total;
       u += (int64_t)gridDim.x * QTHREADS) {
    int64_t j = u / nblk, b = u - j * nblk;
    const uint4* src = reinterpret_cast<const uint4*>(
        w + (int64_t)ids[j] * hidden + b * 16);
    const uint4 v0 = src[0], v1 = src[1];
    uint32_t x[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t bm = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t a = abs_bf16_pair_max(x[i]);
      bm = bm > a ? bm : a;
    }
    const float bmax = bf16_to_f32(bm);
    const float s = bmax / six_gs;
    const uint32_t sc = e4m3_encode_nonneg(s);
    const float s_dec = e4m3_decode_nonneg(sc);
    const float d = s_dec * gs;
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t bits = (x[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu;
      uint32_t nib = (bits >> 15) << 3;  // sign bit of the BF16 input
      if (s_dec != 0.0f) {
        const float q = bf16_to_f32(bits) / d;
        nib |= e2m1_encode_mag(fabsf(q));
      }
      out[i >> 3] |= nib << ((i & 7) * 4);
    }
    *reinterpret_cast<uint2*>(packed + j * (hidden / 2) + b * 8) =
        make_uint2(out[0], out[1]);
    scales[j * nblk + b] = (uint8_t)sc;
  }
}

__device__ __forceinline__ float e4m3_scale_from(uint32_t amax_bits) {
  float amax = __uint_as_float(amax_bits);
  return fmaxf(amax, 1e-12f) / 448.0f;
}

__global__ __launch_bounds__(QTHREADS) void k_e4m3_encode(
    const uint16_t* __restrict__ w, int64_t hidden,
    const int32_t* __restrict__ ids, int64_t n_rows,
    const uint32_t* __restrict__ amax_bits, uint8_t* __restrict__ q) {
  const int64_t upr = hidden / 8;  // 16-byte input units per row
  const int64_t total = n_rows * upr;
  const float scale = e4m3_scale_from(*amax_bits);
  for (int64_t u = (int64_t)blockIdx.x * QTHREADS + threadIdx.x; u < total;
       u += (int64_t)gridDim.x * QTHREADS) {
    const int64_t j = u / upr, k = u - j * upr;
    const uint4 v =
        *reinterpret_cast<const uint4*>(w + (int64_t)ids[j] * hidden + k * 8);
    const uint32_t x[4] = {v.x, v.y, v.z, v.w};
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t bits = (x[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu;
      float t = bf16_to_f32(bits) / scale;
      t = fminf(fmaxf(t, -448.0f), 448.0f);
      const uint32_t code =
          e4m3_encode_nonneg(fabsf(t)) | ((__float_as_uint(t) >> 31) << 7);
      out[i >> 2] |= code << ((i & 3) * 8);
    }
    *reinterpret_cast<uint2*>(q + j * hidden + k * 8) =
        make_uint2(out[0], out[1]);
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

int grid_for(int64_t units, int cus) {
  int64_t want = (units + QTHREADS - 1) / QTHREADS;
  int64_t cap = (int64_t)cus * 16;
  if (want > cap) want = cap;
  return (int)(want < 1 ? 1 : want);
}

}  // namespace

hipError_t launch_nvfp4_quantize(const QuantArgs& a, hipStream_t s) {
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  uint32_t* amax = reinterpret_cast<uint32_t*>(a.ws + WS_AMAX);
  k_gather_amax<<<grid_for(a.n_rows * (a.hidden / 8), di.cus), QTHREADS, 0,
                  s>>>(a.w, a.hidden, a.ids, a.n_rows, amax);
  k_nvfp4_encode<<<grid_for(a.n_rows * (a.hidden / 16), di.cus), QTHREADS, 0,
                   s>>>(a.w, a.hidden, a.ids, a.n_rows, amax, a.packed,
                        a.scales);
  k_quant_finish<false><<<1, 64, 0, s>>>(amax, a.global_scale);
  return hipGetLastError();
}

hipError_t launch_e4m3_quantize(const QuantE4m3Args& a, hipStream_t s) {
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  uint32_t* amax = reinterpret_cast<uint32_t*>(a.ws + WS_AMAX);
  const int grid = grid_for(a.n_rows * (a.hidden / 8), di.cus);
  k_gather_amax<<<grid, QTHREADS, 0, s>>>(a.w, a.hidden, a.ids, a.n_rows,
                                          amax);
  k_e4m3_encode<<<grid, QTHREADS, 0, s>>>(a.w, a.hidden, a.ids, a.n_rows,
                                          amax, a.q);
  k_quant_finish<true><<<1, 64, 0, s>>>(amax, a.scale);
  return hipGetLastError();
}

}  // namespace dh
