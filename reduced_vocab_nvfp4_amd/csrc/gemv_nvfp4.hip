// W4A16 NVFP4 GEMV fused with the two-level argmax and the id remap, and
// its logits-scatter variant.
//
// What is computed (page 1, "q38_draft.py": get_top_tokens takes the argmax
// of the draft head's output over the kept rows and maps it through dh_idx;
// compute_logits writes the head's float32 output into a -inf filled
// batch x vocab tensor at the kept ids):
//   logit[b, j] = sum_k e2m1(q[j,k]) * e4m3(s[j, k/16]) * h[b, k]   (fp32)
//   top token   = dh_idx[lowest j with the largest logit]
//   logits      = gs * logit[b, j] scattered to out[b, dh_idx[j]], j < n_kept
// The positive global scale gs does not change the argmax and is applied
// only on the logits path.
//
// Layout: packed [n_rows][hidden/2] (element k in byte k/2, low nibble for
// even k), scales [n_rows][hidden/16] E4M3.  The kernel is a stream over
// hidden/2 + hidden/16 bytes per row, so HBM bandwidth bounds it at batch 1.
//
// Work mapping (fast path, hidden = 32*G*C): a wave is 64/G groups of G
// lanes, one head row per group per iteration.  A "chunk" is 16 packed
// bytes (32 weights, two scale blocks); lane g of a group owns chunks
// g, g+G, ..., g+(C-1)G of every row, so
//   * each 128-bit load instruction reads G*16 contiguous bytes per row
//     (256 B for G=16): fully coalesced;
//   * the lane's slice of h is the same for every row and, at batch 1, stays
//     in VGPRs (C*16 registers of BF16 pairs) for the whole kernel; at
//     batch > 1 it is read from LDS.
// Weights are dequantized in registers: v_cvt_scalef32_pk_bf16_fp4 turns
// one byte (two e2m1 codes, low nibble first) into a BF16 pair with scale
// 1.0 (exact), v_dot2_f32_bf16 accumulates the pair against h, each
// 16-element block's partial is multiplied by its E4M3 scale
// (v_cvt_f32_fp8, exact), and a DPP reduction over the G lanes finishes the
// row.  Row groups are double-buffered so one group's loads are in flight
// while the previous one is computed.
//
// Argmax: every lane keeps (best value, its row) over the rows it saw in
// ascending order; the block reduces them (wave shuffles, then LDS) to one
// (value, row) partial per batch row, written to the workspace; the last
// block to arrive (agent-scope acq_rel counter) reduces all partials, ties
// going to the lowest row, writes dh_idx[row] and resets the counter.
#include <limits.h>

#include "dh_device.h"
#include "dh_internal.h"

namespace dh {
namespace {

constexpr int THREADS = 256;
constexpr int WAVES = THREADS / 64;
constexpr int LDS_BUDGET = 64 * 1024;

struct KArgs {
  const uint8_t* packed;
  const uint8_t* scales;
  const float* global_scale;
  const int32_t* dh_idx;
  int64_t n_rows, hidden;
  const uint16_t* h;  // [B][hidden] for this launch's batch slice
  int32_t* out_ids;   // [B]
  float* out_logits;  // [B][vocab]
  int64_t n_kept, vocab;
  uint8_t* ws;
};

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) {
  return __builtin_bit_cast(bf16x2, u);
}

// Eight weights (one dword of packed nibbles) against four BF16 pairs.
__device__ __forceinline__ float dot8(uint32_t w, const uint32_t* hp,
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

// One 16-element block (two dwords of codes, eight BF16 pairs of h).
__device__ __forceinline__ float block_dot(uint32_t w0, uint32_t w1,
                                           const uint32_t* hp) {
  return dot8(w1, hp + 4, dot8(w0, hp, 0.0f));
}

// One 16-byte chunk: two blocks, their scales in the low two bytes of sb.
__device__ __forceinline__ float chunk_dot(const uint4& p, uint32_t sb,
                                           const uint32_t* hp, float acc) {
  const float b0 = block_dot(p.x, p.y, hp);
  const float b1 = block_dot(p.z, p.w, hp + 8);
  acc = fmaf(__builtin_amdgcn_cvt_f32_fp8(sb, 0), b0, acc);
  acc = fmaf(__builtin_amdgcn_cvt_f32_fp8(sb, 1), b1, acc);
  return acc;
}

__device__ __forceinline__ uint64_t pack_partial(float v, int r) {
  return ((uint64_t)(uint32_t)r << 32) | (uint64_t)__float_as_uint(v);
}

// Block-level (value,row) reduction, partial write, and the last block's
// final pass.  best_v/best_r are this lane's per-batch candidates.
template <int B>
__device__ __forceinline__ void argmax_finish(float (&best_v)[B],
                                              int (&best_r)[B],
                                              const KArgs& a) {
  __shared__ float sv[WAVES][B];
  __shared__ int sr[WAVES][B];
  __shared__ int is_last;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t* part = reinterpret_cast<uint64_t*>(a.ws + WS_PARTIALS);
  uint32_t* counter = reinterpret_cast<uint32_t*>(a.ws + WS_COUNTER);
#pragma unroll
  for (int b = 0; b < B; ++b) {
    wave_argmax(best_v[b], best_r[b]);
    if (lane == 0) {
      sv[wave][b] = best_v[b];
      sr[wave][b] = best_r[b];
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int b = 0; b < B; ++b) {
      float v = sv[0][b];
      int r = sr[0][b];
      for (int w = 1; w < WAVES; ++w)
        if (better(sv[w][b], sr[w][b], v, r)) {
          v = sv[w][b];
          r = sr[w][b];
        }
      __hip_atomic_store(&part[(int64_t)blockIdx.x * B + b],
                         pack_partial(v, r), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    const uint32_t ticket = __hip_atomic_fetch_add(
        counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    is_last = (ticket == gridDim.x - 1);
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();
#pragma unroll
  for (int b = 0; b < B; ++b) {
    float v = -INFINITY;
    int r = INT_MAX;
    for (int i = threadIdx.x; i < (int)gridDim.x; i += THREADS) {
      const uint64_t p = __hip_atomic_load(&part[(int64_t)i * B + b],
                                           __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      const float pv = __uint_as_float((uint32_t)p);
      const int pr = (int)(p >> 32);
      if (better(pv, pr, v, r)) {
        v = pv;
        r = pr;
      }
    }
    wave_argmax(v, r);
    if (lane == 0) {
      sv[wave][b] = v;
      sr[wave][b] = r;
    }
  }
  __syncthreads();
  if (threadIdx.x < B) {
    const int b = threadIdx.x;
    float v = sv[0][b];
    int r = sr[0][b];
    for (int w = 1; w < WAVES; ++w)
      if (better(sv[w][b], sr[w][b], v, r)) {
        v = sv[w][b];
        r = sr[w][b];
      }
    if (r < 0 || r >= a.n_rows) r = 0;  // only reachable with NaN inputs
    a.out_ids[b] = a.dh_idx[r];
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Copy h [B][hidden] into LDS as BF16 pairs.
template <int B>
__device__ __forceinline__ void stage_h(const uint16_t* h, int64_t hidden,
                                        uint32_t* hs) {
  const uint4* src = reinterpret_cast<const uint4*>(h);
  uint4* dst = reinterpret_cast<uint4*>(hs);
  const int n = (int)(B * hidden / 8);
  for (int t = threadIdx.x; t < n; t += THREADS) dst[t] = src[t];
  __syncthreads();
}

template <int G, int C>
struct Rows {
  uint4 p[C];
  uint32_t s[C];
};

template <int G, int C>
__device__ __forceinline__ void load_rows(Rows<G, C>& r, const KArgs& a,
                                          int64_t row, int g) {
  const uint4* prow =
      reinterpret_cast<const uint4*>(a.packed + row * (a.hidden / 2));
  const uint16_t* srow =
      reinterpret_cast<const uint16_t*>(a.scales + row * (a.hidden / 16));
#pragma unroll
  for (int i = 0; i < C; ++i) {
    r.p[i] = prow[g + G * i];
    r.s[i] = srow[g + G * i];
  }
}

template <int G, int C, int B, bool LOGITS>
__device__ __forceinline__ void compute_rows(
    const Rows<G, C>& r, const KArgs& a, int64_t row, int g,
    const uint32_t* hreg, const uint32_t* hs, float gs, float (&best_v)[B],
    int (&best_r)[B]) {
  float acc[B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = 0.0f;
#pragma unroll
  for (int i = 0; i < C; ++i) {
    if constexpr (B == 1) {
      acc[0] = chunk_dot(r.p[i], r.s[i], hreg + i * 16, acc[0]);
    } else {
      const int c = g + G * i;
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const uint4* hp4 =
            reinterpret_cast<const uint4*>(hs + b * (a.hidden / 2) + c * 16);
        uint32_t hp[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 v = hp4[q];
          hp[4 * q + 0] = v.x;
          hp[4 * q + 1] = v.y;
          hp[4 * q + 2] = v.z;
          hp[4 * q + 3] = v.w;
        }
        acc[b] = chunk_dot(r.p[i], r.s[i], hp, acc[b]);
      }
    }
  }
#pragma unroll
  for (int b = 0; b < B; ++b) {
    const float v = group_sum<G>(acc[b]);
    if constexpr (LOGITS) {
      if (g == 0 && row < a.n_kept)
        a.out_logits[b * a.vocab + a.dh_idx[row]] = v * gs;
    } else {
      // rows reach a lane in ascending order: strict > keeps the lowest
      if (v > best_v[b]) {
        best_v[b] = v;
        best_r[b] = (int)row;
      }
    }
  }
}

template <int G, int C, int B, bool LOGITS>
__global__ __launch_bounds__(THREADS) void k_nvfp4_fast(const KArgs a) {
  constexpr int R = 64 / G;  // rows per wave iteration
  extern __shared__ uint32_t hs[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane / G, g = lane % G;

  uint32_t hreg[B == 1 ? C * 16 : 1];
  if constexpr (B == 1) {
    const uint4* h4 = reinterpret_cast<const uint4*>(a.h);
#pragma unroll
    for (int i = 0; i < C; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 v = h4[(g + G * i) * 4 + q];
        hreg[i * 16 + 4 * q + 0] = v.x;
        hreg[i * 16 + 4 * q + 1] = v.y;
        hreg[i * 16 + 4 * q + 2] = v.z;
        hreg[i * 16 + 4 * q + 3] = v.w;
      }
    }
  } else {
    stage_h<B>(a.h, a.hidden, hs);
  }
  const float gs = LOGITS ? *a.global_scale : 1.0f;

  float best_v[B];
  int best_r[B];
#pragma unroll
  for (int b = 0; b < B; ++b) {
    best_v[b] = -INFINITY;
    best_r[b] = INT_MAX;
  }

  const int64_t T = a.n_rows / R;  // row groups
  const int64_t rg0 = (int64_t)blockIdx.x * T / gridDim.x;
  const int64_t rg1 = (int64_t)(blockIdx.x + 1) * T / gridDim.x;
  Rows<G, C> ra, rb;
  int64_t rg = rg0 + wave;
  if (rg < rg1) load_rows<G, C>(ra, a, rg * R + grp, g);
  while (rg < rg1) {
    int64_t rn = rg + WAVES;
    if (rn < rg1) load_rows<G, C>(rb, a, rn * R + grp, g);
    compute_rows<G, C, B, LOGITS>(ra, a, rg * R + grp, g, hreg, hs, gs,
                                  best_v, best_r);
    rg = rn;
    if (rg >= rg1) break;
    rn = rg + WAVES;
    if (rn < rg1) load_rows<G, C>(ra, a, rn * R + grp, g);
    compute_rows<G, C, B, LOGITS>(rb, a, rg * R + grp, g, hreg, hs, gs,
                                  best_v, best_r);
    rg = rn;
  }
  if constexpr (!LOGITS) argmax_finish<B>(best_v, best_r, a);
}

// Any hidden % 16 == 0: one row per wave iteration, 8-byte (one block)
// units strided over the 64 lanes, h for every batch row in LDS.
template <int B, bool LOGITS>
__global__ __launch_bounds__(THREADS) void k_nvfp4_generic(const KArgs a) {
  extern __shared__ uint32_t hs[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  stage_h<B>(a.h, a.hidden, hs);
  const float gs = LOGITS ? *a.global_scale : 1.0f;
  float best_v[B];
  int best_r[B];
#pragma unroll
  for (int b = 0; b < B; ++b) {
    best_v[b] = -INFINITY;
    best_r[b] = INT_MAX;
  }
  const int64_t nblk = a.hidden / 16;
  const int64_t r0 = (int64_t)blockIdx.x * a.n_rows / gridDim.x;
  const int64_t r1 = (int64_t)(blockIdx.x + 1) * a.n_rows / gridDim.x;
  for (int64_t row = r0 + wave; row < r1; row += WAVES) {
    const uint2* prow =
        reinterpret_cast<const uint2*>(a.packed + row * (a.hidden / 2));
    const uint8_t* srow = a.scales + row * nblk;
    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.0f;
    for (int64_t c = lane; c < nblk; c += 64) {
      const uint2 p = prow[c];
      const float sc = __builtin_amdgcn_cvt_f32_fp8((uint32_t)srow[c], 0);
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const uint32_t* hp = hs + b * (a.hidden / 2) + c * 8;
        acc[b] = fmaf(sc, block_dot(p.x, p.y, hp), acc[b]);
      }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float v = group_sum<64>(acc[b]);
      if constexpr (LOGITS) {
        if (lane == 0 && row < a.n_kept)
          a.out_logits[b * a.vocab + a.dh_idx[row]] = v * gs;
      } else if (v > best_v[b]) {
        best_v[b] = v;
        best_r[b] = (int)row;
      }
    }
  }
  if constexpr (!LOGITS) argmax_finish<B>(best_v, best_r, a);
}

__global__ __launch_bounds__(THREADS) void k_fill_neg_inf(float* out,
                                                          int64_t n) {
  const int64_t n4 = n / 4;
  float4* o4 = reinterpret_cast<float4*>(out);
  const float ninf = -INFINITY;
  for (int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * THREADS)
    o4[i] = make_float4(ninf, ninf, ninf, ninf);
  for (int64_t i = n4 * 4 + (int64_t)blockIdx.x * THREADS + threadIdx.x;
       i < n; i += (int64_t)gridDim.x * THREADS)
    out[i] = ninf;
}

// ------------------------------------------------------------- dispatch

typedef void (*KernelFn)(const KArgs);

struct Variant {
  KernelFn fn;
  int rows_per_iter;  // rows a wave covers per iteration
  bool fast;
};

template <int G, int C, int B, bool L>
Variant fast_variant() {
  return Variant{k_nvfp4_fast<G, C, B, L>, 64 / G, true};
}

template <bool L>
bool pick_variant(int64_t hidden, int bc, Variant* v) {
  // The register-resident fast path serves batch 1 (the draft step); batch
  // slices of 2-8 rows use the LDS-staged kernel.
  if (bc == 1 && hidden % 32 == 0) {
    switch (hidden / 32) {  // 16-byte chunks per row = G * C
      case 8: *v = fast_variant<8, 1, 1, L>(); return true;
      case 16: *v = fast_variant<16, 1, 1, L>(); return true;
      case 32: *v = fast_variant<32, 1, 1, L>(); return true;
      case 64: *v = fast_variant<64, 1, 1, L>(); return true;
      case 80: *v = fast_variant<16, 5, 1, L>(); return true;
      case 128: *v = fast_variant<32, 4, 1, L>(); return true;
      case 160: *v = fast_variant<32, 5, 1, L>(); return true;
    }
  }
  switch (bc) {
    case 1: *v = Variant{k_nvfp4_generic<1, L>, 1, false}; return true;
    case 2: *v = Variant{k_nvfp4_generic<2, L>, 1, false}; return true;
    case 4: *v = Variant{k_nvfp4_generic<4, L>, 1, false}; return true;
    case 8: *v = Variant{k_nvfp4_generic<8, L>, 1, false}; return true;
  }
  return false;
}

// Largest batch slice in {8,4,2,1} that fits the remaining rows and LDS.
int batch_slice(int64_t remaining, int64_t hidden) {
  for (int bc = 8; bc > 1; bc >>= 1)
    if (bc <= remaining && (int64_t)bc * hidden * 2 <= LDS_BUDGET) return bc;
  return 1;
}

hipError_t launch_gemv(const GemvArgs& ga, bool logits, hipStream_t s) {
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  if (logits) {
    const int64_t n = ga.batch * ga.vocab;
    int64_t blocks = (n / 4 + THREADS - 1) / THREADS;
    if (blocks > (int64_t)di.cus * 8) blocks = (int64_t)di.cus * 8;
    if (blocks < 1) blocks = 1;
    k_fill_neg_inf<<<(int)blocks, THREADS, 0, s>>>(ga.out_logits, n);
  }
  for (int64_t b0 = 0; b0 < ga.batch;) {
    const int bc = batch_slice(ga.batch - b0, ga.hidden);
    Variant v;
    bool ok = logits ? pick_variant<true>(ga.hidden, bc, &v)
                     : pick_variant<false>(ga.hidden, bc, &v);
    if (!ok) return hipErrorInvalidValue;
    const size_t lds = v.fast ? 0 : (size_t)bc * (size_t)ga.hidden * 2;
    int occ = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &occ, reinterpret_cast<const void*>(v.fn), THREADS, lds);
    if (e != hipSuccess) return e;
    if (occ < 1) occ = 1;
    // one resident wave of blocks, but at least one row group per wave
    const int64_t groups = ga.n_rows / v.rows_per_iter;
    int64_t grid = (int64_t)di.cus * occ;
    const int64_t by_work = (groups + WAVES - 1) / WAVES;
    if (grid > by_work) grid = by_work;
    if (grid > MAX_GRID) grid = MAX_GRID;
    if (grid < 1) grid = 1;
    KArgs k;
    k.packed = ga.packed;
    k.scales = ga.scales;
    k.global_scale = ga.global_scale;
    k.dh_idx = ga.dh_idx;
    k.n_rows = ga.n_rows;
    k.hidden = ga.hidden;
    k.h = ga.h + b0 * ga.hidden;
    k.out_ids = logits ? nullptr : ga.out_ids + b0;
    k.out_logits = logits ? ga.out_logits + b0 * ga.vocab : nullptr;
    k.n_kept = ga.n_kept;
    k.vocab = ga.vocab;
    k.ws = ga.ws;
    void* kargs[] = {&k};
    e = hipLaunchKernel(reinterpret_cast<const void*>(v.fn),
                        dim3((unsigned)grid), dim3(THREADS), kargs, lds, s);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return e;
    b0 += bc;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_nvfp4_top_tokens(const GemvArgs& a, hipStream_t s) {
  return launch_gemv(a, false, s);
}

hipError_t launch_nvfp4_logits(const GemvArgs& a, hipStream_t s) {
  return launch_gemv(a, true, s);
}

}  // namespace dh
