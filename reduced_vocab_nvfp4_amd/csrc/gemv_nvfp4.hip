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
// Batch-1 kernel (hidden = 32*G*C): a wave is 64/G groups of G lanes, one
// head row per group per iteration.  A "chunk" is 16 packed bytes (32
// weights, two scale blocks); lane g of a group owns chunks g, g+G, ...,
// g+(C-1)G of every row, so
//   * each 128-bit load instruction reads G*16 contiguous bytes per row
//     (256 B for G=16): fully coalesced;
//   * the lane's slice of h is the same for every row: it is staged once per
//     wave through LDS and then held in C*16 VGPRs for the whole kernel.
// Weights are dequantized in registers: v_cvt_scalef32_pk_bf16_fp4 turns one
// byte (two e2m1 codes, low nibble first) into a BF16 pair with scale 1.0
// (exact), v_dot2_f32_bf16 accumulates the pair against h, each 16-element
// block's partial is multiplied by its E4M3 scale (v_cvt_f32_fp8, exact),
// and a DPP reduction over the G lanes finishes the row.  A ring of NB
// register buffers keeps NB-1 row groups in flight while one is reduced.
//
// Argmax: every lane keeps (best value, its row) over the rows it saw in
// ascending order; the block reduces them (wave shuffles, then LDS) to one
// (value, row) partial per batch row; the last block to arrive reduces all
// partials, ties going to the lowest row, writes dh_idx[row] and resets the
// arrival counter (see argmax_finish for the cross-block protocol).
#include <limits.h>

#include "dh_device.h"
#include "dh_internal.h"

namespace dh {
namespace {

constexpr int THREADS = 256;  // block size of the generic and fill kernels
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

// Block-level (value,row) reduction, the partial write and the last block's
// final pass.  best_v/best_r are this lane's per-batch candidates.
//
// Cross-block protocol.  Each block publishes its partials with agent-scope
// atomic stores (performed at the device-coherent level, past the per-XCD
// L2) and waits for them to complete (s_waitcnt vmcnt(0)) before it counts
// its arrival.  Arrivals are counted in two levels: block b adds to the
// counter of group b % ARRIVAL_GROUPS (counters 4 KB apart, in different
// memory channels: same-address atomics serialize at ~10 ns each, so one
// counter for the whole grid costs microseconds), the last arriver of a
// group adds to the top counter, and the block that completes the top count
// has seen every other block arrive after its partials were complete; it
// reads them with agent-scope atomic loads.  This is the release/acquire
// pairing restricted to the only locations that cross blocks; a general
// agent-scope release fence would also write back the whole L2 in every
// block, which costs tens of microseconds over a grid.  Every counter is
// returned to zero by the block that completes it.
template <int B, int NT>
__device__ __forceinline__ void argmax_finish(float (&best_v)[B],
                                              int (&best_r)[B],
                                              const KArgs& a) {
  constexpr int NW = NT / 64;
  __shared__ float sv[NW][B];
  __shared__ int sr[NW][B];
  __shared__ int is_last;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t* part = reinterpret_cast<uint64_t*>(a.ws + WS_PARTIALS);
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
      for (int w = 1; w < NW; ++w)
        if (better(sv[w][b], sr[w][b], v, r)) {
          v = sv[w][b];
          r = sr[w][b];
        }
      __hip_atomic_store(&part[(int64_t)blockIdx.x * B + b],
                         pack_partial(v, r), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);  // the partial stores have completed
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const uint32_t nb = gridDim.x;
    const uint32_t ng = nb < ARRIVAL_GROUPS ? nb : ARRIVAL_GROUPS;
    const uint32_t grp = blockIdx.x % ARRIVAL_GROUPS;
    const uint32_t gsize = (nb - grp + ARRIVAL_GROUPS - 1) / ARRIVAL_GROUPS;
    uint32_t* gcount =
        reinterpret_cast<uint32_t*>(a.ws + WS_GROUP + grp * WS_GSTEP);
    uint32_t* top = reinterpret_cast<uint32_t*>(a.ws + WS_TOP);
    int last = 0;
    const uint32_t t = __hip_atomic_fetch_add(gcount, 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    if (t == gsize - 1) {
      __hip_atomic_store(gcount, 0u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t u = __hip_atomic_fetch_add(top, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
      if (u == ng - 1) {
        __hip_atomic_store(top, 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        last = 1;
      }
    }
    is_last = last;
  }
  __syncthreads();
  if (!is_last) return;
#pragma unroll
  for (int b = 0; b < B; ++b) {
    float v = -INFINITY;
    int r = INT_MAX;
    for (int i = threadIdx.x; i < (int)gridDim.x; i += NT) {
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
    for (int w = 1; w < NW; ++w)
      if (better(sv[w][b], sr[w][b], v, r)) {
        v = sv[w][b];
        r = sr[w][b];
      }
    if (r < 0 || r >= a.n_rows) r = 0;  // only reachable with NaN inputs
    a.out_ids[b] = a.dh_idx[r];
  }
}

// Copy h [B][hidden] into LDS as BF16 pairs.
template <int NT>
__device__ __forceinline__ void stage_h(const uint16_t* h, int64_t count,
                                        uint32_t* hs) {
  const uint4* src = reinterpret_cast<const uint4*>(h);
  uint4* dst = reinterpret_cast<uint4*>(hs);
  const int n = (int)(count / 8);
  for (int t = threadIdx.x; t < n; t += NT) dst[t] = src[t];
  __syncthreads();
}

template <int C>
struct Rows {
  uint4 p[C];
  uint32_t s[C];
};

template <int G, int C>
__device__ __forceinline__ void load_rows(Rows<C>& r, const KArgs& a,
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

template <int G, int C, bool LOGITS>
__device__ __forceinline__ void compute_rows(const Rows<C>& r, const KArgs& a,
                                             int64_t row, int g,
                                             const uint32_t* hreg, float gs,
                                             float& best_v, int& best_r) {
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < C; ++i) acc = chunk_dot(r.p[i], r.s[i], hreg + i * 16, acc);
  const float v = group_sum<G>(acc);
  if constexpr (LOGITS) {
    if (g == 0 && row < a.n_kept) a.out_logits[a.dh_idx[row]] = v * gs;
  } else if (v > best_v) {
    // rows reach a lane in ascending order: strict > keeps the lowest
    best_v = v;
    best_r = (int)row;
  }
}

// Batch-1 kernel: G lanes per row, C chunks per lane, NB register buffers,
// NT threads per block.
template <int G, int C, bool LOGITS, int NB, int NT>
__global__ __launch_bounds__(NT) void k_nvfp4_b1(const KArgs a) {
  constexpr int R = 64 / G;  // rows per wave iteration
  constexpr int NW = NT / 64;
  constexpr int HU4 = 4 * G * C;  // h as uint4 (hidden = 32*G*C BF16)
  static_assert(HU4 % 64 == 0 || HU4 < 64, "h staging covers HU4 exactly");
  __shared__ uint4 hl[NW][HU4 < 64 ? 64 : HU4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane / G, g = lane % G;
  const int wv = __builtin_amdgcn_readfirstlane(wave);

  // Row groups are dealt to the grid's waves round-robin (grid stride):
  // wave w of the grid takes groups w, w + TW, w + 2 TW, ...  The per-wave
  // trip count is wave-uniform so loop control stays scalar.
  const int64_t T = a.n_rows / R;
  const int64_t TW = (int64_t)gridDim.x * NW;
  const int64_t first = (int64_t)blockIdx.x * NW + wv;
  const int n_it = first < T ? (int)((T - first + TW - 1) / TW) : 0;

  // A ring of NB register buffers: the loads of group it+NB-1 are issued
  // before group it is reduced, so NB-1 groups stay in flight.  The trip
  // count is rounded up to a multiple of NB and row indices past the wave's
  // last group are clamped to it: every load in the loop is unconditional
  // (which keeps the compiler's wait counts exact) and the surplus loads hit
  // in L2; the reduction of those padded iterations is skipped.
  // (A wave without row groups, possible only on tiny heads, reads group 0
  // in its prologue and never reduces it.)
  const int n_pad = (n_it + NB - 1) / NB * NB;
  const int64_t base = n_it > 0 ? first : 0;
  const int last = n_it > 0 ? n_it - 1 : 0;
  auto row_of = [&](int it) {
    const int c = it < last ? it : last;
    return (base + (int64_t)c * TW) * R + grp;
  };
  // Prologue.  h is copied straight into this wave's LDS slice with
  // global_load_lds_dwordx4 (lane i's 16 bytes land at slice + 16*i; no
  // VGPRs, no block barrier), then the first weight row groups are issued,
  // so only h has to arrive before the ring starts.  Every lane then keeps
  // its C chunks of h in VGPRs.
  constexpr int HJ = (HU4 + 63) / 64;  // h copies per lane
  const uint4* h4 = reinterpret_cast<const uint4*>(a.h);
  // lanes past the end of h (only when HU4 < 64) re-read its last uint4
  const int hl0 = (HU4 % 64 == 0 || lane < HU4) ? lane : HU4 - 1;
#pragma unroll
  for (int j = 0; j < HJ; ++j) {
    // global_load_lds_dwordx4: M0 holds the wave's LDS destination.  It is
    // issued as inline assembly so that the compiler's wait-count pass,
    // which does not order LDS reads after these copies correctly, leaves
    // them alone; the explicit wait below covers them.
    const uint32_t lds_dst = (uint32_t)(uintptr_t)(
        (__attribute__((address_space(3))) void*)(&hl[wv][64 * j]));
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "global_load_lds_dwordx4 %0, off"
        :
        : "v"(h4 + hl0 + 64 * j), "s"(lds_dst)
        : "memory", "m0");
  }
  __builtin_amdgcn_sched_barrier(0);
  Rows<C> buf[NB];
#pragma unroll
  for (int k = 0; k < NB - 1; ++k) load_rows<G, C>(buf[k], a, row_of(k), g);
  // Memory loads retire in issue order, so once no more than the weight
  // loads just issued are outstanding, the h copies have landed in LDS.
  // (The wait is explicit: the compiler does not order LDS reads after
  // global_load_lds on its own.)  The "memory" clobber keeps the LDS reads
  // below it.
  constexpr int WEIGHT_LOADS = (NB - 1) * 2 * C;
  static_assert(WEIGHT_LOADS <= 63, "vmcnt field is 6 bits");
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(WEIGHT_LOADS) : "memory");
  __builtin_amdgcn_sched_barrier(0);
  uint32_t hreg[C * 16];
#pragma unroll
  for (int i = 0; i < C; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = hl[wave][(g + G * i) * 4 + q];
      hreg[i * 16 + 4 * q + 0] = v.x;
      hreg[i * 16 + 4 * q + 1] = v.y;
      hreg[i * 16 + 4 * q + 2] = v.z;
      hreg[i * 16 + 4 * q + 3] = v.w;
    }
  }
  const float gs = LOGITS ? *a.global_scale : 1.0f;
  float best_v = -INFINITY;
  int best_r = INT_MAX;

  if (n_it > 0) {
    for (int it = 0; it < n_pad; it += NB) {
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        load_rows<G, C>(buf[(k + NB - 1) % NB], a, row_of(it + k + NB - 1), g);
        __builtin_amdgcn_sched_barrier(0);
        if (it + k < n_it)  // wave-uniform: padded iterations only load
          compute_rows<G, C, LOGITS>(buf[k], a, row_of(it + k), g, hreg, gs,
                                     best_v, best_r);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if constexpr (!LOGITS) {
    float bv[1] = {best_v};
    int br[1] = {best_r};
    argmax_finish<1, NT>(bv, br, a);
  }
}

// Any hidden % 16 == 0 and batch slices of 1-8 rows: one head row per wave
// iteration, 8-byte (one block) units strided over the 64 lanes, h for
// every batch row in LDS.
template <int B, bool LOGITS>
__global__ __launch_bounds__(THREADS) void k_nvfp4_generic(const KArgs a) {
  constexpr int NW = THREADS / 64;
  extern __shared__ uint32_t hs[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  stage_h<THREADS>(a.h, B * a.hidden, hs);
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
  for (int64_t row = r0 + wave; row < r1; row += NW) {
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
  if constexpr (!LOGITS) argmax_finish<B, THREADS>(best_v, best_r, a);
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
  int threads;
  bool fast;
};

// Batch-1 kernel shape: two register buffers, 256-thread blocks (the
// occupancy query then fits three blocks per CU at <= 168 VGPRs).
constexpr int RING = 2;
constexpr int B1_THREADS = 256;

template <int G, int C, bool L>
Variant b1_variant() {
  return Variant{k_nvfp4_b1<G, C, L, RING, B1_THREADS>, 64 / G, B1_THREADS,
                 true};
}

template <bool L>
bool pick_variant(int64_t hidden, int bc, Variant* v) {
  if (bc == 1 && hidden % 32 == 0) {
    switch (hidden / 32) {  // 16-byte chunks per row = G * C
      case 8: *v = b1_variant<8, 1, L>(); return true;
      case 16: *v = b1_variant<16, 1, L>(); return true;
      case 32: *v = b1_variant<32, 1, L>(); return true;
      case 64: *v = b1_variant<64, 1, L>(); return true;
      case 80: *v = b1_variant<16, 5, L>(); return true;
      case 128: *v = b1_variant<32, 4, L>(); return true;
      case 160: *v = b1_variant<32, 5, L>(); return true;
    }
  }
  switch (bc) {
    case 1: *v = Variant{k_nvfp4_generic<1, L>, 1, THREADS, false}; return true;
    case 2: *v = Variant{k_nvfp4_generic<2, L>, 1, THREADS, false}; return true;
    case 4: *v = Variant{k_nvfp4_generic<4, L>, 1, THREADS, false}; return true;
    case 8: *v = Variant{k_nvfp4_generic<8, L>, 1, THREADS, false}; return true;
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
        &occ, reinterpret_cast<const void*>(v.fn), v.threads, lds);
    if (e != hipSuccess) return e;
    if (occ < 1) occ = 1;
    // one resident wave of blocks, but at least one row group per wave
    const int waves = v.threads / 64;
    const int64_t groups = ga.n_rows / v.rows_per_iter;
    int64_t grid = (int64_t)di.cus * occ;
    const int64_t by_work = (groups + waves - 1) / waves;
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
                        dim3((unsigned)grid), dim3(v.threads), kargs, lds, s);
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
