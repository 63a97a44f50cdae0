// Pieces shared by the GEMV kernel families (batch-1 stream, MFMA, generic):
// the per-launch argument block, the cross-block argmax finish, and the
// kernel descriptors the dispatcher picks from.
//
// What every kernel computes (page 1, "q38_draft.py": get_top_tokens takes
// the argmax of the draft head's output over the kept rows and maps it
// through dh_idx; compute_logits writes the head's float32 output into a
// -inf filled batch x vocab tensor at the kept ids):
//   logit[b, j] = sum_k w(j, k) * h[b, k]       w the decoded weight, fp32
//   top token   = dh_idx[lowest j with the largest logit]
//   logits      = scale * logit[b, j] at out[b, dh_idx[j]] for j < n_kept
// The positive tensor scale (NVFP4 global scale, E4M3 tensor scale) does not
// change the argmax and is applied only on the logits path.
#pragma once

#include <limits.h>

#include "dh_internal.h"
#include "formats.h"

namespace dh {

// One launch = one batch slice of at most 16 rows.
struct KArgs {
  const uint8_t* w;       // weight rows (format-specific bytes)
  const uint8_t* scales;  // NVFP4 block scales, else unused
  const float* scale;     // tensor scale (logits only); null = 1
  const int32_t* dh_idx;
  int64_t n_rows, hidden;
  const uint16_t* h;  // [nb][hidden] BF16, this slice
  int nb;             // batch rows in this slice
  int32_t* out_ids;   // [nb], top-token mode
  float* out_logits;  // [nb][vocab], logits mode
  int64_t n_kept, vocab;
  uint8_t* ws;
};

// Kernel descriptor used by the dispatcher.
struct KernelDesc {
  const void* fn;
  int threads;
  int rows_per_unit;  // rows one wave owns per work unit
  size_t lds_bytes;   // dynamic LDS
  bool spread;        // units dealt wave-major: one block per unit suffices
};

// Kernel families; each returns false when it has no kernel for the shape.
bool b1_kernel(int fmt, int64_t hidden, bool logits, KernelDesc* out);
bool mfma_kernel(int fmt, int64_t hidden, int nb, bool logits,
                 int lds_per_block, KernelDesc* out);
bool generic_kernel(int fmt, int nb, int64_t hidden, bool logits,
                    KernelDesc* out);
// Largest batch slice the MFMA kernel can stage for this hidden size.
int mfma_max_slice(int64_t hidden, int lds_per_block);
// LDS bytes of one staged h row in the MFMA kernel: whole 1 KB pieces plus
// 16 bytes of bank skew.
__host__ __device__ inline int mfma_lds_row_bytes(int64_t hidden) {
  return (int)((hidden * 2 + 1023) / 1024 * 1024 + 16);
}

__device__ __forceinline__ uint64_t pack_partial(float v, int r) {
  return ((uint64_t)(uint32_t)r << 32) | (uint64_t)__float_as_uint(v);
}

__device__ __forceinline__ float tensor_scale(const KArgs& a) {
  return a.scale ? *a.scale : 1.0f;
}

// Block-level (value,row) reduction, the partial write and the last block's
// final pass.  best_v/best_r are this lane's candidates for the B batch
// columns of the slice (B = the slice's compile-time capacity; only the
// first a.nb are written out).
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
  static_assert(B >= 1 && B <= 64 && (B & (B - 1)) == 0 && NT % 64 == 0,
                "batch slots are a power of two within a wave");
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
  if (threadIdx.x < B) {
    const int b = threadIdx.x;
    float v = sv[0][b];
    int r = sr[0][b];
    for (int w = 1; w < NW; ++w)
      if (better(sv[w][b], sr[w][b], v, r)) {
        v = sv[w][b];
        r = sr[w][b];
      }
    __hip_atomic_store(&part[(int64_t)blockIdx.x * B + b], pack_partial(v, r),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (threadIdx.x < 64) {
    // all partial stores of the block come from wave 0 (B <= 64)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);  // the partial stores have completed
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  }
  if (threadIdx.x == 0) {
    const uint32_t nblk = gridDim.x;
    const uint32_t ng = nblk < ARRIVAL_GROUPS ? nblk : ARRIVAL_GROUPS;
    const uint32_t grp = blockIdx.x % ARRIVAL_GROUPS;
    const uint32_t gsize = (nblk - grp + ARRIVAL_GROUPS - 1) / ARRIVAL_GROUPS;
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
  // Final pass over gridDim.x * B partials: thread t reads the partials of
  // batch row t % B from blocks t / B, t / B + NT / B, ... (all its loads are
  // issued before any is used), then lanes of the same batch row (B apart in
  // a wave) and the waves combine.
  constexpr int PER = NT / B;  // blocks one round covers
  constexpr int UNR = 8;
  const int bt = threadIdx.x % B;
  float v = -INFINITY;
  int r = INT_MAX;
  for (int i0 = threadIdx.x / B; i0 < (int)gridDim.x; i0 += PER * UNR) {
    uint64_t pv[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int i = i0 + u * PER;
      pv[u] = i < (int)gridDim.x
                  ? __hip_atomic_load(&part[(int64_t)i * B + bt],
                                      __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT)
                  : pack_partial(-INFINITY, INT_MAX);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const float fv = __uint_as_float((uint32_t)pv[u]);
      const int fr = (int)(pv[u] >> 32);
      if (better(fv, fr, v, r)) {
        v = fv;
        r = fr;
      }
    }
  }
#pragma unroll
  for (int off = B; off < 64; off <<= 1) {
    const float ov = __shfl_xor(v, off, 64);
    const int orow = __shfl_xor(r, off, 64);
    if (better(ov, orow, v, r)) {
      v = ov;
      r = orow;
    }
  }
  if (lane < B) {
    sv[wave][lane] = v;
    sr[wave][lane] = r;
  }
  __syncthreads();
  if (threadIdx.x < B && threadIdx.x < a.nb) {
    const int b = threadIdx.x;
    float fv = sv[0][b];
    int fr = sr[0][b];
    for (int w = 1; w < NW; ++w)
      if (better(sv[w][b], sr[w][b], fv, fr)) {
        fv = sv[w][b];
        fr = sr[w][b];
      }
    if (fr < 0 || fr >= a.n_rows) fr = 0;  // only reachable with NaN inputs
    a.out_ids[b] = a.dh_idx[fr];
  }
}

}  // namespace dh
