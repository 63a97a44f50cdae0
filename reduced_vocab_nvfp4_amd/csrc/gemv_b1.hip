// Batch-1 GEMV fused with the argmax (or the logits scatter): the draft step
// at batch 1 is a stream over the head's bytes, so HBM bandwidth bounds it
// (page 4, "Qwen3.8-27B-NVFP4-DGX-SPARK": the draft step is dominated by
// reading the lm_head).
//
// Shape: hidden = EPC*G*C for the format's EPC elements per 16-byte chunk.
// A wave is 64/G groups of G lanes, one head row per group per iteration;
// lane g of a group owns chunks g, g+G, ..., g+(C-1)G of every row, so
//   * each 128-bit load instruction reads G*16 contiguous bytes per row
//     (256 B for G=16): fully coalesced;
//   * the lane's slice of h is the same for every row: it is staged once per
//     wave through LDS and then held in C*EPC/2 VGPRs for the whole kernel.
// Weights are decoded in registers (formats.h), multiplied against h with
// v_dot2_f32_bf16, NVFP4 block partials are scaled by their E4M3 scale, and
// a DPP reduction over the G lanes finishes the row.  A ring of NB register
// buffers keeps NB-1 row groups in flight while one is reduced.
//
// Argmax: every lane keeps (best value, its row) over the rows it saw in
// ascending order; argmax_finish reduces them across the block and the grid.
#include "gemv_common.h"

namespace dh {
namespace {

// A wave-uniform 64-bit value moved to scalar registers.
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

template <class F, int C>
struct Rows {
  uint4 p[C];
  uint32_t s[C];
  int32_t id;  // scatter modes: dh_idx of the group's rows (see load_rows)
};

// Loads the C chunks (and their scales) of one row group for this lane.
// row0 is the group's first row (wave-uniform), lane_chunk = grp * CPR + g
// the lane's first chunk within the group (loop-invariant): the address is a
// scalar base plus a fixed per-lane offset, so no per-iteration address
// registers are written while earlier loads are still outstanding.
template <class F, int G, int C, int MODE>
__device__ __forceinline__ void load_rows(Rows<F, C>& r, const KArgs& a,
                                          int64_t row0, uint32_t lane_chunk) {
  constexpr int64_t CPR = (int64_t)G * C;  // chunks per row
  // the group offset is made explicitly scalar, so the loads take the
  // scalar-base + lane-offset form
  const uint64_t woff = uniform_u64((uint64_t)row0 * (uint64_t)(CPR * 16));
  const uint8_t* wb = a.w + woff;
  // the head is read once per call: non-temporal loads keep it from
  // displacing h and the scales in the caches
#pragma unroll
  for (int i = 0; i < C; ++i) {
    const u32x4 t = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(wb + 16u * (lane_chunk + G * i)));
    r.p[i] = make_uint4(t[0], t[1], t[2], t[3]);
  }
  if constexpr (F::SCALED) {
    // two E4M3 scales per chunk
    const uint8_t* sb = a.scales + (woff >> 3);
#pragma unroll
    for (int i = 0; i < C; ++i)
      r.s[i] =
          *reinterpret_cast<const uint16_t*>(sb + 2u * (lane_chunk + G * i));
  }
  if constexpr (is_scatter(MODE)) {
    // lane l < R + 1 loads dh_idx[row0 - 1 + l] (the kept id before the
    // group, then the group's R ids); the other lanes repeat lane R's
    constexpr int R = 64 / G;
    const int l = (int)(threadIdx.x & 63);
    const int64_t j = row0 - 1 + (l < R ? l : R);
    r.id = a.dh_idx[j < 0 ? 0 : j];
  }
}

// Logits of one row group (scatter modes): the wave writes the id range its
// kept rows own (owned_ids), the group's logits at their ids and -inf
// between them.  Called by the whole wave; row0 is wave-uniform and every
// lane of group i holds row row0 + i's sum v.
template <int G, int MODE>
__device__ __forceinline__ void scatter_group(const KArgs& a, int64_t row0,
                                              int32_t id, float v, float sc) {
  constexpr int R = 64 / G;
  if (row0 >= a.n_kept) return;  // pad rows only
  const int64_t left = a.n_kept - row0;
  const int nk = left < R ? (int)left : R;
  int32_t ids[R];
  float vals[R];
  int32_t last_id = 0;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    ids[i] = __builtin_amdgcn_readlane(id, i + 1);
    vals[i] = __int_as_float(
                  __builtin_amdgcn_readlane(__float_as_int(v), i * G)) *
              sc;
    if (i < nk) last_id = ids[i];
  }
  const IdRange rg = owned_ids(row0, nk, __builtin_amdgcn_readlane(id, 0),
                               last_id, a.n_kept, a.vocab);
  const int lane = (int)(threadIdx.x & 63);
  for (int64_t p0 = rg.lo; p0 < rg.hi; p0 += 64) {
    const int64_t p = p0 + lane;
    float out = not_kept_value<MODE>();
#pragma unroll
    for (int i = 0; i < R; ++i)
      if (i < nk && p == ids[i]) out = vals[i];
    if (p < rg.hi) store_logit<MODE>(a.out_logits, p, out);
  }
}

template <class F, int G, int C, int MODE>
__device__ __forceinline__ void compute_rows(const Rows<F, C>& r,
                                             const KArgs& a, int64_t row,
                                             int g, const uint32_t* hreg,
                                             float sc, float& best_v,
                                             int& best_r) {
  constexpr int HD = F::EPC / 2;  // h dwords per chunk
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < C; ++i)
    acc = F::chunk_dot(r.p[i], F::SCALED ? r.s[i] : 0u, hreg + i * HD, acc);
  const float v = group_sum<G>(acc);
  if constexpr (is_scatter(MODE)) {
    scatter_group<G, MODE>(a, row - (int64_t)(threadIdx.x & 63) / G, r.id, v,
                           sc);
  } else if constexpr (MODE == OUT_DENSE) {
    if (g == 0 && row < a.n_kept) store_logit<MODE>(a.out_logits, row, v * sc);
  } else {
    const float c = top_value<MODE>(v, sc);
    if (better(c, (int)row, best_v, best_r)) {
      // (the waves of a block share its groups, so a lane's rows do not
      // come in ascending order: equal values keep the lower row)
      best_v = c;
      best_r = (int)row;
    }
  }
}

// Format F, G lanes per row, C chunks per lane, NT threads per block.
//
// Work: the row groups (R = 64/G rows each) are cut into one contiguous
// slice per block, and the waves of a block take the groups of its slice
// one at a time from a counter in LDS.  A CU's waves then finish within a
// group of each other whatever the issue arbitration favours (with a
// static per-wave split the oldest waves finished in half the time of the
// youngest and the last ones streamed alone), and each block reads its
// slice in address order.  A ring of two register buffers keeps one group
// in flight while another is reduced: each step takes the next group's
// index from the counter, issues its loads, then reduces the group loaded
// one step earlier.
template <class F, int G, int C, int MODE, int NT>
__global__ __launch_bounds__(NT) void k_b1(const KArgs a) {
  constexpr bool LOGITS = !is_top(MODE);
  constexpr int R = 64 / G;  // rows per wave iteration
  constexpr int NW = NT / 64;
  constexpr int HD = F::EPC / 2;           // h dwords per chunk
  constexpr int HQ = F::EPC / 8;           // h uint4 per chunk
  constexpr int HU4 = HQ * G * C;          // h as uint4
  constexpr int HJ = (HU4 + 63) / 64;      // 1 KB pieces of h
  constexpr uint32_t NONE = 0xFFFFFFFFu;   // no group left
  __shared__ uint4 hl[HJ * 64];
  __shared__ uint32_t next_group;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane / G, g = lane % G;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const FinishState st = LOGITS ? FinishState{} : finish_state(a);

  // The block's slice [g0, g0 + NG) of the T row groups; the host launches
  // no more blocks than groups, so NG >= 1.
  const int64_t T = a.n_rows / R;
  const int64_t g0 = (int64_t)blockIdx.x * T / gridDim.x;
  const uint32_t NG =
      (uint32_t)((int64_t)(blockIdx.x + 1) * T / gridDim.x - g0);
  const uint32_t lane_chunk = (uint32_t)(grp * G * C + g);
  auto row0_of = [&](uint32_t gi) { return (g0 + gi) * R; };

  // Prologue.  The block's one copy of h goes straight into LDS with
  // global_load_lds_dwordx4, a 1 KB piece per wave (lane i's 16 bytes land
  // at piece + 16*i; lanes past the end of h re-read its last uint4 into
  // the slack).  Wave w then issues the loads of group w; its explicit
  // wait covers its own copies (vector loads retire in issue order), and
  // the barrier covers every wave's.  The counter starts past the groups
  // the waves took here.
  // Every wave issues the same number of copies, in straight-line code
  // (pieces past the last are clamped to it: a second copy of the same
  // bytes), so the compiler keeps them ahead of the weight loads that the
  // explicit wait below counts.
  const uint4* h4 = reinterpret_cast<const uint4*>(a.h);
  constexpr int CPW = (HJ + NW - 1) / NW;  // copies per wave
#pragma unroll
  for (int t = 0; t < CPW; ++t) {
    const int j = wv + NW * t < HJ ? wv + NW * t : HJ - 1;
    const int src = (HU4 % 64 == 0 || 64 * j + lane < HU4) ? 64 * j + lane
                                                            : HU4 - 1;
    lds_copy_x4(h4 + src, lds_addr(&hl[64 * j]));
  }
  if (threadIdx.x == 0) next_group = NW;
  __builtin_amdgcn_sched_barrier(0);
  Rows<F, C> buf[2];
  uint32_t gi[2];
  gi[0] = (uint32_t)wv < NG ? (uint32_t)wv : NONE;
  load_rows<F, G, C, MODE>(buf[0], a, row0_of(gi[0] != NONE ? gi[0] : NG - 1),
                           lane_chunk);
  constexpr int WEIGHT_LOADS =
      (F::SCALED ? 2 : 1) * C + (is_scatter(MODE) ? 1 : 0);
  static_assert(WEIGHT_LOADS <= 63, "vmcnt field is 6 bits");
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(WEIGHT_LOADS) : "memory");
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
  uint32_t hreg[C * HD];
#pragma unroll
  for (int i = 0; i < C; ++i) {
#pragma unroll
    for (int q = 0; q < HQ; ++q) {
      const uint4 v = hl[(g + G * i) * HQ + q];
      hreg[i * HD + 4 * q + 0] = v.x;
      hreg[i * HD + 4 * q + 1] = v.y;
      hreg[i * HD + 4 * q + 2] = v.z;
      hreg[i * HD + 4 * q + 3] = v.w;
    }
  }
  const float sc = MODE != OUT_TOP ? logit_scale(a, 0) : 1.0f;
  float best_v = -INFINITY;
  int best_r = INT_MAX;
  // next group of the slice, or NONE (one LDS atomic per wave and step)
  auto take = [&]() {
    uint32_t n = 0;
    if (lane == 0)
      n = __hip_atomic_fetch_add(&next_group, 1u, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WORKGROUP);
    n = __builtin_amdgcn_readfirstlane(n);
    return n < NG ? n : NONE;
  };
  // The ring: step k issues the loads of the next group into the buffer
  // freed one step earlier, then reduces buffer k.  Groups come from the
  // counter in increasing order, so the first NONE ends the wave's work.
  // Every step loads (a NONE step re-reads the slice's last group, an L2
  // hit that is never reduced): loads that depend on the counter would cost
  // the loop exact wait counts.
  bool live = gi[0] != NONE;
  while (live) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t nx = take();
      gi[1 - k] = nx;
      load_rows<F, G, C, MODE>(buf[1 - k], a,
                               row0_of(nx != NONE ? nx : NG - 1), lane_chunk);
      __builtin_amdgcn_sched_barrier(0);
      if (gi[k] == NONE) {
        live = false;
        break;
      }
      compute_rows<F, G, C, MODE>(buf[k], a, row0_of(gi[k]) + grp, g, hreg,
                                  sc, best_v, best_r);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if constexpr (!LOGITS) {
    float bv[1] = {best_v};
    int br[1] = {best_r};
    // 2 slots per thread: the grid is two 256-thread blocks per CU
    argmax_finish<1, NT, 2>(bv, br, a, st);
  }
}

// Kernel shape: 256-thread blocks, two per CU (eight waves per CU; a third
// block measured slower: its waves start late and its extra loads buy no
// bandwidth).
constexpr int B1_THREADS = 256;
constexpr int B1_BLOCKS_PER_CU = 2;

template <class F, int G, int C>
constexpr bool fits() {
  return (((F::EPC / 8) * G * C + 63) / 64) * 64 * 16 <= 64 * 1024;
}

template <class F, int G, int C, int L>
bool desc(KernelDesc* d) {
  if constexpr (fits<F, G, C>()) {
    *d = KernelDesc{reinterpret_cast<const void*>(k_b1<F, G, C, L, B1_THREADS>),
                    B1_THREADS, 64 / G, 0, false, 0, B1_BLOCKS_PER_CU};
    return true;
  }
  return false;
}

// (G, C) for a row of n chunks: G*C == n, G a power of two <= 64, C <= 5.
template <class F, int L>
bool pick(int64_t chunks, KernelDesc* d) {
  switch (chunks) {
    case 8: return desc<F, 8, 1, L>(d);
    case 16: return desc<F, 16, 1, L>(d);
    case 32: return desc<F, 32, 1, L>(d);
    case 64: return desc<F, 64, 1, L>(d);
    case 80: return desc<F, 16, 5, L>(d);
    case 128: return desc<F, 32, 4, L>(d);
    case 160: return desc<F, 32, 5, L>(d);
    case 256: return desc<F, 64, 4, L>(d);
    case 320: return desc<F, 64, 5, L>(d);
  }
  return false;
}

template <class F>
bool pick_fmt(int64_t hidden, int mode, KernelDesc* d) {
  if (hidden % F::EPC != 0) return false;
  const int64_t chunks = hidden / F::EPC;
  switch (mode) {
    case OUT_TOP: return pick<F, OUT_TOP>(chunks, d);
    case OUT_SCATTER: return pick<F, OUT_SCATTER>(chunks, d);
    case OUT_DENSE:
      if constexpr (F::kFmt == FMT_NVFP4) return pick<F, OUT_DENSE>(chunks, d);
      return false;
    case OUT_TOP_BF16:
      if constexpr (F::kFmt == FMT_NVFP4)
        return pick<F, OUT_TOP_BF16>(chunks, d);
      return false;
    case OUT_SCATTER_BF16:
      if constexpr (F::kFmt == FMT_NVFP4)
        return pick<F, OUT_SCATTER_BF16>(chunks, d);
      return false;
  }
  return false;
}

}  // namespace

bool b1_kernel(int fmt, int64_t hidden, int mode, KernelDesc* out) {
  switch (fmt) {
    case FMT_NVFP4: return pick_fmt<Nvfp4>(hidden, mode, out);
    case FMT_E4M3: return pick_fmt<E4m3>(hidden, mode, out);
    case FMT_BF16: return pick_fmt<Bf16>(hidden, mode, out);
  }
  return false;
}

}  // namespace dh
