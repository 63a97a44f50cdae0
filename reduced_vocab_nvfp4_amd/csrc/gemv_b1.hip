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
    if (c > best_v) {
      // rows reach a lane in ascending order: strict > keeps the lowest
      best_v = c;
      best_r = (int)row;
    }
  }
}

// Format F, G lanes per row, C chunks per lane, NB register buffers, NT
// threads per block.
template <class F, int G, int C, int MODE, int NB, int NT>
__global__ __launch_bounds__(NT) void k_b1(const KArgs a) {
  constexpr bool LOGITS = !is_top(MODE);
  constexpr int R = 64 / G;  // rows per wave iteration
  constexpr int NW = NT / 64;
  constexpr int HD = F::EPC / 2;           // h dwords per chunk
  constexpr int HQ = F::EPC / 8;           // h uint4 per chunk
  constexpr int HU4 = HQ * G * C;          // h as uint4
  constexpr int HJ = (HU4 + 63) / 64;      // h copies per lane
  __shared__ uint4 hl[NW][HJ * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane / G, g = lane % G;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const FinishState st = LOGITS ? FinishState{} : finish_state(a);

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
  auto row0_of = [&](int it) {  // first row of the group (wave-uniform)
    const int c = it < last ? it : last;
    return (base + (int64_t)c * TW) * R;
  };
  const uint32_t lane_chunk = (uint32_t)(grp * G * C + g);
  // Prologue.  h is copied straight into this wave's LDS slice with
  // global_load_lds_dwordx4 (lane i's 16 bytes land at slice + 16*i; no
  // VGPRs, no block barrier), then the first weight row groups are issued,
  // so only h has to arrive before the ring starts.  Every lane then keeps
  // its C chunks of h in VGPRs.
  const uint4* h4 = reinterpret_cast<const uint4*>(a.h);
#pragma unroll
  for (int j = 0; j < HJ; ++j) {
    // lanes past the end of h (when HU4 % 64 != 0) re-read its last uint4
    // into the slack of the slice
    const int src = (HU4 % 64 == 0 || 64 * j + lane < HU4) ? 64 * j + lane
                                                            : HU4 - 1;
    lds_copy_x4(h4 + src, lds_addr(&hl[wv][64 * j]));
  }
  __builtin_amdgcn_sched_barrier(0);
  Rows<F, C> buf[NB];
#pragma unroll
  for (int k = 0; k < NB - 1; ++k)
    load_rows<F, G, C, MODE>(buf[k], a, row0_of(k), lane_chunk);
  // Memory loads retire in issue order, so once no more than the weight
  // loads just issued are outstanding, the h copies have landed in LDS.
  // (The wait is explicit: the compiler does not order LDS reads after
  // global_load_lds on its own.)  The "memory" clobber keeps the LDS reads
  // below it.
  constexpr int WEIGHT_LOADS =
      (NB - 1) * ((F::SCALED ? 2 : 1) * C + (is_scatter(MODE) ? 1 : 0));
  static_assert(WEIGHT_LOADS <= 63, "vmcnt field is 6 bits");
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(WEIGHT_LOADS) : "memory");
  __builtin_amdgcn_sched_barrier(0);
  uint32_t hreg[C * HD];
#pragma unroll
  for (int i = 0; i < C; ++i) {
#pragma unroll
    for (int q = 0; q < HQ; ++q) {
      const uint4 v = hl[wave][(g + G * i) * HQ + q];
      hreg[i * HD + 4 * q + 0] = v.x;
      hreg[i * HD + 4 * q + 1] = v.y;
      hreg[i * HD + 4 * q + 2] = v.z;
      hreg[i * HD + 4 * q + 3] = v.w;
    }
  }
  const float sc = MODE != OUT_TOP ? logit_scale(a, 0) : 1.0f;
  float best_v = -INFINITY;
  int best_r = INT_MAX;

  if (n_it > 0) {
    for (int it = 0; it < n_pad; it += NB) {
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        load_rows<F, G, C, MODE>(buf[(k + NB - 1) % NB], a,
                                 row0_of(it + k + NB - 1), lane_chunk);
        __builtin_amdgcn_sched_barrier(0);
        if (it + k < n_it)  // wave-uniform: padded iterations only load
          compute_rows<F, G, C, MODE>(buf[k], a, row0_of(it + k) + grp, g,
                                        hreg, sc,
                                        best_v, best_r);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if constexpr (!LOGITS) {
    float bv[1] = {best_v};
    int br[1] = {best_r};
    argmax_finish<1, NT>(bv, br, a, st);
  }
}

// Kernel shape: two register buffers, 256-thread blocks (the occupancy
// query then fits three blocks per CU at <= 168 VGPRs).
constexpr int RING = 2;
constexpr int B1_THREADS = 256;

// Static LDS of the per-wave h slices must stay within 64 KB.
template <class F, int G, int C>
constexpr bool fits() {
  return (B1_THREADS / 64) * (((F::EPC / 8) * G * C + 63) / 64) * 64 * 16 <=
         64 * 1024;
}

template <class F, int G, int C, int L>
bool desc(KernelDesc* d) {
  if constexpr (fits<F, G, C>()) {
    *d = KernelDesc{reinterpret_cast<const void*>(
                        k_b1<F, G, C, L, RING, B1_THREADS>),
                    B1_THREADS, 64 / G, 0, false};
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
