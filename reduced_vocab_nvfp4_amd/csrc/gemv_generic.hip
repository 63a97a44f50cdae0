// GEMV for every shape the batch-1 and MFMA kernels do not cover (any
// hidden % 16 == 0, batch slices of 1, 2, 4 or 8 rows): one head row per wave
// iteration, 8-byte units (one NVFP4 block, 8 E4M3 or 4 BF16 elements)
// strided over the 64 lanes, h of every batch row of the slice in LDS.
// Computes what gemv_common.h states; fused with the argmax or the logits
// scatter.
#include "gemv_common.h"

namespace dh {
namespace {

constexpr int THREADS = 256;

template <class F, int B, int MODE>
__global__ __launch_bounds__(THREADS) void k_generic(const KArgs a) {
  constexpr bool LOGITS = !is_top(MODE);
  constexpr int NW = THREADS / 64;
  constexpr int HD = F::EPU / 2;  // h dwords per unit
  extern __shared__ uint4 hs4[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const FinishState st = LOGITS ? FinishState{} : finish_state(a);
  {
    const uint4* src = reinterpret_cast<const uint4*>(a.h);
    const int n = (int)(B * a.hidden / 8);
    for (int t = threadIdx.x; t < n; t += THREADS) hs4[t] = src[t];
    __syncthreads();
  }
  const uint32_t* hs = reinterpret_cast<const uint32_t*>(hs4);
  const float sc = MODE != OUT_TOP ? tensor_scale(a) : 1.0f;
  float best_v[B];
  int best_r[B];
#pragma unroll
  for (int b = 0; b < B; ++b) {
    best_v[b] = -INFINITY;
    best_r[b] = INT_MAX;
  }
  const int64_t nu = a.hidden / F::EPU;  // units per row
  const int64_t r0 = (int64_t)blockIdx.x * a.n_rows / gridDim.x;
  const int64_t r1 = (int64_t)(blockIdx.x + 1) * a.n_rows / gridDim.x;
  for (int64_t row = r0 + wave; row < r1; row += NW) {
    const uint2* prow = reinterpret_cast<const uint2*>(a.w) + row * nu;
    const uint8_t* srow = a.scales + row * nu;  // NVFP4: one scale per unit
    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.0f;
    for (int64_t c = lane; c < nu; c += 64) {
      const uint2 p = prow[c];
      const uint32_t s = F::SCALED ? (uint32_t)srow[c] : 0u;
#pragma unroll
      for (int b = 0; b < B; ++b)
        acc[b] = F::unit_dot(p, s, hs + b * (a.hidden / 2) + c * HD, acc[b]);
    }
    if constexpr (is_scatter(MODE)) {
      // the row's logits at its id and -inf over the ids it owns
      // (owned_ids): the wave writes them for every batch row
      if (row < a.n_kept) {  // wave-uniform
        const int32_t id = a.dh_idx[row];
        const IdRange rg = owned_ids(row, 1, row > 0 ? a.dh_idx[row - 1] : 0,
                                     id, a.n_kept, a.vocab);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const float v = group_sum<64>(acc[b]) *
                          (a.row_scale ? sc * a.row_scale[b] : sc);
          for (int64_t p = rg.lo + lane; p < rg.hi; p += 64)
            store_logit<MODE>(a.out_logits, b * a.vocab + p,
                              p == id ? v : not_kept_value<MODE>());
        }
      }
      continue;
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float v = group_sum<64>(acc[b]);
      if constexpr (MODE == OUT_DENSE) {
        if (lane == 0)
          store_logit<MODE>(a.out_logits, b * a.vocab + row,
                            v * (a.row_scale ? sc * a.row_scale[b] : sc));
      } else {
        const float c = top_value<MODE>(v, sc);
        if (c > best_v[b]) {
          best_v[b] = c;
          best_r[b] = (int)row;
        }
      }
    }
  }
  // 4 slots per thread: the grid may hold several blocks per CU
  if constexpr (!LOGITS)
    argmax_finish<B, THREADS, 4>(best_v, best_r, a, st);
}

template <class F, int L>
bool pick(int nb, KernelDesc* d) {
  const void* fn = nullptr;
  switch (nb) {
    case 1: fn = reinterpret_cast<const void*>(k_generic<F, 1, L>); break;
    case 2: fn = reinterpret_cast<const void*>(k_generic<F, 2, L>); break;
    case 4: fn = reinterpret_cast<const void*>(k_generic<F, 4, L>); break;
    case 8: fn = reinterpret_cast<const void*>(k_generic<F, 8, L>); break;
    default: return false;
  }
  *d = KernelDesc{fn, THREADS, 1, 0, false};
  return true;
}

template <class F>
bool pick_fmt(int nb, int64_t hidden, int mode, KernelDesc* d) {
  if (hidden % F::EPU != 0) return false;
  bool ok = false;
  switch (mode) {
    case OUT_TOP: ok = pick<F, OUT_TOP>(nb, d); break;
    case OUT_SCATTER: ok = pick<F, OUT_SCATTER>(nb, d); break;
    case OUT_DENSE:
      if constexpr (F::kFmt == FMT_NVFP4) ok = pick<F, OUT_DENSE>(nb, d);
      break;
    case OUT_TOP_BF16:
      if constexpr (F::kFmt == FMT_NVFP4) ok = pick<F, OUT_TOP_BF16>(nb, d);
      break;
    case OUT_SCATTER_BF16:
      if constexpr (F::kFmt == FMT_NVFP4)
        ok = pick<F, OUT_SCATTER_BF16>(nb, d);
      break;
  }
  if (!ok) return false;
  d->lds_bytes = (size_t)nb * (size_t)hidden * 2;
  return true;
}

}  // namespace

bool generic_kernel(int fmt, int nb, int64_t hidden, int mode,
                    KernelDesc* out) {
  switch (fmt) {
    case FMT_NVFP4: return pick_fmt<Nvfp4>(nb, hidden, mode, out);
    case FMT_E4M3: return pick_fmt<E4m3>(nb, hidden, mode, out);
    case FMT_BF16: return pick_fmt<Bf16>(nb, hidden, mode, out);
  }
  return false;
}

}  // namespace dh
