// Batched GEMV on the matrix cores: for a batch slice of up to 16 hidden
// states the head's weights are decoded to BF16 in registers (exactly) and
// multiplied with v_mfma_f32_16x16x32_bf16, fp32 accumulation, fused with the
// argmax (or the logits scatter) as in the batch-1 kernel.  Page 3
// ("...MTP-NVFP4-h98k", "How it was built") gives the NVFP4 recipe, page 2
// the per-tensor E4M3 head; the batch-16 decode step of the 98 304-row head
// is the workload this kernel is shaped for.
//
// MFMA operands (16x16x32, wave64):
//   A = h          lane l holds 8 BF16 of batch row m = l%16, k-slot group
//                  l/16;
//   B = weights^T  lane l holds 8 decoded weights of head row n = l%16, the
//                  same k-slot group;
//   D[m][n]        lane l, register j: m = 4*(l/16) + j, n = l%16.
// Which k a slot stands for is free as long as A and B agree, so each lane
// loads one 16-byte chunk of its own head row per step (chunk 4*step + l/16,
// 64 contiguous bytes per row per load instruction) and the A operand reads
// h at the matching k from LDS.  A chunk holds EPC/8 MFMA operands.
//
// Work: a wave owns units of RT row tiles (16 rows each) and walks the whole
// hidden dimension for each unit, one chunk per lane per tile per step, with
// a ring of NB register buffers (NB-1 steps of loads in flight).  h of the
// slice is staged once per block in LDS (row stride 2*hidden+16 bytes, so the
// 16 batch rows of a read fall on different banks), plus one zero row that
// the A-operand lanes of batch rows past the slice read.
#include "gemv_common.h"

namespace dh {
namespace {

constexpr int MFMA_THREADS = 1024;
constexpr int MFMA_RT = 2;  // 16-row tiles per work unit
constexpr int MFMA_NB = 3;  // register buffers in the ring

template <class F, int RT>
struct Step {
  uint4 p[RT];
  uint32_t s[RT];
};

// Scalar cursor over (unit, step) pairs of one wave, with the row base of
// the unit.
struct Cursor {
  int64_t row0;  // first row of the unit
  int it;        // step within the unit
};

// The EPC/8 MFMAs of one step: operand O of every tile's chunk against the
// h slots O of the lane's chunk.
template <class F, int O, int RT>
__device__ __forceinline__ void mfma_ops(const Step<F, RT>& b, const char* hp,
                                         f32x4 (&acc)[RT]) {
  if constexpr (O < F::EPC / 8) {
    const bf16x8 av = *reinterpret_cast<const bf16x8*>(hp + 16 * O);
#pragma unroll
    for (int t = 0; t < RT; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          av, F::template operand<O>(b.p[t], b.s[t]), acc[t], 0, 0, 0);
    mfma_ops<F, O + 1, RT>(b, hp, acc);
  }
}

template <class F, int RT, int NB, bool LOGITS, int NT>
__global__ __launch_bounds__(NT) void k_mfma(const KArgs a) {
  constexpr int NW = NT / 64;
  constexpr int UR = 16 * RT;       // rows per unit
  extern __shared__ uint4 hs[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, q = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int64_t hidden = a.hidden;
  const int nb = a.nb;

  // Stage h [nb][hidden] and one zero row into LDS (row stride SB4 uint4).
  const int64_t HU4 = hidden / 8;
  const int64_t SB4 = HU4 + 1;
  {
    const uint4* h4 = reinterpret_cast<const uint4*>(a.h);
    const int64_t tot = (int64_t)(nb + 1) * SB4;
    for (int64_t i = threadIdx.x; i < tot; i += NT) {
      const int64_t r = i / SB4, c = i - r * SB4;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (r < nb && c < HU4) v = h4[r * HU4 + c];
      hs[i] = v;
    }
  }
  __syncthreads();

  const int64_t U = a.n_rows / UR;
  const int64_t TW = (int64_t)gridDim.x * NW;
  const int64_t first = (int64_t)blockIdx.x * NW + wv;
  const int n_u = first < U ? (int)((U - first + TW - 1) / TW) : 0;
  const int64_t CPR = hidden / F::EPC;  // 16-byte chunks per row
  const int NI = (int)(CPR / 4);        // steps per unit
  const int n_s = n_u * NI;
  const int n_pad = (n_s + NB - 1) / NB * NB;
  const int64_t RB = CPR * 16;          // weight bytes per row
  const int64_t SPR = hidden / 16;      // scale bytes per row (NVFP4)

  // Per-lane constant parts of the addresses.
  uint32_t woff[RT], soff[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    woff[t] = (uint32_t)((16 * t + n) * RB + q * 16);
    soff[t] = (uint32_t)((16 * t + n) * SPR + q * 2);
  }
  // A-operand LDS address of this lane at step 0: batch row min(m, nb)
  // (row nb is zero), chunk q.
  const int mrow = n < nb ? n : nb;
  const uint32_t hoff = (uint32_t)(mrow * SB4 * 16 + q * F::EPC * 2);
  const char* hsb = reinterpret_cast<const char*>(hs);

  const Cursor start{(n_u > 0 ? first : 0) * UR, 0};
  const int64_t unit_stride = TW * UR;
  auto advance = [&](Cursor& c) {
    if (++c.it == NI) {
      c.it = 0;
      c.row0 += unit_stride;
    }
  };
  auto load = [&](Step<F, RT>& b, const Cursor& c) {
    const uint8_t* wb = a.w + c.row0 * RB + (int64_t)c.it * 64;
#pragma unroll
    for (int t = 0; t < RT; ++t)
      b.p[t] = *reinterpret_cast<const uint4*>(wb + woff[t]);
    if constexpr (F::SCALED) {
      const uint8_t* sb = a.scales + c.row0 * SPR + (int64_t)c.it * 8;
#pragma unroll
      for (int t = 0; t < RT; ++t)
        b.s[t] = *reinterpret_cast<const uint16_t*>(sb + soff[t]);
    }
  };

  f32x4 acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const float sc = LOGITS ? tensor_scale(a) : 1.0f;
  float best_v[4];
  int best_r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    best_v[j] = -INFINITY;
    best_r[j] = INT_MAX;
  }

  // The load cursor stops at the wave's last step: the surplus loads of the
  // padded ring re-read it (L2 hits) and are never computed.
  Cursor ld = start;
  int ld_count = 0;
  auto advance_ld = [&]() {
    if (ld_count + 1 < n_s) {
      advance(ld);
      ++ld_count;
    }
  };
  Step<F, RT> buf[NB];
#pragma unroll
  for (int k = 0; k < NB - 1; ++k) {
    load(buf[k], ld);
    advance_ld();
  }
  Cursor cp = start;
  for (int s = 0; s < n_pad; s += NB) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      load(buf[(k + NB - 1) % NB], ld);
      advance_ld();
      __builtin_amdgcn_sched_barrier(0);
      if (s + k < n_s) {  // wave-uniform
        mfma_ops<F, 0, RT>(buf[k], hsb + hoff + cp.it * (4 * F::EPC * 2), acc);
        if (cp.it == NI - 1) {
          // unit done: rows row0 + 16t + n, batch rows 4q + j
#pragma unroll
          for (int t = 0; t < RT; ++t) {
            const int64_t row = cp.row0 + 16 * t + n;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float v = acc[t][j];
              if constexpr (LOGITS) {
                const int m = 4 * q + j;
                if (m < nb && row < a.n_kept)
                  a.out_logits[(int64_t)m * a.vocab + a.dh_idx[row]] = v * sc;
              } else if (v > best_v[j]) {
                // a lane's rows ascend: strict > keeps the lowest
                best_v[j] = v;
                best_r[j] = (int)row;
              }
            }
            acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
          }
        }
        advance(cp);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if constexpr (!LOGITS) {
    // batch row b lives in register b%4 of the lanes with l/16 == b/4
    float bv[16];
    int br[16];
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      const bool own = q == (b >> 2);
      bv[b] = own ? best_v[b & 3] : -INFINITY;
      br[b] = own ? best_r[b & 3] : INT_MAX;
    }
    argmax_finish<16, NT>(bv, br, a);
  }
}

template <class F, bool L>
KernelDesc desc() {
  return KernelDesc{reinterpret_cast<const void*>(
                        k_mfma<F, MFMA_RT, MFMA_NB, L, MFMA_THREADS>),
                    MFMA_THREADS, 16 * MFMA_RT, 0};
}

template <class F>
bool pick(int64_t hidden, int nb, bool logits, int lds_per_block,
          KernelDesc* d) {
  if (hidden % (4 * F::EPC) != 0) return false;
  if (nb < 1 || nb > mfma_max_slice(hidden, lds_per_block)) return false;
  *d = logits ? desc<F, true>() : desc<F, false>();
  d->lds_bytes = (size_t)(nb + 1) * (size_t)(hidden * 2 + 16);
  return true;
}

}  // namespace

int mfma_max_slice(int64_t hidden, int lds_per_block) {
  const int64_t row = hidden * 2 + 16;
  int64_t nb = (int64_t)lds_per_block / row - 1;
  if (nb > 16) nb = 16;
  return nb < 0 ? 0 : (int)nb;
}

bool mfma_kernel(int fmt, int64_t hidden, int nb, bool logits,
                 int lds_per_block, KernelDesc* out) {
  switch (fmt) {
    case FMT_NVFP4: return pick<Nvfp4>(hidden, nb, logits, lds_per_block, out);
    case FMT_E4M3: return pick<E4m3>(hidden, nb, logits, lds_per_block, out);
    case FMT_BF16: return pick<Bf16>(hidden, nb, logits, lds_per_block, out);
  }
  return false;
}

}  // namespace dh
