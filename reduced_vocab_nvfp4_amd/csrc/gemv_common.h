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

// What a GEMV launch writes: the top token per batch row (through the
// argmax finish), the fp32 logits scattered to the full vocabulary at
// dh_idx[j] for j < n_kept, or the fp32 output of every row densely,
// out[b][j] (the plain linear).  The two BF16 modes are the pages' own
// numerics (their linear returns BF16): the top token of the logits
// (tensor scale applied) rounded to BF16, lowest row on ties, and the BF16
// logits scattered.
enum OutMode : int {
  OUT_TOP = 0,
  OUT_SCATTER = 1,
  OUT_DENSE = 2,
  OUT_TOP_BF16 = 3,
  OUT_SCATTER_BF16 = 4
};

constexpr bool is_top(int mode) {
  return mode == OUT_TOP || mode == OUT_TOP_BF16;
}

// Stores one logit (already scaled) in the mode's output type.
template <int MODE>
__device__ __forceinline__ void store_logit(float* out, int64_t off,
                                            float v) {
  if constexpr (MODE == OUT_SCATTER_BF16)
    reinterpret_cast<__bf16*>(out)[off] = (__bf16)v;  // round to nearest even
  else
    out[off] = v;
}

// The value the argmax compares: the unscaled logit (a positive scale does
// not change the order), or in the BF16 mode the scaled logit rounded to
// BF16, as the pages' argmax sees it.
template <int MODE>
__device__ __forceinline__ float top_value(float v, float sc) {
  if constexpr (MODE == OUT_TOP_BF16) return (float)(__bf16)(v * sc);
  return v;
}

// Output column of row j in the logits modes.
template <int MODE>
__device__ __forceinline__ int64_t out_col(const int32_t* dh_idx,
                                           int64_t row) {
  if constexpr (MODE == OUT_DENSE) return row;
  return dh_idx[row];
}

constexpr bool is_scatter(int mode) {
  return mode == OUT_SCATTER || mode == OUT_SCATTER_BF16;
}

// The value the scatter writes at ids that were not kept.
template <int MODE>
__device__ __forceinline__ float not_kept_value() {
  return -INFINITY;  // 0xFF800000, or 0xFF80 once rounded to BF16
}

// The id range of the logits that kept rows [r0, r0 + nk) own, nk >= 1,
// r0 + nk <= n_kept: from just past the previous kept id (0 for row 0) up to
// their last id, or to the end of the vocabulary for the group holding the
// last kept row.  The ranges of consecutive groups tile [0, vocab), so
// every logit is written exactly once, by the wave that owns the kept ids
// it holds or lies between: the -inf fill needs no launch of its own.  The
// bounds are clamped to [0, vocab), so ids outside the contract (out of
// range, not ascending) give wrong logits but never a store out of bounds.
struct IdRange {
  int64_t lo, hi;
};
__device__ __forceinline__ IdRange owned_ids(int64_t r0, int nk,
                                             int32_t prev_id,
                                             int32_t last_id,
                                             int64_t n_kept, int64_t vocab) {
  int64_t lo = r0 == 0 ? 0 : (int64_t)prev_id + 1;
  int64_t hi = r0 + nk == n_kept ? vocab : (int64_t)last_id + 1;
  if (lo < 0) lo = 0;
  if (hi > vocab) hi = vocab;
  return IdRange{lo, hi};
}

// One launch = one batch slice of at most 16 rows.
struct KArgs {
  const uint8_t* w;       // weight rows (format-specific bytes)
  const uint8_t* scales;  // NVFP4 block scales, else unused
  const float* scale;     // tensor scale (logits, BF16 top token); null = 1
  const int32_t* dh_idx;
  int64_t n_rows, hidden;
  const uint16_t* h;  // [nb][hidden] BF16, this slice
  int nb;             // batch rows in this slice
  int32_t* out_ids;   // [nb], top-token mode
  float* out_logits;  // [nb][vocab], logits mode
  int64_t n_kept, vocab;  // dense mode: n_kept = n_rows, vocab = row stride
  uint8_t* ws;
  int ks_log2;  // MFMA dense mode: log2 of the waves that share a unit
  const float* row_scale;  // logits: factor of batch row b (slice), or null
};

// Kernel descriptor used by the dispatcher.
struct KernelDesc {
  const void* fn;
  int threads;
  int rows_per_unit;  // rows one wave owns per work unit
  size_t lds_bytes;   // dynamic LDS
  bool spread;        // units dealt wave-major: one block per unit suffices
  int split_slots;    // > 0: the waves of a block may split a unit's
                      // split_slots slots over the hidden dimension
  int per_cu;         // > 0: blocks per CU to launch (else as many as fit)
  bool fp8_act = false;  // reads h as E4M3 codes (GemvArgs::h_fp8)
};

// Kernel families; each returns false when it has no kernel for the shape.
// mode is an OutMode; the dense mode exists for NVFP4 only.
bool b1_kernel(int fmt, int64_t hidden, int mode, KernelDesc* out);
// fp8_act: h holds E4M3 codes (the W8A8 step), one byte per element.
bool mfma_kernel(int fmt, int64_t hidden, int nb, int mode,
                 int lds_per_block, bool fp8_act, KernelDesc* out);
bool generic_kernel(int fmt, int nb, int64_t hidden, int mode,
                    KernelDesc* out);
// Largest batch slice the MFMA kernel can stage for this hidden size.
int mfma_max_slice(int64_t hidden, int lds_per_block, int h_bytes = 2);
// LDS the MFMA kernels declare statically (the finish's tables), kept out of
// the h slice's budget; a CPU test checks the built kernels against it.
constexpr int MFMA_STATIC_LDS = 4096;

// LDS bytes of one staged h row in the MFMA kernel: whole 1 KB pieces plus
// 16 bytes of bank skew.
__host__ __device__ inline int mfma_lds_row_bytes(int64_t hidden,
                                                  int h_bytes = 2) {
  return (int)((hidden * h_bytes + 1023) / 1024 * 1024 + 16);
}

__device__ __forceinline__ uint64_t pack_partial(float v, int r) {
  return ((uint64_t)(uint32_t)r << 32) | (uint64_t)__float_as_uint(v);
}

__device__ __forceinline__ float tensor_scale(const KArgs& a) {
  return a.scale ? *a.scale : 1.0f;
}

// The logits factor of batch row m of the slice: the tensor scale times the
// row's own scale when there is one (m < nb).
__device__ __forceinline__ float logit_scale(const KArgs& a, int m) {
  const float s = tensor_scale(a);
  return a.row_scale ? s * a.row_scale[m] : s;
}

// State of the argmax finish kept in the workspace: the call counter of the
// slots, the sticky give-up status and the polling-round bound.  A call's
// blocks tag their slots with counter + 1 (0 is skipped: a zero-filled slot
// is never valid) and the collecting block stores the tag back as the new
// counter once it has read every slot.  The previous call's store is
// visible to this one by stream order, and no block of this call reads the
// counter after the collector writes it (every block reads it before it
// publishes), so a plain load suffices.  Every wave issues it at the
// kernel's start, unconditionally, and only the argmax finish uses the
// values: their latency then hides behind the kernel's own work.  (They are
// atomic loads only to keep the compiler from turning them into scalar
// loads, whose wait would coincide with the first LDS wait.)
struct FinishState {
  uint64_t word;  // WS_EPOCH .. WS_SPIN
  __device__ uint32_t epoch() const { return (uint32_t)word; }
  __device__ uint32_t status() const { return (uint32_t)(word >> 32) & 0xFFFFu; }
  __device__ uint32_t spin() const { return (uint32_t)(word >> 48); }
};

__device__ __forceinline__ FinishState finish_state(const KArgs& a) {
  return FinishState{
      __hip_atomic_load(reinterpret_cast<uint64_t*>(a.ws + WS_EPOCH),
                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)};
}

// Block-level (value,row) reduction, the partial write and the collection
// of the partials.  best_v/best_r are this lane's candidates for the B batch
// columns of the slice (B = the slice's compile-time capacity; only the
// first a.nb are written out).  st = finish_state(a), loaded at the
// kernel's start (only thread 0's value is used).
//
// Cross-block protocol.  Every block publishes its (value, row) per batch
// column in a slot of two 64-bit words, (tag, value bits) and (tag, row),
// each written by an agent-scope atomic store (single-copy atomic, performed
// past the per-XCD L2), and exits without waiting for them.  The last block,
// after its own share of the rows, polls the slots of column 0 with
// agent-scope atomic loads until both words carry this call's tag; a slot
// can only hold that tag once this call's owner wrote it, and the values
// travel inside the atomics, so relaxed ordering suffices.  Column b is
// collected the same way by block gridDim.x - 1 - b % gridDim.x.  A
// collector keeps two polling rounds in flight, so it learns of the last
// slot about half a memory round trip after it lands, where counting
// arrivals costs a completion wait and an atomic round trip per counter
// level.  At batch 1 it also fetches dh_idx of its running best row after
// each round, so the winner's id is in hand when the last slot arrives;
// otherwise the thread holding the winner fetches it at the end.
//
// Termination: only the collectors (at most 16 blocks) wait, and only for
// slots that the other blocks publish without waiting on anything, so those
// blocks run to completion wherever and whenever they are dispatched and
// every wait ends.  The wait is also bounded: after FINISH_SPIN_LIMIT empty
// polling rounds (each waits out a memory round trip, so at least a few
// tenths of a second; the workspace's WS_SPIN word can lower the bound) a
// collector gives up, writes -1 for its batch row and sets the workspace's
// status word.  A block that had not started by then may still publish a
// slot with a tag the next call would also use, so a workspace whose status
// is set is never polled again: every later call's collectors write -1 at
// once, until the caller zero-fills the workspace (after the failed call
// has completed, so no block of it still runs).
constexpr int FINISH_SPIN_LIMIT = 1 << 22;

struct FinishSlot {
  uint64_t tv;  // tag << 32 | value bits
  uint64_t tr;  // tag << 32 | row
};

// Per-wave candidates of a block, one per batch column, in LDS.
template <int B, int NT>
struct WaveBest {
  float v[NT / 64][B];
  int r[NT / 64][B];
};

// The block's part once every wave has put its per-column best in w.  A
// collecting thread polls UNR slots per round: the kernel picks it so that
// one round covers its usual grid (the slot count) with NT threads and no
// thread loads a slot twice.
template <int B, int NT, int UNR>
__device__ __forceinline__ void finish_from_waves(const WaveBest<B, NT>& w,
                                                  const KArgs& a,
                                                  const FinishState& st) {
  static_assert(B >= 1 && B <= 64 && NT % 64 == 0, "columns within a wave");
  constexpr int NW = NT / 64;
  const float(&sv)[NW][B] = w.v;
  const int(&sr)[NW][B] = w.r;
  __shared__ float cv[NW];  // collection: per-wave best of one column
  __shared__ int cr[NW];
  __shared__ int failed;
  __shared__ uint32_t block_tag;
  __shared__ int spin_limit;  // -1: give up without polling
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  FinishSlot* slot = reinterpret_cast<FinishSlot*>(a.ws + WS_SLOTS);
  if (threadIdx.x == 0) {
    // The state word was loaded at the kernel's start; the empty asm keeps
    // the compiler from moving its first use (a move to scalar registers,
    // which waits for the load) up there.
    FinishState fs = st;
    asm volatile("" : "+v"(fs.word));
    failed = 0;
    block_tag = fs.epoch() + 1 == 0 ? 1u : fs.epoch() + 1;
    // rounds a collector may poll; a workspace whose status is set is never
    // polled again (see above), and a bound of 0 rounds gives up at once
    const uint32_t sp = fs.spin();
    const int lim = sp == 0 ? FINISH_SPIN_LIMIT : (int)sp - 1;
    spin_limit = (fs.status() != 0 || lim == 0) ? -1 : lim;
  }
  lds_barrier();  // LDS only: see lds_barrier
  const uint32_t tg = block_tag;
  if (threadIdx.x < B) {
    const int b = threadIdx.x;
    float v = sv[0][b];
    int r = sr[0][b];
    for (int w = 1; w < NW; ++w)
      if (better(sv[w][b], sr[w][b], v, r)) {
        v = sv[w][b];
        r = sr[w][b];
      }
    const uint64_t hi = (uint64_t)tg << 32;
    FinishSlot* s = slot + (int64_t)blockIdx.x * B + b;
    __hip_atomic_store(&s->tv, hi | __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&s->tr, hi | (uint32_t)r, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  // Collection.  Batch column b < min(nb, B) is collected by block
  // gridDim.x - 1 - b % gridDim.x: the columns of a wide slice are polled
  // from different CUs (the uncached polling loads of one CU are served one
  // after another), and the collectors are the blocks dispatched last,
  // which tend to finish last, so most slots are there by their first poll.
  // Thread t polls the slots of blocks t + k * NT, UNR of them per round
  // (further rounds if the grid has more than NT * UNR blocks).
  // Two rounds are in flight: round k+1 is issued before round k is
  // checked.  Every load of a round is issued whether or not its slot is
  // still pending (slot indices past the grid wrap to one of the thread's
  // own slots, and their results are ignored), so the number of loads
  // outstanding is the same on every path and the wait before a check
  // covers only the older round.
  const int nblk = (int)gridDim.x;
  const int ncol = a.nb < B ? a.nb : B;
  for (int b = nblk - 1 - (int)blockIdx.x; b < ncol; b += nblk) {
    float v = -INFINITY;
    int r = INT_MAX;
    int id = 0, id_row = -1;  // dh_idx[id_row] (batch 1: after each round)
    if (spin_limit < 0 && threadIdx.x == 0) failed = 1;
    for (int i0 = threadIdx.x; spin_limit >= 0 && i0 < nblk;
         i0 += NT * UNR) {
      uint32_t pending = 0;
      const FinishSlot* ps[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int i = i0 + u * NT;
        if (i < nblk) pending |= 1u << u;
        // past the grid: one of this thread's own slots again (a second
        // load of a line it polls anyway; a common clamp to the last slot
        // sends every thread's surplus loads to one address)
        ps[u] = slot + (int64_t)(i < nblk ? i : i % nblk) * B + b;
      }
      uint64_t v0[UNR], r0[UNR], v1[UNR], r1[UNR];
      auto issue = [&](uint64_t (&tv)[UNR], uint64_t (&tr)[UNR]) {
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          tv[u] = __hip_atomic_load(&ps[u]->tv, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
          tr[u] = __hip_atomic_load(&ps[u]->tr, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
        }
      };
      // takes the slots of a round that carry this call's tag in both words
      auto check = [&](const uint64_t (&tv)[UNR], const uint64_t (&tr)[UNR]) {
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          if (!((pending >> u) & 1u) || (tv[u] >> 32) != tg ||
              (tr[u] >> 32) != tg)
            continue;
          pending &= ~(1u << u);
          const float fv = __uint_as_float((uint32_t)tv[u]);
          const int fr = (int)(uint32_t)tr[u];
          if (better(fv, fr, v, r)) {
            v = fv;
            r = fr;
          }
        }
        // one load per round, also unconditional (row 0 until a row wins);
        // at batch 1 only: the wider slices measured faster fetching the
        // winner's id once, at the end
        if constexpr (B == 1) {
          id_row = (r >= 0 && r < a.n_rows) ? r : 0;
          id = a.dh_idx[id_row];
        }
      };
      issue(v0, r0);
      for (int spin = 0; pending != 0; spin += 2) {
        issue(v1, r1);
        check(v0, r0);
        if (pending == 0) break;
        issue(v0, r0);
        check(v1, r1);
        if (pending != 0 && spin >= spin_limit) {
          failed = 1;
          break;
        }
      }
    }
    // Block argmax of (v, r); the thread holding the winning row (rows are
    // unique within a column) writes its id, so no thread waits for another
    // thread's dh_idx fetch.
    float wvv = v;
    int wr = r;
    wave_argmax(wvv, wr);
    if (lane == 0) {
      cv[wave] = wvv;
      cr[wave] = wr;
    }
    lds_barrier();
    float fv = cv[0];
    int fr = cr[0];
    for (int w = 1; w < NW; ++w)
      if (better(cv[w], cr[w], fv, fr)) {
        fv = cv[w];
        fr = cr[w];
      }
    if (fr >= 0 && fr < a.n_rows) {
      if (r == fr)
        a.out_ids[b] = failed ? -1 : (id_row == r ? id : a.dh_idx[fr]);
    } else if (threadIdx.x == 0) {
      // no row won: only reachable when every logit is NaN (or when the
      // collector gave up before its first poll)
      a.out_ids[b] = failed ? -1 : a.dh_idx[0];
    }
    if (failed && threadIdx.x == 0)  // the status half of the dword at 4
      __hip_atomic_fetch_or(reinterpret_cast<uint32_t*>(a.ws + WS_STATUS), 1u,
                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    lds_barrier();  // cv/cr are reused by the next column
  }
  // The last block collects column 0, so it has seen every block's slot, and
  // with it every block's read of the counter, before it advances the
  // counter.
  if ((int)blockIdx.x == nblk - 1 && threadIdx.x == 0)
    __hip_atomic_store(reinterpret_cast<uint32_t*>(a.ws + WS_EPOCH), tg,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every lane holds a candidate for each of the B columns: one wave argmax
// per column.
template <int B, int NT, int UNR>
__device__ __forceinline__ void argmax_finish(float (&best_v)[B],
                                              int (&best_r)[B],
                                              const KArgs& a,
                                              const FinishState& st) {
  static_assert((B & (B - 1)) == 0, "batch slots are a power of two");
  __shared__ WaveBest<B, NT> w;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int b = 0; b < B; ++b) {
    wave_argmax(best_v[b], best_r[b]);
    if (lane == 0) {
      w.v[wave][b] = best_v[b];
      w.r[wave][b] = best_r[b];
    }
  }
  finish_from_waves<B, NT, UNR>(w, a, st);
}

// MFMA output layout: the 16 lanes of row q = lane / 16 hold the candidates
// of columns 4q + j in register j.  Four 16-lane DPP reductions, which run
// on the four rows at once, replace sixteen whole-wave ones.
template <int NT, int UNR>
__device__ __forceinline__ void argmax_finish_rows(float (&best_v)[4],
                                                   int (&best_r)[4],
                                                   const KArgs& a,
                                                   const FinishState& st) {
  __shared__ WaveBest<16, NT> w;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    row_argmax(best_v[j], best_r[j]);
    if ((lane & 15) == 0) {
      w.v[wave][4 * (lane >> 4) + j] = best_v[j];
      w.r[wave][4 * (lane >> 4) + j] = best_r[j];
    }
  }
  finish_from_waves<16, NT, UNR>(w, a, st);
}

}  // namespace dh
