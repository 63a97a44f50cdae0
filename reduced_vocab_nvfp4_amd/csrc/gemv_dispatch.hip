// Launch planning of the GEMV calls: the batch is cut into slices, each slice
// goes to the batch-1 stream kernel (one row, a hidden size it has a shape
// for), the MFMA kernel (two or more rows, hidden a multiple of four
// chunks, h fits LDS) or the generic kernel, and the grid is sized to one
// resident wave of blocks (never more blocks than work units).  In the
// logits modes each launch also writes -inf at the ids that were not kept
// (page 1, "q38_draft.py", compute_logits), in the same pass (owned_ids in
// gemv_common.h): one launch per slice.
#include "gemv_common.h"

#include <mutex>

namespace dh {
namespace {

constexpr int GENERIC_LDS = 64 * 1024;

// Largest generic slice in {8,4,2,1} that fits the remaining rows and LDS.
int generic_slice(int64_t remaining, int64_t hidden) {
  for (int bc = 8; bc > 1; bc >>= 1)
    if (bc <= remaining && (int64_t)bc * hidden * 2 <= GENERIC_LDS) return bc;
  return 1;
}

int out_mode(const GemvArgs& ga) {
  if (ga.out_logits == nullptr) return ga.bf16_logits ? OUT_TOP_BF16 : OUT_TOP;
  if (ga.dense) return OUT_DENSE;
  return ga.bf16_logits ? OUT_SCATTER_BF16 : OUT_SCATTER;
}

// Blocks of a kernel shape that fit one CU, queried once per (kernel, block
// size, dynamic LDS, device) and kept.  A kernel that needs more than 64 KB
// of dynamic LDS has its limit raised the first time, and raised again
// only when a later shape needs more (the limit never shrinks, so a cached
// shape stays launchable).  The lock makes the tables safe for concurrent
// host threads; the queries are a few microseconds, the lookup is not.
hipError_t occupancy(const KernelDesc& d, int dev, int* occ) {
  struct Occ {
    const void* fn;
    int dev, threads;
    size_t lds;
    int occ;
  };
  struct Lim {
    const void* fn;
    int dev;
    size_t lds;
  };
  constexpr int N = 512;
  static std::mutex mu;
  static Occ occs[N];
  static Lim lims[N];
  static int n_occ = 0, n_lim = 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < n_occ; ++i)
    if (occs[i].fn == d.fn && occs[i].dev == dev &&
        occs[i].threads == d.threads && occs[i].lds == d.lds_bytes) {
      *occ = occs[i].occ;
      return hipSuccess;
    }
  hipError_t e;
  if (d.lds_bytes > 64 * 1024) {
    int li = 0;
    while (li < n_lim && !(lims[li].fn == d.fn && lims[li].dev == dev)) ++li;
    if (li == n_lim || lims[li].lds < d.lds_bytes) {
      e = hipFuncSetAttribute(d.fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)d.lds_bytes);
      if (e != hipSuccess) return e;
      if (li == n_lim && n_lim < N) ++n_lim;
      if (li < N) lims[li] = Lim{d.fn, dev, d.lds_bytes};
    }
  }
  int o = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, d.fn, d.threads,
                                                   d.lds_bytes);
  if (e != hipSuccess) return e;
  if (o < 1) o = 1;
  if (n_occ < N) occs[n_occ++] = Occ{d.fn, dev, d.threads, d.lds_bytes, o};
  *occ = o;
  return hipSuccess;
}

hipError_t plan_slice(const GemvArgs& ga, int64_t remaining,
                      const DeviceInfo& di, KernelDesc* d, int* bc) {
  const int mode = out_mode(ga);
  if (remaining == 1 && b1_kernel(ga.fmt, ga.hidden, mode, d)) {
    *bc = 1;
    return hipSuccess;
  }
  if (remaining >= 2) {
    const bool fp8 = ga.h_fp8 != nullptr;
    int nb = mfma_max_slice(ga.hidden, di.lds_per_block, fp8 ? 1 : 2);
    if (nb > remaining) nb = (int)remaining;
    if (nb >= 2 && mfma_kernel(ga.fmt, ga.hidden, nb, mode, di.lds_per_block,
                               fp8, d)) {
      *bc = nb;
      return hipSuccess;
    }
  }
  *bc = generic_slice(remaining, ga.hidden);
  return generic_kernel(ga.fmt, *bc, ga.hidden, mode, d)
             ? hipSuccess
             : hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemv(const GemvArgs& ga, hipStream_t s) {
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  const bool logits = ga.out_logits != nullptr;
  for (int64_t b0 = 0; b0 < ga.batch;) {
    KernelDesc d;
    int bc = 0;
    e = plan_slice(ga, ga.batch - b0, di, &d, &bc);
    if (e != hipSuccess) return e;
    int occ = 0;
    e = occupancy(d, di.dev, &occ);
    if (e != hipSuccess) return e;
    if (d.per_cu > 0 && d.per_cu < occ) occ = d.per_cu;
    const int waves = d.threads / 64;
    const int64_t units = ga.n_rows / d.rows_per_unit;
    int64_t grid = (int64_t)di.cus * occ;
    const int64_t by_work = d.spread ? units : (units + waves - 1) / waves;
    if (grid > by_work) grid = by_work;
    // Fewer units than twice the resident blocks leave most waves idle and
    // each busy one a long chain of dependent slots: then 2^kl waves of a
    // block share a unit over the hidden dimension, as many as keep every
    // group to one unit and every wave to at least one slot.  The grid stays
    // one block per CU, so the decode spreads over every CU.  (With more
    // units the split's closing barrier costs more than it saves.)
    int kl = 0;
    if (d.split_slots > 0 && units < 2 * (int64_t)di.cus * occ) {
      const int64_t resident = (int64_t)di.cus * occ * waves;
      while ((2 << kl) <= waves && (2 << kl) <= d.split_slots &&
             units * (2 << kl) <= resident)
        ++kl;
    }
    if (grid > MAX_GRID) grid = MAX_GRID;
    if (grid < 1) grid = 1;
    KArgs k;
    k.w = ga.w;
    k.scales = ga.scales;
    k.scale = ga.scale;
    k.dh_idx = ga.dense ? nullptr : ga.dh_idx;
    k.n_rows = ga.n_rows;
    k.hidden = ga.hidden;
    // the W8A8 step's FP8 kernel reads the codes, every other kernel h
    k.h = d.fp8_act ? reinterpret_cast<const uint16_t*>(ga.h_fp8 + b0 * ga.hidden)
                    : ga.h + b0 * ga.hidden;
    k.nb = bc;
    k.out_ids = logits ? nullptr : ga.out_ids + b0;
    // dense: every row is written, out has n_rows columns
    const int64_t cols = ga.dense ? ga.n_rows : ga.vocab;
    // the slice's first output row (BF16 logits take two bytes each)
    k.out_logits =
        logits ? reinterpret_cast<float*>(
                     reinterpret_cast<char*>(ga.out_logits) +
                     b0 * cols * (ga.bf16_logits ? 2 : 4))
               : nullptr;
    k.n_kept = ga.dense ? ga.n_rows : ga.n_kept;
    k.vocab = cols;
    k.ws = ga.ws;
    k.ks_log2 = kl;
    k.row_scale = ga.row_scale ? ga.row_scale + b0 : nullptr;
    void* kargs[] = {&k};
    e = hipLaunchKernel(d.fn, dim3((unsigned)grid), dim3(d.threads), kargs,
                        d.lds_bytes, s);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return e;
    b0 += bc;
  }
  return hipSuccess;
}

}  // namespace dh
