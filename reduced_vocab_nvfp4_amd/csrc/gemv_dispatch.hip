// Launch planning of the GEMV calls: the batch is cut into slices, each slice
// goes to the batch-1 stream kernel (one row, a hidden size it has a shape
// for), the MFMA kernel (two or more rows, hidden a multiple of four
// chunks, h fits LDS) or the generic kernel, and the grid is sized to one
// resident wave of blocks (never more blocks than work units).  The logits
// path first fills the output with -inf (page 1, "q38_draft.py",
// compute_logits: ids that were not kept score -inf).
#include "gemv_common.h"

namespace dh {
namespace {

constexpr int FILL_THREADS = 256;
constexpr int GENERIC_LDS = 64 * 1024;

__global__ __launch_bounds__(FILL_THREADS) void k_fill_neg_inf(float* out,
                                                               int64_t n) {
  const int64_t n4 = n / 4;
  float4* o4 = reinterpret_cast<float4*>(out);
  const float ninf = -INFINITY;
  const int64_t stride = (int64_t)gridDim.x * FILL_THREADS;
  for (int64_t i = (int64_t)blockIdx.x * FILL_THREADS + threadIdx.x; i < n4;
       i += stride)
    o4[i] = make_float4(ninf, ninf, ninf, ninf);
  for (int64_t i = n4 * 4 + (int64_t)blockIdx.x * FILL_THREADS + threadIdx.x;
       i < n; i += stride)
    out[i] = ninf;
}

// The same fill for BF16 logits: -inf is 0xFF80, eight to a 16-byte store.
__global__ __launch_bounds__(FILL_THREADS) void k_fill_neg_inf_bf16(
    uint16_t* out, int64_t n) {
  const int64_t n8 = n / 8;
  uint4* o8 = reinterpret_cast<uint4*>(out);
  const uint32_t w = 0xFF80FF80u;
  const int64_t stride = (int64_t)gridDim.x * FILL_THREADS;
  for (int64_t i = (int64_t)blockIdx.x * FILL_THREADS + threadIdx.x; i < n8;
       i += stride)
    o8[i] = make_uint4(w, w, w, w);
  for (int64_t i = n8 * 8 + (int64_t)blockIdx.x * FILL_THREADS + threadIdx.x;
       i < n; i += stride)
    out[i] = 0xFF80u;
}

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

hipError_t plan_slice(const GemvArgs& ga, int64_t remaining,
                      const DeviceInfo& di, KernelDesc* d, int* bc) {
  const int mode = out_mode(ga);
  if (remaining == 1 && b1_kernel(ga.fmt, ga.hidden, mode, d)) {
    *bc = 1;
    return hipSuccess;
  }
  if (remaining >= 2) {
    int nb = mfma_max_slice(ga.hidden, di.lds_per_block);
    if (nb > remaining) nb = (int)remaining;
    if (nb >= 2 &&
        mfma_kernel(ga.fmt, ga.hidden, nb, mode, di.lds_per_block, d)) {
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
  if (logits && !ga.dense) {
    const int64_t n = ga.batch * ga.vocab;
    int64_t blocks = (n / 4 + FILL_THREADS - 1) / FILL_THREADS;
    if (blocks > (int64_t)di.cus * 8) blocks = (int64_t)di.cus * 8;
    if (blocks < 1) blocks = 1;
    if (ga.bf16_logits)
      k_fill_neg_inf_bf16<<<(int)blocks, FILL_THREADS, 0, s>>>(
          reinterpret_cast<uint16_t*>(ga.out_logits), n);
    else
      k_fill_neg_inf<<<(int)blocks, FILL_THREADS, 0, s>>>(ga.out_logits, n);
  }
  for (int64_t b0 = 0; b0 < ga.batch;) {
    KernelDesc d;
    int bc = 0;
    e = plan_slice(ga, ga.batch - b0, di, &d, &bc);
    if (e != hipSuccess) return e;
    if (d.lds_bytes > 64 * 1024) {
      e = hipFuncSetAttribute(d.fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)d.lds_bytes);
      if (e != hipSuccess) return e;
    }
    int occ = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, d.fn, d.threads,
                                                     d.lds_bytes);
    if (e != hipSuccess) return e;
    if (occ < 1) occ = 1;
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
    k.h = ga.h + b0 * ga.hidden;
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
