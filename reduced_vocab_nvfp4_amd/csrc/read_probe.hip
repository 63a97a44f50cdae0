// A plain streaming read of a head's bytes, for the measurement: page 4
// ("autotrust/Qwen3.8-27B-NVFP4-DGX-SPARK", "Why native MTP plateaus at
// 37") treats the draft step as a stream of lm_head bytes, so the rate at
// which the device can stream those same bytes, with nothing else to do, is
// the practical ceiling the GEMV kernels are compared with.
//
// Shape (the fastest plain read measured for a 92 MB head): 256-thread
// blocks, three per CU; the two buffers are one sequence of 1 KB lines, and
// each wave reads its own contiguous run of lines, four lines (one 16-byte
// non-temporal load per lane each) in flight.  Each wave folds what it read
// into one 32-bit XOR and stores it to sink[0] only when it equals
// DRAFTHEAD_READ_PROBE_MAGIC, so the loads cannot be dropped and a test can
// check that every byte was read.
#include "drafthead.h"

#include "dh_device.h"
#include "dh_internal.h"
#include "formats.h"

namespace dh {
namespace {

constexpr int RP_THREADS = 256;
constexpr int RP_WAVES = RP_THREADS / 64;
constexpr int RP_BLOCKS_PER_CU = 3;
constexpr int RP_DEPTH = 4;

__global__ __launch_bounds__(RP_THREADS) void k_read_probe(
    const u32x4* __restrict__ a, int64_t na16, const u32x4* __restrict__ b,
    int64_t nb16, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t n16 = na16 + nb16;
  const int64_t lines = (n16 + 63) / 64;
  const int64_t nw = (int64_t)gridDim.x * RP_WAVES;
  const int64_t w = (int64_t)blockIdx.x * RP_WAVES +
                    __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t l0 = w * lines / nw, l1 = (w + 1) * lines / nw;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t l = l0; l < l1; l += RP_DEPTH) {
    u32x4 v[RP_DEPTH];
#pragma unroll
    for (int k = 0; k < RP_DEPTH; ++k) {
      const int64_t i = (l + k) * 64 + lane;
      v[k] = u32x4{0u, 0u, 0u, 0u};
      if (l + k < l1 && i < n16)
        v[k] = __builtin_nontemporal_load(i < na16 ? a + i : b + (i - na16));
    }
#pragma unroll
    for (int k = 0; k < RP_DEPTH; ++k) acc ^= v[k];
  }
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1)
    x ^= (uint32_t)__shfl_xor((int)x, off, 64);
  if (lane == 0 && x == DRAFTHEAD_READ_PROBE_MAGIC) sink[0] = x;
}

}  // namespace

hipError_t launch_read_probe(const void* a, size_t a_bytes, const void* b,
                             size_t b_bytes, uint32_t* sink, hipStream_t s) {
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  const int64_t n16 = (int64_t)((a_bytes + b_bytes) / 16);
  const int64_t lines = (n16 + 63) / 64;
  int64_t grid = (int64_t)di.cus * RP_BLOCKS_PER_CU;
  const int64_t by_work = (lines + RP_WAVES - 1) / RP_WAVES;
  if (grid > by_work) grid = by_work;
  if (grid < 1) grid = 1;
  k_read_probe<<<(unsigned)grid, RP_THREADS, 0, s>>>(
      static_cast<const u32x4*>(a), (int64_t)(a_bytes / 16),
      static_cast<const u32x4*>(b), (int64_t)(b_bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace dh
