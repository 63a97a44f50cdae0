// Internal interface between the C-ABI layer (api.hip) and the kernel
// launchers.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dh {

// Workspace layout (bytes).  The caller zero-fills it once; after that it
// carries state from call to call and must not be modified between calls.
//   WS_EPOCH   uint32 call counter of the argmax finish (tags its slots)
//   WS_STATUS  uint16, nonzero once a collector of the argmax finish gave
//              up waiting; sticky: every later top-token call on this
//              workspace writes -1 until the caller zero-fills it again
//              (DH_WS_STATUS_OFFSET in drafthead.h)
//   WS_SPIN    uint16 bound on a collector's empty polling rounds: 0 = the
//              default FINISH_SPIN_LIMIT, n > 0 = n - 1 rounds, so 1 gives
//              up before the first poll (DH_WS_SPIN_LIMIT_OFFSET)
//   (the three share the 64-bit word at 0, which every block loads once)
//   WS_AMAX    amax bits of the quantizers, returned to zero by each call
//   WS_SLOTS   16-byte tagged (value, row) slots, one per block per batch
//              row of a slice (at most MAX_SLICE)
constexpr size_t WS_EPOCH = 0;
constexpr size_t WS_STATUS = 4;
constexpr size_t WS_SPIN = 6;
constexpr size_t WS_AMAX = 64;
constexpr size_t WS_SLOTS = 256;
constexpr int MAX_GRID = 4096;  // upper bound of any argmax grid
constexpr int MAX_BATCH = 64;
constexpr int MAX_SLICE = 16;   // batch rows per kernel launch
constexpr int64_t MAX_TOKENS = 1 << 16;  // rows of one token quantization

size_t workspace_bytes(int64_t n_rows, int64_t batch);

// Properties of the current device, queried once per device.
struct DeviceInfo {
  int dev;
  int cus;
  int lds_per_block;
};
hipError_t device_info(DeviceInfo* out);

struct QuantArgs {
  const uint16_t* w;
  int64_t vocab, hidden;
  const int32_t* ids;
  int64_t n_rows;
  uint8_t* packed;
  uint8_t* scales;
  float* global_scale;
  uint8_t* ws;
  bool f16 = false;  // w holds binary16 values instead of BF16
};
hipError_t launch_nvfp4_quantize(const QuantArgs& a, hipStream_t s);

struct QuantE4m3Args {
  const uint16_t* w;
  int64_t vocab, hidden;
  const int32_t* ids;
  int64_t n_rows;
  uint8_t* q;
  float* scale;
  uint8_t* ws;
};
hipError_t launch_e4m3_quantize(const QuantE4m3Args& a, hipStream_t s);

// Per-token E4M3 quantization of h [batch][hidden] (hidden % 8 == 0): codes
// to qx, their exact BF16 values to hq (either may be null), scales to sx.
hipError_t launch_fp8_tokens(const uint16_t* h, int64_t batch, int64_t hidden,
                             uint8_t* qx, uint16_t* hq, float* sx,
                             hipStream_t s);

// One GEMV call: weight format (WeightFormat in formats.h), the head, h and
// either out_ids (top tokens) or out_logits (logits scatter).
struct GemvArgs {
  int fmt;
  const uint8_t* w;       // NVFP4 packed codes, E4M3 bytes or BF16 rows
  const uint8_t* scales;  // NVFP4 block scales, else null
  const float* scale;     // NVFP4 global / E4M3 tensor scale; null for BF16
  const int32_t* dh_idx;
  int64_t n_rows, hidden;
  const uint16_t* h;
  int64_t batch;
  int32_t* out_ids;   // top-token mode
  float* out_logits;  // logits mode when non-null
  int64_t n_kept, vocab;
  uint8_t* ws;
  // Dense output (the linear): out_logits[b][j] for every row j, no index,
  // no -inf fill; dh_idx, n_kept and vocab are ignored.
  bool dense = false;
  // Logits only: one more factor per batch row (the W8A8 head's token
  // scales), null for none.
  const float* row_scale = nullptr;
  // The W8A8 step (E4M3 head): the tokens' E4M3 codes [batch][hidden]
  // beside their BF16 values in h; the batched slices multiply the codes on
  // the FP8 matrix cores, the others use h.  Null otherwise.
  const uint8_t* h_fp8 = nullptr;
  // The pages' own numerics (NVFP4 only): the top token of the scaled
  // logits rounded to BF16, or BF16 logits (out_logits then points to
  // BF16 [batch][vocab]).
  bool bf16_logits = false;
};
hipError_t launch_gemv(const GemvArgs& a, hipStream_t s);

// The plain streaming read of a then b (drafthead_read_probe).
hipError_t launch_read_probe(const void* a, size_t a_bytes, const void* b,
                             size_t b_bytes, uint32_t* sink, hipStream_t s);

}  // namespace dh
