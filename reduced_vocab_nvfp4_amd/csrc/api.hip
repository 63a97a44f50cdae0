// extern "C" entry points of the draft-head library: argument checks on the
// host (before any HIP call, so every error path runs without a device),
// then the kernel launchers.  Semantics and citations are documented at the
// declarations in include/drafthead.h.
#include "drafthead.h"

#include <mutex>

#include "dh_internal.h"
#include "formats.h"

namespace dh {

static bool aligned(const void* p, uintptr_t n) {
  return (reinterpret_cast<uintptr_t>(p) % n) == 0;
}

size_t workspace_bytes(int64_t n_rows, int64_t batch) {
  if (n_rows < 1 || batch < 1 || batch > MAX_BATCH) return 0;
  // A batch of one runs the one-row kernels (one argmax slot per block);
  // any larger batch may run a kernel with MAX_SLICE slots per block.
  const int64_t slots = batch == 1 ? 1 : MAX_SLICE;
  return WS_SLOTS + (size_t)MAX_GRID * (size_t)slots * 16;
}

// Queried once per device under a lock, so two host threads making their
// first call at the same time do not race on the cache.
hipError_t device_info(DeviceInfo* out) {
  constexpr int MAX_DEV = 64;
  static std::mutex mu;
  static DeviceInfo cache[MAX_DEV];
  static bool have[MAX_DEV];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= 0 && dev < MAX_DEV && have[dev]) {
    *out = cache[dev];
    return hipSuccess;
  }
  DeviceInfo d{};
  d.dev = dev;
  e = hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&d.lds_per_block,
                            hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess) return e;
  if (d.cus < 1) d.cus = 1;
  if (dev >= 0 && dev < MAX_DEV) {
    cache[dev] = d;
    have[dev] = true;
  }
  *out = d;
  return hipSuccess;
}

static int status(hipError_t e) { return e == hipSuccess ? DH_OK : DH_EHIP; }

// Shape and pointer checks shared by the GEMV entry points.  `scales` is
// checked only for NVFP4 and `scale` only for the scaled formats.
static int check_head(int fmt, const void* w, const uint8_t* scales,
                      const float* scale, const int32_t* dh_idx,
                      int64_t n_rows, int64_t hidden, const void* h,
                      int64_t batch, const void* ws, size_t ws_bytes) {
  if (!w || !dh_idx || !h) return DH_EINVAL;
  if (fmt == FMT_NVFP4 && (!scales || !aligned(scales, 16))) return DH_EINVAL;
  if (fmt != FMT_BF16 && (!scale || !aligned(scale, 4))) return DH_EINVAL;
  if (hidden < 16 || hidden > 16384 || hidden % 16 != 0) return DH_EINVAL;
  if (n_rows < 64 || n_rows % 64 != 0 || n_rows > INT32_MAX) return DH_EINVAL;
  if (batch < 1 || batch > MAX_BATCH) return DH_EINVAL;
  if (!aligned(w, 16) || !aligned(h, 16) || !aligned(dh_idx, 4))
    return DH_EINVAL;
  if (!ws || !aligned(ws, 16) || ws_bytes < workspace_bytes(n_rows, batch))
    return DH_EWORKSPACE;
  return DH_OK;
}

// Scratch of draft_head_top_tokens_noalloc: the largest workspace any batch
// needs, in static device storage (zero at load, one copy per GPU).  In host
// code `scratch` names a host-side stand-in, not device memory: the address
// kernels use is the one hipGetSymbolAddress returns with the device
// current, fetched on a device's first call and kept per device.
constexpr size_t NOALLOC_SCRATCH_BYTES =
    WS_SLOTS + (size_t)MAX_GRID * (size_t)MAX_SLICE * 16;
static_assert(NOALLOC_SCRATCH_BYTES == DRAFTHEAD_NOALLOC_SCRATCH_BYTES,
              "the header states the scratch size");
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

static hipError_t scratch_address(void** out) {
  constexpr int MAX_DEV = 64;
  static std::mutex mu;
  static void* addr[MAX_DEV];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEV) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

static int top_tokens(int fmt, const void* w, const uint8_t* scales,
                      const float* scale, const int32_t* dh_idx,
                      int64_t n_rows, int64_t hidden, const void* h,
                      int64_t batch, int32_t* out_ids, void* ws,
                      size_t ws_bytes, void* stream, bool bf16 = false) {
  if (!out_ids || !aligned(out_ids, 4)) return DH_EINVAL;
  const int rc = check_head(fmt, w, scales, scale, dh_idx, n_rows, hidden, h,
                            batch, ws, ws_bytes);
  if (rc != DH_OK) return rc;
  GemvArgs a{};
  a.fmt = fmt;
  a.w = static_cast<const uint8_t*>(w);
  a.scales = scales;
  a.scale = scale;
  a.dh_idx = dh_idx;
  a.n_rows = n_rows;
  a.hidden = hidden;
  a.h = static_cast<const uint16_t*>(h);
  a.batch = batch;
  a.out_ids = out_ids;
  a.ws = static_cast<uint8_t*>(ws);
  a.bf16_logits = bf16;
  return status(launch_gemv(a, static_cast<hipStream_t>(stream)));
}

static int logits(int fmt, const void* w, const uint8_t* scales,
                  const float* scale, const int32_t* dh_idx, int64_t n_rows,
                  int64_t n_kept, int64_t hidden, int64_t vocab, const void* h,
                  int64_t batch, float* out, void* ws, size_t ws_bytes,
                  void* stream, bool bf16 = false) {
  if (!out || !aligned(out, 16)) return DH_EINVAL;
  if (n_kept < 1 || n_kept > n_rows || vocab < n_kept || vocab > INT32_MAX)
    return DH_EINVAL;
  const int rc = check_head(fmt, w, scales, scale, dh_idx, n_rows, hidden, h,
                            batch, ws, ws_bytes);
  if (rc != DH_OK) return rc;
  GemvArgs a{};
  a.fmt = fmt;
  a.w = static_cast<const uint8_t*>(w);
  a.scales = scales;
  a.scale = scale;
  a.dh_idx = dh_idx;
  a.n_rows = n_rows;
  a.hidden = hidden;
  a.h = static_cast<const uint16_t*>(h);
  a.batch = batch;
  a.out_logits = out;
  a.n_kept = n_kept;
  a.vocab = vocab;
  a.ws = static_cast<uint8_t*>(ws);
  a.bf16_logits = bf16;
  return status(launch_gemv(a, static_cast<hipStream_t>(stream)));
}

static int check_quant(const void* w, int64_t vocab, int64_t hidden,
                       const int32_t* ids, int64_t n_rows, const void* out,
                       uintptr_t out_align, const float* scale,
                       const void* ws, size_t ws_bytes);

// NVFP4 quantization of a BF16 or FP16 head.
static int quantize_nvfp4(const void* w, bool f16, int64_t vocab,
                          int64_t hidden, const int32_t* row_ids,
                          int64_t n_rows, uint8_t* packed, uint8_t* scales,
                          float* global_scale, void* ws, size_t ws_bytes,
                          void* stream) {
  if (!scales) return DH_EINVAL;
  const int rc = check_quant(w, vocab, hidden, row_ids, n_rows, packed, 8,
                             global_scale, ws, ws_bytes);
  if (rc != DH_OK) return rc;
  QuantArgs a;
  a.w = static_cast<const uint16_t*>(w);
  a.vocab = vocab;
  a.hidden = hidden;
  a.ids = row_ids;
  a.n_rows = n_rows;
  a.packed = packed;
  a.scales = scales;
  a.global_scale = global_scale;
  a.ws = static_cast<uint8_t*>(ws);
  a.f16 = f16;
  return status(launch_nvfp4_quantize(a, static_cast<hipStream_t>(stream)));
}

// W8A8 workspace: the argmax state of any top-token call (the slots of the
// widest batch, so a workspace shared with other calls never overlaps
// them), then the tokens' activations (the BF16 values of their E4M3 codes,
// [batch][hidden]), their codes ([batch][hidden] bytes) and their scales,
// scratch that each call rewrites before reading.  total == 0 for an
// invalid shape.
struct W8a8Layout {
  size_t act, codes, sx, total;
};

static W8a8Layout w8a8_layout(int64_t n_rows, int64_t batch, int64_t hidden) {
  W8a8Layout l{};
  if (workspace_bytes(n_rows, batch) == 0 || hidden < 16 || hidden > 16384 ||
      hidden % 16 != 0)
    return l;
  const size_t state = workspace_bytes(n_rows, MAX_BATCH);
  l.act = (state + 255) / 256 * 256;
  l.codes = l.act + ((size_t)batch * (size_t)hidden * 2 + 255) / 256 * 256;
  l.sx = l.codes + ((size_t)batch * (size_t)hidden + 255) / 256 * 256;
  l.total = l.sx + ((size_t)batch * 4 + 255) / 256 * 256;
  return l;
}

// The FP8 head's step: per-token E4M3 quantization of h into the
// workspace (codes and their exact BF16 values), then the E4M3 GEMV: the
// batched slices multiply the codes with the head's bytes on the FP8 matrix
// cores, a batch-1 slice (a stream kernel) uses the BF16 values; either way
// each product is a product of two E4M3 values, as in an FP8 GEMM.  The
// logits carry each token's scale; the top token does not need it (a
// positive factor per batch row leaves the row's argmax unchanged).
static int w8a8(const uint8_t* q, const float* scale, const int32_t* dh_idx,
                int64_t n_rows, int64_t n_kept, int64_t hidden, int64_t vocab,
                const void* h, int64_t batch, int32_t* out_ids, float* out,
                void* ws, size_t ws_bytes, void* stream) {
  if (out_ids) {
    if (!aligned(out_ids, 4)) return DH_EINVAL;
  } else {
    if (!out || !aligned(out, 16)) return DH_EINVAL;
    if (n_kept < 1 || n_kept > n_rows || vocab < n_kept || vocab > INT32_MAX)
      return DH_EINVAL;
  }
  const int rc = check_head(FMT_E4M3, q, nullptr, scale, dh_idx, n_rows,
                            hidden, h, batch, ws, ws_bytes);
  if (rc != DH_OK) return rc;
  const W8a8Layout l = w8a8_layout(n_rows, batch, hidden);
  if (ws_bytes < l.total) return DH_EWORKSPACE;
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  uint16_t* hq = reinterpret_cast<uint16_t*>(wsb + l.act);
  uint8_t* qx = wsb + l.codes;
  float* sx = reinterpret_cast<float*>(wsb + l.sx);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = launch_fp8_tokens(static_cast<const uint16_t*>(h),
                                         batch, hidden, qx, hq, sx, s);
  if (e != hipSuccess) return DH_EHIP;
  GemvArgs a{};
  a.fmt = FMT_E4M3;
  a.w = q;
  a.scale = scale;
  a.dh_idx = dh_idx;
  a.n_rows = n_rows;
  a.hidden = hidden;
  a.h = hq;
  a.h_fp8 = qx;
  a.batch = batch;
  a.ws = wsb;
  if (out_ids) {
    a.out_ids = out_ids;
  } else {
    a.out_logits = out;
    a.n_kept = n_kept;
    a.vocab = vocab;
    a.row_scale = sx;
  }
  return status(launch_gemv(a, s));
}

// Checks shared by the quantizers.
static int check_quant(const void* w, int64_t vocab, int64_t hidden,
                       const int32_t* ids, int64_t n_rows, const void* out,
                       uintptr_t out_align, const float* scale,
                       const void* ws, size_t ws_bytes) {
  if (!w || !ids || !out || !scale) return DH_EINVAL;
  if (vocab < 1 || vocab > INT32_MAX || n_rows < 1 || n_rows > INT32_MAX)
    return DH_EINVAL;
  if (hidden < 16 || hidden > 16384 || hidden % 16 != 0) return DH_EINVAL;
  if (!aligned(w, 16) || !aligned(out, out_align) || !aligned(ids, 4) ||
      !aligned(scale, 4))
    return DH_EINVAL;
  if (!ws || !aligned(ws, 16) || ws_bytes < workspace_bytes(n_rows, 1))
    return DH_EWORKSPACE;
  return DH_OK;
}

}  // namespace dh

extern "C" {

int drafthead_abi_version(void) { return DRAFTHEAD_ABI_VERSION; }

const char* drafthead_error_string(int s) {
  switch (s) {
    case DH_OK: return "ok";
    case DH_EINVAL: return "invalid argument (null pointer, size or shape)";
    case DH_EWORKSPACE: return "workspace missing or too small";
    case DH_EHIP: return "HIP runtime or kernel launch error";
  }
  return "unknown status";
}

int64_t draft_head_build_index(const uint8_t* keep_mask, int64_t vocab,
                               int32_t* dh_idx, int64_t capacity,
                               int64_t* n_kept) {
  if (!keep_mask || !dh_idx || !n_kept || vocab < 1 || vocab > INT32_MAX)
    return DH_EINVAL;
  int64_t n = 0;
  for (int64_t v = 0; v < vocab; ++v) {
    if (!keep_mask[v]) continue;
    if (n >= capacity) return DH_EINVAL;
    dh_idx[n++] = (int32_t)v;
  }
  if (n == 0) return DH_EINVAL;
  const int64_t rows = (n + 63) / 64 * 64;
  if (rows > capacity) return DH_EINVAL;
  for (int64_t j = n; j < rows; ++j) dh_idx[j] = dh_idx[0];
  *n_kept = n;
  return rows;
}

size_t draft_head_workspace_bytes(int64_t n_rows, int64_t batch) {
  return dh::workspace_bytes(n_rows, batch);
}

int nvfp4_quantize_rows(const void* w_bf16, int64_t vocab, int64_t hidden,
                        const int32_t* row_ids, int64_t n_rows,
                        uint8_t* packed, uint8_t* scales, float* global_scale,
                        void* workspace, size_t workspace_bytes,
                        void* stream) {
  return dh::quantize_nvfp4(w_bf16, false, vocab, hidden, row_ids, n_rows,
                            packed, scales, global_scale, workspace,
                            workspace_bytes, stream);
}

int nvfp4_quantize_rows_f16(const void* w_f16, int64_t vocab, int64_t hidden,
                            const int32_t* row_ids, int64_t n_rows,
                            uint8_t* packed, uint8_t* scales,
                            float* global_scale, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return dh::quantize_nvfp4(w_f16, true, vocab, hidden, row_ids, n_rows,
                            packed, scales, global_scale, workspace,
                            workspace_bytes, stream);
}

int e4m3_quantize_rows_per_tensor(const void* w_bf16, int64_t vocab,
                                  int64_t hidden, const int32_t* row_ids,
                                  int64_t n_rows, uint8_t* q, float* scale,
                                  void* workspace, size_t workspace_bytes,
                                  void* stream) {
  const int rc = dh::check_quant(w_bf16, vocab, hidden, row_ids, n_rows, q, 8,
                                 scale, workspace, workspace_bytes);
  if (rc != DH_OK) return rc;
  dh::QuantE4m3Args a;
  a.w = static_cast<const uint16_t*>(w_bf16);
  a.vocab = vocab;
  a.hidden = hidden;
  a.ids = row_ids;
  a.n_rows = n_rows;
  a.q = q;
  a.scale = scale;
  a.ws = static_cast<uint8_t*>(workspace);
  return dh::status(
      dh::launch_e4m3_quantize(a, static_cast<hipStream_t>(stream)));
}

int draft_head_top_tokens(const uint8_t* packed, const uint8_t* scales,
                          const float* global_scale, const int32_t* dh_idx,
                          int64_t n_rows, int64_t hidden, const void* h_bf16,
                          int64_t batch, int32_t* out_ids, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return dh::top_tokens(dh::FMT_NVFP4, packed, scales, global_scale, dh_idx,
                        n_rows, hidden, h_bf16, batch, out_ids, workspace,
                        workspace_bytes, stream);
}

int draft_head_top_tokens_noalloc(const uint8_t* packed,
                                  const uint8_t* scales,
                                  const float* global_scale,
                                  const int32_t* dh_idx, int64_t n_rows,
                                  int64_t hidden, const void* h_bf16,
                                  int64_t batch, int32_t* out_ids,
                                  void* stream) {
  // every argument error is reported before the first HIP call: the checks
  // run against an aligned stand-in for the scratch's address
  const size_t need = dh::workspace_bytes(n_rows, batch);
  if (need > dh::NOALLOC_SCRATCH_BYTES) return DH_EWORKSPACE;
  if (!out_ids || !dh::aligned(out_ids, 4)) return DH_EINVAL;
  int rc = dh::check_head(dh::FMT_NVFP4, packed, scales, global_scale, dh_idx,
                          n_rows, hidden, h_bf16, batch,
                          reinterpret_cast<void*>(uintptr_t{256}),
                          dh::NOALLOC_SCRATCH_BYTES);
  if (rc != DH_OK) return rc;
  void* ws = nullptr;
  if (dh::scratch_address(&ws) != hipSuccess) return DH_EHIP;
  return dh::top_tokens(dh::FMT_NVFP4, packed, scales, global_scale, dh_idx,
                        n_rows, hidden, h_bf16, batch, out_ids, ws,
                        dh::NOALLOC_SCRATCH_BYTES, stream);
}

int draft_head_logits(const uint8_t* packed, const uint8_t* scales,
                      const float* global_scale, const int32_t* dh_idx,
                      int64_t n_rows, int64_t n_kept, int64_t hidden,
                      int64_t vocab, const void* h_bf16, int64_t batch,
                      float* out_logits, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return dh::logits(dh::FMT_NVFP4, packed, scales, global_scale, dh_idx,
                    n_rows, n_kept, hidden, vocab, h_bf16, batch, out_logits,
                    workspace, workspace_bytes, stream);
}

int draft_head_top_tokens_compat(const uint8_t* packed,
                                 const uint8_t* scales,
                                 const float* global_scale,
                                 const int32_t* dh_idx, int64_t n_rows,
                                 int64_t hidden, const void* h_bf16,
                                 int64_t batch, int32_t* out_ids,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return dh::top_tokens(dh::FMT_NVFP4, packed, scales, global_scale, dh_idx,
                        n_rows, hidden, h_bf16, batch, out_ids, workspace,
                        workspace_bytes, stream, true);
}

int draft_head_logits_compat(const uint8_t* packed, const uint8_t* scales,
                             const float* global_scale,
                             const int32_t* dh_idx, int64_t n_rows,
                             int64_t n_kept, int64_t hidden, int64_t vocab,
                             const void* h_bf16, int64_t batch,
                             void* out_logits_bf16, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return dh::logits(dh::FMT_NVFP4, packed, scales, global_scale, dh_idx,
                    n_rows, n_kept, hidden, vocab, h_bf16, batch,
                    static_cast<float*>(out_logits_bf16), workspace,
                    workspace_bytes, stream, true);
}

int nvfp4_linear(const uint8_t* packed, const uint8_t* scales,
                 const float* global_scale, int64_t n_rows, int64_t hidden,
                 const void* h_bf16, int64_t batch, float* out,
                 void* stream) {
  using namespace dh;
  if (!packed || !scales || !global_scale || !h_bf16 || !out)
    return DH_EINVAL;
  if (!aligned(packed, 16) || !aligned(scales, 16) ||
      !aligned(global_scale, 4) || !aligned(h_bf16, 16) || !aligned(out, 16))
    return DH_EINVAL;
  if (hidden < 16 || hidden > 16384 || hidden % 16 != 0) return DH_EINVAL;
  if (n_rows < 64 || n_rows % 64 != 0 || n_rows > INT32_MAX) return DH_EINVAL;
  if (batch < 1 || batch > MAX_BATCH) return DH_EINVAL;
  GemvArgs a{};
  a.fmt = FMT_NVFP4;
  a.w = packed;
  a.scales = scales;
  a.scale = global_scale;
  a.n_rows = n_rows;
  a.hidden = hidden;
  a.h = static_cast<const uint16_t*>(h_bf16);
  a.batch = batch;
  a.out_logits = out;
  a.dense = true;
  return status(launch_gemv(a, static_cast<hipStream_t>(stream)));
}

int draft_head_top_tokens_e4m3(const uint8_t* q, const float* scale,
                               const int32_t* dh_idx, int64_t n_rows,
                               int64_t hidden, const void* h_bf16,
                               int64_t batch, int32_t* out_ids,
                               void* workspace, size_t workspace_bytes,
                               void* stream) {
  return dh::top_tokens(dh::FMT_E4M3, q, nullptr, scale, dh_idx, n_rows,
                        hidden, h_bf16, batch, out_ids, workspace,
                        workspace_bytes, stream);
}

int draft_head_logits_e4m3(const uint8_t* q, const float* scale,
                           const int32_t* dh_idx, int64_t n_rows,
                           int64_t n_kept, int64_t hidden, int64_t vocab,
                           const void* h_bf16, int64_t batch,
                           float* out_logits, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return dh::logits(dh::FMT_E4M3, q, nullptr, scale, dh_idx, n_rows, n_kept,
                    hidden, vocab, h_bf16, batch, out_logits, workspace,
                    workspace_bytes, stream);
}

size_t draft_head_workspace_bytes_w8a8(int64_t n_rows, int64_t batch,
                                       int64_t hidden) {
  return dh::w8a8_layout(n_rows, batch, hidden).total;
}

int fp8_quantize_tokens(const void* h_bf16, int64_t batch, int64_t hidden,
                        uint8_t* qx, float* sx, void* stream) {
  using namespace dh;
  if (!h_bf16 || !qx || !sx) return DH_EINVAL;
  if (!aligned(h_bf16, 16) || !aligned(qx, 8) || !aligned(sx, 4))
    return DH_EINVAL;
  if (hidden < 16 || hidden > 16384 || hidden % 16 != 0) return DH_EINVAL;
  if (batch < 1 || batch > MAX_TOKENS) return DH_EINVAL;
  return status(launch_fp8_tokens(static_cast<const uint16_t*>(h_bf16), batch,
                                  hidden, qx, nullptr, sx,
                                  static_cast<hipStream_t>(stream)));
}

int draft_head_top_tokens_w8a8(const uint8_t* q, const float* scale,
                               const int32_t* dh_idx, int64_t n_rows,
                               int64_t hidden, const void* h_bf16,
                               int64_t batch, int32_t* out_ids,
                               void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (!out_ids) return DH_EINVAL;
  return dh::w8a8(q, scale, dh_idx, n_rows, 0, hidden, 0, h_bf16, batch,
                  out_ids, nullptr, workspace, workspace_bytes, stream);
}

int draft_head_logits_w8a8(const uint8_t* q, const float* scale,
                           const int32_t* dh_idx, int64_t n_rows,
                           int64_t n_kept, int64_t hidden, int64_t vocab,
                           const void* h_bf16, int64_t batch,
                           float* out_logits, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return dh::w8a8(q, scale, dh_idx, n_rows, n_kept, hidden, vocab, h_bf16,
                  batch, nullptr, out_logits, workspace, workspace_bytes,
                  stream);
}

int draft_head_top_tokens_bf16(const void* w_bf16, const int32_t* dh_idx,
                               int64_t n_rows, int64_t hidden,
                               const void* h_bf16, int64_t batch,
                               int32_t* out_ids, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return dh::top_tokens(dh::FMT_BF16, w_bf16, nullptr, nullptr, dh_idx,
                        n_rows, hidden, h_bf16, batch, out_ids, workspace,
                        workspace_bytes, stream);
}

int draft_head_logits_bf16(const void* w_bf16, const int32_t* dh_idx,
                           int64_t n_rows, int64_t n_kept, int64_t hidden,
                           int64_t vocab, const void* h_bf16, int64_t batch,
                           float* out_logits, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return dh::logits(dh::FMT_BF16, w_bf16, nullptr, nullptr, dh_idx, n_rows,
                    n_kept, hidden, vocab, h_bf16, batch, out_logits,
                    workspace, workspace_bytes, stream);
}

static constexpr size_t kMaxProbeBytes = (size_t)1 << 48;

int drafthead_read_probe(const void* a, size_t a_bytes, const void* b,
                         size_t b_bytes, uint32_t* sink, void* stream) {
  if (!a || !sink || !dh::aligned(a, 16) || !dh::aligned(sink, 4))
    return DH_EINVAL;
  if (a_bytes % 16 != 0 || b_bytes % 16 != 0 || a_bytes + b_bytes == 0)
    return DH_EINVAL;
  // no buffer is that large; this also keeps the sum from wrapping
  if (a_bytes > kMaxProbeBytes || b_bytes > kMaxProbeBytes) return DH_EINVAL;
  if (b_bytes != 0 && (!b || !dh::aligned(b, 16))) return DH_EINVAL;
  return dh::status(dh::launch_read_probe(a, a_bytes, b, b_bytes, sink,
                                          static_cast<hipStream_t>(stream)));
}

}  // extern "C"
