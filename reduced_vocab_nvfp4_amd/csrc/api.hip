// extern "C" entry points of the draft-head library: argument checks on the
// host (before any HIP call, so every error path runs without a device),
// then the kernel launchers.  Semantics and citations are documented at the
// declarations in include/drafthead.h.
#include "drafthead.h"

#include "dh_internal.h"

namespace dh {

static bool aligned(const void* p, uintptr_t n) {
  return (reinterpret_cast<uintptr_t>(p) % n) == 0;
}

size_t workspace_bytes(int64_t n_rows, int64_t batch) {
  if (n_rows < 1 || batch < 1 || batch > MAX_BATCH) return 0;
  const int64_t slice = batch < 8 ? batch : 8;
  return WS_PARTIALS + (size_t)MAX_GRID * (size_t)slice * sizeof(uint64_t);
}

hipError_t device_info(DeviceInfo* out) {
  static DeviceInfo cache[64];
  static bool have[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64 && have[dev]) {
    *out = cache[dev];
    return hipSuccess;
  }
  DeviceInfo d{};
  e = hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&d.lds_per_block,
                            hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess) return e;
  if (d.cus < 1) d.cus = 1;
  if (dev >= 0 && dev < 64) {
    cache[dev] = d;
    have[dev] = true;
  }
  *out = d;
  return hipSuccess;
}

static int status(hipError_t e) { return e == hipSuccess ? DH_OK : DH_EHIP; }

// Shape and pointer checks shared by the GEMV entry points.
static int check_head(const uint8_t* packed, const uint8_t* scales,
                      const float* gs, const int32_t* dh_idx, int64_t n_rows,
                      int64_t hidden, const void* h, int64_t batch,
                      const void* ws, size_t ws_bytes) {
  if (!packed || !scales || !gs || !dh_idx || !h) return DH_EINVAL;
  if (hidden < 16 || hidden > 16384 || hidden % 16 != 0) return DH_EINVAL;
  if (n_rows < 64 || n_rows % 64 != 0 || n_rows > INT32_MAX) return DH_EINVAL;
  if (batch < 1 || batch > MAX_BATCH) return DH_EINVAL;
  if (!aligned(packed, 16) || !aligned(scales, 16) || !aligned(h, 16) ||
      !aligned(gs, 4) || !aligned(dh_idx, 4))
    return DH_EINVAL;
  if (!ws || !aligned(ws, 16) || ws_bytes < workspace_bytes(n_rows, batch))
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
  if (!w_bf16 || !row_ids || !packed || !scales || !global_scale)
    return DH_EINVAL;
  if (vocab < 1 || vocab > INT32_MAX || n_rows < 1 || n_rows > INT32_MAX)
    return DH_EINVAL;
  if (hidden < 16 || hidden > 16384 || hidden % 16 != 0) return DH_EINVAL;
  if (!dh::aligned(w_bf16, 16) || !dh::aligned(packed, 8) ||
      !dh::aligned(row_ids, 4) || !dh::aligned(global_scale, 4))
    return DH_EINVAL;
  if (!workspace || !dh::aligned(workspace, 16) ||
      workspace_bytes < dh::workspace_bytes(n_rows, 1))
    return DH_EWORKSPACE;
  dh::QuantArgs a;
  a.w = static_cast<const uint16_t*>(w_bf16);
  a.vocab = vocab;
  a.hidden = hidden;
  a.ids = row_ids;
  a.n_rows = n_rows;
  a.packed = packed;
  a.scales = scales;
  a.global_scale = global_scale;
  a.ws = static_cast<uint8_t*>(workspace);
  return dh::status(
      dh::launch_nvfp4_quantize(a, static_cast<hipStream_t>(stream)));
}

int draft_head_top_tokens(const uint8_t* packed, const uint8_t* scales,
                          const float* global_scale, const int32_t* dh_idx,
                          int64_t n_rows, int64_t hidden, const void* h_bf16,
                          int64_t batch, int32_t* out_ids, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!out_ids || !dh::aligned(out_ids, 4)) return DH_EINVAL;
  int rc = dh::check_head(packed, scales, global_scale, dh_idx, n_rows, hidden,
                          h_bf16, batch, workspace, workspace_bytes);
  if (rc != DH_OK) return rc;
  dh::GemvArgs a{};
  a.packed = packed;
  a.scales = scales;
  a.global_scale = global_scale;
  a.dh_idx = dh_idx;
  a.n_rows = n_rows;
  a.hidden = hidden;
  a.h = static_cast<const uint16_t*>(h_bf16);
  a.batch = batch;
  a.out_ids = out_ids;
  a.ws = static_cast<uint8_t*>(workspace);
  return dh::status(
      dh::launch_nvfp4_top_tokens(a, static_cast<hipStream_t>(stream)));
}

int draft_head_logits(const uint8_t* packed, const uint8_t* scales,
                      const float* global_scale, const int32_t* dh_idx,
                      int64_t n_rows, int64_t n_kept, int64_t hidden,
                      int64_t vocab, const void* h_bf16, int64_t batch,
                      float* out_logits, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (!out_logits || !dh::aligned(out_logits, 16)) return DH_EINVAL;
  if (n_kept < 1 || n_kept > n_rows || vocab < n_kept || vocab > INT32_MAX)
    return DH_EINVAL;
  int rc = dh::check_head(packed, scales, global_scale, dh_idx, n_rows, hidden,
                          h_bf16, batch, workspace, workspace_bytes);
  if (rc != DH_OK) return rc;
  dh::GemvArgs a{};
  a.packed = packed;
  a.scales = scales;
  a.global_scale = global_scale;
  a.dh_idx = dh_idx;
  a.n_rows = n_rows;
  a.hidden = hidden;
  a.h = static_cast<const uint16_t*>(h_bf16);
  a.batch = batch;
  a.out_logits = out_logits;
  a.n_kept = n_kept;
  a.vocab = vocab;
  a.ws = static_cast<uint8_t*>(workspace);
  return dh::status(
      dh::launch_nvfp4_logits(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
