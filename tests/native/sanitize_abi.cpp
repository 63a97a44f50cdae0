// Drives the host side of the C-ABI (csrc/api.hip, compiled for the host
// only) under -fsanitize=address,undefined: argument validation, the row
// index, the workspace sizes and the argument marshalling up to the kernel
// launchers.  The launchers and the two HIP queries the layer makes are
// stubs here that record the call and return success, so no device is
// touched.  Every entry point is called with invalid arguments (each must be
// refused before any launch) and with valid ones (each must reach its
// launcher).  Exits 0 when every call returned what it should.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "dh_internal.h"
#include "drafthead.h"

static int launches = 0;
static int failures = 0;

namespace dh {
hipError_t launch_gemv(const GemvArgs& a, hipStream_t) {
  if (a.n_rows < 1 || a.batch < 1 || a.hidden < 16) return hipErrorInvalidValue;
  ++launches;
  return hipSuccess;
}
hipError_t launch_nvfp4_quantize(const QuantArgs& a, hipStream_t) {
  if (a.n_rows < 1) return hipErrorInvalidValue;
  ++launches;
  return hipSuccess;
}
hipError_t launch_e4m3_quantize(const QuantE4m3Args& a, hipStream_t) {
  if (a.n_rows < 1) return hipErrorInvalidValue;
  ++launches;
  return hipSuccess;
}
hipError_t launch_fp8_tokens(const uint16_t*, int64_t batch, int64_t hidden,
                             uint8_t*, uint16_t*, float*, hipStream_t) {
  if (batch < 1 || hidden < 16) return hipErrorInvalidValue;
  ++launches;
  return hipSuccess;
}
hipError_t launch_read_probe(const void*, size_t a_bytes, const void*,
                             size_t b_bytes, uint32_t*, hipStream_t) {
  if (a_bytes % 16 != 0 || b_bytes % 16 != 0 || a_bytes + b_bytes == 0)
    return hipErrorInvalidValue;
  ++launches;
  return hipSuccess;
}
}  // namespace dh

extern "C" hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
// api.hip holds one static device array (the scratch of the no-allocation
// entry point): its registration at load and the address query are stubbed
// too; the address is a fake aligned pointer, never dereferenced.
static int symbol_queries = 0;
extern "C" void** __hipRegisterFatBinary(const void*) {
  static void* handle = nullptr;
  return &handle;
}
extern "C" void __hipUnregisterFatBinary(void**) {}
extern "C" void __hipRegisterVar(void**, void*, char*, char*, int, size_t,
                                 int, int) {}
extern "C" hipError_t hipGetSymbolAddress(void** p, const void*) {
  *p = reinterpret_cast<void*>(uintptr_t(3) << 40);
  ++symbol_queries;
  return hipSuccess;
}
extern "C" hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t,
                                            int) {
  *v = 256;
  return hipSuccess;
}

static void expect(bool ok, const char* what, int line) {
  if (!ok) {
    printf("FAILED line %d: %s\n", line, what);
    ++failures;
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

// Refused before any launch.
#define REFUSED(call, code)              \
  do {                                   \
    const int before = launches;         \
    const int rc = (call);               \
    EXPECT(rc == (code));                \
    EXPECT(launches == before);          \
  } while (0)
// Reaches its launcher (a W8A8 step launches twice).
#define LAUNCHED(call, n)                \
  do {                                   \
    const int before = launches;         \
    const int rc = (call);               \
    EXPECT(rc == DH_OK);                 \
    EXPECT(launches == before + (n));    \
  } while (0)

int main() {
  // fake device pointers: never dereferenced on the host
  void* P = reinterpret_cast<void*>(uintptr_t(1) << 40);
  uint8_t* P8 = static_cast<uint8_t*>(P);
  float* PF = static_cast<float*>(P);
  int32_t* PI = static_cast<int32_t*>(P);
  void* MIS = reinterpret_cast<void*>((uintptr_t(1) << 40) + 2);
  const int64_t N = 64064, H = 2560, V = 248320;
  const size_t ws1 = draft_head_workspace_bytes(N, 1);
  const size_t ws16 = draft_head_workspace_bytes(N, 16);
  EXPECT(ws1 > 0 && ws16 >= ws1);

  // workspace sizes at and past the limits
  EXPECT(draft_head_workspace_bytes(0, 1) == 0);
  EXPECT(draft_head_workspace_bytes(64, 0) == 0);
  EXPECT(draft_head_workspace_bytes(64, 65) == 0);
  EXPECT(draft_head_workspace_bytes(INT64_MAX, 64) > 0);
  EXPECT(draft_head_workspace_bytes(INT64_MIN, 1) == 0);
  EXPECT(draft_head_workspace_bytes_w8a8(N, 16, H) > ws16);
  EXPECT(draft_head_workspace_bytes_w8a8(N, 16, 8) == 0);
  EXPECT(draft_head_workspace_bytes_w8a8(N, 16, INT64_MAX) == 0);
  EXPECT(draft_head_workspace_bytes_w8a8(INT64_MAX, 64, 16384) > 0);
  for (int s = -5; s <= 1; ++s) EXPECT(drafthead_error_string(s) != nullptr);
  EXPECT(drafthead_abi_version() == DRAFTHEAD_ABI_VERSION);

  // row index: masks with and without kept ids, too small a capacity
  {
    std::vector<uint8_t> keep(4097);
    std::vector<int32_t> idx(4097 + 64);
    int64_t nk = -1;
    REFUSED((int)draft_head_build_index(keep.data(), 4097, idx.data(),
                                        (int64_t)idx.size(), &nk),
            DH_EINVAL);
    keep[4096] = 1;
    EXPECT(draft_head_build_index(keep.data(), 4097, idx.data(),
                                  (int64_t)idx.size(), &nk) == 64);
    EXPECT(nk == 1 && idx[0] == 4096 && idx[63] == 4096);
    for (size_t v = 0; v < keep.size(); ++v) keep[v] = (v * 7919) % 3 == 0;
    const int64_t n = draft_head_build_index(
        keep.data(), 4097, idx.data(), (int64_t)idx.size(), &nk);
    EXPECT(n > 0 && n % 64 == 0 && nk <= n);
    REFUSED((int)draft_head_build_index(keep.data(), 4097, idx.data(), 10,
                                        &nk),
            DH_EINVAL);
    REFUSED((int)draft_head_build_index(keep.data(), 4097, idx.data(), nk,
                                        &nk),
            nk % 64 ? DH_EINVAL : (int)nk);
    REFUSED((int)draft_head_build_index(nullptr, 4097, idx.data(), 99, &nk),
            DH_EINVAL);
    REFUSED((int)draft_head_build_index(keep.data(), 0, idx.data(), 99, &nk),
            DH_EINVAL);
    REFUSED((int)draft_head_build_index(keep.data(), INT64_MAX, idx.data(),
                                        99, &nk),
            DH_EINVAL);
  }

  // quantizers
  LAUNCHED(nvfp4_quantize_rows(P, V, H, PI, N, P8, P8, PF, P, ws1, nullptr), 1);
  LAUNCHED(nvfp4_quantize_rows_f16(P, V, H, PI, N, P8, P8, PF, P, ws1, nullptr),
           1);
  REFUSED(nvfp4_quantize_rows(P, V, H, PI, N, P8, nullptr, PF, P, ws1, nullptr),
          DH_EINVAL);
  REFUSED(nvfp4_quantize_rows(P, V, 24, PI, N, P8, P8, PF, P, ws1, nullptr),
          DH_EINVAL);
  REFUSED(nvfp4_quantize_rows(P, V, 32768, PI, N, P8, P8, PF, P, ws1, nullptr),
          DH_EINVAL);
  REFUSED(nvfp4_quantize_rows(MIS, V, H, PI, N, P8, P8, PF, P, ws1, nullptr),
          DH_EINVAL);
  REFUSED(nvfp4_quantize_rows(P, 0, H, PI, N, P8, P8, PF, P, ws1, nullptr),
          DH_EINVAL);
  REFUSED(nvfp4_quantize_rows(P, V, H, PI, 0, P8, P8, PF, P, ws1, nullptr),
          DH_EINVAL);
  REFUSED(nvfp4_quantize_rows(P, V, H, PI, INT64_MAX, P8, P8, PF, P, ws1,
                              nullptr),
          DH_EINVAL);
  REFUSED(nvfp4_quantize_rows(P, V, H, PI, N, P8, P8, PF, P, 8, nullptr),
          DH_EWORKSPACE);
  REFUSED(nvfp4_quantize_rows(P, V, H, PI, N, P8, P8, PF, nullptr, ws1,
                              nullptr),
          DH_EWORKSPACE);
  LAUNCHED(e4m3_quantize_rows_per_tensor(P, V, H, PI, N, P8, PF, P, ws1,
                                         nullptr),
           1);
  REFUSED(e4m3_quantize_rows_per_tensor(P, V, H, PI, N, P8, nullptr, P, ws1,
                                        nullptr),
          DH_EINVAL);

  // top tokens and logits, every format
  LAUNCHED(draft_head_top_tokens(P8, P8, PF, PI, N, H, P, 1, PI, P, ws1,
                                 nullptr),
           1);
  LAUNCHED(draft_head_top_tokens(P8, P8, PF, PI, N, H, P, 16, PI, P, ws16,
                                 nullptr),
           1);
  // the scratch address is queried once per device, then kept
  LAUNCHED(draft_head_top_tokens_noalloc(P8, P8, PF, PI, N, H, P, 1, PI,
                                         nullptr),
           1);
  LAUNCHED(draft_head_top_tokens_noalloc(P8, P8, PF, PI, N, H, P, 64, PI,
                                         nullptr),
           1);
  EXPECT(symbol_queries == 1);
  REFUSED(draft_head_top_tokens_noalloc(nullptr, P8, PF, PI, N, H, P, 1, PI,
                                        nullptr),
          DH_EINVAL);
  REFUSED(draft_head_top_tokens_noalloc(P8, P8, PF, PI, N, H, P, 65, PI,
                                        nullptr),
          DH_EINVAL);
  REFUSED(draft_head_top_tokens_noalloc(P8, P8, PF, PI, N, H, P, 1,
                                        reinterpret_cast<int32_t*>(MIS),
                                        nullptr),
          DH_EINVAL);
  LAUNCHED(draft_head_top_tokens_compat(P8, P8, PF, PI, N, H, P, 3, PI, P,
                                        ws16, nullptr),
           1);
  LAUNCHED(draft_head_logits(P8, P8, PF, PI, N, 64026, H, V, P, 8, PF, P,
                             ws16, nullptr),
           1);
  LAUNCHED(draft_head_logits_compat(P8, P8, PF, PI, N, 64026, H, V, P, 8, P,
                                    P, ws16, nullptr),
           1);
  LAUNCHED(draft_head_top_tokens_e4m3(P8, PF, PI, N, H, P, 4, PI, P, ws16,
                                      nullptr),
           1);
  LAUNCHED(draft_head_logits_e4m3(P8, PF, PI, N, 64026, H, V, P, 2, PF, P,
                                  ws16, nullptr),
           1);
  LAUNCHED(draft_head_top_tokens_bf16(P, PI, N, H, P, 1, PI, P, ws1, nullptr),
           1);
  LAUNCHED(draft_head_logits_bf16(P, PI, N, N, H, V, P, 1, PF, P, ws1,
                                  nullptr),
           1);
  LAUNCHED(nvfp4_linear(P8, P8, PF, 5120, H, P, 16, PF, nullptr), 1);
  const size_t w8 = draft_head_workspace_bytes_w8a8(N, 16, H);
  LAUNCHED(draft_head_top_tokens_w8a8(P8, PF, PI, N, H, P, 16, PI, P, w8,
                                      nullptr),
           2);
  LAUNCHED(draft_head_logits_w8a8(P8, PF, PI, N, 64026, H, V, P, 16, PF, P,
                                  w8, nullptr),
           2);
  LAUNCHED(fp8_quantize_tokens(P, 16, H, P8, PF, nullptr), 1);
  uint32_t* PU = static_cast<uint32_t*>(P);
  LAUNCHED(drafthead_read_probe(P, 1 << 20, P, 160 << 10, PU, nullptr), 1);
  LAUNCHED(drafthead_read_probe(P, 1 << 20, nullptr, 0, PU, nullptr), 1);

  // refused shapes and pointers
  REFUSED(draft_head_top_tokens(nullptr, P8, PF, PI, N, H, P, 1, PI, P, ws1,
                                nullptr),
          DH_EINVAL);
  REFUSED(draft_head_top_tokens(P8, nullptr, PF, PI, N, H, P, 1, PI, P, ws1,
                                nullptr),
          DH_EINVAL);
  REFUSED(draft_head_top_tokens(P8, P8, nullptr, PI, N, H, P, 1, PI, P, ws1,
                                nullptr),
          DH_EINVAL);
  REFUSED(draft_head_top_tokens(P8, P8, PF, PI, N + 1, H, P, 1, PI, P, ws1,
                                nullptr),
          DH_EINVAL);
  REFUSED(draft_head_top_tokens(P8, P8, PF, PI, 0, H, P, 1, PI, P, ws1,
                                nullptr),
          DH_EINVAL);
  REFUSED(draft_head_top_tokens(P8, P8, PF, PI, INT64_MAX - 63, H, P, 1, PI,
                                P, ws1, nullptr),
          DH_EINVAL);
  REFUSED(draft_head_top_tokens(P8, P8, PF, PI, N, 8, P, 1, PI, P, ws1,
                                nullptr),
          DH_EINVAL);
  REFUSED(draft_head_top_tokens(P8, P8, PF, PI, N, H, P, 0, PI, P, ws1,
                                nullptr),
          DH_EINVAL);
  REFUSED(draft_head_top_tokens(P8, P8, PF, PI, N, H, P, 65, PI, P, ws1,
                                nullptr),
          DH_EINVAL);
  REFUSED(draft_head_top_tokens(P8, P8, PF, PI, N, H, MIS, 1, PI, P, ws1,
                                nullptr),
          DH_EINVAL);
  REFUSED(draft_head_top_tokens(P8, P8, PF, PI, N, H, P, 1, PI, P, ws1 - 1,
                                nullptr),
          DH_EWORKSPACE);
  REFUSED(draft_head_top_tokens(P8, P8, PF, PI, N, H, P, 16, PI, P, ws1,
                                nullptr),
          DH_EWORKSPACE);
  REFUSED(draft_head_logits(P8, P8, PF, PI, N, 0, H, V, P, 1, PF, P, ws1,
                            nullptr),
          DH_EINVAL);
  REFUSED(draft_head_logits(P8, P8, PF, PI, N, N + 1, H, V, P, 1, PF, P, ws1,
                            nullptr),
          DH_EINVAL);
  REFUSED(draft_head_logits(P8, P8, PF, PI, N, 64026, H, 100, P, 1, PF, P,
                            ws1, nullptr),
          DH_EINVAL);
  REFUSED(draft_head_logits(P8, P8, PF, PI, N, 64026, H, INT64_MAX, P, 1, PF,
                            P, ws1, nullptr),
          DH_EINVAL);
  REFUSED(draft_head_logits(P8, P8, PF, PI, N, 64026, H, V, P, 1,
                            static_cast<float*>(MIS), P, ws1, nullptr),
          DH_EINVAL);
  REFUSED(nvfp4_linear(P8, P8, PF, 5120, H, P, 0, PF, nullptr), DH_EINVAL);
  REFUSED(nvfp4_linear(P8, P8, PF, 5100, H, P, 1, PF, nullptr), DH_EINVAL);
  REFUSED(draft_head_top_tokens_w8a8(P8, PF, PI, N, H, P, 16, PI, P, ws16,
                                     nullptr),
          DH_EWORKSPACE);
  REFUSED(draft_head_top_tokens_w8a8(P8, PF, PI, N, H, P, 16, nullptr, P, w8,
                                     nullptr),
          DH_EINVAL);
  REFUSED(fp8_quantize_tokens(P, 0, H, P8, PF, nullptr), DH_EINVAL);
  REFUSED(fp8_quantize_tokens(P, (1 << 16) + 1, H, P8, PF, nullptr),
          DH_EINVAL);
  REFUSED(fp8_quantize_tokens(P, 4, 40, P8, PF, nullptr), DH_EINVAL);
  REFUSED(drafthead_read_probe(nullptr, 16, nullptr, 0, PU, nullptr),
          DH_EINVAL);
  REFUSED(drafthead_read_probe(MIS, 16, nullptr, 0, PU, nullptr), DH_EINVAL);
  REFUSED(drafthead_read_probe(P, 24, nullptr, 0, PU, nullptr), DH_EINVAL);
  REFUSED(drafthead_read_probe(P, 16, nullptr, 16, PU, nullptr), DH_EINVAL);
  REFUSED(drafthead_read_probe(P, 16, MIS, 16, PU, nullptr), DH_EINVAL);
  REFUSED(drafthead_read_probe(P, 0, nullptr, 0, PU, nullptr), DH_EINVAL);
  REFUSED(drafthead_read_probe(P, 16, nullptr, 0, nullptr, nullptr),
          DH_EINVAL);
  REFUSED(drafthead_read_probe(P, 16, nullptr, 0,
                               reinterpret_cast<uint32_t*>(P8 + 2), nullptr),
          DH_EINVAL);
  // sizes whose sum wraps around
  REFUSED(drafthead_read_probe(P, SIZE_MAX - 15, P, 32, PU, nullptr),
          DH_EINVAL);

  printf("C-ABI host sanitizer run: %d launches, %d failures\n", launches,
         failures);
  return failures ? 1 : 0;
}
