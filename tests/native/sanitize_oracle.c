/* Drives every entry point of oracle/oracle.c on small inputs, including
 * the edge cases the tests use (empty and one-id masks, pad rows, all-zero
 * and wide-range heads, invalid shapes), so that a build with
 * -fsanitize=address,undefined reports any out-of-bounds access, overflow
 * or other undefined behaviour in the oracle.  The values are checked by
 * the Python pins; this program only checks return codes.  Exits 0 when
 * every call returned what it should. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float oracle_f16_value(uint16_t bits);
uint16_t oracle_bf16_code(float x);
double oracle_e4m3_value(uint8_t code);
uint8_t oracle_e4m3_code(float s);
double oracle_e2m1_value(uint8_t nib);
uint8_t oracle_e2m1_code(float q);
int64_t oracle_build_index(const uint8_t* keep, int64_t vocab, int32_t* idx,
                           int64_t capacity, int64_t* n_kept);
int oracle_nvfp4_quantize(const uint16_t* w, int64_t vocab, int64_t hidden,
                          const int32_t* idx, int64_t n_rows, uint8_t* packed,
                          uint8_t* scales, float* gs_out);
int oracle_nvfp4_quantize_f16(const uint16_t* w, int64_t vocab,
                              int64_t hidden, const int32_t* idx,
                              int64_t n_rows, uint8_t* packed,
                              uint8_t* scales, float* gs_out);
int oracle_nvfp4_logits(const uint8_t* packed, const uint8_t* scales,
                        float gs, int64_t n_rows, int64_t hidden,
                        const uint16_t* h, int64_t batch, double* L);
int oracle_argmax_remap(const double* L, int64_t batch, int64_t n_rows,
                        const int32_t* idx, int64_t* rows, int32_t* ids);
int oracle_logits_scatter(const double* L, int64_t batch, int64_t n_rows,
                          int64_t n_kept, const int32_t* idx, int64_t vocab,
                          float* out);
int oracle_logits_to_bf16(const double* L, int64_t n, uint16_t* out);
int oracle_logits_scatter_bf16(const uint16_t* Lb, int64_t batch,
                               int64_t n_rows, int64_t n_kept,
                               const int32_t* idx, int64_t vocab,
                               uint16_t* out);
int oracle_bf16_logits(const uint16_t* w, int64_t vocab, int64_t hidden,
                       const int32_t* idx, int64_t n_rows, const uint16_t* h,
                       int64_t batch, double* L);
int oracle_e4m3_tensor_quantize(const uint16_t* w, int64_t vocab,
                                int64_t hidden, const int32_t* idx,
                                int64_t n_rows, uint8_t* q, float* scale);
int oracle_e4m3_tensor_logits(const uint8_t* q, float scale, int64_t n_rows,
                              int64_t hidden, const uint16_t* h,
                              int64_t batch, double* L);
int oracle_fp8_tokens_quantize(const uint16_t* h, int64_t batch,
                               int64_t hidden, uint8_t* qx, float* sx);
int oracle_w8a8_logits(const uint8_t* q, float sw, int64_t n_rows,
                       int64_t hidden, const uint8_t* qx, const float* sx,
                       int64_t batch, double* L);
int oracle_num_threads(void);
void oracle_set_threads(int n);

static int failures = 0;

static void expect(int ok, const char* what) {
  if (!ok) {
    printf("FAILED: %s\n", what);
    ++failures;
  }
}

static uint64_t rng_state = 0x243F6A8885A308D3ull;
static uint32_t next_u32(void) {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return (uint32_t)(rng_state >> 16);
}

/* bf16 bits of a value with a random sign, exponent in [lo, hi] and
 * mantissa; exponent 0 gives subnormals and zeros. */
static uint16_t rand_bf16(int lo, int hi) {
  const uint32_t e = (uint32_t)(lo + (int)(next_u32() % (uint32_t)(hi - lo + 1)));
  return (uint16_t)(((next_u32() & 1u) << 15) | (e << 7) | (next_u32() & 0x7Fu));
}

static void one_head(int64_t vocab, int64_t hidden, int64_t batch,
                     const uint8_t* keep, int exp_lo, int exp_hi) {
  int32_t* idx = malloc(sizeof(int32_t) * (size_t)(vocab + 64));
  int64_t n_kept = 0;
  const int64_t n = oracle_build_index(keep, vocab, idx, vocab + 64, &n_kept);
  if (n <= 0) {
    expect(n_kept == 0, "empty mask");
    free(idx);
    return;
  }
  expect(n % 64 == 0 && n_kept >= 1 && n_kept <= n, "index shape");
  uint16_t* w = malloc(2 * (size_t)(vocab * hidden));
  for (int64_t i = 0; i < vocab * hidden; ++i) w[i] = rand_bf16(exp_lo, exp_hi);
  uint16_t* h = malloc(2 * (size_t)(batch * hidden));
  for (int64_t i = 0; i < batch * hidden; ++i) h[i] = rand_bf16(100, 130);
  uint8_t* packed = malloc((size_t)(n * hidden / 2));
  uint8_t* scales = malloc((size_t)(n * hidden / 16));
  uint8_t* q = malloc((size_t)(n * hidden));
  uint8_t* qx = malloc((size_t)(batch * hidden));
  float* sx = malloc(sizeof(float) * (size_t)batch);
  double* L = malloc(sizeof(double) * (size_t)(batch * n));
  uint16_t* Lb = malloc(2 * (size_t)(batch * n));
  float* out = malloc(sizeof(float) * (size_t)(batch * vocab));
  uint16_t* outb = malloc(2 * (size_t)(batch * vocab));
  int64_t* rows = malloc(sizeof(int64_t) * (size_t)batch);
  int32_t* ids = malloc(sizeof(int32_t) * (size_t)batch);
  float gs = 0.0f, sc = 0.0f;
  expect(oracle_nvfp4_quantize(w, vocab, hidden, idx, n, packed, scales, &gs) == 0,
         "nvfp4_quantize");
  expect(oracle_nvfp4_quantize_f16(w, vocab, hidden, idx, n, packed, scales,
                                   &gs) == 0,
         "nvfp4_quantize_f16");
  expect(oracle_nvfp4_logits(packed, scales, gs, n, hidden, h, batch, L) == 0,
         "nvfp4_logits");
  expect(oracle_argmax_remap(L, batch, n, idx, rows, ids) == 0, "argmax");
  expect(oracle_logits_scatter(L, batch, n, n_kept, idx, vocab, out) == 0,
         "scatter");
  expect(oracle_logits_to_bf16(L, batch * n, Lb) == 0, "to_bf16");
  expect(oracle_logits_scatter_bf16(Lb, batch, n, n_kept, idx, vocab, outb) == 0,
         "scatter_bf16");
  expect(oracle_bf16_logits(w, vocab, hidden, idx, n, h, batch, L) == 0,
         "bf16_logits");
  expect(oracle_e4m3_tensor_quantize(w, vocab, hidden, idx, n, q, &sc) == 0,
         "e4m3_quantize");
  expect(oracle_e4m3_tensor_logits(q, sc, n, hidden, h, batch, L) == 0,
         "e4m3_logits");
  expect(oracle_fp8_tokens_quantize(h, batch, hidden, qx, sx) == 0,
         "fp8_tokens");
  expect(oracle_w8a8_logits(q, sc, n, hidden, qx, sx, batch, L) == 0,
         "w8a8_logits");
  /* invalid shapes are refused, not read */
  expect(oracle_nvfp4_logits(packed, scales, gs, n, hidden - 8, h, batch, L) != 0,
         "nvfp4_logits rejects hidden % 16");
  expect(oracle_nvfp4_logits(packed, scales, gs, 0, hidden, h, batch, L) != 0,
         "nvfp4_logits rejects n_rows 0");
  free(w); free(h); free(packed); free(scales); free(q); free(qx); free(sx);
  free(L); free(Lb); free(out); free(outb); free(rows); free(ids); free(idx);
}

int main(void) {
  oracle_set_threads(2);
  expect(oracle_num_threads() >= 1, "threads");
  /* element codecs over every input they take */
  for (uint32_t c = 0; c < 256; ++c) {
    (void)oracle_e4m3_value((uint8_t)c);
    (void)oracle_e2m1_value((uint8_t)(c & 15));
  }
  for (uint32_t b = 0; b < 65536; ++b) {
    const float x = oracle_f16_value((uint16_t)b);
    (void)oracle_bf16_code(x);
    if (x >= 0.0f) (void)oracle_e4m3_code(x);
    (void)oracle_e2m1_code(x);
  }
  const int64_t V = 700;
  uint8_t* keep = calloc((size_t)V, 1);
  /* empty mask: refused */
  int32_t idx0[64];
  int64_t nk0 = -1;
  expect(oracle_build_index(keep, V, idx0, 64, &nk0) < 0, "empty mask refused");
  /* one id; the last id; every id; a random third; wide and narrow heads */
  keep[V / 2] = 1;
  one_head(V, 32, 1, keep, 110, 125);
  memset(keep, 0, (size_t)V);
  keep[V - 1] = 1;
  one_head(V, 48, 3, keep, 0, 254);
  memset(keep, 1, (size_t)V);
  one_head(V, 16, 2, keep, 120, 126);
  for (int64_t v = 0; v < V; ++v) keep[v] = (uint8_t)(next_u32() % 3 == 0);
  one_head(V, 64, 5, keep, 60, 200);
  memset(keep, 0, (size_t)V);
  for (int64_t v = 0; v < V; ++v) keep[v] = 1;
  /* an all-zero head (the 1e-12 floor) */
  {
    int32_t* idx = malloc(sizeof(int32_t) * (size_t)(V + 64));
    int64_t nk = 0;
    const int64_t n = oracle_build_index(keep, V, idx, V + 64, &nk);
    uint16_t* w = calloc((size_t)(V * 32), 2);
    uint8_t* p = malloc((size_t)(n * 16));
    uint8_t* s = malloc((size_t)(n * 2));
    float gs = 0.0f;
    expect(oracle_nvfp4_quantize(w, V, 32, idx, n, p, s, &gs) == 0, "zero head");
    free(idx); free(w); free(p); free(s);
  }
  /* capacity too small: refused */
  {
    int32_t small[8];
    int64_t nk = 0;
    expect(oracle_build_index(keep, V, small, 8, &nk) < 0,
           "small capacity refused");
  }
  free(keep);
  printf("oracle sanitizer run: %d failures\n", failures);
  return failures ? 1 : 0;
}
