/*
 * Oracle for the reduced-vocabulary NVFP4 draft head.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or helper with the
 * HIP library; the two meet only at seeded inputs.
 *
 * What it computes, step by step, in the order of the pages:
 *   C1  build the draft-head row index (kept ids ascending, padded to a
 *       multiple of 64 with the first kept id)        -- page 1, q38_draft.py,
 *       load_draft_model
 *   C2  global scale gs = max(amax, 1e-12) / (6*448)   -- page 3 (98K head),
 *       "How it was built", NVFP4 recipe; the 1e-12 floor is the one page 2
 *       (FP8 MTP draft stack) uses in _fp8_convert_draft_head
 *   C3  per-16 E4M3 block scale, round-to-nearest-even, saturating
 *   C4  e2m1 element codes, round-to-nearest-even, two per byte
 *   C5  W4A16 logits, accumulated in float64
 *   C6  argmax over the kept rows (first maximal row), then the id remap
 *                                                      -- page 1,
 *       get_top_tokens
 *   C7  fp32 logits scattered to the full vocabulary, -inf elsewhere
 *                                                      -- page 1,
 *       compute_logits; page 2, compute_logits
 *   C8  BF16 stock head logits (identity index)        -- page 1, _Bf16 and
 *       the no-mask branch of load_draft_model
 *   C9  E4M3 per-tensor head: scale = max(amax,1e-12)/448, clamp, E4M3 cast
 *                                                      -- page 2,
 *       _fp8_convert_draft_head; page 3, "How it was built" (98K head)
 *   C10 per-token dynamic E4M3 activations: each row of h gets its own
 *       scale max(amax_row, 1e-12)/448, then the same clamp and cast as C9
 *                                                      -- page 2,
 *       _Fp8DraftHeadMethod.apply (per-token dynamic activation quant)
 *   C11 W8A8 logits: both operands E4M3, scaled by the token's and the
 *       head's scale, accumulated in float64              -- page 2,
 *       _Fp8DraftHeadMethod.apply (the scaled GEMM)
 *   C12 reference-compatible mode: an FP16 head is accepted (its values
 *       decoded exactly) -- page 1, q38_draft.py, the install step's check
 *       that the head is BF16 or FP16; the logits are float32 values
 *       rounded to BF16 before the argmax and the scatter, as the BF16
 *       output of the pages' linear is (page 1, get_top_tokens; page 2,
 *       compute_logits keeps the processor's dtype)
 *
 * Floating point: every float operation below is one IEEE binary32 operation
 * rounded to nearest-even (built with -ffp-contract=off, no fast-math, SSE).
 * Encodings are written as "nearest value of a finite grid, ties to the code
 * whose last bit is 0" and found by scanning the grid, not by bit tricks.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)

/* ---------------------------------------------------------------- helpers */

static float bf16_value(uint16_t bits) {
    /* A BF16 number is the upper half of the binary32 with the same value. */
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* An IEEE binary16 number: sign, 5 exponent bits (bias 15), 10 mantissa
 * bits; exponent 0 is subnormal (m * 2^-24).  Every value is exact in
 * binary32. */
static float f16_value(uint16_t bits) {
    int sign = (bits >> 15) & 1;
    int e = (bits >> 10) & 31;
    int m = bits & 1023;
    double mag;
    if (e == 31)
        mag = m ? NAN : INFINITY;
    else if (e == 0)
        mag = ldexp((double)m, -24);
    else
        mag = ldexp(1.0 + m / 1024.0, e - 15);
    return (float)(sign ? -mag : mag);
}

float oracle_f16_value(uint16_t bits) { return f16_value(bits); }

/* BF16 bits of a binary32 rounded to nearest, ties to the even code: of
 * the two BF16 neighbours of x (x with its low 16 bits cleared, and the
 * next value away from zero) take the closer one; on a tie the one whose
 * last bit is 0.  Past the largest finite BF16 the upper neighbour is the
 * infinity code, whose distance is measured from 2^128, as if the exponent
 * went on (IEEE overflow). */
uint16_t oracle_bf16_code(float x) {
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    uint32_t lo = u & 0xFFFF0000u, hi = lo + 0x10000u;
    float flo, fhi;
    memcpy(&flo, &lo, sizeof flo);
    memcpy(&fhi, &hi, sizeof fhi);
    double dhi_val = (double)fhi;
    if ((hi & 0x7F800000u) == 0x7F800000u)
        dhi_val = copysign(ldexp(1.0, 128), (double)x);
    double dlo = fabs((double)x - (double)flo);
    double dhi = fabs(dhi_val - (double)x);
    if (dlo < dhi) return (uint16_t)(lo >> 16);
    if (dhi < dlo) return (uint16_t)(hi >> 16);
    return (uint16_t)(((lo >> 16) & 1) ? (hi >> 16) : (lo >> 16));
}

/* ------------------------------------------------------------ E4M3 (OCP) */

/* Value of an OCP e4m3fn byte: sign, 4 exponent bits (bias 7), 3 mantissa
 * bits; exponent 0 is subnormal (m * 2^-9); 0x7F and 0xFF are NaN; there are
 * no infinities, so the largest finite magnitude is 0x7E = 448. */
double oracle_e4m3_value(uint8_t code) {
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -mag : mag;
}

static double E4M3_GRID[127]; /* magnitudes of codes 0x00..0x7E, ascending */
static double E2M1_GRID[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
static int grids_ready = 0;

static void init_grids(void) {
    if (grids_ready) return;
    for (int c = 0; c < 127; ++c) E4M3_GRID[c] = oracle_e4m3_value((uint8_t)c);
    grids_ready = 1;
}

/* Round a non-negative magnitude onto a finite ascending grid: nearest grid
 * value, a tie goes to the even code, anything above the top value
 * saturates to the top code.  The midpoint of two grid values is exact in
 * float64, so every comparison is exact. */
static int round_to_grid(double x, const double* grid, int n) {
    for (int c = 0; c + 1 < n; ++c) {
        double mid = 0.5 * (grid[c] + grid[c + 1]);
        if (x < mid) return c;
        if (x == mid) return (c % 2 == 0) ? c : c + 1;
    }
    return n - 1;
}

/* E4M3 code of a non-negative float: RNE, values past 448 saturate to 0x7E
 * (0x7F, the NaN, is never produced). */
uint8_t oracle_e4m3_code(float s) {
    init_grids();
    return (uint8_t)round_to_grid((double)s, E4M3_GRID, 127);
}

/* ------------------------------------------------------------------ e2m1 */

/* Value of an e2m1 nibble: bit 3 is the sign, bits 0-2 index
 * {0, 0.5, 1, 1.5, 2, 3, 4, 6}. */
double oracle_e2m1_value(uint8_t nib) {
    double mag = E2M1_GRID[nib & 7];
    return (nib & 8) ? -mag : mag;
}

/* e2m1 nibble of a float: the sign is the float's sign bit (so -0 and
 * negatives that round to zero keep it), the magnitude is RNE onto the grid
 * with saturation at 6. */
uint8_t oracle_e2m1_code(float q) {
    uint8_t mag = (uint8_t)round_to_grid(fabs((double)q), E2M1_GRID, 8);
    return (uint8_t)((signbit(q) ? 8 : 0) | mag);
}

/* -------------------------------------------------------------- C1 index */

/* Draft-head row index from a bool keep mask: the kept ids in ascending
 * order, then (-n) mod 64 copies of the first kept id.  Returns the padded
 * row count, or -1 for an empty mask or too small an output buffer. */
int64_t oracle_build_index(const uint8_t* keep, int64_t vocab, int32_t* idx,
                           int64_t cap, int64_t* n_kept_out) {
    int64_t n = 0;
    for (int64_t v = 0; v < vocab; ++v) {
        if (keep[v]) {
            if (n >= cap) return -1;
            idx[n++] = (int32_t)v;
        }
    }
    if (n == 0) return -1;
    int64_t pad = (64 - n % 64) % 64;
    if (n + pad > cap) return -1;
    for (int64_t p = 0; p < pad; ++p) idx[n + p] = idx[0];
    if (n_kept_out) *n_kept_out = n;
    return n + pad;
}

/* ---------------------------------------------------- C2-C4 NVFP4 encode */

/* Quantize the gathered rows W[idx[j]] (BF16 bits, row-major [vocab,hidden])
 * to NVFP4.  Outputs: packed[j*hidden/2 + k/2] holds element k in the low
 * nibble when k is even and in the high nibble when k is odd;
 * scales[j*hidden/16 + k/16] is the E4M3 byte of block k/16; *gs the global
 * scale.  A value decodes as e2m1(nibble) * e4m3(scale) * gs. */
typedef float (*elem_fn)(uint16_t);

static int nvfp4_quantize(const uint16_t* w, elem_fn value, int64_t vocab,
                          int64_t hidden, const int32_t* idx, int64_t n_rows,
                          uint8_t* packed, uint8_t* scales, float* gs_out) {
    if (hidden <= 0 || hidden % 16 != 0 || n_rows <= 0) return ORACLE_EINVAL;
    for (int64_t j = 0; j < n_rows; ++j)
        if (idx[j] < 0 || idx[j] >= vocab) return ORACLE_EINVAL;
    init_grids();

    /* C2: amax over the gathered rows, then one binary32 division. */
    float amax = 0.0f;
#pragma omp parallel for reduction(max : amax) schedule(static)
    for (int64_t j = 0; j < n_rows; ++j) {
        const uint16_t* row = w + (int64_t)idx[j] * hidden;
        for (int64_t k = 0; k < hidden; ++k) {
            float a = fabsf(value(row[k]));
            if (a > amax) amax = a;
        }
    }
    float gs = fmaxf(amax, 1e-12f) / 2688.0f; /* 2688 = 6 * 448 */
    float six_gs = 6.0f * gs;
    *gs_out = gs;

    int64_t nblk = hidden / 16;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n_rows; ++j) {
        const uint16_t* row = w + (int64_t)idx[j] * hidden;
        for (int64_t b = 0; b < nblk; ++b) {
            const uint16_t* blk = row + b * 16;
            /* C3: block amax, then scale = bmax / (6 * gs), E4M3. */
            float bmax = 0.0f;
            for (int i = 0; i < 16; ++i) {
                float a = fabsf(value(blk[i]));
                if (a > bmax) bmax = a;
            }
            float s = bmax / six_gs;
            uint8_t sc = oracle_e4m3_code(s);
            scales[j * nblk + b] = sc;
            float s_dec = (float)oracle_e4m3_value(sc);
            float d = s_dec * gs;
            /* C4: element codes. */
            for (int i = 0; i < 16; ++i) {
                float x = value(blk[i]);
                uint8_t nib;
                if (s_dec == 0.0f)
                    nib = (uint8_t)(signbit(x) ? 8 : 0);
                else
                    nib = oracle_e2m1_code(x / d);
                int64_t k = b * 16 + i;
                uint8_t* byte = &packed[j * (hidden / 2) + k / 2];
                if (k % 2 == 0)
                    *byte = (uint8_t)((*byte & 0xF0) | nib);
                else
                    *byte = (uint8_t)((*byte & 0x0F) | (nib << 4));
            }
        }
    }
    return ORACLE_OK;
}

int oracle_nvfp4_quantize(const uint16_t* w, int64_t vocab, int64_t hidden,
                          const int32_t* idx, int64_t n_rows, uint8_t* packed,
                          uint8_t* scales, float* gs_out) {
    return nvfp4_quantize(w, bf16_value, vocab, hidden, idx, n_rows, packed,
                          scales, gs_out);
}

/* C12: the same recipe on an FP16 head. */
int oracle_nvfp4_quantize_f16(const uint16_t* w, int64_t vocab,
                              int64_t hidden, const int32_t* idx,
                              int64_t n_rows, uint8_t* packed,
                              uint8_t* scales, float* gs_out) {
    return nvfp4_quantize(w, f16_value, vocab, hidden, idx, n_rows, packed,
                          scales, gs_out);
}

/* ------------------------------------------------------------- C5 logits */

/* L[b*n_rows + j] = gs * sum_k e2m1(q[j,k]) * e4m3(s[j,k/16]) * h[b,k],
 * float64 throughout; every product is exact in float64. */
int oracle_nvfp4_logits(const uint8_t* packed, const uint8_t* scales,
                        float gs, int64_t n_rows, int64_t hidden,
                        const uint16_t* h, int64_t batch, double* L) {
    if (hidden <= 0 || hidden % 16 != 0 || n_rows <= 0 || batch <= 0)
        return ORACLE_EINVAL;
    int64_t nblk = hidden / 16;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t j = 0; j < n_rows; ++j) {
            double acc = 0.0;
            for (int64_t k = 0; k < hidden; ++k) {
                uint8_t byte = packed[j * (hidden / 2) + k / 2];
                uint8_t nib = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
                double wk = oracle_e2m1_value(nib) *
                            oracle_e4m3_value(scales[j * nblk + k / 16]);
                acc += wk * (double)bf16_value(h[b * hidden + k]);
            }
            L[b * n_rows + j] = (double)gs * acc;
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------ C6 argmax, remap */

/* For every batch row: the first row index holding the largest logit, and
 * the target id idx[row] it maps to. */
int oracle_argmax_remap(const double* L, int64_t batch, int64_t n_rows,
                        const int32_t* idx, int64_t* row_out,
                        int32_t* id_out) {
    if (batch <= 0 || n_rows <= 0) return ORACLE_EINVAL;
    for (int64_t b = 0; b < batch; ++b) {
        const double* l = L + b * n_rows;
        int64_t best = 0;
        for (int64_t j = 1; j < n_rows; ++j)
            if (l[j] > l[best]) best = j;
        if (row_out) row_out[b] = best;
        id_out[b] = idx[best];
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------ C7 scatter */

/* out[b, v] = -inf for every id v, then out[b, idx[j]] = (float)L[b, j] for
 * the n_kept kept rows (the pad rows are left out). */
int oracle_logits_scatter(const double* L, int64_t batch, int64_t n_rows,
                          int64_t n_kept, const int32_t* idx, int64_t vocab,
                          float* out) {
    if (batch <= 0 || n_kept <= 0 || n_kept > n_rows) return ORACLE_EINVAL;
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t v = 0; v < vocab; ++v) out[b * vocab + v] = -INFINITY;
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t j = 0; j < n_kept; ++j) {
            if (idx[j] < 0 || idx[j] >= vocab) return ORACLE_EINVAL;
            out[b * vocab + idx[j]] = (float)L[b * n_rows + j];
        }
    return ORACLE_OK;
}

/* C12: the logits as the pages' BF16 linear returns them: each float64
 * logit rounded to binary32 (the accumulator's precision), then to BF16. */
int oracle_logits_to_bf16(const double* L, int64_t n, uint16_t* out) {
    if (n <= 0) return ORACLE_EINVAL;
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_code((float)L[i]);
    return ORACLE_OK;
}

/* C12: the scatter of C7 in BF16: -inf is 0xFF80; the pad rows are left
 * out. */
int oracle_logits_scatter_bf16(const uint16_t* Lb, int64_t batch,
                               int64_t n_rows, int64_t n_kept,
                               const int32_t* idx, int64_t vocab,
                               uint16_t* out) {
    if (batch <= 0 || n_kept <= 0 || n_kept > n_rows) return ORACLE_EINVAL;
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t v = 0; v < vocab; ++v) out[b * vocab + v] = 0xFF80u;
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t j = 0; j < n_kept; ++j) {
            if (idx[j] < 0 || idx[j] >= vocab) return ORACLE_EINVAL;
            out[b * vocab + idx[j]] = Lb[b * n_rows + j];
        }
    return ORACLE_OK;
}

/* ------------------------------------------------------- C8 BF16 logits */

/* L[b*n_rows + j] = sum_k W[rows[j], k] * h[b, k] in float64 (each product
 * of two BF16 numbers is exact). */
int oracle_bf16_logits(const uint16_t* w, int64_t vocab, int64_t hidden,
                       const int32_t* rows, int64_t n_rows, const uint16_t* h,
                       int64_t batch, double* L) {
    if (hidden <= 0 || n_rows <= 0 || batch <= 0) return ORACLE_EINVAL;
    for (int64_t j = 0; j < n_rows; ++j)
        if (rows[j] < 0 || rows[j] >= vocab) return ORACLE_EINVAL;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t j = 0; j < n_rows; ++j) {
            const uint16_t* row = w + (int64_t)rows[j] * hidden;
            double acc = 0.0;
            for (int64_t k = 0; k < hidden; ++k)
                acc += (double)bf16_value(row[k]) *
                       (double)bf16_value(h[b * hidden + k]);
            L[b * n_rows + j] = acc;
        }
    }
    return ORACLE_OK;
}

/* ---------------------------------------------- C9 E4M3 per-tensor head */

/* scale = max(amax, 1e-12) / 448 over the gathered rows; each element is
 * x / scale, clamped to [-448, 448], cast to E4M3 (RNE, sign kept). */
int oracle_e4m3_tensor_quantize(const uint16_t* w, int64_t vocab,
                                int64_t hidden, const int32_t* idx,
                                int64_t n_rows, uint8_t* q, float* scale_out) {
    if (hidden <= 0 || n_rows <= 0) return ORACLE_EINVAL;
    for (int64_t j = 0; j < n_rows; ++j)
        if (idx[j] < 0 || idx[j] >= vocab) return ORACLE_EINVAL;
    init_grids();
    float amax = 0.0f;
#pragma omp parallel for reduction(max : amax) schedule(static)
    for (int64_t j = 0; j < n_rows; ++j) {
        const uint16_t* row = w + (int64_t)idx[j] * hidden;
        for (int64_t k = 0; k < hidden; ++k) {
            float a = fabsf(bf16_value(row[k]));
            if (a > amax) amax = a;
        }
    }
    float scale = fmaxf(amax, 1e-12f) / 448.0f;
    *scale_out = scale;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n_rows; ++j) {
        const uint16_t* row = w + (int64_t)idx[j] * hidden;
        for (int64_t k = 0; k < hidden; ++k) {
            float v = bf16_value(row[k]) / scale;
            if (v > 448.0f) v = 448.0f;
            if (v < -448.0f) v = -448.0f;
            uint8_t mag = oracle_e4m3_code(fabsf(v));
            q[j * hidden + k] = (uint8_t)((signbit(v) ? 0x80 : 0) | mag);
        }
    }
    return ORACLE_OK;
}

/* L[b*n_rows + j] = scale * sum_k e4m3(q[j,k]) * h[b,k] in float64. */
int oracle_e4m3_tensor_logits(const uint8_t* q, float scale, int64_t n_rows,
                              int64_t hidden, const uint16_t* h, int64_t batch,
                              double* L) {
    if (hidden <= 0 || n_rows <= 0 || batch <= 0) return ORACLE_EINVAL;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t j = 0; j < n_rows; ++j) {
            double acc = 0.0;
            for (int64_t k = 0; k < hidden; ++k)
                acc += oracle_e4m3_value(q[j * hidden + k]) *
                       (double)bf16_value(h[b * hidden + k]);
            L[b * n_rows + j] = (double)scale * acc;
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------- C10 per-token E4M3 activations */

/* For every row b of h: sx[b] = max(amax_b, 1e-12) / 448 with amax_b the
 * largest |h[b,k]|; each element is h / sx[b], clamped to [-448, 448] and
 * cast to E4M3 (RNE, sign kept) -- the head's recipe of C9, one scale per
 * token instead of one per tensor. */
int oracle_fp8_tokens_quantize(const uint16_t* h, int64_t batch,
                               int64_t hidden, uint8_t* qx, float* sx) {
    if (hidden <= 0 || batch <= 0) return ORACLE_EINVAL;
    init_grids();
    for (int64_t b = 0; b < batch; ++b) {
        const uint16_t* row = h + b * hidden;
        float amax = 0.0f;
        for (int64_t k = 0; k < hidden; ++k) {
            float a = fabsf(bf16_value(row[k]));
            if (a > amax) amax = a;
        }
        float scale = fmaxf(amax, 1e-12f) / 448.0f;
        sx[b] = scale;
        for (int64_t k = 0; k < hidden; ++k) {
            float v = bf16_value(row[k]) / scale;
            if (v > 448.0f) v = 448.0f;
            if (v < -448.0f) v = -448.0f;
            uint8_t mag = oracle_e4m3_code(fabsf(v));
            qx[b * hidden + k] = (uint8_t)((signbit(v) ? 0x80 : 0) | mag);
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------ C11 W8A8 logits */

/* L[b*n_rows + j] = sx[b] * sw * sum_k e4m3(q[j,k]) * e4m3(qx[b,k]) in
 * float64 (each product of two E4M3 values is exact). */
int oracle_w8a8_logits(const uint8_t* q, float sw, int64_t n_rows,
                       int64_t hidden, const uint8_t* qx, const float* sx,
                       int64_t batch, double* L) {
    if (hidden <= 0 || n_rows <= 0 || batch <= 0) return ORACLE_EINVAL;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t j = 0; j < n_rows; ++j) {
            double acc = 0.0;
            for (int64_t k = 0; k < hidden; ++k)
                acc += oracle_e4m3_value(q[j * hidden + k]) *
                       oracle_e4m3_value(qx[b * hidden + k]);
            L[b * n_rows + j] = (double)sx[b] * (double)sw * acc;
        }
    }
    return ORACLE_OK;
}

/* Threads an OpenMP region of this library uses, and a way to set them. */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
