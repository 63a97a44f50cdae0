/*
 * drafthead.h — C-ABI of the MI355X (gfx950) reduced-vocabulary NVFP4 draft
 * head.
 *
 * The method (page 1, "q38_draft.py", module docstring and load_draft_model;
 * page 4, "Qwen3.8-27B-NVFP4-DGX-SPARK", section on why native MTP plateaus):
 * a speculative drafter scores only a kept subset of the vocabulary.  The kept
 * rows of the BF16 target lm_head are gathered, re-quantized to NVFP4, and
 * every draft step runs a W4A16 GEMV of the hidden state against them, takes
 * the argmax over the kept rows and maps the winning row back to a target id.
 *
 * Conventions shared by every entry point below
 * ---------------------------------------------
 *  - Pointers marked [device] are device memory of the current HIP device;
 *    [host] pointers are ordinary host memory.  The caller owns every buffer;
 *    the library allocates nothing, keeps no per-call state and never
 *    synchronizes.  All device work is enqueued on `stream` (a hipStream_t
 *    passed as void*; NULL is the null stream) and is complete only when the
 *    caller synchronizes that stream.
 *  - Layouts are row-major.  Device pointers to weights, scales and hidden
 *    states, and the logits output, must be 16-byte aligned (every torch
 *    allocation is); ids, scalars and the workspace need 4 / 4 / 16 bytes.
 *    An NVFP4 head of n_rows x hidden is
 *      packed [n_rows][hidden/2]  uint8: element k of a row sits in byte k/2,
 *                                 low nibble for even k, high nibble for odd k;
 *                                 a nibble is sign (bit 3) + e2m1 magnitude
 *                                 index (bits 0-2) into {0,.5,1,1.5,2,3,4,6};
 *      scales [n_rows][hidden/16] uint8: OCP E4M3 (e4m3fn) scale of the
 *                                 16-element block k/16;
 *      global_scale               one float32; an element decodes to
 *                                 e2m1 * e4m3 * global_scale.
 *    A per-tensor E4M3 head is q [n_rows][hidden] OCP e4m3fn bytes and one
 *    float32 scale; an element decodes to e4m3 * scale.  A BF16 head is
 *    [n_rows][hidden] BF16.  BF16 tensors are raw 16-bit patterns.  Row
 *    indices are int32.
 *  - The row index dh_idx has n_rows entries, n_rows a multiple of 64: the
 *    n_kept kept target ids in ascending order, then copies of dh_idx[0]
 *    (page 1, load_draft_model pads the index so the NVFP4 GEMM row count is
 *    a multiple of 64).  draft_head_build_index produces it.
 *  - Workspace: device memory of at least draft_head_workspace_bytes() bytes,
 *    zero-filled once by the caller before its first use.  From then on it
 *    carries state from call to call (a call counter and per-block results
 *    tagged with it), so the caller must not modify it between calls; calls
 *    may share it whatever their head or batch size, and replaying a
 *    captured call is safe.  Calls that may run concurrently need distinct
 *    workspaces.
 *  - Give-up: the top-token calls combine per-block results across the
 *    grid, and a collecting block waits at most a bounded number of polling
 *    rounds (a fraction of a second or more; exceeded only if the device
 *    starves some blocks of the call).  A collector that gives up writes -1
 *    for its batch row and sets the uint16 at byte DH_WS_STATUS_OFFSET of
 *    the workspace.  The status is sticky: a block of the failed call that
 *    had not started may still leave a result the next call would take for
 *    its own, so every later top-token call on that workspace writes -1 for
 *    every batch row at once, without waiting, until the caller zero-fills
 *    the workspace again (on the same stream, or after the failed call has
 *    completed).  The uint16 at DH_WS_SPIN_LIMIT_OFFSET (0 after the
 *    zero-fill) lowers the bound: n > 0 allows n - 1 empty rounds, so 1
 *    gives up before the first poll; tests use it to reach this path
 *    without starving the device.
 *  - Every function returns DH_OK (0) or a negative DH_E* code; no C++
 *    exception crosses this interface.  Arguments are checked on the host
 *    before any device work is enqueued.  Ids outside [0, vocab) and
 *    non-finite inputs are outside the contract and are not checked on the
 *    device.
 */
#ifndef DRAFTHEAD_H
#define DRAFTHEAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DH_OK 0
#define DH_EINVAL (-1)     /* null pointer, bad size or shape */
#define DH_EWORKSPACE (-2) /* workspace pointer null or too small */
#define DH_EHIP (-3)       /* a HIP runtime call or kernel launch failed */

#define DRAFTHEAD_ABI_VERSION 5

/* Byte offsets of the two uint16 fields of a workspace a caller may read or
 * write (see "Give-up" above). */
#define DH_WS_STATUS_OFFSET 4
#define DH_WS_SPIN_LIMIT_OFFSET 6

int drafthead_abi_version(void);

/* Static text for a status code (never NULL). */
const char* drafthead_error_string(int status);

/*
 * Row index from a keep mask (page 1, load_draft_model: the kept ids come
 * from the mask's nonzero entries; with no mask every id is kept; the list is
 * padded to a multiple of 64 with copies of its first id).
 *   keep_mask [host]  vocab bytes, nonzero = kept
 *   dh_idx    [host]  out: capacity int32 slots
 *   n_kept    [host]  out: number of kept ids
 * Returns n_rows (>= 64) or DH_EINVAL (null pointer, vocab < 1, empty mask,
 * capacity < n_rows).  Host only; touches no device.
 */
int64_t draft_head_build_index(const uint8_t* keep_mask, int64_t vocab,
                               int32_t* dh_idx, int64_t capacity,
                               int64_t* n_kept);

/* Workspace bytes the calls below need for a head of n_rows rows at this
 * batch size.  Returns 0 for n_rows < 1, batch < 1 or batch > 64. */
size_t draft_head_workspace_bytes(int64_t n_rows, int64_t batch);

/*
 * Gather + NVFP4 quantization of the kept rows (page 3, "...MTP-NVFP4-h98k",
 * "How it was built": global scale amax/(6*448), E4M3 block scales per 16
 * elements, e2m1 codes rounded to nearest-even; page 1: the quantizer is fed
 * the gathered rows W[dh_idx]).
 *   w_bf16       [device] vocab x hidden BF16 target head
 *   row_ids      [device] n_rows int32 ids in [0, vocab) (dh_idx)
 *   packed       [device] out: n_rows x hidden/2
 *   scales       [device] out: n_rows x hidden/16
 *   global_scale [device] out: one float32
 * Arithmetic (float32, round-to-nearest-even): amax over the gathered rows;
 * gs = max(amax, 1e-12) / 2688; per block s = bmax / (6*gs) rounded to E4M3
 * (saturating at 448); element code = e2m1 of x / (e4m3(s)*gs), sign kept.
 * Errors: DH_EINVAL for null pointers, hidden < 16, hidden > 16384 or
 * hidden % 16 != 0, n_rows < 1, vocab < 1, packed not 8-byte aligned;
 * DH_EWORKSPACE; DH_EHIP.
 */
int nvfp4_quantize_rows(const void* w_bf16, int64_t vocab, int64_t hidden,
                        const int32_t* row_ids, int64_t n_rows,
                        uint8_t* packed, uint8_t* scales, float* global_scale,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same quantization of an FP16 head (page 1, "q38_draft.py", the
 * install step accepts a BF16 or an FP16 head).
 *   w_f16 [device] vocab x hidden IEEE binary16
 * Every binary16 value is exact in float32; the recipe, the outputs and the
 * errors are those of nvfp4_quantize_rows.
 */
int nvfp4_quantize_rows_f16(const void* w_f16, int64_t vocab, int64_t hidden,
                            const int32_t* row_ids, int64_t n_rows,
                            uint8_t* packed, uint8_t* scales,
                            float* global_scale, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * Greedy draft tokens (page 1, get_top_tokens: the argmax over the kept rows
 * of the draft head's output, mapped through dh_idx).
 *   packed, scales, global_scale [device] the NVFP4 head (layout above)
 *   dh_idx   [device] n_rows int32
 *   h_bf16   [device] batch x hidden BF16 hidden states
 *   out_ids  [device] out: batch int32 target ids
 * For each batch row b: logit_j = sum_k e2m1*e4m3*h[b,k] accumulated in
 * float32 (the positive global scale does not change the argmax and is not
 * applied); row = lowest j with the largest logit; out_ids[b] = dh_idx[row].
 * Errors: DH_EINVAL for null pointers, hidden % 16 != 0, hidden < 16,
 * hidden > 16384, n_rows < 64 or n_rows % 64 != 0, batch < 1 or batch > 64,
 * misaligned pointers; DH_EWORKSPACE; DH_EHIP.
 */
int draft_head_top_tokens(const uint8_t* packed, const uint8_t* scales,
                          const float* global_scale, const int32_t* dh_idx,
                          int64_t n_rows, int64_t hidden, const void* h_bf16,
                          int64_t batch, int32_t* out_ids, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * draft_head_top_tokens without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  The finish state a
 * workspace would carry lives in a static device array of the library
 * (DRAFTHEAD_NOALLOC_SCRATCH_BYTES, the largest workspace any batch needs;
 * each GPU holds its own copy until the process ends); the call allocates
 * nothing.  Arguments, results and errors are those of
 * draft_head_top_tokens, whose kernels it runs; a workspace size beyond the
 * array, which no valid batch reaches, returns DH_EWORKSPACE.
 * The array starts zeroed and carries the state from call to call as a
 * workspace does, so nothing is cleared per call.  Every call on a GPU
 * shares that GPU's array: calls that may overlap on one GPU (unordered
 * streams, several host threads) race and must not be issued.  A give-up
 * (see above) is sticky for the rest of the process on that GPU, since
 * nothing can zero-fill the array again: draft_head_top_tokens with a
 * workspace of the caller's remains available.
 */
#define DRAFTHEAD_NOALLOC_SCRATCH_BYTES 1048832
int draft_head_top_tokens_noalloc(const uint8_t* packed,
                                  const uint8_t* scales,
                                  const float* global_scale,
                                  const int32_t* dh_idx, int64_t n_rows,
                                  int64_t hidden, const void* h_bf16,
                                  int64_t batch, int32_t* out_ids,
                                  void* stream);

/*
 * Draft logits over the full vocabulary (page 1, compute_logits: the draft
 * head's output in float32, written into a batch x vocab tensor filled with
 * -inf at the kept ids; page 2, compute_logits does the same scatter).
 *   out_logits [device] out: batch x vocab float32
 * out[b, v] = -inf for every v not among dh_idx[0:n_kept];
 * out[b, dh_idx[j]] = global_scale * logit_j (float32) for j < n_kept (the
 * pad rows are not written).  dh_idx[0:n_kept] must be strictly ascending,
 * as draft_head_build_index makes it: the -inf fill is part of the same
 * pass (one launch per batch slice of up to 16 rows), each kept row writing
 * the ids from just past the previous kept id up to its own, so a mask
 * with a long run of dropped ids costs the wave owning that run about
 * run/64 store rounds.  Ids that are not ascending or not below vocab give
 * wrong logits but no store outside out_logits.
 * Errors: as draft_head_top_tokens, plus DH_EINVAL for n_kept < 1,
 * n_kept > n_rows, vocab < n_kept.
 */
int draft_head_logits(const uint8_t* packed, const uint8_t* scales,
                      const float* global_scale, const int32_t* dh_idx,
                      int64_t n_rows, int64_t n_kept, int64_t hidden,
                      int64_t vocab, const void* h_bf16, int64_t batch,
                      float* out_logits, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * The pages' own numerics, for a caller that must reproduce them (page 1,
 * get_top_tokens, and page 2, compute_logits, take the argmax and the
 * scatter of the BF16 output of the drafter's linear).
 * draft_head_top_tokens_compat: as draft_head_top_tokens, with the argmax
 *   over c_j = bf16(gs * logit_j) -- the float32 logit times the global
 *   scale in float32, rounded to nearest-even BF16 -- and the lowest j
 *   among equal c_j (BF16 values tie often).
 * draft_head_logits_compat: as draft_head_logits with BF16 output:
 *   out[b, dh_idx[j]] = bf16(gs * logit_j) for j < n_kept, -inf (0xFF80)
 *   elsewhere; out_logits_bf16 is batch x vocab BF16, 16-byte aligned.
 * Errors: as draft_head_top_tokens / draft_head_logits.
 */
int draft_head_top_tokens_compat(const uint8_t* packed,
                                 const uint8_t* scales,
                                 const float* global_scale,
                                 const int32_t* dh_idx, int64_t n_rows,
                                 int64_t hidden, const void* h_bf16,
                                 int64_t batch, int32_t* out_ids,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream);
int draft_head_logits_compat(const uint8_t* packed, const uint8_t* scales,
                             const float* global_scale,
                             const int32_t* dh_idx, int64_t n_rows,
                             int64_t n_kept, int64_t hidden, int64_t vocab,
                             const void* h_bf16, int64_t batch,
                             void* out_logits_bf16, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * NVFP4 W4A16 linear for the drafter's other projections (page 1,
 * "q38_draft.py", install: every 2-D BF16 weight of the MTP block named in
 * its key list, with N % 64 == 0 and K % 16 == 0, is quantized with the same
 * recipe and its forward returns the quantized linear's output).  Quantize
 * the weight with nvfp4_quantize_rows and an identity row_ids.
 *   packed, scales, global_scale [device] the NVFP4 weight, n_rows x hidden
 *   h_bf16  [device] batch x hidden BF16 inputs
 *   out     [device] out: batch x n_rows float32, row-major
 * out[b, j] = global_scale * sum_k e2m1*e4m3*h[b,k], accumulated in float32
 * (never rounded to BF16).  No workspace: nothing crosses blocks.
 * Errors: DH_EINVAL for null or misaligned pointers (out 16 bytes), hidden %
 * 16 != 0, hidden < 16, hidden > 16384, n_rows < 64 or n_rows % 64 != 0,
 * batch < 1 or batch > 64; DH_EHIP.
 */
int nvfp4_linear(const uint8_t* packed, const uint8_t* scales,
                 const float* global_scale, int64_t n_rows, int64_t hidden,
                 const void* h_bf16, int64_t batch, float* out, void* stream);

/*
 * Per-tensor E4M3 head from the same gathered rows (page 2, "FP8 MTP draft
 * stack for vLLM", _fp8_convert_draft_head: the FP8 head it ships scales the whole head by amax/448, divides, clamps to
 * +-448 and casts to e4m3fn; page 3 lists the FP8 head next to the NVFP4 one).
 *   w_bf16  [device] vocab x hidden BF16 target head
 *   row_ids [device] n_rows int32 ids in [0, vocab)
 *   q       [device] out: n_rows x hidden e4m3fn bytes
 *   scale   [device] out: one float32
 * Arithmetic (float32, round-to-nearest-even): amax over the gathered rows;
 * scale = max(amax, 1e-12) / 448; q = e4m3(clamp(x / scale, -448, 448)),
 * sign kept (0x80 for a negative zero quotient).
 * Errors: as nvfp4_quantize_rows (q must be 8-byte aligned).
 */
int e4m3_quantize_rows_per_tensor(const void* w_bf16, int64_t vocab,
                                  int64_t hidden, const int32_t* row_ids,
                                  int64_t n_rows, uint8_t* q, float* scale,
                                  void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * Greedy draft tokens of a per-tensor E4M3 head (page 1, get_top_tokens, as
 * for the NVFP4 head; page 2's FP8 head).  Activations stay BF16 (W8A16):
 * logit_j = sum_k e4m3(q[j,k]) * h[b,k] in float32, the scale (positive) is
 * not applied; out_ids[b] = dh_idx[lowest j with the largest logit].
 * Errors: as draft_head_top_tokens.
 */
int draft_head_top_tokens_e4m3(const uint8_t* q, const float* scale,
                               const int32_t* dh_idx, int64_t n_rows,
                               int64_t hidden, const void* h_bf16,
                               int64_t batch, int32_t* out_ids,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * Logits of a per-tensor E4M3 head (page 2, compute_logits): as
 * draft_head_logits with out[b, dh_idx[j]] = scale * logit_j.
 * Errors: as draft_head_logits.
 */
int draft_head_logits_e4m3(const uint8_t* q, const float* scale,
                           const int32_t* dh_idx, int64_t n_rows,
                           int64_t n_kept, int64_t hidden, int64_t vocab,
                           const void* h_bf16, int64_t batch,
                           float* out_logits, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Per-token dynamic E4M3 quantization of hidden states (page 2, "FP8 MTP
 * draft stack for vLLM", _Fp8DraftHeadMethod.apply: the FP8 head quantizes
 * each token's activations with a scale of its own before the scaled GEMM).
 *   h_bf16 [device] batch x hidden BF16, 16-byte aligned
 *   qx     [device] out: batch x hidden e4m3fn bytes, 8-byte aligned
 *   sx     [device] out: batch float32 scales
 * Arithmetic (float32, round-to-nearest-even), per row b: amax over the
 * row; sx[b] = max(amax, 1e-12) / 448; qx = e4m3(clamp(x / sx[b], -448,
 * 448)), sign kept -- the head's recipe with one scale per token.
 * Errors: DH_EINVAL for a null or misaligned pointer, hidden not a multiple
 * of 16 in [16, 16384], batch < 1 or > 65536; DH_EHIP.
 */
int fp8_quantize_tokens(const void* h_bf16, int64_t batch, int64_t hidden,
                        uint8_t* qx, float* sx, void* stream);

/* Workspace bytes for the W8A8 head calls below (0 for an invalid shape):
 * the state of any top-token call (its largest batch) plus scratch for the
 * quantized tokens, so one workspace can serve these and the other calls. */
size_t draft_head_workspace_bytes_w8a8(int64_t n_rows, int64_t batch,
                                       int64_t hidden);

/*
 * Greedy draft tokens of the FP8 head as page 2 applies it, W8A8 (page 2,
 * _Fp8DraftHeadMethod.apply: per-token dynamic activation quantization,
 * then a GEMM scaled by the token's and the head's scale; page 1,
 * get_top_tokens for the argmax and the remap).  q and scale come from
 * e4m3_quantize_rows_per_tensor.  The call quantizes h as
 * fp8_quantize_tokens does, into the workspace, then
 * logit_j = sum_k e4m3(q[j,k]) * e4m3(qx[b,k]) in float32 (each product is
 * exact); the scales are positive and leave the argmax unchanged.
 * out_ids[b] = dh_idx[lowest j with the largest logit].
 *   workspace  zero-filled once, draft_head_workspace_bytes_w8a8 bytes; it
 *              carries state from call to call as for draft_head_top_tokens
 * Errors: as draft_head_top_tokens.
 */
int draft_head_top_tokens_w8a8(const uint8_t* q, const float* scale,
                               const int32_t* dh_idx, int64_t n_rows,
                               int64_t hidden, const void* h_bf16,
                               int64_t batch, int32_t* out_ids,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * Logits of the W8A8 FP8 head (page 2, apply and compute_logits): as
 * draft_head_logits with
 * out[b, dh_idx[j]] = sx[b] * scale * sum_k e4m3(q[j,k]) * e4m3(qx[b,k]).
 * Errors: as draft_head_logits; the workspace as above.
 */
int draft_head_logits_w8a8(const uint8_t* q, const float* scale,
                           const int32_t* dh_idx, int64_t n_rows,
                           int64_t n_kept, int64_t hidden, int64_t vocab,
                           const void* h_bf16, int64_t batch,
                           float* out_logits, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Greedy tokens of an unquantized BF16 head (page 4: the stock drafter reads
 * the full BF16 lm_head every draft step; page 1, get_top_tokens).  For the
 * stock head pass all vocab rows and the identity index.
 *   w_bf16 [device] n_rows x hidden BF16 rows (row j scores id dh_idx[j])
 * logit_j = sum_k w[j,k] * h[b,k] in float32; out_ids[b] = dh_idx[lowest j
 * with the largest logit].
 * Errors: as draft_head_top_tokens.
 */
int draft_head_top_tokens_bf16(const void* w_bf16, const int32_t* dh_idx,
                               int64_t n_rows, int64_t hidden,
                               const void* h_bf16, int64_t batch,
                               int32_t* out_ids, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * Logits of a BF16 head (page 1 and page 2, compute_logits): as
 * draft_head_logits with out[b, dh_idx[j]] = logit_j.
 * Errors: as draft_head_logits.
 */
int draft_head_logits_bf16(const void* w_bf16, const int32_t* dh_idx,
                           int64_t n_rows, int64_t n_kept, int64_t hidden,
                           int64_t vocab, const void* h_bf16, int64_t batch,
                           float* out_logits, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Measurement aid: streams a_bytes at a, then b_bytes at b, once, with
 * nothing else to do (page 4, "autotrust/Qwen3.8-27B-NVFP4-DGX-SPARK", "Why
 * native MTP plateaus at 37": a draft step is a stream of lm_head bytes).
 * Timed on a head's own buffers (codes and scales), it gives the rate at
 * which the device streams those bytes: the practical ceiling of the
 * draft-head calls above.  Nothing is computed and nothing written, except
 * that every wave of the read folds the 32-bit words it read into one XOR
 * and stores it to sink[0] when it equals DRAFTHEAD_READ_PROBE_MAGIC (so
 * the reads cannot be skipped, and a buffer that holds the constant once
 * among zeros shows that every byte was read).
 *   a      [device] 16-byte aligned, a_bytes a multiple of 16
 *   b      [device] 16-byte aligned, b_bytes a multiple of 16; NULL when
 *                   b_bytes is 0
 *   sink   [device] one uint32, 4-byte aligned
 * Errors: DH_EINVAL for a null or misaligned pointer, a size that is not a
 * multiple of 16 or above 2^48 bytes, or nothing to read; DH_EHIP.
 */
#define DRAFTHEAD_READ_PROBE_MAGIC 0x9E3779B9u
int drafthead_read_probe(const void* a, size_t a_bytes, const void* b,
                         size_t b_bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DRAFTHEAD_H */
