// Batched GEMV on the matrix cores: for a batch slice of up to 16 hidden
// states the head's weights are decoded to BF16 in registers (exactly) and
// multiplied with v_mfma_f32_16x16x32_bf16, fp32 accumulation, fused with the
// argmax (or the logits scatter) as in the batch-1 kernel.  Page 3
// ("...MTP-NVFP4-h98k", "How it was built") gives the NVFP4 recipe, page 2
// the per-tensor E4M3 head; the batch-16 decode step of the 98 304-row head
// is the workload this kernel is shaped for.  Page 2's W8A8 step
// (_Fp8DraftHeadMethod.apply) runs the same kernel on E4M3 token codes and
// the head's E4M3 bytes as they are, with v_mfma_f32_16x16x32_fp8_fp8
// (format E4m3Fp8 in formats.h): no weight decode.
//
// MFMA operands (16x16x32, wave64):
//   A = h          lane l holds 8 BF16 of batch row m = l%16, k-slot group
//                  l/16;
//   B = weights^T  lane l holds 8 decoded weights of head row n = l%16, the
//                  same k-slot group;
//   D[m][n]        lane l, register j: m = 4*(l/16) + j, n = l%16.
// Which k a slot stands for is free as long as A and B agree, so each lane
// loads one 16-byte chunk of its own head row per step (chunk 4*step + l/16,
// 64 contiguous bytes per row per load instruction) and the A operand reads
// h at the matching k from LDS.  A chunk holds EPC/8 MFMA operands.
//
// Work: a wave owns units of RT row tiles (16 rows each) and walks the whole
// hidden dimension for each unit, one chunk per lane per tile per step.  (In
// the dense mode a small matrix has fewer units than the grid has waves:
// then ks = 2^ks_log2 waves of a block share a unit, each walks a contiguous
// part of its slots, and the block adds the parts through LDS, part 0 first.)  A
// ring of NB register slots of SPS steps each keeps NB-1 slots of loads in
// flight; the SPS loads of a tile are issued back to back so that DRAM sees
// SPS*64 contiguous bytes of each row at once.  h of the
// slice is staged once per block in LDS (row stride 2*hidden+16 bytes, so the
// 16 batch rows of a read fall on different banks), plus one zero row that
// the A-operand lanes of batch rows past the slice read.
#include "gemv_common.h"

namespace dh {
namespace {

// A work unit is RT 16-row tiles; a "slot" of the register ring holds SPS
// consecutive steps of every tile, loaded back to back so that each head row
// is read SPS*64 contiguous bytes at a time.
//
// Block scales (NVFP4): step c of a slot needs the two scale bytes of chunk
// 4c + q, 8 bytes apart from step to step.
//   * Four steps per slot (the NVFP4 shape): the slot's 32 scale bytes of a
//     row are 4 x 4 pairs, pair (c, q) at byte 8c + 2q.  Lane (n, q) loads
//     the 8 bytes 8q .. 8q+7, which are step q's pairs of the row's four
//     lanes, and a transpose over the wave's four 16-lane rows
//     (transpose_scale_pairs) hands each lane its own pairs of steps 0..3.
//     One 8-byte load per lane per slot, no byte loaded twice.
//   * Another even SPS: the slot's 8*SPS scale bytes of the lane's row are
//     loaded as SPS/2 16-byte pieces (the four lanes of a row load the same
//     pieces) and each step picks its two bytes out of them.
//   * An odd SPS loads them as one 16-bit value per step.
template <class F, int SPS>
constexpr bool pair_scales() {
  return F::SCALED && SPS == 4;
}
template <class F, int SPS>
constexpr bool wide_scales() {
  return F::SCALED && SPS % 2 == 0 && !pair_scales<F, SPS>();
}

template <class F, int RT, int SPS>
struct Slot {
  uint4 p[RT][SPS];
  uint32_t s[RT][F::SCALED && SPS % 2 == 1 ? SPS : 1];
  uint4 sw[RT][wide_scales<F, SPS>() ? SPS / 2 : 1];
  uint2 sp[RT];  // pair_scales: the lane's 8 bytes, as loaded
  // scatter modes: lane l holds dh_idx[r0 - 1 + min(l, 16)] of tile t (r0
  // its first row; row -1 reads row 0): the kept id before the tile, then
  // the tile's 16 ids.  The address depends on the lane, so this is a
  // vector load, which the prologue's wait count relies on.
  int32_t ids[RT];
};

// pair_scales: lane (n, q) holds v, bytes 8q .. 8q+7 of the slot's 32 scale
// bytes of head row n, which are pairs (q, 0..3), pair (c, r) being the two
// scale bytes of chunk 4c + r.  Returns pairs (0..3, q), the lane's own
// pairs of steps 0..3 (step c in half c%2 of word c/2): a 4x4 transpose of
// 16-bit values over the wave's four 16-lane rows.
//   1. v_permlane32_swap trades word 1 of rows 0, 1 for word 0 of rows 2, 3.
//      Rows 0, 1 then hold pairs (q, 0..1) in a and (q+2, 0..1) in b, rows
//      2, 3 pairs (q-2, 2..3) in a and (q, 2..3) in b.
//   2. In each row pair (0, 1) and (2, 3) the even row sends the high
//      halves of a and b and keeps the low ones, the odd row the reverse
//      (v_perm_b32 with the lane's selector sel.s); v_permlane16_swap trades
//      the sent words between the two rows, and two more v_perm_b32 put the
//      kept and the received halves in step order.
struct PairSel {
  uint32_t s, y0, y1;  // byte selectors of v_perm_b32 for this lane's row
  bool odd;            // the lane's row q is odd
};

__device__ __forceinline__ PairSel pair_selectors(int q) {
  const bool odd = (q & 1) != 0;
  // v_perm_b32(hi, lo, sel): selector byte i picks byte i of the result,
  // 0-3 from lo, 4-7 from hi
  return odd ? PairSel{0x05040100u, 0x03020504u, 0x03020706u, true}
             : PairSel{0x07060302u, 0x05040100u, 0x07060100u, false};
}

__device__ __forceinline__ uint2 transpose_scale_pairs(uint2 v,
                                                       const PairSel& sel) {
  const auto w = __builtin_amdgcn_permlane32_swap(v.x, v.y, false, false);
  const uint32_t a = w[0], b = w[1];
  const uint32_t s = __builtin_amdgcn_perm(b, a, sel.s);
  // odd rows of the first operand trade with even rows of the second: an
  // even row finds its partner's word in the second result, an odd row in
  // the first
  const auto x = __builtin_amdgcn_permlane16_swap(s, s, false, false);
  const uint32_t r = sel.odd ? x[0] : x[1];
  return make_uint2(__builtin_amdgcn_perm(r, a, sel.y0),
                    __builtin_amdgcn_perm(r, b, sel.y1));
}

// The two scale bytes of step C for a lane of k-slot group q.
template <class F, int RT, int SPS, int C>
__device__ __forceinline__ uint32_t slot_scale(const Slot<F, RT, SPS>& b,
                                               int t, int q) {
  if constexpr (wide_scales<F, SPS>()) {
    // bytes 8C + 2q: dword 2C + q/2, half q%2
    constexpr int D0 = 2 * C;
    const uint4 lo = b.sw[t][D0 / 4];
    const uint32_t w0 = (D0 % 4 == 0) ? lo.x : lo.z;
    const uint32_t w1 = (D0 % 4 == 0) ? lo.y : lo.w;
    const uint32_t w = (q & 2) ? w1 : w0;
    return (q & 1) ? (w >> 16) : (w & 0xFFFFu);
  } else if constexpr (F::SCALED) {
    return b.s[t][C];
  } else {
    return 0u;
  }
}

// Bytes of one staged h element: BF16, or an E4M3 code (W8A8).
template <class F>
constexpr int h_elem_bytes() {
  return F::FP8_ACT ? 1 : 2;
}

// The EPC/8 MFMAs of one step: operand O of every tile's chunk against the
// h slots O of the lane's chunk.  The chunk's scale bytes are bytes SB and
// SB + 1 of sc[t].
template <class F, int O, int RT, int SPS, int SB>
__device__ __forceinline__ void mfma_ops(const Slot<F, RT, SPS>& b, int c,
                                         const uint32_t (&sc)[RT],
                                         const char* hp, f32x4 (&acc)[RT]) {
  if constexpr (O < F::EPC / 8) {
    if constexpr (F::FP8_ACT) {
      // eight E4M3 codes of h against eight E4M3 weights
      const uint64_t av = *reinterpret_cast<const uint64_t*>(hp + 8 * O);
#pragma unroll
      for (int t = 0; t < RT; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(
            (long)av, (long)F::template operand8<O>(b.p[t][c]), acc[t], 0, 0,
            0);
    } else {
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(hp + 16 * O);
#pragma unroll
      for (int t = 0; t < RT; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            av, F::template operand<O, SB>(b.p[t][c], sc[t]), acc[t], 0, 0,
            0);
    }
    mfma_ops<F, O + 1, RT, SPS, SB>(b, c, sc, hp, acc);
  }
}

// The SPS steps of one slot (pr: the transposed scale pairs, pair_scales).
template <class F, int C, int RT, int SPS>
__device__ __forceinline__ void slot_steps(const Slot<F, RT, SPS>& b,
                                           const uint2 (&pr)[RT], int q,
                                           const char* hp, f32x4 (&acc)[RT]) {
  if constexpr (C < SPS) {
    uint32_t sc[RT];
    const char* hc = hp + C * (4 * F::EPC * h_elem_bytes<F>());
    if constexpr (pair_scales<F, SPS>()) {
#pragma unroll
      for (int t = 0; t < RT; ++t) sc[t] = C < 2 ? pr[t].x : pr[t].y;
      mfma_ops<F, 0, RT, SPS, 2 * (C % 2)>(b, C, sc, hc, acc);
    } else {
#pragma unroll
      for (int t = 0; t < RT; ++t) sc[t] = slot_scale<F, RT, SPS, C>(b, t, q);
      mfma_ops<F, 0, RT, SPS, 0>(b, C, sc, hc, acc);
    }
    slot_steps<F, C + 1, RT, SPS>(b, pr, q, hp, acc);
  }
}

// Logits of one 16-row tile (scatter modes), written by the whole wave: the
// id range the tile's kept rows own (owned_ids in gemv_common.h), each batch
// row's logit at its row's id and -inf between them.  Lane l holds
// id = dh_idx[r0 - 1 + min(l, 16)] (Slot::ids) and, in register j, the
// scaled logit of batch row 4(l/16) + j and tile row l%16 (the MFMA output
// layout).  For a position p of the range, the kept rows below it are
// counted against the tile's ids (ascending), which names the only row
// that can hold p; its logits come over with ds_bpermute.
template <int MODE>
__device__ __forceinline__ void scatter_tile(const KArgs& a, int64_t r0,
                                             int32_t id, const f32x4& val,
                                             int nb) {
  if (r0 >= a.n_kept) return;  // pad rows only
  const int64_t left = a.n_kept - r0;
  const int nk = left < 16 ? (int)left : 16;
  int32_t ids[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) ids[i] = __builtin_amdgcn_readlane(id, i + 1);
  const IdRange rg =
      owned_ids(r0, nk, __builtin_amdgcn_readlane(id, 0),
                __builtin_amdgcn_readlane(id, nk), a.n_kept, a.vocab);
  const int lane = (int)(threadIdx.x & 63);
  for (int64_t p0 = rg.lo; p0 < rg.hi; p0 += 64) {
    const int p = (int)(p0 + lane);  // vocab <= INT32_MAX
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) cnt += (i < nk && ids[i] < p) ? 1 : 0;
    const int c = cnt < 15 ? cnt : 15;
    // every ds_bpermute runs with the whole wave active: a lane reading from
    // a lane the exec mask left out would get 0
    const int at = __builtin_amdgcn_ds_bpermute(4 * (c + 1), id);
    const bool kept = cnt < nk && at == p;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      if (m < nb) {  // wave-uniform
        const float lv = __int_as_float(__builtin_amdgcn_ds_bpermute(
            4 * ((m >> 2) * 16 + c), __float_as_int(val[m & 3])));
        if (p < rg.hi)
          store_logit<MODE>(a.out_logits, (int64_t)m * a.vocab + p,
                            kept ? lv : not_kept_value<MODE>());
      }
    }
  }
}

template <class F, int RT, int SPS, int NB, int MODE, int NT>
__global__ __launch_bounds__(NT) void k_mfma(const KArgs a) {
  constexpr bool LOGITS = !is_top(MODE);
  constexpr int NW = NT / 64;
  constexpr int UR = 16 * RT;  // rows per unit
  extern __shared__ uint4 hs[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, q = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const FinishState st = LOGITS ? FinishState{} : finish_state(a);
  const int64_t hidden = a.hidden;
  const int nb = a.nb;

  // h [nb][hidden] and one zero row are staged in LDS; a row takes whole
  // 1 KB pieces plus 16 bytes (SB bytes), so the 16 batch rows of an A-operand
  // read fall on different banks.
  constexpr int HB = h_elem_bytes<F>();
  const int RBH = (int)(hidden * HB);  // h bytes per row
  const int PPR = (RBH + 1023) / 1024;
  const int SB = mfma_lds_row_bytes(hidden, HB);

  // Units are dealt to groups of ks waves, group-major (unit u goes to group
  // u / gridDim.x of block u % gridDim.x), so every block gets work even when
  // there are fewer units than groups in the grid.  Wave kp of a group takes
  // slots [js0, js1) of each of its units; with ks > 1 the host guarantees
  // at most one unit per group.
  const int kl = MODE == OUT_DENSE ? a.ks_log2 : 0;
  const int ks = 1 << kl;
  const int gw = wv >> kl, kp = wv & (ks - 1);
  const int64_t U = a.n_rows / UR;
  const int64_t TW = (int64_t)gridDim.x * (NW >> kl);
  const int64_t first = (int64_t)gw * gridDim.x + blockIdx.x;
  const int n_u = first < U ? (int)((U - first + TW - 1) / TW) : 0;
  const int64_t CPR = hidden / F::EPC;     // 16-byte chunks per row
  const int NSU = (int)(CPR / (4 * SPS));  // slots per unit
  const int js0 = (kp * NSU) >> kl, js1 = ((kp + 1) * NSU) >> kl;
  const int NS = js1 - js0;                // slots of this wave per unit
  const int n_s = n_u * NS;
  const int n_pad = (n_s + NB - 1) / NB * NB;
  const int64_t RB = CPR * 16;      // weight bytes per row
  const int64_t SPR = hidden / 16;  // scale bytes per row (NVFP4)

  // Per-lane constant parts of the addresses.
  uint32_t woff[RT], soff[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    woff[t] = (uint32_t)((16 * t + n) * RB + q * 16);
    soff[t] = (uint32_t)((16 * t + n) * SPR +
                         (wide_scales<F, SPS>()   ? 0
                          : pair_scales<F, SPS>() ? q * 8
                                                  : q * 2));
  }
  const PairSel psel = pair_selectors(q);
  // A-operand LDS address of this lane at step 0: batch row min(m, nb)
  // (row nb is zero), chunk q.
  const int mrow = n < nb ? n : nb;
  const uint32_t hoff = (uint32_t)(mrow * SB + q * F::EPC * HB);
  const char* hsb = reinterpret_cast<const char*>(hs);

  // Scalar cursor over (unit, slot) pairs: first row of the unit, slot.
  int64_t ld_row0 = (n_u > 0 ? first : 0) * UR;
  int ld_js = js0, ld_count = 0;
  const int64_t unit_stride = TW * UR;
  auto load = [&](Slot<F, RT, SPS>& b) {
    // The cursor is passed through an opaque asm so that the compiler never
    // folds the repeated loads of a clamped cursor into copies: the prologue
    // wait below counts on every slot load being issued.
    int64_t row0 = ld_row0;
    int js = ld_js;
    asm volatile("" : "+s"(row0), "+s"(js));
    const uint8_t* wb = a.w + row0 * RB + (int64_t)js * (64 * SPS);
    const uint8_t* sb = a.scales + row0 * SPR + (int64_t)js * (8 * SPS);
    // pair scales first: the transpose needs only them, so it can run while
    // the slot's code loads are still arriving
    if constexpr (pair_scales<F, SPS>()) {
#pragma unroll
      for (int t = 0; t < RT; ++t)
        b.sp[t] = *reinterpret_cast<const uint2*>(sb + soff[t]);
    }
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int c = 0; c < SPS; ++c)
        b.p[t][c] = *reinterpret_cast<const uint4*>(wb + woff[t] + 64 * c);
    if constexpr (F::SCALED && !pair_scales<F, SPS>()) {
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int c = 0; c < SPS; ++c)
          if constexpr (wide_scales<F, SPS>()) {
            if (c < SPS / 2)
              b.sw[t][c] =
                  *reinterpret_cast<const uint4*>(sb + soff[t] + 16 * c);
          } else {
            b.s[t][c] =
                *reinterpret_cast<const uint16_t*>(sb + soff[t] + 8 * c);
          }
    }
    if constexpr (is_scatter(MODE)) {
      const int64_t l = lane < 16 ? lane : 16;
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const int64_t j = row0 + 16 * t - 1 + l;
        b.ids[t] = a.dh_idx[j > 0 ? j : 0];
      }
    }
    // The cursor stops at the wave's last slot: the surplus loads of the
    // padded ring re-read it (L2 hits) and are never computed.
    if (ld_count + 1 < n_s) {
      ++ld_count;
      if (++ld_js == js1) {
        ld_js = js0;
        ld_row0 += unit_stride;
      }
    }
  };

  f32x4 acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // Logits factor of batch row 4q + j (rows past the slice are never
  // written): the tensor scale times the row's own scale.  Both are loaded
  // here and first used when a unit completes (lane_scales), so their
  // latency hides behind the loop instead of delaying the first loads.
  const float tsc = MODE != OUT_TOP ? tensor_scale(a) : 1.0f;
  float rsc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = 4 * q + j < nb ? 4 * q + j : nb - 1;
    rsc[j] = MODE != OUT_TOP && a.row_scale ? a.row_scale[m] : 1.0f;
  }
  // (the empty asm keeps the compiler from forming the products, and so
  // waiting for the loads, before the loop)
  auto lane_scales = [&](float (&lsc)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float t = tsc, r = rsc[j];
      asm volatile("" : "+v"(t), "+v"(r));
      lsc[j] = t * r;
    }
  };
  float best_v[4];
  int best_r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    best_v[j] = -INFINITY;
    best_r[j] = INT_MAX;
  }

  // Prologue.  h goes straight into LDS with global_load_lds_dwordx4 (a
  // wave copies 1 KB pieces: lane i's 16 bytes land at M0 + 16 i; lanes past
  // the end of a row re-read its last 16 bytes into the row's padding), the
  // zero row is written, and the first weight slots are issued, so the
  // staging overlaps their latency.  Memory loads retire in issue order:
  // once no more than the weight loads are outstanding, this wave's copies
  // have landed; the barrier then covers every wave's.  (The wait is
  // explicit, see lds_copy_x4; a __syncthreads fence would also wait for the
  // weight loads.)
  {
    const char* hb = reinterpret_cast<const char*>(a.h);
    const uint32_t lds_base = lds_addr(hs);
    const int pieces = nb * PPR;
    for (int pc = wv; pc < pieces; pc += NW) {
      const int r = pc / PPR, j = pc - r * PPR;
      const int off = j * 1024 + 16 * lane;
      const int src = off < RBH ? off : RBH - 16;
      lds_copy_x4(hb + (int64_t)r * RBH + src,
                  lds_base + (uint32_t)(r * SB + j * 1024));
    }
    uint4* zrow = hs + nb * (SB / 16);
    for (int i = threadIdx.x; i < SB / 16; i += NT)
      zrow[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  // Every wave has issued its copies before any wave issues weight loads:
  // the CU's memory pipeline serves requests in order, so the copies (L2
  // hits) do not queue behind the block's first HBM reads.
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  Slot<F, RT, SPS> buf[NB];
#pragma unroll
  for (int k = 0; k < NB - 1; ++k) load(buf[k]);
  constexpr int SCALE_LOADS = pair_scales<F, SPS>()   ? 1
                              : wide_scales<F, SPS>() ? SPS / 2
                              : F::SCALED             ? SPS
                                                      : 0;
  constexpr int WEIGHT_LOADS =
      (NB - 1) * (RT * (SPS + SCALE_LOADS) + (is_scatter(MODE) ? RT : 0));
  static_assert(WEIGHT_LOADS <= 63, "vmcnt field is 6 bits");
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(WEIGHT_LOADS)
               : "memory");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  int64_t cp_row0 = (n_u > 0 ? first : 0) * UR;
  int cp_js = js0;
  for (int s0 = 0; s0 < n_pad; s0 += NB) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      load(buf[(k + NB - 1) % NB]);
      __builtin_amdgcn_sched_barrier(0);
      if (s0 + k < n_s) {  // wave-uniform
        const Slot<F, RT, SPS>& b = buf[k];
        uint2 pr[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t)
          pr[t] = pair_scales<F, SPS>() ? transpose_scale_pairs(b.sp[t], psel)
                                        : make_uint2(0u, 0u);
        slot_steps<F, 0, RT, SPS>(
            b, pr, q, hsb + hoff + cp_js * SPS * (4 * F::EPC * HB), acc);
        if (cp_js == js1 - 1) {
          // unit done: rows row0 + 16t + n, batch rows 4q + j (a split
          // unit's parts are added after the loop)
          float lsc[4];
          lane_scales(lsc);
          if constexpr (is_scatter(MODE)) {
#pragma unroll
            for (int t = 0; t < RT; ++t) {
              f32x4 sv;
#pragma unroll
              for (int j = 0; j < 4; ++j) sv[j] = acc[t][j] * lsc[j];
              scatter_tile<MODE>(a, cp_row0 + 16 * t, b.ids[t], sv, nb);
              acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
          }
#pragma unroll
          for (int t = 0; t < RT && ks == 1 && !is_scatter(MODE); ++t) {
            const int64_t row = cp_row0 + 16 * t + n;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float v = acc[t][j];
              if constexpr (MODE == OUT_DENSE) {
                const int m = 4 * q + j;
                if (m < nb && row < a.n_kept)
                  store_logit<MODE>(a.out_logits, (int64_t)m * a.vocab + row,
                                    v * lsc[j]);
              } else {
                const float c = top_value<MODE>(v, lsc[j]);
                if (c > best_v[j]) {
                  // a lane's rows ascend: strict > keeps the lowest
                  best_v[j] = c;
                  best_r[j] = (int)row;
                }
              }
            }
            acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
          }
          cp_js = js0;
          cp_row0 += unit_stride;
        } else {
          ++cp_js;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if constexpr (MODE == OUT_DENSE) {
    if (ks > 1) {  // block-uniform
      // Every wave is done with h: its LDS takes the partial tiles.
      __syncthreads();
      f32x4* red = reinterpret_cast<f32x4*>(hs);
#pragma unroll
      for (int t = 0; t < RT; ++t) red[(wv * RT + t) * 64 + lane] = acc[t];
      __syncthreads();
      if (kp == 0 && n_u > 0) {
        float lsc[4];
        lane_scales(lsc);
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          f32x4 v = acc[t];
          for (int p = 1; p < ks; ++p) {
            const f32x4 o = red[((wv + p) * RT + t) * 64 + lane];
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] += o[j];
          }
          const int64_t row = first * UR + 16 * t + n;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int m = 4 * q + j;
            if (m < nb)
              a.out_logits[(int64_t)m * a.vocab + row] = v[j] * lsc[j];
          }
        }
      }
    }
  }
  if constexpr (!LOGITS) {
    // batch row b lives in register b%4 of the lanes with l/16 == b/4
    // one slot per thread: the grid is one block (512 or 1024 threads) per
    // CU
    argmax_finish_rows<NT, 1>(best_v, best_r, a, st);
  }
}

// Launch shape: one 16-row tile per unit, a double-buffered ring of slots,
// one block per CU (the h slice fills most of the LDS; see desc), 512
// threads (two waves per SIMD, 256 VGPRs each).
//   * NVFP4: slots of four steps.  On the 98K head at batch 16 this is 7%
//     faster than 1024 threads: the 6144 tiles then make three units for
//     every wave instead of one and a half, and the extra waves bought no
//     latency cover.  768 threads (two units per wave), a third ring slot
//     and slots of ten steps measured the same or slower.
//   * E4M3 and BF16 (and the W8A8 codes): slots of ten steps (ten 1 KB
//     loads per slot), 2% faster than the NVFP4 shape on the 98K E4M3 head.
constexpr int MFMA_RT = 1;
constexpr int MFMA_NB = 2;

template <class F>
struct MfmaShape {
  static constexpr int THREADS = 512;
  static constexpr int SPS = 10;  // preferred steps per slot
};
template <>
struct MfmaShape<Nvfp4> {
  static constexpr int THREADS = 512;
  static constexpr int SPS = 4;
};

// steps = hidden / (4 * EPC), the MFMA steps of a unit.
template <class F, int SPS, int L>
KernelDesc desc(int64_t steps) {
  constexpr int NT = MfmaShape<F>::THREADS;
  // one block per CU: the units are dealt over the grid's waves, and a
  // second block (which fits when h is staged as one-byte codes) would
  // leave the waves of the 98K head with one and a half units each
  return KernelDesc{
      reinterpret_cast<const void*>(k_mfma<F, MFMA_RT, SPS, MFMA_NB, L, NT>),
      NT, 16 * MFMA_RT, 0, true, L == OUT_DENSE ? (int)(steps / SPS) : 0, 1};
}

// Steps per slot: the format's preferred size if it divides the steps of a
// unit, else the largest of 10, 4, 2, 1 that does.
template <class F, int L>
KernelDesc desc_for(int64_t steps) {
  constexpr int P = MfmaShape<F>::SPS;
  if (steps % P == 0) return desc<F, P, L>(steps);
  if (steps % 10 == 0) return desc<F, 10, L>(steps);
  if (steps % 4 == 0) return desc<F, 4, L>(steps);
  if (steps % 2 == 0) return desc<F, 2, L>(steps);
  return desc<F, 1, L>(steps);
}

// The dense mode (the linear) and the BF16 modes exist for NVFP4 only; an
// absent kernel is an empty descriptor.
template <class F, int L>
constexpr bool has_mode() {
  return F::kFmt == FMT_NVFP4 || L == OUT_TOP || L == OUT_SCATTER;
}

template <class F, int L>
KernelDesc desc_mode(bool one_step, int64_t steps) {
  if constexpr (has_mode<F, L>())
    return one_step ? desc<F, 1, L>(steps) : desc_for<F, L>(steps);
  return KernelDesc{nullptr, 0, 0, 0, false};
}

template <class F>
bool pick(int64_t hidden, int nb, int mode, int lds_per_block,
          KernelDesc* d) {
  constexpr int HB = h_elem_bytes<F>();
  if (hidden % (4 * F::EPC) != 0) return false;
  if (nb < 1 || nb > mfma_max_slice(hidden, lds_per_block, HB)) return false;
  const int64_t steps = hidden / (4 * F::EPC);
  // 16-byte scale pieces need 16-byte aligned scale rows; otherwise one step
  // per slot (the odd slot size loads the scales as 16-bit values)
  const bool one = F::SCALED && (hidden / 16) % 16 != 0;
  switch (mode) {
    case OUT_TOP: *d = desc_mode<F, OUT_TOP>(one, steps); break;
    case OUT_SCATTER: *d = desc_mode<F, OUT_SCATTER>(one, steps); break;
    case OUT_DENSE: *d = desc_mode<F, OUT_DENSE>(one, steps); break;
    case OUT_TOP_BF16: *d = desc_mode<F, OUT_TOP_BF16>(one, steps); break;
    case OUT_SCATTER_BF16:
      *d = desc_mode<F, OUT_SCATTER_BF16>(one, steps);
      break;
    default: return false;
  }
  if (!d->fn) return false;
  d->lds_bytes = (size_t)(nb + 1) * (size_t)mfma_lds_row_bytes(hidden, HB);
  d->fp8_act = F::FP8_ACT;
  if (mode == OUT_DENSE) {
    // a split unit's parts are added through LDS: one f32x4 per lane and
    // tile of every wave
    const size_t red = (size_t)d->threads * MFMA_RT * 16;
    if (d->lds_bytes < red) d->lds_bytes = red;
  }
  return true;
}

}  // namespace

int mfma_max_slice(int64_t hidden, int lds_per_block, int h_bytes) {
  const int64_t row = mfma_lds_row_bytes(hidden, h_bytes);
  // the kernels' static LDS (the finish's tables) comes out of the same
  // budget as the h slice
  int64_t nb = ((int64_t)lds_per_block - MFMA_STATIC_LDS) / row - 1;
  if (nb > 16) nb = 16;
  return nb < 0 ? 0 : (int)nb;
}

bool mfma_kernel(int fmt, int64_t hidden, int nb, int mode,
                 int lds_per_block, bool fp8_act, KernelDesc* out) {
  if (fp8_act)  // the W8A8 step: an E4M3 head only
    return fmt == FMT_E4M3 &&
           pick<E4m3Fp8>(hidden, nb, mode, lds_per_block, out);
  switch (fmt) {
    case FMT_NVFP4: return pick<Nvfp4>(hidden, nb, mode, lds_per_block, out);
    case FMT_E4M3: return pick<E4m3>(hidden, nb, mode, lds_per_block, out);
    case FMT_BF16: return pick<Bf16>(hidden, nb, mode, lds_per_block, out);
  }
  return false;
}

}  // namespace dh
