"""The pages' own numerics (page 1, "q38_draft.py": the install step takes
a BF16 or FP16 head and the drafter's linear returns BF16, which
get_top_tokens hands to argmax; page 2, compute_logits scatters in that
dtype), GPU against the oracle through the C-ABI.

* FP16 head: codes, scales and gs bit-exact.
* Top tokens over the logits rounded to BF16 (global scale applied), lowest
  row on ties: equal to the oracle's id, or a documented exception where the
  two rows' float64 logits lie within the float32 logit tolerance; and equal
  to the first maximum of the GPU's own BF16 logits, bit for bit.
* BF16 logits: every value equals the oracle's BF16 rounding of its float32
  logit, except where the float64 logit lies within FP32_ERR of a BF16
  rounding boundary (then either neighbour passes).  FP32_ERR bounds the
  float32 GEMV's error against the float64 oracle with room to spare: the
  fp32 logit tests measure at most 2e-6 on logits of size ~5.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import reduced_vocab_nvfp4_amd as dh
from reduced_vocab_nvfp4_amd import workloads as wl
from tests import helpers as H
from tests.test_gpu_parity import head

pytestmark = pytest.mark.gpu
DEV = "cuda"
FP32_ERR_ABS, FP32_ERR_REL = 1e-5, 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _f16_bits(w: torch.Tensor) -> np.ndarray:
    return w.cpu().view(torch.int16).numpy().view(np.uint16)


def _f16_case(w16, idx, tag):
    p, s, g = dh.nvfp4_quantize_rows(w16.to(DEV), torch.from_numpy(idx).to(DEV))
    op, os_, og = oracle.nvfp4_quantize_f16(_f16_bits(w16), idx)
    say(f"[f16 quantize] {tag}: rows={idx.shape[0]}")
    assert np.float32(g.item()) == og, tag
    sn, pn = s.cpu().numpy(), p.cpu().numpy()
    assert np.array_equal(sn, os_), (tag, np.argwhere(sn != os_)[:5])
    assert np.array_equal(pn, op), (tag, np.argwhere(pn != op)[:5])
    return p, s, g, (op, os_, og)


@pytest.mark.parametrize("name", ["tiny", "flash_next_64k"])
def test_f16_head_quantize_bit_exact(name):
    hd = head(name)
    _f16_case(hd.w.to(torch.float16), hd.idx_o, name)


def test_f16_quantize_edge_cases():
    """FP16 subnormals down to 2^-24, the largest value 65504, signed zeros,
    an all-zero head (the floor), and a ragged gather with repeats."""
    rng = np.random.default_rng(31)
    x = rng.standard_normal((128, 64)) * np.exp2(rng.integers(-20, 8, (128, 1)))
    x[0, 0] = 65504.0
    x[1, :4] = [2.0 ** -24, -(2.0 ** -24), 3 * 2.0 ** -24, -0.0]
    x[2] = 0.0
    w16 = torch.from_numpy(x.astype(np.float16))
    _f16_case(w16, np.arange(128, dtype=np.int32), "wide range")
    _f16_case(torch.zeros((64, 32), dtype=torch.float16),
              np.arange(64, dtype=np.int32), "all-zero head")
    idx = np.concatenate([rng.permutation(128)[:50],
                          np.full(14, 3)]).astype(np.int32)
    _f16_case(w16, idx, "ragged gather with repeats")


def _oracle_compat(hd_o, h):
    """float64 logits and their BF16 bits as the pages' linear rounds them."""
    L = oracle.nvfp4_logits(*hd_o, wl.bf16_bits(h))
    return L, oracle.logits_to_bf16(L)


def _first_max_rows(vals: np.ndarray) -> np.ndarray:
    return np.argmax(vals, axis=1)  # numpy: the first maximal index


def _check_compat_top(ids, L, Lb, idx, n_kept, row_scale):
    """Returns (exceptions, ties): ties counts batch rows whose BF16 maximum
    is shared by several kept rows (decided by the lowest-row rule).  The
    absolute part of the tolerance scales with the batch row's scale (the
    float32 error of a logit is proportional to the magnitude of h)."""
    vals = oracle.bf16_bits_value(Lb)
    rows = _first_max_rows(vals)
    exc = ties = 0
    for b in range(L.shape[0]):
        top = vals[b].max()
        if (vals[b, :n_kept] == top).sum() > 1:
            ties += 1
        if int(ids[b]) == int(idx[rows[b]]):
            continue
        r = np.flatnonzero(idx[:n_kept] == int(ids[b]))
        assert r.size == 1, f"batch {b}: id {ids[b]} is not a kept id"
        lw, lg = L[b, rows[b]], L[b, r[0]]
        assert abs(lw - lg) <= H.ATOL * row_scale[b] + H.RTOL * abs(lw), (
            f"batch {b}: got id {ids[b]} (logit {lg}), want {idx[rows[b]]} "
            f"(logit {lw})")
        exc += 1
    return exc, ties


def _check_compat_logits(out_bits, L, idx, n_kept, vocab, tag, row_scale):
    """out_bits: GPU BF16 [B, V] as uint16; row_scale [B] as in
    _check_compat_top."""
    Lb = oracle.logits_to_bf16(L)
    ref = oracle.logits_scatter_bf16(Lb, n_kept, idx, vocab)
    bad = out_bits != ref
    if bad.any():
        # a value may differ only where the float64 logit is within the
        # float32 error of a BF16 rounding boundary: it must then be a BF16
        # value between the roundings of L - err and L + err (near zero that
        # window holds several)
        err = FP32_ERR_ABS * row_scale[:, None] + FP32_ERR_REL * np.abs(L)
        lo = oracle.bf16_bits_value(oracle.logits_scatter_bf16(
            oracle.logits_to_bf16(L - err), n_kept, idx, vocab))
        hi = oracle.bf16_bits_value(oracle.logits_scatter_bf16(
            oracle.logits_to_bf16(L + err), n_kept, idx, vocab))
        got = oracle.bf16_bits_value(out_bits)
        ok = (got >= lo) & (got <= hi)
        assert ok[bad].all(), (tag, np.argwhere(bad & ~ok)[:5])
    say(f"[compat logits] {tag}: {int(bad.sum())} boundary values of "
        f"{out_bits.size}")
    assert ((out_bits == 0xFF80).sum(axis=1) == vocab - n_kept).all()


def _compat_case(hd, h, tag, packed=None, scales=None, gs=None, o=None,
                 row_scale=None):
    packed = hd.packed if packed is None else packed
    scales = hd.scales if scales is None else scales
    gs = hd.gs if gs is None else gs
    o = (hd.o_packed, hd.o_scales, hd.o_gs) if o is None else o
    hg = h.to(DEV)
    ids = dh.draft_head_top_tokens_compat(packed, scales, gs, hd.idx_gpu,
                                          hg).cpu().numpy()
    out = dh.draft_head_logits_compat(packed, scales, gs, hd.idx_gpu,
                                      hd.n_kept, hd.vocab, hg)
    bits = out.cpu().view(torch.int16).numpy().view(np.uint16)
    L, Lb = _oracle_compat(o, h)
    rs = np.ones(h.shape[0]) if row_scale is None else np.asarray(row_scale)
    exc, ties = _check_compat_top(ids, L, Lb, hd.idx_o, hd.n_kept, rs)
    # the top token is the first maximum of the GPU's own BF16 logits
    kept_vals = oracle.bf16_bits_value(bits[:, hd.idx_o[:hd.n_kept]])
    assert np.array_equal(ids, hd.idx_o[:hd.n_kept][_first_max_rows(kept_vals)])
    _check_compat_logits(bits, L, hd.idx_o, hd.n_kept, hd.vocab, tag, rs)
    say(f"[compat top] {tag}: B={h.shape[0]} exceptions={exc} "
        f"bf16 ties at the top={ties}")
    return exc


@pytest.mark.parametrize("B", [1, 5, 16, 33])
def test_compat_tiny(B):
    hd = head("tiny")
    assert _compat_case(hd, wl.hidden_states(B, hd.hidden, 300 + B),
                        f"tiny B={B}") == 0


def test_compat_flash_b1():
    hd = head("flash_next_64k")
    exc = sum(_compat_case(hd, wl.hidden_states(1, hd.hidden, 310 + s),
                           f"flash s{s}") for s in range(3))
    assert exc <= 1


def test_compat_h98k_b16():
    hd = head("h98k_b16")
    assert _compat_case(hd, wl.hidden_states(16, hd.hidden, 320),
                        "h98k B=16") <= 1


def test_compat_f16_head_end_to_end():
    """An FP16 head quantized on the GPU, then the BF16-rounded step."""
    hd = head("flash_next_64k")
    w16 = hd.w.to(torch.float16)
    p, s, g, o = _f16_case(w16, hd.idx_o, "flash as FP16")
    assert _compat_case(hd, wl.hidden_states(4, hd.hidden, 330), "flash FP16 B=4",
                        packed=p, scales=s, gs=g, o=o) <= 1


def test_compat_ties_take_the_lowest_row():
    """A BF16 tie that float32 breaks the other way: row 0 becomes a copy of
    the winning row with one element halved, chosen (on the oracle) so that
    its float32 logit is just below the winner's but rounds to the same
    BF16 value.  The BF16 argmax must return row 0's id, the float32 argmax
    the winner's."""
    hd = head("tiny")
    h = wl.hidden_states(1, hd.hidden, 340)
    best = int(np.argmax(hd.oracle_logits(h)[0]))
    assert best > 0
    src, dst = int(hd.idx_o[best]), int(hd.idx_o[0])
    found = None
    for k in range(hd.hidden):
        w = hd.w.clone()
        w[dst] = w[src]
        w[dst, k] = w[src, k] * 0.5
        o = oracle.nvfp4_quantize(wl.bf16_bits(w), hd.idx_o)
        Lo = oracle.nvfp4_logits(*o, wl.bf16_bits(h))[0]
        Lb = oracle.bf16_bits_value(oracle.logits_to_bf16(Lo))
        f32 = Lo.astype(np.float32)
        if (Lb[0] == Lb.max() and Lb[best] == Lb[0] and
                int(np.argmax(Lo)) == best and f32[0] < f32[best] and
                Lo[best] - Lo[0] > 1e-4):
            found = (k, w)
            break
    assert found is not None, "no element gives a BF16-only tie"
    k, w = found
    say(f"[compat tie] element {k} of row 0 halved")
    p, sc, g = dh.nvfp4_quantize_rows(w.to(DEV), hd.idx_gpu)
    hg = h.to(DEV)
    assert int(dh.draft_head_top_tokens_compat(p, sc, g, hd.idx_gpu, hg)
               .item()) == dst
    assert int(dh.draft_head_top_tokens(p, sc, g, hd.idx_gpu, hg)
               .item()) == src


@pytest.mark.parametrize("hid", [48, 272])
def test_compat_generic_kernel(hid):
    """Hidden sizes no batch-1 or MFMA shape tiles run the generic kernel,
    in both BF16 modes, at batch 1, 3 and 9 (slices of 8 and 1)."""
    from tests.test_gpu_parity import Head
    hd = Head("tiny", hidden=hid)
    for B in (1, 3, 9):
        assert _compat_case(hd, wl.hidden_states(B, hid, 350 + B),
                            f"generic H={hid} B={B}") == 0
