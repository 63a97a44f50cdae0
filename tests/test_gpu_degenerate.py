"""Degenerate inputs of the draft-head step, GPU against the oracle through
the C-ABI, at full head sizes in the launch configurations the library picks
(batch-1 kernel, MFMA slices):

* Zero hidden states, signed zeros mixed in.  Every logit is zero and the
  whole head ties, so every step kind must return the first kept id: the
  lowest row wins a tie (page 1, get_top_tokens takes the first maximal
  index).  Logits are zero at the kept ids, -inf elsewhere; the linear's
  output is zero.
* One-hot hidden states.  Each logit is one exact product (a dequantized
  weight times one BF16 value) scaled once in float32, so the GPU's float32
  logits equal the oracle's rounded to float32, and the maximum is shared by
  rows that lie far apart in the head (different blocks of the grid).  Ids
  must equal the oracle's lowest row with no tolerance, in the float32 and
  the BF16-rounded modes and for the E4M3 head (W8A16 and W8A8).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import reduced_vocab_nvfp4_amd as dh
from reduced_vocab_nvfp4_amd import workloads as wl
from tests import helpers as H
from tests.test_gpu_formats import _index, _logits_ok, e4m3_head
from tests.test_gpu_parity import head

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _zero_h(B, hidden):
    h = torch.zeros(B, hidden, dtype=torch.bfloat16)
    h[:, 1::2] = -0.0
    bits = wl.bf16_bits(h)
    assert (bits[:, 1::2] == 0x8000).all() and (bits[:, 0::2] == 0).all()
    return h


def _one_hot_h(B, hidden):
    """Row b is zero but for one element: positions spread over the hidden
    dimension (both ends, block edges), values of both signs."""
    pos = [0, hidden - 1, 1, 17, 15, 16, 31, 32, hidden // 2, hidden // 3,
           2, 3, hidden - 16, hidden - 17, 640 % hidden, 1919 % hidden]
    val = [1.0, -1.0, 0.375, -3.0]
    h = torch.zeros(B, hidden, dtype=torch.bfloat16)
    for b in range(B):
        h[b, pos[b % len(pos)]] = val[b % len(val)] * (1 + b // len(pos))
    return h


def _bf16_out_bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _unsigned_zero(bits):
    return np.where((bits & 0x7FFF) == 0, 0, bits)


def _first_max_ids(vals, idx, n_kept):
    """Target id of the first maximum over the kept rows of each row of
    vals (float64 [B, n_rows])."""
    rows, ids = oracle.argmax_remap(vals[:, :n_kept], idx[:n_kept])
    return ids


@pytest.mark.parametrize("name,B", [("tiny", 1), ("tiny", 5),
                                    ("flash_next_64k", 1),
                                    ("flash_next_64k", 16)])
def test_zero_hidden_state_nvfp4_every_step_kind(name, B):
    hd = head(name)
    h = _zero_h(B, hd.hidden)
    hg = h.to(DEV)
    L = hd.oracle_logits(h)
    rows, want = oracle.argmax_remap(L, hd.idx_o)
    assert (L == 0).all() and (rows == 0).all() and (want == hd.idx_o[0]).all()
    ids = dh.draft_head_top_tokens(hd.packed, hd.scales, hd.gs, hd.idx_gpu, hg)
    assert np.array_equal(ids.cpu().numpy(), want), ids
    kept = hd.idx_o[:hd.n_kept]
    out = dh.draft_head_logits(hd.packed, hd.scales, hd.gs, hd.idx_gpu,
                               hd.n_kept, hd.vocab, hg).cpu().numpy()
    _logits_ok(out, oracle.logits_scatter(L, hd.n_kept, hd.idx_o, hd.vocab),
               f"{name} zero h B={B}")
    assert (out[:, kept] == 0).all()
    ids_b = dh.draft_head_top_tokens_compat(hd.packed, hd.scales, hd.gs,
                                            hd.idx_gpu, hg)
    assert np.array_equal(ids_b.cpu().numpy(), want), ids_b
    bits = _bf16_out_bits(dh.draft_head_logits_compat(
        hd.packed, hd.scales, hd.gs, hd.idx_gpu, hd.n_kept, hd.vocab, hg))
    assert ((bits[:, kept] & 0x7FFF) == 0).all()
    assert ((bits == 0xFF80).sum(axis=1) == hd.vocab - hd.n_kept).all()
    y = dh.nvfp4_linear(hd.packed, hd.scales, hd.gs, hg).cpu().numpy()
    assert y.shape == (B, hd.n_rows) and (y == 0).all()
    say(f"[zero h] {name} B={B}: every step kind returns id {want[0]}")


@pytest.mark.parametrize("B", [1, 16])
def test_zero_hidden_state_e4m3_w8a8_and_bf16_heads(B):
    e4 = e4m3_head("tiny")
    h = _zero_h(B, e4.hidden)
    hg = h.to(DEV)
    first = np.full(B, e4.idx[0], dtype=np.int32)
    ids = dh.draft_head_top_tokens_e4m3(e4.q, e4.scale, e4.idx_gpu, hg)
    assert np.array_equal(ids.cpu().numpy(), first)
    # W8A8: a zero row quantizes with the 1e-12 floor to zero codes
    qx, sx = oracle.fp8_tokens_quantize(wl.bf16_bits(h))
    L8 = oracle.w8a8_logits(e4.o_q, e4.o_scale, qx, sx)
    _, want8 = oracle.argmax_remap(L8, e4.idx)
    assert (L8 == 0).all() and np.array_equal(want8, first)
    ids8 = dh.draft_head_top_tokens_w8a8(e4.q, e4.scale, e4.idx_gpu, hg)
    assert np.array_equal(ids8.cpu().numpy(), first)
    out8 = dh.draft_head_logits_w8a8(e4.q, e4.scale, e4.idx_gpu, e4.n_kept,
                                     e4.vocab, hg).cpu().numpy()
    assert (out8[:, e4.idx[:e4.n_kept]] == 0).all()
    # BF16 head of gathered rows
    idx, n_kept = _index("tiny")
    w = H.head_weight(4096, 256)
    rows = w[torch.from_numpy(idx.astype(np.int64))].contiguous().to(DEV)
    idx_g = torch.from_numpy(idx).to(DEV)
    ids16 = dh.draft_head_top_tokens_bf16(rows, idx_g, _zero_h(B, 256).to(DEV))
    assert np.array_equal(ids16.cpu().numpy(), np.full(B, idx[0], np.int32))
    say(f"[zero h] E4M3 W8A16, W8A8 and BF16 heads B={B}: id {idx[0]}")


@pytest.mark.parametrize("name,B", [("flash_next_64k", 1),
                                    ("flash_next_64k", 4),
                                    ("h98k_b16", 16)])
def test_one_hot_hidden_states_nvfp4_exact(name, B):
    """At batch 1, four single rows in turn (the batch-1 kernel); otherwise
    one batch of B rows."""
    hd = head(name)
    h = _one_hot_h(max(B, 4), hd.hidden)
    hs = [h[b:b + 1] for b in range(4)] if B == 1 else [h]
    ties = sum((_one_hot_nvfp4_case(hd, x, name) for x in hs), [])
    assert max(ties) >= 2


def _one_hot_nvfp4_case(hd, h, name):
    B = h.shape[0]
    hg = h.to(DEV)
    L = hd.oracle_logits(h)
    kept = hd.idx_o[:hd.n_kept]
    want = _first_max_ids(L, hd.idx_o, hd.n_kept)
    ties = [int((L[b, :hd.n_kept] == L[b, :hd.n_kept].max()).sum())
            for b in range(B)]
    say(f"[one-hot] {name} B={B}: rows at the maximum {ties}")
    ids = dh.draft_head_top_tokens(hd.packed, hd.scales, hd.gs, hd.idx_gpu,
                                   hg).cpu().numpy()
    assert np.array_equal(ids, want), (ids, want)
    # float32 logits: the oracle's value rounded once
    out = dh.draft_head_logits(hd.packed, hd.scales, hd.gs, hd.idx_gpu,
                               hd.n_kept, hd.vocab, hg).cpu().numpy()
    ref = oracle.logits_scatter(L, hd.n_kept, hd.idx_o, hd.vocab)
    assert np.array_equal(out[:, kept], ref[:, kept]), name
    assert (out.view(np.uint32)[~np.isfinite(ref)] == 0xFF800000).all()
    # BF16-rounded mode: ties widen, the lowest row still wins
    Lb = oracle.bf16_bits_value(oracle.logits_to_bf16(L))
    want_b = _first_max_ids(Lb, hd.idx_o, hd.n_kept)
    ids_b = dh.draft_head_top_tokens_compat(hd.packed, hd.scales, hd.gs,
                                            hd.idx_gpu, hg).cpu().numpy()
    assert np.array_equal(ids_b, want_b), (ids_b, want_b)
    bits = _bf16_out_bits(dh.draft_head_logits_compat(
        hd.packed, hd.scales, hd.gs, hd.idx_gpu, hd.n_kept, hd.vocab, hg))
    ref_b = oracle.logits_scatter_bf16(oracle.logits_to_bf16(L), hd.n_kept,
                                       hd.idx_o, hd.vocab)
    # a zero product may carry either sign on either side
    assert np.array_equal(_unsigned_zero(bits), _unsigned_zero(ref_b))
    # the linear: every output is one rounded product
    y = dh.nvfp4_linear(hd.packed, hd.scales, hd.gs, hg).cpu().numpy()
    assert np.array_equal(y, L.astype(np.float32))
    return ties


@pytest.mark.parametrize("B", [1, 16])
def test_one_hot_hidden_states_e4m3_exact(B):
    e4 = e4m3_head("h98k_b16")
    h = _one_hot_h(max(B, 4), e4.hidden)[3 if B == 1 else 0:][:B]
    hg = h.to(DEV)
    L = e4.oracle_logits(h)
    ids = dh.draft_head_top_tokens_e4m3(e4.q, e4.scale, e4.idx_gpu,
                                        hg).cpu().numpy()
    assert np.array_equal(ids, _first_max_ids(L, e4.idx, e4.n_kept))
    qx, sx = oracle.fp8_tokens_quantize(wl.bf16_bits(h))
    L8 = oracle.w8a8_logits(e4.o_q, e4.o_scale, qx, sx)
    want8 = _first_max_ids(L8, e4.idx, e4.n_kept)
    ids8 = dh.draft_head_top_tokens_w8a8(e4.q, e4.scale, e4.idx_gpu,
                                         hg).cpu().numpy()
    assert np.array_equal(ids8, want8), (ids8, want8)
    ties = [int((L8[b, :e4.n_kept] == L8[b, :e4.n_kept].max()).sum())
            for b in range(B)]
    say(f"[one-hot] E4M3 h98k B={B}: W8A8 rows at the maximum {ties}")
    assert max(ties) >= 2
