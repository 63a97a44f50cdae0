"""The FP8 head applied W8A8 (page 2, "FP8 MTP draft stack for vLLM",
_Fp8DraftHeadMethod.apply): per-token dynamic E4M3 activations, then the
GEMM scaled by the token's and the head's scale.  GPU against the oracle
through the C-ABI: token codes and scales bit-exact, token ids exact (or a
top-2 gap below the logit tolerance), logits within
|gpu - oracle| <= 1e-4 + 1e-3 * |oracle|.  The 98 304 x 2560 head runs at
its full size, in the launch configurations the library picks."""
import sys

import numpy as np
import pytest
import torch

import oracle
import reduced_vocab_nvfp4_amd as dh
from reduced_vocab_nvfp4_amd import workloads as wl
from tests import helpers as H
from tests.test_gpu_formats import _logits_ok, e4m3_head

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _tokens_case(h, tag):
    qx, sx = dh.fp8_quantize_tokens(h.to(DEV))
    oq, os_ = oracle.fp8_tokens_quantize(wl.bf16_bits(h))
    qn, sn = qx.cpu().numpy(), sx.cpu().numpy()
    say(f"[w8a8 tokens] {tag}: B={h.shape[0]} H={h.shape[1]}")
    assert np.array_equal(sn, os_), (tag, sn, os_)
    assert np.array_equal(qn, oq), (tag, np.argwhere(qn != oq)[:5])
    return qn, sn


@pytest.mark.parametrize("B,hid", [(1, 2560), (16, 2560), (3, 5120),
                                   (64, 16), (5, 16384), (2, 272)])
def test_token_quantize_bit_exact(B, hid):
    _tokens_case(wl.hidden_states(B, hid, 70 + B), f"{B}x{hid}")


def test_token_quantize_edge_rows():
    """An all-zero row (the 1e-12 floor), signed zeros, a row whose scale is
    exactly 1 with ties between E4M3 values, subnormal codes and their
    underflow to a signed zero, values spread over 2^-30..2^30, and the row
    where dividing and multiplying by the reciprocal disagree."""
    rng = np.random.default_rng(21)
    x = np.zeros((6, 64), dtype=np.float32)
    x[1, 7] = -0.0
    x[1, 8] = 0.0
    x[2, 0] = 448.0
    x[2, 1:9] = [336.0, -336.0, 2.0 ** -9, 2.0 ** -10, -(2.0 ** -10),
                 3 * 2.0 ** -11, 17.0, 19.0]
    x[3] = rng.standard_normal(64) * np.exp2(rng.integers(-30, 30, 64))
    x[4, 0], x[4, 1] = 4.75, -3.5625
    x[5] = -1e-38
    x[5, 3] = -1.0
    qn, sn = _tokens_case(torch.from_numpy(x).to(torch.bfloat16), "edge rows")
    assert sn[0] == np.float32(np.float32(1e-12) / np.float32(448.0))
    assert sn[2] == 1.0 and qn[2, 1] == 0x7A and qn[2, 2] == 0xFA
    assert qn[1, 7] == 0x80 and qn[1, 8] == 0x00
    assert qn[4, 1] == 0xFA


def _top_check(hd, h, tag):
    ids = dh.draft_head_top_tokens_w8a8(hd.q, hd.scale, hd.idx_gpu,
                                        h.to(DEV)).cpu().numpy()
    qx, sx = oracle.fp8_tokens_quantize(wl.bf16_bits(h))
    L = oracle.w8a8_logits(hd.o_q, hd.o_scale, qx, sx)
    _, want = oracle.argmax_remap(L, hd.idx)
    exc = H.check_top_tokens(ids, L, hd.idx, hd.n_kept, want)
    say(f"[w8a8 top] {tag}: B={h.shape[0]} exceptions={exc}")
    return exc


def test_w8a8_top_tokens_h98k_b16():
    hd = e4m3_head("h98k_b16")
    exc = 0
    for s in range(2):
        exc += _top_check(hd, wl.hidden_states(16, hd.hidden, 80 + s),
                          f"h98k s{s}")
    assert exc <= 1


@pytest.mark.parametrize("batch", [1, 3, 17])
def test_w8a8_top_tokens_other_batches(batch):
    hd = e4m3_head("h98k_b16")
    assert _top_check(hd, wl.hidden_states(batch, hd.hidden, 90 + batch),
                      f"h98k B={batch}") <= 1


def test_w8a8_top_tokens_tiny():
    hd = e4m3_head("tiny")
    for B in (1, 5, 16):
        assert _top_check(hd, wl.hidden_states(B, hd.hidden, 95 + B),
                          f"tiny B={B}") == 0


def _logits_check(hd, h, tag):
    out = dh.draft_head_logits_w8a8(hd.q, hd.scale, hd.idx_gpu, hd.n_kept,
                                    hd.vocab, h.to(DEV)).cpu().numpy()
    qx, sx = oracle.fp8_tokens_quantize(wl.bf16_bits(h))
    L = oracle.w8a8_logits(hd.o_q, hd.o_scale, qx, sx)
    ref = oracle.logits_scatter(L, hd.n_kept, hd.idx, hd.vocab)
    _logits_ok(out, ref, tag)
    # the token quantization is visible at this tolerance: the W8A16 logits
    # of the same head would not pass
    w16 = oracle.e4m3_tensor_logits(hd.o_q, hd.o_scale, wl.bf16_bits(h))
    assert not H.close(w16, L).all()


def test_w8a8_logits():
    tiny = e4m3_head("tiny")
    _logits_check(tiny, wl.hidden_states(1, tiny.hidden, 31), "tiny B=1")
    _logits_check(tiny, wl.hidden_states(5, tiny.hidden, 32), "tiny B=5")
    big = e4m3_head("h98k_b16")
    _logits_check(big, wl.hidden_states(16, big.hidden, 33), "h98k B=16")
    _logits_check(big, wl.hidden_states(3, big.hidden, 34), "h98k B=3")


def test_w8a8_workspace_is_reused_across_calls():
    """One workspace for a sequence of calls of different batches, top
    tokens and logits interleaved, as a decode loop uses it."""
    hd = e4m3_head("tiny")
    ws = dh.new_workspace_w8a8(hd.n_rows, 16, hd.hidden, DEV)
    for i, B in enumerate((16, 1, 7, 16, 2)):
        h = wl.hidden_states(B, hd.hidden, 200 + i)
        ids = dh.draft_head_top_tokens_w8a8(hd.q, hd.scale, hd.idx_gpu,
                                            h.to(DEV), workspace=ws)
        qx, sx = oracle.fp8_tokens_quantize(wl.bf16_bits(h))
        L = oracle.w8a8_logits(hd.o_q, hd.o_scale, qx, sx)
        _, want = oracle.argmax_remap(L, hd.idx)
        assert H.check_top_tokens(ids.cpu().numpy(), L, hd.idx, hd.n_kept,
                                  want) == 0
        out = dh.draft_head_logits_w8a8(hd.q, hd.scale, hd.idx_gpu, hd.n_kept,
                                        hd.vocab, h.to(DEV), workspace=ws)
        _logits_ok(out.cpu().numpy(),
                   oracle.logits_scatter(L, hd.n_kept, hd.idx, hd.vocab),
                   f"reuse {i} B={B}")


@pytest.mark.parametrize("hid", [48, 272])
def test_w8a8_generic_kernel(hid):
    """The W8A8 step on hidden sizes that only the generic kernel tiles."""
    name = "tiny"
    w_ = wl.WORKLOADS[name]
    w = H.head_weight(w_.vocab, hid)
    idx, n_kept = oracle.build_index(wl.keep_mask(w_))
    idx_g = torch.from_numpy(idx).to(DEV)
    q, sc = dh.e4m3_quantize_rows_per_tensor(w.to(DEV), idx_g)
    oq, os_ = oracle.e4m3_tensor_quantize(wl.bf16_bits(w), idx)
    assert np.array_equal(q.cpu().numpy(), oq)
    for B in (1, 3, 9):
        h = wl.hidden_states(B, hid, 360 + B)
        qx, sx = oracle.fp8_tokens_quantize(wl.bf16_bits(h))
        L = oracle.w8a8_logits(oq, os_, qx, sx)
        ids = dh.draft_head_top_tokens_w8a8(q, sc, idx_g, h.to(DEV))
        _, want = oracle.argmax_remap(L, idx)
        assert H.check_top_tokens(ids.cpu().numpy(), L, idx, n_kept, want) == 0
        out = dh.draft_head_logits_w8a8(q, sc, idx_g, n_kept, w_.vocab,
                                        h.to(DEV))
        _logits_ok(out.cpu().numpy(),
                   oracle.logits_scatter(L, n_kept, idx, w_.vocab),
                   f"w8a8 generic H={hid} B={B}")


def test_w8a8_and_other_calls_share_a_workspace():
    """A workspace sized for the W8A8 calls at batch 1 also serves the
    W16 top-token calls of the same head at batch 16, interleaved: the
    tokens' scratch lies past every call's argmax state."""
    hd = e4m3_head("tiny")
    ws = dh.new_workspace_w8a8(hd.n_rows, 1, hd.hidden, DEV)
    assert ws.numel() >= dh.draft_head_workspace_bytes(hd.n_rows, 16)
    for i in range(4):
        h1 = wl.hidden_states(1, hd.hidden, 400 + i)
        ids = dh.draft_head_top_tokens_w8a8(hd.q, hd.scale, hd.idx_gpu,
                                            h1.to(DEV), workspace=ws)
        qx, sx = oracle.fp8_tokens_quantize(wl.bf16_bits(h1))
        L = oracle.w8a8_logits(hd.o_q, hd.o_scale, qx, sx)
        _, want = oracle.argmax_remap(L, hd.idx)
        assert H.check_top_tokens(ids.cpu().numpy(), L, hd.idx, hd.n_kept,
                                  want) == 0
        h16 = wl.hidden_states(16, hd.hidden, 410 + i)
        ids16 = dh.draft_head_top_tokens_e4m3(hd.q, hd.scale, hd.idx_gpu,
                                              h16.to(DEV), workspace=ws)
        L16 = hd.oracle_logits(h16)
        _, want16 = oracle.argmax_remap(L16, hd.idx)
        assert H.check_top_tokens(ids16.cpu().numpy(), L16, hd.idx,
                                  hd.n_kept, want16) == 0
