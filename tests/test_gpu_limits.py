"""The boundary's limits, GPU against the oracle: the largest batch (64,
four MFMA slices of 16) and the largest hidden size (16 384, where the MFMA
kernel stages at most three batch rows per slice and batch 1 runs the
generic kernel) on the smallest head (64 rows), for every step kind:
top tokens and logits (fp32 and BF16), the W8A8 head and the linear.  At
hidden 16 384 the W8A8 head's FP8 kernel stages one-byte token codes, eight
batch rows per slice, so batch 9 runs a slice of eight on the FP8 matrix
cores and one on the stream kernel."""
import sys

import numpy as np
import pytest
import torch

import oracle
import reduced_vocab_nvfp4_amd as dh
from reduced_vocab_nvfp4_amd import workloads as wl
from tests import helpers as H
from tests.test_gpu_formats import _logits_ok, e4m3_head
from tests.test_gpu_parity import _synthetic_head, head

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_batch_64_every_step_kind():
    hd = head("tiny")
    h = wl.hidden_states(64, hd.hidden, 500)
    hg = h.to(DEV)
    L = hd.oracle_logits(h)
    _, want = oracle.argmax_remap(L, hd.idx_o)
    ids = dh.draft_head_top_tokens(hd.packed, hd.scales, hd.gs, hd.idx_gpu, hg)
    assert H.check_top_tokens(ids.cpu().numpy(), L, hd.idx_o, hd.n_kept,
                              want) == 0
    out = dh.draft_head_logits(hd.packed, hd.scales, hd.gs, hd.idx_gpu,
                               hd.n_kept, hd.vocab, hg)
    _logits_ok(out.cpu().numpy(),
               oracle.logits_scatter(L, hd.n_kept, hd.idx_o, hd.vocab),
               "tiny B=64")
    # BF16-rounded top tokens: the first maximum of the GPU's BF16 logits
    ids_b = dh.draft_head_top_tokens_compat(hd.packed, hd.scales, hd.gs,
                                            hd.idx_gpu, hg).cpu().numpy()
    lb = dh.draft_head_logits_compat(hd.packed, hd.scales, hd.gs, hd.idx_gpu,
                                     hd.n_kept, hd.vocab, hg)
    bits = lb.cpu().view(torch.int16).numpy().view(np.uint16)
    kept = oracle.bf16_bits_value(bits[:, hd.idx_o[:hd.n_kept]])
    assert np.array_equal(ids_b, hd.idx_o[:hd.n_kept][np.argmax(kept, axis=1)])
    # the linear over the gathered rows
    y = dh.nvfp4_linear(hd.packed, hd.scales, hd.gs, hg).cpu().numpy()
    assert H.close(y, L).all()
    # the W8A8 head
    e4 = e4m3_head("tiny")
    ids8 = dh.draft_head_top_tokens_w8a8(e4.q, e4.scale, e4.idx_gpu, hg)
    qx, sx = oracle.fp8_tokens_quantize(wl.bf16_bits(h))
    L8 = oracle.w8a8_logits(e4.o_q, e4.o_scale, qx, sx)
    _, want8 = oracle.argmax_remap(L8, e4.idx)
    assert H.check_top_tokens(ids8.cpu().numpy(), L8, e4.idx, e4.n_kept,
                              want8) == 0
    say("[limits] batch 64: top, logits, BF16 modes, linear, W8A8")


@pytest.mark.parametrize("B", [1, 3, 7])
def test_hidden_16384_on_a_64_row_head(B):
    rng = np.random.default_rng(600 + B)
    n, hid = 64, 16384
    packed, scales = _synthetic_head(rng, n, hid)
    idx = rng.permutation(200000)[:n].astype(np.int32)
    idx.sort()
    V = 200000
    gs = np.float32(0.25)
    h = wl.hidden_states(B, hid, 610 + B)
    L = oracle.nvfp4_logits(packed, scales, gs, wl.bf16_bits(h))
    pg = torch.from_numpy(packed).to(DEV)
    sg = torch.from_numpy(scales).to(DEV)
    gg = torch.full((1,), float(gs), device=DEV)
    ig = torch.from_numpy(idx).to(DEV)
    hg = h.to(DEV)
    _, want = oracle.argmax_remap(L, idx)
    ids = dh.draft_head_top_tokens(pg, sg, gg, ig, hg).cpu().numpy()
    assert H.check_top_tokens(ids, L, idx, n, want) <= 1
    out = dh.draft_head_logits(pg, sg, gg, ig, n, V, hg).cpu().numpy()
    _logits_ok(out, oracle.logits_scatter(L, n, idx, V),
               f"H=16384 B={B}")
    y = dh.nvfp4_linear(pg, sg, gg, hg).cpu().numpy()
    assert H.close(y, L).all()
    say(f"[limits] hidden 16384, 64 rows, B={B}")


@pytest.mark.parametrize("B", [3, 9])
def test_hidden_16384_w8a8(B):
    rng = np.random.default_rng(620 + B)
    n, hid, V = 64, 16384, 200000
    w = torch.from_numpy(rng.standard_normal((n, hid)).astype(np.float32)
                         * 0.02).to(torch.bfloat16)
    idx = np.arange(n, dtype=np.int32)
    q, sc = dh.e4m3_quantize_rows_per_tensor(w.to(DEV),
                                             torch.from_numpy(idx).to(DEV))
    oq, osc = oracle.e4m3_tensor_quantize(wl.bf16_bits(w), idx)
    assert np.array_equal(q.cpu().numpy(), oq)
    ids_kept = np.sort(rng.permutation(V)[:n]).astype(np.int32)
    ig = torch.from_numpy(ids_kept).to(DEV)
    h = wl.hidden_states(B, hid, 630 + B)
    hg = h.to(DEV)
    qx, sx = oracle.fp8_tokens_quantize(wl.bf16_bits(h))
    L = oracle.w8a8_logits(oq, osc, qx, sx)
    _, want = oracle.argmax_remap(L, ids_kept)
    ids = dh.draft_head_top_tokens_w8a8(q, sc, ig, hg).cpu().numpy()
    assert H.check_top_tokens(ids, L, ids_kept, n, want) <= 1
    out = dh.draft_head_logits_w8a8(q, sc, ig, n, V, hg).cpu().numpy()
    _logits_ok(out, oracle.logits_scatter(L, n, ids_kept, V),
               f"W8A8 H=16384 B={B}")
    say(f"[limits] W8A8 hidden 16384, 64 rows, B={B}")
