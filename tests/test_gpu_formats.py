"""Parity of the per-tensor E4M3 head, the BF16 stock head and the batched
(MFMA) NVFP4 path with the CPU oracle, through the C-ABI.

Bit-exact: E4M3 codes and tensor scale, token ids (except a top-2 gap below
the logit tolerance, where either id passes).  Logits:
|gpu - oracle| <= 1e-4 + 1e-3 * |oracle|.  Every case runs at the full
sizes of its workload, in the launch configuration the library picks for
that batch (batch-1 stream kernel, MFMA slices of up to 16, generic kernel).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import reduced_vocab_nvfp4_amd as dh
from reduced_vocab_nvfp4_amd import workloads as wl
from tests import helpers as H

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _index(name):
    keep = wl.keep_mask(wl.WORKLOADS[name])
    idx, n_kept = oracle.build_index(keep)
    return idx, n_kept


def _logits_ok(out, ref, tag):
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(out), fin), tag
    assert (out.view(np.uint32)[~fin] == 0xFF800000).all(), tag
    ok = H.close(out[fin], ref[fin])
    say(f"[logits] {tag}: max abs err "
        f"{np.abs(out[fin].astype(np.float64) - ref[fin]).max():.3e}")
    assert ok.all(), (tag, np.argwhere(~ok)[:5])


# ------------------------------------------------------------ E4M3 head

class E4m3Head:
    def __init__(self, name):
        w_ = wl.WORKLOADS[name]
        self.vocab, self.hidden = w_.vocab, w_.hidden
        say(f"[setup e4m3] {name}: V={self.vocab} H={self.hidden}")
        self.w = H.head_weight(self.vocab, self.hidden)
        self.idx, self.n_kept = _index(name)
        self.n_rows = self.idx.shape[0]
        self.idx_gpu = torch.from_numpy(self.idx).to(DEV)
        self.q, self.scale = dh.e4m3_quantize_rows_per_tensor(
            self.w.to(DEV), self.idx_gpu)
        torch.cuda.synchronize()
        self.o_q, self.o_scale = oracle.e4m3_tensor_quantize(
            wl.bf16_bits(self.w), self.idx)

    def oracle_logits(self, h):
        return oracle.e4m3_tensor_logits(self.o_q, self.o_scale,
                                         wl.bf16_bits(h))


_e4 = {}


def e4m3_head(name):
    if name not in _e4:
        _e4[name] = E4m3Head(name)
    return _e4[name]


@pytest.mark.parametrize("name", ["tiny", "h98k_b16"])
def test_e4m3_quantize_bit_exact(name):
    hd = e4m3_head(name)
    say(f"[e4m3 quantize] {name} rows={hd.n_rows}")
    assert np.float32(hd.scale.item()) == hd.o_scale
    q = hd.q.cpu().numpy()
    assert np.array_equal(q, hd.o_q), np.argwhere(q != hd.o_q)[:5]


def _e4m3_quant_case(w, idx, tag):
    say(f"[e4m3 quantize] {tag}")
    q, s = dh.e4m3_quantize_rows_per_tensor(w.to(DEV),
                                            torch.from_numpy(idx).to(DEV))
    oq, os_ = oracle.e4m3_tensor_quantize(wl.bf16_bits(w), idx)
    assert np.float32(s.item()) == os_, tag
    qn = q.cpu().numpy()
    assert np.array_equal(qn, oq), (tag, np.argwhere(qn != oq)[:5])
    return qn, s.item()


def test_e4m3_quantize_edge_cases():
    rng = np.random.default_rng(5)
    z = torch.zeros((64, 32), dtype=torch.bfloat16)
    z[1, 3] = -0.0
    q, s = _e4m3_quant_case(z, np.arange(64, dtype=np.int32), "all-zero head")
    assert s == np.float32(np.float32(1e-12) / np.float32(448.0))
    assert q[1, 3] == 0x80 and (np.delete(q.ravel(), 32 + 3) == 0).all()
    x = rng.standard_normal((128, 48)) * np.exp2(rng.integers(-30, 4, (128, 1)))
    x[0, 0] = 448.0 * 2.0 ** 3  # sets amax: scale = 8
    x[0, 1:7] = np.array([448, -448, 2.0 ** -9, 2.0 ** -10, -(2.0 ** -10),
                          3 * 2.0 ** -11]) * 8.0
    _e4m3_quant_case(torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16),
                     np.arange(128, dtype=np.int32),
                     "wide range: clamp, subnormal codes, ties to even")
    w = torch.from_numpy((rng.standard_normal((300, 80)) * 0.02)
                         .astype(np.float32)).to(torch.bfloat16)
    idx = np.concatenate([rng.permutation(300)[:100],
                          np.full(28, 11)]).astype(np.int32)
    _e4m3_quant_case(w, idx, "hidden=80, ragged gather with repeats")


def _e4m3_top_check(hd, h, tag):
    ids = dh.draft_head_top_tokens_e4m3(hd.q, hd.scale, hd.idx_gpu,
                                        h.to(DEV)).cpu().numpy()
    L = hd.oracle_logits(h)
    _, want = oracle.argmax_remap(L, hd.idx)
    exc = H.check_top_tokens(ids, L, hd.idx, hd.n_kept, want)
    say(f"[e4m3 top] {tag}: B={h.shape[0]} exceptions={exc}")
    return exc


def test_e4m3_top_tokens_h98k_b16():
    hd = e4m3_head("h98k_b16")
    exc = 0
    for s in range(2):
        exc += _e4m3_top_check(hd, wl.hidden_states(16, hd.hidden, s),
                               f"h98k s{s}")
    assert exc <= 1


@pytest.mark.parametrize("batch", [1, 3, 17])
def test_e4m3_top_tokens_other_batches(batch):
    hd = e4m3_head("h98k_b16")
    assert _e4m3_top_check(hd, wl.hidden_states(batch, hd.hidden, 40 + batch),
                           f"h98k B={batch}") <= 1


def _e4m3_logits_check(hd, h, tag):
    out = dh.draft_head_logits_e4m3(hd.q, hd.scale, hd.idx_gpu, hd.n_kept,
                                    hd.vocab, h.to(DEV)).cpu().numpy()
    ref = oracle.logits_scatter(hd.oracle_logits(h), hd.n_kept, hd.idx,
                                hd.vocab)
    _logits_ok(out, ref, tag)


def test_e4m3_logits():
    tiny = e4m3_head("tiny")
    _e4m3_logits_check(tiny, wl.hidden_states(1, tiny.hidden, 3), "tiny B=1")
    _e4m3_logits_check(tiny, wl.hidden_states(5, tiny.hidden, 4), "tiny B=5")
    big = e4m3_head("h98k_b16")
    _e4m3_logits_check(big, wl.hidden_states(16, big.hidden, 5), "h98k B=16")


# ------------------------------------------------------- BF16 stock head

class StockHead:
    def __init__(self):
        w_ = wl.WORKLOADS["stock_bf16"]
        self.vocab, self.hidden = w_.vocab, w_.hidden
        say(f"[setup bf16] V={self.vocab} H={self.hidden}")
        self.w = H.head_weight(self.vocab, self.hidden)
        self.w_bits = wl.bf16_bits(self.w)
        self.idx, self.n_kept = _index("stock_bf16")
        assert np.array_equal(self.idx, np.arange(self.vocab))
        self.w_gpu = self.w.to(DEV)
        self.idx_gpu = torch.from_numpy(self.idx).to(DEV)

    def oracle_logits(self, h):
        return oracle.bf16_logits(self.w_bits, self.idx, wl.bf16_bits(h))


_stock = []


def stock():
    if not _stock:
        _stock.append(StockHead())
    return _stock[0]


@pytest.mark.parametrize("batch", [1, 4])
def test_bf16_stock_top_tokens(batch):
    """The stock 248 320 x 2560 BF16 head: sixteen hidden states at batch 1
    (the stock-head workload), one batch of four."""
    hd = stock()
    exc = 0
    for s in range(16 if batch == 1 else 1):
        h = wl.hidden_states(batch, hd.hidden, 60 + s)
        ids = dh.draft_head_top_tokens_bf16(hd.w_gpu, hd.idx_gpu,
                                            h.to(DEV)).cpu().numpy()
        L = hd.oracle_logits(h)
        _, want = oracle.argmax_remap(L, hd.idx)
        exc += H.check_top_tokens(ids, L, hd.idx, hd.n_kept, want)
        say(f"[bf16 top] stock B={batch} s{s}: ids={ids[:4]} exceptions={exc}")
    assert exc <= 1


def test_bf16_logits_gathered_rows():
    """A BF16 head of gathered rows W[dh_idx] with the tiny mask."""
    idx, n_kept = _index("tiny")
    w = H.head_weight(4096, 256)
    rows = w[torch.from_numpy(idx.astype(np.int64))].contiguous()
    for B in (1, 5):
        h = wl.hidden_states(B, 256, 70 + B)
        out = dh.draft_head_logits_bf16(
            rows.to(DEV), torch.from_numpy(idx).to(DEV), n_kept, 4096,
            h.to(DEV)).cpu().numpy()
        L = oracle.bf16_logits(wl.bf16_bits(w), idx, wl.bf16_bits(h))
        _logits_ok(out, oracle.logits_scatter(L, n_kept, idx, 4096),
                   f"bf16 tiny B={B}")


# ------------------------------------------- NVFP4 through the MFMA path

class Nvfp4Head:
    def __init__(self, name):
        w_ = wl.WORKLOADS[name]
        self.vocab, self.hidden = w_.vocab, w_.hidden
        say(f"[setup nvfp4] {name}: V={self.vocab} H={self.hidden}")
        w = H.head_weight(self.vocab, self.hidden)
        self.idx, self.n_kept = _index(name)
        self.idx_gpu = torch.from_numpy(self.idx).to(DEV)
        self.packed, self.scales, self.gs = dh.nvfp4_quantize_rows(
            w.to(DEV), self.idx_gpu)
        torch.cuda.synchronize()
        self.o_packed, self.o_scales, self.o_gs = oracle.nvfp4_quantize(
            wl.bf16_bits(w), self.idx)
        assert np.array_equal(self.packed.cpu().numpy(), self.o_packed)
        assert np.array_equal(self.scales.cpu().numpy(), self.o_scales)

    def oracle_logits(self, h):
        return oracle.nvfp4_logits(self.o_packed, self.o_scales, self.o_gs,
                                   wl.bf16_bits(h))


_nv = {}


def nvfp4_head(name):
    if name not in _nv:
        _nv[name] = Nvfp4Head(name)
    return _nv[name]


def _nvfp4_top_check(hd, h, tag):
    ids = dh.draft_head_top_tokens(hd.packed, hd.scales, hd.gs, hd.idx_gpu,
                                   h.to(DEV)).cpu().numpy()
    L = hd.oracle_logits(h)
    _, want = oracle.argmax_remap(L, hd.idx)
    exc = H.check_top_tokens(ids, L, hd.idx, hd.n_kept, want)
    say(f"[nvfp4 top] {tag}: B={h.shape[0]} exceptions={exc}")
    return exc


def test_nvfp4_top_tokens_h98k_b16():
    hd = nvfp4_head("h98k_b16")
    exc = sum(_nvfp4_top_check(hd, wl.hidden_states(16, hd.hidden, s),
                               f"h98k s{s}") for s in range(2))
    assert exc <= 1


def test_nvfp4_dense27b_b8_top_tokens_and_logits_16_draws():
    """The 27B-shaped head (64 064 x 5120 NVFP4) at batch 8: sixteen seeded
    batches, the ids and every logit of the full-vocabulary output of each
    against the oracle."""
    hd = nvfp4_head("dense27b_64k_b8")
    exc = 0
    for s in range(16):
        h = wl.hidden_states(8, hd.hidden, s)
        L = hd.oracle_logits(h)
        ids = dh.draft_head_top_tokens(hd.packed, hd.scales, hd.gs,
                                       hd.idx_gpu, h.to(DEV)).cpu().numpy()
        _, want = oracle.argmax_remap(L, hd.idx)
        exc += H.check_top_tokens(ids, L, hd.idx, hd.n_kept, want)
        out = dh.draft_head_logits(hd.packed, hd.scales, hd.gs, hd.idx_gpu,
                                   hd.n_kept, hd.vocab,
                                   h.to(DEV)).cpu().numpy()
        _logits_ok(out, oracle.logits_scatter(L, hd.n_kept, hd.idx, hd.vocab),
                   f"dense27b B=8 s{s}")
    say(f"[nvfp4] dense27b: 16 batches of 8, near-tie exceptions {exc}")
    assert exc <= 2


# ------------------------------------------------ shapes of every kernel

@pytest.mark.parametrize("fmt", ["e4m3", "bf16"])
def test_other_formats_on_small_and_odd_shapes(fmt):
    """hidden not a multiple of the chunk tiling (generic kernel), a 64-row
    head, and batch slices that mix kernels."""
    rng = np.random.default_rng(81)
    for n, Hd, B in ((64, 48, 1), (192, 48, 3), (64, 2560, 1), (128, 272, 2),
                     (256, 256, 19)):
        ids = rng.permutation(100000)[:n].astype(np.int32)
        w = torch.from_numpy((rng.standard_normal((n, Hd)) * 0.02)
                             .astype(np.float32)).to(torch.bfloat16)
        h = wl.hidden_states(B, Hd, n + Hd)
        rows = np.arange(n, dtype=np.int32)
        if fmt == "e4m3":
            q, s = oracle.e4m3_tensor_quantize(wl.bf16_bits(w), rows)
            L = oracle.e4m3_tensor_logits(q, s, wl.bf16_bits(h))
            got = dh.draft_head_top_tokens_e4m3(
                torch.from_numpy(q).to(DEV),
                torch.full((1,), float(s), device=DEV),
                torch.from_numpy(ids).to(DEV), h.to(DEV))
        else:
            L = oracle.bf16_logits(wl.bf16_bits(w), rows, wl.bf16_bits(h))
            got = dh.draft_head_top_tokens_bf16(
                w.to(DEV), torch.from_numpy(ids).to(DEV), h.to(DEV))
        _, want = oracle.argmax_remap(L, ids)
        say(f"[{fmt} shapes] n={n} H={Hd} B={B}")
        H.check_top_tokens(got.cpu().numpy(), L, ids, n, want)


@pytest.mark.parametrize("batch", [2, 16, 33])
def test_nvfp4_mfma_slices_on_tiny(batch):
    """Batch slices through the MFMA kernel, logits and top tokens."""
    hd = nvfp4_head("tiny")
    h = wl.hidden_states(batch, hd.hidden, 90 + batch)
    _nvfp4_top_check(hd, h, f"tiny B={batch}")
    out = dh.draft_head_logits(hd.packed, hd.scales, hd.gs, hd.idx_gpu,
                               hd.n_kept, hd.vocab, h.to(DEV)).cpu().numpy()
    ref = oracle.logits_scatter(hd.oracle_logits(h), hd.n_kept, hd.idx,
                                hd.vocab)
    _logits_ok(out, ref, f"tiny B={batch}")
