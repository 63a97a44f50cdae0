"""Parity of the HIP path with the CPU oracle, through the C-ABI.

Bit-exact: packed codes, block scales, global scale, token ids (except a
top-2 gap below the logit tolerance, where either id passes).  Logits:
|gpu - oracle| <= 1e-4 + 1e-3 * |oracle|.
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


class Head:
    """A workload's head quantized by both sides."""

    def __init__(self, name, vocab=None, hidden=None):
        w_ = wl.WORKLOADS[name]
        self.wl = w_
        self.vocab = vocab or w_.vocab
        self.hidden = hidden or w_.hidden
        say(f"[setup] {name}: V={self.vocab} H={self.hidden}")
        self.w = H.head_weight(self.vocab, self.hidden)
        self.w_bits = wl.bf16_bits(self.w)
        keep = wl.keep_mask(w_)
        self.idx_o, self.n_kept = oracle.build_index(keep)
        idx_t, nk = dh.draft_head_build_index(keep)
        assert nk == self.n_kept and np.array_equal(idx_t.numpy(), self.idx_o)
        self.n_rows = self.idx_o.shape[0]
        self.w_gpu = self.w.to(DEV)
        self.idx_gpu = idx_t.to(DEV)
        self.packed, self.scales, self.gs = dh.nvfp4_quantize_rows(
            self.w_gpu, self.idx_gpu)
        torch.cuda.synchronize()
        self.o_packed, self.o_scales, self.o_gs = oracle.nvfp4_quantize(
            self.w_bits, self.idx_o)

    def oracle_logits(self, h):
        return oracle.nvfp4_logits(self.o_packed, self.o_scales, self.o_gs,
                                   wl.bf16_bits(h))


_heads = {}


def head(name):
    if name not in _heads:
        _heads[name] = Head(name)
    return _heads[name]


# ------------------------------------------------------------ quantizer

@pytest.mark.parametrize("name", ["tiny", "flash_next_64k", "h98k_b16"])
def test_quantize_bit_exact(name):
    hd = head(name)
    say(f"[quantize] {name} rows={hd.n_rows}")
    assert np.float32(hd.gs.item()) == hd.o_gs
    s = hd.scales.cpu().numpy()
    assert np.array_equal(s, hd.o_scales), np.argwhere(s != hd.o_scales)[:5]
    p = hd.packed.cpu().numpy()
    assert np.array_equal(p, hd.o_packed), np.argwhere(p != hd.o_packed)[:5]


def _quant_case(w, idx):
    w_gpu = w.to(DEV)
    idx_gpu = torch.from_numpy(idx).to(DEV)
    p, s, g = dh.nvfp4_quantize_rows(w_gpu, idx_gpu)
    op, os_, og = oracle.nvfp4_quantize(wl.bf16_bits(w), idx)
    assert np.float32(g.item()) == og
    assert np.array_equal(s.cpu().numpy(), os_)
    assert np.array_equal(p.cpu().numpy(), op)
    return p, s, g


def test_quantize_edge_cases():
    rng = np.random.default_rng(21)
    say("[quantize] hidden=48, ragged gather with repeats")
    w = torch.from_numpy(rng.standard_normal((300, 48)).astype(np.float32)
                         * 0.02).to(torch.bfloat16)
    idx = np.concatenate([rng.permutation(300)[:90], np.full(38, 7)]).astype(np.int32)
    _quant_case(w, idx)
    say("[quantize] all-zero head with signed zeros")
    z = torch.zeros((64, 32), dtype=torch.bfloat16)
    z[3, 5] = -0.0
    _quant_case(z, np.arange(64, dtype=np.int32))
    say("[quantize] wide dynamic range: powers of two, ties, subnormal scales")
    x = rng.standard_normal((128, 64)) * np.exp2(rng.integers(-20, 6, (128, 1)))
    x[0, :16] = [6.0 * 2.0 ** -8 * v for v in
                 [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, 6, -0.25, -0.75, -1.25,
                  -1.75, -2.5, -3.5, -5, -6]]
    _quant_case(torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16),
                np.arange(128, dtype=np.int32))
    say("[quantize] the block-scale op-order case")
    w = torch.zeros((64, 32), dtype=torch.float32)
    w[0, 0] = 2.4375
    w[1, 0] = 0.00011157989501953125
    _, s, _ = _quant_case(w.to(torch.bfloat16), np.arange(64, dtype=np.int32))
    assert s[1, 0].item() == 11
    say("[quantize] the round-trip construction")
    from tests.test_oracle_pins import _roundtrip_construction
    packed, scales, wt = _roundtrip_construction(rng, 128, 64)
    p, s, g = _quant_case(wt, np.arange(128, dtype=np.int32))
    assert np.array_equal(p.cpu().numpy(), packed) and g.item() == 2.0 ** -8


def _sweep_head(rng, e_lo, e_hi):
    """BF16 head whose blocks of 16 put every positive bf16 value x with a
    biased exponent in [e_lo, e_hi) (subnormals too when e_lo == 0) beside a
    block maximum x*f for twelve factors f, so that the quotient x/d of the
    element code falls near every e2m1 midpoint; the other 13 elements are
    x times seeded factors in [0, 1) with seeded signs."""
    ex = np.arange(e_lo, e_hi, dtype=np.uint32)
    x = ((ex[:, None] << 7) | np.arange(128, dtype=np.uint32)[None, :]).ravel()
    x = x[x > 0]
    xf = (x << 16).view(np.float32)
    factors = np.array([1, 1.25, 1.5, 2, 2.5, 3, 4, 5, 6, 8, 12, 24],
                       dtype=np.float32)
    nb = x.size * factors.size
    blk = np.empty((nb, 16), dtype=np.float32)
    xs = np.repeat(xf, factors.size)
    big = xs.astype(np.float64) * np.tile(factors, x.size)
    # below the largest finite bf16, and never below x after rounding
    blk[:, 0] = np.maximum(np.minimum(big, 3.38e38), xs).astype(np.float32)
    blk[:, 1] = xs
    blk[:, 2] = -xs
    blk[:, 3:] = (xs[:, None] * rng.random((nb, 13), dtype=np.float32)
                  * rng.choice(np.array([-1, 1], dtype=np.float32), (nb, 13)))
    pad = -nb % 16  # whole rows of 256: repeat the first blocks
    blk = np.concatenate([blk, blk[:pad]])
    w = torch.from_numpy(blk.reshape(-1, 256)).to(torch.bfloat16)
    # the block maximum stays the largest magnitude after rounding to bf16
    a = w.float().abs().view(-1, 16)
    assert bool((a[:, 0] >= a.max(dim=1).values).all())
    return w


def test_quantizers_on_every_finite_bf16_value():
    """Both quantizers against the oracle, bit for bit, over every finite
    bf16 magnitude: windows of eight binades (so every block scale lands in
    the E4M3 range) cover the exponent field, each value beside twelve block
    maxima.  Pins the kernels' quotient (one reciprocal per divisor plus a
    correction) and their hardware fp4/fp8 converts, including the windows
    above 2^60 that take the division."""
    rng = np.random.default_rng(77)
    for e_lo in range(0, 255, 8):
        e_hi = min(e_lo + 8, 255)
        w = _sweep_head(rng, e_lo, e_hi)
        idx = np.arange(w.shape[0], dtype=np.int32)
        say(f"[quantize sweep] exponents [{e_lo}, {e_hi}) rows={w.shape[0]}")
        _quant_case(w, idx)
        q, sc = dh.e4m3_quantize_rows_per_tensor(w.to(DEV),
                                                 torch.from_numpy(idx).to(DEV))
        oq, os_ = oracle.e4m3_tensor_quantize(wl.bf16_bits(w), idx)
        assert np.float32(sc.item()) == os_
        qn = q.cpu().numpy()
        assert np.array_equal(qn, oq), (e_lo, np.argwhere(qn != oq)[:5])


# ------------------------------------------------------------ top tokens

def _top_tokens_check(hd, h, tag):
    h_gpu = h.to(DEV)
    ids = dh.draft_head_top_tokens(hd.packed, hd.scales, hd.gs, hd.idx_gpu,
                                   h_gpu).cpu().numpy()
    L = hd.oracle_logits(h)
    _, want = oracle.argmax_remap(L, hd.idx_o)
    exc = H.check_top_tokens(ids, L, hd.idx_o, hd.n_kept, want)
    say(f"[top_tokens] {tag}: B={h.shape[0]} ids={ids[:4]}... near-tie "
        f"exceptions={exc}")
    return exc


def test_top_tokens_tiny_16_draws():
    hd = head("tiny")
    exc = sum(_top_tokens_check(hd, wl.hidden_states(1, hd.hidden, s), f"tiny s{s}")
              for s in range(16))
    assert exc <= 1


def test_top_tokens_flash_next_64k_16_draws():
    """The headline workload (64 064 x 2560 NVFP4, batch 1) on sixteen
    seeded hidden states, each id against the oracle's."""
    hd = head("flash_next_64k")
    exc = 0
    for s in range(16):
        exc += _top_tokens_check(hd, wl.hidden_states(1, hd.hidden, s),
                                 f"flash_next_64k s{s}")
    assert exc <= 1


@pytest.mark.parametrize("batch", [2, 3, 5, 8, 13])
def test_top_tokens_ragged_batches(batch):
    hd = head("tiny")
    _top_tokens_check(hd, wl.hidden_states(batch, hd.hidden, 100 + batch),
                      f"tiny B={batch}")


def test_top_tokens_back_to_back_calls_reuse_the_workspace():
    """Calls on one workspace agree with calls on fresh ones; the call
    counter that tags the argmax slots advances once per launch and the
    quantizer's amax slot stays zero."""
    hd = head("flash_next_64k")
    ws = dh.new_workspace(hd.n_rows, 1)
    hs = [wl.hidden_states(1, hd.hidden, 50 + s).to(DEV) for s in range(4)]
    outs = [torch.empty(1, dtype=torch.int32, device=DEV) for _ in range(200)]
    for i, o in enumerate(outs):
        dh.draft_head_top_tokens(hd.packed, hd.scales, hd.gs, hd.idx_gpu,
                                 hs[i % 4], out_ids=o, workspace=ws)
    torch.cuda.synchronize()
    first = [dh.draft_head_top_tokens(hd.packed, hd.scales, hd.gs, hd.idx_gpu,
                                      hs[i]).item() for i in range(4)]
    assert all(o.item() == first[i % 4] for i, o in enumerate(outs))
    w = ws.cpu().numpy()
    assert int(w[:4].view(np.uint32)[0]) == 200
    assert not w[64:68].any()


def test_top_tokens_call_counter_wraps_past_zero():
    """The slot tag skips 0 (the tag of a zero-filled slot) when the call
    counter wraps."""
    hd = head("tiny")
    ws = dh.new_workspace(hd.n_rows, 4)
    ws[:4].view(torch.int32).fill_(-2)  # counter 0xFFFFFFFE
    h = wl.hidden_states(4, hd.hidden, 77).to(DEV)
    fresh = dh.draft_head_top_tokens(hd.packed, hd.scales, hd.gs, hd.idx_gpu,
                                     h).cpu()
    for k in range(3):
        out = dh.draft_head_top_tokens(hd.packed, hd.scales, hd.gs,
                                       hd.idx_gpu, h, workspace=ws).cpu()
        assert torch.equal(out, fresh), k
    # tags 0xFFFFFFFF, 1, 2
    assert int(ws[:4].cpu().numpy().view(np.uint32)[0]) == 2


def test_top_tokens_workspace_shared_across_heads_and_batches():
    """Slots left by a call with a larger grid or another batch never pass
    for a later call's results."""
    big, tiny = head("flash_next_64k"), head("tiny")
    ws = dh.new_workspace(big.n_rows, 16)
    for k in range(3):
        for hd, b in ((big, 1), (tiny, 16), (big, 3), (tiny, 1), (tiny, 7)):
            h = wl.hidden_states(b, hd.hidden, 300 + 10 * k + b).to(DEV)
            shared = dh.draft_head_top_tokens(hd.packed, hd.scales, hd.gs,
                                              hd.idx_gpu, h, workspace=ws)
            fresh = dh.draft_head_top_tokens(hd.packed, hd.scales, hd.gs,
                                             hd.idx_gpu, h)
            assert torch.equal(shared.cpu(), fresh.cpu()), (k, b)


@pytest.mark.parametrize("name,batch", [("flash_next_64k", 1), ("tiny", 16)])
def test_top_tokens_graph_replay(name, batch):
    """A captured top-token call replayed with new hidden states matches the
    eager call every time: the call counter in the workspace advances on the
    device, so replays never mistake the previous replay's slots for theirs."""
    hd = head(name)
    ws = dh.new_workspace(hd.n_rows, batch)
    h_static = torch.zeros(batch, hd.hidden, dtype=torch.bfloat16, device=DEV)
    out = torch.full((batch,), -7, dtype=torch.int32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up call outside the capture
        dh.draft_head_top_tokens(hd.packed, hd.scales, hd.gs, hd.idx_gpu,
                                 h_static, out_ids=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dh.draft_head_top_tokens(hd.packed, hd.scales, hd.gs, hd.idx_gpu,
                                 h_static, out_ids=out, workspace=ws)
    for k in range(5):
        h = wl.hidden_states(batch, hd.hidden, 900 + k).to(DEV)
        want = dh.draft_head_top_tokens(hd.packed, hd.scales, hd.gs,
                                        hd.idx_gpu, h).cpu()
        h_static.copy_(h)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.cpu(), want), k


def _synthetic_head(rng, n_rows, hidden):
    packed = rng.integers(0, 256, size=(n_rows, hidden // 2), dtype=np.uint8)
    scales = rng.integers(0x20, 0x48, size=(n_rows, hidden // 16), dtype=np.uint8)
    return packed, scales


def test_top_tokens_exact_ties_pick_the_lowest_row():
    """Copies of the best row, below and above it, tie bit-exactly (every
    row is reduced in the same order wherever it sits); the lowest wins."""
    rng = np.random.default_rng(31)
    n, Hd = 4096, 2560
    packed, scales = _synthetic_head(rng, n, Hd)
    h = wl.hidden_states(1, Hd, 7)
    L = oracle.nvfp4_logits(packed, scales, np.float32(1.0), wl.bf16_bits(h))
    best = int(np.argmax(L[0]))
    lower = best // 2
    for r in {lower, min(best + 1, n - 1), n - 1}:
        packed[r] = packed[best]
        scales[r] = scales[best]
    idx = np.arange(n, dtype=np.int32) * 3 + 1
    L = oracle.nvfp4_logits(packed, scales, np.float32(1.0), wl.bf16_bits(h))
    rows, want = oracle.argmax_remap(L, idx)
    assert rows[0] == min(lower, best)
    ids = dh.draft_head_top_tokens(
        torch.from_numpy(packed).to(DEV), torch.from_numpy(scales).to(DEV),
        torch.ones(1, device=DEV), torch.from_numpy(idx).to(DEV),
        h.to(DEV)).cpu().numpy()
    say(f"[ties] best row {best}, copies at {lower}, {best + 1}, {n - 1}; "
        f"oracle row {rows[0]}, got id {ids[0]}")
    assert ids[0] == want[0]


def test_top_tokens_generic_path_and_minimal_head():
    """hidden % 32 != 0 (the 8-byte-unit kernel) and a 64-row head."""
    rng = np.random.default_rng(41)
    for n, Hd, B in ((64, 48, 1), (192, 48, 3), (64, 2560, 1), (128, 272, 2)):
        packed, scales = _synthetic_head(rng, n, Hd)
        idx = rng.permutation(100000)[:n].astype(np.int32)
        h = wl.hidden_states(B, Hd, n + Hd)
        L = oracle.nvfp4_logits(packed, scales, np.float32(0.5), wl.bf16_bits(h))
        _, want = oracle.argmax_remap(L, idx)
        ids = dh.draft_head_top_tokens(
            torch.from_numpy(packed).to(DEV), torch.from_numpy(scales).to(DEV),
            torch.full((1,), 0.5, device=DEV), torch.from_numpy(idx).to(DEV),
            h.to(DEV)).cpu().numpy()
        say(f"[generic] n={n} H={Hd} B={B}")
        H.check_top_tokens(ids, L, idx, n, want)


@pytest.mark.parametrize("B", [1, 3])
def test_top_tokens_generic_kernel_on_a_wide_grid(B):
    """hidden 48 on 16 384 rows: the generic kernel's grid is as many blocks
    as the device holds (more than a collector covers in one pass of four
    slots per thread), so the argmax collection takes several passes."""
    rng = np.random.default_rng(43 + B)
    n, Hd = 16384, 48
    packed, scales = _synthetic_head(rng, n, Hd)
    idx = np.sort(rng.permutation(200000)[:n]).astype(np.int32)
    h = wl.hidden_states(B, Hd, 4300 + B)
    L = oracle.nvfp4_logits(packed, scales, np.float32(0.5), wl.bf16_bits(h))
    _, want = oracle.argmax_remap(L, idx)
    ids = dh.draft_head_top_tokens(
        torch.from_numpy(packed).to(DEV), torch.from_numpy(scales).to(DEV),
        torch.full((1,), 0.5, device=DEV), torch.from_numpy(idx).to(DEV),
        h.to(DEV)).cpu().numpy()
    say(f"[generic wide grid] n={n} H={Hd} B={B}")
    assert H.check_top_tokens(ids, L, idx, n, want) == 0


# ---------------------------------------------------------------- logits

def _logits_check(hd, h, tag):
    out = dh.draft_head_logits(hd.packed, hd.scales, hd.gs, hd.idx_gpu,
                               hd.n_kept, hd.vocab, h.to(DEV)).cpu().numpy()
    L = hd.oracle_logits(h)
    ref = oracle.logits_scatter(L, hd.n_kept, hd.idx_o, hd.vocab)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(out), fin), tag
    assert (out.view(np.uint32)[~fin] == 0xFF800000).all(), tag
    ok = H.close(out[fin], ref[fin])
    say(f"[logits] {tag}: max abs err "
        f"{np.abs(out[fin].astype(np.float64) - ref[fin]).max():.3e}")
    assert ok.all(), (tag, np.argwhere(~ok)[:5])


def test_logits_tiny():
    hd = head("tiny")
    for s in range(4):
        _logits_check(hd, wl.hidden_states(1, hd.hidden, s), f"tiny s{s}")
    _logits_check(hd, wl.hidden_states(5, hd.hidden, 9), "tiny B=5")


def test_logits_flash_next_batch_1():
    hd = head("flash_next_64k")
    for s in (3, 11):
        _logits_check(hd, wl.hidden_states(1, hd.hidden, s),
                      f"flash_next_64k B=1 s{s}")
