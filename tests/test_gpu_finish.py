"""The cross-block argmax finish and the one-pass logits scatter, through the
C-ABI on the GPU.

* Give-up path: a collecting block that waits too long writes -1 and sets the
  workspace's status word, and a workspace whose status is set answers -1
  without polling until it is zero-filled.  The tests reach that path through
  the workspace's spin-bound field (a bound of 0 rounds gives up before the
  first poll), so every kernel runs to its normal end.
* Logits scatter: each kept row writes the ids from just past the previous
  kept id up to its own, -inf between them, in the GEMV launch itself.  The
  masks below put long runs of dropped ids at the start, the end and in the
  middle of the vocabulary, on each kernel family (batch-1 stream, MFMA
  slices, generic), in float32 and BF16.
* Soak: ten thousand back-to-back top-token calls on one workspace, cycling
  over three heads whose calls run the three kernel families on grids of
  different sizes, each compared with the eager result of its hidden state
  (itself checked against the oracle).
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


class SmallHead:
    """A random BF16 head of vocab x hidden with a given keep mask, quantized
    by both sides."""

    def __init__(self, vocab, hidden, keep, seed):
        rng = np.random.default_rng(seed)
        self.vocab, self.hidden = vocab, hidden
        self.w = torch.from_numpy(
            (rng.standard_normal((vocab, hidden)) * 0.02).astype(np.float32)
        ).to(torch.bfloat16)
        self.idx, self.n_kept = oracle.build_index(np.asarray(keep))
        idx_t, nk = dh.draft_head_build_index(np.asarray(keep))
        assert nk == self.n_kept and np.array_equal(idx_t.numpy(), self.idx)
        self.n_rows = self.idx.shape[0]
        self.idx_gpu = idx_t.to(DEV)
        self.packed, self.scales, self.gs = dh.nvfp4_quantize_rows(
            self.w.to(DEV), self.idx_gpu)
        self.o_packed, self.o_scales, self.o_gs = oracle.nvfp4_quantize(
            wl.bf16_bits(self.w), self.idx)
        assert np.array_equal(self.packed.cpu().numpy(), self.o_packed)

    def logits(self, h):
        return oracle.nvfp4_logits(self.o_packed, self.o_scales, self.o_gs,
                                   wl.bf16_bits(h))

    def top(self, h, **kw):
        return dh.draft_head_top_tokens(self.packed, self.scales, self.gs,
                                        self.idx_gpu, h.to(DEV), **kw)


# ------------------------------------------------------------ give-up path

def _keep_random(vocab, n, seed):
    keep = np.zeros(vocab, bool)
    keep[np.random.default_rng(seed).permutation(vocab)[:n]] = True
    return keep


@pytest.mark.parametrize("hidden,batch", [(256, 1), (256, 16), (48, 1),
                                          (48, 3), (2560, 1)])
def test_give_up_sets_the_status_and_stays_until_zero_filled(hidden, batch):
    """Batch 1 on the stream kernel (hidden 256, 2560), 16 on the MFMA
    kernel, hidden 48 on the generic kernel."""
    hd = SmallHead(4096, hidden, _keep_random(4096, 1000, hidden + batch),
                   hidden)
    h = wl.hidden_states(batch, hidden, 500 + batch)
    want = hd.top(h).cpu()
    L = hd.logits(h)
    _, oracle_ids = oracle.argmax_remap(L, hd.idx)
    H.check_top_tokens(want.numpy(), L, hd.idx, hd.n_kept, oracle_ids)
    ws = dh.new_workspace(hd.n_rows, batch)
    assert not dh.workspace_gave_up(ws)
    # one good call first, so the slots hold this head's tagged results
    assert torch.equal(hd.top(h, workspace=ws).cpu(), want)
    dh.set_workspace_spin_limit(ws, 0)
    got = hd.top(h, workspace=ws).cpu()
    say(f"[give-up] H={hidden} B={batch}: ids after a bound of 0 rounds "
        f"{got.tolist()[:4]}")
    assert (got == -1).all()
    assert dh.workspace_gave_up(ws)
    # the default bound again, but the status stays: no polling, -1 at once
    ws[dh.WS_SPIN_LIMIT_OFFSET:dh.WS_SPIN_LIMIT_OFFSET + 2].zero_()
    assert (hd.top(h, workspace=ws).cpu() == -1).all()
    assert dh.workspace_gave_up(ws)
    # zero-filled: the workspace works again
    ws.zero_()
    for _ in range(3):
        assert torch.equal(hd.top(h, workspace=ws).cpu(), want)
    assert not dh.workspace_gave_up(ws)


def test_a_generous_spin_bound_changes_nothing():
    hd = SmallHead(4096, 256, _keep_random(4096, 2000, 3), 3)
    ws = dh.new_workspace(hd.n_rows, 4)
    dh.set_workspace_spin_limit(ws, 60000)
    for s in range(4):
        h = wl.hidden_states(4, 256, 600 + s)
        assert torch.equal(hd.top(h, workspace=ws).cpu(), hd.top(h).cpu())
    assert not dh.workspace_gave_up(ws)


# ----------------------------------------------------- one-pass scatter

def _masks(vocab):
    rng = np.random.default_rng(5)
    m = {}
    k = np.zeros(vocab, bool)
    k[-64:] = True
    m["last 64 only"] = k
    k = np.zeros(vocab, bool)
    k[:5] = True
    m["first 5 only"] = k
    k = np.zeros(vocab, bool)
    k[vocab // 2] = True
    m["one id"] = k
    m["every id"] = np.ones(vocab, bool)
    k = np.zeros(vocab, bool)
    k[rng.permutation(vocab)[:700]] = True
    k[1000:3000] = False  # a long run dropped in the middle
    k[100:180] = True     # and a long run kept
    m["runs"] = k
    return m


def _scatter_ok(out, ref, tag):
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(out), fin), tag
    assert (out.view(np.uint32)[~fin] == 0xFF800000).all(), tag
    assert H.close(out[fin], ref[fin]).all(), tag


@pytest.mark.parametrize("hidden,batch", [(256, 1), (2560, 1), (256, 2),
                                          (256, 16), (256, 19), (48, 1),
                                          (48, 5)])
def test_logits_scatter_on_masks_with_long_runs(hidden, batch):
    """hidden 256 / 2560 at batch 1: stream kernel (8 and 4 rows per wave
    group); batch 2, 16, 19: MFMA slices; hidden 48: generic kernel."""
    V = 4096
    for name, keep in _masks(V).items():
        hd = SmallHead(V, hidden, keep, hidden + 7)
        h = wl.hidden_states(batch, hidden, 700 + batch)
        out = dh.draft_head_logits(hd.packed, hd.scales, hd.gs, hd.idx_gpu,
                                   hd.n_kept, V, h.to(DEV)).cpu().numpy()
        ref = oracle.logits_scatter(hd.logits(h), hd.n_kept, hd.idx, V)
        say(f"[scatter] {name}: H={hidden} B={batch} kept={hd.n_kept}")
        _scatter_ok(out, ref, name)


@pytest.mark.parametrize("batch", [1, 16])
def test_bf16_logits_scatter_on_masks_with_long_runs(batch):
    """BF16 logits: each value equal to the oracle's rounding, or within the
    float32 GEMV's error of a rounding boundary (the reference-mode tests'
    rule); -inf at exactly the ids that were not kept."""
    from tests.test_gpu_compat import _check_compat_logits
    V = 4096
    for name, keep in _masks(V).items():
        hd = SmallHead(V, 256, keep, 11)
        h = wl.hidden_states(batch, 256, 800 + batch)
        out = dh.draft_head_logits_compat(
            hd.packed, hd.scales, hd.gs, hd.idx_gpu, hd.n_kept, V,
            h.to(DEV)).cpu().view(torch.int16).numpy().view(np.uint16)
        _check_compat_logits(out, hd.logits(h), hd.idx, hd.n_kept, V,
                             f"{name} B={batch}", np.ones(batch))


@pytest.mark.parametrize("fmt", ["e4m3", "bf16"])
def test_other_formats_scatter_on_masks_with_long_runs(fmt):
    V, Hd = 4096, 256
    rng = np.random.default_rng(13)
    w = torch.from_numpy((rng.standard_normal((V, Hd)) * 0.02)
                         .astype(np.float32)).to(torch.bfloat16)
    for name, keep in _masks(V).items():
        idx, n_kept = oracle.build_index(keep)
        idx_gpu = torch.from_numpy(idx).to(DEV)
        for B in (1, 3):
            h = wl.hidden_states(B, Hd, 900 + B)
            if fmt == "e4m3":
                q, s = oracle.e4m3_tensor_quantize(wl.bf16_bits(w), idx)
                L = oracle.e4m3_tensor_logits(q, s, wl.bf16_bits(h))
                out = dh.draft_head_logits_e4m3(
                    torch.from_numpy(q).to(DEV),
                    torch.full((1,), float(s), device=DEV), idx_gpu, n_kept,
                    V, h.to(DEV))
            else:
                rows = w[torch.from_numpy(idx.astype(np.int64))].contiguous()
                L = oracle.bf16_logits(wl.bf16_bits(w), idx, wl.bf16_bits(h))
                out = dh.draft_head_logits_bf16(rows.to(DEV), idx_gpu, n_kept,
                                                V, h.to(DEV))
            say(f"[{fmt} scatter] {name}: B={B}")
            _scatter_ok(out.cpu().numpy(),
                        oracle.logits_scatter(L, n_kept, idx, V), name)


# ------------------------------------------------------------------ soak

def test_soak_ten_thousand_calls_over_three_kernel_families():
    """Calls cycle over (head, hidden state): the 64 064 x 2560 head at batch
    1 (stream kernel, 768 blocks), a 98 304 x 2560 head at batch 16 (MFMA
    kernel, 256 blocks) and a 16 384 x 48 head at batch 1 (generic kernel),
    all on one workspace, so each call's slots sit over slots another grid
    left.  Every result is compared with the eager result of its hidden
    state; the first mismatch fails the test."""
    heads = []
    for name in ("flash_next_64k", "h98k_b16"):
        w_ = wl.WORKLOADS[name]
        w = H.head_weight(w_.vocab, w_.hidden)
        idx, n_kept = oracle.build_index(wl.keep_mask(w_))
        idx_gpu = torch.from_numpy(idx).to(DEV)
        p, s, g = dh.nvfp4_quantize_rows(w.to(DEV), idx_gpu)
        heads.append((name, p, s, g, idx, n_kept, idx_gpu, w_.hidden,
                      w_.batch))
    rng = np.random.default_rng(17)
    n, Hd = 16384, 48
    pk = rng.integers(0, 256, size=(n, Hd // 2), dtype=np.uint8)
    sc = rng.integers(0x20, 0x48, size=(n, Hd // 16), dtype=np.uint8)
    gidx = np.sort(rng.permutation(200000)[:n]).astype(np.int32)
    heads.append(("generic 16384x48", torch.from_numpy(pk).to(DEV),
                  torch.from_numpy(sc).to(DEV),
                  torch.full((1,), 0.5, device=DEV), gidx, n,
                  torch.from_numpy(gidx).to(DEV), Hd, 1))
    NH = 4  # hidden states per head
    ws = dh.new_workspace(98304, 16)
    refs = []
    for (name, p, s, g, idx, n_kept, idx_gpu, Hd, B) in heads:
        hs = [wl.hidden_states(B, Hd, 1000 + k) for k in range(NH)]
        hg = [x.to(DEV) for x in hs]
        want = [dh.draft_head_top_tokens(p, s, g, idx_gpu, x).cpu()
                for x in hg]
        # the eager results against the oracle (one hidden state per head)
        if name.startswith("generic"):
            L = oracle.nvfp4_logits(pk, sc, np.float32(0.5),
                                    wl.bf16_bits(hs[0]))
        else:
            L = oracle.nvfp4_logits(p.cpu().numpy(), s.cpu().numpy(),
                                    np.float32(g.item()), wl.bf16_bits(hs[0]))
        _, oid = oracle.argmax_remap(L, idx)
        H.check_top_tokens(want[0].numpy(), L, idx, n_kept, oid)
        refs.append((hg, want))
    N = 10000
    out = torch.full((N, 16), -7, dtype=torch.int32, device=DEV)
    L = dh.lib()
    ptrs = []
    for (name, p, s, g, idx, n_kept, idx_gpu, Hd, B) in heads:
        ptrs.append((p.data_ptr(), s.data_ptr(), g.data_ptr(),
                     idx_gpu.data_ptr(), p.shape[0], Hd, B))
    hptr = [[x.data_ptr() for x in hg] for hg, _ in refs]
    out_p = out.data_ptr()
    sp = torch.cuda.current_stream().cuda_stream
    say(f"[soak] {N} calls over {len(heads)} heads")
    for i in range(N):
        k = i % len(heads)
        pp, ss, gg, ii, nr, Hd, B = ptrs[k]
        rc = L.draft_head_top_tokens(pp, ss, gg, ii, nr, Hd,
                                     hptr[k][(i // len(heads)) % NH], B,
                                     out_p + 64 * i, ws.data_ptr(),
                                     ws.numel(), sp)
        assert rc == 0, (i, rc)
    torch.cuda.synchronize()
    got = out.cpu()
    for i in range(N):
        k = i % len(heads)
        B = ptrs[k][6]
        want = refs[k][1][(i // len(heads)) % NH]
        if not torch.equal(got[i, :B], want):
            raise AssertionError(f"call {i} ({heads[k][0]}): {got[i, :B]} "
                                 f"!= {want}")
    assert not dh.workspace_gave_up(ws)
    say(f"[soak] {N} calls agree")
