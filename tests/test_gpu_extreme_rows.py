"""Hidden states with extreme per-row ranges through the batched (MFMA)
kernel, GPU against the oracle through the C-ABI.  The kernel multiplies
BF16 h by BF16 dequantized weights with fp32 accumulation, which holds every
BF16 input exactly, so no range of h is special to it; this pins that down
for rows near 2^+-40 and 2^+-100, a zero row, one element 2^60 times the
rest (where that element's weight is zero, the logit is the sum of the
ordinary terms), and elements spread over 24 binades.

Every mode that reads the staged rows is checked: top tokens, fp32 logits,
BF16 top tokens and logits, and the dense linear.  Rows scaled as a whole
are compared after dividing by their scale, so the elementwise tolerance
keeps its meaning (an argmax does not change under a positive scale); the
other rows unscaled.  Slices of 16 and 5 rows, with hidden 256 (a wave's
pieces of h span two rows) and 2688 (one-step slots)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import reduced_vocab_nvfp4_amd as dh
from reduced_vocab_nvfp4_amd import workloads as wl
from tests import helpers as H
from tests.test_gpu_compat import _compat_case
from tests.test_gpu_parity import Head

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def extreme_rows(B, hidden, seed):
    """BF16 [B, hidden] rows cycling through eight kinds, and each row's
    scale (the factor its logits carry)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, hidden))
    scale = np.ones(B)
    for b in range(B):
        kind = b % 8
        if kind == 1:
            x[b] *= 2.0 ** 40
            scale[b] = 2.0 ** 40
        elif kind == 2:
            x[b] *= 2.0 ** -40
            scale[b] = 2.0 ** -40
        elif kind == 3:
            x[b] *= 2.0 ** 100
            scale[b] = 2.0 ** 100
        elif kind == 4:
            x[b] = 0.0
        elif kind == 5:
            x[b, 7] = 2.0 ** 60
        elif kind == 6:
            x[b] *= 2.0 ** -100
            scale[b] = 2.0 ** -100
        elif kind == 7:
            x[b] *= np.exp2(rng.integers(-12, 13, hidden))
    return torch.from_numpy(x).to(torch.bfloat16), scale


_heads = {}


def _head(hidden):
    if hidden not in _heads:
        _heads[hidden] = Head("tiny", hidden=hidden)
    return _heads[hidden]


@pytest.mark.parametrize("hidden", [256, 2688])
@pytest.mark.parametrize("B", [16, 5])
def test_extreme_rows(hidden, B):
    hd = _head(hidden)
    h, scale = extreme_rows(B, hidden, 700 + B + hidden)
    tag = f"hidden={hidden} B={B}"
    say(f"[extreme rows] {tag}")
    hg = h.to(DEV)
    L = hd.oracle_logits(h)
    assert np.isfinite(L).all()
    # top tokens: the argmax of each row is that of the row divided by its
    # scale
    ids = dh.draft_head_top_tokens(hd.packed, hd.scales, hd.gs, hd.idx_gpu,
                                   hg).cpu().numpy()
    _, want = oracle.argmax_remap(L, hd.idx_o)
    exc = H.check_top_tokens(ids, L / scale[:, None], hd.idx_o, hd.n_kept,
                             want)
    # the zero row: every logit is 0, so the lowest kept row wins
    for b in range(B):
        if b % 8 == 4:
            assert ids[b] == hd.idx_o[0], (tag, b)
    # fp32 logits
    out = dh.draft_head_logits(hd.packed, hd.scales, hd.gs, hd.idx_gpu,
                               hd.n_kept, hd.vocab, hg).cpu().numpy()
    ref = oracle.logits_scatter(L, hd.n_kept, hd.idx_o, hd.vocab)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(out), fin), tag
    s = np.broadcast_to(scale[:, None], ref.shape)
    ok = H.close(out[fin] / s[fin], ref[fin] / s[fin])
    assert ok.all(), (tag, np.argwhere(~ok)[:5])
    # BF16 top tokens and logits
    exc += _compat_case(hd, h, tag)
    # the dense linear over the kept rows' weights
    y = dh.nvfp4_linear(hd.packed, hd.scales, hd.gs, hg).cpu().numpy()
    ok = H.close(y / scale[:, None], L / scale[:, None])
    assert ok.all(), (tag, np.argwhere(~ok)[:5])
    say(f"[extreme rows] {tag}: near-tie exceptions {exc}")
