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
pieces of h span two rows) and 2688 (one-step slots).

A row holding an infinity or a NaN leaves the slice's other rows alone, and
its own logits carry the oracle's pattern of NaN and +-inf."""
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
    exc += _compat_case(hd, h, tag, row_scale=scale)
    # the dense linear over the kept rows' weights
    y = dh.nvfp4_linear(hd.packed, hd.scales, hd.gs, hg).cpu().numpy()
    ok = H.close(y / scale[:, None], L / scale[:, None])
    assert ok.all(), (tag, np.argwhere(~ok)[:5])
    say(f"[extreme rows] {tag}: near-tie exceptions {exc}")


def _zero_weight_column(hd):
    """The hidden column at which the most kept rows have a zero weight."""
    lo = hd.o_packed[: hd.n_kept] & 0x7
    hi = (hd.o_packed[: hd.n_kept] >> 4) & 0x7
    zeros = np.empty((hd.n_kept, hd.hidden), dtype=bool)
    zeros[:, 0::2] = lo == 0
    zeros[:, 1::2] = hi == 0
    return int(np.argmax(zeros.sum(axis=0)))


@pytest.mark.parametrize("hidden", [256, 2560])
@pytest.mark.parametrize("special", ["inf", "nan"])
def test_row_with_a_non_finite_element(hidden, special):
    """Batch row 4 of a 16-row slice holds +inf or NaN at the column where
    the most head rows have a zero weight.  The other rows' top tokens,
    fp32 logits and dense linear are the oracle's; row 4's logits have the
    oracle's pattern of NaN and +-inf (a sum holding a NaN term, or
    infinities of both signs, is NaN in any order; else it is the infinity:
    0 * inf makes NaN where the weight is zero)."""
    hd = _head(hidden)
    col = _zero_weight_column(hd)
    B = 16
    x = np.random.default_rng(970 + hidden).standard_normal((B, hidden))
    x[4, col] = np.inf if special == "inf" else np.nan
    h = torch.from_numpy(x).to(torch.bfloat16)
    tag = f"{special} hidden={hidden} col={col}"
    say(f"[non-finite row] {tag}")
    hg = h.to(DEV)
    L = hd.oracle_logits(h)
    rows = np.array([b for b in range(B) if b != 4])
    ids = dh.draft_head_top_tokens(hd.packed, hd.scales, hd.gs, hd.idx_gpu,
                                   hg).cpu().numpy()
    _, want = oracle.argmax_remap(L[rows], hd.idx_o)
    H.check_top_tokens(ids[rows], L[rows], hd.idx_o, hd.n_kept, want)
    out = dh.draft_head_logits(hd.packed, hd.scales, hd.gs, hd.idx_gpu,
                               hd.n_kept, hd.vocab, hg).cpu().numpy()
    ref = oracle.logits_scatter(L, hd.n_kept, hd.idx_o, hd.vocab)
    fin = np.isfinite(ref[rows])
    assert np.array_equal(np.isfinite(out[rows]), fin), tag
    ok = H.close(out[rows][fin], ref[rows][fin])
    assert ok.all(), (tag, np.argwhere(~ok)[:5])
    y = dh.nvfp4_linear(hd.packed, hd.scales, hd.gs, hg).cpu().numpy()
    ok = H.close(y[rows], L[rows])
    assert ok.all(), (tag, np.argwhere(~ok)[:5])
    got, want4 = out[4], ref[4]
    assert np.array_equal(np.isnan(got), np.isnan(want4)), tag
    assert np.array_equal(np.isposinf(got), np.isposinf(want4)), tag
    assert np.array_equal(np.isneginf(got), np.isneginf(want4)), tag
    kept = want4[hd.idx_o[: hd.n_kept]]
    if special == "inf":  # rows with a zero weight there, and the others
        assert np.isnan(kept).any() and np.isinf(kept).any(), tag
    else:
        assert np.isnan(kept).all(), tag
