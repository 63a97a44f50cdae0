"""NVFP4 W4A16 linear (the drafter's other projections, page 1,
"q38_draft.py", install: the MTP block's 2-D weights with N % 64 == 0 and
K % 16 == 0 get the same quantized linear): GPU against the oracle's float64
GEMV of the same codes, within the logits tolerance."""
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


# (n_rows, hidden, batch): the drafter's fc projection (2 x 2560 -> 2560)
# and expanding / contracting projections at its hidden sizes, at batch 1
# (one-row kernel), 4 and 16 (MFMA) and 33 (two slices); a hidden size
# that only the generic kernel tiles; the smallest shape.  On the MFMA
# kernel the waves of a block split a unit's hidden dimension when the
# matrix has few 16-row units: 2560 x 5120 splits 8 ways over 10 slots,
# 5120 x 2560 4 ways over 5 slots (uneven parts), 1024 rows 4 ways;
# 24 000 and 40 960 rows do not split; hidden 2688 takes one-step slots (21
# per unit, split 16 ways); hidden 256 has one slot per unit and cannot
# split.
SHAPES = [(2560, 5120, 1), (10240, 2560, 1), (2560, 10240, 1),
          (5120, 2560, 4), (2560, 5120, 16), (1024, 2560, 33),
          (24000, 2560, 2), (40960, 2560, 16), (640, 2688, 8),
          (64, 256, 2), (128, 272, 3), (64, 16, 1)]


@pytest.mark.parametrize("n,hid,batch", SHAPES)
def test_linear_matches_the_oracle(n, hid, batch):
    rng = np.random.default_rng(n * 7 + hid + batch)
    w = torch.from_numpy((rng.standard_normal((n, hid)) * 0.02)
                         .astype(np.float32)).to(torch.bfloat16)
    rows = np.arange(n, dtype=np.int32)
    packed, scales, gs = dh.nvfp4_quantize_rows(
        w.to(DEV), torch.from_numpy(rows).to(DEV))
    op, os_, og = oracle.nvfp4_quantize(wl.bf16_bits(w), rows)
    assert np.array_equal(packed.cpu().numpy(), op)
    assert np.array_equal(scales.cpu().numpy(), os_)
    h = wl.hidden_states(batch, hid, 500 + batch)
    y = dh.nvfp4_linear(packed, scales, gs, h.to(DEV)).cpu().numpy()
    ref = oracle.nvfp4_logits(op, os_, og, wl.bf16_bits(h))
    assert y.shape == (batch, n) and np.isfinite(y).all()
    ok = H.close(y, ref)
    err = np.abs(y.astype(np.float64) - ref).max()
    say(f"[linear] {n}x{hid} B={batch}: max abs err {err:.3e}")
    assert ok.all(), np.argwhere(~ok)[:5]


def test_linear_writes_only_its_output():
    """The dense output covers exactly batch x n_rows floats: a guard band
    around it keeps its sentinel."""
    n, hid, batch = 256, 2560, 4
    rng = np.random.default_rng(3)
    w = torch.from_numpy((rng.standard_normal((n, hid)) * 0.02)
                         .astype(np.float32)).to(torch.bfloat16)
    packed, scales, gs = dh.nvfp4_quantize_rows(
        w.to(DEV), torch.arange(n, dtype=torch.int32, device=DEV))
    buf = torch.full((batch * n + 128,), 7.0, dtype=torch.float32, device=DEV)
    out = buf[64:64 + batch * n].view(batch, n)
    h = wl.hidden_states(batch, hid, 9).to(DEV)
    dh.nvfp4_linear(packed, scales, gs, h, out=out)
    b = buf.cpu().numpy()
    assert (b[:64] == 7.0).all() and (b[64 + batch * n:] == 7.0).all()
    assert np.isfinite(b[64:64 + batch * n]).all()
