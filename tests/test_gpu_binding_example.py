"""The Python calls the README shows for one draft step (build the index,
quantize, a workspace, top tokens and logits), run as written on the tiny
workload at batch 16 and checked against the oracle: ids equal, logits
within the parity tolerance, -inf exactly where ids were not kept."""
import sys

import numpy as np
import pytest
import torch

import oracle
import reduced_vocab_nvfp4_amd as dh
from reduced_vocab_nvfp4_amd import workloads as wl
from tests import helpers as H

pytestmark = pytest.mark.gpu


def test_readme_draft_step():
    print("[binding example] tiny, batch 16", flush=True)
    sys.stdout.flush()
    w_ = wl.WORKLOADS["tiny"]
    w = wl.head_weight(w_.vocab, w_.hidden).cuda()
    keep = torch.from_numpy(wl.keep_mask(w_))
    h = wl.hidden_states(16, w_.hidden, 0).cuda()

    dh_idx, n_kept = dh.draft_head_build_index(keep)
    dh_idx = dh_idx.cuda()
    packed, scales, gs = dh.nvfp4_quantize_rows(w, dh_idx)
    ws = dh.new_workspace(dh_idx.shape[0], batch=16)
    ids = dh.draft_head_top_tokens(packed, scales, gs, dh_idx, h, workspace=ws)
    logits = dh.draft_head_logits(packed, scales, gs, dh_idx, n_kept,
                                  w.shape[0], h, workspace=ws)

    idx_o, nk = oracle.build_index(keep.numpy())
    assert nk == n_kept
    o = oracle.nvfp4_quantize(wl.bf16_bits(w.cpu()), idx_o)
    L = oracle.nvfp4_logits(*o, wl.bf16_bits(h.cpu()))
    _, want = oracle.argmax_remap(L, idx_o)
    H.check_top_tokens(ids.cpu().numpy(), L, idx_o, nk, want)
    ref = oracle.logits_scatter(L, nk, idx_o, w.shape[0])
    got = logits.cpu().numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin)
    assert np.all(got[~fin] == -np.inf)
    assert H.close(got[fin], ref[fin]).all()
