"""draft_head_top_tokens_noalloc (the library's own static scratch in place
of a caller's workspace) against draft_head_top_tokens, through the C-ABI:
the same ids, bit for bit, on consecutive calls whose batch shrinks (16 then
3 rows, 64 then 1: the batched and the one-row kernels), on two head
shapes; both also against the oracle's argmax.  A batch beyond the largest
the scratch holds is refused."""
import sys

import numpy as np
import pytest
import torch

import oracle
import reduced_vocab_nvfp4_amd as dh
from reduced_vocab_nvfp4_amd import workloads as wl
from tests import helpers as H
from tests.test_gpu_parity import Head

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _args(hd, h, out):
    return (hd.packed.data_ptr(), hd.scales.data_ptr(), hd.gs.data_ptr(),
            hd.idx_gpu.data_ptr(), hd.n_rows, hd.hidden, h.data_ptr(),
            h.shape[0], out.data_ptr())


def _pair(hd, h):
    """(ids from the no-allocation call, ids from the workspace call)."""
    L = dh.lib()
    stream = torch.cuda.current_stream().cuda_stream
    out_a = torch.full((h.shape[0],), -7, dtype=torch.int32, device=DEV)
    out_b = torch.full((h.shape[0],), -7, dtype=torch.int32, device=DEV)
    rc = L.draft_head_top_tokens_noalloc(*_args(hd, h, out_a), stream)
    assert rc == dh.DH_OK, dh.error_string(rc)
    ws = dh.new_workspace(hd.n_rows, h.shape[0], DEV)
    rc = L.draft_head_top_tokens(*_args(hd, h, out_b), ws.data_ptr(),
                                 ws.numel(), stream)
    assert rc == dh.DH_OK, dh.error_string(rc)
    torch.cuda.synchronize()
    return out_a.cpu().numpy(), out_b.cpu().numpy()


@pytest.mark.parametrize("hidden", [256, 2560])
def test_noalloc_matches_the_workspace_entry_point(hidden):
    hd = Head("tiny", hidden=hidden)
    for seq in ((16, 3), (64, 1)):
        for i, B in enumerate(seq):
            say(f"[noalloc] hidden={hidden} call {i + 1} of {seq}: B={B}")
            h = wl.hidden_states(B, hidden, 800 + 10 * B + hidden).to(DEV)
            a, b = _pair(hd, h)
            assert np.array_equal(a, b), (hidden, B, a, b)
            L64 = hd.oracle_logits(h.cpu())
            _, want = oracle.argmax_remap(L64, hd.idx_o)
            H.check_top_tokens(a, L64, hd.idx_o, hd.n_kept, want)


def test_noalloc_refuses_a_batch_beyond_the_scratch():
    hd = Head("tiny")
    h = torch.zeros((65, hd.hidden), dtype=torch.bfloat16, device=DEV)
    out = torch.zeros(65, dtype=torch.int32, device=DEV)
    rc = dh.lib().draft_head_top_tokens_noalloc(
        *_args(hd, h, out), torch.cuda.current_stream().cuda_stream)
    assert rc == dh.DH_EINVAL
