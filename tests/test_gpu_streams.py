"""Calls on different streams with distinct workspaces run concurrently
and share no state: three step kinds enqueued on three streams (default
priority) without synchronizing between them give the results of the same
calls run alone."""
import pytest
import torch

import reduced_vocab_nvfp4_amd as dh
from reduced_vocab_nvfp4_amd import workloads as wl
from tests.test_gpu_formats import e4m3_head
from tests.test_gpu_parity import head

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_concurrent_calls_on_separate_streams():
    big = head("flash_next_64k")
    tiny = head("tiny")
    e4 = e4m3_head("tiny")
    hb = [wl.hidden_states(1, big.hidden, 1600 + i).to(DEV) for i in range(6)]
    ht = [wl.hidden_states(16, tiny.hidden, 1700 + i).to(DEV) for i in range(6)]
    # references, one call at a time
    ref_b = [dh.draft_head_top_tokens(big.packed, big.scales, big.gs,
                                      big.idx_gpu, h).clone() for h in hb]
    ref_t = [dh.draft_head_logits(tiny.packed, tiny.scales, tiny.gs,
                                  tiny.idx_gpu, tiny.n_kept, tiny.vocab,
                                  h).clone() for h in ht]
    ref_8 = [dh.draft_head_top_tokens_w8a8(e4.q, e4.scale, e4.idx_gpu,
                                           h).clone() for h in ht]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(3)]
    ws = [dh.new_workspace(big.n_rows, 1, DEV),
          dh.new_workspace(tiny.n_rows, 16, DEV),
          dh.new_workspace_w8a8(e4.n_rows, 16, e4.hidden, DEV)]
    outs_b = [torch.empty(1, dtype=torch.int32, device=DEV) for _ in hb]
    outs_t = [torch.empty((16, tiny.vocab), dtype=torch.float32, device=DEV)
              for _ in ht]
    outs_8 = [torch.empty(16, dtype=torch.int32, device=DEV) for _ in ht]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for i in range(6):
        dh.draft_head_top_tokens(big.packed, big.scales, big.gs, big.idx_gpu,
                                 hb[i], out_ids=outs_b[i], workspace=ws[0],
                                 stream=streams[0])
        dh.draft_head_logits(tiny.packed, tiny.scales, tiny.gs, tiny.idx_gpu,
                             tiny.n_kept, tiny.vocab, ht[i], out=outs_t[i],
                             workspace=ws[1], stream=streams[1])
        dh.draft_head_top_tokens_w8a8(e4.q, e4.scale, e4.idx_gpu, ht[i],
                                      out_ids=outs_8[i], workspace=ws[2],
                                      stream=streams[2])
    torch.cuda.synchronize()
    for i in range(6):
        assert torch.equal(outs_b[i], ref_b[i]), i
        assert torch.equal(outs_t[i], ref_t[i]), i
        assert torch.equal(outs_8[i], ref_8[i]), i


def test_calls_on_a_side_stream_allocate_there():
    """stream= without a workspace or outputs: the binding allocates them on
    that stream, so the workspace's zero-fill is ordered before the kernels
    and the memory is not handed to other work while they run.  The current
    stream is kept busy meanwhile (a long device sleep), so work wrongly
    ordered on it would come after the side stream's kernels."""
    tiny = head("tiny")
    w = tiny.w_gpu
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    hs = [wl.hidden_states(4, tiny.hidden, 1800 + i).to(DEV) for i in range(8)]
    ref = [dh.draft_head_top_tokens(tiny.packed, tiny.scales, tiny.gs,
                                    tiny.idx_gpu, h).clone() for h in hs]
    ref_q = dh.nvfp4_quantize_rows(w, tiny.idx_gpu)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(5e7))  # holds the current stream
    got = [dh.draft_head_top_tokens(tiny.packed, tiny.scales, tiny.gs,
                                    tiny.idx_gpu, h, stream=side)
           for h in hs]
    q = dh.nvfp4_quantize_rows(w, tiny.idx_gpu, stream=side)
    side.synchronize()
    for i in range(8):
        assert torch.equal(got[i], ref[i]), i
    for a, b in zip(q, ref_q):
        assert torch.equal(a, b)
    torch.cuda.synchronize()
