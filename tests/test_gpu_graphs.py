"""HIP graph replay of every step kind: a call captured once and replayed
with new inputs gives the eager result on every replay (no kernel here
records a memset, the workspace state advances on the device, and the W8A8
scratch is rewritten before it is read).  Eager runs and replays alternate
with synchronizations between them."""
import sys

import pytest
import torch

import reduced_vocab_nvfp4_amd as dh
from reduced_vocab_nvfp4_amd import workloads as wl
from tests.test_gpu_formats import e4m3_head
from tests.test_gpu_parity import head

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _check_replays(run, B, hidden, seed, tag, replays=5):
    """run(h, out=None, fresh=False) -> out tensor.  Captured once with a
    static h and output, replayed with fresh h against an eager call
    (fresh=True: its own workspace and output)."""
    h_static = torch.zeros(B, hidden, dtype=torch.bfloat16, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up call outside the capture
        out_static = run(h_static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(h_static, out=out_static)
    for k in range(replays):
        h = wl.hidden_states(B, hidden, seed + k).to(DEV)
        want = run(h, fresh=True).clone()
        torch.cuda.synchronize()
        h_static.copy_(h)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_static.view(torch.uint8),
                           want.view(torch.uint8)), (tag, k)
    say(f"[graph] {tag}: {replays} replays match")


def _runner(call, ws_size):
    """Wraps call(h, out, ws) with a persistent workspace for the captured
    call and a separate one for the eager reference."""
    ws_cap = torch.zeros(ws_size, dtype=torch.uint8, device=DEV) if ws_size else None
    ws_ref = torch.zeros(ws_size, dtype=torch.uint8, device=DEV) if ws_size else None

    def run(h, out=None, fresh=False):
        return call(h, out, ws_ref if fresh else ws_cap)
    return run


@pytest.mark.parametrize("B", [1, 16])
def test_graph_w8a8_top_tokens(B):
    e4 = e4m3_head("tiny")
    run = _runner(lambda h, out, ws: dh.draft_head_top_tokens_w8a8(
        e4.q, e4.scale, e4.idx_gpu, h, out_ids=out, workspace=ws),
        dh.draft_head_workspace_bytes_w8a8(e4.n_rows, B, e4.hidden))
    _check_replays(run, B, e4.hidden, 1000 + B, f"w8a8 top B={B}")


def test_graph_w8a8_logits():
    e4 = e4m3_head("tiny")
    B = 5
    run = _runner(lambda h, out, ws: dh.draft_head_logits_w8a8(
        e4.q, e4.scale, e4.idx_gpu, e4.n_kept, e4.vocab, h, out=out,
        workspace=ws),
        dh.draft_head_workspace_bytes_w8a8(e4.n_rows, B, e4.hidden))
    _check_replays(run, B, e4.hidden, 1100, "w8a8 logits B=5")


@pytest.mark.parametrize("name,B", [("flash_next_64k", 1), ("tiny", 5)])
def test_graph_logits_fp32_and_bf16(name, B):
    hd = head(name)
    ws = dh.draft_head_workspace_bytes(hd.n_rows, B)
    run = _runner(lambda h, out, w: dh.draft_head_logits(
        hd.packed, hd.scales, hd.gs, hd.idx_gpu, hd.n_kept, hd.vocab, h,
        out=out, workspace=w), ws)
    _check_replays(run, B, hd.hidden, 1200 + B, f"{name} logits B={B}")
    run = _runner(lambda h, out, w: dh.draft_head_logits_compat(
        hd.packed, hd.scales, hd.gs, hd.idx_gpu, hd.n_kept, hd.vocab, h,
        out=out, workspace=w), ws)
    _check_replays(run, B, hd.hidden, 1300 + B, f"{name} BF16 logits B={B}")
    run = _runner(lambda h, out, w: dh.draft_head_top_tokens_compat(
        hd.packed, hd.scales, hd.gs, hd.idx_gpu, h, out_ids=out,
        workspace=w), ws)
    _check_replays(run, B, hd.hidden, 1400 + B, f"{name} BF16 top B={B}")


@pytest.mark.parametrize("B", [1, 16])
def test_graph_linear(B):
    hd = head("tiny")
    run = _runner(lambda h, out, ws: dh.nvfp4_linear(
        hd.packed, hd.scales, hd.gs, h, out=out), 0)
    _check_replays(run, B, hd.hidden, 1500 + B, f"linear B={B}")
