"""The plain streaming read (drafthead_read_probe), the measurement aid
bench.py times beside each step.  It must read every byte of both buffers:
a buffer of zeros holding DRAFTHEAD_READ_PROBE_MAGIC once makes exactly one
wave's XOR equal the constant, whatever the grid, so the sink is written;
all zeros leave it alone.  The constant is placed at the first word of a,
at the last 16 bytes of b, and where a ends inside a 1 KB line of the
joined sequence."""
import sys

import pytest
import torch

import reduced_vocab_nvfp4_amd as dh

pytestmark = pytest.mark.gpu
DEV = "cuda"
M = dh.READ_PROBE_MAGIC


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _buf(n_bytes):
    return torch.zeros(n_bytes // 4, dtype=torch.int32, device=DEV)


def _put(t, word_index):
    t[word_index] = torch.tensor(M, dtype=torch.int64).to(torch.int32)


def _sink_after(a, b):
    sink = dh.read_probe(a, b)
    torch.cuda.synchronize()
    return int(sink.item()) & 0xFFFFFFFF


@pytest.mark.parametrize("na,nb", [(1 << 20, 160 << 10),
                                   ((1 << 20) + 48, (3 << 20) + 16 * 7),
                                   (92257292 // 16 * 16, 0)])
def test_read_probe_reads_every_byte(na, nb):
    say(f"[read probe] a={na} b={nb}")
    a = _buf(na)
    b = _buf(nb) if nb else None
    assert _sink_after(a, b) == 0
    _put(a, 0)
    assert _sink_after(a, b) == M
    a.zero_()
    if b is not None:
        _put(b, nb // 4 - 4)          # the last 16 bytes of b
        assert _sink_after(a, b) == M
        b.zero_()
        _put(b, 0)                    # right after a's last byte
        assert _sink_after(a, b) == M
    else:
        _put(a, na // 4 - 1)          # a's last word
        assert _sink_after(a, b) == M
