"""The C-ABI library without a GPU: it loads, exports what the header
declares, builds the row index exactly like the oracle, and rejects bad
arguments on the host before any device work."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import reduced_vocab_nvfp4_amd as dh
from reduced_vocab_nvfp4_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    for hdr in os.listdir(os.path.join(ROOT, "include")):
        if not hdr.endswith(".h"):
            continue
        text = open(os.path.join(ROOT, "include", hdr)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*([a-z_0-9]+)\s*\(",
                            text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert {"nvfp4_quantize_rows", "draft_head_top_tokens",
            "draft_head_logits"} <= set(names)
    L = ctypes.CDLL(dh.LIB_PATH)
    for n in names:
        assert hasattr(L, n), f"{n} declared but not exported"
    assert dh.lib().drafthead_abi_version() == 5
    assert dh.error_string(dh.DH_EINVAL).startswith("invalid")


def test_build_checks_the_version_the_header_declares():
    """__graft_entry__.build() compares the library's ABI version with the
    one include/drafthead.h declares, not with a copy of it."""
    import __graft_entry__ as ge
    assert ge.header_abi_version() == dh.lib().drafthead_abi_version()


@pytest.mark.parametrize("name", ["tiny", "flash_next_64k", "h98k_b16"])
def test_build_index_matches_oracle(name):
    keep = wl.keep_mask(wl.WORKLOADS[name])
    got, n_kept = dh.draft_head_build_index(keep)
    want, want_kept = oracle.build_index(keep)
    assert n_kept == want_kept
    assert np.array_equal(got.numpy(), want)


def test_build_index_edge_cases():
    for keep in ([True] * 64, [True] * 65, [False] * 99 + [True], [True]):
        got, n = dh.draft_head_build_index(np.array(keep))
        want, wn = oracle.build_index(np.array(keep))
        assert n == wn and np.array_equal(got.numpy(), want)
    with pytest.raises(dh.DraftHeadError):
        dh.draft_head_build_index(np.zeros(50, bool))


def test_workspace_bytes():
    assert dh.draft_head_workspace_bytes(64064, 1) >= 256 + 8 * 1024
    # a batch above one may run kernels with 16 partials per block
    assert (dh.draft_head_workspace_bytes(64064, 2)
            >= dh.draft_head_workspace_bytes(64064, 1) + 4096 * 15 * 8)
    assert (dh.draft_head_workspace_bytes(64064, 64)
            == dh.draft_head_workspace_bytes(64064, 2))
    assert dh.draft_head_workspace_bytes(0, 1) == 0
    assert dh.draft_head_workspace_bytes(64, 0) == 0
    assert dh.draft_head_workspace_bytes(64, 65) == 0


FAKE = 1 << 20  # an aligned non-null address that is never dereferenced


def test_quantize_rejects_bad_arguments_on_the_host():
    L = dh.lib()
    ws = dh.draft_head_workspace_bytes(64, 1)
    args = dict(w=FAKE, V=1000, H=256, ids=FAKE, n=64, p=FAKE, s=FAKE, g=FAKE,
                ws=FAKE, wsb=ws)

    def call(**kw):
        a = {**args, **kw}
        return L.nvfp4_quantize_rows(a["w"], a["V"], a["H"], a["ids"], a["n"],
                                     a["p"], a["s"], a["g"], a["ws"], a["wsb"],
                                     None)
    assert call(w=None) == dh.DH_EINVAL
    assert call(ids=None) == dh.DH_EINVAL
    assert call(H=24) == dh.DH_EINVAL
    assert call(H=0) == dh.DH_EINVAL
    assert call(n=0) == dh.DH_EINVAL
    assert call(V=0) == dh.DH_EINVAL
    assert call(w=FAKE + 2) == dh.DH_EINVAL
    assert call(ws=None) == dh.DH_EWORKSPACE
    assert call(wsb=ws - 1) == dh.DH_EWORKSPACE


def test_top_tokens_and_logits_reject_bad_arguments_on_the_host():
    L = dh.lib()
    ws = dh.draft_head_workspace_bytes(128, 8)
    base = dict(p=FAKE, s=FAKE, g=FAKE, idx=FAKE, n=128, H=256, h=FAKE, B=1,
                out=FAKE, ws=FAKE, wsb=ws)

    def top(**kw):
        a = {**base, **kw}
        return L.draft_head_top_tokens(a["p"], a["s"], a["g"], a["idx"], a["n"],
                                       a["H"], a["h"], a["B"], a["out"], a["ws"],
                                       a["wsb"], None)

    def logits(n_kept=100, vocab=1000, **kw):
        a = {**base, **kw}
        return L.draft_head_logits(a["p"], a["s"], a["g"], a["idx"], a["n"],
                                   n_kept, a["H"], vocab, a["h"], a["B"],
                                   a["out"], a["ws"], a["wsb"], None)
    for f in (top, logits):
        assert f(p=None) == dh.DH_EINVAL
        assert f(s=None) == dh.DH_EINVAL
        assert f(g=None) == dh.DH_EINVAL
        assert f(idx=None) == dh.DH_EINVAL
        assert f(h=None) == dh.DH_EINVAL
        assert f(out=None) == dh.DH_EINVAL
        assert f(n=100) == dh.DH_EINVAL       # not a multiple of 64
        assert f(n=0) == dh.DH_EINVAL
        assert f(H=40) == dh.DH_EINVAL        # not a multiple of 16
        assert f(H=0) == dh.DH_EINVAL
        assert f(B=0) == dh.DH_EINVAL
        assert f(B=65) == dh.DH_EINVAL
        assert f(p=FAKE + 8) == dh.DH_EINVAL  # packed must be 16-byte aligned
        assert f(ws=None) == dh.DH_EWORKSPACE
        assert f(wsb=16) == dh.DH_EWORKSPACE
    assert logits(n_kept=0) == dh.DH_EINVAL
    assert logits(n_kept=129) == dh.DH_EINVAL
    assert logits(vocab=50) == dh.DH_EINVAL
    assert logits(out=FAKE + 4) == dh.DH_EINVAL


def test_noalloc_top_tokens_rejects_bad_arguments_on_the_host():
    """The entry point without a workspace checks every argument before its
    first HIP call (the scratch address is fetched only after them)."""
    L = dh.lib()
    base = dict(p=FAKE, s=FAKE, g=FAKE, idx=FAKE, n=128, H=256, h=FAKE, B=1,
                out=FAKE)

    def top(**kw):
        a = {**base, **kw}
        return L.draft_head_top_tokens_noalloc(
            a["p"], a["s"], a["g"], a["idx"], a["n"], a["H"], a["h"], a["B"],
            a["out"], None)
    assert top(p=None) == dh.DH_EINVAL
    assert top(s=None) == dh.DH_EINVAL
    assert top(g=None) == dh.DH_EINVAL
    assert top(idx=None) == dh.DH_EINVAL
    assert top(h=None) == dh.DH_EINVAL
    assert top(out=None) == dh.DH_EINVAL
    assert top(out=FAKE + 2) == dh.DH_EINVAL
    assert top(n=100) == dh.DH_EINVAL
    assert top(H=40) == dh.DH_EINVAL
    assert top(B=0) == dh.DH_EINVAL
    assert top(B=65) == dh.DH_EINVAL     # beyond the largest batch
    assert top(p=FAKE + 8) == dh.DH_EINVAL
    # the largest workspace any batch needs is the scratch's size
    assert (dh.draft_head_workspace_bytes(1 << 20, 64)
            <= 1048832 == dh.draft_head_workspace_bytes(128, 64))


def test_read_probe_rejects_bad_arguments_on_the_host():
    """The measurement aid checks pointers, alignment and sizes before it
    launches anything."""
    L = dh.lib()

    def probe(a=FAKE, na=4096, b=FAKE, nb=4096, sink=FAKE):
        return L.drafthead_read_probe(a, na, b, nb, sink, None)
    assert probe(a=None) == dh.DH_EINVAL
    assert probe(sink=None) == dh.DH_EINVAL
    assert probe(a=FAKE + 8) == dh.DH_EINVAL
    assert probe(b=FAKE + 4) == dh.DH_EINVAL
    assert probe(sink=FAKE + 2) == dh.DH_EINVAL
    assert probe(na=100) == dh.DH_EINVAL
    assert probe(nb=24) == dh.DH_EINVAL
    assert probe(na=0, nb=0) == dh.DH_EINVAL
    assert probe(b=None) == dh.DH_EINVAL          # b_bytes > 0 needs b
    assert dh.READ_PROBE_MAGIC == 0x9E3779B9


def test_e4m3_quantize_rejects_bad_arguments_on_the_host():
    L = dh.lib()
    ws = dh.draft_head_workspace_bytes(64, 1)
    args = dict(w=FAKE, V=1000, H=256, ids=FAKE, n=64, q=FAKE, s=FAKE,
                ws=FAKE, wsb=ws)

    def call(**kw):
        a = {**args, **kw}
        return L.e4m3_quantize_rows_per_tensor(a["w"], a["V"], a["H"],
                                               a["ids"], a["n"], a["q"],
                                               a["s"], a["ws"], a["wsb"], None)
    for bad in (dict(w=None), dict(ids=None), dict(q=None), dict(s=None),
                dict(H=24), dict(H=0), dict(H=16400), dict(n=0), dict(V=0),
                dict(w=FAKE + 2), dict(q=FAKE + 4), dict(s=FAKE + 2)):
        assert call(**bad) == dh.DH_EINVAL, bad
    assert call(ws=None) == dh.DH_EWORKSPACE
    assert call(wsb=ws - 1) == dh.DH_EWORKSPACE


def test_e4m3_and_bf16_heads_reject_bad_arguments_on_the_host():
    L = dh.lib()
    ws = dh.draft_head_workspace_bytes(128, 8)
    base = dict(w=FAKE, s=FAKE, idx=FAKE, n=128, H=256, h=FAKE, B=1, out=FAKE,
                ws=FAKE, wsb=ws)

    def e4_top(**kw):
        a = {**base, **kw}
        return L.draft_head_top_tokens_e4m3(a["w"], a["s"], a["idx"], a["n"],
                                            a["H"], a["h"], a["B"], a["out"],
                                            a["ws"], a["wsb"], None)

    def e4_logits(n_kept=100, vocab=1000, **kw):
        a = {**base, **kw}
        return L.draft_head_logits_e4m3(a["w"], a["s"], a["idx"], a["n"],
                                        n_kept, a["H"], vocab, a["h"], a["B"],
                                        a["out"], a["ws"], a["wsb"], None)

    def bf_top(**kw):
        a = {**base, **kw}
        return L.draft_head_top_tokens_bf16(a["w"], a["idx"], a["n"], a["H"],
                                            a["h"], a["B"], a["out"], a["ws"],
                                            a["wsb"], None)

    def bf_logits(n_kept=100, vocab=1000, **kw):
        a = {**base, **kw}
        return L.draft_head_logits_bf16(a["w"], a["idx"], a["n"], n_kept,
                                        a["H"], vocab, a["h"], a["B"],
                                        a["out"], a["ws"], a["wsb"], None)
    for f in (e4_top, e4_logits, bf_top, bf_logits):
        for bad in (dict(w=None), dict(idx=None), dict(h=None),
                    dict(out=None), dict(n=100), dict(n=0), dict(H=40),
                    dict(H=0), dict(B=0), dict(B=65), dict(w=FAKE + 8),
                    dict(h=FAKE + 4)):
            assert f(**bad) == dh.DH_EINVAL, (f.__name__, bad)
        assert f(ws=None) == dh.DH_EWORKSPACE
        assert f(wsb=16) == dh.DH_EWORKSPACE
    assert e4_top(s=None) == dh.DH_EINVAL   # the E4M3 head needs its scale
    for f in (e4_logits, bf_logits):
        assert f(n_kept=0) == dh.DH_EINVAL
        assert f(n_kept=129) == dh.DH_EINVAL
        assert f(vocab=50) == dh.DH_EINVAL
        assert f(out=FAKE + 4) == dh.DH_EINVAL


def test_linear_rejects_bad_arguments_on_the_host():
    L = dh.lib()
    base = dict(p=FAKE, s=FAKE, g=FAKE, n=128, H=256, h=FAKE, B=1, out=FAKE)

    def lin(**kw):
        a = {**base, **kw}
        return L.nvfp4_linear(a["p"], a["s"], a["g"], a["n"], a["H"], a["h"],
                              a["B"], a["out"], None)
    assert lin(p=None) == dh.DH_EINVAL
    assert lin(s=None) == dh.DH_EINVAL
    assert lin(g=None) == dh.DH_EINVAL
    assert lin(h=None) == dh.DH_EINVAL
    assert lin(out=None) == dh.DH_EINVAL
    assert lin(n=100) == dh.DH_EINVAL        # not a multiple of 64
    assert lin(n=0) == dh.DH_EINVAL
    assert lin(H=40) == dh.DH_EINVAL         # not a multiple of 16
    assert lin(H=16400) == dh.DH_EINVAL
    assert lin(B=0) == dh.DH_EINVAL
    assert lin(B=65) == dh.DH_EINVAL
    assert lin(p=FAKE + 8) == dh.DH_EINVAL   # 16-byte alignment
    assert lin(out=FAKE + 4) == dh.DH_EINVAL
    assert lin(g=FAKE + 2) == dh.DH_EINVAL


def test_token_quantize_rejects_bad_arguments_on_the_host():
    L = dh.lib()
    base = dict(h=FAKE, B=4, H=256, qx=FAKE, sx=FAKE)

    def tq(**kw):
        a = {**base, **kw}
        return L.fp8_quantize_tokens(a["h"], a["B"], a["H"], a["qx"], a["sx"],
                                     None)
    assert tq(h=None) == dh.DH_EINVAL
    assert tq(qx=None) == dh.DH_EINVAL
    assert tq(sx=None) == dh.DH_EINVAL
    assert tq(B=0) == dh.DH_EINVAL
    assert tq(B=65537) == dh.DH_EINVAL
    assert tq(H=8) == dh.DH_EINVAL
    assert tq(H=40) == dh.DH_EINVAL
    assert tq(H=16400) == dh.DH_EINVAL
    assert tq(h=FAKE + 8) == dh.DH_EINVAL    # 16-byte alignment
    assert tq(qx=FAKE + 4) == dh.DH_EINVAL   # 8-byte alignment
    assert tq(sx=FAKE + 2) == dh.DH_EINVAL


def test_w8a8_workspace_and_arguments_on_the_host():
    """The W8A8 workspace is the top-token workspace plus the tokens' BF16
    activations, their E4M3 codes and scales; every call checks it on the
    host."""
    base = dh.draft_head_workspace_bytes(98304, 16)
    w = dh.draft_head_workspace_bytes_w8a8(98304, 16, 2560)
    assert w >= base + 16 * 2560 * 2 + 16 * 2560 + 16 * 4
    assert dh.draft_head_workspace_bytes_w8a8(98304, 16, 5120) > w
    assert dh.draft_head_workspace_bytes_w8a8(98304, 16, 40) == 0
    assert dh.draft_head_workspace_bytes_w8a8(0, 16, 2560) == 0
    assert dh.draft_head_workspace_bytes_w8a8(128, 65, 2560) == 0
    L = dh.lib()
    n, H, B = 128, 256, 4
    need = dh.draft_head_workspace_bytes_w8a8(n, B, H)
    args = dict(q=FAKE, s=FAKE, idx=FAKE, n=n, H=H, h=FAKE, B=B, out=FAKE,
                ws=FAKE, wsn=need)

    def top(**kw):
        a = {**args, **kw}
        return L.draft_head_top_tokens_w8a8(
            a["q"], a["s"], a["idx"], a["n"], a["H"], a["h"], a["B"], a["out"],
            a["ws"], a["wsn"], None)

    def lg(**kw):
        a = {**args, **kw}
        return L.draft_head_logits_w8a8(
            a["q"], a["s"], a["idx"], a["n"], a.get("nk", n), a["H"],
            a.get("V", 4096), a["h"], a["B"], a["out"], a["ws"], a["wsn"],
            None)
    for f in (top, lg):
        assert f(q=None) == dh.DH_EINVAL
        assert f(s=None) == dh.DH_EINVAL
        assert f(out=None) == dh.DH_EINVAL
        assert f(n=100) == dh.DH_EINVAL
        assert f(H=40) == dh.DH_EINVAL
        assert f(B=65) == dh.DH_EINVAL
        assert f(ws=None) == dh.DH_EWORKSPACE
        # big enough for the top-token workspace, not for the tokens
        assert f(wsn=dh.draft_head_workspace_bytes(n, B)) == dh.DH_EWORKSPACE
        assert f(wsn=need - 1) == dh.DH_EWORKSPACE
    assert lg(nk=0) == dh.DH_EINVAL
    assert lg(nk=n + 1) == dh.DH_EINVAL
    assert lg(V=64) == dh.DH_EINVAL
    assert lg(out=FAKE + 4) == dh.DH_EINVAL


def test_compat_calls_and_f16_quantize_reject_bad_arguments_on_the_host():
    L = dh.lib()
    n, H, B = 128, 256, 2
    ws = dh.draft_head_workspace_bytes(n, B)
    a = dict(p=FAKE, s=FAKE, g=FAKE, idx=FAKE, n=n, H=H, h=FAKE, B=B,
             out=FAKE, ws=FAKE, wsn=ws)

    def top(**kw):
        x = {**a, **kw}
        return L.draft_head_top_tokens_compat(
            x["p"], x["s"], x["g"], x["idx"], x["n"], x["H"], x["h"], x["B"],
            x["out"], x["ws"], x["wsn"], None)

    def lg(**kw):
        x = {**a, **kw}
        return L.draft_head_logits_compat(
            x["p"], x["s"], x["g"], x["idx"], x["n"], x.get("nk", n), x["H"],
            x.get("V", 4096), x["h"], x["B"], x["out"], x["ws"], x["wsn"], None)
    for f in (top, lg):
        assert f(p=None) == dh.DH_EINVAL
        assert f(s=None) == dh.DH_EINVAL
        assert f(g=None) == dh.DH_EINVAL
        assert f(out=None) == dh.DH_EINVAL
        assert f(n=100) == dh.DH_EINVAL
        assert f(B=0) == dh.DH_EINVAL
        assert f(ws=None) == dh.DH_EWORKSPACE
        assert f(wsn=ws - 1) == dh.DH_EWORKSPACE
    assert lg(nk=n + 1) == dh.DH_EINVAL
    assert lg(out=FAKE + 2) == dh.DH_EINVAL

    def q16(**kw):
        x = dict(w=FAKE, V=4096, H=256, ids=FAKE, n=128, p=FAKE, s=FAKE,
                 g=FAKE, ws=FAKE, wsn=dh.draft_head_workspace_bytes(128, 1))
        x.update(kw)
        return L.nvfp4_quantize_rows_f16(x["w"], x["V"], x["H"], x["ids"],
                                         x["n"], x["p"], x["s"], x["g"],
                                         x["ws"], x["wsn"], None)
    assert q16(w=None) == dh.DH_EINVAL
    assert q16(s=None) == dh.DH_EINVAL
    assert q16(H=40) == dh.DH_EINVAL
    assert q16(p=FAKE + 4) == dh.DH_EINVAL
    assert q16(ws=None) == dh.DH_EWORKSPACE


def test_binding_fails_loudly_without_the_library():
    """No CPU fallback: with the HIP library missing, the first call raises
    instead of computing anything another way."""
    import subprocess
    import sys
    code = ("import reduced_vocab_nvfp4_amd as dh\n"
            "dh.LIB_PATH = '/nonexistent/libdrafthead.so'\n"
            "dh._lib = None\n"
            "try:\n"
            "    dh.draft_head_workspace_bytes(64, 1)\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root,
                       capture_output=True, text=True, timeout=300)
    assert "raised:" in r.stdout and "not built" in r.stdout, r.stdout + r.stderr
