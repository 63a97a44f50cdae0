"""Pins of the CPU oracle against things other than itself.

Every step of the oracle is checked here against a library routine, a
closed form, a brute-force search with exact rationals, a hand-derived
fixture, or an invariant, chosen so that a dropped term, a wrong sign, a
swapped nibble or index, a wrong constant or a wrong tie rule fails a test.
None of these tests needs a GPU.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from reduced_vocab_nvfp4_amd import workloads as wl
from tests import helpers as H

# --------------------------------------------------------------- E4M3 pins


def _torch_e4m3_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_all_codes_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert list(np.flatnonzero(nan)) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_e4m3_encode_roundtrips_every_finite_code():
    for c in range(127):
        assert oracle.e4m3_code(oracle.e4m3_value(c)) == c


def test_e4m3_encode_every_midpoint_ties_to_even_and_neighbours_round():
    for c in range(126):
        lo, hi = oracle.e4m3_value(c), oracle.e4m3_value(c + 1)
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2  # exact in binary32
        even = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_code(mid) == even
        assert oracle.e4m3_code(np.nextafter(mid, np.float32(0))) == c
        assert oracle.e4m3_code(np.nextafter(mid, np.float32(1e9))) == c + 1
        assert _torch_e4m3_bits(np.array([mid]))[0] == even


def test_e4m3_encode_matches_torch_cast_on_random_values():
    rng = np.random.default_rng(123)
    x = np.concatenate([
        np.exp2(rng.uniform(-14, 9, 20000)),
        rng.uniform(0, 448, 20000),
        rng.uniform(0, 2.0 ** -6, 5000),
        np.array([0.0, 2.0 ** -10, 2.0 ** -10 * 3, 17.0, 19.0, 448.0]),
    ]).astype(np.float32)
    want = _torch_e4m3_bits(np.minimum(x, np.float32(448)))
    got = np.array([oracle.e4m3_code(v) for v in x], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_e4m3_encode_saturates_instead_of_nan():
    for v in [448.0, 448.5, 463.99, 464.0, 480.0, 1e30, float("inf")]:
        assert oracle.e4m3_code(v) == 0x7E
    assert oracle.e4m3_code(2.0 ** -10) == 0x00   # tie between 0 and 2^-9
    assert oracle.e4m3_code(17.0) == 0x58          # 16
    assert oracle.e4m3_code(19.0) == 0x5A          # 20


# --------------------------------------------------------------- e2m1 pins

def _e2m1_bruteforce(q: float) -> int:
    """Nearest e2m1 magnitude by exact rationals, ties to the code whose
    mantissa bit is 0, saturating at 6; sign from the float's sign bit."""
    x = abs(Fraction(float(q)))
    best = None
    for code in range(8):
        v = H.e2m1_from_bits(code)
        d = abs(x - v)
        key = (d, code & 1)
        if best is None or key < best[0]:
            best = (key, code)
    code = best[1]
    if x > 6:
        code = 7
    sign = 8 if np.signbit(np.float32(q)) else 0
    return sign | code


def test_e2m1_values_match_bit_field_definition():
    for n in range(16):
        assert oracle.e2m1_value(n) == float(H.e2m1_from_bits(n))


def test_e2m1_encode_matches_bruteforce():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    vals = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, 6.0001, 7.0, 1e9, 1e-30]
    xs = []
    for m in mids + vals:
        m = np.float32(m)
        xs += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1e9))]
    rng = np.random.default_rng(7)
    xs += list(rng.uniform(0, 7, 4000).astype(np.float32))
    xs += [-x for x in xs]
    xs += [np.float32(-0.0), np.float32(-1e-30)]
    for x in xs:
        assert oracle.e2m1_code(x) == _e2m1_bruteforce(x), x
    # the tie cases, spelled out
    assert [oracle.e2m1_code(v) for v in mids] == [0, 2, 2, 4, 4, 6, 6]
    assert oracle.e2m1_code(-0.0) == 8 and oracle.e2m1_code(-0.1) == 8


# ------------------------------------------------------------- C1 row index

def test_build_index_properties_on_the_workloads():
    for name, pads in [("tiny", 0), ("flash_next_64k", 38)]:
        w = wl.WORKLOADS[name]
        keep = wl.keep_mask(w)
        idx, n_kept = oracle.build_index(keep)
        assert n_kept == w.n_keep
        assert idx.shape[0] % 64 == 0 and idx.shape[0] - n_kept == pads
        assert np.array_equal(idx[:n_kept], np.flatnonzero(keep))
        assert np.all(idx[n_kept:] == idx[0])
    idx, n = oracle.build_index(np.ones(64, bool))
    assert n == 64 and np.array_equal(idx, np.arange(64))
    keep = np.zeros(200, bool)
    keep[[5, 7, 100]] = True
    idx, n = oracle.build_index(keep)
    assert n == 3 and idx.shape[0] == 64 and list(idx[:4]) == [5, 7, 100, 5]
    with pytest.raises(ValueError):
        oracle.build_index(np.zeros(10, bool))


# ----------------------------------------------------- C2-C4 quantization

def _bits(t: torch.Tensor) -> np.ndarray:
    return wl.bf16_bits(t)


def _unpack(packed: np.ndarray) -> np.ndarray:
    n, H2 = packed.shape
    out = np.empty((n, 2 * H2), dtype=np.uint8)
    out[:, 0::2] = packed & 15
    out[:, 1::2] = packed >> 4
    return out


def _pack(nib: np.ndarray) -> np.ndarray:
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def _roundtrip_construction(rng, n_rows, hidden):
    """Codes and scales chosen so that quantizing their exact product must
    give them back: every block holds a +-6, one block has scale 448, so
    amax = 6*448*2^-8 = 10.5 and gs = 10.5/2688 = 2^-8 exactly."""
    nblk = hidden // 16
    nib = rng.integers(0, 16, size=(n_rows, hidden)).astype(np.uint8)
    pos = rng.integers(0, 16, size=(n_rows, nblk))
    for j in range(n_rows):
        for b in range(nblk):
            nib[j, b * 16 + pos[j, b]] = 7 | (8 * rng.integers(0, 2))
    scales = rng.integers(1, 0x7E, size=(n_rows, nblk)).astype(np.uint8)
    scales[0, 0] = 0x7E
    vals = H.E2M1_TABLE[nib]
    sc = torch.from_numpy(scales).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    w = vals * np.repeat(sc, 16, axis=1) * 2.0 ** -8
    wt = torch.from_numpy(w).to(torch.bfloat16)
    assert np.array_equal(wt.to(torch.float64).numpy(), w)  # exact in BF16
    return _pack(nib), scales, wt


def test_quantize_roundtrip_construction_is_exact():
    rng = np.random.default_rng(11)
    packed, scales, wt = _roundtrip_construction(rng, 128, 64)
    idx = np.arange(128, dtype=np.int32)
    p2, s2, gs = oracle.nvfp4_quantize(_bits(wt), idx)
    assert gs == np.float32(2.0 ** -8)
    assert np.array_equal(s2, scales)
    assert np.array_equal(p2, packed)


def test_quantize_invariants():
    rng = np.random.default_rng(5)
    w = torch.from_numpy(rng.standard_normal((300, 96)).astype(np.float32) * 0.02
                         ).to(torch.bfloat16)
    idx = rng.permutation(300)[:128].astype(np.int32)
    p, s, gs = oracle.nvfp4_quantize(_bits(w), idx)
    # gs comes from the gathered rows only, in one float32 division
    amax = np.float32(np.abs(w.float().numpy()[idx]).max())
    assert gs == np.float32(max(amax, np.float32(1e-12)) / np.float32(2688))
    # the block holding amax gets the largest scale; no NaN code appears
    assert (s == 0x7E).any() and not ((s & 0x7F) == 0x7F).any()
    # scaling by a power of two leaves codes alone and scales gs exactly
    for k in (-4, 3):
        p2, s2, gs2 = oracle.nvfp4_quantize(_bits(w * 2.0 ** k), idx)
        assert np.array_equal(p2, p) and np.array_equal(s2, s)
        assert gs2 == np.float32(gs * 2.0 ** k)
    # negation flips exactly the sign bit of every nibble
    p3, s3, gs3 = oracle.nvfp4_quantize(_bits(-w), idx)
    assert np.array_equal(s3, s) and gs3 == gs
    assert np.array_equal(p3, p ^ 0x88)
    # permuting the index permutes the rows
    perm = rng.permutation(128)
    p4, s4, gs4 = oracle.nvfp4_quantize(_bits(w), idx[perm])
    assert gs4 == gs and np.array_equal(p4, p[perm]) and np.array_equal(s4, s[perm])
    # pad rows (copies of the first id) repeat row 0
    idxp = np.concatenate([idx[:100], np.full(28, idx[0], np.int32)])
    p5, s5, _ = oracle.nvfp4_quantize(_bits(w), idxp)
    assert np.all(p5[100:] == p5[0]) and np.all(s5[100:] == s5[0])


def test_quantize_zero_head_uses_the_floor():
    w = torch.zeros((64, 32), dtype=torch.bfloat16)
    w[3, 5] = -0.0
    p, s, gs = oracle.nvfp4_quantize(_bits(w), np.arange(64, dtype=np.int32))
    assert gs == np.float32(np.float32(1e-12) / np.float32(2688))
    assert not s.any()
    nib = _unpack(p)
    assert nib[3, 5] == 8 and nib.sum() == 8


def test_quantize_matches_an_independent_float32_recipe():
    """The NVFP4 recipe restated with numpy float32 array ops and torch's
    float8 cast (scales) on random data; element codes through the
    brute-force e2m1 encoder."""
    rng = np.random.default_rng(9)
    w = torch.from_numpy(rng.standard_normal((70, 48)).astype(np.float32) * 0.02
                         ).to(torch.bfloat16)
    idx = rng.permutation(70)[:64].astype(np.int32)
    p, s, gs = oracle.nvfp4_quantize(_bits(w), idx)
    x = w.float().numpy()[idx]
    amax = np.abs(x).max()
    gs_ref = np.float32(np.maximum(amax, np.float32(1e-12)) / np.float32(2688))
    bmax = np.abs(x.reshape(64, 3, 16)).max(axis=2)
    sref = _torch_e4m3_bits(bmax / (np.float32(6) * gs_ref))
    assert gs == gs_ref and np.array_equal(s, sref)
    sdec = torch.from_numpy(sref).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    d = (sdec * gs_ref).astype(np.float32)
    q = (x.reshape(64, 3, 16) / d[:, :, None]).reshape(64, 48)
    nib = np.array([[_e2m1_bruteforce(v) for v in row] for row in q], np.uint8)
    assert np.array_equal(_unpack(p), nib)


# --------------------------------------------------------------- C5 GEMV

def test_logits_hand_cases():
    g = H.golden("gemv_hand_cases.json")
    for case in g["cases"]:
        packed, scales, gs, h_bits, expected, amax_row = H.load_gemv_case(
            case, g["hidden"], g["rows"])
        L = oracle.nvfp4_logits(packed, scales, gs, h_bits)
        assert np.array_equal(L[0], expected), case["name"]
        rows, ids = oracle.argmax_remap(L, np.arange(g["rows"], dtype=np.int32))
        assert rows[0] == amax_row


def test_logits_match_torch_float64_matmul():
    rng = np.random.default_rng(3)
    n, Hd, B = 192, 96, 3
    packed = rng.integers(0, 256, size=(n, Hd // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, size=(n, Hd // 16), dtype=np.uint8)
    gs = np.float32(0.0123)
    h = torch.from_numpy(rng.standard_normal((B, Hd))).to(torch.bfloat16)
    L = oracle.nvfp4_logits(packed, scales, gs, _bits(h))
    Wd = H.dequant_nvfp4_torch(packed, scales, gs)
    ref = (h.to(torch.float64) @ Wd.T).numpy()
    np.testing.assert_allclose(L, ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------ C6 argmax + remap

def test_argmax_first_maximal_row_and_remap():
    rng = np.random.default_rng(4)
    L = rng.standard_normal((5, 256))
    L[1, 17] = L[1, 200] = L[1].max() + 1.0     # tie: the lower row wins
    L[2, :] = 0.0
    L[2, 3] = -0.0                                # -0 == +0: row 0 wins
    L[3, 0] = L[3].max() + 1.0
    L[3, 250:] = L[3, 0]                          # pads duplicate row 0
    idx = rng.permutation(10000)[:256].astype(np.int32)
    rows, ids = oracle.argmax_remap(L, idx)
    ref = torch.argmax(torch.from_numpy(L), dim=1).numpy()
    assert np.array_equal(rows, ref)
    assert rows[1] == 17 and rows[2] == 0 and rows[3] == 0
    assert np.array_equal(ids, idx[rows])


# --------------------------------------------------------------- C7 scatter

def test_scatter_matches_index_copy_and_skips_pads():
    rng = np.random.default_rng(6)
    V, n_kept = 1000, 100
    keep = np.zeros(V, bool)
    keep[rng.choice(V, n_kept, replace=False)] = True
    idx, nk = oracle.build_index(keep)
    L = rng.standard_normal((2, idx.shape[0]))
    out = oracle.logits_scatter(L, nk, idx, V)
    ref = torch.full((2, V), float("-inf"), dtype=torch.float32)
    ref.index_copy_(1, torch.from_numpy(idx[:nk]).long(),
                    torch.from_numpy(L[:, :nk]).float())
    assert np.array_equal(out, ref.numpy())
    assert (np.isfinite(out).sum(axis=1) == nk).all()
    assert (out.view(np.uint32)[~np.isfinite(out)] == 0xFF800000).all()


# ---------------------------------------------------------- C8 BF16 head

def test_bf16_logits_match_torch_float64_matmul():
    rng = np.random.default_rng(8)
    w = torch.from_numpy(rng.standard_normal((300, 80)) * 0.02).to(torch.bfloat16)
    h = torch.from_numpy(rng.standard_normal((2, 80))).to(torch.bfloat16)
    rows = np.arange(300, dtype=np.int32)
    L = oracle.bf16_logits(_bits(w), rows, _bits(h))
    ref = (h.to(torch.float64) @ w.to(torch.float64).T).numpy()
    np.testing.assert_allclose(L, ref, rtol=1e-13, atol=1e-13)


# -------------------------------------------------- C9 E4M3 per-tensor head

def test_e4m3_tensor_quantize_matches_the_torch_recipe():
    """Bit-exact against the FP8 head conversion written with torch ops:
    float32 amax with a 1e-12 floor, divide by 448, divide, clamp, cast."""
    rng = np.random.default_rng(10)
    w = torch.from_numpy(rng.standard_normal((200, 64)).astype(np.float32) * 0.02
                         ).to(torch.bfloat16)
    w[7, 3] = -0.0
    idx = rng.permutation(200)[:128].astype(np.int32)
    q, scale = oracle.e4m3_tensor_quantize(_bits(w), idx)
    wf = w[torch.from_numpy(idx).long()].float()
    fmax = torch.finfo(torch.float8_e4m3fn).max
    amax = wf.abs().amax().clamp_min(1e-12)
    sref = amax / fmax
    qref = (wf / sref).clamp(-fmax, fmax).to(torch.float8_e4m3fn).view(torch.uint8)
    assert scale == np.float32(sref.item())
    assert np.array_equal(q, qref.numpy())
    h = torch.from_numpy(rng.standard_normal((2, 64))).to(torch.bfloat16)
    L = oracle.e4m3_tensor_logits(q, scale, _bits(h))
    ref = (h.to(torch.float64) @ (qref.view(torch.float8_e4m3fn).to(torch.float64)
                                  * float(scale)).T).numpy()
    np.testing.assert_allclose(L, ref, rtol=1e-12, atol=1e-12)


def _torch_token_recipe(hf: torch.Tensor):
    """Per-token dynamic E4M3 quantization written with torch ops: float32
    row amax with a 1e-12 floor, divide by 448, divide, clamp, cast."""
    fmax = torch.finfo(torch.float8_e4m3fn).max
    sref = hf.abs().amax(dim=1).clamp_min(1e-12) / fmax
    qref = (hf / sref[:, None]).clamp(-fmax, fmax).to(torch.float8_e4m3fn)
    return qref.view(torch.uint8), sref


def test_fp8_tokens_quantize_matches_the_torch_recipe():
    """Bit-exact against the torch recipe, one scale per row: rows of random
    values, an all-zero row (the 1e-12 floor), signed zeros, a row with one
    large value among tiny ones (codes that underflow to zero keep their
    sign), and a row whose scale is a power of two."""
    rng = np.random.default_rng(11)
    h = torch.from_numpy(rng.standard_normal((7, 96))).to(torch.bfloat16)
    h[1] = 0.0
    h[2, 5] = -0.0
    h[3] = torch.from_numpy(rng.standard_normal(96) * 1e-6).to(torch.bfloat16)
    h[3, 0] = 1000.0
    h[4] = torch.linspace(-3.5, 3.5, 96).to(torch.bfloat16)
    h[4, 0] = 448.0  # scale exactly 1
    qx, sx = oracle.fp8_tokens_quantize(_bits(h))
    qref, sref = _torch_token_recipe(h.float())
    assert np.array_equal(sx, sref.numpy())
    assert np.array_equal(qx, qref.numpy())
    assert sx[1] == np.float32(np.float32(1e-12) / np.float32(448))
    assert sx[4] == 1.0
    assert (qx[3] == 0x80).any() and qx[3, 0] == 0x7E


def test_fp8_tokens_scale_is_per_row():
    """Scaling one row of h by a power of two scales its sx by the same
    factor, leaves its codes unchanged and leaves every other row alone --
    which a per-tensor scale would not."""
    rng = np.random.default_rng(12)
    h = torch.from_numpy(rng.standard_normal((3, 64))).to(torch.bfloat16)
    q0, s0 = oracle.fp8_tokens_quantize(_bits(h))
    h2 = h.clone()
    h2[1] *= 2.0 ** 5
    q1, s1 = oracle.fp8_tokens_quantize(_bits(h2))
    assert np.array_equal(q0, q1)
    assert s1[1] == s0[1] * np.float32(32) and s1[0] == s0[0] and s1[2] == s0[2]


def test_w8a8_logits_match_a_float64_matmul():
    """The W8A8 logits against a float64 torch matmul of both operands
    decoded through torch's float8_e4m3fn dtype, times sx[b] * sw; and the
    hand case of one nonzero code on each side."""
    rng = np.random.default_rng(13)
    w = torch.from_numpy(rng.standard_normal((128, 80)).astype(np.float32) * 0.02
                         ).to(torch.bfloat16)
    q, sw = oracle.e4m3_tensor_quantize(_bits(w), np.arange(128, dtype=np.int32))
    h = torch.from_numpy(rng.standard_normal((3, 80))).to(torch.bfloat16)
    qx, sx = oracle.fp8_tokens_quantize(_bits(h))
    L = oracle.w8a8_logits(q, sw, qx, sx)
    dw = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64)
    dx = torch.from_numpy(qx).view(torch.float8_e4m3fn).to(torch.float64)
    ref = (dx @ dw.T) * torch.from_numpy(sx).double()[:, None] * float(sw)
    np.testing.assert_allclose(L, ref.numpy(), rtol=1e-12, atol=0)
    # one code of 2.0 (0x40) in the head against one of -0.5 (0xB0) in the
    # token at the same k: sx * sw * 2 * -0.5
    qh = np.zeros((64, 16), dtype=np.uint8)
    qh[9, 4] = 0x40
    qt = np.zeros((1, 16), dtype=np.uint8)
    qt[0, 4] = 0xB0
    L1 = oracle.w8a8_logits(qh, np.float32(0.25), qt, np.array([8.0], np.float32))
    assert L1[0, 9] == -2.0 and np.count_nonzero(L1) == 1


# ------------------------------------- reference-compatible mode (C12)

def test_f16_decode_all_codes_matches_numpy():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = codes.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_value(c) for c in range(65536)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert oracle.f16_value(0x0001) == 2.0 ** -24
    assert oracle.f16_value(0x7BFF) == 65504.0


def test_nvfp4_quantize_f16_roundtrip_construction():
    """The exact construction of the BF16 pin, stored as FP16 (every value
    is exact there too): the FP16 quantizer returns its codes and scales."""
    rng = np.random.default_rng(14)
    packed, scales, wt = _roundtrip_construction(rng, 128, 64)
    w64 = wt.to(torch.float64).numpy()
    w16 = w64.astype(np.float16)
    assert np.array_equal(w16.astype(np.float64), w64)
    p2, s2, gs = oracle.nvfp4_quantize_f16(w16.view(np.uint16),
                                           np.arange(128, dtype=np.int32))
    assert gs == np.float32(2.0 ** -8)
    assert np.array_equal(s2, scales) and np.array_equal(p2, packed)


def test_nvfp4_quantize_f16_agrees_with_bf16_on_shared_values():
    """A head whose values are exact in both FP16 and BF16 quantizes to the
    same codes, scales and gs from either; an FP16-only mantissa changes
    codes where the BF16 rounding of the same head would."""
    rng = np.random.default_rng(15)
    # magnitudes in [2^-12, 0.1]: FP16 normals, where every BF16 value fits
    mag = rng.uniform(2.0 ** -12, 0.1, (256, 96))
    sign = np.where(rng.integers(0, 2, (256, 96)) == 1, -1.0, 1.0)
    w = torch.from_numpy((mag * sign).astype(np.float32)).to(torch.bfloat16)
    w64 = w.to(torch.float64).numpy()
    w16 = w64.astype(np.float16)
    assert np.array_equal(w16.astype(np.float64), w64)
    idx = rng.permutation(256)[:128].astype(np.int32)
    a = oracle.nvfp4_quantize(_bits(w), idx)
    b = oracle.nvfp4_quantize_f16(w16.view(np.uint16), idx)
    assert a[2] == b[2] and np.array_equal(a[1], b[1]) and np.array_equal(a[0], b[0])
    x = (rng.standard_normal((128, 96)) * 0.02).astype(np.float16)
    c = oracle.nvfp4_quantize_f16(x.view(np.uint16), np.arange(128, dtype=np.int32))
    d = oracle.nvfp4_quantize(_bits(torch.from_numpy(x.astype(np.float32))
                                    .to(torch.bfloat16)),
                              np.arange(128, dtype=np.int32))
    assert not np.array_equal(c[0], d[0])


def test_bf16_code_matches_torch():
    """Round to nearest, ties to even, against torch's float32 -> bfloat16
    cast: random magnitudes over 2^-126..2^120 of both signs, every exact
    tie of a range of BF16 pairs, and values just off the ties."""
    rng = np.random.default_rng(16)
    x = (rng.standard_normal(4000) * np.exp2(rng.integers(-126, 120, 4000))
         ).astype(np.float32)
    top = np.array([3.3895e38, 3.39e38, 3.3961e38, 3.3962e38, 3.4e38],
                   dtype=np.float32)  # around the largest BF16 and overflow
    x = np.concatenate([x, top, -top])
    base = np.arange(0x3F80, 0x3F80 + 256, dtype=np.uint32) << 16
    ties = (base | 0x8000).view(np.float32)
    near = np.concatenate([np.nextafter(ties, np.float32(0)),
                           np.nextafter(ties, np.float32(np.inf))])
    vals = np.concatenate([x, ties, -ties, near, [0.0, -0.0]]).astype(np.float32)
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy()
    got = np.array([oracle.bf16_code(v) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref.view(np.uint16))


def test_logits_to_bf16_rounds_through_float32():
    """The float64 logit goes to float32 first (the accumulator's
    precision), then to BF16: 1 + 2^-8 + 2^-30 becomes the tie 1 + 2^-8 in
    float32 and then 1.0, where a direct rounding would give 1 + 2^-7."""
    L = np.array([[1 + 2.0 ** -8 + 2.0 ** -30, -(1 + 2.0 ** -8 + 2.0 ** -30),
                   3.0, -0.0, 1e-40, 3.4e38, -3.39e38, 3.38e38]])
    got = oracle.logits_to_bf16(L)
    ref = torch.from_numpy(L).float().to(torch.bfloat16).view(torch.int16)
    assert np.array_equal(got, ref.numpy().view(np.uint16))
    assert got[0, 0] == 0x3F80 and got[0, 1] == 0xBF80


def test_scatter_bf16_matches_index_copy():
    rng = np.random.default_rng(17)
    idx = np.concatenate([np.sort(rng.choice(500, 100, replace=False)),
                          np.zeros(28, dtype=np.int64)]).astype(np.int32)
    idx[100:] = idx[0]
    Lb = oracle.logits_to_bf16(rng.standard_normal((3, 128)))
    out = oracle.logits_scatter_bf16(Lb, 100, idx, 500)
    ref = torch.full((3, 500), float("-inf"), dtype=torch.bfloat16)
    ref.index_copy_(1, torch.from_numpy(idx[:100]).long(),
                    torch.from_numpy(Lb[:, :100].view(np.int16)).view(torch.bfloat16))
    assert np.array_equal(out, ref.view(torch.int16).numpy().view(np.uint16))
    assert ((out == 0xFF80).sum(axis=1) == 400).all()


# ------------------------------------------- readings of silent float steps

def test_block_scale_reading_is_bmax_over_six_gs():
    """The pages fix the recipe's constants but not the float32 operation
    order of the block scale.  The reading taken is bmax / (6 * gs) in two
    roundings.  For amax = 2.4375 and a block maximum of 2^-13 * 0.914 the
    two plausible orders disagree: bmax/(6*gs) lands on E4M3 code 11,
    (bmax/6)/gs on code 10."""
    w = torch.zeros((64, 32), dtype=torch.float32)
    w[0, 0] = 2.4375
    w[1, 0] = 0.00011157989501953125
    wb = w.to(torch.bfloat16)
    assert wb.float()[1, 0].item() == 0.00011157989501953125
    p, s, gs = oracle.nvfp4_quantize(_bits(wb), np.arange(64, dtype=np.int32))
    assert gs == np.float32(np.float32(2.4375) / np.float32(2688))
    assert s[1, 0] == 11
    assert s[0, 0] == 0x7E


def test_e4m3_tensor_reading_divides_by_the_scale():
    """Page 2's conversion divides by the scale; multiplying by its
    reciprocal differs here: x / scale gives code 26, x * (1/scale) 27."""
    w = torch.zeros((64, 16), dtype=torch.float32)
    w[0, 0] = 0.0062255859375
    w[5, 3] = 1.1399388313293457e-06
    wb = w.to(torch.bfloat16)
    assert wb.float()[5, 3].item() == 1.1399388313293457e-06
    q, scale = oracle.e4m3_tensor_quantize(_bits(wb), np.arange(64, dtype=np.int32))
    assert q[5, 3] == 26 and q[0, 0] == 0x7E


def test_fp8_tokens_reading_divides_by_the_scale():
    """The per-token quant divides by the row's scale, as page 2's head
    conversion does.  With amax 4.75, x = -3.5625 gives x / sx = -336
    exactly, a tie between 320 and 352 that goes to the even code 0xFA;
    x * (1/sx) is -336.00003 and would give 0xFB."""
    h = torch.zeros((1, 16), dtype=torch.float32)
    h[0, 0] = 4.75
    h[0, 1] = -3.5625
    qx, sx = oracle.fp8_tokens_quantize(_bits(h.to(torch.bfloat16)))
    assert qx[0, 1] == 0xFA and qx[0, 0] == 0x7E


def test_markstein_quotient_equals_the_division(tmp_path):
    """The quantizer kernels' per-element quotient (one reciprocal per
    divisor, Markstein's fma correction) is the correctly rounded division
    over every bf16 input in its range, for a seeded sample of divisors: the
    arithmetic fact the kernels rely on, checked on the CPU's IEEE float32
    with a correctly rounded fmaf."""
    import subprocess
    src = os.path.join(os.path.dirname(__file__), "native", "markstein_check.c")
    exe = str(tmp_path / "markstein_check")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", src,
                    "-o", exe, "-lm"], check=True)
    r = subprocess.run([exe, "1500"], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout
    assert "mismatches 0 " in r.stdout, r.stdout
