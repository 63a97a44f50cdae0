"""Test-side helpers: golden-case loading, an independent dequantizer for the
library pins, and the argmax acceptance rule used by the parity tests.

Nothing here is used by the library; nothing here is used by the oracle.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# Logit tolerance for floating-point parity (allclose semantics).
RTOL = 1e-3
ATOL = 1e-4


def e2m1_from_bits(nib: int) -> Fraction:
    """e2m1 value straight from the bit fields: sign bit 3, exponent bits 2-1
    (bias 1), mantissa bit 0; exponent 0 is subnormal (m * 1/2)."""
    s = (nib >> 3) & 1
    e = (nib >> 1) & 3
    m = nib & 1
    mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
    return -mag if s else mag


# float table; code 0x8 is -0.0 (a Fraction has no signed zero)
E2M1_TABLE = np.array([np.copysign(float(abs(e2m1_from_bits(n))),
                                   -1.0 if n & 8 else 1.0) for n in range(16)])


def dequant_nvfp4_torch(packed: np.ndarray, scales: np.ndarray, gs) -> torch.Tensor:
    """float64 [n, H] weights from NVFP4 codes, decoded without the oracle:
    scales through torch's float8_e4m3fn dtype, nibbles through the bit-field
    table above."""
    n, H2 = packed.shape
    lo = packed & 15
    hi = packed >> 4
    nib = np.empty((n, H2 * 2), dtype=np.uint8)
    nib[:, 0::2] = lo
    nib[:, 1::2] = hi
    vals = torch.from_numpy(E2M1_TABLE[nib])
    sc = torch.from_numpy(np.ascontiguousarray(scales)).view(
        torch.float8_e4m3fn).to(torch.float64)
    sc = sc.repeat_interleave(16, dim=1)
    return vals * sc * float(gs)


def load_gemv_case(case: dict, hidden: int, rows: int):
    """(packed, scales, gs, h_bits, expected float64[rows], argmax_row)."""
    packed = np.zeros((rows, hidden // 2), dtype=np.uint8)
    for r, b in case.get("bytes_all", {}).items():
        packed[int(r), :] = int(b, 16)
    for r, cols in case.get("bytes", {}).items():
        for c, b in cols.items():
            packed[int(r), int(c)] = int(b, 16)
    scales = np.full((rows, hidden // 16), int(case["scales_default"], 16),
                     dtype=np.uint8)
    for r, lst in case.get("scales", {}).items():
        scales[int(r), :] = [int(x, 16) for x in lst]
    h = np.full(hidden, case["h_default"], dtype=np.float32)
    for k, v in case.get("h", {}).items():
        h[int(k)] = v
    h_bits = torch.from_numpy(h).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)[None, :].copy()
    expected = np.full(rows, case["expected_default"], dtype=np.float64)
    for r, v in case["expected"].items():
        expected[int(r)] = v
    return packed, scales, np.float32(case["gs"]), h_bits, expected, case["argmax_row"]


def golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def close(got, want, rtol=RTOL, atol=ATOL):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    return np.abs(got - want) <= atol + rtol * np.abs(want)


def check_top_tokens(got_ids, L: np.ndarray, idx: np.ndarray, n_kept: int,
                     want_ids, rtol=RTOL, atol=ATOL):
    """Argmax acceptance rule.  A returned id passes when it equals the
    oracle's id, or when it is a kept id whose oracle logit is within the
    logit tolerance of the oracle's maximum (a top-2 gap below tolerance).
    Returns the number of such near-tie exceptions; raises on a failure."""
    L = np.atleast_2d(L)
    exceptions = 0
    for b, (g, w) in enumerate(zip(np.asarray(got_ids), np.asarray(want_ids))):
        if int(g) == int(w):
            continue
        rows = np.flatnonzero(idx[:n_kept] == int(g))
        assert rows.size == 1, f"batch {b}: id {g} is not a kept id"
        lmax = L[b].max()
        lg = L[b, rows[0]]
        assert abs(lg - lmax) <= atol + rtol * abs(lmax), (
            f"batch {b}: got id {g} (logit {lg}) but oracle id {w} "
            f"(logit {lmax}); gap {lmax - lg}")
        exceptions += 1
    return exceptions


_WEIGHTS = {}


def head_weight(vocab: int, hidden: int):
    """The seeded BF16 head of this shape, drawn once per test session."""
    if (vocab, hidden) not in _WEIGHTS:
        from reduced_vocab_nvfp4_amd import workloads
        _WEIGHTS[(vocab, hidden)] = workloads.head_weight(vocab, hidden)
    return _WEIGHTS[(vocab, hidden)]
