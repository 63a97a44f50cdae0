"""CPU oracle for the reduced-vocabulary NVFP4 draft head.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the library and its Python binding
never do.  The arithmetic lives in ``oracle.c`` (plain C, built with gcc,
no fast-math, no FMA contraction); this module only builds it and marshals
numpy arrays through ctypes.

Function-by-function citations are in ``oracle.c``.  Every function here has
a pin in ``tests/test_oracle_pins.py`` against something other than the
oracle itself (library casts, closed forms, brute force, constructions).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
             "-fno-fast-math", "-ffp-contract=off", "-fexcess-precision=standard",
             "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc; returns the path."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None

c_i64 = ctypes.c_int64
c_ptr = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or (
                os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build()
        L = ctypes.CDLL(_LIB)
        L.oracle_e4m3_value.restype = ctypes.c_double
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_code.restype = ctypes.c_uint8
        L.oracle_e4m3_code.argtypes = [ctypes.c_float]
        L.oracle_e2m1_value.restype = ctypes.c_double
        L.oracle_e2m1_value.argtypes = [ctypes.c_uint8]
        L.oracle_e2m1_code.restype = ctypes.c_uint8
        L.oracle_e2m1_code.argtypes = [ctypes.c_float]
        L.oracle_build_index.restype = c_i64
        L.oracle_build_index.argtypes = [c_ptr, c_i64, c_ptr, c_i64, c_ptr]
        L.oracle_nvfp4_quantize.argtypes = [c_ptr, c_i64, c_i64, c_ptr, c_i64,
                                            c_ptr, c_ptr, c_ptr]
        L.oracle_nvfp4_logits.argtypes = [c_ptr, c_ptr, ctypes.c_float, c_i64,
                                          c_i64, c_ptr, c_i64, c_ptr]
        L.oracle_argmax_remap.argtypes = [c_ptr, c_i64, c_i64, c_ptr, c_ptr,
                                          c_ptr]
        L.oracle_logits_scatter.argtypes = [c_ptr, c_i64, c_i64, c_i64, c_ptr,
                                            c_i64, c_ptr]
        L.oracle_bf16_logits.argtypes = [c_ptr, c_i64, c_i64, c_ptr, c_i64,
                                         c_ptr, c_i64, c_ptr]
        L.oracle_e4m3_tensor_quantize.argtypes = [c_ptr, c_i64, c_i64, c_ptr,
                                                  c_i64, c_ptr, c_ptr]
        L.oracle_e4m3_tensor_logits.argtypes = [c_ptr, ctypes.c_float, c_i64,
                                                c_i64, c_ptr, c_i64, c_ptr]
        L.oracle_fp8_tokens_quantize.argtypes = [c_ptr, c_i64, c_i64, c_ptr,
                                                 c_ptr]
        L.oracle_w8a8_logits.argtypes = [c_ptr, ctypes.c_float, c_i64, c_i64,
                                         c_ptr, c_ptr, c_i64, c_ptr]
        L.oracle_f16_value.restype = ctypes.c_float
        L.oracle_f16_value.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_code.restype = ctypes.c_uint16
        L.oracle_bf16_code.argtypes = [ctypes.c_float]
        L.oracle_nvfp4_quantize_f16.argtypes = [c_ptr, c_i64, c_i64, c_ptr,
                                                c_i64, c_ptr, c_ptr, c_ptr]
        L.oracle_logits_to_bf16.argtypes = [c_ptr, c_i64, c_ptr]
        L.oracle_logits_scatter_bf16.argtypes = [c_ptr, c_i64, c_i64, c_i64,
                                                 c_ptr, c_i64, c_ptr]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments (rc={rc})")


# ----------------------------------------------------------------- scalars

def e4m3_value(code: int) -> float:
    return lib().oracle_e4m3_value(int(code) & 0xFF)


def e4m3_code(s: float) -> int:
    """E4M3 code of a non-negative float32 (RNE, saturating at 448)."""
    return lib().oracle_e4m3_code(float(np.float32(s)))


def e2m1_value(nib: int) -> float:
    return lib().oracle_e2m1_value(int(nib) & 0xF)


def e2m1_code(q: float) -> int:
    return lib().oracle_e2m1_code(float(np.float32(q)))


# ------------------------------------------------------------------- steps

def build_index(keep: np.ndarray):
    """C1: (idx int32[n_rows], n_kept) from a bool keep mask."""
    keep = np.ascontiguousarray(keep, dtype=np.uint8)
    V = keep.shape[0]
    cap = V + 64
    idx = np.empty(cap, dtype=np.int32)
    n_kept = c_i64(0)
    n = lib().oracle_build_index(_p(keep), V, _p(idx), cap,
                                 ctypes.addressof(n_kept))
    if n < 0:
        raise ValueError("oracle build_index: empty keep mask")
    return idx[:n].copy(), int(n_kept.value)


def nvfp4_quantize(w_bits: np.ndarray, idx: np.ndarray):
    """C2-C4: (packed u8[n,H/2], scales u8[n,H/16], gs float32)."""
    w_bits = np.ascontiguousarray(w_bits, dtype=np.uint16)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    V, H = w_bits.shape
    n = idx.shape[0]
    packed = np.zeros((n, H // 2), dtype=np.uint8)
    scales = np.zeros((n, H // 16), dtype=np.uint8)
    gs = np.zeros(1, dtype=np.float32)
    _check(lib().oracle_nvfp4_quantize(_p(w_bits), V, H, _p(idx), n,
                                       _p(packed), _p(scales), _p(gs)),
           "nvfp4_quantize")
    return packed, scales, np.float32(gs[0])


def nvfp4_logits(packed: np.ndarray, scales: np.ndarray, gs,
                 h_bits: np.ndarray) -> np.ndarray:
    """C5: float64 [B, n_rows] logits."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    h_bits = np.ascontiguousarray(np.atleast_2d(h_bits), dtype=np.uint16)
    n, H2 = packed.shape
    B, H = h_bits.shape
    assert H2 * 2 == H and scales.shape == (n, H // 16)
    L = np.empty((B, n), dtype=np.float64)
    _check(lib().oracle_nvfp4_logits(_p(packed), _p(scales), float(gs), n, H,
                                     _p(h_bits), B, _p(L)), "nvfp4_logits")
    return L


def argmax_remap(L: np.ndarray, idx: np.ndarray):
    """C6: (rows int64[B], ids int32[B])."""
    L = np.ascontiguousarray(np.atleast_2d(L), dtype=np.float64)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    B, n = L.shape
    rows = np.empty(B, dtype=np.int64)
    ids = np.empty(B, dtype=np.int32)
    _check(lib().oracle_argmax_remap(_p(L), B, n, _p(idx), _p(rows), _p(ids)),
           "argmax_remap")
    return rows, ids


def logits_scatter(L: np.ndarray, n_kept: int, idx: np.ndarray,
                   vocab: int) -> np.ndarray:
    """C7: float32 [B, vocab] with -inf for ids not kept."""
    L = np.ascontiguousarray(np.atleast_2d(L), dtype=np.float64)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    B, n = L.shape
    out = np.empty((B, vocab), dtype=np.float32)
    _check(lib().oracle_logits_scatter(_p(L), B, n, n_kept, _p(idx), vocab,
                                       _p(out)), "logits_scatter")
    return out


def bf16_logits(w_bits: np.ndarray, rows: np.ndarray,
                h_bits: np.ndarray) -> np.ndarray:
    """C8: float64 [B, len(rows)] logits of a BF16 head."""
    w_bits = np.ascontiguousarray(w_bits, dtype=np.uint16)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    h_bits = np.ascontiguousarray(np.atleast_2d(h_bits), dtype=np.uint16)
    V, H = w_bits.shape
    B = h_bits.shape[0]
    L = np.empty((B, rows.shape[0]), dtype=np.float64)
    _check(lib().oracle_bf16_logits(_p(w_bits), V, H, _p(rows), rows.shape[0],
                                    _p(h_bits), B, _p(L)), "bf16_logits")
    return L


def e4m3_tensor_quantize(w_bits: np.ndarray, idx: np.ndarray):
    """C9: (q u8[n,H], scale float32)."""
    w_bits = np.ascontiguousarray(w_bits, dtype=np.uint16)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    V, H = w_bits.shape
    n = idx.shape[0]
    q = np.empty((n, H), dtype=np.uint8)
    scale = np.zeros(1, dtype=np.float32)
    _check(lib().oracle_e4m3_tensor_quantize(_p(w_bits), V, H, _p(idx), n,
                                             _p(q), _p(scale)),
           "e4m3_tensor_quantize")
    return q, np.float32(scale[0])


def e4m3_tensor_logits(q: np.ndarray, scale, h_bits: np.ndarray) -> np.ndarray:
    """C9: float64 [B, n] logits of an E4M3 per-tensor head."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    h_bits = np.ascontiguousarray(np.atleast_2d(h_bits), dtype=np.uint16)
    n, H = q.shape
    B = h_bits.shape[0]
    L = np.empty((B, n), dtype=np.float64)
    _check(lib().oracle_e4m3_tensor_logits(_p(q), float(scale), n, H,
                                           _p(h_bits), B, _p(L)),
           "e4m3_tensor_logits")
    return L


def fp8_tokens_quantize(h_bits: np.ndarray):
    """C10: (qx u8[B,H], sx float32[B]), one E4M3 scale per row of h."""
    h_bits = np.ascontiguousarray(np.atleast_2d(h_bits), dtype=np.uint16)
    B, H = h_bits.shape
    qx = np.empty((B, H), dtype=np.uint8)
    sx = np.empty(B, dtype=np.float32)
    _check(lib().oracle_fp8_tokens_quantize(_p(h_bits), B, H, _p(qx), _p(sx)),
           "fp8_tokens_quantize")
    return qx, sx


def w8a8_logits(q: np.ndarray, sw, qx: np.ndarray,
                sx: np.ndarray) -> np.ndarray:
    """C11: float64 [B, n] logits of an E4M3 head against E4M3 tokens."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    qx = np.ascontiguousarray(np.atleast_2d(qx), dtype=np.uint8)
    sx = np.ascontiguousarray(sx, dtype=np.float32)
    n, H = q.shape
    B = qx.shape[0]
    if qx.shape[1] != H or sx.shape != (B,):
        raise ValueError("w8a8_logits: shapes do not agree")
    L = np.empty((B, n), dtype=np.float64)
    _check(lib().oracle_w8a8_logits(_p(q), float(sw), n, H, _p(qx), _p(sx),
                                    B, _p(L)), "w8a8_logits")
    return L


def f16_value(bits: int) -> float:
    return float(lib().oracle_f16_value(int(bits)))


def bf16_code(x: float) -> int:
    """C12: BF16 bits of a float32, round to nearest, ties to even."""
    return int(lib().oracle_bf16_code(float(x)))


def nvfp4_quantize_f16(w_bits: np.ndarray, idx: np.ndarray):
    """C12: NVFP4 quantization of an FP16 head (binary16 bits)."""
    w_bits = np.ascontiguousarray(w_bits, dtype=np.uint16)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    V, H = w_bits.shape
    n = idx.shape[0]
    packed = np.zeros((n, H // 2), dtype=np.uint8)
    scales = np.zeros((n, H // 16), dtype=np.uint8)
    gs = np.zeros(1, dtype=np.float32)
    _check(lib().oracle_nvfp4_quantize_f16(_p(w_bits), V, H, _p(idx), n,
                                           _p(packed), _p(scales), _p(gs)),
           "nvfp4_quantize_f16")
    return packed, scales, np.float32(gs[0])


def logits_to_bf16(L: np.ndarray) -> np.ndarray:
    """C12: BF16 bits (uint16) of float64 logits rounded to float32, then
    to BF16."""
    L = np.ascontiguousarray(L, dtype=np.float64)
    out = np.empty(L.shape, dtype=np.uint16)
    _check(lib().oracle_logits_to_bf16(_p(L), L.size, _p(out)),
           "logits_to_bf16")
    return out


def bf16_bits_value(bits: np.ndarray) -> np.ndarray:
    """float64 values of BF16 bit patterns (the upper half of a float32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def logits_scatter_bf16(Lb: np.ndarray, n_kept: int, idx: np.ndarray,
                        vocab: int) -> np.ndarray:
    """C12: BF16 bits [B, vocab], 0xFF80 (-inf) at ids not kept."""
    Lb = np.ascontiguousarray(np.atleast_2d(Lb), dtype=np.uint16)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    B, n = Lb.shape
    out = np.empty((B, vocab), dtype=np.uint16)
    _check(lib().oracle_logits_scatter_bf16(_p(Lb), B, n, int(n_kept),
                                            _p(idx), int(vocab), _p(out)),
           "logits_scatter_bf16")
    return out


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))
