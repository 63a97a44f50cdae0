"""Python binding of the MI355X reduced-vocabulary NVFP4 draft head.

Argument marshalling only: every function here checks tensor dtypes and
devices, allocates outputs with torch when the caller does not pass them,
and calls the C-ABI of ``libdrafthead.so`` (declared in include/drafthead.h)
on the current HIP stream.  Every step of the computation runs in the HIP
kernels; there is no fallback.  If the library is not built, importing the
functions works but the first call raises.

Method: page 1 ("q38_draft.py", load_draft_model / get_top_tokens /
compute_logits) and page 3 ("...MTP-NVFP4-h98k", "How it was built", the
NVFP4 recipe).
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdrafthead.so")

DH_OK = 0
DH_EINVAL = -1
DH_EWORKSPACE = -2
DH_EHIP = -3


class DraftHeadError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {error_string(status)} (status {status})")


_lib = None
_c_i64 = ctypes.c_int64
_c_ptr = ctypes.c_void_p
_c_size = ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python __graft_entry__.py` "
                "or reduced_vocab_nvfp4_amd._build.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.drafthead_abi_version.restype = ctypes.c_int
        L.drafthead_error_string.restype = ctypes.c_char_p
        L.drafthead_error_string.argtypes = [ctypes.c_int]
        L.draft_head_build_index.restype = _c_i64
        L.draft_head_build_index.argtypes = [_c_ptr, _c_i64, _c_ptr, _c_i64,
                                             _c_ptr]
        L.draft_head_workspace_bytes.restype = _c_size
        L.draft_head_workspace_bytes.argtypes = [_c_i64, _c_i64]
        L.nvfp4_quantize_rows.restype = ctypes.c_int
        L.nvfp4_quantize_rows.argtypes = [_c_ptr, _c_i64, _c_i64, _c_ptr,
                                          _c_i64, _c_ptr, _c_ptr, _c_ptr,
                                          _c_ptr, _c_size, _c_ptr]
        L.nvfp4_quantize_rows_f16.restype = ctypes.c_int
        L.nvfp4_quantize_rows_f16.argtypes = L.nvfp4_quantize_rows.argtypes
        L.draft_head_top_tokens_compat.restype = ctypes.c_int
        L.draft_head_top_tokens_compat.argtypes = [
            _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i64, _c_i64, _c_ptr, _c_i64,
            _c_ptr, _c_ptr, _c_size, _c_ptr]
        L.draft_head_logits_compat.restype = ctypes.c_int
        L.draft_head_logits_compat.argtypes = [
            _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i64, _c_i64, _c_i64, _c_i64,
            _c_ptr, _c_i64, _c_ptr, _c_ptr, _c_size, _c_ptr]
        L.draft_head_top_tokens.restype = ctypes.c_int
        L.draft_head_top_tokens.argtypes = [_c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                            _c_i64, _c_i64, _c_ptr, _c_i64,
                                            _c_ptr, _c_ptr, _c_size, _c_ptr]
        L.draft_head_top_tokens_noalloc.restype = ctypes.c_int
        L.draft_head_top_tokens_noalloc.argtypes = [
            _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i64, _c_i64, _c_ptr, _c_i64,
            _c_ptr, _c_ptr]
        L.drafthead_read_probe.restype = ctypes.c_int
        L.drafthead_read_probe.argtypes = [_c_ptr, _c_size, _c_ptr, _c_size,
                                           _c_ptr, _c_ptr]
        L.draft_head_logits.restype = ctypes.c_int
        L.draft_head_logits.argtypes = [_c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                        _c_i64, _c_i64, _c_i64, _c_i64,
                                        _c_ptr, _c_i64, _c_ptr, _c_ptr,
                                        _c_size, _c_ptr]
        L.nvfp4_linear.restype = ctypes.c_int
        L.nvfp4_linear.argtypes = [_c_ptr, _c_ptr, _c_ptr, _c_i64, _c_i64,
                                   _c_ptr, _c_i64, _c_ptr, _c_ptr]
        L.e4m3_quantize_rows_per_tensor.restype = ctypes.c_int
        L.e4m3_quantize_rows_per_tensor.argtypes = [
            _c_ptr, _c_i64, _c_i64, _c_ptr, _c_i64, _c_ptr, _c_ptr, _c_ptr,
            _c_size, _c_ptr]
        L.draft_head_top_tokens_e4m3.restype = ctypes.c_int
        L.draft_head_top_tokens_e4m3.argtypes = [
            _c_ptr, _c_ptr, _c_ptr, _c_i64, _c_i64, _c_ptr, _c_i64, _c_ptr,
            _c_ptr, _c_size, _c_ptr]
        L.draft_head_logits_e4m3.restype = ctypes.c_int
        L.draft_head_logits_e4m3.argtypes = [
            _c_ptr, _c_ptr, _c_ptr, _c_i64, _c_i64, _c_i64, _c_i64, _c_ptr,
            _c_i64, _c_ptr, _c_ptr, _c_size, _c_ptr]
        L.fp8_quantize_tokens.restype = ctypes.c_int
        L.fp8_quantize_tokens.argtypes = [_c_ptr, _c_i64, _c_i64, _c_ptr,
                                          _c_ptr, _c_ptr]
        L.draft_head_workspace_bytes_w8a8.restype = _c_size
        L.draft_head_workspace_bytes_w8a8.argtypes = [_c_i64, _c_i64, _c_i64]
        L.draft_head_top_tokens_w8a8.restype = ctypes.c_int
        L.draft_head_top_tokens_w8a8.argtypes = [
            _c_ptr, _c_ptr, _c_ptr, _c_i64, _c_i64, _c_ptr, _c_i64, _c_ptr,
            _c_ptr, _c_size, _c_ptr]
        L.draft_head_logits_w8a8.restype = ctypes.c_int
        L.draft_head_logits_w8a8.argtypes = [
            _c_ptr, _c_ptr, _c_ptr, _c_i64, _c_i64, _c_i64, _c_i64, _c_ptr,
            _c_i64, _c_ptr, _c_ptr, _c_size, _c_ptr]
        L.draft_head_top_tokens_bf16.restype = ctypes.c_int
        L.draft_head_top_tokens_bf16.argtypes = [
            _c_ptr, _c_ptr, _c_i64, _c_i64, _c_ptr, _c_i64, _c_ptr, _c_ptr,
            _c_size, _c_ptr]
        L.draft_head_logits_bf16.restype = ctypes.c_int
        L.draft_head_logits_bf16.argtypes = [
            _c_ptr, _c_ptr, _c_i64, _c_i64, _c_i64, _c_i64, _c_ptr, _c_i64,
            _c_ptr, _c_ptr, _c_size, _c_ptr]
        _lib = L
    return _lib


def error_string(status: int) -> str:
    return lib().drafthead_error_string(int(status)).decode()


def _check(fn: str, rc: int) -> None:
    if rc != DH_OK:
        raise DraftHeadError(fn, rc)


def _dev(t: torch.Tensor, name: str, dtype) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(device: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream)


def _alloc_stream(stream):
    """Context for the tensors a call allocates for the caller (outputs, a
    fresh workspace): on the call's stream, so a workspace's zero-fill is
    ordered before the kernels that read it, and the caching allocator does
    not hand its memory to work on another stream while the kernels may
    still use it."""
    return contextlib.nullcontext() if stream is None else \
        torch.cuda.stream(stream)


# --------------------------------------------------------------- A1 index

def draft_head_build_index(keep_mask) -> tuple[torch.Tensor, int]:
    """Row index from a bool keep mask (host): (dh_idx int32 CPU tensor of
    n_rows entries, n_kept)."""
    m = keep_mask.cpu().numpy() if isinstance(keep_mask, torch.Tensor) \
        else np.asarray(keep_mask)
    m = np.ascontiguousarray(m.astype(np.uint8))
    V = m.shape[0]
    cap = V + 64
    out = np.empty(cap, dtype=np.int32)
    n_kept = ctypes.c_int64(0)
    n = lib().draft_head_build_index(m.ctypes.data, V, out.ctypes.data, cap,
                                     ctypes.addressof(n_kept))
    if n < 0:
        raise DraftHeadError("draft_head_build_index", int(n))
    return torch.from_numpy(out[:n].copy()), int(n_kept.value)


def draft_head_workspace_bytes(n_rows: int, batch: int) -> int:
    return int(lib().draft_head_workspace_bytes(int(n_rows), int(batch)))


# Workspace fields a caller may read or write (DH_WS_STATUS_OFFSET and
# DH_WS_SPIN_LIMIT_OFFSET in drafthead.h): two uint16.
WS_STATUS_OFFSET = 4
WS_SPIN_LIMIT_OFFSET = 6


def workspace_gave_up(workspace: torch.Tensor) -> bool:
    """True once a collecting block of a top-token call on this workspace
    gave up waiting (its call wrote -1 ids; every later call on it writes -1
    until the workspace is zero-filled again).  Reads device memory, so it
    waits for the work queued on the current stream."""
    return bool(workspace[WS_STATUS_OFFSET:WS_STATUS_OFFSET + 2]
                .view(torch.int16).item() != 0)


def set_workspace_spin_limit(workspace: torch.Tensor, rounds: int) -> None:
    """Bound a collecting block's empty polling rounds on this workspace
    (0 = give up before the first poll); a zero-filled workspace has the
    library's default bound."""
    if not 0 <= rounds < 0xFFFF:
        raise ValueError("rounds must be in [0, 65534]")
    v = rounds + 1  # the uint16 field, written through a signed view
    workspace[WS_SPIN_LIMIT_OFFSET:WS_SPIN_LIMIT_OFFSET + 2].view(
        torch.int16).fill_(v - 65536 if v >= 32768 else v)


def new_workspace(n_rows: int, batch: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace for heads of n_rows rows up to this batch."""
    n = draft_head_workspace_bytes(n_rows, batch)
    if n == 0:
        raise ValueError("invalid n_rows/batch for a workspace")
    return torch.zeros(n, dtype=torch.uint8, device=device)


# ------------------------------------------------------------ A2 quantize

def nvfp4_quantize_rows(w: torch.Tensor, row_ids: torch.Tensor, *,
                        packed=None, scales=None, global_scale=None,
                        workspace=None, stream=None):
    """Gather W[row_ids] and quantize to NVFP4 on the GPU; w is BF16 or
    FP16.  Returns (packed u8 [n,H/2], scales u8 [n,H/16], global_scale
    f32 [1])."""
    V, H = w.shape
    n = row_ids.shape[0]
    dev = w.device
    with _alloc_stream(stream):
        if packed is None:
            packed = torch.empty((n, H // 2), dtype=torch.uint8, device=dev)
        if scales is None:
            scales = torch.empty((n, H // 16), dtype=torch.uint8, device=dev)
        if global_scale is None:
            global_scale = torch.empty(1, dtype=torch.float32, device=dev)
        if workspace is None:
            workspace = new_workspace(max(n, 1), 1, dev)
    f16 = w.dtype == torch.float16
    fn = lib().nvfp4_quantize_rows_f16 if f16 else lib().nvfp4_quantize_rows
    rc = fn(
        _dev(w, "w", torch.float16 if f16 else torch.bfloat16), V, H,
        _dev(row_ids, "row_ids", torch.int32), n,
        _dev(packed, "packed", torch.uint8), _dev(scales, "scales", torch.uint8),
        _dev(global_scale, "global_scale", torch.float32),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream(dev, stream))
    _check("nvfp4_quantize_rows_f16" if f16 else "nvfp4_quantize_rows", rc)
    return packed, scales, global_scale


# ------------------------------------------------------- A3+A4 top tokens

def draft_head_top_tokens(packed, scales, global_scale, dh_idx, h, *,
                          out_ids=None, workspace=None, stream=None):
    """Greedy draft tokens: int32 [B] target ids."""
    n, H2 = packed.shape
    B, H = h.shape
    dev = h.device
    with _alloc_stream(stream):
        if out_ids is None:
            out_ids = torch.empty(B, dtype=torch.int32, device=dev)
        if workspace is None:
            workspace = new_workspace(n, B, dev)
    rc = lib().draft_head_top_tokens(
        _dev(packed, "packed", torch.uint8), _dev(scales, "scales", torch.uint8),
        _dev(global_scale, "global_scale", torch.float32),
        _dev(dh_idx, "dh_idx", torch.int32), n, H,
        _dev(h, "h", torch.bfloat16), B,
        _dev(out_ids, "out_ids", torch.int32),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream(dev, stream))
    _check("draft_head_top_tokens", rc)
    return out_ids


def draft_head_top_tokens_noalloc(packed, scales, global_scale, dh_idx, h, *,
                                  out_ids=None, stream=None):
    """draft_head_top_tokens on the library's own static scratch (the C call
    allocates nothing; calls that overlap on one GPU race): int32 [B] ids."""
    n, H2 = packed.shape
    B, H = h.shape
    dev = h.device
    if out_ids is None:
        with _alloc_stream(stream):
            out_ids = torch.empty(B, dtype=torch.int32, device=dev)
    rc = lib().draft_head_top_tokens_noalloc(
        _dev(packed, "packed", torch.uint8), _dev(scales, "scales", torch.uint8),
        _dev(global_scale, "global_scale", torch.float32),
        _dev(dh_idx, "dh_idx", torch.int32), n, H,
        _dev(h, "h", torch.bfloat16), B,
        _dev(out_ids, "out_ids", torch.int32), _stream(dev, stream))
    _check("draft_head_top_tokens_noalloc", rc)
    return out_ids


# Measurement aid (drafthead_read_probe): the constant a wave's XOR of the
# words it read must equal for the probe to store it.
READ_PROBE_MAGIC = 0x9E3779B9


def read_probe(a: torch.Tensor, b: torch.Tensor = None, *, sink=None,
               stream=None) -> torch.Tensor:
    """One plain streaming read of a's bytes, then b's (contiguous device
    tensors, 16-byte aligned, sizes multiples of 16 bytes): the device's
    rate for streaming a head's own buffers.  Returns the sink (int32 [1],
    written only by a wave whose XOR equals READ_PROBE_MAGIC)."""
    def ptr(t, name):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        return t.data_ptr(), t.numel() * t.element_size()
    pa, na = ptr(a, "a")
    pb, nb = ptr(b, "b") if b is not None else (None, 0)
    if sink is None:
        with _alloc_stream(stream):
            sink = torch.zeros(1, dtype=torch.int32, device=a.device)
    rc = lib().drafthead_read_probe(pa, na, pb, nb,
                                    _dev(sink, "sink", torch.int32),
                                    _stream(a.device, stream))
    _check("drafthead_read_probe", rc)
    return sink


# ------------------------------------------------------------- A5 logits

def draft_head_logits(packed, scales, global_scale, dh_idx, n_kept: int,
                      vocab: int, h, *, out=None, workspace=None, stream=None):
    """float32 [B, vocab] logits, -inf at ids that were not kept."""
    n, H2 = packed.shape
    B, H = h.shape
    dev = h.device
    with _alloc_stream(stream):
        if out is None:
            out = torch.empty((B, vocab), dtype=torch.float32, device=dev)
        if workspace is None:
            workspace = new_workspace(n, B, dev)
    rc = lib().draft_head_logits(
        _dev(packed, "packed", torch.uint8), _dev(scales, "scales", torch.uint8),
        _dev(global_scale, "global_scale", torch.float32),
        _dev(dh_idx, "dh_idx", torch.int32), n, int(n_kept), H, int(vocab),
        _dev(h, "h", torch.bfloat16), B, _dev(out, "out", torch.float32),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream(dev, stream))
    _check("draft_head_logits", rc)
    return out


# --------------------------------- the pages' own numerics (BF16 logits)

def draft_head_top_tokens_compat(packed, scales, global_scale, dh_idx, h, *,
                                 out_ids=None, workspace=None, stream=None):
    """Greedy draft tokens over the logits rounded to BF16 (global scale
    applied, lowest row on ties), as the pages' BF16 linear feeds the
    argmax: int32 [B] target ids."""
    n = packed.shape[0]
    B, H = h.shape
    dev = h.device
    with _alloc_stream(stream):
        if out_ids is None:
            out_ids = torch.empty(B, dtype=torch.int32, device=dev)
        if workspace is None:
            workspace = new_workspace(n, B, dev)
    rc = lib().draft_head_top_tokens_compat(
        _dev(packed, "packed", torch.uint8), _dev(scales, "scales", torch.uint8),
        _dev(global_scale, "global_scale", torch.float32),
        _dev(dh_idx, "dh_idx", torch.int32), n, H,
        _dev(h, "h", torch.bfloat16), B, _dev(out_ids, "out_ids", torch.int32),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream(dev, stream))
    _check("draft_head_top_tokens_compat", rc)
    return out_ids


def draft_head_logits_compat(packed, scales, global_scale, dh_idx,
                             n_kept: int, vocab: int, h, *, out=None,
                             workspace=None, stream=None):
    """BF16 [B, vocab] logits (global scale applied, rounded to nearest
    even), -inf at ids that were not kept."""
    n = packed.shape[0]
    B, H = h.shape
    dev = h.device
    with _alloc_stream(stream):
        if out is None:
            out = torch.empty((B, vocab), dtype=torch.bfloat16, device=dev)
        if workspace is None:
            workspace = new_workspace(n, B, dev)
    rc = lib().draft_head_logits_compat(
        _dev(packed, "packed", torch.uint8), _dev(scales, "scales", torch.uint8),
        _dev(global_scale, "global_scale", torch.float32),
        _dev(dh_idx, "dh_idx", torch.int32), n, int(n_kept), H, int(vocab),
        _dev(h, "h", torch.bfloat16), B, _dev(out, "out", torch.bfloat16),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream(dev, stream))
    _check("draft_head_logits_compat", rc)
    return out


# ---------------------------------------------- NVFP4 W4A16 linear (N1)

def nvfp4_linear(packed, scales, global_scale, h, *, out=None, stream=None):
    """float32 [B, n_rows] = global_scale * (NVFP4 weight) @ h^T, for a
    weight quantized by nvfp4_quantize_rows (identity row_ids)."""
    n, H2 = packed.shape
    B, H = h.shape
    dev = h.device
    with _alloc_stream(stream):
        if out is None:
            out = torch.empty((B, n), dtype=torch.float32, device=dev)
    rc = lib().nvfp4_linear(
        _dev(packed, "packed", torch.uint8), _dev(scales, "scales", torch.uint8),
        _dev(global_scale, "global_scale", torch.float32), n, H,
        _dev(h, "h", torch.bfloat16), B, _dev(out, "out", torch.float32),
        _stream(dev, stream))
    _check("nvfp4_linear", rc)
    return out


# ------------------------------------------- per-tensor E4M3 head (FP8)

def e4m3_quantize_rows_per_tensor(w: torch.Tensor, row_ids: torch.Tensor, *,
                                  q=None, scale=None, workspace=None,
                                  stream=None):
    """Gather W[row_ids] and quantize to E4M3 with one tensor scale.
    Returns (q u8 [n,H], scale f32 [1])."""
    V, H = w.shape
    n = row_ids.shape[0]
    dev = w.device
    with _alloc_stream(stream):
        if q is None:
            q = torch.empty((n, H), dtype=torch.uint8, device=dev)
        if scale is None:
            scale = torch.empty(1, dtype=torch.float32, device=dev)
        if workspace is None:
            workspace = new_workspace(max(n, 1), 1, dev)
    rc = lib().e4m3_quantize_rows_per_tensor(
        _dev(w, "w", torch.bfloat16), V, H,
        _dev(row_ids, "row_ids", torch.int32), n, _dev(q, "q", torch.uint8),
        _dev(scale, "scale", torch.float32),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream(dev, stream))
    _check("e4m3_quantize_rows_per_tensor", rc)
    return q, scale


def draft_head_top_tokens_e4m3(q, scale, dh_idx, h, *, out_ids=None,
                               workspace=None, stream=None):
    """Greedy draft tokens of an E4M3 head: int32 [B] target ids."""
    n, H = q.shape
    B = h.shape[0]
    dev = h.device
    with _alloc_stream(stream):
        if out_ids is None:
            out_ids = torch.empty(B, dtype=torch.int32, device=dev)
        if workspace is None:
            workspace = new_workspace(n, B, dev)
    rc = lib().draft_head_top_tokens_e4m3(
        _dev(q, "q", torch.uint8), _dev(scale, "scale", torch.float32),
        _dev(dh_idx, "dh_idx", torch.int32), n, H,
        _dev(h, "h", torch.bfloat16), B, _dev(out_ids, "out_ids", torch.int32),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream(dev, stream))
    _check("draft_head_top_tokens_e4m3", rc)
    return out_ids


def draft_head_logits_e4m3(q, scale, dh_idx, n_kept: int, vocab: int, h, *,
                           out=None, workspace=None, stream=None):
    """float32 [B, vocab] logits of an E4M3 head, -inf at ids not kept."""
    n, H = q.shape
    B = h.shape[0]
    dev = h.device
    with _alloc_stream(stream):
        if out is None:
            out = torch.empty((B, vocab), dtype=torch.float32, device=dev)
        if workspace is None:
            workspace = new_workspace(n, B, dev)
    rc = lib().draft_head_logits_e4m3(
        _dev(q, "q", torch.uint8), _dev(scale, "scale", torch.float32),
        _dev(dh_idx, "dh_idx", torch.int32), n, int(n_kept), H, int(vocab),
        _dev(h, "h", torch.bfloat16), B, _dev(out, "out", torch.float32),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream(dev, stream))
    _check("draft_head_logits_e4m3", rc)
    return out


# ------------------------------------------------- W8A8 (FP8) head, page 2

def fp8_quantize_tokens(h, *, qx=None, sx=None, stream=None):
    """Per-token dynamic E4M3 quantization of BF16 h [B, H]:
    (qx uint8 [B, H] e4m3fn codes, sx float32 [B] scales)."""
    B, H = h.shape
    dev = h.device
    with _alloc_stream(stream):
        if qx is None:
            qx = torch.empty((B, H), dtype=torch.uint8, device=dev)
        if sx is None:
            sx = torch.empty(B, dtype=torch.float32, device=dev)
    rc = lib().fp8_quantize_tokens(
        _dev(h, "h", torch.bfloat16), B, H, _dev(qx, "qx", torch.uint8),
        _dev(sx, "sx", torch.float32), _stream(dev, stream))
    _check("fp8_quantize_tokens", rc)
    return qx, sx


def draft_head_workspace_bytes_w8a8(n_rows: int, batch: int,
                                    hidden: int) -> int:
    return int(lib().draft_head_workspace_bytes_w8a8(n_rows, batch, hidden))


def new_workspace_w8a8(n_rows: int, batch: int, hidden: int,
                       device="cuda") -> torch.Tensor:
    """A zero-filled workspace for the W8A8 head calls."""
    n = draft_head_workspace_bytes_w8a8(n_rows, batch, hidden)
    if n == 0:
        raise ValueError("invalid n_rows/batch/hidden for a workspace")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def draft_head_top_tokens_w8a8(q, scale, dh_idx, h, *, out_ids=None,
                               workspace=None, stream=None):
    """Greedy draft tokens of an E4M3 head applied W8A8 (the tokens are
    quantized per token inside the call): int32 [B] target ids."""
    n, H = q.shape
    B = h.shape[0]
    dev = h.device
    with _alloc_stream(stream):
        if out_ids is None:
            out_ids = torch.empty(B, dtype=torch.int32, device=dev)
        if workspace is None:
            workspace = new_workspace_w8a8(n, B, H, dev)
    rc = lib().draft_head_top_tokens_w8a8(
        _dev(q, "q", torch.uint8), _dev(scale, "scale", torch.float32),
        _dev(dh_idx, "dh_idx", torch.int32), n, H,
        _dev(h, "h", torch.bfloat16), B, _dev(out_ids, "out_ids", torch.int32),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream(dev, stream))
    _check("draft_head_top_tokens_w8a8", rc)
    return out_ids


def draft_head_logits_w8a8(q, scale, dh_idx, n_kept: int, vocab: int, h, *,
                           out=None, workspace=None, stream=None):
    """float32 [B, vocab] W8A8 logits of an E4M3 head, -inf at ids not
    kept."""
    n, H = q.shape
    B = h.shape[0]
    dev = h.device
    with _alloc_stream(stream):
        if out is None:
            out = torch.empty((B, vocab), dtype=torch.float32, device=dev)
        if workspace is None:
            workspace = new_workspace_w8a8(n, B, H, dev)
    rc = lib().draft_head_logits_w8a8(
        _dev(q, "q", torch.uint8), _dev(scale, "scale", torch.float32),
        _dev(dh_idx, "dh_idx", torch.int32), n, int(n_kept), H, int(vocab),
        _dev(h, "h", torch.bfloat16), B, _dev(out, "out", torch.float32),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream(dev, stream))
    _check("draft_head_logits_w8a8", rc)
    return out


# ------------------------------------------------------- BF16 (stock) head

def draft_head_top_tokens_bf16(w, dh_idx, h, *, out_ids=None, workspace=None,
                               stream=None):
    """Greedy tokens of a BF16 head [n_rows, H] (row j scores dh_idx[j])."""
    n, H = w.shape
    B = h.shape[0]
    dev = h.device
    with _alloc_stream(stream):
        if out_ids is None:
            out_ids = torch.empty(B, dtype=torch.int32, device=dev)
        if workspace is None:
            workspace = new_workspace(n, B, dev)
    rc = lib().draft_head_top_tokens_bf16(
        _dev(w, "w", torch.bfloat16), _dev(dh_idx, "dh_idx", torch.int32), n,
        H, _dev(h, "h", torch.bfloat16), B,
        _dev(out_ids, "out_ids", torch.int32),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream(dev, stream))
    _check("draft_head_top_tokens_bf16", rc)
    return out_ids


def draft_head_logits_bf16(w, dh_idx, n_kept: int, vocab: int, h, *,
                           out=None, workspace=None, stream=None):
    """float32 [B, vocab] logits of a BF16 head, -inf at ids not kept."""
    n, H = w.shape
    B = h.shape[0]
    dev = h.device
    with _alloc_stream(stream):
        if out is None:
            out = torch.empty((B, vocab), dtype=torch.float32, device=dev)
        if workspace is None:
            workspace = new_workspace(n, B, dev)
    rc = lib().draft_head_logits_bf16(
        _dev(w, "w", torch.bfloat16), _dev(dh_idx, "dh_idx", torch.int32), n,
        int(n_kept), H, int(vocab), _dev(h, "h", torch.bfloat16), B,
        _dev(out, "out", torch.float32),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream(dev, stream))
    _check("draft_head_logits_bf16", rc)
    return out


__all__ = [
    "DraftHeadError", "lib", "error_string", "draft_head_build_index",
    "draft_head_workspace_bytes", "new_workspace", "workspace_gave_up",
    "set_workspace_spin_limit", "nvfp4_quantize_rows",
    "draft_head_top_tokens", "draft_head_logits",
    "draft_head_top_tokens_compat", "draft_head_logits_compat",
    "nvfp4_linear",
    "e4m3_quantize_rows_per_tensor", "draft_head_top_tokens_e4m3",
    "draft_head_logits_e4m3", "fp8_quantize_tokens",
    "draft_head_workspace_bytes_w8a8", "new_workspace_w8a8",
    "draft_head_top_tokens_w8a8", "draft_head_logits_w8a8",
    "draft_head_top_tokens_bf16", "draft_head_logits_bf16",
]
