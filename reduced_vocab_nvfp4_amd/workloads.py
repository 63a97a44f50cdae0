"""Seeded synthetic inputs for the reduced-vocabulary draft head.

This module only draws data: head weights, hidden states and keep masks.
It holds none of the method's arithmetic (no index building, no encoding,
no contraction), so both the HIP path and the CPU oracle can be fed from it
without sharing a single step of the computation.

The shapes follow the pages:
  * "Qwen3.8-Flash-Next ... q38_draft.py" (page 1, module docstring): a
    248 320 x 2560 BF16 head, batch-1 drafting, a 64k draft vocabulary with
    special tokens always kept.
  * "Qwen3.8-27B-NVFP4-DGX-SPARK" (page 4, repository layout): a bool mask
    over 248 320 ids with 64 026 kept, giving a 64 064-row head once padded.
  * "...MTP-NVFP4-h98k" (page 3, "How it was built"): a 98 304-row head.
The trained weights and the corpus-derived masks are not available, so:
  W ~ N(0, 0.02) in float32, rounded to BF16 (round-to-nearest-even);
  h ~ N(0, 1) in float64, rounded to BF16;
  the keep mask forces the last ids (stand-ins for special tokens) and then
  walks a seeded random permutation (a stand-in for the frequency ranking:
  only the rank order matters for which ids are kept).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

SEED_W = 0
SEED_KEEP = 1
SEED_H0 = 2  # hidden-state seed for step s is SEED_H0 + s


@dataclass(frozen=True)
class Workload:
    name: str
    vocab: int
    hidden: int
    batch: int
    n_keep: int            # ids kept by the mask (== vocab for the identity head)
    forced_tail: int       # the last `forced_tail` ids are always kept
    formats: tuple = ("nvfp4",)
    logits: bool = False   # the step also scatters fp32 logits to the full vocab
    identity: bool = False  # stock head: every id kept, no mask
    tiny_choice: bool = False  # keep = forced tail + a random choice (small case)
    linear: bool = False   # a plain NVFP4 linear: vocab = output rows, dense out
    note: str = field(default="", compare=False)


WORKLOADS = {
    "tiny": Workload(
        "tiny", vocab=4096, hidden=256, batch=1, n_keep=1024, forced_tail=32,
        logits=True, tiny_choice=True,
        note="V=4096 H=256, last 32 ids + 992 random ids -> 1024 rows, B=1, "
             "top token and full-vocab logits"),
    "flash_next_64k": Workload(
        "flash_next_64k", vocab=248320, hidden=2560, batch=1, n_keep=64026,
        forced_tail=256,
        note="V=248320 H=2560, 64026 kept -> 64064 rows (38 pads), NVFP4 "
             "W4A16, B=1, top token"),
    "stock_bf16": Workload(
        "stock_bf16", vocab=248320, hidden=2560, batch=1, n_keep=248320,
        forced_tail=0, formats=("bf16",), identity=True,
        note="full 248320 x 2560 BF16 head, B=1, argmax over every row"),
    "dense27b_64k_b8": Workload(
        "dense27b_64k_b8", vocab=248320, hidden=5120, batch=8, n_keep=64026,
        forced_tail=256, logits=True,
        note="V=248320 H=5120, 64064 rows, NVFP4, B=8, top tokens and "
             "fp32 logits scattered to the full vocab"),
    # The drafter's other NVFP4 linears (page 1, "q38_draft.py", install:
    # the MTP block's 2-D weights with N % 64 == 0 and K % 16 == 0): shapes
    # at the draft head's hidden size, output rows x input features.
    "linear_2560x5120_b1": Workload(
        "linear_2560x5120_b1", vocab=2560, hidden=5120, batch=1, n_keep=2560,
        forced_tail=0, identity=True, linear=True,
        note="NVFP4 W4A16 linear, 2560 outputs from 5120 inputs (two "
             "2560-wide vectors concatenated), B=1, dense fp32 out"),
    "linear_10240x2560_b1": Workload(
        "linear_10240x2560_b1", vocab=10240, hidden=2560, batch=1,
        n_keep=10240, forced_tail=0, identity=True, linear=True,
        note="NVFP4 W4A16 linear, 10240 outputs from 2560 inputs, B=1"),
    "linear_5120x2560_b16": Workload(
        "linear_5120x2560_b16", vocab=5120, hidden=2560, batch=16,
        n_keep=5120, forced_tail=0, identity=True, linear=True,
        note="NVFP4 W4A16 linear, 5120 outputs from 2560 inputs, B=16 (MFMA)"),
    "h98k_b16": Workload(
        "h98k_b16", vocab=248320, hidden=2560, batch=16, n_keep=98304,
        forced_tail=256, formats=("nvfp4", "e4m3", "w8a8"),
        note="V=248320 H=2560, 98304 kept, NVFP4 and E4M3 per-tensor "
             "(W8A16, or W8A8 with per-token E4M3 activations), B=16"),
}


def keep_mask(wl: Workload, seed: int = SEED_KEEP) -> np.ndarray:
    """bool[vocab] keep mask drawn from `seed` (see the module docstring)."""
    V = wl.vocab
    keep = np.zeros(V, dtype=bool)
    if wl.identity:
        keep[:] = True
        return keep
    rng = np.random.default_rng(seed)
    if wl.forced_tail:
        keep[V - wl.forced_tail:] = True
    if wl.tiny_choice:
        extra = rng.choice(V - wl.forced_tail, wl.n_keep - wl.forced_tail,
                           replace=False)
        keep[extra] = True
    else:
        perm = rng.permutation(V)
        need = wl.n_keep - int(keep.sum())
        fresh = perm[~keep[perm]]
        keep[fresh[:need]] = True
    assert int(keep.sum()) == wl.n_keep
    return keep


def head_weight(vocab: int, hidden: int, seed: int = SEED_W,
                chunk_rows: int = 16384) -> torch.Tensor:
    """BF16 [vocab, hidden] CPU tensor, N(0, 0.02) drawn in row chunks."""
    rng = np.random.default_rng(seed)
    out = torch.empty((vocab, hidden), dtype=torch.bfloat16)
    for r0 in range(0, vocab, chunk_rows):
        r1 = min(vocab, r0 + chunk_rows)
        x = rng.standard_normal((r1 - r0, hidden), dtype=np.float32)
        x *= np.float32(0.02)
        out[r0:r1] = torch.from_numpy(x).to(torch.bfloat16)
    return out


def hidden_states(batch: int, hidden: int, step: int = 0) -> torch.Tensor:
    """BF16 [batch, hidden] CPU tensor, N(0, 1), seed SEED_H0 + step."""
    rng = np.random.default_rng(SEED_H0 + step)
    x = rng.standard_normal((batch, hidden))
    return torch.from_numpy(x).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """uint16 view of a contiguous BF16 CPU tensor (no copy of values)."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)
