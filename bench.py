#!/usr/bin/env python3
"""Draft-head step benchmark on one MI355X.

One step = one draft-head call, the hot path of the method (page 1,
"q38_draft.py", get_top_tokens / compute_logits; page 4,
"Qwen3.8-27B-NVFP4-DGX-SPARK", why native MTP plateaus: the head GEMV
dominates a draft step): a GEMV of BF16 hidden states against the kept head
rows fused with the argmax and the id remap (or with the fp32 logits
scatter).  The row index and the quantization happen once, at load, outside
the timed region (the quantizer is timed separately).

Workloads (reduced_vocab_nvfp4_amd/workloads.py; seeded synthetic inputs):
  flash_next_64k   NVFP4 64 064 x 2560, batch 1, top token  (default)
  h98k_b16         NVFP4 (or --format e4m3, or w8a8: the E4M3 head with
                   per-token E4M3 activations) 98 304 x 2560, batch 16
  dense27b_64k_b8  NVFP4 64 064 x 5120, batch 8, fp32 logits to 248 320 ids
  stock_bf16       BF16 248 320 x 2560 (every id), batch 1, top token
  tiny             NVFP4 1024 x 256, batch 1 (launch-bound; correctness)
  linear_*         NVFP4 W4A16 linears of the drafter's block (nvfp4_linear,
                   dense fp32 out; no index, no argmax)

The timed region streams from HBM: R copies of the head rotate so that
R x head bytes exceeds twice the 256 MB Infinity Cache.  Timing: HIP events
recorded on the launch stream before and after K back-to-back calls
(preceded by a short GPU sleep so the host enqueues ahead of the device),
repeated (5 times by default); `value` is algorithmic bytes per step / the
median GPU time per step.  When profiles/ holds a rocprofv3 kernel-trace
figure taken on the current kernel sources, the line carries it too.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import reduced_vocab_nvfp4_amd as dh  # noqa: E402
from reduced_vocab_nvfp4_amd import workloads as wl  # noqa: E402

METRIC = ("draft-head µs/step and HBM GB/s (% peak), NVFP4 64064x2560 "
          "GEMV+argmax, batch 1")


def metric_name(case) -> str:
    """The headline metric for the default workload; the same measure named
    for the workload otherwise."""
    if case.name == "flash_next_64k" and case.op == "top":
        return METRIC
    if case.op == "linear":
        return (f"NVFP4 W4A16 linear µs/step and HBM GB/s (% peak), "
                f"{case.n_rows}x{case.H}, batch {case.B}")
    what = {"top": "GEMV+argmax", "logits": "GEMV+logits scatter",
            "top_bf16": "GEMV+argmax over BF16-rounded logits",
            "logits_bf16": "GEMV+BF16 logits scatter"}[case.op]
    return (f"draft-head µs/step and HBM GB/s (% peak), {case.fmt.upper()} "
            f"{case.n_rows}x{case.H} {what}, batch {case.B}")
HBM_PEAK_GBS = 8000.0
INFINITY_CACHE = 256 << 20
RTOL, ATOL = 1e-3, 1e-4


def weight_bytes(fmt, n_rows, hidden):
    return {"nvfp4": n_rows * hidden // 2 + n_rows * hidden // 16,
            "e4m3": n_rows * hidden, "w8a8": n_rows * hidden,
            "bf16": n_rows * hidden * 2}[fmt]


def algorithmic_bytes(fmt, n_rows, hidden, batch, op, vocab):
    """Bytes a step must move: the head (codes and scales), h, the tensor
    scale, then either the winning dh_idx entries and the out ids, or the
    dh_idx column and the full fp32 logits.  (The W8A8 step's quantized
    tokens are an intermediate, not counted.)"""
    b = weight_bytes(fmt, n_rows, hidden) + batch * hidden * 2
    b += 4 if fmt != "bf16" else 0
    if op == "logits":
        b += n_rows * 4 + batch * vocab * 4
    elif op == "logits_bf16":
        b += n_rows * 4 + batch * vocab * 2
    elif op == "linear":
        b += batch * n_rows * 4
    else:
        b += batch * 4 + batch * 4
    return b


def code_text(src: str) -> str:
    """C/C++/HIP source without comments and with whitespace collapsed: what
    the compiler sees, so a comment edit does not mark measurements stale.
    (The kernel sources hold no "//" or "/*" inside string literals.)"""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_source_hash(csrc=None):
    """Hash of the kernel sources' code (comments and layout excluded)."""
    h = hashlib.sha256()
    csrc = csrc or os.path.join(ROOT, "reduced_vocab_nvfp4_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode() + code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def _profile(kind, case, kernel_hash):
    """A committed profiles/<kind>_<case>.json, only if it was taken on the
    current kernel sources."""
    p = os.path.join(ROOT, "profiles", f"{kind}_{case}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_hash:
        return None
    return t


def load_traffic(case, kernel_hash):
    """HBM traffic per step from committed rocprofv3 counter runs."""
    t = _profile("traffic", case, kernel_hash)
    return t.get("hbm_bytes_per_step") if t else None


def load_kernel_time(case, kernel_hash):
    """Kernel time per step (µs, summed over the step's kernels) from a
    committed rocprofv3 --kernel-trace --stats run."""
    t = _profile("kernel_time", case, kernel_hash)
    return t.get("kernel_us_per_step") if t else None


class Case:
    """One workload in one format: the head on the GPU, a lean per-step
    call (pointers resolved once: argument marshalling only) and the oracle's
    version of the step."""

    def __init__(self, config, fmt, op, dev, stream):
        self.config, self.fmt = config, fmt
        w_ = wl.WORKLOADS[config]
        if fmt not in w_.formats:
            raise SystemExit(f"workload {config} has no {fmt} head "
                             f"(formats: {', '.join(w_.formats)})")
        self.V, self.H, self.B = w_.vocab, w_.hidden, w_.batch
        default_op = ("linear" if w_.linear else
                      "logits" if w_.logits and w_.batch > 1 else "top")
        if w_.linear and op not in (None, "linear"):
            raise SystemExit(f"workload {config} is a linear; --op does not "
                             f"apply")
        self.op = op or default_op
        if self.op in ("top_bf16", "logits_bf16") and fmt != "nvfp4":
            raise SystemExit("the BF16-rounded ops run on the NVFP4 head")
        self.name = config if fmt == w_.formats[0] else f"{config}_{fmt}"
        if self.op != default_op:
            self.name += f"_{self.op}"
        t0 = time.perf_counter()
        self.w = wl.head_weight(self.V, self.H)
        keep = wl.keep_mask(w_)
        idx, self.n_kept = dh.draft_head_build_index(keep)
        self.idx = idx.numpy()
        self.n_rows = idx.shape[0]
        self.idx_gpu = idx.to(dev)
        self.ws = (dh.new_workspace_w8a8(self.n_rows, self.B, self.H, dev)
                   if fmt == "w8a8" else
                   dh.new_workspace(self.n_rows, self.B, dev))
        w_gpu = self.w.to(dev)
        self.quant_us = None
        if fmt == "nvfp4":
            packed, scales, self.scale = dh.nvfp4_quantize_rows(
                w_gpu, self.idx_gpu, workspace=self.ws)
            quant = lambda: dh.nvfp4_quantize_rows(  # noqa: E731
                w_gpu, self.idx_gpu, packed=packed, scales=scales,
                global_scale=self.scale, workspace=self.ws)
            tensors = (packed, scales)
        elif fmt in ("e4m3", "w8a8"):
            q, self.scale = dh.e4m3_quantize_rows_per_tensor(
                w_gpu, self.idx_gpu, workspace=self.ws)
            quant = lambda: dh.e4m3_quantize_rows_per_tensor(  # noqa: E731
                w_gpu, self.idx_gpu, q=q, scale=self.scale,
                workspace=self.ws)
            tensors = (q,)
        else:
            rows = w_gpu if w_.identity else \
                w_gpu[self.idx_gpu.long()].contiguous()
            self.scale, quant, tensors = None, None, (rows,)
        torch.cuda.synchronize()
        if quant is not None:
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            for _ in range(5):
                quant()
            ev[1].record(stream)
            torch.cuda.synchronize()
            self.quant_us = ev[0].elapsed_time(ev[1]) * 1000.0 / 5
        del w_gpu, quant
        self.head_bytes = weight_bytes(fmt, self.n_rows, self.H)
        self.nbytes = algorithmic_bytes(fmt, self.n_rows, self.H, self.B,
                                        self.op, self.V)
        self.setup_s = time.perf_counter() - t0
        self.tensors = tensors

    def rotate(self, R):
        self.R = R
        self.heads = [self.tensors] + [tuple(t.clone() for t in self.tensors)
                                       for _ in range(R - 1)]

    def make_step(self, h_ptrs, out, stream):
        L = dh.lib()
        sp = int(stream.cuda_stream)
        heads = [tuple(t.data_ptr() for t in hd) for hd in self.heads]
        sc = self.scale.data_ptr() if self.scale is not None else None
        idx_p, ws_p, ws_n = (self.idx_gpu.data_ptr(), self.ws.data_ptr(),
                             self.ws.numel())
        n, H, B, R, nh = self.n_rows, self.H, self.B, self.R, len(h_ptrs)
        out_p = out.data_ptr()
        fmt = self.fmt
        if self.op == "linear":
            stride = B * n * 4

            def step(i):
                hd = heads[i % R]
                rc = L.nvfp4_linear(hd[0], hd[1], sc, n, H, h_ptrs[i % nh], B,
                                    out_p + stride * (i % 2), sp)
                if rc:
                    raise dh.DraftHeadError("linear", rc)
            return step
        if self.op == "logits_bf16":
            stride = B * self.V * 2
            nk, V = self.n_kept, self.V

            def step(i):
                hd = heads[i % R]
                rc = L.draft_head_logits_compat(
                    hd[0], hd[1], sc, idx_p, n, nk, H, V, h_ptrs[i % nh], B,
                    out_p + stride * (i % 2), ws_p, ws_n, sp)
                if rc:
                    raise dh.DraftHeadError("logits (BF16)", rc)
            return step
        if self.op == "logits":
            stride = B * self.V * 4
            nk, V = self.n_kept, self.V

            if fmt == "nvfp4":
                def lcall(hd, hp, o):
                    return L.draft_head_logits(hd[0], hd[1], sc, idx_p, n, nk,
                                               H, V, hp, B, o, ws_p, ws_n, sp)
            elif fmt == "e4m3":
                def lcall(hd, hp, o):
                    return L.draft_head_logits_e4m3(hd[0], sc, idx_p, n, nk,
                                                    H, V, hp, B, o, ws_p,
                                                    ws_n, sp)
            elif fmt == "w8a8":
                def lcall(hd, hp, o):
                    return L.draft_head_logits_w8a8(hd[0], sc, idx_p, n, nk,
                                                    H, V, hp, B, o, ws_p,
                                                    ws_n, sp)
            else:
                def lcall(hd, hp, o):
                    return L.draft_head_logits_bf16(hd[0], idx_p, n, nk, H, V,
                                                    hp, B, o, ws_p, ws_n, sp)

            def step(i):
                rc = lcall(heads[i % R], h_ptrs[i % nh],
                           out_p + stride * (i % 2))
                if rc:
                    raise dh.DraftHeadError(f"logits ({fmt})", rc)
            return step
        if self.op == "top_bf16":
            def call(hd, hp, o):
                return L.draft_head_top_tokens_compat(hd[0], hd[1], sc, idx_p,
                                                      n, H, hp, B, o, ws_p,
                                                      ws_n, sp)
        elif fmt == "nvfp4":
            def call(hd, hp, o):
                return L.draft_head_top_tokens(hd[0], hd[1], sc, idx_p, n, H,
                                               hp, B, o, ws_p, ws_n, sp)
        elif fmt == "e4m3":
            def call(hd, hp, o):
                return L.draft_head_top_tokens_e4m3(hd[0], sc, idx_p, n, H,
                                                    hp, B, o, ws_p, ws_n, sp)
        elif fmt == "w8a8":
            def call(hd, hp, o):
                return L.draft_head_top_tokens_w8a8(hd[0], sc, idx_p, n, H,
                                                    hp, B, o, ws_p, ws_n, sp)
        else:
            def call(hd, hp, o):
                return L.draft_head_top_tokens_bf16(hd[0], idx_p, n, H, hp,
                                                    B, o, ws_p, ws_n, sp)

        def step(i):
            rc = call(heads[i % R], h_ptrs[i % nh], out_p + 4 * B * i)
            if rc:
                raise dh.DraftHeadError(f"top tokens ({fmt})", rc)
        return step

    # ---- the oracle's step ------------------------------------------------
    def oracle_setup(self):
        import oracle
        bits = wl.bf16_bits(self.w)
        t0 = time.perf_counter()
        if self.fmt == "nvfp4":
            self.o_head = oracle.nvfp4_quantize(bits, self.idx)
        elif self.fmt in ("e4m3", "w8a8"):
            self.o_head = oracle.e4m3_tensor_quantize(bits, self.idx)
        else:
            self.o_head = bits
        return time.perf_counter() - t0

    def oracle_gemv_rows(self, h, m):
        """The oracle's GEMV over the first m rows only (the part of a step
        that scales with the head): times a single-thread sample."""
        import oracle
        hb = wl.bf16_bits(h)
        if self.fmt == "nvfp4":
            p, sc, g = self.o_head
            return oracle.nvfp4_logits(p[:m], sc[:m], g, hb)
        if self.fmt == "e4m3":
            q, sc = self.o_head
            return oracle.e4m3_tensor_logits(q[:m], sc, hb)
        if self.fmt == "w8a8":
            q, sc = self.o_head
            return oracle.w8a8_logits(q[:m], sc,
                                      *oracle.fp8_tokens_quantize(hb))
        return oracle.bf16_logits(self.o_head, self.idx[:m], hb)

    def oracle_step(self, h):
        import oracle
        hb = wl.bf16_bits(h)
        if self.fmt == "nvfp4":
            L = oracle.nvfp4_logits(*self.o_head, hb)
        elif self.fmt == "e4m3":
            L = oracle.e4m3_tensor_logits(*self.o_head, hb)
        elif self.fmt == "w8a8":
            L = oracle.w8a8_logits(*self.o_head,
                                   *oracle.fp8_tokens_quantize(hb))
        else:
            L = oracle.bf16_logits(self.o_head, self.idx, hb)
        if self.op == "logits":
            return L, oracle.logits_scatter(L, self.n_kept, self.idx, self.V)
        if self.op == "linear":
            return L, L
        if self.op in ("top_bf16", "logits_bf16"):
            Lb = oracle.logits_to_bf16(L)
            if self.op == "logits_bf16":
                return L, oracle.logits_scatter_bf16(Lb, self.n_kept,
                                                     self.idx, self.V)
            rows = np.argmax(oracle.bf16_bits_value(Lb), axis=1)
            return L, self.idx[rows]
        return L, oracle.argmax_remap(L, self.idx)[1]


def time_read_probe(case, K, reps, stream):
    """The plain streaming read of the step's own head buffers, in the same
    rotation and with the same timing as the step (drafthead_read_probe):
    the rate at which this device streams those bytes with nothing else to
    do, the practical ceiling of the step's weight stream.  Median µs per
    read over the repeats."""
    L = dh.lib()
    sp = int(stream.cuda_stream)
    sink = torch.zeros(1, dtype=torch.int32, device=case.heads[0][0].device)
    sk = sink.data_ptr()
    bufs = []
    for hd in case.heads:
        a = hd[0]
        b = hd[1] if len(hd) > 1 else None
        bufs.append((a.data_ptr(), a.numel() * a.element_size(),
                     b.data_ptr() if b is not None else None,
                     b.numel() * b.element_size() if b is not None else 0))
    R = len(bufs)

    def call(i):
        pa, na, pb, nb = bufs[i % R]
        rc = L.drafthead_read_probe(pa, na, pb, nb, sk, sp)
        if rc != 0:
            raise RuntimeError(f"drafthead_read_probe: {dh.error_string(rc)}")
    for i in range(2 * R):
        call(i)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    us = []
    for _ in range(reps):
        torch.cuda.synchronize()
        try:
            torch.cuda._sleep(int(2e7))
        except (AttributeError, RuntimeError):
            pass
        e0.record(stream)
        for i in range(K):
            call(i)
        e1.record(stream)
        torch.cuda.synchronize()
        us.append(e0.elapsed_time(e1) * 1000.0 / K)
    return float(np.median(us))


def cpu_baseline(case, h_list, budget_s):
    """The oracle's step (float64 GEMV over every row, then argmax + remap
    or the logits scatter) on the host, repeated on full steps until
    budget_s elapse (at least one step)."""
    import oracle
    t_quant = case.oracle_setup()
    times, results = [], []
    t_start = time.perf_counter()
    i = 0
    while True:
        h = h_list[i % len(h_list)]
        t0 = time.perf_counter()
        r = case.oracle_step(h)
        times.append(time.perf_counter() - t0)
        if i < len(h_list):
            results.append(r)
        i += 1
        if time.perf_counter() - t_start > budget_s or i >= 64:
            break
    threads = oracle.num_threads()
    step_s = float(np.median(times))
    # one step on one thread: the full step when it fits the budget (about
    # threads x the parallel step), else the GEMV over a leading slice of
    # rows scaled to all of them (the rest of a step is a small part of it)
    single_s, single_rows = None, None
    oracle.set_threads(1)
    try:
        if step_s * threads <= budget_s:
            t0 = time.perf_counter()
            case.oracle_step(h_list[0])
            single_s = time.perf_counter() - t0
        else:
            m = max(64, int(case.n_rows * budget_s / 4 / (step_s * threads)))
            m = min(m - m % 64, case.n_rows)
            t0 = time.perf_counter()
            case.oracle_gemv_rows(h_list[0], m)
            single_s = (time.perf_counter() - t0) * case.n_rows / m
            single_rows = m
    finally:
        oracle.set_threads(threads)
    return {"step_s": step_s, "steps": len(times), "threads": threads,
            "single_thread_s": single_s, "single_thread_rows": single_rows,
            "quantize_s": t_quant, "results": results}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def check_top(ids, results, case, n_h):
    """Ids of every timed step whose h the oracle ran, with the near-tie
    rule: a different id passes when its oracle logit is within the logit
    tolerance of the oracle's maximum."""
    parity = {"checked_steps": 0, "mismatches": 0, "near_tie_exceptions": 0}
    for hi, (Lo, want) in enumerate(results):
        for b in range(case.B):
            lmax = Lo[b].max()
            for g in ids[hi::n_h, b]:  # every step that used this h
                parity["checked_steps"] += 1
                if int(g) == int(want[b]):
                    continue
                r = np.flatnonzero(case.idx[:case.n_kept] == g)
                gap = lmax - Lo[b, r[0]] if r.size else np.inf
                if gap <= ATOL + RTOL * abs(lmax):
                    parity["near_tie_exceptions"] += 1
                else:
                    parity["mismatches"] += 1
    return parity


def check_logits(out, ref):
    fin = np.isfinite(ref)
    bad = int((np.isfinite(out) != fin).sum())
    bad += int((out.view(np.uint32)[~fin] != 0xFF800000).sum())
    err = np.abs(out[fin].astype(np.float64) - ref[fin])
    bad += int((err > ATOL + RTOL * np.abs(ref[fin])).sum())
    return {"checked_values": int(out.size), "mismatches": bad,
            "max_abs_err": float(err.max()) if err.size else 0.0}


def check_logits_bf16(got, ref, L64, case):
    """BF16 logits: equal to the oracle's rounding, or (where the float64
    logit is within the float32 GEMV's error of a rounding boundary) a BF16
    value between the roundings of L - err and L + err."""
    import oracle
    bad = got != ref
    n_bad = 0
    if bad.any():
        err = 1e-5 + 1e-5 * np.abs(L64)
        lo = oracle.bf16_bits_value(oracle.logits_scatter_bf16(
            oracle.logits_to_bf16(L64 - err), case.n_kept, case.idx, case.V))
        hi = oracle.bf16_bits_value(oracle.logits_scatter_bf16(
            oracle.logits_to_bf16(L64 + err), case.n_kept, case.idx, case.V))
        v = oracle.bf16_bits_value(got)
        n_bad = int((bad & ~((v >= lo) & (v <= hi))).sum())
    return {"checked_values": int(got.size), "mismatches": n_bad,
            "boundary_values": int(bad.sum()) - n_bad}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed runs of --steps calls; the median is "
                         "reported")
    ap.add_argument("--config", default="flash_next_64k",
                    choices=sorted(wl.WORKLOADS))
    ap.add_argument("--format", default=None,
                    choices=["nvfp4", "e4m3", "w8a8", "bf16"],
                    help="head format (default: the workload's first)")
    ap.add_argument("--op", default=None,
                    choices=["top", "logits", "top_bf16", "logits_bf16"],
                    help="step kind of a head workload (default: logits for "
                         "the batch-8 logits workload, else top tokens); "
                         "the linear workloads always run the linear")
    ap.add_argument("--rotate", type=int, default=0,
                    help="head copies to rotate (0: enough for 2x MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--seed", type=int, default=0,
                    help="first hidden-state step: the timed steps use the "
                         "seeds SEED_H0 + seed .. SEED_H0 + seed + 7")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="before the timed region, copy a MIB-MiB device "
                         "buffer 5 times (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.seed < 0:
        ap.error("--seed must be at least 0")

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU "
              "path (the head is replicated per GPU)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    fmt = args.format or wl.WORKLOADS[args.config].formats[0]
    case = Case(args.config, fmt, args.op, dev, stream)
    B, H, V = case.B, case.H, case.V

    if args.calibrate_copy:
        src = torch.empty(args.calibrate_copy << 20, dtype=torch.uint8,
                          device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.rotate:
        R = args.rotate
    elif case.head_bytes >= 2 * INFINITY_CACHE:
        R = 1
    else:
        # enough copies that every step reads its weights from HBM, as a
        # decode step does when the model's weights exceed the cache
        R = min(4096, -(-2 * INFINITY_CACHE // case.head_bytes) + 1)
    case.rotate(R)
    n_h = 8
    # the timed steps cycle through n_h hidden states, seeds SEED_H0 +
    # args.seed + i
    h_steps = [args.seed + i for i in range(n_h)]
    h_cpu = [wl.hidden_states(B, H, s) for s in h_steps]
    h_gpu = [x.to(dev) for x in h_cpu]
    h_ptrs = [x.data_ptr() for x in h_gpu]
    K, W = args.steps, args.warmup
    if case.op == "logits":
        out = torch.empty((2, B, V), dtype=torch.float32, device=dev)
    elif case.op == "logits_bf16":
        out = torch.empty((2, B, V), dtype=torch.bfloat16, device=dev)
    elif case.op == "linear":
        out = torch.empty((2, B, case.n_rows), dtype=torch.float32,
                          device=dev)
    else:
        out = torch.zeros((K + W, B), dtype=torch.int32, device=dev)
    step = case.make_step(h_ptrs, out, stream)
    for i in range(W):
        step(K + i if case.op in ("top", "top_bf16") else i)
    torch.cuda.synchronize()

    # Timed region: K back-to-back calls between two events recorded on the
    # launch stream (per-step event records would add their own gaps),
    # repeated; the median repeat is reported.  A short device-side sleep
    # before each repeat lets the host enqueue ahead of the GPU.
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    reps = max(1, args.repeats)
    rep_us, host_us = [], []
    t_wall = 0.0
    for _ in range(reps):
        torch.cuda.synchronize()
        t_wall0 = time.perf_counter()
        try:
            torch.cuda._sleep(int(2e7))
        except (AttributeError, RuntimeError):
            pass
        e0.record(stream)
        t_host0 = time.perf_counter()
        for i in range(K):
            step(i)
        # host time to enqueue the K calls (the device is still busy): when
        # it exceeds the device time per step, the device waits for the host
        host_us.append((time.perf_counter() - t_host0) * 1e6 / K)
        e1.record(stream)
        torch.cuda.synchronize()
        t_wall += time.perf_counter() - t_wall0
        rep_us.append(e0.elapsed_time(e1) * 1000.0 / K)
    us_step = float(np.median(rep_us))
    gbs = case.nbytes / (us_step * 1e-6) / 1e9
    read_us = time_read_probe(case, K, reps, stream)
    read_gbs = case.head_bytes / (read_us * 1e-6) / 1e9

    # ---- parity against the oracle, and the CPU leg -----------------------
    result_cpu, parity = None, None
    if not args.no_cpu_baseline:
        cb = cpu_baseline(case, h_cpu, args.cpu_budget)
        if case.op == "logits_bf16":
            hi = (K - 1) % n_h
            L64, ref = (cb["results"][hi] if hi < len(cb["results"])
                        else case.oracle_step(h_cpu[hi]))
            got = out[(K - 1) % 2].cpu().view(torch.int16).numpy().view(
                np.uint16)
            parity = check_logits_bf16(got, ref, L64, case)
        elif case.op in ("logits", "linear"):
            # the last timed step used h[(K-1) % n_h] and buffer (K-1) % 2
            hi = (K - 1) % n_h
            ref = (cb["results"][hi] if hi < len(cb["results"])
                   else case.oracle_step(h_cpu[hi]))[1]
            parity = check_logits(out[(K - 1) % 2].cpu().numpy(), ref)
        else:
            parity = check_top(out[:K].cpu().numpy(), cb["results"], case,
                               n_h)
        what = {"logits": "logits scatter", "linear": "dense fp32 out",
                "top": "argmax, remap",
                "top_bf16": "BF16 rounding, argmax, remap",
                "logits_bf16": "BF16 logits scatter"}[case.op]
        result_cpu = {
            "value": round(case.nbytes / cb["step_s"] / 1e9, 3),
            "unit": "GB/s",
            "us_per_step": round(cb["step_s"] * 1e6, 1),
            "cores": cb["threads"],
            "kind": "oracle",
            "single_thread_us_per_step": (
                round(cb["single_thread_s"] * 1e6, 1)
                if cb["single_thread_s"] is not None else None),
            # when set: the single-thread figure is the GEMV over this many
            # leading rows, scaled to the whole head
            "single_thread_sampled_rows": cb["single_thread_rows"],
            "quantize_ms": (round(cb["quantize_s"] * 1e3, 1)
                            if cb["quantize_s"] is not None else None),
            "sample": (f"{cb['steps']} full steps of {case.name} (float64 "
                       f"GEMV over {case.n_rows} rows x {H}, batch {B}, "
                       f"{what}), median; host {os.cpu_count()} visible "
                       f"CPUs, {cpu_model()}"),
        }

    khash = kernel_source_hash()
    k_us = load_kernel_time(case.name, khash)
    rec = {
        "metric": metric_name(case),
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(us_step / 1000.0, 6),
        "us_per_step": round(us_step, 3),
        "repeats": reps,
        "us_per_step_repeats": [round(x, 3) for x in rep_us],
        "host_enqueue_us_per_call": round(float(np.median(host_us)), 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": case.name, "vocab": V, "hidden": H, "batch": B,
            "n_rows": case.n_rows, "n_kept": case.n_kept,
            "format": {"nvfp4": "nvfp4-w4a16", "e4m3": "e4m3-w8a16",
                       "w8a8": "e4m3-w8a8", "bf16": "bf16"}[fmt],
            "step": {"top": "top tokens",
                     "top_bf16": "top tokens over BF16-rounded logits",
                     "logits_bf16": "BF16 logits to the full vocab",
                     "logits": "fp32 logits to the full vocab",
                     "linear": "NVFP4 W4A16 linear, fp32 out"}[case.op],
            "rotated_head_copies": R, "parallelism": "none (1 GPU)",
            "h_seeds": [wl.SEED_H0 + s for s in h_steps],
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": load_traffic(case.name, khash),
            "bytes_per_step": case.nbytes,
            "launches_per_step": 1 + (1 if fmt == "w8a8" else 0),
            # the committed rocprofv3 kernel-trace time of this step on the
            # current kernel sources (null when the sources changed since)
            "rocprof_kernel_us": k_us,
            "rocprof_frac": (round(case.nbytes / (k_us * 1e-6) / 1e9
                                   / HBM_PEAK_GBS, 4) if k_us else None),
            # a plain streaming read of the same head buffers, timed the same
            # way in the same run: the step's weight stream against the rate
            # this device reaches for those bytes with nothing else to do
            "plain_read": {
                "us": round(read_us, 3),
                "bytes": case.head_bytes,
                "gbs": round(read_gbs, 2),
                "frac": round(read_gbs / HBM_PEAK_GBS, 4),
                "step_over_plain_read": round(read_us / us_step, 4),
            },
        },
        "cpu_baseline": result_cpu,
        "parity": parity,
        "quantize_us": round(case.quant_us, 1) if case.quant_us else None,
        "setup_s": round(case.setup_s, 1),
        "wall_s_timed": round(t_wall, 4),
        "kernel_source_hash": khash,
    }
    print(json.dumps(rec), flush=True)
    if parity and parity["mismatches"]:
        sys.exit(1)


if __name__ == "__main__":
    main()
