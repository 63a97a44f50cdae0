#!/usr/bin/env python3
"""Draft-head step benchmark on one MI355X.

One step = one greedy draft-head call, the hot path of the method
(page 1, "q38_draft.py", get_top_tokens; page 4, "Qwen3.8-27B-NVFP4-DGX-SPARK",
why native MTP plateaus: the head GEMV dominates a draft step): a W4A16
NVFP4 GEMV of a BF16 hidden state against the kept rows, the argmax over them
and the id remap, all in one kernel launch.  The row index and the NVFP4
quantization happen once, at load, outside the timed region.

Default workload: the Flash-Next-shaped head, 248 320 x 2560 BF16 target
head, 64 026 kept ids padded to 64 064 rows, batch 1.  Inputs are seeded and
synthetic (see reduced_vocab_nvfp4_amd/workloads.py).

The timed region streams from HBM: R copies of the quantized head rotate so
that R x 92 MB exceeds twice the 256 MB Infinity Cache.  Timing: HIP events
recorded on the launch stream before and after K back-to-back launches
(preceded by a short GPU sleep so the host enqueues ahead of the device);
`value` is algorithmic bytes per step / GPU time per step.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
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
HBM_PEAK_GBS = 8000.0
INFINITY_CACHE = 256 << 20


def algorithmic_bytes(n_rows, hidden, batch, logits_vocab=0):
    """Bytes a step must move: packed codes, E4M3 scales, h, the global
    scale, the out ids (and the dh_idx / logits traffic on the logits
    path)."""
    b = n_rows * hidden // 2 + n_rows * hidden // 16 + batch * hidden * 2 + 4
    if logits_vocab:
        b += n_rows * 4 + batch * logits_vocab * 4
    else:
        b += 4 + batch * 4  # the winning dh_idx entry and the out ids
    return b


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "reduced_vocab_nvfp4_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_hash):
    """HBM traffic per launch from committed rocprofv3 counter runs, only if
    they were taken on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", "traffic_flash_next_64k.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_hash:
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(head, h_list, budget_s=10.0):
    """The oracle's top-token step (float64 GEMV over every row, argmax,
    remap) on the host, repeated on full steps until budget_s elapse."""
    import oracle
    t0 = time.perf_counter()
    op, os_, ogs = oracle.nvfp4_quantize(head["w_bits"], head["idx"])
    t_quant = time.perf_counter() - t0
    times = []
    ids = []
    t_start = time.perf_counter()
    i = 0
    while True:
        h = h_list[i % len(h_list)]
        t0 = time.perf_counter()
        L = oracle.nvfp4_logits(op, os_, ogs, wl.bf16_bits(h))
        _, idd = oracle.argmax_remap(L, head["idx"])
        times.append(time.perf_counter() - t0)
        ids.append((i % len(h_list), int(idd[0]), L))
        i += 1
        if time.perf_counter() - t_start > budget_s or i >= 64:
            break
    return {
        "step_s": float(np.median(times)),
        "steps": len(times),
        "threads": oracle.num_threads(),
        "quantize_s": t_quant,
        "ids": ids,
        "oracle_head": (op, os_, ogs),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="flash_next_64k",
                    choices=sorted(wl.WORKLOADS))
    ap.add_argument("--rotate", type=int, default=0,
                    help="head copies to rotate (0: enough for 2x MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="before the timed region, copy a MIB-MiB device "
                         "buffer 5 times (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU "
              "path (the head is replicated per GPU; see DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    w_ = wl.WORKLOADS[args.config]
    if "nvfp4" not in w_.formats:
        print(f"workload {args.config} has no NVFP4 head", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    V, H, B = w_.vocab, w_.hidden, w_.batch

    # ---- setup (untimed): weights, index, quantization ------------------
    t0 = time.perf_counter()
    w = wl.head_weight(V, H)
    keep = wl.keep_mask(w_)
    idx, n_kept = dh.draft_head_build_index(keep)
    n_rows = idx.shape[0]
    w_gpu = w.to(dev)
    idx_gpu = idx.to(dev)
    ws = dh.new_workspace(n_rows, B, dev)
    packed, scales, gs = dh.nvfp4_quantize_rows(w_gpu, idx_gpu, workspace=ws)
    torch.cuda.synchronize()
    # quantizer timing (load-time step), a few repetitions
    qe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    qe[0].record(stream)
    for _ in range(5):
        dh.nvfp4_quantize_rows(w_gpu, idx_gpu, packed=packed, scales=scales,
                               global_scale=gs, workspace=ws)
    qe[1].record(stream)
    torch.cuda.synchronize()
    quant_us = qe[0].elapsed_time(qe[1]) * 1000.0 / 5
    del w_gpu
    setup_s = time.perf_counter() - t0

    if args.calibrate_copy:
        src = torch.empty(args.calibrate_copy << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    head_bytes = n_rows * H // 2 + n_rows * H // 16
    R = args.rotate or max(1, -(-2 * INFINITY_CACHE // head_bytes) + 1)
    heads = [(packed, scales)] + [(packed.clone(), scales.clone())
                                  for _ in range(R - 1)]
    n_h = 8
    h_cpu = [wl.hidden_states(B, H, s) for s in range(n_h)]
    h_gpu = [x.to(dev) for x in h_cpu]
    K, W = args.steps, args.warmup
    out = torch.zeros((K + W, B), dtype=torch.int32, device=dev)

    # Lean per-step call: pointers resolved once (argument marshalling only).
    L = dh.lib()
    sp = int(stream.cuda_stream)
    heads_p = [(p.data_ptr(), s.data_ptr()) for p, s in heads]
    h_p = [x.data_ptr() for x in h_gpu]
    gs_p, idx_p, ws_p, ws_n = gs.data_ptr(), idx_gpu.data_ptr(), ws.data_ptr(), ws.numel()
    out_p = out.data_ptr()

    def step(i):
        p, s = heads_p[i % R]
        rc = L.draft_head_top_tokens(p, s, gs_p, idx_p, n_rows, H,
                                     h_p[i % n_h], B, out_p + 4 * B * i,
                                     ws_p, ws_n, sp)
        if rc != 0:
            raise dh.DraftHeadError("draft_head_top_tokens", rc)

    for i in range(W):
        step(K + i)
    torch.cuda.synchronize()

    # Timed region: K back-to-back launches between two events recorded on
    # the launch stream (per-step event records would add their own gaps).
    # A short device-side sleep first lets the host enqueue ahead of the GPU.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    try:
        torch.cuda._sleep(int(2e7))
    except (AttributeError, RuntimeError):
        pass
    e0.record(stream)
    for i in range(K):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    total_us = e0.elapsed_time(e1) * 1000.0
    us_step = total_us / K

    nbytes = algorithmic_bytes(n_rows, H, B)
    gbs = nbytes / (us_step * 1e-6) / 1e9
    ids = out[:K].cpu().numpy()

    # ---- parity of sampled steps against the oracle, and the CPU leg ----
    result_cpu = None
    parity = {"checked_steps": 0, "mismatches": 0, "near_tie_exceptions": 0}
    if not args.no_cpu_baseline:
        cb = cpu_baseline({"w_bits": wl.bf16_bits(w), "idx": idx.numpy()},
                          h_cpu, args.cpu_budget)
        import oracle
        idx_np = idx.numpy()
        for hi, _, Lo in cb["ids"][:n_h]:
            _, want = oracle.argmax_remap(Lo, idx_np)
            for b in range(B):
                lmax = Lo[b].max()
                for g in ids[hi::n_h, b]:  # every step that used this h
                    parity["checked_steps"] += 1
                    if int(g) == int(want[b]):
                        continue
                    r = np.flatnonzero(idx_np[:n_kept] == g)
                    gap = lmax - Lo[b, r[0]] if r.size else np.inf
                    if gap <= 1e-4 + 1e-3 * abs(lmax):
                        parity["near_tie_exceptions"] += 1
                    else:
                        parity["mismatches"] += 1
        cpu_us = cb["step_s"] * 1e6
        result_cpu = {
            "value": round(nbytes / cb["step_s"] / 1e9, 3),
            "unit": "GB/s",
            "us_per_step": round(cpu_us, 1),
            "cores": cb["threads"],
            "kind": "oracle",
            "sample": (f"{cb['steps']} full steps of {args.config} (float64 "
                       f"GEMV over {n_rows} rows x {H}, argmax, remap), "
                       f"median; host {os.cpu_count()} visible CPUs"),
        }

    khash = kernel_source_hash()
    rec = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(us_step / 1000.0, 6),
        "us_per_step": round(us_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": args.config, "vocab": V, "hidden": H, "batch": B,
            "n_rows": n_rows, "n_kept": n_kept, "format": "nvfp4-w4a16",
            "rotated_head_copies": R, "parallelism": "none (1 GPU)",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": load_traffic(khash),
            "bytes_per_launch": nbytes,
        },
        "cpu_baseline": result_cpu,
        "parity": parity,
        "quantize_us": round(quant_us, 1),
        "setup_s": round(setup_s, 1),
        "wall_s_timed": round(t_wall, 4),
        "kernel_source_hash": khash,
    }
    print(json.dumps(rec), flush=True)
    if parity["mismatches"]:
        sys.exit(1)


if __name__ == "__main__":
    main()
