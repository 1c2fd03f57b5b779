"""Throughput of the DSA indexer -> top-2,048 -> sparse MLA read on one MI355X.

One step = one pass of the whole read over one batch (index scores, top-k,
then the sparse MLA read of every layer that shares the selection), through
the C ABI, with all inputs resident in HBM.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 0..4] [--no-cpu]

The default workload is the decode batch of 64 sequences at 32,768 positions
(bf16).  `roofline` describes the dominant kernel (the indexer): algorithmic
bytes (or FLOP) per launch over its average duration, timed with HIP events
on the launch stream inside the timed region.  `cpu_baseline` times the CPU
oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
FP32_VALU_PEAK_TFLOPS = 157.3   # MI355X fp32 vector, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=1)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU oracle sample budget")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(every workload runs on a single MI355X); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from sparse_attention_12_amd import binding as B
    from sparse_attention_12_amd import costmodel, workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_gen = time.time()
    w = workloads.config(args.config)
    print(f"[bench] workload {w.name}: nq={w.nq} layers={w.n_layers} max_len={w.max_len} "
          f"(generated in {time.time() - t_gen:.1f}s)", file=sys.stderr, flush=True)
    t = w.to_torch(dev)
    batch = B.Batch(t["q_seq"], t["q_pos"], t["seq_len"], t["seq_row0"], w.max_len)
    k, L = w.k, w.n_layers
    scores = torch.empty((w.nq, w.max_len), dtype=torch.float32, device=dev)
    idx = torch.empty((w.nq, k), dtype=torch.int32, device=dev)
    count = torch.empty((w.nq,), dtype=torch.int32, device=dev)
    outs = [torch.empty((w.nq, 64, 512), dtype=torch.float32, device=dev) for _ in range(L)]
    lses = [torch.empty((w.nq, 64), dtype=torch.float32, device=dev) for _ in range(L)]
    tk_ws_n = B.dsa_topk_workspace_size(w.nq, w.max_len, k)
    tk_ws = torch.empty(max(tk_ws_n, 256), dtype=torch.uint8, device=dev)
    mla_ws = torch.empty(max(B.mla_sparse_attend_workspace_size(w.nq, k, 1), 256), dtype=torch.uint8,
                         device=dev)
    stream = torch.cuda.current_stream()

    ev_idx = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]

    def step(i=None):
        if i is not None:
            ev_idx[i][0].record(stream)
        B.dsa_index_score(batch, t["qI"], t["w"], t["kI"], scores)
        if i is not None:
            ev_idx[i][1].record(stream)
        B.dsa_topk(batch, scores, k, idx, count, tk_ws if tk_ws_n else None)
        for l in range(L):
            B.mla_sparse_attend(batch, t["q"][l], t["kv"][l], idx, k, w.tau, outs[l], lses[l], mla_ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t0.elapsed_time(t1) / args.steps
    idx_ms = sum(a.elapsed_time(b) for a, b in ev_idx) / args.steps
    print(f"[bench] {args.steps} steps: {ms_per_step:.4f} ms/step (wall {wall * 1e3 / args.steps:.4f}); "
          f"indexer {idx_ms:.4f} ms", file=sys.stderr, flush=True)

    # the fused entry point (one call: indexer, top-k, every layer's MLA)
    fused_ws = torch.empty(B.dsa_mla_decode_fused_workspace_size(w.nq, w.max_len, k, L), dtype=torch.uint8,
                           device=dev)
    fused_ms = None
    if w.kind == "decode":
        for _ in range(max(2, args.warmup)):
            B.dsa_mla_decode_fused(batch, t["qI"], t["w"], t["kI"], k, t["q"], t["kv"], outs, w.tau, lses, idx,
                                   fused_ws)
        f0 = torch.cuda.Event(enable_timing=True)
        f1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        f0.record(stream)
        for _ in range(args.steps):
            B.dsa_mla_decode_fused(batch, t["qI"], t["w"], t["kI"], k, t["q"], t["kv"], outs, w.tau, lses, idx,
                                   fused_ws)
        f1.record(stream)
        torch.cuda.synchronize()
        fused_ms = f0.elapsed_time(f1) / args.steps

    tr = costmodel.path_traffic(w.seq_len, w.q_seq, w.q_pos, w.dtype, L, k)
    value = w.nq / (ms_per_step / 1e3)
    if w.kind == "prefill":
        achieved = tr["indexer"]["flop"] / (idx_ms / 1e3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=BF16_MFMA_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / BF16_MFMA_PEAK_TFLOPS, 4), traffic=None,
                    kernel="idx_prefill_bf16", per_launch=tr["indexer"]["flop"], per_launch_unit="FLOP")
    elif w.dtype == "bf16":
        achieved = tr["indexer"]["bytes"] / (idx_ms / 1e3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBPS, 4), traffic=None,
                    kernel="idx_decode_bf16", per_launch=tr["indexer"]["bytes"], per_launch_unit="B")
    else:
        achieved = tr["indexer"]["flop"] / (idx_ms / 1e3) / 1e12
        roof = dict(bound="alu", achieved=round(achieved, 3), peak=FP32_VALU_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / FP32_VALU_PEAK_TFLOPS, 4), traffic=None,
                    kernel="idx_decode_f32", per_launch=tr["indexer"]["flop"], per_launch_unit="FLOP")
    path_gbps = tr["path_bytes"] / (ms_per_step / 1e3) / 1e9

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(w, args.cpu_seconds)

    rec = {
        "metric": "query-tokens/s for DSA index+top-2048+sparse MLA attn; % HBM/MFMA peak",
        "value": round(value, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; integer indexer inputs in [-3,3], weights in [1,4], N(0,1) queries and cache)",
        "config": {"workload": w.name, "queries": w.nq, "sequences": w.nseq, "max_context": w.max_len,
                   "layers_sharing_selection": L, "topk": k, "kind": w.kind},
        "roofline": roof,
        "cpu_baseline": cpu,
        "path": {"algorithmic_bytes": tr["path_bytes"], "algorithmic_flop": tr["path_flop"],
                 "GBps": round(path_gbps, 1), "hbm_frac": round(path_gbps / HBM_PEAK_GBPS, 4),
                 "indexer_ms": round(idx_ms, 5),
                 "fused_entry_ms_per_step": None if fused_ms is None else round(fused_ms, 5)},
    }
    print(json.dumps(rec))


def cpu_baseline(w, budget_s: float):
    """The CPU oracle, as it stands, on the first queries of the workload until
    the time budget is spent (at least one query)."""
    import numpy as np

    import oracle

    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        oracle.build(force=False)
    threads = oracle.max_threads()
    done = 0
    el = 0.0
    qIw = w.widen(w.qI)
    while done < w.nq and el < budget_s:
        qi = done
        s = int(w.q_seq[qi])
        n = oracle.n_candidates(int(w.q_pos[qi]), int(w.seq_len[s]))
        kI = w.widen(w.seq_rows(w.kI, s))
        qs = [w.widen(x[qi]) for x in w.q]
        kvs = [w.widen(w.seq_rows(x, s)) for x in w.kv]
        t0 = time.perf_counter()
        oracle.decode_query(qIw[qi], w.w[qi], kI, qs, kvs, n, w.k, w.tau)
        el += time.perf_counter() - t0
        done += 1
    return {"value": round(done / el, 3), "unit": "query-tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {done} of {w.nq} queries of the same workload ({el:.1f} s of oracle time, "
                      f"fp64 C oracle, OpenMP over positions and heads)"}


if __name__ == "__main__":
    main()
