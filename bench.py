"""Throughput of the DSA indexer -> top-2,048 -> sparse MLA read on one MI355X.

One step = one pass of the whole read over one batch (index scores, top-k,
then the sparse MLA read of every layer that shares the selection), through
the C ABI, with all inputs resident in HBM: the fused decode entry for decode
batches, the three calls in turn for a prefill chunk.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 0..4] [--no-cpu]
                  [--index-dtype fp8]
  python bench.py --model-layers 72 [--model-batch 64] [--model-context 32768]
      one decode step of every layer of the model's schedule (indexer layers,
      selection reuse, rotary-free layers, shared cache), inputs drawn on the
      GPU from a seeded generator (the caches of 63 layers do not fit a
      host-side draw in reasonable time); prints its own JSON line.

The default workload is the decode batch of 64 sequences at 32,768 positions
(bf16).  `roofline` describes the dominant kernel (the indexer): algorithmic
bytes (or FLOP) per launch over its average duration, timed with HIP events
on the launch stream over a timed loop of that kernel alone.  `cpu_baseline` times the CPU
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
FP8_MFMA_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 matrix, published
FP32_VALU_PEAK_TFLOPS = 157.3   # MI355X fp32 vector, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=1)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--index-dtype", choices=["bf16", "fp8"], default=None,
                    help="store the indexer's query and keys in this type (default: the workload's)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU oracle sample budget")
    ap.add_argument("--cold-reps", type=int, default=10,
                    help="extra steps, each after reading a 512 MiB buffer that evicts L2 and the Infinity Cache "
                         "(reported apart from the warm value)")
    ap.add_argument("--model-layers", type=int, default=0,
                    help="time a decode step over this many layers of the model's schedule instead")
    ap.add_argument("--model-batch", type=int, default=64)
    ap.add_argument("--model-context", type=int, default=32768)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the run, copy a device buffer of this size (for counter calibration)")
    return ap.parse_args()


def kernel_source_digest(kind: str) -> str:
    """sha256 of the HIP source holding the dominant kernel (counter data is
    only reused while it is unchanged)."""
    import hashlib
    src = os.path.join(ROOT, "sparse_attention_12_amd", "csrc", "indexer.hip")
    return hashlib.sha256(open(src, "rb").read()).hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    counter summary (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy of
    known size), or None if absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(f"{kernel}/{workload}")
    if not rec or rec.get("source_sha256") != kernel_source_digest(kernel):
        return None
    return rec["bytes_per_launch"]


def indexer_kernel(w) -> str:
    """The indexer kernel the library launches for this batch (same rules as
    its dispatch: batches of one sequence with 32 or more queries use the
    blocked matrix kernel, up to 1,024 decode queries the balanced range
    kernel)."""
    if w.index_dtype == "f32":
        return "idx_decode_f32"
    t = "fp8" if w.index_dtype == "fp8" else "bf16"
    if w.nseq == 1 and w.nq >= 32:
        return f"idx_prefill_{t}"
    return f"idx_decode_{t}_bal" if w.nq <= 1024 else f"idx_decode_{t}"


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(every workload runs on a single MI355X); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from sparse_attention_12_amd import binding as B
    from sparse_attention_12_amd import costmodel, workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.model_layers:
        model_step(args, dev)
        return
    t_gen = time.time()
    w = workloads.config(args.config, args.index_dtype)
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

    fused_ws = torch.empty(max(B.dsa_mla_decode_fused_workspace_size(w.nq, w.max_len, k, L), 256),
                           dtype=torch.uint8, device=dev)

    def step():
        if w.kind == "decode":
            # the decode read as one call: indexer, top-k, every layer's MLA
            B.dsa_mla_decode_fused(batch, t["qI"], t["w"], t["kI"], k, t["q"], t["kv"], outs, w.tau, lses, idx,
                                   fused_ws)
        else:
            B.dsa_index_score(batch, t["qI"], t["w"], t["kI"], scores)
            B.dsa_topk(batch, scores, k, idx, count, tk_ws if tk_ws_n else None)
            for l in range(L):
                B.mla_sparse_attend(batch, t["q"][l], t["kv"][l], idx, k, w.tau, outs[l], lses[l], mla_ws)

    def timed(fn, n):
        """Average ms per call of fn over n calls, HIP events on the launch stream."""
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ms_per_step = timed(step, args.steps)
    wall = time.perf_counter() - wall0

    # cold steps: before each, a read of a 512 MiB buffer evicts the 4 MB
    # L2s and the 256 MB Infinity Cache (with clean lines, so no write-back
    # competes with the step), so every input comes from HBM; only the step
    # is timed
    cold_ms = None
    if args.cold_reps > 0:
        flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
        tot = 0.0
        for _ in range(args.cold_reps):
            flush.sum()
            c0 = torch.cuda.Event(enable_timing=True)
            c1 = torch.cuda.Event(enable_timing=True)
            c0.record(stream)
            step()
            c1.record(stream)
            torch.cuda.synchronize()
            tot += c0.elapsed_time(c1)
        cold_ms = tot / args.cold_reps
        del flush

    # per-stage timings of the same kernels, same launch configurations
    idx_fn = lambda: B.dsa_index_score(batch, t["qI"], t["w"], t["kI"], scores)
    idx_fn()
    idx_ms = timed(idx_fn, args.steps)
    tk_fn = lambda: B.dsa_topk(batch, scores, k, idx, count, tk_ws if tk_ws_n else None)
    tk_ms = timed(tk_fn, args.steps)
    mla_fn = lambda: B.mla_sparse_attend(batch, t["q"][0], t["kv"][0], idx, k, w.tau, outs[0], lses[0], mla_ws)
    mla_ms = timed(mla_fn, args.steps)
    print(f"[bench] {args.steps} steps: {ms_per_step:.4f} ms/step (wall {wall * 1e3 / args.steps:.4f}); "
          f"indexer {idx_ms:.4f} ms, top-k {tk_ms:.4f} ms, one-layer MLA {mla_ms:.4f} ms",
          file=sys.stderr, flush=True)

    tr = costmodel.path_traffic(w.seq_len, w.q_seq, w.q_pos, w.dtype, L, k, index_dtype=w.index_dtype)
    value = w.nq / (ms_per_step / 1e3)
    kname = indexer_kernel(w)
    if w.kind == "prefill" and w.index_dtype != "f32":
        peak = FP8_MFMA_PEAK_TFLOPS if w.index_dtype == "fp8" else BF16_MFMA_PEAK_TFLOPS
        achieved = tr["indexer"]["flop"] / (idx_ms / 1e3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=peak, unit="TFLOP/s",
                    frac=round(achieved / peak, 4), traffic=None,
                    kernel=kname, per_launch=tr["indexer"]["flop"], per_launch_unit="FLOP")
    elif w.index_dtype != "f32":
        achieved = tr["indexer"]["bytes"] / (idx_ms / 1e3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBPS, 4), traffic=None,
                    kernel=kname, per_launch=tr["indexer"]["bytes"], per_launch_unit="B")
    else:
        achieved = tr["indexer"]["flop"] / (idx_ms / 1e3) / 1e12
        roof = dict(bound="alu", achieved=round(achieved, 3), peak=FP32_VALU_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / FP32_VALU_PEAK_TFLOPS, 4), traffic=None,
                    kernel="idx_decode_f32", per_launch=tr["indexer"]["flop"], per_launch_unit="FLOP")
    path_gbps = tr["path_bytes"] / (ms_per_step / 1e3) / 1e9
    roof["traffic"] = measured_traffic(roof["kernel"], w.name)

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

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
                   "layers_sharing_selection": L, "topk": k, "kind": w.kind,
                   "indexer_dtype": w.index_dtype},
        "roofline": roof,
        "cpu_baseline": cpu,
        "cold": None if cold_ms is None else {
            "reps": args.cold_reps, "ms_per_step": round(cold_ms, 5),
            "value": round(w.nq / (cold_ms / 1e3), 1),
            "note": "each step after a 512 MiB read that evicts L2 and the Infinity Cache"},
        "path": {"algorithmic_bytes": tr["path_bytes"], "algorithmic_flop": tr["path_flop"],
                 "GBps": round(path_gbps, 1), "hbm_frac": round(path_gbps / HBM_PEAK_GBPS, 4),
                 "step_entry": "dsa_mla_decode_fused" if w.kind == "decode" else
                               "dsa_index_score + dsa_topk + mla_sparse_attend",
                 "indexer_ms": round(idx_ms, 5), "topk_ms": round(tk_ms, 5),
                 "mla_one_layer_ms": round(mla_ms, 5)},
    }
    print(json.dumps(rec))


def model_step(args, dev):
    """Decode step over the first `--model-layers` layers of the model's
    schedule: per layer its own query; indexer inputs for the layers that run
    the indexer; a cache for the layers that own one (rotary layers 576-wide,
    the others 512-wide; from layer 39 the rotary-free layers read layer
    35's).  One call of dsa_mla_decode_layers per step."""
    import torch

    from sparse_attention_12_amd import binding as B

    nl, nq, L, k = args.model_layers, args.model_batch, args.model_context, 2048
    plan = B.dsa_ml4_layer_plan(nl)
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    t_gen = time.time()
    bf = torch.bfloat16
    ints = lambda shape: torch.randint(-3, 4, shape, generator=g, device=dev, dtype=torch.int8).to(bf)
    rows = nq * L
    qI, wI, kI, q, kv = [], [], [], [], []
    for l, (runs, rope, src) in enumerate(plan):
        W = 512 + rope
        qI.append(ints((nq, 32, 128)) if runs else None)
        wI.append(torch.randint(1, 5, (nq, 32), generator=g, device=dev).float() if runs else None)
        kI.append(ints((rows, 128)) if runs else None)
        q.append(torch.randn((nq, 64, W), generator=g, device=dev, dtype=bf))
        kv.append(torch.randn((rows, W), generator=g, device=dev, dtype=bf) if src == l else None)
    torch.cuda.synchronize()
    print(f"[bench] model step: {nl} layers ({sum(p[0] for p in plan)} run the indexer), {nq} x {L}, "
          f"inputs drawn on the GPU in {time.time() - t_gen:.1f}s", file=sys.stderr, flush=True)
    seq_len = torch.full((nq,), L, dtype=torch.int32, device=dev)
    batch = B.Batch(torch.arange(nq, dtype=torch.int32, device=dev), seq_len - 1, seq_len,
                    torch.arange(nq, device=dev, dtype=torch.int64) * L, L)
    outs = [torch.empty((nq, 64, 512), device=dev) for _ in plan]
    ws = torch.empty(B.dsa_mla_decode_layers_workspace_size(nq, L, k, plan), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    tau = 1.0 / math.sqrt(192.0)
    step = lambda: B.dsa_mla_decode_layers(batch, plan, qI, wI, kI, k, q, kv, outs, tau, ws=ws)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # algorithmic bytes: indexer keys and queries of the indexer layers, the
    # selected rows, queries and outputs of every layer
    n_sel = min(k, L)
    idx_bytes = sum(nq * (L * 256 + 32 * 128 * 2 + 32 * 4) for r, _, _ in plan if r)
    mla_bytes = sum(nq * (n_sel * (512 + rope) * 2 + 64 * (512 + rope) * 2 + 64 * (512 * 4 + 4))
                    for _, rope, _ in plan)
    gbps = (idx_bytes + mla_bytes) / (ms / 1e3) / 1e9
    rec = {
        "metric": "query-tokens/s for the attention read of every layer of the model's schedule",
        "value": round(nq / (ms / 1e3), 1), "unit": "query-tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic, drawn on the GPU (seeded torch generator): integer indexer inputs, N(0,1) queries and caches",
        "config": {"workload": f"decode_b{nq}_L{L}_bf16_{nl}layer_schedule", "queries": nq, "max_context": L,
                   "layers": nl, "indexer_layers": sum(p[0] for p in plan), "topk": k},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None, "kernel": "whole step",
                     "per_launch": idx_bytes + mla_bytes, "per_launch_unit": "B"},
        "cpu_baseline": None,
    }
    print(json.dumps(rec))


def cpu_baseline(w, budget_s: float):
    """The CPU oracle, as it stands, on the queries of the workload in order
    until the time budget is spent (at least one query).  When one pass over
    the workload takes less than the budget, each query's oracle call is
    repeated so that the timed work lasts about the budget (the inputs of a
    query are widened once, outside the timed calls)."""
    import math as _m

    import oracle

    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        oracle.build(force=False)
    threads = oracle.max_threads()
    done = 0
    el = 0.0
    reps = 2
    qIw = w.widen(w.qI)
    for qi in range(w.nq):
        if el >= budget_s:
            break
        s = int(w.q_seq[qi])
        n = oracle.n_candidates(int(w.q_pos[qi]), int(w.seq_len[s]))
        kI = w.widen(w.seq_rows(w.kI, s))
        qs = [w.widen(x[qi]) for x in w.q]
        kvs = [w.widen(w.seq_rows(x, s)) for x in w.kv]
        r = 0
        while r < reps:
            t0 = time.perf_counter()
            oracle.decode_query(qIw[qi], w.w[qi], kI, qs, kvs, n, w.k, w.tau)
            el += time.perf_counter() - t0
            done += 1
            r += 1
            if qi == 0 and r == 2:   # size the repeats from the first two calls' time
                reps = max(2, _m.ceil(budget_s / (el / 2 * w.nq)))
    return {"value": round(done / el, 3), "unit": "query-tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"{done} oracle calls over the first {min(w.nq, qi + 1)} of {w.nq} queries of the same "
                       f"workload (each run {reps}x; {el:.1f} s of oracle time; fp64 C "
                       f"oracle, OpenMP over positions and heads)")}


if __name__ == "__main__":
    main()
