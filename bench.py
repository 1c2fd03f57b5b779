"""Throughput of the DSA indexer -> top-2,048 -> sparse MLA read on one MI355X.

One step = one pass of the whole read over one batch (index scores, top-k,
then the sparse MLA read of every layer that shares the selection), through
the C ABI, with all inputs resident in HBM: the fused decode entry for decode
batches, the three calls in turn for a prefill chunk.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 0..4] [--no-cpu]
                  [--no-extras] [--index-dtype fp8]
  python bench.py --model-layers 72 [--model-batch 64] [--model-context 32768]
      one decode step of every layer of the model's schedule (indexer layers,
      selection reuse, rotary-free layers, shared cache), inputs drawn on the
      GPU from a seeded generator; prints its own JSON line.

The default workload is the largest one: 4 sequences at 2^20 positions
(bf16).  Timing: W untimed warmup steps; then K steps, each after a read of
a 512 MiB buffer that evicts the L2s and the 256 MB Infinity Cache, each
timed alone with HIP events on the launch stream; `value` and `ms_per_step`
are the median of the K.  A warm figure (K steps back to back) is reported
beside it.  `roofline` describes the dominant kernel (the indexer):
algorithmic bytes (or FLOP) per launch over its average duration in a timed
loop of that kernel alone on the same stream.  `bars` holds, from the same
run, the two workloads that carry targets -- the ragged 4-layer decode batch
reaching 131,072 positions (whole-step HBM fraction, median of 50 flushed
steps) and the 2,048-query prefill chunk (indexer MFMA fraction) -- and the
single fp32 query (median of 50 flushed steps).  `cpu_baseline` times the CPU
oracle on a bounded sample of the headline workload, and single-threaded on
one query of the single-query, 64 x 32,768 and 2^20 shapes.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
FP8_MFMA_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 matrix, published
FP32_VALU_PEAK_TFLOPS = 157.3   # MI355X fp32 vector, published
HEADLINE_CONFIG = 4


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=HEADLINE_CONFIG)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extras", action="store_true", help="skip the other workloads' bar figures")
    ap.add_argument("--index-dtype", choices=["bf16", "fp8"], default=None,
                    help="store the indexer's query and keys in this type (default: the workload's)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU oracle sample budget")
    ap.add_argument("--cold-reps", type=int, default=50,
                    help="flushed steps whose median the bar workloads report")
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


def measured_traffic(kernel: str, workload: str, algorithmic_bytes: int):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    counter summary (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy of
    known size), or None if absent, taken on a different kernel source or on
    other inputs (different algorithmic bytes)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(f"{kernel}/{workload}")
    if not rec or rec.get("source_sha256") != kernel_source_digest(kernel):
        return None
    if rec.get("algorithmic_bytes") != algorithmic_bytes:
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


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class Runner:
    """One workload resident on the GPU, its step and its stages."""

    def __init__(self, w, dev):
        import torch

        from sparse_attention_12_amd import binding as B

        self.w, self.B, self.dev = w, B, dev
        self.t = t = w.to_torch(dev)
        self.batch = B.Batch(t["q_seq"], t["q_pos"], t["seq_len"], t["seq_row0"], w.max_len)
        k, L = w.k, w.n_layers
        self.scores = torch.empty((w.nq, w.max_len), dtype=torch.float32, device=dev)
        self.idx = torch.empty((w.nq, k), dtype=torch.int32, device=dev)
        self.count = torch.empty((w.nq,), dtype=torch.int32, device=dev)
        self.outs = [torch.empty((w.nq, 64, 512), dtype=torch.float32, device=dev) for _ in range(L)]
        self.lses = [torch.empty((w.nq, 64), dtype=torch.float32, device=dev) for _ in range(L)]
        n = B.dsa_topk_workspace_size(w.nq, w.max_len, k)
        self.tk_ws = torch.empty(n, dtype=torch.uint8, device=dev) if n else None
        self.mla_ws = torch.empty(max(B.mla_sparse_attend_workspace_size(w.nq, k, 1), 256), dtype=torch.uint8,
                                  device=dev)
        self.fused_ws = torch.empty(max(B.dsa_mla_decode_fused_workspace_size(w.nq, w.max_len, k, L), 256),
                                    dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream()

    def step(self):
        w, t, B = self.w, self.t, self.B
        if w.kind == "decode":
            # the decode read as one call: indexer, top-k, every layer's MLA
            B.dsa_mla_decode_fused(self.batch, t["qI"], t["w"], t["kI"], w.k, t["q"], t["kv"], self.outs, w.tau,
                                   self.lses, self.idx, self.fused_ws)
        else:
            self.indexer()
            self.topk()
            for l in range(w.n_layers):
                B.mla_sparse_attend(self.batch, t["q"][l], t["kv"][l], self.idx, w.k, w.tau, self.outs[l],
                                    self.lses[l], self.mla_ws)

    def indexer(self):
        t = self.t
        self.B.dsa_index_score(self.batch, t["qI"], t["w"], t["kI"], self.scores)

    def topk(self):
        self.B.dsa_topk(self.batch, self.scores, self.w.k, self.idx, self.count, self.tk_ws)

    def mla(self):
        w, t = self.w, self.t
        self.B.mla_sparse_attend(self.batch, t["q"][0], t["kv"][0], self.idx, w.k, w.tau, self.outs[0],
                                 self.lses[0], self.mla_ws)

    def timed(self, fn, n):
        """Average ms per call of fn over n calls back to back, HIP events on
        the launch stream."""
        import torch
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(self.stream)
        for _ in range(n):
            fn()
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    def stage(self, fn, n, flush):
        """ms of one stage (fn launches its kernels and nothing else), timed
        like the step: the median of n calls, each alone after the
        cache-evicting read (so the 190 MB of keys of the ragged batch are not
        served from the 256 MB Infinity Cache by the previous call), HIP
        events on the launch stream around the call; while the flush runs the
        host has already queued the call, so no per-call host cost is
        timed."""
        fn()
        return statistics.median(self.flushed(fn, n, flush))

    def flushed(self, fn, n, flush):
        """ms of each of n calls of fn, each after `flush` (outside its events)."""
        import torch
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        torch.cuda.synchronize()
        for a, b in ev:
            flush()
            a.record(self.stream)
            fn()
            b.record(self.stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    def traffic(self):
        from sparse_attention_12_amd import costmodel
        w = self.w
        return costmodel.path_traffic(w.seq_len, w.q_seq, w.q_pos, w.dtype, w.n_layers, w.k,
                                      index_dtype=w.index_dtype)

    def indexer_roofline(self, idx_ms):
        w = self.w
        tr = self.traffic()
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
        roof["traffic"] = measured_traffic(roof["kernel"], w.name, tr["indexer"]["bytes"])
        return roof

    def release(self):
        import torch
        del self.t, self.scores, self.outs, self.lses, self.fused_ws, self.mla_ws, self.tk_ws
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(every workload runs on a single MI355X); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from sparse_attention_12_amd import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.model_layers:
        model_step(args, dev)
        return
    # before each flushed step: a read of 512 MiB (clean lines, so no
    # write-back competes with the step) evicts the 4 MB L2s and the 256 MB
    # Infinity Cache
    flush_buf = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    flush = lambda: flush_buf.sum()

    t_gen = time.time()
    w = workloads.config(args.config, args.index_dtype)
    print(f"[bench] workload {w.name}: nq={w.nq} layers={w.n_layers} max_len={w.max_len} "
          f"(generated in {time.time() - t_gen:.1f}s)", file=sys.stderr, flush=True)
    R = Runner(w, dev)

    for _ in range(args.warmup):
        R.step()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    per_step = R.flushed(R.step, args.steps, flush)
    wall = time.perf_counter() - wall0
    ms_per_step = statistics.median(per_step)
    warm_ms = R.timed(R.step, args.steps)

    # per-stage timings of the same kernels, same launch configurations
    R.indexer()
    idx_ms = R.stage(R.indexer, args.steps, flush)
    tk_ms = R.stage(R.topk, args.steps, flush)
    mla_ms = R.stage(R.mla, args.steps, flush)
    print(f"[bench] {args.steps} flushed steps: median {ms_per_step:.4f} ms (min {min(per_step):.4f}, "
          f"max {max(per_step):.4f}; region {wall:.2f} s); warm {warm_ms:.4f} ms; indexer {idx_ms:.4f} ms, "
          f"top-k {tk_ms:.4f} ms, one-layer MLA {mla_ms:.4f} ms", file=sys.stderr, flush=True)

    tr = R.traffic()
    value = w.nq / (ms_per_step / 1e3)
    roof = R.indexer_roofline(idx_ms)
    path_gbps = tr["path_bytes"] / (ms_per_step / 1e3) / 1e9

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    headline = w
    R.release()
    del R
    bars = None if args.no_extras else extras(args, dev, flush)
    del flush_buf

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(headline, args.cpu_seconds)

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
                   "layers_sharing_selection": w.n_layers, "topk": w.k, "kind": w.kind,
                   "indexer_dtype": w.index_dtype,
                   "timing": "median of the timed steps, each after a 512 MiB read that evicts L2 and the "
                             "Infinity Cache"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "warm": {"ms_per_step": round(warm_ms, 5), "value": round(w.nq / (warm_ms / 1e3), 1),
                 "note": "the same steps back to back"},
        "path": {"algorithmic_bytes": tr["path_bytes"], "algorithmic_flop": tr["path_flop"],
                 "GBps": round(path_gbps, 1), "hbm_frac": round(path_gbps / HBM_PEAK_GBPS, 4),
                 "step_entry": "dsa_mla_decode_fused" if w.kind == "decode" else
                               "dsa_index_score + dsa_topk + mla_sparse_attend",
                 "step_ms_min": round(min(per_step), 5), "step_ms_max": round(max(per_step), 5),
                 "indexer_ms": round(idx_ms, 5), "topk_ms": round(tk_ms, 5),
                 "mla_one_layer_ms": round(mla_ms, 5),
                 "stage_timing": "each stage through its own entry point (dsa_index_score, dsa_topk without the "
                                 "indexer's histogram, mla_sparse_attend), median of K calls, each after the same "
                                 "cache-evicting read as the steps"},
        "bars": bars,
    }
    print(json.dumps(rec))


def extras(args, dev, flush):
    """The workloads that carry targets, timed in the same run: the ragged
    4-layer decode batch (whole step against HBM peak, median of flushed
    steps), the prefill chunk (its indexer against the matrix peak) and the
    single fp32 query (median of flushed steps)."""
    from sparse_attention_12_amd import workloads
    out = {}
    reps = max(args.cold_reps, 1)
    # ragged decode batch: whole-step HBM fraction (target 0.60)
    w = workloads.config(2, args.index_dtype)
    R = Runner(w, dev)
    for _ in range(args.warmup):
        R.step()
    cold = R.flushed(R.step, reps, flush)
    warm = R.timed(R.step, reps)
    R.indexer()
    idx_ms = R.stage(R.indexer, args.steps, flush)
    tk_ms = R.stage(R.topk, args.steps, flush)
    tr = R.traffic()
    med = statistics.median(cold)
    gbps = tr["path_bytes"] / (med / 1e3) / 1e9
    out["ragged_decode_128K"] = {
        "workload": w.name, "reps": reps, "ms_per_step": round(med, 5), "value": round(w.nq / (med / 1e3), 1),
        "unit": "query-tokens/s", "warm_ms_per_step": round(warm, 5), "path_bytes": tr["path_bytes"],
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4), "warm_hbm_frac": round(tr["path_bytes"] / (warm / 1e3) / 1e9
                                                                          / HBM_PEAK_GBPS, 4),
        "target_hbm_frac": 0.60, "indexer_ms": round(idx_ms, 5), "topk_ms": round(tk_ms, 5),
        "indexer_roofline": R.indexer_roofline(idx_ms)}
    print(f"[bench] {w.name}: median of {reps} flushed steps {med:.4f} ms ({gbps / HBM_PEAK_GBPS:.3f} of HBM "
          f"peak), warm {warm:.4f} ms", file=sys.stderr, flush=True)
    R.release()
    del R, w
    # prefill chunk: indexer against the matrix peak (target 0.40 in bf16)
    w = workloads.config(3, args.index_dtype)
    R = Runner(w, dev)
    for _ in range(max(2, args.warmup // 2)):
        R.step()
    R.indexer()
    idx_ms = R.stage(R.indexer, args.steps, flush)
    cold = R.flushed(R.step, max(10, reps // 5), flush)
    med = statistics.median(cold)
    roof = R.indexer_roofline(idx_ms)
    out["causal_prefill_2048q"] = {
        "workload": w.name, "reps": len(cold), "ms_per_step": round(med, 5),
        "value": round(w.nq / (med / 1e3), 1), "unit": "query-tokens/s", "indexer_ms": round(idx_ms, 5),
        "indexer_mfma_frac": roof["frac"], "target_mfma_frac": 0.40, "indexer_roofline": roof}
    print(f"[bench] {w.name}: indexer {idx_ms:.4f} ms ({roof['frac']:.3f} of the matrix peak), step "
          f"{med:.4f} ms", file=sys.stderr, flush=True)
    R.release()
    del R, w
    # single fp32 query
    w = workloads.config(0)
    R = Runner(w, dev)
    for _ in range(args.warmup):
        R.step()
    cold = R.flushed(R.step, reps, flush)
    med = statistics.median(cold)
    out["decode_b1_L4096_f32"] = {"workload": w.name, "reps": reps, "ms_per_step": round(med, 5),
                                  "value": round(w.nq / (med / 1e3), 1), "unit": "query-tokens/s",
                                  "warm_ms_per_step": round(R.timed(R.step, reps), 5)}
    print(f"[bench] {w.name}: median of {reps} flushed steps {med:.4f} ms", file=sys.stderr, flush=True)
    R.release()
    return out


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
    query are widened once, outside the timed calls).  Then the oracle on one
    thread, one query of each decode shape (single query at 4,096, one
    sequence of 32,768 and of 2^20 positions)."""
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
    nq_done = min(w.nq, qi + 1)
    del qIw, kI, qs, kvs
    single = single_thread_oracle()
    oracle.set_threads(threads)
    return {"value": round(done / el, 3), "unit": "query-tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": (f"{done} oracle calls over the first {nq_done} of {w.nq} queries of the same "
                       f"workload (each run {reps}x; {el:.1f} s of oracle time; fp64 C "
                       f"oracle, OpenMP over positions and heads)"),
            "single_thread": single}


def single_thread_oracle():
    """Seconds of one oracle call on one thread, one query per decode shape
    (inputs drawn like the workloads'; the oracle's time does not depend on
    the values)."""
    import oracle
    from sparse_attention_12_amd import workloads as wl
    oracle.set_threads(1)
    out = {}
    for name, L, dt in (("decode_b1_L4096_f32", 4096, "f32"), ("decode_b64_L32768_bf16", 32768, "bf16"),
                        ("decode_b4_L1048576_bf16", 1 << 20, "bf16")):
        w = wl.make_decode([L], dt, 1, seed=77, split_kv=(dt == "f32"))
        args = (w.widen(w.qI)[0], w.w[0], w.widen(w.kI), [w.widen(w.q[0])[0]], [w.widen(w.kv[0])], L, w.k, w.tau)
        t0 = time.perf_counter()
        oracle.decode_query(*args)
        sec = time.perf_counter() - t0
        out[name] = {"seconds_per_query": round(sec, 3), "query_tokens_per_s": round(1.0 / sec, 4),
                     "sample": f"one query at {L:,} positions on one thread"}
        del w, args
    return out


if __name__ == "__main__":
    main()
