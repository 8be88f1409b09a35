"""Benchmark: paged decode attention on one MI355X, effective KV GB/s against HBM peak.

One "step" is one full decode-attention call (kvd_decode_attn_paged: partition kernel + LSE
reduce) over a synthetic batch already resident in HBM.  The default workload is the
FP8-E4M3 cache at 32K context (16 sequences, 64 query / 8 KV heads, head_dim 128, 512-token
partitions).  The K timed steps are timed with one HIP event pair each, on the stream the
kernels run on, around the whole call.  No event sits between the two launches: a marker
there delays the second launch by 2-7 us, which a caller never pays.  The partition kernel's
own duration (for `roofline`) comes from a second event-timed loop of K steps that brackets
only the partition launch; the reduce follows outside the events.  Between steps (outside
the events) a 512 MiB buffer is read.  That evicts the 256 MB Infinity Cache without leaving
dirty lines behind; a rewrite would leave write-backs that land inside the next timed call.

Prints ONE JSON line.  `value` = algorithmic KV bytes per call / mean call time.
`roofline` = the partition kernel's algorithmic bytes / its mean duration against 8 TB/s.
`cpu_baseline` = the fp64 oracle timed on this host's cores over a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention: effective KV GB/s (% of HBM peak) at 32K context"
HBM_PEAK_GBS = 8000.0
KV_NAMES = {"bf16": "bf16", "fp8": "fp8_e4m3", "turbo4": "turbo4 (K4/V4 rotated codebook)",
            "turbo3": "turbo3 (K3/V4 rotated codebook)",
            "turbo8": "turbo8 (FP8 K + V4 rotated codebook)"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # 50: the first calls after start-up run slow (FP8 32K: ~260 us mean over the first 50
    # calls, 208-209 us from then on); the default warm-up reaches the steady state
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="c4",
                    help="c1 c2 c3 c4 c5-t4 c5-t3 c5-t8 m-bf16 m-t4 m-t3 m-t8 mq-fp8 mq-t4 mq-t3 mqa-fp8 mqa-t4 "
                         "(see kvgen.SPECS)")
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--partitions-per-wave", type=int, default=0,
                    help="launch tuning of the partition kernel (0 = the library's choice)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, time a plain device-to-device copy of this "
                         "many MiB (calibrates HBM byte counters against a known size)")
    ap.add_argument("--append", type=int, default=0, metavar="T",
                    help="instead of decode attention, time the KV append (quantize-on-write) "
                         "of T new tokens per sequence into the workload's cache")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "hbm_traffic.json"),
                    help="JSON with HBM bytes per partition-kernel launch measured by rocprofv3 "
                         "(used only while the kernel sources are unchanged since)")
    return ap.parse_args()


def cpu_baseline(inp, seconds):
    """Time the oracle (unchanged) on a bounded sample of (sequence, KV head) pairs."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    s = inp.spec
    spans = inp.spans()
    per_pair = kvgen_bytes_per_token_head(s)
    done_bytes = 0
    pairs = 0
    t0 = time.perf_counter()
    order = [(b, hk) for b in range(s.num_seqs) for hk in range(s.num_kv_heads)]
    fn = oracle.decode_attention if s.queries_per_seq == 1 else oracle.multi_query_attention
    for b, hk in order:
        fn(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.context_lens, s.fmt, inp.scales,
           inp.codebook, inp.sign, inp.softmax_scale, inp.window, inp.softcap, s.num_kv_heads,
           s.head_dim, seqs=[b], kv_heads=[hk])
        done_bytes += int(spans[b]) * per_pair
        pairs += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{pairs} of {len(order)} (sequence, KV head) pairs, {done_bytes / 1e6:.1f} MB "
                      f"of KV in {dt:.1f} s (NumPy fp64 oracle; host cores {os.cpu_count()}, "
                      f"{len(os.sched_getaffinity(0))} in this process's affinity, BLAS threads "
                      f"{threads})"}


KERNEL_SOURCES = [os.path.join(ROOT, "quantized_kv_cache_split_amd", "csrc", f)
                  for f in ("kvd_kernels.hip", "kvd_api.cpp", "kvd_internal.h")]


def kernel_source_hash() -> str:
    """SHA-256 over the HIP kernel and launch sources (ties counter readings to a kernel)."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(path, workload):
    """HBM bytes per partition-kernel launch from the counter record, or None when the record
    is missing, covers another workload or predates the current kernel sources."""
    if not path or not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    entry = rec.get("workloads", {}).get(workload)
    return None if entry is None else entry.get("hbm_bytes_per_launch")


def kvgen_bytes_per_token_head(s):
    import kvgen
    return kvgen.kv_bytes_per_token_head(s.fmt, s.head_dim)


def copy_probe(mib, steps):
    """A plain copy kernel of known size: reads and writes mib MiB per launch."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    dt = e0.elapsed_time(e1) * 1e-3 / steps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": steps + 3,
                      "copy_gbps_read_plus_write": round(2 * n / dt / 1e9, 2)}), flush=True)


def append_bench(args):
    """KV append: T new fp32 tokens per sequence (K and V, all KV heads) encoded into the
    workload's paged cache.  Algorithmic bytes per (token, KV head): the fp32 K and V read
    (8 D) plus the cache bytes written (K and V codes, and for the codebook formats 8 bytes of
    norms).  The new tokens overwrite the last T of each sequence (their pages are mapped)."""
    import torch

    import kvgen
    import quantized_kv_cache_split_amd as kvd
    from kvgen.torch_io import dims_kwargs, to_torch

    spec = kvgen.SPECS[args.workload]
    inp = kvgen.make_inputs(spec)
    t = to_torch(inp, "cuda:0")
    T = args.append
    B, Hkv, D = spec.num_seqs, spec.num_kv_heads, spec.head_dim
    dims = kvd.Dims(**dims_kwargs(inp, 0))
    g = torch.Generator(device="cuda:0").manual_seed(1)
    kn = torch.randn((B, T, Hkv, D), generator=g, device="cuda:0", dtype=torch.float32)
    vn = torch.randn((B, T, Hkv, D), generator=g, device="cuda:0", dtype=torch.float32)
    pos = (t["context_lens"] - T).clamp(min=0).to(torch.int32)
    call = (dims, spec.fmt, kn, vn, t["block_table"], pos, T, t["k_cache"], t["v_cache"],
            t["scales"], t["codebook"], t["sign_pattern"])
    flush = torch.ones(64 << 20, dtype=torch.int64, device="cuda:0")
    sink = torch.empty(1, dtype=torch.int64, device="cuda:0")
    for _ in range(args.warmup):
        kvd.append_kv(*call)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in ev:
        torch.sum(flush, dim=0, keepdim=True, out=sink)
        e[0].record()
        kvd.append_kv(*call)
        e[1].record()
    torch.cuda.synchronize()
    ts = np.array([e[0].elapsed_time(e[1]) for e in ev]) * 1e-3
    per = 8 * D + kvgen.kv_bytes_per_token_head(spec.fmt, D)
    nbytes = B * T * Hkv * per
    mean = float(ts.mean())
    res = {"metric": "kv append (quantize-on-write): GB/s of fp32 input read + cache written",
           "value": round(nbytes / mean / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(mean * 1e3, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f32->" + spec.fmt, "data": "synthetic",
           "config": {"workload": f"{args.workload}: {spec.name}", "new_tokens_per_seq": T,
                      "num_seqs": B, "num_kv_heads": Hkv, "head_dim": D,
                      "bytes_per_token_head": per, "bytes_per_call": nbytes},
           "tokens_per_s": round(B * T / mean, 1),
           "ms_per_step_p10_p50_p90": [round(float(np.percentile(ts, q)) * 1e3, 4) for q in (10, 50, 90)],
           "roofline": {"bound": "hbm", "achieved": round(nbytes / mean / 1e9, 2),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(nbytes / mean / 1e9 / HBM_PEAK_GBS, 4), "traffic": None}}
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only; multi-GPU runs are not supported "
              "(the per-(sequence, KV head, partition) work would shard by sequence or KV head "
              "with no exchange, see DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe(args.copy_probe, args.steps)
        return
    if args.append:
        append_bench(args)
        return

    import torch

    import kvgen
    import quantized_kv_cache_split_amd as kvd
    from kvgen.torch_io import dims_kwargs, to_torch

    spec = kvgen.SPECS[args.workload]
    t_gen = time.perf_counter()
    inp = kvgen.make_inputs(spec)
    t_gen = time.perf_counter() - t_gen
    dev = "cuda:0"
    torch.cuda.set_device(0)
    t = to_torch(inp, dev)
    ps = args.partition_size if args.partition_size is not None else spec.partition_size
    dims = kvd.Dims(**dims_kwargs(inp, ps, args.partitions_per_wave))
    out = torch.empty(tuple(inp.q.shape), dtype=torch.float32, device=dev)   # [B, (n_q,) Hq, D]
    nws = kvd.workspace_bytes(dims)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev) if nws else None
    flush = None if args.no_flush else torch.ones(64 << 20, dtype=torch.int64, device=dev)
    sink = torch.empty(1, dtype=torch.int64, device=dev)

    def evict():   # read 512 MiB (no dirty lines), outside the timed events
        if flush is not None:
            torch.sum(flush, dim=0, keepdim=True, out=sink)
    call_args = (dims, t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["context_lens"],
                 spec.fmt, t["scales"], t["codebook"], t["sign_pattern"],
                 float(inp.softmax_scale), t["window"], float(inp.softcap), out, ws)
    kv_bytes = inp.kv_bytes()

    def step(ev=None):   # one full call, the entry point a caller uses
        if ev is not None:
            ev[0].record()
        kvd.decode_attn_paged(*call_args)
        if ev is not None:
            ev[1].record()

    def partition_step(ev):   # the partition kernel alone inside the events
        ev[0].record()
        kvd.decode_partitions(*call_args)
        ev[1].record()
        kvd.reduce_partitions(*call_args)

    def timed(fn):
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        w = time.perf_counter()
        for i in range(args.steps):
            evict()
            fn(events[i])
        torch.cuda.synchronize()
        w = time.perf_counter() - w
        return np.array([e[0].elapsed_time(e[1]) for e in events]) * 1e-3, w   # seconds

    for _ in range(args.warmup):
        evict()
        step()
    torch.cuda.synchronize()
    t_call, wall = timed(step)
    assert np.isfinite(out.cpu().numpy()).all(), "non-finite output"
    t_part, _ = timed(partition_step)

    mean_call = float(t_call.mean())
    value = kv_bytes / mean_call / 1e9
    achieved = kv_bytes / float(t_part.mean()) / 1e9
    traffic = measured_traffic(args.traffic, args.workload)
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mean_call * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: {spec.name}",
            "num_seqs": spec.num_seqs, "num_q_heads": spec.num_q_heads,
            "num_kv_heads": spec.num_kv_heads, "head_dim": spec.head_dim,
            "context": spec.context if spec.context else list(spec.ctx_range),
            "window": spec.window, "softcap": spec.softcap,
            "kv_format": KV_NAMES[spec.fmt], "block_size": 16,
            "partition_size": ps if ps else 512, "kv_bytes_per_step": kv_bytes,
            "queries_per_seq": spec.queries_per_seq,
            "mfma_operands": "bf16 for BF16/FP8 K and V, fp16 for codebook K and V (Turbo8: "
                             "bf16 QK, fp16 PV); fp32 accumulate",
        },
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "decode_tokens_per_s": round(spec.num_seqs * spec.queries_per_seq / mean_call, 1),
        "ms_per_step_p10_p50_p90": [round(float(np.percentile(t_call, q)) * 1e3, 4) for q in (10, 50, 90)],
        "partition_kernel_ms": round(float(t_part.mean()) * 1e3, 4),
        "call_minus_partition_ms": round(float(t_call.mean() - t_part.mean()) * 1e3, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "input_gen_s": round(t_gen, 1),
        "timed_wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
