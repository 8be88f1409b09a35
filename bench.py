"""Benchmark: paged decode attention on one MI355X, effective KV GB/s against HBM peak.

One "step" is one full decode-attention call (kvd_decode_attn_paged: partition kernel, then
the LSE reduce unless every sequence is one workgroup's walk) over a synthetic batch already
resident in HBM.  The default workload is the
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
`other_formats` = the other formats' 32K workloads (BF16, Turbo4, Turbo3 by default), timed the
same way in the same run with fewer steps.  Their warm-up runs at least the W warm-up steps and
at least `--settle-s` seconds of calls: measured from an idle GPU (as after the seconds of
input generation), Turbo3 32K calls took 70 us for the first few steps, 80 us over the next
thirty and 66 us from about the hundredth on, while FP8 32K calls were flat from the first.  `dtype` names the operand precision of the
headline format's matrix products (accumulation is fp32 everywhere).

`--read-probe` instead measures the HBM read ceiling (kvd_read_probe): a plain read stream and
random-chunk reads of the paged layouts' chunk sizes.
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
                    help="c1 c2 c3 c4 c5-t4 c5-t3 c5-t8 s-t4 s-t3 b6-fp8 b6-bf16 b6-t4 b1-fp8 "
                         "b1-t4 m-bf16 m-t4 m-t3 m-t8 mq-fp8 mq8-fp8 mq-t4 mq-t3 mqa-fp8 mqa-bf16 "
                         "mqa-t4 mqa-t8 b64-fp8 "
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
    ap.add_argument("--read-probe", action="store_true",
                    help="instead of decode attention, measure the HBM read ceiling: a plain "
                         "read stream and random-chunk reads of the paged layouts' chunk sizes")
    ap.add_argument("--formats", default="m-bf16,m-t4,m-t3",
                    help="other 32K workloads timed after the headline one, in the same run "
                         "(comma separated; empty = none)")
    ap.add_argument("--settle-s", type=float, default=0.1,
                    help="least warm-up time (s) of each workload in --formats")
    ap.add_argument("--format-steps", type=int, default=30,
                    help="timed steps of each workload in --formats (warm-up: --warmup)")
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


def read_probe(args):
    """HBM read ceiling on this GPU: chunks of a 4 GiB buffer read in order (a plain stream) or
    in a random order (a paged cache's pages sit at random places in the pool), with the chunk
    sizes of the paged layouts (1 KB Turbo4 page chunks ... 4 KB BF16) and 8 waves per CU."""
    import torch

    import quantized_kv_cache_split_amd as kvd
    buf_bytes = 4 << 30
    buf = torch.empty(buf_bytes, dtype=torch.uint8, device="cuda:0")
    buf.fill_(1)
    props = torch.cuda.get_device_properties(0)
    sink = torch.empty(props.multi_processor_count * 32 * 64, dtype=torch.int32, device="cuda:0")
    g = torch.Generator(device="cpu").manual_seed(7)
    cases = [("stream", 65536, 8, 16), ("stream", 65536, 8, 8)]
    for cb in (1024, 2048, 4096):
        for fl in (4, 8, 16):
            cases.append(("random", cb, 8, fl))
    res = []
    for kind, cb, wpc, fl in cases:
        n = buf_bytes // cb
        ids = torch.arange(n, dtype=torch.int32) if kind == "stream" else \
            torch.randperm(n, generator=g).to(torch.int32)
        ids = ids.to("cuda:0")
        for _ in range(3):
            kvd.read_probe(buf, ids, cb, wpc, fl, sink)
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for e in ev:
            e[0].record()
            kvd.read_probe(buf, ids, cb, wpc, fl, sink)
            e[1].record()
        torch.cuda.synchronize()
        t = np.array([e[0].elapsed_time(e[1]) for e in ev]) * 1e-3
        med = float(np.median(t))
        res.append({"order": kind, "chunk_bytes": cb, "waves_per_cu": wpc,
                    "kb_in_flight_per_wave": fl, "bytes_per_launch": buf_bytes,
                    "median_ms": round(med * 1e3, 4), "gbps": round(buf_bytes / med / 1e9, 1),
                    "frac_of_8tbs": round(buf_bytes / med / 1e9 / HBM_PEAK_GBS, 4)})
        print(json.dumps(res[-1]), flush=True)
    best = {k: max(r["gbps"] for r in res if r["order"] == k) for k in ("stream", "random")}
    print(json.dumps({"metric": "HBM read ceiling (kvd_read_probe)", "value": best["random"],
                      "unit": "GB/s", "stream_gbps": best["stream"], "random_chunk_gbps": best["random"],
                      "cases": res}), flush=True)


# Operand precision of each format's matrix products (the accumulators are fp32 throughout).
DTYPES = {
    "bf16": "bf16 K/V/q operands, P as a bf16 hi+lo pair; fp32 accumulate",
    "fp8": "bf16 operands (E4M3 K/V exactly), P as a bf16 hi+lo pair; fp32 accumulate",
    "turbo8": "QK bf16 (E4M3 K exactly); PV fp16 (V levels and P' fp16); fp32 accumulate",
    "turbo4": "fp16 operands (K levels and rotated q as hi+lo; V levels and P' fp16); fp32 accumulate",
    "turbo3": "fp16 operands (K levels and rotated q as hi+lo; V levels and P' fp16); fp32 accumulate",
}


def time_workload(name, steps, warmup, partition_size=None, partitions_per_wave=0, flush=True,
                  settle_s=0.0):
    """Generate workload `name` and time full calls and partition launches on cuda:0, after
    `warmup` untimed steps (continued until `settle_s` seconds of them have run).
    Returns a dict of the measurements (seconds arrays and sizes)."""
    import torch

    import kvgen
    import quantized_kv_cache_split_amd as kvd
    from kvgen.torch_io import dims_kwargs, to_torch

    spec = kvgen.SPECS[name]
    t_gen = time.perf_counter()
    inp = kvgen.make_inputs(spec)
    t_gen = time.perf_counter() - t_gen
    dev = "cuda:0"
    t = to_torch(inp, dev)
    ps = partition_size if partition_size is not None else spec.partition_size
    dims = kvd.Dims(**dims_kwargs(inp, ps, partitions_per_wave))
    out = torch.empty(tuple(inp.q.shape), dtype=torch.float32, device=dev)   # [B, (n_q,) Hq, D]
    nws = kvd.workspace_bytes(dims)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev) if nws else None
    fl = torch.ones(64 << 20, dtype=torch.int64, device=dev) if flush else None
    sink = torch.empty(1, dtype=torch.int64, device=dev)

    def evict():   # read 512 MiB (no dirty lines), outside the timed events
        if fl is not None:
            torch.sum(fl, dim=0, keepdim=True, out=sink)
    call_args = (dims, t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["context_lens"],
                 spec.fmt, t["scales"], t["codebook"], t["sign_pattern"],
                 float(inp.softmax_scale), t["window"], float(inp.softcap), out, ws)

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
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        torch.cuda.synchronize()
        w = time.perf_counter()
        for i in range(steps):
            evict()
            fn(events[i])
        torch.cuda.synchronize()
        w = time.perf_counter() - w
        return np.array([e[0].elapsed_time(e[1]) for e in events]) * 1e-3, w   # seconds

    n_warm, w0 = 0, time.perf_counter()
    while n_warm < warmup or time.perf_counter() - w0 < settle_s:
        evict()
        step()
        n_warm += 1
        if settle_s and n_warm % 16 == 0:
            torch.cuda.synchronize()   # the host stays within 16 steps of the GPU
    torch.cuda.synchronize()
    t_call, wall = timed(step)
    assert np.isfinite(out.cpu().numpy()).all(), "non-finite output"
    t_part, _ = timed(partition_step)
    res = dict(spec=spec, inp=inp, ps=ps, t_call=t_call, t_part=t_part, wall=wall, t_gen=t_gen,
               kv_bytes=inp.kv_bytes(), warmup_steps=n_warm)
    del t, out, ws, fl
    torch.cuda.empty_cache()
    return res


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

    if args.read_probe:
        read_probe(args)
        return

    import torch
    torch.cuda.set_device(0)
    m = time_workload(args.workload, args.steps, args.warmup, args.partition_size,
                      args.partitions_per_wave, flush=not args.no_flush)
    spec, inp, ps, t_call, t_part = m["spec"], m["inp"], m["ps"], m["t_call"], m["t_part"]
    kv_bytes = m["kv_bytes"]
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
        "dtype": DTYPES[spec.fmt],
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
        },
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "decode_tokens_per_s": round(spec.num_seqs * spec.queries_per_seq / mean_call, 1),
        "ms_per_step_p10_p50_p90": [round(float(np.percentile(t_call, q)) * 1e3, 4) for q in (10, 50, 90)],
        "partition_kernel_ms": round(float(t_part.mean()) * 1e3, 4),
        "call_minus_partition_ms": round(float(t_call.mean() - t_part.mean()) * 1e3, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "input_gen_s": round(m["t_gen"], 1),
        "timed_wall_s": round(m["wall"], 3),
    }
    # the other formats' 32K workloads, timed in the same run (fewer steps)
    others = {}
    for name in [w for w in args.formats.split(",") if w and w != args.workload]:
        o = time_workload(name, args.format_steps, args.warmup, flush=not args.no_flush,
                          settle_s=args.settle_s)
        oc, op = float(o["t_call"].mean()), float(o["t_part"].mean())
        others[name] = {"workload": o["spec"].name, "dtype": DTYPES[o["spec"].fmt],
                        "kv_bytes_per_step": o["kv_bytes"], "steps": args.format_steps,
                        "warmup_steps": o["warmup_steps"],
                        "call_ms": round(oc * 1e3, 4), "partition_kernel_ms": round(op * 1e3, 4),
                        "gbps": round(o["kv_bytes"] / oc / 1e9, 2),
                        "frac_of_hbm_peak": round(o["kv_bytes"] / oc / 1e9 / HBM_PEAK_GBS, 4),
                        "partition_kernel_frac": round(o["kv_bytes"] / op / 1e9 / HBM_PEAK_GBS, 4),
                        "decode_tokens_per_s": round(o["spec"].num_seqs * o["spec"].queries_per_seq / oc, 1)}
        del o
    if others:
        res["other_formats"] = others
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
