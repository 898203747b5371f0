#!/usr/bin/env python3
"""Benchmark of the exact tiled attention path on one MI355X.

One step = one full pass of the hot path over one batch of synthetic input resident in HBM:
fa_forward (O, LSE) followed by the backward (preprocess delta, dK/dV, dQ -- the three
stages fa_backward runs, launched individually here so each kernel can be timed with HIP
events on the stream it runs on).

Workload (default): B=4, H=32, N=4096, d=128, causal, bf16, Q, K, V, dO ~ N(0,1) from seed
1004, scale = 1/sqrt(d). Counted FLOPs: forward F = 4*B*H*N^2*d, halved for causal
("Triton 05: Flash Attention", section on why throughput stops at a fraction of peak: the
two matmuls of the forward); backward 2.5 F; a step counts 3.5 F.

Prints ONE JSON line on stdout. Progress goes to stderr.

Options beyond the contract (--gpus, --steps, --warmup):
  --sweep                    also time, as 11 single runs each, every workload (forward,
                             fa_backward, split-KV forward) and the strided, packed, other
                             head-dim and decode (one query against a key cache) problems
  --copy-calibration-mib M   after the timed region, one plain device copy of M MiB: the
                             kernel of known traffic that scales the HBM byte counters
  --ingest-counters F W      no GPU work: turn the counter files of a FETCH_SIZE and a
                             WRITE_SIZE rocprofv3 run into profiles/traffic.json
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16/fp16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "fwd": ["fa_fwd.hip", "fa_common.hpp", "fa_kernels.hpp"],
    "bwd_preprocess": ["fa_bwd.hip", "fa_common.hpp", "fa_kernels.hpp"],
    "bwd_dkv": ["fa_bwd_dkv.hip", "fa_common.hpp", "fa_kernels.hpp"],
    "bwd_dq": ["fa_bwd.hip", "fa_common.hpp", "fa_kernels.hpp"],
}
# Kernel-name fragments of each timed kernel in a profiler's per-dispatch records.
KERNEL_SYMBOLS = {"fwd": "fwd_kernel", "bwd_preprocess": "bwd_preprocess_kernel", "bwd_dkv": "bwd_dkv_kernel",
                  "bwd_dq": "bwd_dq_kernel"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "exact_attention_27_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter runs, or None when absent or stale."""
    try:
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        return None
    rec = table.get(kernel)
    if not rec or rec.get("workload") != workload or rec.get("source_sha") != source_sha(kernel):
        return None
    return rec.get("bytes_per_launch")


def ingest_counters(fetch_csv: str, write_csv: str, copy_mib: int, workload: str) -> dict:
    """HBM bytes per launch of every timed kernel from two rocprofv3 --pmc runs of this script
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled by what the same counter read
    for the plain device copy of copy_mib MiB that --copy-calibration-mib runs last. Writes
    profiles/traffic.json with the current kernel source hashes and returns the table."""
    import csv
    import collections

    def per_kernel(path, counter):
        per = collections.defaultdict(list)
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    per[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return per

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    copies = [k for k in fetch if "copy" in k.lower()]
    if len(copies) != 1 or copies[0] not in write:
        raise SystemExit(f"expected one copy kernel in both counter files, found {copies}")
    copy_bytes = copy_mib * (1 << 20)
    f_factor = copy_bytes / (fetch[copies[0]][-1] * 1024)
    w_factor = copy_bytes / (write[copies[0]][-1] * 1024)

    def find(per, frag):
        hits = [k for k in per if frag in k]
        if len(hits) != 1:
            raise SystemExit(f"expected one kernel matching {frag}, found {len(hits)}")
        return per[hits[0]]

    out = {}
    for name, frag in KERNEL_SYMBOLS.items():
        fv, wv = find(fetch, frag), find(write, frag)
        fb = sum(fv) / len(fv) * 1024 * f_factor
        wb = sum(wv) / len(wv) * 1024 * w_factor
        out[name] = {"workload": workload, "source_sha": source_sha(name), "bytes_per_launch": round(fb + wb),
                     "fetch_bytes": round(fb), "write_bytes": round(wb), "fetch_kib_raw": sum(fv) / len(fv),
                     "write_kib_raw": sum(wv) / len(wv), "dispatches": len(fv)}
    out["_calibration"] = {"copy_mib": copy_mib, "copy_kernel": copies[0], "fetch_factor": f_factor,
                           "write_factor": w_factor}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    return out


def cpu_baseline(bits, w, heads):
    """The fp64 oracle as it stands, on a bounded sample of heads of the same workload."""
    import numpy as np
    import fa_inputs as FI
    from oracle import attention as ORACLE
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the affinity count
        threads = len(os.sched_getaffinity(0))
    causal = w.causal[0]
    t0 = time.perf_counter()
    for b, h in heads:
        q, k, v, do = (FI.bits_to_f64(bits[n][b, h], w.dtype) for n in FI.TENSOR_ORDER)
        ORACLE.backward(q, k, v, do, w.scale(), causal)
    dt = time.perf_counter() - t0
    per_head = 3.5 * 4.0 * w.N * w.N * w.d * (0.5 if causal else 1.0)
    return {
        "value": len(heads) * per_head / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{len(heads)} of {w.B * w.H} heads (every {w.B * w.H // len(heads)}th (b, h)) of the "
                   f"same workload: fp64 forward+backward materialising S and P, {dt:.2f} s wall; "
                   f"counted 3.5*F per head as for the GPU"),
        "seconds": dt,
        "host": _host_info(),
    }


def _host_info():
    """The host the oracle ran on: CPU model, CPUs this process may use, memory."""
    info = {"affinity_cpus": len(os.sched_getaffinity(0))}
    try:
        with open("/proc/cpuinfo") as f:
            info["cpu_model"] = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
        with open("/proc/meminfo") as f:
            kib = next((int(ln.split()[1]) for ln in f if ln.startswith("MemTotal:")), None)
        info["mem_gib"] = round(kib / 2**20, 1) if kib else None
    except OSError:  # no /proc: report what is known
        pass
    return info


def sweep_configs(fa, FI, torch, np, dev, log):
    """Every workload (and mask setting): forward alone, one fa_backward call, and the split-KV
    forward with 2 and 4 key ranges, each timed as 11 runs bracketed by HIP events on one
    stream, the first discarded; counted FLOPs as above."""
    out = []
    stream = torch.cuda.current_stream(dev)
    for key, w in FI.WORKLOADS.items():
        bits = FI.draw_workload(w)
        tdt = torch.bfloat16 if w.dtype == FI.BF16 else torch.float16
        q, k, v, do = (torch.from_numpy(bits[n].view(np.int16)).to(dev).view(tdt) for n in FI.TENSOR_ORDER)
        o = torch.empty_like(q)
        lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device=dev)
        delta = torch.empty_like(lse)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        for causal in w.causal:
            F = 4.0 * w.B * w.H * w.N * w.N * w.d * (0.5 if causal else 1.0)
            res = {}
            for name, fn in (("fwd", lambda: fa.fa_forward(q, k, v, o, lse, causal, w.scale(), stream)),
                             ("bwd", lambda: fa.fa_backward(q, k, v, o, do, lse, dq, dk, dv, delta, causal,
                                                            w.scale(), stream))):
                ts = []
                for _ in range(11):
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    fn()
                    b.record(stream)
                    torch.cuda.synchronize()
                    ts.append(a.elapsed_time(b))
                ts = np.array(ts[1:]) * 1e3  # us
                res[name] = {"mean_us": float(ts.mean()), "std_us": float(ts.std()), "median_us": float(np.median(ts))}
            # the split-KV forward (fa_forward_splitkv) with 2 and 4 key ranges per Q tile
            for sp in (2, 4):
                nb = fa.fa_forward_splitkv_workspace_bytes(w.B, w.H, w.N, w.d, sp)
                if nb > (1 << 30):
                    continue
                ws = torch.empty(nb // 4, dtype=torch.float32, device=dev)
                ts = []
                for _ in range(11):
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    fa.fa_forward_splitkv(q, k, v, o, lse, causal, w.scale(), sp, ws, stream)
                    b.record(stream)
                    torch.cuda.synchronize()
                    ts.append(a.elapsed_time(b))
                ts = np.array(ts[1:]) * 1e3
                res[f"fwd_split{sp}"] = {"mean_us": float(ts.mean()), "std_us": float(ts.std()),
                                         "median_us": float(np.median(ts))}
                del ws
            fwd_tf = F / (res["fwd"]["mean_us"] * 1e-6) / 1e12
            tot_tf = 3.5 * F / ((res["fwd"]["mean_us"] + res["bwd"]["mean_us"]) * 1e-6) / 1e12
            rec = {"workload": key, "label": w.label, "causal": causal, **res,
                   "fwd_tflops": fwd_tf, "fwd_bwd_tflops": tot_tf}
            log(f"  {key:13s} causal={int(causal)}  fwd {res['fwd']['mean_us']:9.1f} us (sd {res['fwd']['std_us']:.1f})"
                f"  bwd {res['bwd']['mean_us']:9.1f} us (sd {res['bwd']['std_us']:.1f})  fwd {fwd_tf:7.1f} TFLOP/s"
                f"  fwd+bwd {tot_tf:7.1f} TFLOP/s  split-KV fwd: "
                + ", ".join(f"{k[9:]} ranges {v['mean_us']:.1f} us" for k, v in res.items() if k.startswith("fwd_split")))
            out.append(rec)
        del q, k, v, do, o, lse, delta, dq, dk, dv
        torch.cuda.empty_cache()
    return out


def _time11(fn, torch, np, stream):
    """11 runs of fn bracketed by HIP events on `stream`, the first discarded (microseconds)."""
    ts = []
    for _ in range(11):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    ts = np.array(ts[1:]) * 1e3
    return {"mean_us": float(ts.mean()), "std_us": float(ts.std()), "median_us": float(np.median(ts))}


def sweep_extras(fa, FI, torch, np, dev, log):
    """The strided, variable-length and other-head-dim entry points on LLM-layer-sized work:
    forward and backward, each timed as 11 runs (first discarded); FLOPs counted on the work
    the problem defines (for a packed batch, each sequence's own causal triangle)."""
    out = []
    stream = torch.cuda.current_stream(dev)
    H, N, d = 32, 4096, 128

    def rec(label, F, fwd, bwd):
        r = {"extra": label, "fwd": fwd, "bwd": bwd, "counted_flop": F,
             "fwd_tflops": F / (fwd["mean_us"] * 1e-6) / 1e12,
             "fwd_bwd_tflops": 3.5 * F / ((fwd["mean_us"] + bwd["mean_us"]) * 1e-6) / 1e12}
        log(f"  {label:58s} fwd {fwd['mean_us']:9.1f} us  bwd {bwd['mean_us']:9.1f} us  "
            f"fwd {r['fwd_tflops']:7.1f}  fwd+bwd {r['fwd_bwd_tflops']:7.1f} TFLOP/s")
        out.append(r)

    def tensors(shape, dtype, seed):
        bits = FI.draw_bits(shape, dtype, seed)
        tdt = torch.bfloat16 if dtype == FI.BF16 else torch.float16
        return [torch.from_numpy(bits[n].view(np.int16)).to(dev).view(tdt) for n in FI.TENSOR_ORDER]

    # (B, N, H, d) storage at the headline shape, through fa_forward_ex / fa_backward_ex
    q, k, v, do = (t.transpose(1, 2).contiguous() for t in tensors((4, H, N, d), FI.BF16, 1004))
    o = torch.empty_like(q)
    lse = torch.empty(4, H, N, dtype=torch.float32, device=dev)
    delta, dq, dk, dv = torch.empty_like(lse), torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    F = 4.0 * 4 * H * N * N * d * 0.5
    rec("B=4 H=32 N=4096 d=128 causal bf16, (B,N,H,d) strided", F,
        _time11(lambda: fa.fa_forward_ex(q, k, v, o, lse, True, d ** -0.5, "bnhd", stream=stream), torch, np, stream),
        _time11(lambda: fa.fa_backward_ex(q, k, v, o, do, lse, dq, dk, dv, delta, True, d ** -0.5, "bnhd",
                                          stream=stream), torch, np, stream))
    del q, k, v, do, o, lse, delta, dq, dk, dv

    # a packed batch of 8 sequences with a seeded length mix, and the same batch padded to
    # its longest sequence (what the variable-length interface saves)
    lengths = FI.varlen_lengths(8, N, 3001)
    T = int(lengths.sum())
    q, k, v, do = (t[0].transpose(0, 1).contiguous() for t in tensors((1, H, T, d), FI.BF16, 3002))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty(H, T, dtype=torch.float32, device=dev)
    delta, dq, dk, dv = torch.empty_like(lse), torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    F = float(sum(4.0 * H * n * n * d * 0.5 for n in lengths))
    rec(f"varlen 8 seqs, {T} tokens (max {N}) H=32 d=128 causal bf16", F,
        _time11(lambda: fa.fa_forward_ex(q, k, v, o, lse, True, d ** -0.5, cu_seqlens=cu, max_seqlen=N,
                                         stream=stream), torch, np, stream),
        _time11(lambda: fa.fa_backward_ex(q, k, v, o, do, lse, dq, dk, dv, delta, True, d ** -0.5, cu_seqlens=cu,
                                          max_seqlen=N, stream=stream), torch, np, stream))
    del q, k, v, do, o, lse, delta, dq, dk, dv
    q, k, v, do = tensors((8, H, N, d), FI.BF16, 3003)
    o = torch.empty_like(q)
    lse = torch.empty(8, H, N, dtype=torch.float32, device=dev)
    delta, dq, dk, dv = torch.empty_like(lse), torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    rec(f"same batch padded to 8 x {N} (useful work counted)", F,
        _time11(lambda: fa.fa_forward(q, k, v, o, lse, True, d ** -0.5, stream), torch, np, stream),
        _time11(lambda: fa.fa_backward(q, k, v, o, do, lse, dq, dk, dv, delta, True, d ** -0.5, stream), torch, np,
                stream))
    del q, k, v, do, o, lse, delta, dq, dk, dv

    # other head dims at B=4 H=32 N=4096 causal (d = 96 runs 128 wide, 256 at one wave per SIMD)
    for dd, hh in ((96, 32), (256, 16)):
        q, k, v, do = tensors((4, hh, N, dd), FI.BF16, 3100 + dd)
        o = torch.empty_like(q)
        lse = torch.empty(4, hh, N, dtype=torch.float32, device=dev)
        delta, dq, dk, dv = torch.empty_like(lse), torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        F = 4.0 * 4 * hh * N * N * dd * 0.5
        rec(f"B=4 H={hh} N=4096 d={dd} causal bf16", F,
            _time11(lambda: fa.fa_forward(q, k, v, o, lse, True, dd ** -0.5, stream), torch, np, stream),
            _time11(lambda: fa.fa_backward(q, k, v, o, do, lse, dq, dk, dv, delta, True, dd ** -0.5, stream), torch,
                    np, stream))
        del q, k, v, do, o, lse, delta, dq, dk, dv

    # decode: one new query per sequence against a 4096-key cache (B=8 H=32 d=128 bf16), the
    # key range cut into 1..64 ranges. Reading the cache (K and V once) bounds it, so it is
    # reported in GB/s against the HBM peak.
    Bd, Nk = 8, 4096
    bits = FI.draw_bits_rect(Bd, H, 1, Nk, d, FI.BF16, 3200)
    q, k, v = (torch.from_numpy(bits[n].view(np.int16)).to(dev).view(torch.bfloat16) for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty(Bd, H, 1, dtype=torch.float32, device=dev)
    nbytes = 2 * Bd * H * Nk * d * 2 + 2 * Bd * H * d * 2 + Bd * H * 4
    for splits in (0, 4, 8, 16, 32, 64):
        if splits == 0:
            fn = (lambda: fa.fa_forward_ex(q, k, v, o, lse, True, d ** -0.5, "bhnd", stream=stream))
        else:
            need = fa.fa_forward_splitkv_ex_workspace_bytes(q, k, splits, "bhnd")
            ws = torch.empty(need // 4, dtype=torch.float32, device=dev)
            fn = (lambda s=splits, w=ws: fa.fa_forward_splitkv_ex(q, k, v, o, lse, True, d ** -0.5, s, w, "bhnd",
                                                                   stream=stream))
        t = _time11(fn, torch, np, stream)
        gbs = nbytes / (t["mean_us"] * 1e-6) / 1e9
        label = f"decode B={Bd} H={H} Nq=1 Nk={Nk} d={d} causal bf16, " + (f"{splits} ranges" if splits else "no split")
        log(f"  {label:58s} fwd {t['mean_us']:9.1f} us  {gbs:7.0f} GB/s ({gbs / PEAK_HBM_GBS:.1%} of HBM peak)")
        out.append({"extra": label, "fwd": t, "hbm_bytes": nbytes, "gb_per_s": gbs,
                    "frac_of_hbm_peak": gbs / PEAK_HBM_GBS})
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llm_layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=128)
    ap.add_argument("--sweep", action="store_true",
                    help="also time forward and fa_backward on every workload (table on stderr, 'sweep' in the line)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed region, run one plain device-to-device copy of this many MiB "
                         "(a kernel of known traffic for scaling HBM byte counters)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: turn the counter_collection.csv files of a FETCH_SIZE and a WRITE_SIZE "
                         "rocprofv3 --pmc run of this script (with --copy-calibration-mib) into "
                         "profiles/traffic.json, then exit")
    args = ap.parse_args()
    if args.ingest_counters:
        table = ingest_counters(args.ingest_counters[0], args.ingest_counters[1],
                                args.copy_calibration_mib or 256, args.workload)
        print(json.dumps(table, indent=1))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the path shards over batch*heads with no communication, but no multi-GPU run is provided.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import fa_inputs as FI
    import exact_attention_27_amd as fa

    if not torch.cuda.is_available():
        log("bench.py: no GPU visible")
        sys.exit(1)
    fa.load_library()  # raises if libfa.so was not built: there is no fallback
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    w = FI.WORKLOADS[args.workload]
    causal = w.causal[0]
    scale = w.scale()
    log(f"device {props.name} ({getattr(props, 'gcnArchName', '?')}), {props.multi_processor_count} CUs; "
        f"workload {w.label}")

    t0 = time.perf_counter()
    bits = FI.draw_workload(w)
    torch_dt = torch.bfloat16 if w.dtype == FI.BF16 else torch.float16

    def up(name):
        return torch.from_numpy(bits[name].view(np.int16)).to(dev).view(torch_dt)

    q, k, v, do = (up(n) for n in FI.TENSOR_ORDER)
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device=dev)
    delta = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    torch.cuda.synchronize()
    log(f"inputs drawn and resident in HBM in {time.perf_counter() - t0:.1f} s")

    stream = torch.cuda.current_stream(dev)
    names = ["fwd", "bwd_preprocess", "bwd_dkv", "bwd_dq"]

    def step(evs=None):
        if evs:
            evs[0].record(stream)
        fa.fa_forward(q, k, v, o, lse, causal, scale, stream)
        if evs:
            evs[1].record(stream)
        fa.fa_backward_preprocess(o, do, delta, stream)
        if evs:
            evs[2].record(stream)
        fa.fa_backward_dkv(q, k, v, do, lse, delta, dk, dv, causal, scale, stream)
        if evs:
            evs[3].record(stream)
        fa.fa_backward_dq(q, k, v, do, lse, delta, dq, causal, scale, stream)
        if evs:
            evs[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for s in range(args.steps):
        step(ev[s])
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    kern_ms = {n: float(np.mean([ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)]))
               for i, n in enumerate(names)}
    log("per-kernel mean ms: " + ", ".join(f"{n}={t:.4f}" for n, t in kern_ms.items()))

    F = 4.0 * w.B * w.H * w.N * w.N * w.d * (0.5 if causal else 1.0)
    step_flops = 3.5 * F
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    fwd_tflops = F / (kern_ms["fwd"] * 1e-3) / 1e12
    bwd_ms = kern_ms["bwd_preprocess"] + kern_ms["bwd_dkv"] + kern_ms["bwd_dq"]
    bwd_tflops = 2.5 * F / (bwd_ms * 1e-3) / 1e12

    # Algorithmic work per launch: forward F; dK/dV kernel 2F (S, dP,
    # dV, dK); dQ kernel 0.5F (dQ only -- its S and dP recomputation is the price of having
    # no atomics and is not counted); preprocess reads O and dO and writes delta (bytes).
    rows = w.B * w.H * w.N
    algo = {
        "fwd": ("mfma", F / 1e12, "TFLOP/s", PEAK_BF16_TFLOPS),
        "bwd_dkv": ("mfma", 2.0 * F / 1e12, "TFLOP/s", PEAK_BF16_TFLOPS),
        "bwd_dq": ("mfma", 0.5 * F / 1e12, "TFLOP/s", PEAK_BF16_TFLOPS),
        "bwd_preprocess": ("hbm", (2 * rows * w.d * 2 + rows * 4) / 1e9, "GB/s", PEAK_HBM_GBS),
    }
    dominant = max(kern_ms, key=kern_ms.get)
    bound, work, unit, peak = algo[dominant]
    achieved = work / (kern_ms[dominant] * 1e-3)
    roofline = {
        "bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
        "traffic": traffic_for(dominant, w.key), "kernel": dominant, "ms": kern_ms[dominant],
    }
    kernels = {}
    for n in names:
        b_, wk, u, pk = algo[n]
        a_ = wk / (kern_ms[n] * 1e-3)
        kernels[n] = {"ms": kern_ms[n], "achieved": a_, "unit": u, "frac": a_ / pk,
                      "traffic": traffic_for(n, w.key)}

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {args.copy_calibration_mib} MiB read + {args.copy_calibration_mib} MiB written")
        del src, dst

    sweep = None
    if args.sweep:
        log("sweep over the workloads (11 runs each, first discarded):")
        sweep = sweep_configs(fa, FI, torch, np, dev, log)
        log("strided, variable-length and other head dims (11 runs each, first discarded):")
        sweep += sweep_extras(fa, FI, torch, np, dev, log)

    cpu = None
    if not args.no_cpu_baseline:
        n = max(1, min(args.cpu_heads, w.B * w.H))
        heads = [(i // w.H, i % w.H) for i in range(0, w.B * w.H, w.B * w.H // n)][:n]
        log(f"timing the fp64 oracle on {len(heads)} head(s) on the host ...")
        cpu = cpu_baseline(bits, w, heads)

    line = {
        "metric": "fwd+bwd attention TFLOP/s and % of bf16 MFMA peak, N=4096 d=128 causal",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == FI.BF16 else "fp16",
        "data": "synthetic (seeded N(0,1), fixed before any result)",
        "config": {"workload": w.label, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": causal,
                   "seed": w.seed, "counted_flop_per_step": step_flops},
        "frac_of_peak": value / PEAK_BF16_TFLOPS,
        "fwd_tflops": fwd_tflops,
        "fwd_frac_of_peak": fwd_tflops / PEAK_BF16_TFLOPS,
        "bwd_tflops": bwd_tflops,
        "roofline": roofline,
        "kernels": kernels,
        "cpu_baseline": cpu,
        "sweep": sweep,
        "device": {"name": props.name, "cus": props.multi_processor_count},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
