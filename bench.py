#!/usr/bin/env python3
"""Benchmark of the exact tiled attention path on one MI355X.

One step = one full pass of the hot path over one batch of synthetic input resident in HBM:
fa_forward (O, LSE) followed by the backward (dQ computing delta, then dK/dV -- the two
stages fa_backward runs, launched individually here so each kernel can be timed with HIP
events on the stream it runs on).

Workload (default): B=4, H=32, N=4096, d=128, causal, bf16, Q, K, V, dO ~ N(0,1) from seed
1004, scale = 1/sqrt(d). Counted FLOPs: forward F = 4*B*H*N^2*d, halved for causal
("Triton 05: Flash Attention", section on why throughput stops at a fraction of peak: the
two matmuls of the forward); backward 2.5 F; a step counts 3.5 F.

Prints ONE JSON line on stdout. Progress goes to stderr.

Besides the headline steps, the line carries "configs": every workload (and mask setting),
each kernel timed as 11 runs on one stream, each bracketed by its own HIP events, enqueued
back to back, the first discarded: the forward, its ping-pong form, the two backward stages
one by one and one fa_backward call, with counted TFLOP/s, the fraction of the chip's peak, the clock and
matrix-core utilisation each kernel ran at (from committed counter runs, when they match the
current sources) and the fp64 oracle's forward and backward wall times on a sample of heads.

Options beyond the contract (--gpus, --steps, --warmup):
  --no-configs               leave out the per-workload records
  --sweep                    also time the split-KV forward (2 and 4 ranges) on every workload,
                             and the strided, packed, other head-dim and decode (one query
                             against a key cache) problems
  --counter-pass             no timing: launch every workload's kernels (STAGES) 3 times each in
                             a fixed order, for a rocprofv3 --pmc run that --ingest-sq reads
  --ingest-sq SQ [FETCH WRITE]
                             no GPU work: turn the counter_collection.csv files of --counter-pass
                             rocprofv3 runs (GRBM_GUI_ACTIVE, SQ_VALU_MFMA_BUSY_CYCLES,
                             SQ_INSTS_MFMA; then FETCH_SIZE, then WRITE_SIZE with the copy
                             calibration) into profiles/counters.json
  --copy-calibration-mib M   after the timed region, one plain device copy of M MiB: the
                             kernel of known traffic that scales the HBM byte counters
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16/fp16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
SQ_FILE = os.path.join(ROOT, "profiles", "counters.json")
N_SIMDS = 1024              # 256 CUs x 4 SIMDs
N_XCDS = 8                  # GRBM_GUI_ACTIVE sums the 8 XCDs' cycle counts
COUNTER_REPEATS = 3         # launches of each kernel per workload in a --counter-pass run
# the kernels of a step, plus the forward's two-group ping-pong form (fa_forward_pingpong),
# timed and counted beside them on every workload
STAGES = ("fwd", "fwd_pingpong", "bwd_dq_delta", "bwd_dkv")
KERNEL_SOURCES = {
    "fwd": ["fa_fwd.hip", "fa_common.hpp", "fa_kernels.hpp"],
    "fwd_pingpong": ["fa_fwd.hip", "fa_common.hpp", "fa_kernels.hpp"],
    "bwd_dkv": ["fa_bwd_dkv.hip", "fa_common.hpp", "fa_kernels.hpp"],
    "bwd_dq_delta": ["fa_bwd.hip", "fa_common.hpp", "fa_kernels.hpp"],
}
# Kernel-name fragments of each timed kernel in a profiler's per-dispatch records.
KERNEL_SYMBOLS = {"fwd": "fwd_kernel", "fwd_pingpong": "fwd_kernel", "bwd_dkv": "bwd_dkv_kernel",
                  "bwd_dq_delta": "bwd_dq_kernel"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def code_text(src: str) -> str:
    """A kernel source without its comments and with every whitespace run collapsed, so that
    a change of comments alone leaves the hash below, and with it the counter table's claim
    on the kernel, as it is (the sources hold no "//" inside string literals and no block
    comments)."""
    return " ".join(re.sub(r"//[^\n]*", " ", src).split())


def source_sha(kernel: str) -> str:
    """Hash of the code (comments left out) of the sources a kernel is built from."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "exact_attention_27_amd", "csrc", name), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def algorithmic_bytes(kernel: str, w) -> float:
    """HBM bytes a kernel must move once on workload w: its operands read and its outputs
    written, each exactly once (16-bit tensors of B*H*N*d, float32 rows of B*H*N)."""
    t, r = w.B * w.H * w.N * w.d * 2, w.B * w.H * w.N * 4
    return {"fwd": 4 * t + r,                   # Q, K, V in; O, LSE out
            "fwd_pingpong": 4 * t + r,
            "bwd_dkv": 6 * t + 2 * r,           # Q, K, V, dO, LSE, delta in; dK, dV out
            "bwd_dq_delta": 6 * t + 2 * r}[kernel]  # Q, K, V, O, dO, LSE in; dQ, delta out


def traffic_for(kernel: str, workload: str, causal: bool = True):
    """HBM bytes per launch from the committed counter runs, or None when absent or taken on
    other sources."""
    try:
        with open(SQ_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        return None
    rec = table.get(f"{workload}|{int(causal)}|{kernel}")
    if not rec or rec.get("source_sha") != source_sha(kernel):
        return None
    return rec.get("bytes_per_launch")


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
    """The split-KV forward (fa_forward_splitkv) with 2 and 4 key ranges per Q tile on every
    workload and mask setting, 11 runs each bracketed by HIP events on one stream, the first
    discarded (workspaces above 1 GiB are skipped)."""
    out = []
    stream = torch.cuda.current_stream(dev)
    for key, w in FI.WORKLOADS.items():
        bits, t = _config_tensors(FI, torch, np, dev, w)
        for causal in w.causal:
            F = 4.0 * w.B * w.H * w.N * w.N * w.d * (0.5 if causal else 1.0)
            res = {}
            for sp in (2, 4):
                nb = fa.fa_forward_splitkv_workspace_bytes(w.B, w.H, w.N, w.d, sp)
                if nb > (1 << 30):
                    continue
                ws = torch.empty(nb // 4, dtype=torch.float32, device=dev)
                res[f"fwd_split{sp}"] = _time11(lambda: fa.fa_forward_splitkv(t["q"], t["k"], t["v"], t["o"], t["lse"],
                                                                               causal, w.scale(), sp, ws, stream),
                                                torch, np, stream)
                res[f"fwd_split{sp}"]["tflops"] = F / (res[f"fwd_split{sp}"]["mean_us"] * 1e-6) / 1e12
                del ws
            log(f"  {key:13s} causal={int(causal)}  split-KV fwd: "
                + ", ".join(f"{k[9:]} ranges {v['mean_us']:.1f} us" for k, v in res.items()))
            out.append({"workload": key, "label": w.label, "causal": causal, **res})
        del t, bits
        torch.cuda.empty_cache()
    return out


def _time11(fn, torch, np, stream, settle_s=0.05):
    """11 runs of fn, each bracketed by its own pair of HIP events on `stream`, the first
    discarded (microseconds). The runs are enqueued back to back and the host synchronises once
    at the end: with a host synchronisation after every run the GPU clock never settles and
    single launches read 10-20% slower than the same kernels in a training step. Before them fn
    runs back to back for about settle_s seconds, for the same reason: after the host-side
    set-up between workloads the first milliseconds of work ran up to 20% slower and noisier."""
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    once = max(time.perf_counter() - t0, 1e-6)
    for _ in range(min(2000, max(1, int(settle_s / once)))):
        fn()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(11)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    ts = np.array([a.elapsed_time(b) for a, b in evs[1:]]) * 1e3
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


def copy_calibration(torch, dev, mib, log):
    """One plain device copy of `mib` MiB: the kernel of known traffic that scales the HBM byte
    counters."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: {mib} MiB read + {mib} MiB written")
    del src, dst


def config_list(FI):
    """(workload key, causal) of every workload and mask setting, in a fixed order."""
    return [(key, causal) for key, w in FI.WORKLOADS.items() for causal in w.causal]


def _config_tensors(FI, torch, np, dev, w):
    bits = FI.draw_workload(w)
    tdt = torch.bfloat16 if w.dtype == FI.BF16 else torch.float16
    q, k, v, do = (torch.from_numpy(bits[n].view(np.int16)).to(dev).view(tdt) for n in FI.TENSOR_ORDER)
    t = {"q": q, "k": k, "v": v, "do": do, "o": torch.empty_like(q),
         "lse": torch.empty(w.B, w.H, w.N, dtype=torch.float32, device=dev),
         "dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v)}
    t["delta"] = torch.empty_like(t["lse"])
    return bits, t


def _stage_fns(fa, t, causal, scale, stream):
    """The kernels of a step (forward; dQ with delta; dK/dV) and the ping-pong forward, each as
    one call, in an order that lets each consume what the previous ones wrote."""
    return {
        "fwd": lambda: fa.fa_forward(t["q"], t["k"], t["v"], t["o"], t["lse"], causal, scale, stream),
        "fwd_pingpong": lambda: fa.fa_forward_pingpong(t["q"], t["k"], t["v"], t["o"], t["lse"], causal, scale,
                                                       stream),
        "bwd_dkv": lambda: fa.fa_backward_dkv(t["q"], t["k"], t["v"], t["do"], t["lse"], t["delta"], t["dk"], t["dv"],
                                              causal, scale, stream),
        "bwd_dq_delta": lambda: fa.fa_backward_dq_delta(t["q"], t["k"], t["v"], t["o"], t["do"], t["lse"], t["dq"],
                                                        t["delta"], causal, scale, stream),
    }


def kernel_work(name, w, causal):
    """Algorithmic work of one launch of a kernel on workload w: (bound, amount, unit, peak).
    Forward F = 4 B H N^2 d, halved for causal; dK/dV 2F (S, dP, dV, dK); dQ 0.5F (dQ only: its
    S and dP recomputation is the price of having no atomics, and its D computation, are not
    counted)."""
    F = 4.0 * w.B * w.H * w.N * w.N * w.d * (0.5 if causal else 1.0)
    return {
        "fwd": ("mfma", F / 1e12, "TFLOP/s", PEAK_BF16_TFLOPS),
        "fwd_pingpong": ("mfma", F / 1e12, "TFLOP/s", PEAK_BF16_TFLOPS),
        "bwd_dkv": ("mfma", 2.0 * F / 1e12, "TFLOP/s", PEAK_BF16_TFLOPS),
        "bwd_dq_delta": ("mfma", 0.5 * F / 1e12, "TFLOP/s", PEAK_BF16_TFLOPS),
    }[name]


def counters_for(kernel: str, key: str, causal: bool):
    """Clock and matrix-core utilisation of a kernel on a workload, from the committed counter
    run, or None when absent or taken on other sources."""
    try:
        with open(SQ_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        return None
    rec = table.get(f"{key}|{int(causal)}|{kernel}")
    if not rec or rec.get("source_sha") != source_sha(kernel):
        return None
    return {"clock_ghz": rec.get("clock_ghz"), "mfma_busy": rec.get("mfma_busy"),
            "mfma_issued_per_needed": rec.get("mfma_issued_per_needed"), "counter_run_us": rec.get("us"),
            "hbm_bytes": rec.get("bytes_per_launch")}


def oracle_times(bits, w, causal, heads):
    """The fp64 oracle as it stands, forward alone and forward + backward, on `heads`."""
    import fa_inputs as FI
    from oracle import attention as ORACLE
    tf = tb = 0.0
    for b, h in heads:
        q, k, v, do = (FI.bits_to_f64(bits[n][b, h], w.dtype) for n in FI.TENSOR_ORDER)
        t0 = time.perf_counter()
        ORACLE.forward(q, k, v, w.scale(), causal)
        t1 = time.perf_counter()
        ORACLE.backward(q, k, v, do, w.scale(), causal)
        t2 = time.perf_counter()
        tf += t1 - t0
        tb += t2 - t1
    F = 4.0 * w.N * w.N * w.d * (0.5 if causal else 1.0) * len(heads)
    return {"heads": len(heads), "of_heads": w.B * w.H, "fwd_s": tf, "fwd_bwd_s": tb,
            "bwd_s_derived": tb - tf, "fwd_tflops": F / tf / 1e12, "fwd_bwd_tflops": 3.5 * F / tb / 1e12,
            "note": "oracle.backward recomputes the forward it needs: bwd_s_derived = fwd_bwd_s - fwd_s"}


# heads of each workload the oracle is timed on (about 10 s of host work in all)
ORACLE_HEADS = {"single_head": 1, "small_causal": 8, "gpt2_medium": 32, "llm_layer": 8, "long_context": 1}


def config_records(fa, FI, torch, np, dev, log, with_oracle=True):
    """Every workload and mask setting: each kernel and one fa_backward call timed as 11 runs
    bracketed by HIP events on one stream (first discarded), roofline fraction per kernel,
    counter-derived clock and matrix-core utilisation, and the oracle's wall times."""
    out = []
    stream = torch.cuda.current_stream(dev)
    for key, w in FI.WORKLOADS.items():
        bits, t = _config_tensors(FI, torch, np, dev, w)
        for causal in w.causal:
            fns = _stage_fns(fa, t, causal, w.scale(), stream)
            fns["fwd"]()  # O and LSE for the backward stages
            kern = {}
            for name in STAGES:
                tm = _time11(fns[name], torch, np, stream)
                bound, work, unit, peak = kernel_work(name, w, causal)
                ach = work / (tm["mean_us"] * 1e-6)
                kern[name] = {**tm, "bound": bound, "achieved": ach, "unit": unit, "frac": ach / peak,
                              "algorithmic_bytes": algorithmic_bytes(name, w),
                              "counters": counters_for(name, key, causal)}
            bwd = _time11(lambda: fa.fa_backward(t["q"], t["k"], t["v"], t["o"], t["do"], t["lse"], t["dq"], t["dk"],
                                                 t["dv"], t["delta"], causal, w.scale(), stream), torch, np, stream)
            F = 4.0 * w.B * w.H * w.N * w.N * w.d * (0.5 if causal else 1.0)
            fwd_us = kern["fwd"]["mean_us"]
            rec = {"workload": key, "label": w.label, "causal": causal, "counted_fwd_flop": F,
                   "fwd": {k: kern["fwd"][k] for k in ("mean_us", "std_us", "median_us")}, "bwd": bwd,
                   "fwd_tflops": F / (fwd_us * 1e-6) / 1e12,
                   "fwd_frac_of_peak": F / (fwd_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS,
                   "fwd_bwd_tflops": 3.5 * F / ((fwd_us + bwd["mean_us"]) * 1e-6) / 1e12,
                   "kernels": kern}
            rec["fwd_bwd_frac_of_peak"] = rec["fwd_bwd_tflops"] / PEAK_BF16_TFLOPS
            if with_oracle:
                n = min(ORACLE_HEADS.get(key, 1), w.B * w.H)
                stride = (w.B * w.H) // n
                heads = [(i // w.H, i % w.H) for i in range(0, w.B * w.H, stride)][:n]
                rec["oracle"] = oracle_times(bits, w, causal, heads)
                rec["oracle"]["cores"] = len(os.sched_getaffinity(0))
            log(f"  {key:13s} causal={int(causal)}  fwd {fwd_us:8.1f} us  bwd {bwd['mean_us']:8.1f} us  "
                f"fwd {rec['fwd_tflops']:7.1f} TFLOP/s ({rec['fwd_frac_of_peak']:.1%})  fwd+bwd "
                f"{rec['fwd_bwd_tflops']:7.1f} ({rec['fwd_bwd_frac_of_peak']:.1%})  "
                + "  ".join(f"{n}={kern[n]['mean_us']:.1f}us/{kern[n]['frac']:.2f}" for n in STAGES)
                + (f"  oracle fwd {rec['oracle']['fwd_s']:.2f}s fwd+bwd {rec['oracle']['fwd_bwd_s']:.2f}s"
                   f" on {rec['oracle']['heads']} head(s)" if with_oracle else ""))
            out.append(rec)
        del t, bits
        torch.cuda.empty_cache()
    return out


def counter_pass(fa, FI, torch, np, dev, log):
    """For a rocprofv3 --pmc run: every workload and mask setting in config_list order, each of
    the kernels of STAGES launched COUNTER_REPEATS times each in that order, nothing else of ours."""
    stream = torch.cuda.current_stream(dev)
    for key, w in FI.WORKLOADS.items():
        bits, t = _config_tensors(FI, torch, np, dev, w)
        for causal in w.causal:
            fns = _stage_fns(fa, t, causal, w.scale(), stream)
            for name in STAGES:
                for _ in range(COUNTER_REPEATS):
                    fns[name]()
            torch.cuda.synchronize()
            log(f"  counter pass: {key} causal={int(causal)} done")
        del t, bits
        torch.cuda.empty_cache()


def _dispatches(csv_path: str):
    """Our kernels' dispatches of a --counter-pass rocprofv3 run, in launch order: a list of
    {kernel, name, ns, <counter>: value} (kernel: the KERNEL_SYMBOLS family) and the copy
    kernel's counters (or None)."""
    import csv
    import collections
    disp = collections.OrderedDict()
    copy = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if "copy" in name.lower():
                copy[r["Counter_Name"]] = float(r["Counter_Value"])
                continue
            fam = next((fr for fr in set(KERNEL_SYMBOLS.values()) if f"fa::{fr}<" in name), None)
            if fam is None:
                continue
            d = disp.setdefault(int(r["Dispatch_Id"]), {"kernel": fam, "name": name,
                                                        "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
            d[r["Counter_Name"]] = float(r["Counter_Value"])
    return [disp[k] for k in sorted(disp)], (copy or None)


def _attribute(seq):
    """Group launch-ordered dispatches by (workload key, causal, stage), checking the order."""
    import collections
    import fa_inputs as FI
    plan = [(key, causal, st) for key, causal in config_list(FI) for st in STAGES for _ in range(COUNTER_REPEATS)]
    if len(seq) != len(plan):
        raise SystemExit(f"expected {len(plan)} dispatches of our kernels, found {len(seq)}")
    acc = collections.defaultdict(list)
    for d, (key, causal, st) in zip(seq, plan):
        if d["kernel"] != KERNEL_SYMBOLS[st]:
            raise SystemExit(f"dispatch order mismatch: expected {st} for {key}, found {d['name'][:60]}")
        acc[(key, causal, st)].append(d)
    return acc


def ingest_traffic(fetch_csv: str, write_csv: str, copy_mib: int, table: dict) -> dict:
    """Add HBM bytes per launch to `table` (from ingest_sq) from a FETCH_SIZE and a WRITE_SIZE
    --counter-pass run (KiB per dispatch), each scaled by what the same counter read for the
    plain copy of copy_mib MiB that the counter pass runs last."""
    fseq, fcopy = _dispatches(fetch_csv)
    wseq, wcopy = _dispatches(write_csv)
    if not fcopy or not wcopy:
        raise SystemExit("no copy kernel in the counter files (run --counter-pass with --copy-calibration-mib)")
    nbytes = copy_mib * (1 << 20)
    ff = nbytes / (fcopy["FETCH_SIZE"] * 1024)
    wf = nbytes / (wcopy["WRITE_SIZE"] * 1024)
    fa_, wa_ = _attribute(fseq), _attribute(wseq)
    for (key, causal, st), ds in fa_.items():
        rec = table.setdefault(f"{key}|{int(causal)}|{st}", {"workload": key, "causal": causal, "kernel": st,
                                                             "source_sha": source_sha(st)})
        fb = sum(d["FETCH_SIZE"] for d in ds) / len(ds) * 1024 * ff
        wb = sum(d["WRITE_SIZE"] for d in wa_[(key, causal, st)]) / len(ds) * 1024 * wf
        rec.update({"fetch_bytes": round(fb), "write_bytes": round(wb), "bytes_per_launch": round(fb + wb)})
    table["_calibration"] = {"copy_mib": copy_mib, "fetch_factor": ff, "write_factor": wf}
    return table


def ingest_sq(csv_path: str, write: bool = True) -> dict:
    """Per (workload, mask, kernel) clock and matrix-core utilisation from the
    counter_collection.csv of a rocprofv3 --pmc run of --counter-pass, with the dispatches of
    our kernels attributed by launch order (config_list x STAGES x COUNTER_REPEATS).
    clock = GRBM_GUI_ACTIVE / 8 XCDs / dispatch time; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES /
    (1024 SIMDs x GRBM_GUI_ACTIVE / 8); MFMA issued per needed = SQ_INSTS_MFMA / (needed FLOP /
    32768, one 32x32x16 product; for dQ three times its counted work, since it recomputes S
    and dP) for the three matrix kernels."""
    import fa_inputs as FI
    seq, _ = _dispatches(csv_path)
    acc = _attribute(seq)
    out = {}
    for (key, causal, st), ds in acc.items():
        w = FI.WORKLOADS[key]
        cyc = [d["GRBM_GUI_ACTIVE"] / N_XCDS for d in ds]
        rec = {"workload": key, "causal": causal, "kernel": st, "source_sha": source_sha(st),
               "dispatches": len(ds), "us": sum(d["ns"] for d in ds) / len(ds) / 1e3,
               "clock_ghz": sum(c / d["ns"] for c, d in zip(cyc, ds)) / len(ds),
               "mfma_busy": sum(d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (N_SIMDS * c) for c, d in zip(cyc, ds)) / len(ds),
               "kernel_name": ds[0]["name"].split("(")[0]}
        bound, work, unit, _ = kernel_work(st, w, causal)
        if bound == "mfma" and "SQ_INSTS_MFMA" in ds[0]:
            # products the kernel's algorithm needs: the counted work, and for dQ its S and dP too
            executed = {"fwd": 1.0, "fwd_pingpong": 1.0, "bwd_dkv": 1.0, "bwd_dq_delta": 3.0}[st]
            rec["mfma_issued_per_needed"] = (sum(d["SQ_INSTS_MFMA"] for d in ds) / len(ds)) / (work * 1e12 * executed / 32768)
        out[f"{key}|{int(causal)}|{st}"] = rec
    if write:
        with open(SQ_FILE, "w") as f:
            json.dump(out, f, indent=1)
            f.write("\n")
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="llm_layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=128)
    ap.add_argument("--no-configs", action="store_true", help="leave out the per-workload records")
    ap.add_argument("--sweep", action="store_true",
                    help="also time the split-KV forward on every workload and the strided, packed, other head-dim "
                         "and decode problems (table on stderr, 'sweep' in the line)")
    ap.add_argument("--counter-pass", action="store_true",
                    help="no timing: launch every workload's four kernels a fixed number of times (rocprofv3 --pmc)")
    ap.add_argument("--ingest-sq", nargs="+", metavar="CSV",
                    help="no GPU work: counter_collection.csv of an SQ --counter-pass run, optionally followed by "
                         "those of a FETCH_SIZE and a WRITE_SIZE run (with --copy-calibration-mib) -> "
                         "profiles/sq_counters.json")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed region, run one plain device-to-device copy of this many MiB "
                         "(a kernel of known traffic for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.ingest_sq:
        table = ingest_sq(args.ingest_sq[0], write=len(args.ingest_sq) == 1)
        if len(args.ingest_sq) == 3:
            table = ingest_traffic(args.ingest_sq[1], args.ingest_sq[2], args.copy_calibration_mib or 256, table)
            with open(SQ_FILE, "w") as f:
                json.dump(table, f, indent=1)
                f.write("\n")
        print(json.dumps(table, indent=1))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
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
    if args.counter_pass:
        counter_pass(fa, FI, torch, np, dev, log)
        if args.copy_calibration_mib > 0:
            copy_calibration(torch, dev, args.copy_calibration_mib, log)
        return
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
    names = ["fwd", "bwd_dq_delta", "bwd_dkv"]

    def step(evs=None):
        if evs:
            evs[0].record(stream)
        fa.fa_forward(q, k, v, o, lse, causal, scale, stream)
        if evs:
            evs[1].record(stream)
        fa.fa_backward_dq_delta(q, k, v, o, do, lse, dq, delta, causal, scale, stream)
        if evs:
            evs[2].record(stream)
        fa.fa_backward_dkv(q, k, v, do, lse, delta, dk, dv, causal, scale, stream)
        if evs:
            evs[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
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
    bwd_ms = kern_ms["bwd_dq_delta"] + kern_ms["bwd_dkv"]
    bwd_tflops = 2.5 * F / (bwd_ms * 1e-3) / 1e12

    # Algorithmic work per launch (kernel_work): forward F; dK/dV kernel 2F (S, dP, dV, dK);
    # dQ kernel 0.5F (dQ only -- its S and dP recomputation is the price of having no atomics,
    # and its D computation, are not counted).
    algo = {n: kernel_work(n, w, causal) for n in names}
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
        copy_calibration(torch, dev, args.copy_calibration_mib, log)

    configs = None
    if not args.no_configs:
        log("every workload (11 runs per kernel, first discarded; oracle on a sample of heads):")
        configs = config_records(fa, FI, torch, np, dev, log, with_oracle=not args.no_cpu_baseline)

    sweep = None
    if args.sweep:
        log("split-KV forward on every workload (11 runs each, first discarded):")
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
        "configs": configs,
        "sweep": sweep,
        "device": {"name": props.name, "cus": props.multi_processor_count},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
