"""Throughput of the libfa forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload C4]

One step is one call of the whole forward pass (``fa_fwd``: one kernel) over
the workload's inputs, which are resident in HBM before timing starts.  The
default workload is the bf16 long-sequence shape B=1 H=16 N=16384 d=64,
non-causal.  Workloads with grouped K/V heads, their own key length or a key
split (C1s, D1, G1, G2) run through ``fa_fwd_ex`` instead: one step is then
the whole call (the split kernel and, when split, the combine kernel), with
its workspace allocated before timing.  ``--pass bwd`` times the backward
pass instead (``fa_bwd``: row dot products, dK/dV, dQ; for grouped K/V heads
``fa_bwd_ex`` with its default head parts, plus their part sum) on the same
workloads, after one forward call that provides O and LSE; its FLOPs follow
the usual convention of 2.5x the forward's (five products of 2*d FLOPs per
visible pair).  Prints ONE JSON line with:

  value / ms_per_step   whole-job throughput (metric FLOPs 4*B*H*N^2*d, halved
                        when causal) from a wall clock around K steps,
                        bracketed by stream synchronisation;
  roofline              the kernel's own average duration from HIP events
                        recorded on the launch stream around each of K more
                        launches, queued behind a delay kernel of the probe
                        library (libfa_probe.so) so that they run back to back
                        and the host's launch gap stays out of the events,
                        against the MI355X dense MFMA peak of the
                        input dtype, or against HBM bandwidth (8 TB/s)
                        when the workload's FLOP per algorithmic byte is
                        below the ridge point; ``hbm_gbs`` is the algorithmic
                        bytes (Q, K, V read once, O and LSE written once) over
                        that duration; ``traffic`` is the HBM bytes per launch
                        from the committed rocprofv3 counter summary when it
                        was taken on the current kernel source, else null;
                        ``kernel_ms_cold_median`` times further calls made
                        right after reading a 512 MiB buffer (L2 and MALL
                        flushed), so K/V start from HBM; ``mfma_loop_tflops``
                        is the rate of a plain MFMA loop of the same input
                        type on every SIMD (libfa_probe.so), measured after
                        the timed steps at the clock the chip then holds, and
                        ``frac_of_mfma_loop`` the kernel's rate against it;
  cpu_baseline          the fp64 oracle timed on the host cores on a bounded
                        row sample of the same workload (reported baseline),
                        with the CPU model, the host's core counts, the
                        threads used, and the whole C1 workload on one thread.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "fwd attention TFLOP/s & % MFMA peak, bf16 B=1 H=16 N=16384 d=64 (1 GPU)"
# MI355X published dense peaks (TFLOP/s) per input dtype, and HBM bandwidth.
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
COLD_FLUSH_BYTES = 512 << 20
# Sources of the forward kernels of each input-type family (a committed
# traffic summary counts only while these hash to the value it records).
FWD_SOURCES = {
    "h16": ["fa_device.hpp", "fa_h16.hpp", "fa_lds_dma.hpp", "fa_fwd_h16.hip", "fa_api.hip",
            "fa_api_util.hpp", "fa_combine.hip"],
    "f32": ["fa_device.hpp", "fa_fwd_f32.hip", "fa_api.hip", "fa_api_util.hpp", "fa_combine.hip"],
}


BWD_SOURCES = ["fa_device.hpp", "fa_h16.hpp", "fa_lds_dma.hpp", "fa_bwd.hpp", "fa_bwd_h16.hip",
               "fa_bwd_f32.hip", "fa_api_bwd.hip", "fa_api_util.hpp"]


def fwd_sources(dtype: str):
    return FWD_SOURCES["f32" if dtype == "f32" else "h16"]


def kernel_source_hash(names=FWD_SOURCES["h16"]) -> str:
    h = hashlib.sha256()
    for name in names:
        h.update((ROOT / "exact_attention_13_amd" / "csrc" / name).read_bytes())
    return h.hexdigest()[:16]


def read_traffic(workload: str, dtype: str):
    """HBM bytes per launch from the committed counter summary, or None."""
    path = ROOT / "profiles" / f"fa_fwd_{workload}_hbm_traffic.txt"
    if not path.exists():
        return None
    fields = {}
    for line in path.read_text().splitlines():
        m = re.match(r"^([a-z_]+):\s*(\S+)", line)
        if m:
            fields[m.group(1)] = m.group(2)
    if fields.get("kernel_source_sha") != kernel_source_hash(fwd_sources(dtype)):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, q, k, v, target_s: float):
    """fp64 oracle on a bounded row sample, scaled to TFLOP/s."""
    import numpy as np
    import oracle
    from oracle.reference import default_threads

    threads = default_threads()
    pair_flops = 4.0 * w.d
    nk = w.n_kv

    def rows_flops(rows):
        i = rows % w.N
        vis = np.clip(i + 1 + nk - w.N, 0, nk) if w.causal else np.full(rows.shape, nk)
        return float(vis.sum()) * pair_flops

    rng = np.random.default_rng(99)
    total = w.B * w.H * w.N
    # Rate from two calibration samples: a small one, then one of about 1.5 s
    # (the small one's fixed start-up cost would understate the rate).
    size = min(256, total)
    for target in (None, 1.5):
        if target is not None:
            size = int(min(total, max(256, target * rate / per_row)))
        calib = np.sort(rng.choice(total, size=size, replace=False)).astype(np.int64)
        t0 = time.perf_counter()
        oracle.fwd_gqa(q, k, v, w.scale, w.causal, rows=calib, threads=threads)
        dt = max(time.perf_counter() - t0, 1e-3)
        rate = rows_flops(calib) / dt
        per_row = max(rows_flops(calib) / len(calib), 1.0)
    want = int(min(total, max(256, target_s * rate / per_row)))
    rows = np.sort(rng.choice(total, size=want, replace=False)).astype(np.int64)
    t0 = time.perf_counter()
    oracle.fwd_gqa(q, k, v, w.scale, w.causal, rows=rows, threads=threads)
    dt = time.perf_counter() - t0
    fl = rows_flops(rows)
    out = {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": f"{want} of {total} query rows (uniform, seed 99) of the same workload, "
                     f"{fl:.3e} FLOPs in {dt:.1f} s, fp64 three-pass, {threads} threads"}
    out.update(host_cpu(threads))
    out["one_thread_C1"] = one_thread_c1()
    return out


def host_cpu(threads: int) -> dict:
    """The host the oracle ran on: CPU model, cores the process may use, and
    the thread count taken (all of them up to 16, the host share of one GPU
    on the measurement boxes)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count() or 1
    return {"cpu_model": model, "host_logical_cpus": os.cpu_count(),
            "affinity_cpus": affinity, "threads_used": threads,
            "thread_cap": "min(affinity, 16)"}


def one_thread_c1() -> dict:
    """The whole C1 workload (fp32, one 512-row head, d = 64) on one thread:
    the kind of single-threaded CPU figure the pages report."""
    from exact_attention_13_amd.inputs import WORKLOADS, make_inputs
    import oracle
    w = WORKLOADS["C1"]
    q, k, v = make_inputs(w)
    oracle.fwd(q, k, v, w.scale, w.causal, threads=1)  # warm (library load)
    best = None
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.fwd(q, k, v, w.scale, w.causal, threads=1)
        dt = time.perf_counter() - t0
        best = dt if best is None else min(best, dt)
    return {"ms": round(best * 1e3, 3), "GFLOP/s": round(w.flops / best / 1e9, 3),
            "workload": "C1: fp32 B=1 H=1 N=512 d=64, fp64 oracle, 1 thread, best of 3"}


def cpu_baseline_bwd(w, q, k, v, dout, target_s: float):
    """fp64 oracle dQ rows on a bounded row sample, scaled to TFLOP/s.

    A dQ row recomputes its scores, weights and output (2 + 2 FLOPs per key
    and column), dP (2) and dQ (2): 8*d FLOPs per visible key.  The oracle's
    row routine runs on one thread.
    """
    import numpy as np
    import oracle

    rng = np.random.default_rng(98)
    total = w.B * w.H * w.N

    def rows_flops(rows):
        nk = w.n_kv
        vis = np.clip(rows % w.N + 1 + (nk - w.N), 0, nk) if w.causal else np.full(rows.shape, nk)
        return float(vis.sum()) * 8.0 * w.d

    calib = np.sort(rng.choice(total, size=min(16, total), replace=False)).astype(np.int64)
    t0 = time.perf_counter()
    oracle.bwd_dq_rows(q, k, v, dout, w.scale, w.causal, calib)
    rate = rows_flops(calib) / max(time.perf_counter() - t0, 1e-6)
    per_row = rows_flops(calib) / len(calib)
    want = int(min(total, max(16, target_s * rate / per_row)))
    rows = np.sort(rng.choice(total, size=want, replace=False)).astype(np.int64)
    t0 = time.perf_counter()
    oracle.bwd_dq_rows(q, k, v, dout, w.scale, w.causal, rows)
    dt = time.perf_counter() - t0
    fl = rows_flops(rows)
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"dQ of {want} of {total} query rows (uniform, seed 98) of the same "
                      f"workload, 8*d FLOPs per visible key, {fl:.3e} FLOPs in {dt:.1f} s, fp64, "
                      f"1 thread"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="C4")
    ap.add_argument("--pass", dest="which", choices=["fwd", "bwd"], default="fwd",
                    help="time the forward pass (default) or the backward pass")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--read-bytes", type=int, default=0,
                    help="instead of attention, time a plain reduction that reads this many "
                         "bytes (the streaming-read rate a bandwidth-bound kernel can expect)")
    ap.add_argument("--splits", type=int, default=None,
                    help="key ranges for fa_fwd_ex workloads (default: the workload's, "
                         "0 = the library's choice)")
    ap.add_argument("--bwd-splits", type=int, default=None,
                    help="head parts of the dK/dV pass for fa_bwd_ex workloads (default: "
                         "the library's choice)")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="calls after the timed steps, each preceded by a 512 MiB read that "
                         "flushes the caches; "
                         "their median duration is roofline.kernel_ms_cold_median (0: skip)")
    ap.add_argument("--no-mfma-loop", action="store_true",
                    help="skip the MFMA-loop rate (roofline.mfma_loop_tflops: independent "
                         "32x32 MFMAs on every SIMD, measured after the timed steps)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of attention, run a plain device copy of this many bytes "
                         "(calibrates the HBM traffic counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the forward pass has no multi-GPU path "
              "in this library (heads shard across GPUs with no exchange).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from exact_attention_13_amd import binding
    from exact_attention_13_amd.inputs import WORKLOADS, make_inputs, make_upstream

    if args.copy_bytes:
        n = args.copy_bytes // 4
        src = torch.rand(n, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n * 4, "launches": max(1, args.steps)}), flush=True)
        return

    if args.read_bytes:
        x = torch.ones(args.read_bytes // 4, dtype=torch.float32, device="cuda:0")
        for _ in range(max(1, args.warmup)):
            x.sum()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(max(1, args.steps)):
            x.sum()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / max(1, args.steps)
        print(json.dumps({"read_bytes": x.numel() * 4, "ms": round(ms, 5),
                          "GB/s": round(x.numel() * 4 / (ms * 1e-3) / 1e9, 1)}), flush=True)
        return

    binding.load()  # fails loudly when libfa.so is missing
    w = WORKLOADS[args.workload]
    if args.splits is not None:
        w = w.with_(splits=args.splits)
    q, k, v = make_inputs(w)
    # SHA-256 of each input's stored bits (host copy, first 16 hex digits):
    # identifies the exact synthetic tensors a run used
    input_sha = {n: hashlib.sha256(t.contiguous().view(torch.uint8).numpy().tobytes()).hexdigest()[:16]
                 for n, t in zip("qkv", (q, k, v))}
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    splits, workspace = 1, None
    if args.which == "bwd":
        dout_h = make_upstream(w, w.seed + 100)
        input_sha["dO"] = hashlib.sha256(
            dout_h.contiguous().view(torch.uint8).numpy().tobytes()).hexdigest()[:16]
        dout = dout_h.to(dev)
        if w.extended:
            binding.fwd_ex(qd, kd, vd, w.scale, w.causal, out=o, lse=lse, stream=stream)
        else:
            binding.fwd(qd, kd, vd, w.scale, w.causal, out=o, lse=lse, stream=stream)
        grads = [torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)]
        delta = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        dt_code = {"f32": binding.FA_F32, "bf16": binding.FA_BF16, "f16": binding.FA_F16}[w.dtype]
        ptrs = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), dout.data_ptr(),
                lse.data_ptr(), *(t.data_ptr() for t in grads), delta.data_ptr())

        if w.extended:
            splits = args.bwd_splits or binding.bwd_default_splits(
                w.B, w.H, w.h_kv, w.N, w.n_kv, w.d, w.causal, dt_code)
            need = binding.bwd_workspace_bytes(w.B, w.H, w.h_kv, w.N, w.n_kv, w.d, splits)
            if need > 0:
                workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        ws_ptr = workspace.data_ptr() if workspace is not None else None
        ws_bytes = workspace.numel() if workspace is not None else 0

        def step():
            if w.extended:
                st = binding.fa_bwd_ex(*ptrs, w.B, w.H, w.h_kv, w.N, w.n_kv, w.d, w.scale,
                                       w.causal, dt_code, splits, ws_ptr, ws_bytes,
                                       stream.cuda_stream)
            else:
                st = binding.fa_bwd(*ptrs, w.B, w.H, w.N, w.d, w.scale, w.causal, dt_code,
                                    stream.cuda_stream)
            if st != 0:
                raise binding.FaError(st)
    elif w.extended:
        dt_code = {"f32": binding.FA_F32, "bf16": binding.FA_BF16, "f16": binding.FA_F16}[w.dtype]
        splits = w.splits or binding.default_splits(w.B, w.H, w.h_kv, w.N, w.n_kv, w.d,
                                                    w.causal, dt_code)
        need = binding.workspace_bytes(w.B, w.H, w.N, w.n_kv, w.d, splits)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)

        def step():
            binding.fwd_ex(qd, kd, vd, w.scale, w.causal, num_splits=splits, out=o, lse=lse,
                           workspace=workspace, stream=stream)
    else:
        def step():
            binding.fwd(qd, kd, vd, w.scale, w.causal, out=o, lse=lse, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Whole-job throughput: K steps between two synchronisations.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    enqueue_s = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # Kernel duration: HIP events on the launch stream around each of K more
    # launches.  They are queued behind a delay kernel that holds the stream
    # for longer than the host takes to enqueue them, so they run back to
    # back and each event pair brackets its launch rather than the host's
    # launch gap, which is longer than the shortest calls.  W untimed
    # launches between the delay and the timed ones bring the clock back up
    # after the near-idle delay.
    from exact_attention_13_amd import probe
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    per_launch_s = enqueue_s / max(1, args.steps)
    probe.delay(min(1000000, int(3e6 * per_launch_s * (args.steps + args.warmup)) + 2000), stream)
    for _ in range(args.warmup):
        step()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    kernel_ms = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    avg_kernel_ms = sum(kernel_ms) / len(kernel_ms)

    # Cold caches: reading a 512 MiB buffer between calls evicts the L2s and
    # the MALL (a read leaves no dirty lines to write back during the next
    # call), so K/V start from HBM; outside the timed steps.
    cold_ms = None
    if args.cold_steps > 0:
        flush = torch.ones(COLD_FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
        sink = torch.empty((), dtype=torch.int64, device=dev)
        cold = []
        for i in range(args.cold_steps):
            torch.sum(flush, dim=0, out=sink)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            step()
            b.record(stream)
            cold.append((a, b))
        torch.cuda.synchronize()
        cold_sorted = sorted(a.elapsed_time(b) for a, b in cold)
        cold_ms = round(cold_sorted[len(cold_sorted) // 2], 5)
        del flush, sink

    # The dense MFMA rate of a plain MFMA loop on this GPU, measured right
    # after the attention calls (same warm chip), for the FLOP-bound lines.
    mfma_loop = None
    if not args.no_mfma_loop:
        mfma_loop = probe.mfma_tflops(w.dtype, stream=stream)

    flops = w.flops * (2.5 if args.which == "bwd" else 1.0)
    value = flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    hbm_bound = args.which == "fwd" and flops / w.io_bytes < peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    if hbm_bound:
        achieved, peak, unit = w.io_bytes / (avg_kernel_ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        achieved, unit = flops / (avg_kernel_ms * 1e-3) / 1e12, "TFLOP/s"
    traffic = read_traffic(w.name, w.dtype) if args.which == "fwd" else None

    if args.which == "bwd":
        metric = f"bwd attention TFLOP/s (2.5x fwd FLOPs), workload {w.name}"
    else:
        metric = METRIC if w.name == "C4" else f"fwd attention TFLOP/s, workload {w.name}"
    out = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": f"synthetic: seeded ({w.dist}, numpy PCG64 seed {w.seed}) Q/K/V rounded to {w.dtype}",
        "config": {"workload": f"{w.name}: {w.dtype} B={w.B} H={w.H} N={w.N} d={w.d} "
                               f"{'causal' if w.causal else 'non-causal'}" + (
                                   (f" H_kv={w.h_kv} N_kv={w.n_kv} head_parts={splits} (fa_bwd_ex)"
                                    if args.which == "bwd" else
                                    f" H_kv={w.h_kv} N_kv={w.n_kv} splits={splits} (fa_fwd_ex)")
                                   if w.extended else ""),
                   "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "flops_per_step": flops, "parallelism": "single GPU",
                   "inputs_sha256": input_sha},
        "roofline": {"bound": "hbm" if hbm_bound else "mfma", "achieved": round(achieved, 2),
                     "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": traffic, "algorithmic_bytes": w.io_bytes,
                     "timed": (("fa_bwd_ex" if w.extended else "fa_bwd") +
                               (" call: row-dot, dK/dV, part-sum and dQ kernels" if splits > 1
                                else " call: row-dot, dK/dV and dQ kernels")
                               if args.which == "bwd"
                               else "fa_fwd_ex call: split kernel + combine kernel" if splits > 1
                               else "one forward kernel"),
                     "hbm_gbs": round(w.io_bytes / (avg_kernel_ms * 1e-3) / 1e9, 1),
                     "kernel_ms_avg": round(avg_kernel_ms, 5),
                     "kernel_ms_min": round(kernel_ms[0], 5),
                     "kernel_ms_median": round(kernel_ms[len(kernel_ms) // 2], 5),
                     "kernel_ms_cold_median": cold_ms},
    }
    if mfma_loop is not None and not hbm_bound:
        out["roofline"]["mfma_loop_tflops"] = round(mfma_loop, 1)
        out["roofline"]["frac_of_mfma_loop"] = round(achieved / mfma_loop, 4)
    if not args.no_cpu_baseline:
        if args.which == "bwd":
            out["cpu_baseline"] = cpu_baseline_bwd(w, q, k, v, dout.cpu(), args.cpu_seconds)
        else:
            out["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
