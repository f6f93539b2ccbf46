#!/usr/bin/env python3
"""Benchmark of the mask-only logits hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input, inputs
already resident in HBM: stream compaction of the token ids into idx (one launch),
read-back of the masked count M, then the fused gather-GEMM logits in row chunks of
max_num_logits rows (one launch per chunk).

Default workload: the logits-dominant long-context case -- L = 32768, d = 4096,
V = 126464 (LLaDA-8B's vocabulary), mask ratio 0.9 (M = 29491), 4096-row chunks,
bf16 inputs and logits, fp32 accumulation.  Prints ONE JSON line on stdout; details
go to stderr.

  value        whole-step TFLOP/s, counting 2*M*d*V per step
  roofline     the gather-GEMM kernel against the dense bf16 MFMA peak (2.5 PFLOP/s):
               achieved = (2*M*d*V of one step) / (GEMM time of one step), with the GEMM
               time measured by HIP events on the stream the kernels run on
  cpu_baseline the CPU oracle (fp64, OpenMP) timed on a bounded sample of rows

Warm-up (untimed): by default at least WARMUP_MIN_STEPS steps and at least
WARMUP_MIN_SECONDS of work.  The clock of a chip that was idle takes some tens of
milliseconds to settle under this load (the first launches of a run are up to 25%
off the steady rate), so a fixed count of 1-ms steps would time that transient
instead of the steady state.  --warmup N runs exactly N steps instead.

--path selects what the step does after compaction (default: logits):
  logits        the bf16 logits of every masked row, stored ([M, V])
  argmax_lse    each masked row reduced in the kernel to (max, first argmax,
                log-sum-exp); no logits buffer exists
  dense_select  the baseline the pages contrast with: logits of all L rows with the
                same kernel and chunking, then the masked rows copied out; `value`
                still counts only 2*M*d*V, so it compares directly with `logits`
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

METRIC = "mask-only logits TFLOP/s (2·M·d·V) and % bf16 MFMA peak at L=32k, d=4096"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
LOWM_VARIANTS = (20,)
DEVICE_COUNT_VARIANT = 22   # the kernel mosaic_masked_logits_device_count runs
WARMUP_MIN_STEPS = 3
WARMUP_MIN_SECONDS = 0.15


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def code_lines(text: str):
    """The lines of a C/C++ source that carry code: comments and blank lines removed."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    out = []
    for line in text.splitlines():
        line = line.split("//", 1)[0].rstrip()
        if line.strip():
            out.append(line)
    return out


def kernel_source_hash(path: str = "logits") -> str:
    """Hash of the code lines of the sources the path's kernels are built from, so that a
    measured traffic figure stays attached to the code it was measured on (comment edits
    keep it): the FP8 kernels for the fp8 path, the bf16/fp32 kernels for the others,
    and the C ABI and launcher header for all."""
    h = hashlib.sha256()
    kernels = "gather_gemm_fp8.hip" if path == "fp8" else "gather_gemm.hip"
    for f in (kernels, "lowm_epilogue.h", "mosaic_abi.cpp", "launch.h"):
        with open(os.path.join(ROOT, "mask_only_logits_amd", "csrc", f), encoding="utf-8") as fh:
            for line in code_lines(fh.read()):
                h.update(line.encode() + b"\n")
    return h.hexdigest()[:16]


def _profile_tag(workload: str, path: str) -> str:
    return workload if path == "logits" else f"{workload}_{path}"


def measured_traffic(workload: str, path: str = "logits", prof_dir: str | None = None):
    """L2-miss (L2-to-fabric) bytes per GEMM launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None.  FETCH_SIZE and
    WRITE_SIZE count what the L2 requests from and sends to the fabric: Infinity-Cache
    hits included, so this is an upper bound on HBM bytes, not HBM bytes."""
    fname = os.path.join(prof_dir or os.path.join(ROOT, "profiles"),
                         f"traffic_gather_gemm_{_profile_tag(workload, path)}.json")
    try:
        with open(fname, encoding="utf-8") as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash(path):
        return None
    return t.get("bytes_per_launch")


def warm_up(step, n_fixed=None, min_steps=WARMUP_MIN_STEPS, min_seconds=WARMUP_MIN_SECONDS, sync=None,
            clock=time.perf_counter) -> int:
    """Run untimed steps; return how many ran.

    n_fixed: exactly that many.  Otherwise at least min_steps, and more until
    min_seconds of wall time have passed with the device synchronized after each step
    (so wall time is device time)."""
    if n_fixed is not None:
        for _ in range(n_fixed):
            step()
        if sync:
            sync()
        return n_fixed
    n, t0 = 0, clock()
    while n < min_steps or clock() - t0 < min_seconds:
        step()
        if sync:
            sync()
        n += 1
    return n


def host_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "affinity_cpus": len(os.sched_getaffinity(0)), "os_cpu_count": os.cpu_count()}


def cpu_baseline(wl, idx_np, target_s: float, path: str = "logits"):
    """Time the oracle on a bounded sample of masked rows (the first rows of idx)."""
    import oracle
    cores = oracle.num_threads()
    flop_row = 2.0 * wl.d * wl.V
    fn = oracle.masked_logits if path == "logits" else oracle.masked_logits_argmax_lse
    t0 = time.perf_counter()
    fn(wl.H, idx_np, wl.W, rows=list(range(2)))
    t_cal = max(1e-3, time.perf_counter() - t0) / 2
    n = int(max(2, min(len(idx_np), target_s / t_cal)))
    rows = list(range(n))
    t0 = time.perf_counter()
    fn(wl.H, idx_np, wl.W, rows=rows)
    dt = time.perf_counter() - t0
    return {"value": round(n * flop_row / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} of {len(idx_np)} masked rows x all {wl.V} vocabulary rows of the same workload "
                      f"(fp64, ascending k{'' if path == 'logits' else ', then max / argmax / log-sum-exp'}), "
                      f"{dt:.1f} s"}


def cpu_per_core(wl, idx_np, path: str = "logits"):
    """The oracle on one thread over one masked row: the per-core rate beside the all-core
    cpu_baseline."""
    import oracle
    cores = oracle.num_threads()
    fn = oracle.masked_logits if path == "logits" else oracle.masked_logits_argmax_lse
    oracle.set_num_threads(1)
    try:
        t0 = time.perf_counter()
        fn(wl.H, idx_np, wl.W, rows=[0])
        t1 = max(1e-4, time.perf_counter() - t0)
        n = int(max(1, min(len(idx_np), 0.5 / t1)))   # about half a second of one core
        t0 = time.perf_counter()
        fn(wl.H, idx_np, wl.W, rows=list(range(n)))
        dt = time.perf_counter() - t0
    finally:
        oracle.set_num_threads(cores)
    return {"value": round(n * 2.0 * wl.d * wl.V / dt / 1e12, 6), "unit": "TFLOP/s", "threads": 1,
            "sample": f"{n} masked rows x all {wl.V} vocabulary rows, {dt:.2f} s"}


def _read_csv(path):
    import csv
    with open(path, newline="", encoding="utf-8") as fh:
        return list(csv.DictReader(fh))


def _find(root, suffix):
    out = []
    for dirpath, _, files in os.walk(root):
        out += [os.path.join(dirpath, f) for f in files if f.endswith(suffix)]
    return sorted(out)


def _roofline_from_log(log_file: str) -> dict:
    """The roofline object of the last JSON result line in a bench log ({} if none)."""
    try:
        with open(log_file, encoding="utf-8") as fh:
            js = [ln for ln in fh if ln.startswith("{")]
        return json.loads(js[-1]).get("roofline", {}) if js else {}
    except (OSError, ValueError):
        return {}


def summarize_profile(root: str, workload: str, copy_mib: int, path: str = "logits", prof_dir: str | None = None):
    """Write profiles/ summaries from rocprofv3 output under `root`: kernel_stats
    (--kernel-trace --stats) and counter_collection (--pmc) CSV files.  `root/commands.txt`,
    if present, holds the rocprofv3 command lines that produced them; it is copied in.
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what they read for the
    copy probe of `copy_mib` MiB, a kernel that reads and writes exactly that much."""
    prof = prof_dir or os.path.join(ROOT, "profiles")
    os.makedirs(prof, exist_ok=True)
    stats = _find(root, "kernel_stats.csv")
    counters = _find(root, "counter_collection.csv")
    tag = _profile_tag(workload, path)
    lines = [f"# rocprofv3 summary: gather-GEMM on workload {workload}"
             + ("" if path == "logits" else f" ({path} path: logits reduced per row, not stored)"), ""]
    cmd_file = os.path.join(root, "commands.txt")
    if os.path.exists(cmd_file):
        lines += ["Commands (run from the repository root):", "```"]
        lines += [ln.rstrip() for ln in open(cmd_file, encoding="utf-8") if ln.strip()]
        lines += ["```", ""]
    for f in stats:
        rows = _read_csv(f)
        lines.append(f"## {os.path.relpath(f, root)}")
        lines.append("| kernel | calls | total ms | avg us | min us | max us | % |")
        lines.append("|---|---|---|---|---|---|---|")
        for r in rows:
            lines.append("| {} | {} | {:.3f} | {:.1f} | {:.1f} | {:.1f} | {:.2f} |".format(
                r["Name"][:90], r["Calls"], float(r["TotalDurationNs"]) / 1e6, float(r["AverageNs"]) / 1e3,
                float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
        lines.append("")
    per_kernel = {}
    for f in counters:
        for r in _read_csv(f):
            name = r.get("Kernel_Name", "")
            key = ("gather_gemm" if "gather_gemm_" in name and "simple" not in name else
                   "copy" if "MulFunctor" in name or "AUnaryFunctor" in name else None)
            if key is None:
                continue
            c = r["Counter_Name"]
            per_kernel.setdefault(key, {}).setdefault(c, []).append(float(r["Counter_Value"]))
    if per_kernel:
        lines.append("## counters (mean per dispatch)")
        lines.append("| kernel | counter | dispatches | mean | ")
        lines.append("|---|---|---|---|")
        for k, cs in sorted(per_kernel.items()):
            for c, v in sorted(cs.items()):
                lines.append(f"| {k} | {c} | {len(v)} | {sum(v) / len(v):.6g} |")
        lines.append("")
    traffic = None
    g, cp = per_kernel.get("gather_gemm", {}), per_kernel.get("copy", {})
    if g.get("FETCH_SIZE") and g.get("WRITE_SIZE") and cp.get("FETCH_SIZE") and cp.get("WRITE_SIZE"):
        known = copy_mib * (1 << 20)
        f_scale = known / (sum(cp["FETCH_SIZE"]) / len(cp["FETCH_SIZE"]) * 1024)
        w_scale = known / (sum(cp["WRITE_SIZE"]) / len(cp["WRITE_SIZE"]) * 1024)
        fetch = sum(g["FETCH_SIZE"]) / len(g["FETCH_SIZE"]) * 1024 * f_scale
        write = sum(g["WRITE_SIZE"]) / len(g["WRITE_SIZE"]) * 1024 * w_scale
        # the hash of the sources the traced run was built from (as it reported it), so that
        # summarising old output after a source change cannot attach it to the new code
        traced = _roofline_from_log(os.path.join(root, "trace.log"))
        traffic = {"kernel_source_hash": traced.get("kernel_source_hash"), "workload": workload, "path": path,
                   "bytes_per_launch": int(fetch + write), "fetch_bytes_per_launch": int(fetch),
                   "write_bytes_per_launch": int(write), "fetch_scale": f_scale, "write_scale": w_scale,
                   "copy_probe_bytes": known}
        with open(os.path.join(prof, f"traffic_gather_gemm_{tag}.json"), "w", encoding="utf-8") as fh:
            json.dump(traffic, fh, indent=1)
        lines.append(f"L2-miss (L2-to-fabric, Infinity-Cache hits included) traffic per GEMM launch, scaled by "
                     f"the copy probe: fetch {fetch / 1e9:.3f} GB, write {write / 1e9:.3f} GB "
                     f"(scales {f_scale:.4f}, {w_scale:.4f})")
        alg = traced.get("algorithmic_bytes_per_launch")
        if alg:
            lines.append(f"Algorithmic bytes per launch (from the traced run's JSON line): {alg / 1e9:.3f} GB; "
                         f"L2-miss / algorithmic = {(fetch + write) / alg:.2f}")
    out = os.path.join(prof, f"gather_gemm_{tag}_rocprof.md")
    with open(out, "w", encoding="utf-8") as fh:
        fh.write("\n".join(lines) + "\n")
    log(f"[bench] wrote {out}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before the timed ones (default: at least %d steps and %.2f s of work)"
                         % (WARMUP_MIN_STEPS, WARMUP_MIN_SECONDS))
    ap.add_argument("--workload", default="long_logits")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--count-on-host", action="store_true",
                    help="single-launch logits and argmax_lse workloads: read the masked count back to the "
                         "host before the GEMM (mosaic_masked_logits, mosaic_masked_logits_argmax_lse) instead "
                         "of letting the kernel read it on the device (mosaic_masked_logits_device_count, "
                         "mosaic_masked_logits_argmax_lse_device_count: the default there)")
    ap.add_argument("--profile-copy-mib", type=int, default=0,
                    help="after the timed steps, run a plain elementwise copy of this many MiB three times "
                         "(a kernel of known traffic that calibrates rocprofv3's FETCH_SIZE/WRITE_SIZE)")
    ap.add_argument("--flush-mib", type=int, default=-1,
                    help="after the timed steps, time as many again with a cache-evicting pass over a buffer of "
                         "this many MiB before each (reported under detail.flushed); default: 512 for the "
                         "HBM-bound low-M kernel, else off")
    ap.add_argument("--compare-vendor", action="store_true",
                    help="after the timed steps, time the vendor GEMM (torch.mm, i.e. hipBLASLt) on the same "
                         "chunks of the masked rows, gathered into a dense matrix beforehand (reported under "
                         "detail.vendor_gemm; bf16 logits path only)")
    ap.add_argument("--summarize-profile", metavar="DIR",
                    help="summarize rocprofv3 CSV output found under DIR into profiles/ and exit")
    ap.add_argument("--path", choices=("logits", "argmax_lse", "dense_select", "fp8"), default="logits",
                    help="logits: store the bf16 logits of every masked row (default); argmax_lse: reduce each "
                         "row to (max, first argmax, log-sum-exp) inside the kernel and store no logits; "
                         "dense_select: the baseline the pages contrast with -- logits of ALL L rows with the "
                         "same kernel and chunking, then the masked rows copied out (value counts only the "
                         "masked rows' 2*M*d*V, so it compares directly with the logits path); fp8: the FP8 "
                         "(E4M3, per-row scales) LM head with W quantized beforehand")
    args = ap.parse_args()

    if args.summarize_profile:
        summarize_profile(args.summarize_profile, args.workload, args.profile_copy_mib or 1024, args.path)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the path is a single-GPU kernel library); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from mask_only_logits_amd import inputs
    from mask_only_logits_amd import mosaic

    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    wl = inputs.make_workload(args.workload)
    log(f"[bench] inputs {args.workload}: L={wl.L} d={wl.d} V={wl.V} in {time.perf_counter() - t0:.1f}s")
    tokens = wl.tokens.to(dev)
    H = wl.H.to(dev)
    W = wl.W.to(dev)
    seq_offsets = wl.seq_offsets.to(dev) if wl.seq_offsets is not None else None
    out_dtype = torch.float32 if wl.out_dtype == "f32" else torch.bfloat16
    L, d, V = wl.L, wl.d, wl.V
    idx = torch.empty(L, dtype=torch.int32, device=dev)
    cnt = torch.empty(max(2, wl.nseq + 1), dtype=torch.int32, device=dev)

    stream = torch.cuda.current_stream()

    # Count once to size the output; every step recomputes it.
    if seq_offsets is not None:
        mosaic.mosaic_mask_compact_batched(tokens, seq_offsets, wl.mask_id, idx=idx, idx_offsets=cnt[: wl.nseq + 1])
        M = int(cnt[wl.nseq].item())
    else:
        mosaic.mosaic_mask_compact(tokens, wl.mask_id, idx=idx, count=cnt[:1])
        M = int(cnt[0].item())
    C = wl.chunk_rows
    launches = mosaic.mosaic_num_chunks(M, C)
    flop = 2.0 * M * d * V
    rows_per_launch = M if launches == 1 else C
    consumer = args.path == "argmax_lse"
    dense = args.path == "dense_select"
    fp8 = args.path == "fp8"
    if fp8:
        if wl.dtype != "bf16" or d % 128:
            log(f"[bench] the fp8 path needs bf16 inputs and d % 128 == 0 ({args.workload} has not)")
            sys.exit(2)
        out = torch.empty((M, V), dtype=torch.bfloat16, device=dev)
        Wq, wsc = mosaic.mosaic_quantize_rows_fp8(W)          # the weights, quantized once
        ws8 = torch.empty(max(16, mosaic.mosaic_logits_fp8_workspace_bytes(M, C, d)), dtype=torch.uint8,
                          device=dev)
        variant = None
        log(f"[bench] M={M} chunk_rows={C} launches={launches} path=fp8 (E4M3 per-row scales) "
            f"out={out.numel() * 2 / 1e9:.2f} GB")
    elif dense:
        out = torch.empty((M, V), dtype=out_dtype, device=dev)
        full = torch.empty((L, V), dtype=out_dtype, device=dev)
        all_rows = torch.arange(L, dtype=torch.int32, device=dev)
        sel = torch.empty(M, dtype=torch.int64, device=dev)
        launches = mosaic.mosaic_num_chunks(L, C)
        variant = mosaic.mosaic_logits_variant(L if launches == 1 else C, V, d, H.dtype, out_dtype)
        log(f"[bench] M={M} L={L} chunk_rows={C} launches={launches} path=dense_select variant={variant} "
            f"peak logits={(full.numel() + out.numel()) * out.element_size() / 1e9:.2f} GB")
    elif consumer:
        if wl.dtype != "bf16" or d % 64:
            log(f"[bench] the argmax_lse path needs bf16 inputs and d % 64 == 0 ({args.workload} has not)")
            sys.exit(2)
        out = None
        rmax = torch.empty(M, dtype=torch.float32, device=dev)
        rarg = torch.empty(M, dtype=torch.int32, device=dev)
        rlse = torch.empty(M, dtype=torch.float32, device=dev)
        ws = torch.empty(max(16, mosaic.mosaic_logits_argmax_lse_workspace_bytes(M, C, V)),
                         dtype=torch.uint8, device=dev)
        variant = None
        log(f"[bench] M={M} chunk_rows={C} launches={launches} path=argmax_lse (no logits stored) "
            f"workspace={ws.numel() / 1e6:.1f} MB")
    else:
        out = torch.empty((M, V), dtype=out_dtype, device=dev)
        variant = mosaic.mosaic_logits_variant(rows_per_launch, V, d, H.dtype, out_dtype)
        log(f"[bench] M={M} chunk_rows={C} launches={launches} variant={variant} "
            f"out={out.numel() * out.element_size() / 1e9:.2f} GB")
    # One launch on the default persistent kernel (logits, or the per-row consumer): the
    # kernel reads the count the compaction left in device memory, so the step has no
    # device-to-host read-back (the output buffers were sized once, from the first count, as a
    # denoising loop whose masked set only shrinks can do).
    count_on_device = (launches == 1 and not args.count_on_host and
                       ((args.path == "logits" and variant == DEVICE_COUNT_VARIANT) or consumer))

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]

    def step(i=None):
        if i is not None:
            ev[i][0].record(stream)
        if seq_offsets is not None:
            mosaic.mosaic_mask_compact_batched(tokens, seq_offsets, wl.mask_id, idx=idx,
                                               idx_offsets=cnt[: wl.nseq + 1], stream=stream)
            cdev = cnt[wl.nseq: wl.nseq + 1]
        else:
            mosaic.mosaic_mask_compact(tokens, wl.mask_id, idx=idx, count=cnt[:1], stream=stream)
            cdev = cnt[:1]
        m = M if count_on_device else int(cdev.item())     # device -> host: sizes the GEMM
        if i is not None:
            ev[i][1].record(stream)
        if consumer and count_on_device:
            mosaic.mosaic_masked_logits_argmax_lse_device_count(H, idx, W, cdev, max_rows=M, row_max=rmax,
                                                                row_argmax=rarg, row_lse=rlse, workspace=ws,
                                                                stream=stream)
        elif consumer:
            mosaic.mosaic_masked_logits_argmax_lse(H, idx, W, M=m, chunk_rows=C, row_max=rmax, row_argmax=rarg,
                                                   row_lse=rlse, workspace=ws, stream=stream)
        elif fp8:
            mosaic.mosaic_masked_logits_fp8(H, idx, Wq, wsc, M=m, out=out, chunk_rows=C, workspace=ws8,
                                            stream=stream)
        elif dense:
            mosaic.mosaic_masked_logits(H, all_rows, W, M=L, out=full, chunk_rows=C, stream=stream)
            sel.copy_(idx[:m])
            torch.index_select(full, 0, sel, out=out)
        elif count_on_device:
            mosaic.mosaic_masked_logits_device_count(H, idx, W, cdev, max_rows=M, out=out, stream=stream)
        else:
            mosaic.mosaic_masked_logits(H, idx, W, M=m, out=out, chunk_rows=C, stream=stream)
        if i is not None:
            ev[i][2].record(stream)
        return m

    n_warmup = warm_up(step, args.warmup, sync=torch.cuda.synchronize)
    log(f"[bench] warm-up: {n_warmup} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        assert step(i) == M
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if count_on_device:   # the count the kernels read (checked after the timed region)
        assert int((cnt[wl.nseq] if seq_offsets is not None else cnt[0]).item()) == M
    ms_per_step = wall * 1e3 / args.steps
    gemm_ms = [a[1].elapsed_time(a[2]) for a in ev]
    compact_ms = [a[0].elapsed_time(a[1]) for a in ev]
    gemm_avg = float(np.mean(gemm_ms))
    gemm_median = float(np.median(gemm_ms))
    value = flop / (ms_per_step / 1e3) / 1e12
    # the kernel's own FLOP: the dense baseline multiplies all L rows
    achieved = (2.0 * L * d * V if dense else flop) / (gemm_avg / 1e3) / 1e12
    log(f"[bench] {ms_per_step:.3f} ms/step ({value:.1f} TFLOP/s); GEMM {gemm_avg:.3f} ms/step "
        f"(min {min(gemm_ms):.3f}) = {achieved:.1f} TFLOP/s = "
        f"{achieved / (PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS):.1%} of {'fp8' if fp8 else 'bf16'} peak; "
        f"{gemm_avg / launches:.3f} ms per launch; compaction+readback {np.mean(compact_ms) * 1e3:.1f} us")

    esize_in = 2 if wl.dtype == "bf16" else 4
    peak = PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS
    out_bytes = M * 12 if consumer else M * V * out.element_size()
    alg_bytes = launches * V * d * esize_in + M * d * esize_in + out_bytes + M * 4
    if fp8:
        # W codes once per chunk + gathered H rows (bf16, quantized per chunk) + codes + out
        alg_bytes = launches * V * d + M * d * 2 + M * V * 2 + M * 4
    if dense:
        # the dense baseline's own work: all L rows
        alg_bytes = launches * V * d * esize_in + L * d * esize_in + (L + 2 * M) * V * out.element_size()
    traffic = measured_traffic(args.workload, args.path)
    fp8_lowm = fp8 and rows_per_launch <= 64 and "fp8lowm=0" not in os.environ.get("MOSAIC_TUNE", "")
    kernel = ("gather_gemm_fp8_lowm_kernel" if fp8_lowm else "gather_gemm_fp8_kernel") if fp8 else \
        "gather_gemm_bf16_defer_kernel" if consumer else {
            0: "gather_gemm_f32_kernel", 2: "gather_gemm_bf16_simple_kernel", 11: "gather_gemm_bf16_persist_kernel",
            12: "gather_gemm_bf16_kernel", 16: "gather_gemm_bf16_defer_kernel", 19: "gather_gemm_bf16_defer_kernel",
            21: "gather_gemm_bf16_defer_kernel", 22: "gather_gemm_bf16_defer_kernel",
            20: "gather_gemm_lowm_shared_kernel"}.get(variant, "gather_gemm")
    if variant in LOWM_VARIANTS or fp8_lowm:
        # streaming W is the bound: algorithmic bytes per launch over the launch time
        achieved_gbs = alg_bytes / launches / (gemm_avg / launches / 1e3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(achieved_gbs / PEAK_HBM_GBS, 4), "traffic": traffic}
    else:
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(achieved / peak, 4), "traffic": traffic}
    roofline.update({"kernel": kernel, "launch_ms_avg": round(gemm_avg / launches, 4),
                     "algorithmic_bytes_per_launch": int(alg_bytes / launches),
                     "algorithmic_flop_per_launch": int(flop / launches),
                     "traffic_kind": "L2-miss bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a copy "
                                     "probe; Infinity-Cache hits included, so an upper bound on HBM bytes)",
                     "traffic_over_algorithmic": (round(traffic / (alg_bytes / launches), 3)
                                                  if traffic is not None else None),
                     "kernel_source_hash": kernel_source_hash(args.path)})
    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": n_warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 (e4m3)" if fp8 else ("bf16" if wl.dtype == "bf16" else "f32"),
        "data": "synthetic (seeded Gaussian H ~ N(0,1), W ~ N(0,0.02); uniform masked positions)",
        "config": {"workload": args.workload, "L": L, "d": d, "V": V, "M": M, "chunk_rows": C,
                   "launches_per_step": launches, "in_dtype": wl.dtype,
                   "out_dtype": "per-row f32 max / i32 argmax / f32 lse" if consumer else wl.out_dtype,
                   "accumulate": "fp32", "path": args.path,
                   "count": "device (no read-back)" if count_on_device else "host (read back before the GEMM)"},
        "roofline": roofline,
        "detail": {"gemm_ms_per_step": round(gemm_avg, 4), "gemm_ms_median": round(gemm_median, 4),
                   "gemm_ms_min": round(min(gemm_ms), 4),
                   "compaction_readback_us": round(float(np.mean(compact_ms)) * 1e3, 2),
                   # logits buffers alive at once: [L, V] + the selected [M, V] (dense_select),
                   # the [M, V] output (logits), none (argmax_lse)
                   "peak_logits_bytes": int((L * V + M * V) * out.element_size()) if dense else
                   (0 if consumer else int(M * V * out.element_size()))},
    }
    flush_mib = args.flush_mib if args.flush_mib >= 0 else (512 if variant in LOWM_VARIANTS or fp8_lowm else 0)
    if flush_mib:
        # W no longer partly in the caches from the previous step: read a buffer larger than
        # the Infinity Cache before each step, outside the GEMM events (a read, so the flush
        # leaves no dirty lines to be written back during the GEMM)
        fl = torch.ones(flush_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
        fsum = torch.empty((), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        fms = []
        for i in range(args.steps):
            torch.sum(fl, dim=0, dtype=torch.float32, out=fsum)
            step(i)
            torch.cuda.synchronize()
            fms.append(ev[i][1].elapsed_time(ev[i][2]))
        del fl
        fmed = float(np.median(fms))
        result["detail"]["flushed"] = {"flush_mib": flush_mib, "gemm_ms_median": round(fmed, 4),
                                       "gemm_ms_min": round(min(fms), 4)}
        if variant in LOWM_VARIANTS or fp8_lowm:
            result["detail"]["flushed"]["achieved_gbs"] = round(alg_bytes / (fmed / 1e3) / 1e9, 1)
        else:
            result["detail"]["flushed"]["achieved_tflops"] = round(flop / (fmed / 1e3) / 1e12, 2)
        log(f"[bench] with a {flush_mib} MiB cache flush before each step: GEMM median {fmed:.3f} ms")

    if args.compare_vendor:
        if wl.dtype != "bf16" or args.path != "logits":
            log("[bench] --compare-vendor times the bf16 logits path only")
        else:
            # The vendor's dense GEMM on the same chunks.  The masked rows are gathered into a
            # dense matrix beforehand, outside the timing, so it does neither the gather nor
            # the compaction: a reference for the GEMM, not an implementation of the path.
            Hg = H[idx[:M].long()].contiguous()
            Wt = W.t()
            rows_c = M if launches == 1 else C
            vout = torch.empty((rows_c, V), dtype=torch.bfloat16, device=dev)

            def vstep():
                for r0 in range(0, M, rows_c):
                    r1 = min(M, r0 + rows_c)
                    torch.mm(Hg[r0:r1], Wt, out=vout[: r1 - r0])

            warm_up(vstep, args.warmup, sync=torch.cuda.synchronize)
            va, vb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            va.record()
            for _ in range(args.steps):
                vstep()
            vb.record()
            torch.cuda.synchronize()
            vms = va.elapsed_time(vb) / args.steps
            vtf = flop / (vms / 1e3) / 1e12
            result["detail"]["vendor_gemm"] = {
                "kernel": "torch.mm (hipBLASLt) on the masked rows gathered beforehand, same chunks",
                "ms_per_step": round(vms, 4), "tflops": round(vtf, 1),
                "gemm_over_vendor": round(achieved / vtf, 4)}
            log(f"[bench] vendor GEMM on pre-gathered rows: {vms:.3f} ms/step = {vtf:.1f} TFLOP/s "
                f"(this GEMM {achieved / vtf:.3f} of it)")
            del Hg, vout

    if args.profile_copy_mib:
        n = args.profile_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)      # reads and writes exactly n * 4 bytes
        torch.cuda.synchronize()
        del src, dst
        log(f"[bench] copy probe: 3 x {args.profile_copy_mib} MiB read + write")

    if fp8 and not args.no_cpu_baseline:
        log("[bench] no cpu_baseline on the fp8 path (its oracle would first quantize all of W)")
        args.no_cpu_baseline = True
    if not args.no_cpu_baseline:
        idx_np = idx[:M].cpu().numpy()
        log("[bench] timing the CPU oracle on a row sample ...")
        result["cpu_baseline"] = cpu_baseline(wl, idx_np, args.cpu_seconds, args.path)
        result["detail"]["cpu_per_core"] = cpu_per_core(wl, idx_np, args.path)
        result["detail"]["host"] = host_info()
        log(f"[bench] cpu_baseline {result['cpu_baseline']}")
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
