#!/usr/bin/env python3
"""Throughput of the fused KroQuant transform + MXFP4 quantizer on one MI355X.

One step = one kq_transform_quant call over one 4608 x 3072 bf16 activation
(the FLUX attention-projection input shape): every 32-channel block is
multiplied by its Kronecker-structured 32x32 transform and quantized to MXFP4.

Inputs are seeded synthetic data (mxfp4_activation_quantizer_amd.inputs),
copied to the GPU before timing.  Steps rotate over several buffer sets whose
total exceeds twice the 256 MB Infinity Cache, so every step reads its input
from HBM, not from a cache that the previous step warmed.

Prints one JSON line.  `value` is GB/s of algorithmic traffic (2 B read +
0.5 B + 1/32 B written per element) over the timed region: W untimed warmup
steps, then exactly K steps bracketed by synchronisations, timed with HIP
events on the stream the kernels run on.  The line also carries the roofline
of the kernel, the CPU oracle timed on the host, and the same-traffic peers
(per-channel scaling, FWHT32, a copy ceiling) on the same input.  Before any
timing, untimed launches run for 0.3 s so that the clocks have settled.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
PEAK_FP4_TFLOPS = 10100.0      # MI355X dense MXFP4 matrix peak
MALL_BYTES = 256 << 20         # Infinity Cache
ADALN_MAX_D = 8192             # channels the AdaLN-fused kernel accepts
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "mxfp4_activation_quantizer_amd", "csrc")


# The files the quantizer kernel is built from: a counter summary stays valid
# until one of them changes.
QUANT_SOURCES = ("kq_quant.hip", "kq_kron.h", "kq_device.h", "kq_host.h", "Makefile")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in QUANT_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str, src_hash: str):
    """HBM bytes per launch from a committed counter summary, or None when
    there is none or the kernel sources changed since it was taken."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != src_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


KERNEL_MATCH = {
    "kq_transform_quant": "KronStage, kq::Mxfp4Sink",
    "kq_transform_quant_mfma": "kron_mfma_kernel",
    "kq_transform_quant_quad": "kron_quad_kernel",
    "kq_smooth_quant": "SmoothStage, kq::Mxfp4Sink",
    "kq_fwht32_quant": "FwhtStage, kq::Mxfp4Sink",
    "kq_copy_ceiling": "IdentityStage, kq::FoldSink",
    "kq_stream_ceiling (read + write)": "stream_kernel<true>",
    "kq_stream_ceiling (read only)": "stream_kernel<false>",
    "kq_dequant_inverse": "KronInverseStage, kq::Bf16Sink",
    "kq_weight_quant": "KronWeightStage, kq::Mxfp4Sink",
    "kq_w4a4_gemm": ("w4a4_gemm_", "gemm_wide_kernel"),  # per-tile, pipelined, 256 x 256
    "kq_adaln_transform_quant": "adaln_kernel<1, true>",
    "kq_adaln_modulate": "adaln_kernel<1, false>",
    "kq_calib_objective": "calib_objective_kernel",
    "kq_calib_es_update": "calib_es_update_kernel",
    "kq_calib_es_step": "calib_es_step_kernel",
}

PROFILE_COMMANDS = """\
cd /tmp && export TMPDIR=/tmp; cd $REPO
python3 bench.py --json-out OUT/bench.json
rocprofv3 --kernel-trace --stats --output-format csv -d OUT/trace -o trace -- python3 bench.py --steps 200 --warmup 50 --no-cpu --no-other-workloads
rocprofv3 --kernel-trace --stats --output-format csv -d OUT/trace_q -o trace_q -- python3 bench.py --kernel-only --steps 200 --warmup 50 --json-out OUT/trace_q.json
rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/FETCH_SIZE -o FETCH_SIZE -- python3 bench.py --kernel-only --steps 20 --warmup 5
rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/WRITE_SIZE -o WRITE_SIZE -- python3 bench.py --kernel-only --steps 20 --warmup 5
rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/copy_FETCH_SIZE -o copy_FETCH_SIZE -- python3 bench.py --copy-calibration --steps 20
rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/copy_WRITE_SIZE -o copy_WRITE_SIZE -- python3 bench.py --copy-calibration --steps 20
rocprofv3 --pmc SQ_WAVES SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_BUSY_CYCLES --output-format csv -d OUT/SQ -o SQ -- python3 bench.py --kernel-only --steps 20 --warmup 5
rocprofv3 --pmc SQ_WAVES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES --output-format csv -d OUT/SQ_mfma -o SQ_mfma -- python3 bench.py --kernel-only --kernel kq_transform_quant_mfma --steps 20 --warmup 5
rocprofv3 --pmc SQ_WAVES SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_BUSY_CYCLES --output-format csv -d OUT/SQ_quad -o SQ_quad -- python3 bench.py --kernel-only --kernel kq_transform_quant_quad --steps 20 --warmup 5
rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/FETCH_quad -o FETCH_quad -- python3 bench.py --kernel-only --kernel kq_transform_quant_quad --steps 20 --warmup 5
rocprofv3 --pmc SQ_WAVES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_BUSY_CYCLES --output-format csv -d OUT/SQ_gemm -o SQ_gemm -- python3 bench.py --kernel-only --kernel kq_w4a4_gemm --steps 20 --warmup 5
rocprofv3 --pmc SQ_WAVES SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_BUSY_CYCLES --output-format csv -d OUT/SQ_adaln -o SQ_adaln -- python3 bench.py --kernel-only --kernel kq_adaln_transform_quant --steps 20 --warmup 5
python3 bench.py --summarize-profiles OUT"""


def oracle_peer_times(oracle, workload: str, x_bits, lu, mult, threads: int) -> dict:
    """The oracle function of each peer entry point timed on a bounded
    sample of the same workload (median of 3 runs on ``threads`` threads),
    in the unit the peer reports: GB/s of its algorithmic bytes, GFLOP/s for
    the GEMM.  Reported beside the GPU figures; never a target."""
    import numpy as np
    from mxfp4_activation_quantizer_amd import inputs
    w = inputs.WORKLOADS[workload]
    d = w.d
    rows = min(1024, w.tokens)
    xs = x_bits[:rows]
    elem = rows * d
    bpe = 2 + 0.5 + 1 / 32  # bytes per element, both directions

    def med(fn):
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return sorted(ts)[1]

    def rec(value, unit, sample):
        return {"value": round(value, 4), "unit": unit, "threads": threads, "sample": sample}

    out = {}
    tag = f"first {rows} rows of {workload}"
    t = med(lambda: oracle.smooth_quant(xs, mult, threads=threads))
    out["smooth_quant"] = rec(elem * bpe / t / 1e9, "GB/s", tag)
    t = med(lambda: oracle.fwht32_quant(xs, threads=threads))
    out["fwht32_quant"] = rec(elem * bpe / t / 1e9, "GB/s", tag)
    t = med(lambda: oracle.transform_quant(xs, lu, oracle.DENSE64, threads=threads))
    out["transform_quant_mfma"] = rec(elem * bpe / t / 1e9, "GB/s", tag + ", fp64 definition mode")
    codes, scales = oracle.transform_quant(xs, lu, oracle.STAGED32, threads=threads)
    t = med(lambda: oracle.dequant_inverse(codes, scales, lu, threads=threads))
    out["dequant_inverse"] = rec(elem * bpe / t / 1e9, "GB/s", tag)
    if d <= ADALN_MAX_D:
        shift, scale = inputs.modulation(workload, 1, d)
        t = med(lambda: oracle.adaln_transform_quant(xs, shift, scale, lu, rows_per_sample=rows,
                                                     threads=threads))
        out["adaln_fused"] = rec(elem * bpe / t / 1e9, "GB/s", tag)
    if d == inputs.GEMM_K:
        wb = inputs.gemm_weight()
        t = med(lambda: oracle.weight_quant(wb[:rows], lu, threads=threads))
        out["weight_quant"] = rec(rows * d * bpe / t / 1e9, "GB/s", f"first {rows} weight rows")
        wc, wsc = oracle.weight_quant(wb, lu, threads=threads)
        W = oracle.mxfp4_dequant(wc, wsc)
        a_rows = 16
        A = oracle.mxfp4_dequant(codes[:a_rows], scales[:a_rows])
        t = med(lambda: oracle.matmul_nt(A, W, threads=threads))
        out["w4a4_gemm"] = rec(2.0 * a_rows * W.shape[0] * d / t / 1e9, "GFLOP/s",
                               f"{a_rows} activation rows x {W.shape[0]} x {d}, fp64 products")
        cal = x_bits[:256]
        t = med(lambda: oracle.calib_objective(cal, lu, threads=threads))
        out["calibration"] = {"value": round(t * 1e3, 3), "unit": "ms per objective evaluation",
                              "threads": threads, "sample": "256 calibration rows"}
    return out


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(directory, suffix):
    for root, _, files in os.walk(directory):
        for name in files:
            if name.endswith(suffix):
                return os.path.join(root, name)
    raise FileNotFoundError(f"no *{suffix} under {directory}")


def _kmatch(entry: str, name: str) -> bool:
    keys = KERNEL_MATCH[entry]
    return any(k in name for k in ((keys,) if isinstance(keys, str) else keys))


def profile_commands(workload: str = "flux_attn") -> list:
    """PROFILE_COMMANDS for a workload: the bench runs take --workload when it
    is not the default one (the copy calibration is the same for all)."""
    from mxfp4_activation_quantizer_amd import inputs
    gemm = inputs.WORKLOADS[workload].d == inputs.GEMM_K  # the consumer takes K = 3072
    adaln = inputs.WORKLOADS[workload].d <= 8192          # one sample's vectors fit LDS
    out = []
    for c in PROFILE_COMMANDS.splitlines():
        if not gemm and "kq_w4a4_gemm" in c:
            continue
        if not adaln and "kq_adaln_transform_quant" in c:
            continue
        if workload != "flux_attn" and "bench.py --" in c and "--copy-calibration" not in c:
            c = c.replace("bench.py --", f"bench.py --workload {workload} --", 1)
        out.append(c)
    return out


def summarize_profiles(out_dir: str, workload: str = "flux_attn") -> int:
    """Turn the rocprofv3 CSV outputs of PROFILE_COMMANDS into the short
    summaries kept under profiles/ (kernel durations; HBM bytes per launch
    from FETCH_SIZE and WRITE_SIZE, each scaled by what the same counter reads
    for a device-to-device copy of 64 MiB)."""
    from mxfp4_activation_quantizer_amd import inputs
    w = inputs.WORKLOADS[workload]
    nbytes = w.algorithmic_bytes
    os.makedirs(PROFILES, exist_ok=True)
    src_hash = kernel_source_hash()

    stats = _csv_rows(_find(os.path.join(out_dir, "trace"), "kernel_stats.csv"))
    # per-dispatch durations, for the median and the 90th percentile
    durations = {}
    for r in _csv_rows(_find(os.path.join(out_dir, "trace"), "kernel_trace.csv")):
        durations.setdefault(r["Kernel_Name"], []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)

    def pct(name, q):
        vals = sorted(v for k, vs in durations.items() if k == name for v in vs)
        return vals[min(len(vals) - 1, int(q * len(vals)))] if vals else float("nan")

    lines = [f"# rocprofv3 --kernel-trace --stats, {workload} {w.tokens}x{w.d} bf16, one MI355X",
             f"# kernel sources {src_hash}; commands (REPO = repository root, OUT = output dir):"]
    lines += ["#   " + c for c in profile_commands(workload)]
    lines.append(f"# algorithmic bytes per launch: {nbytes}")
    lines.append(f"{'entry point':26s} {'calls':>6s} {'avg us':>8s} {'med us':>8s} {'p90 us':>8s} "
                 f"{'min us':>8s} {'max us':>8s} {'GB/s(avg)':>10s}")
    gemm_flops = 2.0 * w.tokens * inputs.GEMM_N * inputs.GEMM_K
    weight_bytes = inputs.GEMM_N * inputs.GEMM_K * (2 + 0.5 + 1 / 32)
    for entry in KERNEL_MATCH:
        for r in stats:
            if _kmatch(entry, r["Name"]):
                avg = float(r["AverageNs"]) / 1e3
                if entry == "kq_w4a4_gemm":
                    kind = "256 x 256 tiles" if "gemm_wide_kernel" in r["Name"] else "128 x 256 tiles"
                    rate = (f"{gemm_flops / (avg * 1e6):10.1f} TFLOP/s ({w.tokens}x{inputs.GEMM_N}x"
                            f"{inputs.GEMM_K}, {kind})")
                elif entry.startswith("kq_stream_ceiling"):
                    rate = f"{'':>10s} (workload-size and 1 GiB streams together)"
                elif entry == "kq_weight_quant":
                    rate = f"{weight_bytes / (avg * 1e3):10.1f} ({inputs.GEMM_N}x{inputs.GEMM_K} weight)"
                elif entry == "kq_adaln_modulate":
                    rate = f"{4 * w.elements / (avg * 1e3):10.1f} (bf16 in, bf16 out)"
                elif entry == "kq_calib_es_update":
                    rate = f"{'':>10s} (update alone, {w.d // 32} blocks)"
                elif entry.startswith("kq_calib"):
                    rate = f"{'':>10s} (one candidate set, 256 x {w.d} calibration rows)"
                else:
                    rate = f"{nbytes / (avg * 1e3):10.1f}"
                lines.append(f"{entry:26s} {int(r['Calls']):6d} {avg:8.3f} "
                             f"{pct(r['Name'], 0.5):8.3f} {pct(r['Name'], 0.9):8.3f} "
                             f"{float(r['MinNs']) / 1e3:8.3f} {float(r['MaxNs']) / 1e3:8.3f} {rate}")
    # the quantizer alone under the trace: its last `steps` dispatches are
    # the timed region of that same process, whose own ms_per_step it printed
    tq_path = os.path.join(out_dir, "trace_q.json")
    if os.path.exists(tq_path):
        with open(tq_path) as f:
            tq = json.loads(f.readline())
        rows = [r for r in _csv_rows(_find(os.path.join(out_dir, "trace_q"), "kernel_trace.csv"))
                if _kmatch("kq_transform_quant", r["Kernel_Name"])]
        rows.sort(key=lambda r: int(r["Start_Timestamp"]))
        timed_rows = rows[-tq["steps"]:]
        dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in timed_rows]
        avg = sum(dur) / len(dur)
        lines += [f"# quantizer alone under the trace (OUT/trace_q, bench.py --kernel-only): its {len(dur)} "
                  f"timed dispatches average {avg:.3f} us (median {sorted(dur)[len(dur) // 2]:.3f}) against "
                  f"that process's own ms_per_step {tq['ms_per_step'] * 1e3:.3f} us "
                  f"({avg / (tq['ms_per_step'] * 1e3):.3f} x); frac from the traced average "
                  f"{nbytes / (avg * 1e3) / PEAK_HBM_GBS:.4f}"]
    bench_rec = None
    bench_path = os.path.join(out_dir, "bench.json")
    if os.path.exists(bench_path):
        with open(bench_path) as f:
            bench_rec = json.loads(f.readline())
        traced = next((float(r["AverageNs"]) / 1e3 for r in stats
                       if KERNEL_MATCH["kq_transform_quant"] in r["Name"]), float("nan"))
        bus = bench_rec["ms_per_step"] * 1e3
        lines += [f"# bench.py run in the same call (OUT/bench.json): ms_per_step {bus:.3f} us "
                  f"({bench_rec['value']} GB/s, frac {bench_rec['roofline']['frac']}); the trace's "
                  f"kq_transform_quant average over all its calls above (warm-up, peers, graph replays "
                  f"and MALL-warm runs included) {traced:.3f} us = {traced / bus:.3f} x"]
    with open(os.path.join(PROFILES, f"kernel_stats_{workload}.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    hc = (bench_rec or {}).get("peers", {}).get("hbm_ceiling")
    if hc:
        frac = bench_rec["roofline"]["frac"]
        gbs = bench_rec["value"]
        hl = [f"# HBM ceilings measured by bench.py ({workload} {w.tokens}x{w.d}) with "
              f"kq_stream_ceiling: wave-contiguous 16-byte loads, no arithmetic, a lane mapping of",
              "# its own (not the quantizer's); 1 GiB streams amortise launch costs; the 64:17 mix is",
              "# the quantizer's bytes per 32-element unit (64 read, 16 + 1 written)",
              f"# kernel sources {src_hash}; command: python3 bench.py --json-out OUT/bench.json"
              + (f" --workload {workload}" if workload != "flux_attn" else ""),
              f"{'stream':44s} {'us':>10s} {'GB/s':>9s} {'of 8 TB/s':>9s}"]
        for key, label, b in (("gib_read_only", "1 GiB read only", 1 << 30),
                              ("gib_read_write_64_17", "1 GiB read + 17/64 written", None)):
            r = hc[key]
            hl.append(f"{label:44s} {r['ms_per_step'] * 1e3:10.2f} {r['GBps']:9.1f} "
                      f"{r['GBps'] / PEAK_HBM_GBS:9.4f}")
        for key, label in (("workload_read_only", f"{w.tokens}x{w.d} size, read only"),
                           ("workload_read_write", f"{w.tokens}x{w.d} size, 64:17, host-issued"),
                           ("workload_read_write_graph", f"{w.tokens}x{w.d} size, 64:17, graph replay")):
            r = hc[key]
            hl.append(f"{label:44s} {r['ms_per_step'] * 1e3:10.3f} {r['GBps']:9.1f} "
                      f"{r['GBps'] / PEAK_HBM_GBS:9.4f}")
        if "torch_copy_gib" in hc:
            r = hc["torch_copy_gib"]
            hl.append(f"{'torch device copy of 1 GiB (read + write)':44s} {r['ms_per_step'] * 1e3:10.2f} "
                      f"{r['GBps_read_plus_write']:9.1f} {r['frac_of_hbm_peak']:9.4f}")
        hl.append(f"{'one-wave pass, host-issued (launch floor)':44s} {hc['one_wave_pass_host_issued_us']:10.3f}")
        hl.append(f"{'one-wave pass, graph replay':44s} {hc['launch_floor_graph_us']:10.3f}")
        hl.append(f"kq_transform_quant in the same run: {gbs} GB/s = frac {frac} of 8 TB/s, "
                  f"{gbs / hc['gib_read_write_64_17']['GBps']:.4f} of the 1 GiB 64:17 stream, "
                  f"{gbs / hc['workload_read_write']['GBps']:.4f} of the same-size 64:17 stream")
        with open(os.path.join(PROFILES, "hbm_ceiling.txt" if workload == "flux_attn"
                               else f"hbm_ceiling_{workload}.txt"), "w") as f:
            f.write("\n".join(hl) + "\n")

    def counter_avg(sub, counter, match):
        rows = _csv_rows(_find(os.path.join(out_dir, sub), "counter_collection.csv"))
        vals = [float(r["Counter_Value"]) for r in rows
                if r["Counter_Name"] == counter and match in r["Kernel_Name"]]
        if not vals:
            raise ValueError(f"{counter}: no dispatch matching {match!r} in {sub}")
        return sum(vals) / len(vals), len(vals)

    copy_kib = (64 << 20) / 1024
    cf, ncf = counter_avg("copy_FETCH_SIZE", "FETCH_SIZE", "copyBuffer")
    cw, ncw = counter_avg("copy_WRITE_SIZE", "WRITE_SIZE", "copyBuffer")
    kf, nkf = counter_avg("FETCH_SIZE", "FETCH_SIZE", KERNEL_MATCH["kq_transform_quant"])
    kw, nkw = counter_avg("WRITE_SIZE", "WRITE_SIZE", KERNEL_MATCH["kq_transform_quant"])
    fs, ws = copy_kib / cf, copy_kib / cw
    read_b, write_b = kf * fs * 1024, kw * ws * 1024
    rec = {"kernel": "kq_transform_quant", "workload": workload, "source_hash": src_hash,
           "fetch_size_kib": round(kf, 2), "write_size_kib": round(kw, 2),
           "copy_fetch_size_kib": round(cf, 2), "copy_write_size_kib": round(cw, 2),
           "fetch_scale": round(fs, 5), "write_scale": round(ws, 5),
           "hbm_read_bytes_per_launch": round(read_b), "hbm_write_bytes_per_launch": round(write_b),
           "hbm_bytes_per_launch": round(read_b + write_b),
           "algorithmic_bytes_per_launch": nbytes,
           "traffic_over_algorithmic": round((read_b + write_b) / nbytes, 4),
           "dispatches": {"kernel_fetch": nkf, "kernel_write": nkw, "copy_fetch": ncf,
                          "copy_write": ncw}}
    with open(os.path.join(PROFILES, f"traffic_kq_transform_quant_{workload}.json"), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    txt = [f"# HBM traffic of kq_transform_quant, {workload} {w.tokens}x{w.d}, from rocprofv3 --pmc",
           f"# kernel sources {src_hash}; commands:"]
    txt += ["#   " + c for c in profile_commands(workload)]
    txt += [f"FETCH_SIZE per dispatch   {kf:12.1f} KiB (x{fs:.4f} copy scale) = {read_b / 1e6:9.3f} MB",
            f"WRITE_SIZE per dispatch   {kw:12.1f} KiB (x{ws:.4f} copy scale) = {write_b / 1e6:9.3f} MB",
            f"64 MiB device copy reads  FETCH_SIZE {cf:10.1f} KiB, WRITE_SIZE {cw:10.1f} KiB",
            f"HBM bytes per launch      {(read_b + write_b) / 1e6:9.3f} MB",
            f"algorithmic bytes         {nbytes / 1e6:9.3f} MB  (ratio {(read_b + write_b) / nbytes:.4f})"]
    with open(os.path.join(PROFILES, f"hbm_traffic_kq_transform_quant_{workload}.txt"), "w") as f:
        f.write("\n".join(txt) + "\n")

    # instruction counters of the hot path, the matrix-core arm, the GEMM and
    # the AdaLN-fused quantizer
    ctr = [f"# SQ counters per dispatch (mean over the dispatches), {workload} "
           f"{w.tokens}x{w.d}, from rocprofv3 --pmc",
           f"# kernel sources {src_hash}; commands:"]
    ctr += ["#   " + c for c in profile_commands(workload)]
    for sub, entry in (("SQ", "kq_transform_quant"), ("SQ_mfma", "kq_transform_quant_mfma"),
                       ("SQ_quad", "kq_transform_quant_quad"),
                       ("SQ_gemm", "kq_w4a4_gemm"), ("SQ_adaln", "kq_adaln_transform_quant")):
        if not any(f"OUT/{sub} " in c for c in profile_commands(workload)):
            continue  # no such pass for this workload
        if not os.path.isdir(os.path.join(out_dir, sub)):
            ctr.append(f"{entry}: no {sub} pass in {out_dir}")
            continue
        rows = _csv_rows(_find(os.path.join(out_dir, sub), "counter_collection.csv"))
        means = {}
        for r in rows:
            if _kmatch(entry, r["Kernel_Name"]):
                means.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        means = {k: sum(v) / len(v) for k, v in means.items()}
        ctr.append(f"{entry}:")
        for k in sorted(means):
            ctr.append(f"  {k:26s} {means[k]:14.1f}")
        if means.get("SQ_WAVES") and entry != "kq_w4a4_gemm":
            ctr.append(f"  VALU instructions per wave {means['SQ_INSTS_VALU'] / means['SQ_WAVES']:14.1f}")
            ctr.append(f"  VALU lane-ops per element  {64 * means['SQ_INSTS_VALU'] / w.elements:14.2f}")
        if means.get("SQ_INSTS_MFMA"):
            ctr.append(f"  MFMA busy cycles per MFMA  {means['SQ_VALU_MFMA_BUSY_CYCLES'] / means['SQ_INSTS_MFMA']:14.1f}")
        if entry == "kq_w4a4_gemm" and means.get("SQ_INSTS_MFMA"):
            ctr.append(f"  (one GEMM, {w.tokens}x{inputs.GEMM_N}x{inputs.GEMM_K}: "
                       f"{2 * w.tokens * inputs.GEMM_N * inputs.GEMM_K / means['SQ_INSTS_MFMA']:.0f} flops per MFMA instruction)")
    if os.path.isdir(os.path.join(out_dir, "FETCH_quad")):
        qf, nqf = counter_avg("FETCH_quad", "FETCH_SIZE", KERNEL_MATCH["kq_transform_quant_quad"])
        ctr.append(f"kq_transform_quant_quad FETCH_SIZE per dispatch {qf:.1f} KiB (x{fs:.4f} copy scale) = "
                   f"{qf * fs * 1024 / 1e6:.3f} MB read, against {read_b / 1e6:.3f} MB for "
                   f"kq_transform_quant ({nqf} dispatches)")
    with open(os.path.join(PROFILES, f"counters_{workload}.txt"), "w") as f:
        f.write("\n".join(ctr) + "\n")
    print("\n".join(lines + txt + ctr))
    return 0


E2M1_VALUES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def round_trip_errors(kq, torch, inputs, np, held, xh, lu_d, start, theta, xa) -> dict:
    """Relative Frobenius error ||x~ - x|| / ||x|| of the MXFP4 round trip on
    the same held-out rows for every transform: the Kronecker transform with
    the workload's random parameters, the Hadamard start and the calibrated
    parameters (GPU quantizer, then the GPU dequantise + inverse, bf16 out),
    per-channel scaling (codes / mult) and FWHT32 (codes times H_32, which is
    its own inverse); the last two decode the GPU codes on the host and round
    to bf16 like the Kronecker inverse."""
    import scipy.linalg
    out = {}
    nx = float(np.linalg.norm(xh))
    for name, lu in (("kron_random_params", lu_d), ("kron_hadamard_start", start),
                     ("kron_calibrated", theta)):
        c, s = kq.transform_quant(held, lu)
        xr = kq.dequant_inverse(c, s, lu)
        xr = inputs.bf16_bits_to_f32(xr.view(torch.int16).cpu().numpy().view(np.uint16))
        out[name] = round(float(np.linalg.norm(xr.astype(np.float64) - xh)) / nx, 5)
    tab = np.array(E2M1_VALUES + tuple(-v for v in E2M1_VALUES))

    def decode(c, s):
        c = c.cpu().numpy()
        nib = np.empty((c.shape[0], c.shape[1] * 2), np.uint8)
        nib[:, 0::2], nib[:, 1::2] = c & 15, c >> 4
        e = np.repeat(s.cpu().numpy().astype(np.float64) - 127.0, 32, axis=1)
        return tab[nib] * 2.0 ** e

    mult = inputs.smooth_multipliers(xa)
    c, s = kq.smooth_quant(held, torch.from_numpy(mult).to(held.device))
    xs = decode(c, s) / mult.astype(np.float64)[None, :]
    xs = inputs.bf16_bits_to_f32(inputs.f64_to_bf16_bits(xs)).astype(np.float64)
    out["smooth"] = round(float(np.linalg.norm(xs - xh)) / nx, 5)
    c, s = kq.fwht32_quant(held)
    H = scipy.linalg.hadamard(32) / np.sqrt(32.0)
    y = decode(c, s)
    xf = (y.reshape(y.shape[0], -1, 32) @ H).reshape(y.shape)
    xf = inputs.bf16_bits_to_f32(inputs.f64_to_bf16_bits(xf)).astype(np.float64)
    out["fwht32"] = round(float(np.linalg.norm(xf - xh)) / nx, 5)
    out["rows"] = "2048..2303 of the workload (held out from calibration)"
    return out


def graph_ms(torch, launch, n):
    """ms per launch of n launches captured in one HIP graph (torch's
    capture) and replayed: no host cost per launch."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(3):
            launch(i, side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cs = torch.cuda.current_stream().cuda_stream
        for i in range(n):
            launch(i, cs)
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    cur = torch.cuda.current_stream()
    e0.record(cur)
    for _ in range(3):
        g.replay()
    e1.record(cur)
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / (3 * n)


def other_workloads(L, torch, dev, sp, steps, warmup, names=("pixart", "flux_mlp")) -> dict:
    """kq_transform_quant on the other activation shapes of the method's
    configurations (PixArt-Sigma 8192 x 1152, FLUX-MLP 4608 x 12288), timed
    like the value: seeded inputs of the workload's recipe, steps rotating
    over buffer sets that together exceed twice the 256 MB MALL."""
    import numpy as np
    from mxfp4_activation_quantizer_amd import inputs, kq
    stream = torch.cuda.current_stream(dev)
    out = {}
    for name in names:
        w = inputs.WORKLOADS[name]
        T, d = w.tokens, w.d
        nb = d // 32
        nbytes = T * d * 2 + T * d // 2 + T * nb
        R = max(2, -(-600_000_000 // nbytes))
        x0 = torch.from_numpy(inputs.activation(name).view(np.int16)).to(dev)
        xs = [x0] + [x0.clone() for _ in range(R - 1)]
        lu = torch.from_numpy(inputs.lu_params(name).astype(np.float32)).to(dev)
        codes = [torch.empty(T, d // 2, dtype=torch.uint8, device=dev) for _ in range(R)]
        scales = [torch.empty(T, nb, dtype=torch.uint8, device=dev) for _ in range(R)]
        args = [(xs[i].data_ptr(), T, d, d, lu.data_ptr(), codes[i].data_ptr(), scales[i].data_ptr(), sp)
                for i in range(R)]
        # untimed launches for 0.3 s (fresh buffers, clocks), then the warmup
        t_end = time.perf_counter() + 0.3
        i = 0
        while time.perf_counter() < t_end or i < warmup:
            st = L.kq_transform_quant(*args[i % R])
            if st != 0:
                raise kq.KQError("kq_transform_quant", st)
            i += 1
            if i % 64 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            L.kq_transform_quant(*args[i % R])
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        g = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"config": f"{name}_{T}x{d}", "ms_per_step": round(ms, 6), "GBps": round(g, 1),
                     "frac_of_hbm_peak": round(g / PEAK_HBM_GBS, 4),
                     "tokens_per_s": round(T / (ms * 1e-3), 1), "rotating_buffer_sets": R}
        del xs, x0, codes, scales, args
        torch.cuda.empty_cache()
    return out


def hbm_ceilings(L, torch, dev, sp, xs, codes, scales, units, steps, warmup) -> dict:
    """What the memory system sustains for the quantizer's traffic, measured
    with kq_stream_ceiling (wave-contiguous loads and stores, no arithmetic, a
    lane mapping of its own): at the workload's size over the same rotating
    buffer sets (read only, and 64 B read + 17 B written per unit), on 1 GiB
    streams (the sustained rate, launch costs amortised), the per-launch floor
    of a one-wave pass, and a torch device-to-device copy of 1 GiB."""
    from mxfp4_activation_quantizer_amd import kq
    stream = torch.cuda.current_stream(dev)

    def ev(call, n, warm):
        for i in range(warm):
            call(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            call(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n  # ms per launch

    def chk(st):
        if st != 0:
            raise kq.KQError("kq_stream_ceiling", st)

    R = len(xs)
    out = {}
    one = torch.empty(64 * 64, dtype=torch.uint8, device=dev)
    ms = ev(lambda i: chk(L.kq_stream_ceiling(xs[i % R].data_ptr(), 64, None, one.data_ptr(), sp)),
            steps, warmup)
    out["one_wave_pass_host_issued_us"] = round(ms * 1e3, 3)
    ms = graph_ms(torch, lambda i, st: chk(L.kq_stream_ceiling(xs[i % R].data_ptr(), 64, None,
                                                        one.data_ptr(), st)), 100)
    out["launch_floor_graph_us"] = round(ms * 1e3, 3)
    rbytes, wbytes = units * 64, units * 17
    ms = ev(lambda i: chk(L.kq_stream_ceiling(xs[i % R].data_ptr(), units, None,
                                              scales[i % R].data_ptr(), sp)), steps, warmup)
    out["workload_read_only"] = {"ms_per_step": round(ms, 6),
                                 "GBps": round(rbytes / (ms * 1e-3) / 1e9, 1)}
    ms = ev(lambda i: chk(L.kq_stream_ceiling(xs[i % R].data_ptr(), units, codes[i % R].data_ptr(),
                                              scales[i % R].data_ptr(), sp)), steps, warmup)
    out["workload_read_write"] = {"ms_per_step": round(ms, 6),
                                  "GBps": round((rbytes + wbytes) / (ms * 1e-3) / 1e9, 1)}
    ms = graph_ms(torch, lambda i, st: chk(L.kq_stream_ceiling(xs[i % R].data_ptr(), units,
                                                        codes[i % R].data_ptr(),
                                                        scales[i % R].data_ptr(), st)), 4 * R)
    out["workload_read_write_graph"] = {"ms_per_step": round(ms, 6),
                                        "GBps": round((rbytes + wbytes) / (ms * 1e-3) / 1e9, 1)}
    gib = 1 << 30
    src = torch.empty(gib, dtype=torch.uint8, device=dev)
    src.fill_(0x3C)
    gu = gib // 64
    gc = torch.empty(gu * 16, dtype=torch.uint8, device=dev)
    gs = torch.empty(gu, dtype=torch.uint8, device=dev)
    n = max(10, steps // 10)
    ms = ev(lambda i: chk(L.kq_stream_ceiling(src.data_ptr(), gu, None, gs.data_ptr(), sp)), n, 3)
    g = gib / (ms * 1e-3) / 1e9
    out["gib_read_only"] = {"ms_per_step": round(ms, 6), "GBps": round(g, 1),
                            "frac_of_hbm_peak": round(g / PEAK_HBM_GBS, 4)}
    ms = ev(lambda i: chk(L.kq_stream_ceiling(src.data_ptr(), gu, gc.data_ptr(), gs.data_ptr(), sp)),
            n, 3)
    g = gu * 81 / (ms * 1e-3) / 1e9
    out["gib_read_write_64_17"] = {"ms_per_step": round(ms, 6), "GBps": round(g, 1),
                                   "frac_of_hbm_peak": round(g / PEAK_HBM_GBS, 4)}
    del gc, gs
    dst = torch.empty_like(src)
    ms = ev(lambda i: dst.copy_(src), n, 3)
    g = 2 * gib / (ms * 1e-3) / 1e9
    out["torch_copy_gib"] = {"ms_per_step": round(ms, 6), "GBps_read_plus_write": round(g, 1),
                             "frac_of_hbm_peak": round(g / PEAK_HBM_GBS, 4)}
    del src, dst
    torch.cuda.empty_cache()
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="flux_attn",
                    choices=["pixart", "flux_attn", "flux_mlp"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the quantizer on the PixArt-Sigma and FLUX-MLP activations")
    ap.add_argument("--no-peers", action="store_true", help="skip the peer kernels")
    ap.add_argument("--kernel-only", action="store_true",
                    help="run only the timed steps of one kernel (for profilers)")
    ap.add_argument("--kernel", default="kq_transform_quant",
                    choices=["kq_transform_quant", "kq_transform_quant_mfma",
                             "kq_transform_quant_quad", "kq_smooth_quant",
                             "kq_fwht32_quant", "kq_copy_ceiling", "kq_stream_ceiling",
                             "kq_dequant_inverse",
                             "kq_weight_quant", "kq_w4a4_gemm", "kq_adaln_transform_quant",
                             "kq_adaln_unfused"],
                    help="the entry point --kernel-only times")
    ap.add_argument("--json-out", metavar="PATH",
                    help="also write the JSON line to PATH")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="summarise rocprofv3 CSV outputs under DIR into profiles/ and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 64 MiB device-to-device copy, the known-size "
                         "reference for the HBM byte counters")
    args = ap.parse_args()

    if args.summarize_profiles:
        return summarize_profiles(args.summarize_profiles, args.workload)
    if args.gpus != 1:
        print(f"bench.py measures one GPU: token rows and channel blocks are independent, so "
              f"the quantizer shards with no exchange and one GPU's figure is the per-GPU "
              f"figure; --gpus {args.gpus} is not supported.", file=sys.stderr)
        return 2
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if world != 1:
        print("bench.py runs as a single process on one GPU", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from mxfp4_activation_quantizer_amd import inputs, kq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = 64 << 20
        srcs = [torch.empty(n // 2, dtype=torch.bfloat16, device=dev) for _ in range(8)]
        dsts = [torch.empty_like(srcs[0]) for _ in range(8)]
        for i in range(args.steps):
            dsts[i % 8].copy_(srcs[i % 8])
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n,
                          "launches": args.steps}), flush=True)
        return 0
    w = inputs.WORKLOADS[args.workload]
    T, d, nb = w.tokens, w.d, w.blocks
    nbytes = w.algorithmic_bytes

    x_bits = inputs.activation(args.workload)
    lu = inputs.lu_params(args.workload)
    mult = inputs.smooth_multipliers(x_bits)

    set_bytes = nbytes
    R = max(2, -(-2 * MALL_BYTES // set_bytes))
    x0 = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    xs = [x0] + [x0.clone() for _ in range(R - 1)]
    x_keep = x0.clone() if not (args.kernel_only or args.no_peers) else None
    codes = [torch.empty((T, d // 2), dtype=torch.uint8, device=dev) for _ in range(R)]
    scales = [torch.empty((T, nb), dtype=torch.uint8, device=dev) for _ in range(R)]
    lu_d = torch.from_numpy(lu).to(dev)
    mult_d = torch.from_numpy(mult).to(dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    L = kq.lib()

    # The consumer of the quantized activation: Y = A W^T with MXFP4 A (the
    # kernel's output) and W (12288 x 3072 prepared by kq_weight_quant).
    gemm = {}
    want_gemm = args.kernel in ("kq_w4a4_gemm", "kq_weight_quant") if args.kernel_only \
        else not args.no_peers
    if want_gemm and d != inputs.GEMM_K:
        if args.kernel_only:
            print(f"the W4A4 consumer takes K = {inputs.GEMM_K} channels", file=sys.stderr)
            return 2
        want_gemm = False
    if want_gemm:
        wn, wk = inputs.GEMM_N, inputs.GEMM_K
        gemm["w"] = torch.from_numpy(inputs.gemm_weight().view(np.int16)).view(torch.bfloat16).to(dev)
        gemm["wc"] = torch.empty((wn, wk // 2), dtype=torch.uint8, device=dev)
        gemm["ws"] = torch.empty((wn, wk // 32), dtype=torch.uint8, device=dev)
        gemm["y"] = [torch.empty((T, wn), dtype=torch.bfloat16, device=dev) for _ in range(2)]
        gemm["lu"] = lu_d
        st = L.kq_weight_quant(gemm["w"].data_ptr(), wn, wk, wk, gemm["lu"].data_ptr(),
                               gemm["wc"].data_ptr(), gemm["ws"].data_ptr(), sp)
        if st != 0:
            raise kq.KQError("kq_weight_quant", st)
        gemm.update(n=wn, k=wk, flops=2.0 * T * wn * wk,
                    weight_bytes=wn * wk * (2 + 0.5 + 1 / 32))

    # AdaLN-fused quantizer: the same rotating inputs read as the pre-norm
    # stream, one sample's shift/scale; the unfused pipeline writes bf16 h.
    shift_np, scale_np = inputs.modulation(args.workload, 1, d)
    shift_d, scale_d = torch.from_numpy(shift_np).to(dev), torch.from_numpy(scale_np).to(dev)
    if args.kernel_only and args.kernel.startswith("kq_adaln") and d > ADALN_MAX_D:
        print(f"the AdaLN-fused kernel takes d <= {ADALN_MAX_D} channels", file=sys.stderr)
        return 2
    need_h = d <= ADALN_MAX_D and ((args.kernel_only and args.kernel == "kq_adaln_unfused") or
                                   not (args.kernel_only or args.no_peers))
    hs = [torch.empty((T, d), dtype=torch.bfloat16, device=dev) for _ in range(R)] if need_h else []

    def argsets(fn_name):
        out = []
        if fn_name == "kq_adaln_transform_quant":
            return [(xs[i].data_ptr(), T, d, d, shift_d.data_ptr(), scale_d.data_ptr(), T,
                     ctypes.c_float(1e-6), lu_d.data_ptr(), codes[i].data_ptr(),
                     scales[i].data_ptr(), sp) for i in range(R)]
        if fn_name == "kq_adaln_modulate":
            return [(xs[i].data_ptr(), T, d, d, shift_d.data_ptr(), scale_d.data_ptr(), T,
                     ctypes.c_float(1e-6), hs[i].data_ptr(), d, sp) for i in range(R)]
        if fn_name == "kq_transform_quant_from_h":
            return [(hs[i].data_ptr(), T, d, d, lu_d.data_ptr(), codes[i].data_ptr(),
                     scales[i].data_ptr(), sp) for i in range(R)]
        if fn_name == "kq_w4a4_gemm":
            for i in range(R):  # A: the quantized activations of set i
                y = gemm["y"][i % 2]
                out.append((codes[i].data_ptr(), scales[i].data_ptr(), gemm["wc"].data_ptr(),
                            gemm["ws"].data_ptr(), T, gemm["n"], gemm["k"], y.data_ptr(),
                            gemm["n"], sp))
            return out
        if fn_name == "kq_weight_quant":
            return [(gemm["w"].data_ptr(), gemm["n"], gemm["k"], gemm["k"], gemm["lu"].data_ptr(),
                     gemm["wc"].data_ptr(), gemm["ws"].data_ptr(), sp)]
        for i in range(R):
            xp, cp, scp = xs[i].data_ptr(), codes[i].data_ptr(), scales[i].data_ptr()
            if fn_name in ("kq_transform_quant", "kq_transform_quant_mfma",
                           "kq_transform_quant_quad"):
                out.append((xp, T, d, d, lu_d.data_ptr(), cp, scp, sp))
            elif fn_name == "kq_stream_ceiling":
                # the same bytes as one quantizer step: T * nb units of 64 B
                out.append((xp, T * nb, cp, scp, sp))
            elif fn_name == "kq_dequant_inverse":
                # codes/scales of set i back to the bf16 buffer of set i
                out.append((cp, scp, T, d, lu_d.data_ptr(), xp, d, sp))
            elif fn_name == "kq_smooth_quant":
                out.append((xp, T, d, d, mult_d.data_ptr(), cp, scp, sp))
            else:
                out.append((xp, T, d, d, cp, scp, sp))
        return out

    def unfused(*a):
        st = L.kq_adaln_modulate(*a[0])
        return st if st != 0 else L.kq_transform_quant(*a[1])

    def timed(fn_name, steps, warmup):
        if fn_name == "kq_adaln_unfused":  # two launches per step
            fn = unfused
            a = list(zip(argsets("kq_adaln_modulate"), argsets("kq_transform_quant_from_h")))
        else:
            fn = getattr(L, fn_name)
            a = argsets(fn_name)
        n_a = len(a)
        for i in range(warmup):
            st = fn(*a[i % n_a])
            if st != 0:
                raise kq.KQError(fn_name, st)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            fn(*a[i % n_a])
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps  # ms per launch

    def timed_one_set(fn_name, steps, warmup):
        """The same launches on buffer set 0 every step: its inputs stay in
        the 256 MB MALL, so this is a cache-warm figure, never the value."""
        fn, a0 = getattr(L, fn_name), argsets(fn_name)[0]
        for _ in range(warmup):
            fn(*a0)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn(*a0)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def settle(seconds=0.3):
        """Untimed launches until the GPU clocks have left their idle state:
        the first timed batch of a fresh process otherwise runs several per
        cent slower than the rest."""
        fn, a = L.kq_transform_quant, argsets("kq_transform_quant")
        t_end = time.perf_counter() + seconds
        while time.perf_counter() < t_end:
            for i in range(200):
                fn(*a[i % R])
            torch.cuda.synchronize()

    settle()
    if args.kernel_only:
        if args.kernel in ("kq_dequant_inverse", "kq_w4a4_gemm"):
            timed("kq_transform_quant", R, 0)  # they read the quantizer's outputs
        ms = timed(args.kernel, args.steps, args.warmup)
        rec = {"kernel": args.kernel, "ms_per_step": ms}
        if args.kernel == "kq_w4a4_gemm":
            rec["TFLOPs"] = gemm["flops"] / (ms * 1e-3) / 1e12
        elif args.kernel in ("kq_adaln_transform_quant", "kq_adaln_unfused"):
            rec["GBps_fused_bytes"] = nbytes / (ms * 1e-3) / 1e9
        elif args.kernel == "kq_weight_quant":
            rec["GBps"] = gemm["weight_bytes"] / (ms * 1e-3) / 1e9
        else:
            rec["GBps"] = nbytes / (ms * 1e-3) / 1e9
        rec["steps"] = args.steps
        print(json.dumps(rec), flush=True)
        if args.json_out:
            with open(args.json_out, "w") as f:
                f.write(json.dumps(rec) + "\n")
        return 0
    ms = timed("kq_transform_quant", args.steps, args.warmup)
    gbs = nbytes / (ms * 1e-3) / 1e9

    extra = {}
    if not args.no_peers:
        for name, fn_name in [("transform_quant_mfma", "kq_transform_quant_mfma"),
                              ("transform_quant_quad", "kq_transform_quant_quad"),
                              ("smooth_quant", "kq_smooth_quant"),
                              ("fwht32_quant", "kq_fwht32_quant"),
                              ("copy_ceiling", "kq_copy_ceiling"),
                              ("dequant_inverse", "kq_dequant_inverse")]:
            pms = timed(fn_name, args.steps, args.warmup)
            pg = nbytes / (pms * 1e-3) / 1e9
            extra[name] = {"ms_per_step": round(pms, 6), "GBps": round(pg, 1),
                           "frac_of_hbm_peak": round(pg / PEAK_HBM_GBS, 4)}
        extra["frac_of_copy_ceiling"] = round(extra["copy_ceiling"]["ms_per_step"] / ms, 4)
        gms = graph_ms(torch, lambda i, st: L.kq_transform_quant(
            xs[i % R].data_ptr(), T, d, d, lu_d.data_ptr(), codes[i % R].data_ptr(),
            scales[i % R].data_ptr(), st), 4 * R)
        extra["transform_quant_graph_replay"] = {
            "ms_per_step": round(gms, 6), "GBps": round(nbytes / (gms * 1e-3) / 1e9, 1),
            "note": "the same steps captured in one HIP graph and replayed; not the value"}
        if args.workload == "flux_attn" and not args.no_other_workloads:
            extra["other_workloads"] = other_workloads(L, torch, dev, sp, args.steps, args.warmup)
        extra["hbm_ceiling"] = hbm_ceilings(L, torch, dev, sp, xs, codes, scales, T * nb,
                                            args.steps, args.warmup)
        wms = timed_one_set("kq_transform_quant", args.steps, args.warmup)
        extra["mall_warm_single_buffer"] = {
            "ms_per_step": round(wms, 6), "GBps": round(nbytes / (wms * 1e-3) / 1e9, 1),
            "note": "one buffer set every step, inputs served from the MALL; not the value"}
        # the copy ceiling and the inverse wrote into the rotating buffers:
        # restore the inputs before the next peers read them
        for xi in xs:
            xi.copy_(x_keep)
        timed("kq_transform_quant", R, 0)
        # AdaLN + quantizer: fused (one pass, same bytes as the quantizer) vs
        # modulate-to-bf16 then quantize (4 more bytes per element through HBM);
        # the fused kernel keeps a sample's vectors in LDS, so d <= 8192
        if d <= ADALN_MAX_D:
            fms = timed("kq_adaln_transform_quant", args.steps, args.warmup)
            ums = timed("kq_adaln_unfused", args.steps, args.warmup)
            extra["adaln_fused"] = {"ms_per_step": round(fms, 6),
                                    "GBps": round(nbytes / (fms * 1e-3) / 1e9, 1),
                                    "frac_of_hbm_peak": round(nbytes / (fms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
            extra["adaln_unfused"] = {"ms_per_step": round(ums, 6),
                                      "GBps_moved": round((nbytes + 4 * T * d) / (ums * 1e-3) / 1e9, 1),
                                      "fused_speedup": round(ums / fms, 3)}
    if not args.no_peers:
        # Calibration of the block parameters from the Hadamard start (per-block
        # (1+1)-ES on the MXFP4 round-trip objective): 150 iterations on 256
        # rows, then the round-trip error on 256 held-out rows.
        xa = inputs.activation(args.workload)
        cal = torch.from_numpy(xa[:256].view(np.int16)).view(torch.bfloat16).to(dev)
        held_rows = slice(2048, 2304)
        held = torch.from_numpy(xa[held_rows].view(np.int16)).view(torch.bfloat16).to(dev)
        start = torch.from_numpy(inputs.hadamard_init(nb)).to(dev)
        noise = torch.from_numpy(inputs.calib_noise(args.workload, 150)).to(dev)
        kq.calibrate(cal, start, noise[:3])  # warm
        torch.cuda.synchronize()
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        theta, _, _ = kq.calibrate(cal, start, noise)
        c1.record(stream)
        torch.cuda.synchronize()
        xh = inputs.bf16_bits_to_f32(xa[held_rows]).astype(np.float64)
        energy = float((xh ** 2).sum())
        f0 = kq.calib_objective(held, start).double().sum().item()
        f1 = kq.calib_objective(held, theta).double().sum().item()
        extra["calibration"] = {
            "iterations": 150, "calibration_rows": 256, "held_out_rows": 256,
            "ms_per_iteration": round(c0.elapsed_time(c1) / 150, 4),
            "held_out_rel_err_hadamard": round((f0 / energy) ** 0.5, 5),
            "held_out_rel_err_calibrated": round((f1 / energy) ** 0.5, 5)}
        extra["round_trip_rel_err"] = round_trip_errors(kq, torch, inputs, np, held, xh, lu_d,
                                                        start, theta, xa)
        if gemm:
            gemm["theta"] = theta
    if gemm:
        timed("kq_transform_quant", R, 0)  # A operands: fresh quantizer outputs
        pms = timed("kq_weight_quant", max(10, args.steps // 10), max(2, args.warmup // 10))
        wg = gemm["weight_bytes"] / (pms * 1e-3) / 1e9
        extra["weight_quant"] = {"ms_per_step": round(pms, 6), "shape": [gemm["n"], gemm["k"]],
                                 "GBps": round(wg, 1), "frac_of_hbm_peak": round(wg / PEAK_HBM_GBS, 4)}
        # at least 50 launches (6 ms): the GEMM's clock moves with its power draw
        pms = timed("kq_w4a4_gemm", max(50, args.steps // 4), max(5, args.warmup // 10))
        tf = gemm["flops"] / (pms * 1e-3) / 1e12
        if "theta" in gemm:
            # end-to-end error of W4A4 against the unquantised X W^T on 24
            # sampled rows, for each transform through the same consumer
            xa = inputs.activation(args.workload)
            wa = inputs.gemm_weight()
            rows = np.sort(np.random.default_rng(9).choice(T, 24, replace=False))
            ref = inputs.bf16_bits_to_f32(xa[rows]).astype(np.float64) @ \
                inputs.bf16_bits_to_f32(wa).astype(np.float64).T
            xdev = torch.from_numpy(xa.view(np.int16)).view(torch.bfloat16).to(dev)
            mult = inputs.smooth_multipliers(xa)
            minv = torch.from_numpy((1.0 / mult.astype(np.float64)).astype(np.float32)).to(dev)
            multd = torch.from_numpy(mult).to(dev)
            pairs = {
                "kron_calibrated": (kq.transform_quant(xdev, gemm["theta"]),
                                    kq.weight_quant(gemm["w"], gemm["theta"])),
                "kron_random_params": (kq.transform_quant(xdev, lu_d), kq.weight_quant(gemm["w"], lu_d)),
                "fwht32": (kq.fwht32_quant(xdev), kq.fwht32_quant(gemm["w"])),
                "smooth": (kq.smooth_quant(xdev, multd), kq.smooth_quant(gemm["w"], minv)),
            }
            e2e = {}
            for name_, ((ac_, as__), (wc_, ws_)) in pairs.items():
                yy = kq.w4a4_gemm(ac_, as__, wc_, ws_)
                got = inputs.bf16_bits_to_f32(
                    yy.view(torch.int16).cpu().numpy().view(np.uint16)[rows]).astype(np.float64)
                e2e[name_] = round(float(np.linalg.norm(got - ref) / np.linalg.norm(ref)), 5)
            extra["w4a4_end_to_end_rel_err"] = e2e
        extra["w4a4_gemm"] = {"ms_per_step": round(pms, 6), "shape_mnk": [T, gemm["n"], gemm["k"]],
                              "TFLOPs": round(tf, 1), "peak_TFLOPs": PEAK_FP4_TFLOPS,
                              "frac": round(tf / PEAK_FP4_TFLOPS, 4)}

    src_hash = kernel_source_hash()
    traffic = load_traffic("kq_transform_quant", args.workload, src_hash)
    roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": nbytes}
    hc = extra.get("hbm_ceiling")
    if hc:
        # the same fraction against what was measured in this run: the
        # streaming reference at this size (launch costs included) and on a
        # 1 GiB stream (the sustained rate for this read:write mix)
        roofline["measured_ceiling_same_size_GBps"] = hc["workload_read_write"]["GBps"]
        roofline["frac_of_measured_ceiling_same_size"] = round(
            gbs / hc["workload_read_write"]["GBps"], 4)
        roofline["measured_ceiling_1gib_GBps"] = hc["gib_read_write_64_17"]["GBps"]
        roofline["frac_of_measured_ceiling_1gib"] = round(gbs / hc["gib_read_write_64_17"]["GBps"], 4)

    cpu = None
    if not args.no_cpu:
        import oracle  # CPU baseline leg only
        cores = len(os.sched_getaffinity(0))
        oracle.transform_quant(x_bits[:64], lu, oracle.STAGED32, threads=cores)  # warm
        times = []
        deadline = time.perf_counter() + 10.0
        while len(times) < 3 or (time.perf_counter() < deadline and len(times) < 20):
            t0 = time.perf_counter()
            oracle.transform_quant(x_bits, lu, oracle.STAGED32, threads=cores)
            times.append(time.perf_counter() - t0)
        tmed = sorted(times)[len(times) // 2]
        cpu = {"value": round(nbytes / tmed / 1e9, 4), "unit": "GB/s", "cores": cores,
               "kind": "oracle",
               "sample": f"the whole {T}x{d} workload, oracle fixed-fp32-order mode, "
                         f"median of {len(times)} runs on {cores} threads"}
        # the same mode on one thread, and the fp64 definition mode on all
        # threads over the first 512 rows (bounded CPU time)
        one = []
        for _ in range(3):
            t0 = time.perf_counter()
            oracle.transform_quant(x_bits, lu, oracle.STAGED32, threads=1)
            one.append(time.perf_counter() - t0)
        rows = min(512, T)
        sub_bytes = nbytes * rows / T
        dense = []
        for _ in range(3):
            t0 = time.perf_counter()
            oracle.transform_quant(x_bits[:rows], lu, oracle.DENSE64, threads=cores)
            dense.append(time.perf_counter() - t0)
        cpu["single_thread_value"] = round(nbytes / sorted(one)[1] / 1e9, 4)
        cpu["dense64_value"] = round(sub_bytes / sorted(dense)[1] / 1e9, 4)
        cpu["dense64_sample"] = f"first {rows} rows, fp64 definition mode, median of 3 on {cores} threads"
        cpu["cpu_model"] = _cpu_model()
        if not args.no_peers:
            cpu["peers"] = oracle_peer_times(oracle, args.workload, x_bits, lu, mult, cores)

    line = {
        "metric": f"fused Kron-transform+MXFP4 quantize GB/s & % HBM peak, {T}x{d} bf16, 1 GPU",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}_{T}x{d}", "tokens": T, "channels": d,
                   "blocks_per_row": nb, "input": "bf16", "output": "mxfp4 (e2m1 + e8m0/32)",
                   "rotating_buffer_sets": R, "parallelism": "single GPU"},
        "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "tokens_per_s": round(T / (ms * 1e-3), 1),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "peers": extra,
        "kernel_source_hash": src_hash,
    }
    print(json.dumps(line), flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(json.dumps(line) + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
