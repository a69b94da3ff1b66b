"""Benchmark of the block-scaled FP8 expert layer on one MI355X.

Default workload: the fully occupied layer, 32 experts, hidden 7168,
intermediate 2048, top-8, 4096 live of 4096 tokens, fp32 activation scales,
plain SwiGLU, weights FP8 E4M3 with 128x128 fp32 block scales: the
full-expert benchmark shape of vLLM PR #59128 (SM100 on B200), the
compute-bound case. One step is one whole forward of the layer (align, act
quant, FC1, SiLU*up+quant, FC2, top-k combine), replayed from a captured HIP
graph with all inputs resident in HBM. Before every step the L2 and the
256 MB Infinity Cache are flushed by reading 1 GiB of unrelated data, so
weights stream from HBM (the pages time with a cold L2, vLLM PR #59128, SM100
on B200). A read leaves the caches clean: flushing by writing would leave
dirty lines whose write-back competes with the layer's own reads.

Printed: one JSON line. `value` is the median cold layer latency in
microseconds as the kernel span of one replay on the GPU timeline: two
one-thread device-clock marks captured at both ends of the graph (the pages
time the span of the layer's kernels, vLLM PR #59128, SM100 on B200). HIP
events around each replay, which add the host-side graph launch latency,
are reported beside it (`latency_us.events_median`). `ms_per_step` is the
wall clock of the bracketed timed loop divided by the steps (it includes the
flush). `roofline` describes the dominant kernel, timed on its own with HIP
events on the stream it runs on: on the decode path the layer is one kernel
(routing, quantization, FC1, SiLU, a grid barrier, FC2 and the combine), so
it is that kernel; elsewhere it is the FC1 grouped GEMM. `per_config` holds
the same layer span for every workload and variant, each with its live-row
TFLOP/s and minimum-bytes HBM rate as fractions of the peaks. `cpu_baseline`
is the CPU oracle on a bounded sample of the headline workload.
"""

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense FP8 MFMA, published
# The pages' own latencies, other GPUs: context only, never a target.
PAGES_CONTEXT_US = {
    "full:4096": {"B200": 1509.025, "H200": 2646.141, "source": "vLLM PR #59128, SM100 on B200 / SM90 on H200"},
    "padded:16": {"B200": 347.456, "H200": 438.144, "source": "vLLM PR #59128, SM100 on B200 / SM90 on H200"},
    "decode:4": {"H200": 64.7, "source": "TensorRT-LLM PR #21250, Performance"},
    "decode:1": {"H200": 28.7, "source": "TensorRT-LLM PR #21250, Performance"},
    "sweep:1": {"Hopper": 36.9, "source": "vLLM PR #65794, layer-time table"},
    "sweep:8": {"Hopper": 92.4, "source": "vLLM PR #65794, layer-time table"},
    "sweep:64": {"Hopper": 280.9, "source": "vLLM PR #65794, layer-time table"},
    "sweep:256": {"Hopper": 337.8, "source": "vLLM PR #65794, layer-time table"},
    "sweep:1024": {"Hopper": 438.0, "source": "vLLM PR #65794, layer-time table"},
    "sweep:4096": {"Hopper": 947.7, "source": "vLLM PR #65794, layer-time table"},
}
FLUSH_BYTES = 1 << 30
MALL_BYTES = 256 << 20       # MI355X Infinity Cache
CAL_BYTES = 256 << 20        # calibration copy for the HBM traffic counters


# SQ_VALU_MFMA_BUSY_CYCLES sums the busy cycles of every SIMD's matrix core
# (256 CUs x 4 SIMDs); GRBM_GUI_ACTIVE sums the active cycles of the 8 XCDs.
MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_LDS_BANK_CONFLICT",
                 "GRBM_GUI_ACTIVE")
N_SIMDS, N_XCDS = 1024, 8


def traffic_file(workload_key):
    """profiles/ file of the dominant kernel's traffic summary of a workload,
    e.g. roofline_kernel_decode_t4_fp32_traffic.json for decode:T4:fp32."""
    return "roofline_kernel_" + workload_key.replace(":", "_").lower() + "_traffic.json"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="full",
                    choices=["tiny", "decode", "padded", "full", "sweep"])
    ap.add_argument("--tokens", type=int, default=None, help="live tokens (default per config)")
    ap.add_argument("--t-cap", type=int, default=None,
                    help="token capacity (default: the config's, or --tokens); live tokens are capped by it")
    ap.add_argument("--fmt", default=None, help="activation scale format")
    ap.add_argument("--act", default="swiglu")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the per-config latency table")
    ap.add_argument("--config-steps", type=int, default=20,
                    help="timed replays per entry of the per-config table")
    ap.add_argument("--no-flush", action="store_true", help="keep caches warm between steps")
    ap.add_argument("--kernel-reps", type=int, default=50)
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs of this command (FETCH_SIZE, then "
                         "WRITE_SIZE) into the FC1 traffic file under profiles/, then exit")
    ap.add_argument("--counters-from", metavar="PMC_DIR",
                    help="summarise a rocprofv3 --pmc run of this command with "
                         f"{' '.join(MFMA_COUNTERS)} into the grouped GEMMs' MFMA utilisation "
                         "file under profiles/, then exit")
    return ap.parse_args()


DEFAULT_TOKENS = {"tiny": (8, 8), "decode": (4, 4), "padded": (512, 16), "full": (4096, 4096),
                  "sweep": (4096, 4096)}


def live_stats(ids, t_live, num_experts):
    import numpy as np
    flat = ids[:t_live].reshape(-1)
    flat = flat[(flat >= 0) & (flat < num_experts)]
    return len(np.unique(flat)), len(flat)


def algorithmic(cfg, n_live_experts, pairs, t_live, weight_fmt="e4m3"):
    """Bytes the layer must move at least, and FLOPs on live rows only.

    Per expert: FC1 codes 2I*H + fp32 block scales (2I/128)(H/128)*4, FC2
    codes H*I + (H/128)(I/128)*4 (MXFP4: half a byte per weight and one
    scale byte per 32). Plus BF16 x in and BF16 out (2*T*H each).
    FLOPs: FC1 2*P*2I*H + FC2 2*P*H*I = 6*P*H*I.
    """
    H, I = cfg.hidden, cfg.inter
    if weight_fmt == "mxfp4":
        per_expert = 3 * I * H // 2 + 3 * I * H // 32
    else:
        per_expert = 2 * I * H + (2 * I // 128) * (H // 128) * 4 + H * I + (H // 128) * (I // 128) * 4
    bmin = n_live_experts * per_expert + 2 * t_live * H * 2
    flops = 6 * pairs * H * I
    return bmin, flops


def fc1_bytes(cfg, n_live_experts, pairs):
    """Algorithmic bytes of one FC1 launch: live experts' FC1 codes + scales,
    the gathered A rows (codes + fp32 scales) and the BF16 output rows."""
    H, I = cfg.hidden, cfg.inter
    per_expert = 2 * I * H + (2 * I // 128) * (H // 128) * 4
    return n_live_experts * per_expert + pairs * (H + (H // 128) * 4) + pairs * 2 * I * 2


def fc1_decode_bytes(cfg, n_live_experts, pairs, t_live):
    """Algorithmic bytes of one decode-path FC1 launch (routing, activation
    quantization, FC1 and SiLU): live experts' FC1 codes + scales, the BF16
    token rows read, the codes + fp32 scales written, the BF16 C1 rows and the
    fp32 SiLU(gate)*up rows."""
    H, I = cfg.hidden, cfg.inter
    per_expert = 2 * I * H + (2 * I // 128) * (H // 128) * 4
    return (n_live_experts * per_expert + t_live * H * 2 + t_live * (H + (H // 128) * 4)
            + pairs * 2 * I * 2 + pairs * I * 4)


def decode_layer_bytes(cfg, n_live_experts, pairs, t_live):
    """Algorithmic bytes of the one-launch decode layer: the FC1 launch's
    bytes (fc1_decode_bytes), the live experts' FC2 codes + scales, the fp32
    SiLU(gate)*up rows read back, the FC2 input codes + fp32 scales and the
    BF16 FC2 rows written to the workspace, the routing weights read and the
    BF16 output rows written."""
    H, I = cfg.hidden, cfg.inter
    per_expert = H * I + (H // 128) * (I // 128) * 4
    return (fc1_decode_bytes(cfg, n_live_experts, pairs, t_live) + n_live_experts * per_expert
            + pairs * I * 4 + pairs * (I + (I // 128) * 4) + pairs * H * 2 + pairs * 4
            + t_live * H * 2)


KERNEL_SOURCES = ("gemm.hip", "fc1_decode.hip", "gemm_device.h", "fc2_decode.h", "device_common.h",
                  "quant_device.h", "kernels.h")


def kernel_source_hash():
    """Hash of the code the dominant kernels compile from (the traffic and
    counter summaries are keyed by it), with comments and whitespace removed,
    so that editing a comment does not make a measurement stale."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "block_fp8_mixture_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(name.encode() + b"\0" + " ".join(text.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(workload_key):
    """HBM traffic of the FC1 kernel from the committed rocprofv3 --pmc summary,
    used only if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", traffic_file(workload_key))
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("gemm_source_sha256_16") != kernel_source_hash() or d.get("workload") != workload_key:
        return None
    return d.get("bytes_per_launch")


def _counter_rows(run_dir, counter):
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    per = {}
    for row in csv.DictReader(open(files[0])):
        if row["Counter_Name"] != counter:
            continue
        key = int(row["Dispatch_Id"])
        name, val = per.get(key, (row["Kernel_Name"], 0.0))
        per[key] = (name, val + float(row["Counter_Value"]))
    return per


def traffic_from(args, fetch_dir, write_dir):
    """FC1 HBM bytes per launch from FETCH_SIZE / WRITE_SIZE runs (KiB per
    dispatch), each scaled by what the same counter reads for the bench's
    256 MiB device copy (the last three copy dispatches of the run)."""
    fmt = args.fmt or __import__("synth").get(args.config).scale_fmts[0]
    t_cap, t_live = DEFAULT_TOKENS[args.config]
    if args.tokens is not None:
        t_cap = t_live = args.tokens
    if args.t_cap is not None:
        t_cap = args.t_cap
        t_live = min(t_live, t_cap)
    want = f"<{'true' if fmt == 'ue8m0' else 'false'}, true"
    want_dec = f"fc1_decode_kernel<{ {'fp32': 0, 'pow2': 1, 'ue8m0': 2}[fmt] }, true,"
    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = _counter_rows(d, counter)
        fc1 = [v for n, v in per.values() if want_dec in n]
        if not fc1:  # the FC1 GEMM: of its kernels, the one that moves the most bytes
            groups = {}
            for n, v in per.values():
                if ("gemm_stream_kernel" in n or "gemm_tiled_kernel" in n) and want in n:
                    groups.setdefault(n, []).append(v)
            if groups:
                fc1 = max(groups.values(), key=sum)
        # the calibration copies are the run's last three copy dispatches
        copies = [per[k][1] for k in sorted(per) if "copyBuffer" in per[k][0]][-3:]
        if not fc1 or not copies:
            raise SystemExit(f"{counter}: FC1 or calibration copy dispatches missing")
        kib = statistics.median(fc1)
        cal_kib = statistics.median(copies)
        scale = (CAL_BYTES / 1024.0) / cal_kib
        out[counter] = {"kib_per_dispatch": round(kib, 1), "dispatches": len(fc1),
                        "copy_kib": round(cal_kib, 1), "scale": round(scale, 4),
                        "bytes": int(kib * 1024 * scale)}
    res = {"workload": f"{args.config}:T{t_live}:{fmt}", "gemm_source_sha256_16": kernel_source_hash(),
           "bytes_per_launch": out["FETCH_SIZE"]["bytes"] + out["WRITE_SIZE"]["bytes"],
           "counters": out}
    path = os.path.join(ROOT, "profiles", traffic_file(res["workload"]))
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(json.dumps(res))


def counters_from(args, pmc_dir):
    """MFMA utilisation of the grouped GEMMs from one rocprofv3 --pmc run with
    MFMA_COUNTERS: per kernel, the medians over its dispatches of the matrix
    cores' busy fraction (busy cycles per SIMD over active cycles), the clock
    those cycles imply, FP8 MFMA ops and LDS bank-conflict cycles."""
    import csv
    import glob
    import re
    files = glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {pmc_dir}")
    per = {}
    for row in csv.DictReader(open(files[0])):
        key = int(row["Dispatch_Id"])
        d = per.setdefault(key, {"name": row["Kernel_Name"],
                                 "us": (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3})
        d[row["Counter_Name"]] = d.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    fmt = args.fmt or __import__("synth").get(args.config).scale_fmts[0]
    t_cap, t_live = DEFAULT_TOKENS[args.config]
    if args.tokens is not None:
        t_cap = t_live = args.tokens
    kernels = {}
    for d in per.values():
        n = d["name"]
        if "gemm_tiled_kernel" not in n and "gemm_stream_kernel" not in n and "fc1_decode_kernel" not in n:
            continue
        cyc = d.get("GRBM_GUI_ACTIVE", 0.0) / N_XCDS
        if cyc <= 0 or d["us"] <= 0:
            continue
        m = re.search(r"(\w+_kernel<[^()]*?>)\(", n)
        k = kernels.setdefault(m.group(1) if m else n, {"dispatches": 0, "us": [], "busy": [], "ghz": [],
                                                   "mops_f8": [], "lds_bank_conflict_cycles": []})
        k["dispatches"] += 1
        k["us"].append(d["us"])
        k["busy"].append(d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / N_SIMDS / cyc)
        k["ghz"].append(cyc / d["us"] / 1e3)
        k["mops_f8"].append(d.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0))
        k["lds_bank_conflict_cycles"].append(d.get("SQ_LDS_BANK_CONFLICT", 0.0))
    out = {}
    for n, k in kernels.items():
        med = {m: statistics.median(k[m]) for m in ("us", "busy", "ghz", "mops_f8", "lds_bank_conflict_cycles")}
        out[n] = {"dispatches": k["dispatches"], "median_us": round(med["us"], 2),
                  "mfma_busy": round(med["busy"], 4), "clock_ghz": round(med["ghz"], 3),
                  "busy_x_clock_over_peak_clock": round(med["busy"] * med["ghz"] / 2.4, 4),
                  "mfma_mops_f8": med["mops_f8"], "lds_bank_conflict_cycles": med["lds_bank_conflict_cycles"]}
    res = {"workload": f"{args.config}:T{t_live}:{fmt}", "gemm_source_sha256_16": kernel_source_hash(),
           "counters": list(MFMA_COUNTERS), "kernels": out}
    path = os.path.join(ROOT, "profiles", "mfma_counters_" + res["workload"].replace(":", "_").lower() + ".json")
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(json.dumps(res))


def cpu_baseline(cfg, x, ids, w, t_live, fmt, act, lim, weights):
    """The oracle on a bounded sample of the workload, on the host's cores.

    The whole 4096-token layer would keep the oracle busy for minutes, so it
    runs on the first S1 and S2 tokens of the same inputs (S2 = 4 S1, each
    about 5-15 s) and the time of the full token count is extrapolated
    linearly from those two points (the oracle's per-expert weight decoding is
    a fixed cost, its GEMMs grow with the tokens). Small workloads run whole.
    The BLAS threads are the process's CPU affinity set.
    """
    import numpy as np
    import oracle
    cores = len(os.sched_getaffinity(0))
    (w1q, w1s), (w2q, w2s) = weights

    def run(n):
        t0 = time.perf_counter()
        oracle.forward(x[:n], ids[:n], w[:n], (w1q, w1s), (w2q, w2s), n, cfg.align_rows, fmt, act,
                       lim)
        return time.perf_counter() - t0

    if t_live <= 64:
        runs = [run(t_live) for _ in range(3)]
        value = statistics.median(runs)
        sample = (f"whole layer, all {t_live} tokens of the benchmarked workload, median of 3 runs "
                  f"of oracle.forward (numpy fp64)")
    else:
        s1 = max(t_live // 32, 16)
        s2 = 4 * s1
        t1, t2 = run(s1), run(s2)
        slope = (t2 - t1) / (s2 - s1)
        value = t2 + slope * (t_live - s2)
        sample = (f"oracle.forward (numpy fp64) on the first {s1} and {s2} of the {t_live} tokens "
                  f"({t1:.1f} s and {t2:.1f} s), extrapolated linearly to {t_live} tokens")
    try:  # the BLAS the oracle's fp64 GEMMs ran on
        b = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except Exception:  # an older numpy without the dict form
        blas = "unknown"
    return {"value": round(value * 1e6, 1), "unit": "us", "cores": cores, "kind": "oracle",
            "blas": blas, "sample": sample}


class Marks:
    """Device-clock marks around a captured layer (bench_clock.hip)."""

    def __init__(self, torch, cap):
        import ctypes
        self.torch = torch
        self.lib = ctypes.CDLL(os.path.join(ROOT, "block_fp8_mixture_amd", "libmoebench.so"))
        self.lib.moe_bench_mark.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint32,
                                            ctypes.c_int, ctypes.c_void_p]
        self.lib.moe_bench_clock_hz.restype = ctypes.c_int64
        self.cap = cap
        dev = torch.device("cuda", 0)
        self.slots = torch.zeros(cap, dtype=torch.int64, device=dev)
        self.ctr = torch.zeros(1, dtype=torch.int32, device=dev)

    def mark(self, closing):
        if self.lib.moe_bench_mark(self.slots.data_ptr(), self.ctr.data_ptr(), self.cap,
                                   int(closing), self.torch.cuda.current_stream().cuda_stream) != 0:
            raise RuntimeError("device-clock mark launch failed")

    def spans_us(self, n):
        hz = self.lib.moe_bench_clock_hz()
        m = self.slots[:2 * n].cpu().numpy().reshape(-1, 2)
        if hz <= 0 or int(self.ctr.item()) != 2 * n or (m[:, 1] <= m[:, 0]).any():
            raise RuntimeError("device-clock marks incomplete")
        return sorted(((m[:, 1] - m[:, 0]) * 1e6 / hz).tolist())


def attainable_peaks(torch):
    """This GPU's attainable peaks, measured by the benchmark library's probes
    (bench_clock.hip): a streaming read of 1 GiB (HBM-resident: larger than
    L2 and the 256 MB Infinity Cache; 2, 4, 8 or 16 workgroups of 256 threads
    per CU, eight 16-byte loads in flight per thread, the best of the four)
    and an FP8 MFMA-only loop (one 8-wave workgroup per CU, four independent
    32x32x64 accumulators per wave). Best of three runs each, after one
    warm-up run."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "block_fp8_mixture_amd", "libmoebench.so"))
    lib.moe_bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                          ctypes.c_int, ctypes.c_void_p]
    lib.moe_bench_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    dev = torch.device("cuda", 0)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream().cuda_stream

    def best(launch):
        ts = []
        for _ in range(4):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            if launch() != 0:
                raise RuntimeError("probe launch failed")
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return min(ts[1:])
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    sink = torch.empty(16 * cus * 256 + cus * 512, dtype=torch.int32, device=dev)
    t_read = min(best(lambda: lib.moe_bench_stream_read(src.data_ptr(), nbytes, sink.data_ptr(), b, stream))
                 for b in (2 * cus, 4 * cus, 8 * cus, 16 * cus))
    del src
    iters = 10000
    t_mfma = best(lambda: lib.moe_bench_mfma_loop(iters, sink.data_ptr(), cus, stream))
    mfma_flops = cus * 8 * 4 * iters * 2 * 32 * 32 * 64
    return {"hbm_read_gbs": round(nbytes / t_read / 1e9, 1),
            "fp8_mfma_tflops": round(mfma_flops / t_mfma / 1e12, 1),
            "method": "streaming read of 1 GiB (best of 2-16 workgroups per CU); FP8 MFMA-only loop (32x32x64, 4 accumulators per "
                      "wave, 8 waves per CU); best of 3 runs each (bench_clock.hip)"}


def time_layer(torch, fwd, steps, warmup, flush_caches, record_events=True):
    """Captures fwd() between two device-clock marks and replays it `steps`
    times after `warmup` replays, flushing the caches before each. Returns the
    sorted spans (us), the sorted HIP-event times (us) and the wall time (s)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            fwd()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    marks = Marks(torch, 2 * (steps + warmup + 8))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        marks.mark(False)
        fwd()
        marks.mark(True)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        flush_caches()
        graph.replay()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    marks.ctr.zero_()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for i in range(steps):
        flush_caches()
        starts[i].record(stream)
        graph.replay()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ev = sorted(a.elapsed_time(b) * 1e3 for a, b in zip(starts, ends))
    spans = marks.spans_us(steps)
    del graph
    return spans, ev, wall


def pct(v, q):
    return v[int(q * (len(v) - 1))]


# Entries of the per-config table: (workload, token capacity, live tokens,
# activation scales, activation, clamp limit[, rows per expert of the
# batched masked-M layout[, weight format]]).
PER_CONFIG = [
    ("tiny", 8, 8, "fp32", "swiglu", float("inf")),
    ("decode", 1, 1, "fp32", "swiglu", float("inf")),
    ("decode", 4, 4, "fp32", "swiglu", float("inf")),
    ("decode", 4, 4, "fp32", "swiglu_clamp", 7.0),
    ("padded", 512, 16, "fp32", "swiglu", float("inf")),
    ("padded", 512, 16, "ue8m0", "swiglu", float("inf")),
    ("full", 4096, 4096, "fp32", "swiglu", float("inf")),
    ("full", 4096, 4096, "ue8m0", "swiglu", float("inf")),
] + [("sweep", m, m, f, "swiglu", float("inf"))
     for m in (1, 8, 64, 256, 1024, 4096) for f in ("fp32", "pow2")] + [
    # the batched masked-M layout ([E, cap] rows, masked_m live; vLLM PR
    # #65794, Details, batched experts): a low-latency dispatch's capacity
    # and the fully occupied layer with room for 1.5x the mean expert load
    ("padded", 512, 16, "fp32", "swiglu", float("inf"), 64),
    ("full", 4096, 4096, "fp32", "swiglu", float("inf"), 1536),
    # MXFP4 weights (E2M1 codes, E8M0 scales per 32 along K) with FP8 activations
    ("decode", 1, 1, "fp32", "swiglu", float("inf"), 0, "mxfp4"),
    ("decode", 4, 4, "fp32", "swiglu", float("inf"), 0, "mxfp4"),
    ("padded", 512, 16, "fp32", "swiglu", float("inf"), 0, "mxfp4"),
    ("full", 4096, 4096, "fp32", "swiglu", float("inf"), 0, "mxfp4"),
    # with UE8M0 token scales the matrix cores apply both scales
    ("full", 4096, 4096, "ue8m0", "swiglu", float("inf"), 0, "mxfp4"),
]


def main():
    args = parse()
    if args.traffic_from:
        traffic_from(args, *args.traffic_from)
        return
    if args.counters_from:
        counters_from(args, args.counters_from)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): this build measures the "
              f"expert layer on a single MI355X; how it would shard is described in DESIGN.md",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import block_fp8_mixture_amd as moe
    import synth

    dev = torch.device("cuda", 0)

    def up(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    flush_sink = torch.empty((), dtype=torch.float32, device=dev)

    def flush_caches():
        if not args.no_flush:
            torch.sum(flush, dim=0, out=flush_sink)

    weights_cache = {}

    def weights_for(name, weight_fmt="e4m3"):
        key = (name, weight_fmt)
        if key not in weights_cache:
            weights_cache.clear()
            torch.cuda.empty_cache()
            cfg_w = synth.get(name)
            gen = synth.ExpertWeightsMxfp4 if weight_fmt == "mxfp4" else synth.ExpertWeights
            host = gen(cfg_w).stacked(threads=min(16, len(os.sched_getaffinity(0))))
            weights_cache[key] = (host, [up(a) for a in (host[0][0], host[0][1], host[1][0], host[1][1])])
        return weights_cache[key]

    def layer_inputs(name, t_cap, t_live, fmt, act, lim, expert_cap=0, weight_fmt="e4m3"):
        cfg_l = synth.get(name)
        x_l, ids_l, w_l = synth.make_workload(cfg_l, t_cap)
        _, d_w_l = weights_for(name, weight_fmt)
        E_l, H_l, I_l, K_l = cfg_l.num_experts, cfg_l.hidden, cfg_l.inter, cfg_l.topk
        lay_l = moe.moe_workspace_plan(E_l, H_l, I_l, K_l, t_cap, cfg_l.align_rows, 0, fmt, act, lim,
                                       expert_cap=expert_cap, weight_fmt=weight_fmt)
        ws_l = torch.zeros(lay_l["total"], dtype=torch.uint8, device=dev)
        out_l = torch.zeros((t_cap, H_l), dtype=torch.int16, device=dev)
        dx_l, dids_l, dw_l = up(x_l), up(ids_l), up(w_l)
        dlive_l = up(np.array([t_live], np.int32))

        def fwd():
            moe.moe_forward(dx_l, dids_l, dw_l, *d_w_l, fmt, act, lim, cfg_l.align_rows, 0,
                            t_live=dlive_l, out=out_l, workspace=ws_l, expert_cap=expert_cap,
                            weight_fmt=weight_fmt)
        return cfg_l, (x_l, ids_l, w_l), fwd, lay_l, ws_l, (dx_l, dids_l, dw_l, dlive_l), out_l

    def rates(cfg_l, ids_l, t_live, span_us, weight_fmt="e4m3"):
        n_e, pairs_l = live_stats(ids_l, t_live, cfg_l.num_experts)
        bmin_l, flops_l = algorithmic(cfg_l, n_e, pairs_l, t_live, weight_fmt)
        return {"live_experts": n_e, "live_pairs": pairs_l,
                "live_tflops": round(flops_l / (span_us * 1e-6) / 1e12, 3),
                "frac_fp8_peak": round(flops_l / (span_us * 1e-6) / 1e12 / FP8_PEAK_TFLOPS, 4),
                "hbm_gbs_min_bytes": round(bmin_l / (span_us * 1e-6) / 1e9, 1),
                "frac_hbm_peak": round(bmin_l / (span_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "min_bytes": bmin_l, "live_flops": flops_l}

    # ---- the headline workload
    cfg = synth.get(args.config)
    t_cap, t_live = DEFAULT_TOKENS[args.config]
    if args.tokens is not None:
        t_cap = t_live = args.tokens
    if args.t_cap is not None:
        t_cap = args.t_cap
        t_live = min(t_live, t_cap)
    fmt = args.fmt or cfg.scale_fmts[0]
    act = args.act
    lim = 7.0 if act != "swiglu" else float("inf")
    E, H, I, K = cfg.num_experts, cfg.hidden, cfg.inter, cfg.topk
    t0 = time.perf_counter()
    cfg, (x, ids, w), fwd, lay, ws, (dx, dids, dw, dlive), out = layer_inputs(
        args.config, t_cap, t_live, fmt, act, lim)
    weights, d_w = weights_for(args.config)
    print(f"# inputs ready in {time.perf_counter() - t0:.1f}s", file=sys.stderr, flush=True)
    lat_us, ev_us, wall = time_layer(torch, fwd, args.steps, args.warmup, flush_caches)
    med, ev_med = statistics.median(lat_us), statistics.median(ev_us)
    p10, p90 = pct(lat_us, 0.1), pct(lat_us, 0.9)
    print(f"# layer kernel span median {med:.2f} us (p10 {p10:.2f}, p90 {p90:.2f}); events around "
          f"the replay {ev_med:.2f} us; over {args.steps} steps", file=sys.stderr, flush=True)

    # ---- dominant kernel alone: FC1 grouped GEMM on the forward's intermediates
    stream = torch.cuda.current_stream()
    n_live_e, pairs = live_stats(ids, t_live, E)
    R = lay["row_cap"]

    def ws_i32(name, n):
        return ws[lay[name]:lay[name] + 4 * n].view(torch.int32)
    counts, offsets = ws_i32("expert_counts", E), ws_i32("expert_offsets", E + 1)
    r2p = ws_i32("row_to_pair", R)
    xq = ws[lay["xq"]:lay["xq"] + t_cap * H].view(t_cap, H)
    sb = 1 if fmt == "ue8m0" else 4
    xs_raw = ws[lay["xs"]:lay["xs"] + (H // 128) * t_cap * sb]
    xs = (xs_raw if fmt == "ue8m0" else xs_raw.view(torch.float32)).view(H // 128, t_cap)
    c1 = torch.empty((R, 2 * I), dtype=torch.int16, device=dev)
    # On the decode path the whole layer is one kernel (within the one-launch
    # limits moe_forward launches the one-launch layer); it is timed
    # through moe_forward on a workspace of its own. Elsewhere the dominant
    # kernel is the FC1 grouped GEMM.
    ws_f = torch.empty_like(ws)
    fused = moe.decode_layer_applies(t_cap, K, H, I)
    out_f = torch.empty_like(out)

    # The kernel alone, back to back over rotating copies of its weights: the
    # copies' live experts together exceed L2 + the 256 MB Infinity Cache, so
    # every launch streams its weights from HBM, while back-to-back launches
    # keep the dispatch overhead out of the average (as a kernel trace
    # measures it).
    per_e = 2 * I * H + (2 * I // 128) * (H // 128) * 4
    if fused:
        per_e += H * I + (H // 128) * (I // 128) * 4
    live_w = max(n_live_e, 1) * per_e
    n_copies = int(min(8, max(2, -(-3 * MALL_BYTES // live_w) + 1)))
    idx = (0, 1, 2, 3) if fused else (0, 1)
    w_copies = [tuple(d_w[j] for j in idx)] + \
        [tuple(d_w[j].clone() for j in idx) for _ in range(n_copies - 1)]
    max_rows = min(pairs, R)

    def fc1(i):
        wc = w_copies[i % n_copies]
        if fused:
            moe.moe_forward(dx, dids, dw, *wc, fmt, act, lim, cfg.align_rows, 0, t_live=dlive,
                            out=out_f, workspace=ws_f)
        else:
            moe.moe_grouped_gemm_fp8(xq, xs, fmt, wc[0], wc[1], counts, offsets, R, a_row_map=r2p,
                                     a_row_div=K, max_rows_per_expert=max_rows, out=c1)
    for i in range(n_copies):
        fc1(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(args.kernel_reps):
        fc1(i)
    b.record(stream)
    torch.cuda.synchronize()
    k_avg = a.elapsed_time(b) * 1e3 / args.kernel_reps
    del w_copies
    fc1_b = decode_layer_bytes(cfg, n_live_e, pairs, t_live) if fused else fc1_bytes(cfg, n_live_e, pairs)
    fc1_flops = 6 * pairs * H * I if fused else 2 * pairs * 2 * I * H
    workload_key = f"{args.config}:T{t_live}:{fmt}"
    traffic = load_traffic(workload_key)
    tiled = pairs > 0 and pairs / max(n_live_e, 1) > moe.GEMM_TILES["stream_max_rows"]
    kname = ("gemm_tiled_kernel" if tiled else "gemm_stream_kernel") + \
        f"<{'true' if fmt == 'ue8m0' else 'false'}, true> (FC1)"
    if fused:
        wide = t_cap * (H + 16) > 24576 or t_cap * (H // 128) > 256  # the 4-deep ring variant
        kname = (f"fc1_decode_kernel<{ {'fp32': 0, 'pow2': 1, 'ue8m0': 2}[fmt] }, true, {4 if wide else 6}, false> "
                 "(the whole decode layer: routing, activation quantization, FC1, SiLU, "
                 "grid barrier, FC2, top-k combine)")
    if tiled:
        roof = {"kernel": kname, "bound": "mfma",
                "achieved": round(fc1_flops / (k_avg * 1e-6) / 1e12, 2), "peak": FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(fc1_flops / (k_avg * 1e-6) / 1e12 / FP8_PEAK_TFLOPS, 4)}
    else:
        roof = {"kernel": kname, "bound": "hbm",
                "achieved": round(fc1_b / (k_avg * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(fc1_b / (k_avg * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    roof.update({"traffic": traffic, "kernel_avg_us": round(k_avg, 3),
                 "algorithmic_bytes": fc1_b, "algorithmic_flops": fc1_flops})
    print(f"# dominant kernel alone: {k_avg:.2f} us, {roof['achieved']} {roof['unit']} "
          f"({roof['frac']:.3f} of peak)", file=sys.stderr, flush=True)

    # A plain 256 MiB device copy, so counter runs (FETCH_SIZE / WRITE_SIZE)
    # can be scaled by what the counters read for a copy of known size.
    cal_src = torch.ones(CAL_BYTES // 4, dtype=torch.float32, device=dev)
    cal_dst = torch.empty_like(cal_src)
    for _ in range(3):
        cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst, ws_f, out_f, c1
    att = attainable_peaks(torch)
    a_peak = att["fp8_mfma_tflops"] if roof["bound"] == "mfma" else att["hbm_read_gbs"]
    roof["attainable"] = a_peak
    roof["frac_attainable"] = round(roof["achieved"] / a_peak, 4)
    print(f"# attainable on this GPU: {att['hbm_read_gbs']} GB/s streaming read, "
          f"{att['fp8_mfma_tflops']} TFLOP/s FP8 MFMA loop; dominant kernel at "
          f"{roof['frac_attainable']:.3f} of its attainable peak", file=sys.stderr, flush=True)

    head_rates = rates(cfg, ids, t_live, med)
    ctx = PAGES_CONTEXT_US.get(f"{args.config}:{t_live}")
    res = {
        "metric": "MoE layer latency (us) + live-row TFLOP/s and HBM GB/s vs roofline",
        "value": round(med, 3),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3",
        "data": "synthetic",
        "config": {
            "workload": f"{args.config}: {E} experts, hidden {H}, intermediate {I}, top-{K}, "
                        f"{t_live} live of {t_cap} tokens, {fmt} activation scales, {act}",
            "experts": E, "hidden": H, "intermediate": I, "topk": K, "tokens": t_live,
            "token_capacity": t_cap, "act_scale_fmt": fmt, "activation": act,
            "cache": "warm" if args.no_flush else "flushed before every step",
        },
        "latency_us": {"median": round(med, 3), "p10": round(p10, 3), "p90": round(p90, 3),
                       "events_median": round(ev_med, 3)},
        "live_experts": head_rates["live_experts"],
        "live_pairs": head_rates["live_pairs"],
        "live_tflops": head_rates["live_tflops"],
        "hbm_gbs_min_bytes": head_rates["hbm_gbs_min_bytes"],
        "frac_fp8_peak": head_rates["frac_fp8_peak"],
        "frac_hbm_peak": head_rates["frac_hbm_peak"],
        "roofline": roof,
        "attainable_peaks": att,
        "pages_context_us": ctx,
    }
    del fwd, ws, out, dx, dids, dw, dlive, d_w

    # ---- every workload and variant, the same protocol with fewer replays
    if not args.no_per_config:
        table = []
        for name, tc, tl, f, ac, li, *extra in PER_CONFIG:
            cap = extra[0] if extra else 0
            wfmt = extra[1] if len(extra) > 1 else "e4m3"
            cfg_l, (xl, idsl, wl), fwd_l, lay_l, ws_l, _, out_l = layer_inputs(name, tc, tl, f, ac, li,
                                                                               cap, wfmt)
            spans, evs, _ = time_layer(torch, fwd_l, args.config_steps, 3, flush_caches)
            m = statistics.median(spans)
            ent = {"workload": name, "tokens": tl, "token_capacity": tc, "act_scale_fmt": f,
                   "activation": ac, "span_us": round(m, 2), "p10_us": round(pct(spans, 0.1), 2),
                   "p90_us": round(pct(spans, 0.9), 2), "events_us": round(statistics.median(evs), 2),
                   "weights": wfmt,
                   "path": ("batched masked-M" if cap else
                            "one launch" if moe.decode_layer_applies(tc, cfg_l.topk, cfg_l.hidden, cfg_l.inter, wfmt)
                            else "general")}
            if cap:
                ent["expert_cap"] = cap
                ovf = int(ws_l[lay_l["overflow"]:lay_l["overflow"] + 4].view(torch.int32).item())
                ent["pairs_dropped"] = ovf
            ent.update(rates(cfg_l, idsl, tl, m, wfmt))
            # the bars: HBM at <= 32 tokens, FP8 MFMA at the fully occupied
            # layer; the tiny layer is launch-bound and reported only
            bar = None if name == "tiny" else ("hbm" if tl <= 32 else ("mfma" if name == "full" else None))
            ent["bar"] = bar
            c = PAGES_CONTEXT_US.get(f"{name}:{tl}")
            if c:
                ent["pages_context_us"] = c
            table.append(ent)
            print(f"# per-config {name} T={tl}/{tc} {f} {ac}{f' cap {cap}' if cap else ''}"
                  f"{' ' + wfmt + ' weights' if wfmt != 'e4m3' else ''}: {m:.1f} us, "
                  f"{ent['frac_fp8_peak']:.3f} FP8, {ent['frac_hbm_peak']:.3f} HBM",
                  file=sys.stderr, flush=True)
            del fwd_l, ws_l, out_l
        res["per_config"] = table
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, x, ids, w, t_live, fmt, act, lim, weights)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
