#!/usr/bin/env python3
"""Benchmark of the W1.58A8 BitLinear forward on one MI355X.

Headline (`value`): HBM GB/s at M = 1 over one step = one decode pass over a
BitNet-100B-shaped slice of 4 layers, each layer's four BitLinears in order,
    QKV 8192->10240 (plain absmax input), O 8192->8192 (subln RMSNorm input),
    up 8192->28672 (plain), down 28672->8192 (ReLU^2 + subln RMSNorm input),
each a call of the fused entry (input quantization, product and rescale), with its
own latent weights per layer (620.8 MB packed per slice) and two copies of the whole
slice rotated step by step (1.24 GB > 256 MB MALL + 32 MB L2), so every step streams its
weights from HBM. Bytes per BitLinear = N*K/4 packed weights + 4 (gamma) + 4*M*K fp32
input [+ 4*K gain] + 4*M*N fp32 output. Every graph is captured before the timed region;
the timed region replays whole graphs and is timed with HIP events on the launch stream
(bracketed by synchronizations), so `value` does not depend on the step count.

Second headline (`prefill`): int8 TOPS at M = 2048 over one step = the four BitLinear
products of a BitNet-2B-shaped layer (QKV 2560->3840, O 2560->2560, up 2560->6912,
down 6912->2560) on pre-quantized activations, timed the same way; ops = 2*M*N*K.

Also printed in the same JSON line:
  roofline      the dominant kernel of the headline step (the down projection, the
                longest launch) timed with HIP events around a graph of back-to-back
                launches over >= 1 GiB of rotating weights, vs 8 TB/s; `traffic` from the
                committed rocprofv3 FETCH_SIZE / WRITE_SIZE counters when they match the
                current kernel source, else null.
  prefill       the M = 2048 figure with its own roofline (int8 matrix cores, 5 POPS).
  cpu_baseline  the CPU oracle on the same bytes the GPU consumed (the first layer of the
                slice, copied back from the device), one thread and then all threads of the
                host share; its outputs are compared with the GPU's.
  extra         per-matrix kernel rates: the slice's matrices, the 2B layer at M in {1,4,8},
                the 100B matrices at M in {8, 32, 64}, prefill at M in {512, 2048}, five codes
                per byte, decode attention, the 30-layer 2B decode stack, packing, and the
                measured peaks of the calibration kernels.

Other modes:
  --profile roofline   only the dominant kernel plus a copy kernel of known size
                       (for rocprofv3 --pmc runs);
  --profile prefill    the same for the prefill figure's roofline kernel (the down
                       projection's GEMM at M = 2048);
  --summarize-pmc F W  turn two rocprofv3 counter CSVs into profiles/ text;
  --summarize-trace T S OUT  turn a rocprofv3 kernel trace and its stats CSV into a
                       profiles/ text (per kernel and grid: calls, average, median, min).
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W1.58A8 BitLinear: GEMV HBM GB/s (%peak) @M=1; int8 TOPS (%peak) @M=2048"
HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0
EPS = 1e-5
ROTATE_BYTES = 1 << 30

# (name, N, K, input mode) of a BitNet-b1.58-2B-shaped layer (hidden 2560, FFN 6912,
# 20 query heads and 5 key/value heads of 128)
LAYER_2B = [("qkv", 3840, 2560, "plain"), ("o", 2560, 2560, "norm"), ("up", 6912, 2560, "plain"),
            ("down", 2560, 6912, "relu2norm")]
# 100B-shaped layer (hidden 8192, FFN 28672)
LAYER_100B = [("qkv", 10240, 8192, "plain"), ("o", 8192, 8192, "norm"), ("up", 28672, 8192, "plain"),
              ("down", 8192, 28672, "relu2norm")]

# One GPU's share of the 100B slice under an 8-way tensor-parallel split (design only; the
# collectives are not part of this build): QKV and up split along N (no exchange), O and
# down along K (an exact int32 all-reduce of the partial products would follow).
LAYER_100B_TP8 = [("qkv", 1280, 8192, "plain"), ("o", 8192, 1024, "norm"), ("up", 3584, 8192, "plain"),
                  ("down", 8192, 3584, "relu2norm")]

SLICE_LAYERS = 4
PREFILL_M = 2048
DOMINANT = "down"      # the longest launch of the headline step: 100B down projection, M = 1
# What decides the measured GEMV's traffic: its kernel, the shared device helpers, and the
# GEMV launch-shape section of the API file (from its "forward dispatch" banner to the MFMA
# GEMM section), so edits elsewhere in the library do not invalidate the counter file.
KERNEL_SRC = ["ternary_weight_linear_w1_amd/csrc/gemv.hpp", "ternary_weight_linear_w1_amd/csrc/device_common.hpp"]
# the launch of one-token tiles (launch_k64 and the one-token dispatch) decides the measured kernel's grid
DISPATCH_SRC = ("ternary_weight_linear_w1_amd/csrc/bitlinear_api.hip", "forward dispatch", "// Two tokens per tile")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_down_100B_M1_traffic.txt")


# The same for the prefill figure's roofline kernel (the down projection's GEMM at M = 2048):
# the GEMM kernel, the shared helpers, and the GEMM tile choice in the API file.
PREFILL_DOMINANT = "down"
KERNEL_SRC_PREFILL = ["ternary_weight_linear_w1_amd/csrc/gemm.hpp", "ternary_weight_linear_w1_amd/csrc/device_common.hpp"]
DISPATCH_SRC_PREFILL = ("ternary_weight_linear_w1_amd/csrc/bitlinear_api.hip", "// Many tokens: int8 MFMA GEMM",
                        "// Few tokens on the matrix cores")
TRAFFIC_FILE_PREFILL = os.path.join(ROOT, "profiles", "gemm_down_2B_M2048_traffic.txt")


def kernel_hash(target="decode") -> str:
    h = hashlib.sha256()
    srcs, (path, start, end) = ((KERNEL_SRC, DISPATCH_SRC) if target == "decode"
                                else (KERNEL_SRC_PREFILL, DISPATCH_SRC_PREFILL))
    for p in srcs:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    with open(os.path.join(ROOT, path), "rb") as f:
        text = f.read()
    i = text.index(start.encode())
    h.update(text[i:text.index(end.encode(), i)])
    return h.hexdigest()[:16]


def layer_bytes(N, K, M, mode, fused=True, residual=False):
    """Algorithmic HBM bytes of one BitLinear: packed weights, gamma, activations in
    (fp32 through the prologue, [gate | up] rows of 2K when gated, or int8 codes and
    scales), the gain, and the fp32 output (read and written again by a residual add)."""
    b = N * K // 4 + 4 + 4 * M * N * (2 if residual else 1)
    b += 4 * M * K * (2 if mode == "gatednorm" else 1) if fused else (M * K + 4 * M)
    if mode in ("norm", "relu2norm", "gatednorm") and fused:
        b += 4 * K
    return b


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- setup

class Mat:
    """One BitLinear: packed weight copies, gamma, input, gain, output."""

    def __init__(self, torch, bl, datagen, cfg, idx, name, N, K, mode, M, copies, dev, layer=0):
        self.name, self.N, self.K, self.mode, self.M = name, N, K, mode, M
        w = datagen.gg_weights_torch(N, K, datagen.stream_id(cfg, layer, idx, 0), dev)
        packed, gamma = bl.bitlinear_pack_weights(w)
        del w
        self.gamma = gamma
        self.copies = [packed] + [packed.clone() for _ in range(copies - 1)]
        self.x = datagen.outlier_acts_torch(M, K, datagen.stream_id(cfg, layer, idx, 1), dev)
        self.gain = datagen.gains_torch(K, datagen.stream_id(cfg, layer, idx, 2), dev) if "norm" in mode else None
        self.relu2 = mode == "relu2norm"
        self.y = torch.empty((M, N), dtype=torch.float32, device=dev)
        self.xq = torch.empty((M, K), dtype=torch.int8, device=dev)
        self.s = torch.empty((M,), dtype=torch.float32, device=dev)
        need = bl.bitlinear_forward_f32_workspace_bytes(M, N, K)
        self.ws = torch.empty((need,), dtype=torch.uint8, device=dev) if need else None

    def fused(self, bl, c):
        bl.bitlinear_forward_f32(self.x, self.copies[c], self.gamma, self.gain, EPS, self.relu2, y=self.y,
                                 workspace=self.ws)

    def prequant(self, bl):
        bl.bitlinear_quantize_act(self.x, self.gain, EPS, self.relu2, xq=self.xq, scale=self.s)

    def forward(self, bl, c, workspace=None, split=True):
        bl.bitlinear_forward(self.xq, self.s, self.copies[c], self.gamma, y=self.y, workspace=workspace, split=split)

    def bytes(self, fused=True):
        return layer_bytes(self.N, self.K, self.M, self.mode, fused)


def n_copies(bytes_per_copy, multiple=1):
    c = max(2, math.ceil(ROTATE_BYTES / bytes_per_copy))
    return int(math.ceil(c / multiple) * multiple)


def time_kernel(torch, fn, copies, reps):
    """Average duration of one launch: `reps` launches captured back to back in a HIP
    graph (weight copies rotating), one replay timed with HIP events on the launch
    stream. The average includes the dispatch gap between consecutive kernels."""
    for i in range(min(reps, 4)):
        fn(i % copies)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(reps):
            fn(i % copies)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e-3 / reps


# ----------------------------------------------------------------------------- CPU baseline

def host_threads():
    """Threads of this process's CPU share (at most 16, the share of one GPU on the box)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(torch, mats, seconds=8.0):
    """The CPU oracle, as it stands, on the bytes the GPU consumed: the packed weights, gamma,
    inputs and gains of `mats` (one layer of the headline slice) are copied from the device,
    unpacked by the oracle, and each BitLinear's quantization + int64 product + rescale is
    run on the host, first on one thread, then with the output rows split over all threads
    of this process's CPU share (the oracle is called once per row range; ctypes releases
    the interpreter lock during the call). The oracle's outputs are compared with the
    GPU's (bit for bit on the plain path, 1e-6 relative on the subln path)."""
    import concurrent.futures
    import numpy as np
    import oracle
    host = []
    for m in mats:
        packed = m.copies[0].cpu().numpy()
        q, bad = oracle.unpack(packed, m.K)
        assert bad == 0
        x = m.x.cpu().numpy()
        gain = None if m.gain is None else m.gain.cpu().numpy()
        host.append((m, q, float(m.gamma.cpu().numpy()[0]), x, gain, m.y.cpu().numpy()))

    def quant(x, gain, mode):
        if mode == "plain":
            return oracle.quantize_act(x)
        return oracle.quantize_act_norm(x, gain, EPS, 1 if mode == "relu2norm" else 0)

    # parity of the sample on the GPU's own bytes
    match = {}
    for m, q, gamma, x, gain, ygpu in host:
        xq, s = quant(x, gain, m.mode)
        _, y = oracle.forward(xq, s, q, gamma)
        if m.mode == "plain":
            match[m.name] = bool(np.array_equal(y, ygpu))
        else:
            match[m.name] = bool(np.all(np.abs(y.astype(np.float64) - ygpu) <= 1e-6 * np.abs(y.astype(np.float64))))
    step_bytes = sum(m.bytes() for m, *_ in host)

    def one_pass(pool=None, nthreads=1):
        for m, q, gamma, x, gain, _ in host:
            xq, s = quant(x, gain, m.mode)
            if pool is None:
                oracle.forward(xq, s, q, gamma)
            else:
                bounds = np.linspace(0, m.N, nthreads + 1).astype(int)
                list(pool.map(lambda r: oracle.forward(xq, s, q[bounds[r]:bounds[r + 1]], gamma), range(nthreads)))

    def timed(pool, nthreads, budget):
        passes, t0 = 0, time.perf_counter()
        while True:
            one_pass(pool, nthreads)
            passes += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return passes, el

    p1, e1 = timed(None, 1, seconds)
    T = host_threads()
    with concurrent.futures.ThreadPoolExecutor(max_workers=T) as pool:
        pT, eT = timed(pool, T, seconds)
    names = "/".join("%s %dx%d" % (m.name, m.N, m.K) for m, *_ in host)
    return {"value": round(step_bytes * pT / eT / 1e9, 4), "unit": "GB/s", "cores": T, "kind": "oracle",
            "sample": "%d passes over layer 0 of the 100B slice at M=1 (%s; %.1f MB per pass, the bytes the GPU "
                      "consumed), quantize + int64 product + rescale on oracle-unpacked codes, output rows split over "
                      "%d threads, %.1f s" % (pT, names, step_bytes / 1e6, T, eT),
            "single_thread": {"value": round(step_bytes * p1 / e1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "sample": "%d passes, %.1f s" % (p1, e1)},
            "cpu_model": cpu_model(), "threads_available": host_threads(),
            "oracle_build": "gcc -O2 -std=c99 -ffp-contract=off -fno-fast-math (plain loops, no intrinsics)",
            "matches_gpu": match}


# ----------------------------------------------------------------------------- traffic

def read_traffic(target="decode"):
    path = TRAFFIC_FILE if target == "decode" else TRAFFIC_FILE_PREFILL
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_hash(target):
        return None
    try:
        return int(float(vals["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def summarize_trace(trace_csv, stats_csv, out, command="--steps 80 --warmup 8 --no-extra --no-cpu-baseline"):
    """Per (kernel, grid) durations from a rocprofv3 kernel trace (End - Start per
    dispatch) and the library rows of its stats table, as text for profiles/."""
    import csv
    import statistics
    rows = {}
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if "bl::" not in name:
                continue
            short = name.replace("void ", "").split("(")[0]
            wg = int(r.get("Workgroup_Size_X", r.get("Workgroup_Size", 256)) or 256)
            key = (short, int(r.get("Grid_Size_X", r.get("Grid_Size", 0))) // wg, int(r.get("Grid_Size_Y", 1)),
                   r.get("VGPR_Count", r.get("Arch_VGPR_Count", "")), r.get("LDS_Block_Size", r.get("LDS_Size", "")))
            rows.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    with open(out, "w") as f:
        f.write("# rocprofv3 kernel trace of bench.py (library kernels; durations End - Start per dispatch, us)\n")
        f.write("# command (GPU box, repository root in $R):\n")
        outdir = os.path.basename(os.path.dirname(os.path.abspath(trace_csv))) or "prof_bench"
        f.write("#   cd /tmp && rocprofv3 --kernel-trace --stats -d $R/gpurun_out/%s -o trace "
                "--output-format csv -- python3 $R/bench.py %s\n" % (outdir, command))
        f.write("#   python3 bench.py --summarize-trace <trace_kernel_trace.csv> <trace_kernel_stats.csv> <this file>%s\n"
                % ("" if command.startswith("--steps 80") else " --trace-command=%s" % command))
        f.write("# WGs = grid X / work-group size X (work-groups per launch row), gridY = grid Y (token tiles; "
                "attention: head groups)\n#\n")
        f.write("# %-48s %5s %5s %5s %6s %6s %8s %8s %8s\n" % ("kernel", "WGs", "gridY", "VGPR", "LDS", "calls", "avg_us",
                                                            "med_us", "min_us"))
        for key in sorted(rows):
            v = rows[key]
            f.write("  %-48s %5d %5d %5s %6s %6d %8.2f %8.2f %8.2f\n" % (key[0][:48], key[1], key[2], key[3], key[4], len(v),
                                                                      sum(v) / len(v), statistics.median(v), min(v)))
        f.write("\n# kernel stats (library rows)\n")
        with open(stats_csv) as g:
            lines = g.read().splitlines()
        f.write(lines[0] + "\n")
        for line in lines[1:]:
            if "bl::" in line:
                f.write(line + "\n")
    log("wrote %s" % out)


def summarize_pmc(fetch_csv, write_csv, copy_bytes, out, target="decode"):
    import csv

    def per_kernel(path, counter):
        rows = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter:
                    continue
                rows.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return rows

    fe = per_kernel(fetch_csv, "FETCH_SIZE")
    wr = per_kernel(write_csv, "WRITE_SIZE")
    # the measured kernel: the library kernel launched most often (200 times in --profile
    # roofline; the packing kernels of the setup run a few times)
    lib_k = [k for k in fe if "bl::" in k and ("gemm" in k) == (target == "prefill")]
    gk = [max(lib_k, key=lambda k: len(fe[k]))] if lib_k else []
    ck = [k for k in fe if "copy" in k.lower()]
    if len(gk) != 1 or not ck:
        raise SystemExit("could not identify kernels: %s" % list(fe))
    # the calibration copy is the largest copy dispatch (copy_bytes read, copy_bytes written)
    copyk = max(ck, key=lambda k: max(wr.get(k, [0.0])))
    copy_fetch_kib, copy_write_kib = max(fe[copyk]), max(wr[copyk])
    f_factor = copy_bytes / (copy_fetch_kib * 1024.0)
    w_factor = copy_bytes / (copy_write_kib * 1024.0)
    g_fetch_kib = sum(fe[gk[0]]) / len(fe[gk[0]])
    g_write_kib = sum(wr[gk[0]]) / len(wr[gk[0]])
    g_fetch = g_fetch_kib * 1024.0 * f_factor
    g_write = g_write_kib * 1024.0 * w_factor
    if target == "decode":
        N, K, mode = [(n, k, m) for (nm, n, k, m) in LAYER_100B if nm == DOMINANT][0]
        alg = layer_bytes(N, K, 1, mode)
        title = "the down-projection product (100B slice, %d->%d, M=1, fused ReLU^2+subln input)" % (K, N)
    else:
        N, K, mode = [(n, k, m) for (nm, n, k, m) in LAYER_2B if nm == PREFILL_DOMINANT][0]
        alg = layer_bytes(N, K, PREFILL_M, mode, fused=False)
        title = ("the down-projection GEMM (2B layer, %d->%d, M=%d, pre-quantized int8 activations)"
                 % (K, N, PREFILL_M))
    with open(out, "w") as f:
        f.write("# HBM traffic of %s\n" % title)
        f.write("# from two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by\n")
        f.write("# the same counter read for a plain copy kernel of %d bytes read and written.\n" % copy_bytes)
        f.write("# commands:\n")
        prof = "roofline" if target == "decode" else "prefill"
        f.write("#   rocprofv3 --pmc FETCH_SIZE -d gpurun_out/pmc_fetch -o fetch --output-format csv -- "
                "python3 bench.py --profile %s\n" % prof)
        f.write("#   rocprofv3 --pmc WRITE_SIZE -d gpurun_out/pmc_write -o write --output-format csv -- "
                "python3 bench.py --profile %s\n" % prof)
        f.write("#   python3 bench.py --summarize-pmc <fetch csv> <write csv>%s\n"
                % ("" if target == "decode" else " --pmc-target prefill"))
        f.write("gemv_kernel = %s\n" % gk[0])
        f.write("copy_kernel = %s\n" % copyk)
        f.write("copy_fetch_kib = %.1f\ncopy_write_kib = %.1f\n" % (copy_fetch_kib, copy_write_kib))
        f.write("fetch_scale = %.4f\nwrite_scale = %.4f\n" % (f_factor, w_factor))
        f.write("gemv_fetch_kib_raw = %.1f\ngemv_write_kib_raw = %.1f\n" % (g_fetch_kib, g_write_kib))
        f.write("gemv_fetch_bytes = %d\ngemv_write_bytes = %d\n" % (g_fetch, g_write))
        f.write("algorithmic_bytes_per_launch = %d\n" % alg)
        f.write("traffic_bytes_per_launch = %d\n" % (g_fetch + g_write))
        f.write("kernel_source_sha256_16 = %s\n" % kernel_hash(target))
    print(open(out).read())


# ----------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--profile", choices=["none", "roofline", "prefill"], default="none")
    ap.add_argument("--pmc-target", choices=["decode", "prefill"], default="decode",
                    help="which kernel --summarize-pmc summarizes")
    ap.add_argument("--no-extra", action="store_true", help="skip the secondary configurations")
    ap.add_argument("--attention-only", action="store_true",
                    help="time only the decode-attention cases (a short program for kernel traces)")
    ap.add_argument("--peaks-only", action="store_true",
                    help="time only the calibration kernels and the vendor GEMM")
    ap.add_argument("--few-tokens-only", action="store_true",
                    help="time only the 4- and 8-token products (a short program for kernel traces)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the M = 2048 prefill products (a short program for counter passes)")
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("COUNTER_CSV", "OUT"),
                    help="matrix-core busy fraction per GEMM launch from a rocprofv3 --pmc pass")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--summarize-trace", nargs=3, metavar=("TRACE_CSV", "STATS_CSV", "OUT"))
    ap.add_argument("--trace-command", default="--steps 80 --warmup 8 --no-extra --no-cpu-baseline",
                    help="bench.py arguments of the traced run (written into the summary)")
    ap.add_argument("--copy-bytes", type=int, default=256 << 20)
    args = ap.parse_args()

    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, command=args.trace_command)
        return 0
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma)
        return 0
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.copy_bytes,
                      TRAFFIC_FILE if args.pmc_target == "decode" else TRAFFIC_FILE_PREFILL, args.pmc_target)
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the W1.58A8 BitLinear path here is a single-GPU build "
              "(no collectives); run it with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import datagen
    import ternary_weight_linear_w1_amd as bl
    from ternary_weight_linear_w1_amd import _build

    if not _build.up_to_date():
        _build.build()
    bl.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.attention_only:
        print(json.dumps({"attention_decode": run_attention(torch, bl, dev)}))
        return 0
    if args.prefill_only:
        print(json.dumps({"2B_prefill_M2048": run_prefill(torch, bl, datagen, dev, 2048)}))
        return 0
    if args.peaks_only:
        print(json.dumps(run_peaks(torch, dev)))
        return 0
    if args.few_tokens_only:
        print(json.dumps(run_few(torch, bl, datagen, dev)))
        return 0

    # ---- headline: the 100B-shaped slice at M = 1
    if args.profile == "roofline":
        N, K, mode = [(n, k, md) for (nm, n, k, md) in LAYER_100B if nm == DOMINANT][0]
        C = n_copies(N * K // 4)
        dom = Mat(torch, bl, datagen, 5, 3, DOMINANT, N, K, mode, 1, C, dev)
        for i in range(200):
            dom.fused(bl, i % C)
        src = torch.empty(args.copy_bytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"profile": "roofline", "kernel_launches": 200, "copy_bytes": args.copy_bytes}))
        return 0

    if args.profile == "prefill":
        i, (name, N, K, mode) = [(i, sp) for i, sp in enumerate(LAYER_2B) if sp[0] == PREFILL_DOMINANT][0]
        m = Mat(torch, bl, datagen, 4, i + 4, name, N, K, mode, PREFILL_M, 2, dev)
        m.x = datagen.heavy_channel_acts_torch(PREFILL_M, K, datagen.stream_id(4, 1, i, 1), dev)
        m.prequant(bl)
        for j in range(50):
            m.forward(bl, j % 2)
        src = torch.empty(args.copy_bytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"profile": "prefill", "kernel_launches": 50, "copy_bytes": args.copy_bytes}))
        return 0

    head = run_headline(torch, bl, datagen, dev, args.steps, args.warmup)
    slice_mats = head.pop("_mats")
    roofline = head.pop("_roofline")
    extra = head.pop("_extra")

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) on layer 0 of the slice ...")
        cpu = cpu_baseline(torch, slice_mats[0], args.cpu_seconds)
        log("cpu baseline: %s" % cpu)
    del slice_mats
    torch.cuda.empty_cache()

    prefill = run_prefill_headline(torch, bl, datagen, dev, PREFILL_M, args.steps, args.warmup)
    torch.cuda.empty_cache()

    if not args.no_extra:
        extra.update(run_extra(torch, bl, datagen, dev))

    out = {
        "metric": METRIC, "value": head["value"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": head["config"],
        "roofline": roofline,
        "prefill": prefill,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)
    return 0


def graph_of(torch, fn):
    """A captured graph, replayed once (its first launch uploads it) before it is timed."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    return g


def timed_replays(torch, graphs_in_order):
    """Replays the given graphs back to back between synchronizations; returns (GPU seconds
    from HIP events on the launch stream, host wall seconds)."""
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for g in graphs_in_order:
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) * 1e-3, wall


def rotation_plan(graphs_pair, graphs_single, start, count):
    """Graph sequence for `count` steps starting at weight copy `start` (0 or 1): pairs of
    steps (copy c then the other one), then one single step if count is odd."""
    seq, c = [], start
    for _ in range(count // 2):
        seq.append(graphs_pair[c])
    if count % 2:
        seq.append(graphs_single[c])
    return seq


def run_headline(torch, bl, datagen, dev, steps, warmup):
    """The 100B-shaped slice (4 layers x QKV, O, up, down), M = 1, fused entry per BitLinear,
    two copies of the whole slice (1.24 GB) alternating step by step."""
    log("setup: 100B slice, %d layers, 2 copies of the packed weights" % SLICE_LAYERS)
    mats = [[Mat(torch, bl, datagen, 5, i, name, N, K, mode, 1, 2, dev, layer=li)
             for i, (name, N, K, mode) in enumerate(LAYER_100B)] for li in range(SLICE_LAYERS)]
    flat = [m for row in mats for m in row]
    step_bytes = sum(m.bytes() for m in flat)
    packed_bytes = sum(m.N * m.K // 4 for m in flat)

    def step(c):
        for m in flat:
            m.fused(bl, c)

    for c in (0, 1):          # eager pass: every kernel loaded before capture
        step(c)
    torch.cuda.synchronize()
    pair = [graph_of(torch, lambda: (step(0), step(1))), graph_of(torch, lambda: (step(1), step(0)))]
    single = [graph_of(torch, lambda: step(0)), graph_of(torch, lambda: step(1))]
    # per-matrix launches of the step (fused entry), each over >= 1 GiB of rotating weights:
    # the slice's 8 instances of the matrix (4 layers x 2 copies) plus clones; timed before the
    # steps, which then run on a GPU that is already busy (clocks up)
    per = {}
    dom_avg = None
    for i, (name, N, K, mode) in enumerate(LAYER_100B):
        inst = [(row[i], c) for row in mats for c in (0, 1)]
        extra_c = max(0, n_copies(N * K // 4) - len(inst))
        clones = [mats[0][i].copies[0].clone() for _ in range(extra_c)]
        m0 = mats[0][i]
        rot = [lambda m=m, c=c: m.fused(bl, c) for m, c in inst] + \
              [lambda w=w: bl.bitlinear_forward_f32(m0.x, w, m0.gamma, m0.gain, EPS, m0.relu2, y=m0.y, workspace=m0.ws)
               for w in clones]
        a = time_kernel(torch, lambda j: rot[j](), len(rot), 200)
        b = m0.bytes()
        per[name] = {"us": round(a * 1e6, 3), "GB/s": round(b / a / 1e9, 1), "frac_hbm": round(b / a / 1e9 / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes": b, "rotating_copies": len(rot)}
        if name == DOMINANT:
            dom_avg, dom_bytes = a, b
        del clones, rot
        torch.cuda.empty_cache()
    log("warmup %d steps" % warmup)
    timed_replays(torch, rotation_plan(pair, single, 0, warmup))
    log("timing %d steps" % steps)
    gpu_s, wall = timed_replays(torch, rotation_plan(pair, single, warmup % 2, steps))
    value = step_bytes * steps / gpu_s / 1e9
    ms_per_step = gpu_s / steps * 1e3
    log("value %.1f GB/s (%.4f ms/step by events; %.4f ms/step by host wall clock)" %
        (value, ms_per_step, wall / steps * 1e3))
    del pair, single

    log("slice per-matrix (fused, M=1): %s" % per)
    achieved = dom_bytes / dom_avg / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": read_traffic(),
                "kernel": "bitlinear_forward_f32 down 28672->8192 (ReLU^2+subln input), M=1",
                "algorithmic_bytes": dom_bytes, "avg_us": round(dom_avg * 1e6, 3),
                "timing": "HIP events around a graph of 200 back-to-back launches on the launch stream, "
                          "weights rotating over >= 1 GiB"}
    step_us = sum(v["us"] for v in per.values()) * SLICE_LAYERS
    config = {"workload": "BitNet-b1.58-100B-shaped layer slice at decode, M=1: %d layers x [QKV 8192->10240 "
                          "(plain absmax input), O 8192->8192 (subln input), up 8192->28672 (plain), down "
                          "28672->8192 (ReLU^2+subln input)], one fused BitLinear call each (quantize + "
                          "W1.58A8 product + rescale), GG(0.846) latents per layer (42/29/29 ternary split), "
                          "2 copies of the slice alternating (%.2f GB) so weights stream from HBM"
                          % (SLICE_LAYERS, 2 * packed_bytes / 1e9),
              "M": 1, "entry": "bitlinear_forward_f32", "step_bytes": step_bytes, "packed_bytes": packed_bytes,
              "graph": "one HIP graph per two steps (both copies), captured before timing",
              "timing": "HIP events around the replays of the timed steps; %.4f ms/step by host wall clock"
                        % (wall / steps * 1e3)}
    extra = {"100B_slice_M1_per_matrix_fused": per,
             "100B_slice_sum_of_launches_us": round(step_us, 2),
             "100B_slice_step_us": round(ms_per_step * 1e3, 2)}
    return {"value": round(value, 2), "ms_per_step": round(ms_per_step, 5), "config": config, "_mats": mats,
            "_roofline": roofline, "_extra": extra}


def run_prefill_headline(torch, bl, datagen, dev, M, steps, warmup):
    """int8 TOPS at M tokens over one step = the four products of the 2B-shaped layer on
    pre-quantized activations (the int8 matrix-core GEMM), two weight copies alternating,
    graphs captured before timing, HIP events around the timed replays."""
    log("setup: prefill M=%d on the 2B layer shapes" % M)
    mats = []
    for i, (name, N, K, mode) in enumerate(LAYER_2B):
        m = Mat(torch, bl, datagen, 4, i + 4, name, N, K, mode, M, 2, dev)
        m.x = datagen.heavy_channel_acts_torch(M, K, datagen.stream_id(4, 1, i, 1), dev)
        m.prequant(bl)
        mats.append(m)
    ops = sum(2.0 * M * m.N * m.K for m in mats)

    def step(c):
        for m in mats:
            m.forward(bl, c)

    for c in (0, 1):
        step(c)
    torch.cuda.synchronize()
    pair = [graph_of(torch, lambda: (step(0), step(1))), graph_of(torch, lambda: (step(1), step(0)))]
    single = [graph_of(torch, lambda: step(0)), graph_of(torch, lambda: step(1))]
    # per-matrix launches first: graphs of 100 launches each, about 40 ms of load, after which
    # the clocks have settled (a cold GPU runs the first ~60 steps up to 15% slower)
    per = {}
    for m in mats:
        a = time_kernel(torch, lambda c, m=m: m.forward(bl, c), 2, 100)
        o = 2.0 * M * m.N * m.K
        per[m.name] = {"us": round(a * 1e6, 2), "TOPS": round(o / a / 1e12, 1),
                       "frac_int8_peak": round(o / a / 1e12 / INT8_PEAK_TOPS, 4)}
    timed_replays(torch, rotation_plan(pair, single, 0, warmup))
    gpu_s, wall = timed_replays(torch, rotation_plan(pair, single, warmup % 2, steps))
    tops = ops * steps / gpu_s / 1e12
    del pair, single
    dom = PREFILL_DOMINANT   # the longest GEMM of the step on the boxes measured (down, with up close)
    dm = [m for m in mats if m.name == dom][0]
    a = per[dom]["us"] * 1e-6
    achieved = 2.0 * M * dm.N * dm.K / a / 1e12
    out = {"metric": "int8 TOPS @M=2048 (W1.58A8 prefill product)", "value": round(tops, 1), "unit": "TOPS",
           "ms_per_step": round(gpu_s / steps * 1e3, 5), "steps": steps, "warmup": warmup,
           "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4),
           "config": {"workload": "BitNet-b1.58-2B-shaped layer products at prefill, M=%d: QKV 2560->3840, "
                                  "O 2560->2560, up 2560->6912, down 6912->2560 on pre-quantized int8 activations "
                                  "(N(0,1) with 1%% Student-t(3) channels), GG(0.846) latents" % M,
                      "M": M, "entry": "bitlinear_forward", "ops_per_step": ops,
                      "timing": "HIP events around graph replays captured before timing; %.4f ms/step by host "
                                "wall clock" % (wall / steps * 1e3)},
           "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": INT8_PEAK_TOPS, "unit": "TOPS",
                        "frac": round(achieved / INT8_PEAK_TOPS, 4), "traffic": read_traffic("prefill"),
                        "algorithmic_bytes": layer_bytes(dm.N, dm.K, M, dm.mode, fused=False),
                        "kernel": "bitlinear_forward %s %d->%d, M=%d (int8 matrix-core GEMM)" % (dom, dm.K, dm.N, M),
                        "avg_us": per[dom]["us"],
                        "timing": "HIP events around a graph of 100 back-to-back launches (two weight copies)"},
           "per_matrix": per}
    log("prefill M=%d: %.1f TOPS (%.4f ms/step); per matrix %s" % (M, tops, gpu_s / steps * 1e3, per))
    del mats
    return out


def run_2b_layer(torch, bl, datagen, dev, steps=400):
    """One BitNet-2B-shaped layer's four BitLinears at M = 1 (fused entry each), weights
    rotating over >= 1 GiB of copies, graphs of 8 steps captured before timing; and each
    matrix's launch alone (graph of back-to-back launches)."""
    layer_copy_bytes = sum(N * K // 4 for _, N, K, _ in LAYER_2B)
    G = 8
    C = n_copies(layer_copy_bytes, G)
    mats = [Mat(torch, bl, datagen, 2, i, *spec, 1, C, dev) for i, spec in enumerate(LAYER_2B)]
    step_bytes = sum(m.bytes() for m in mats)

    def steps_of(c0):
        for c in range(c0, c0 + G):
            for m in mats:
                m.fused(bl, c)

    steps_of(0)
    torch.cuda.synchronize()
    graphs = [graph_of(torch, lambda gi=gi: steps_of(gi * G)) for gi in range(C // G)]
    timed_replays(torch, graphs)
    reps = max(1, steps // (G * len(graphs)))
    gpu_s, _ = timed_replays(torch, graphs * reps)
    n = G * len(graphs) * reps
    out = {"us_per_step": round(gpu_s / n * 1e6, 3), "GB/s": round(step_bytes * n / gpu_s / 1e9, 1),
           "step_bytes": step_bytes, "steps": n, "weight_copies": C}
    del graphs
    per = {}
    for m in mats:
        a = time_kernel(torch, lambda c, m=m: m.fused(bl, c), C, 200)
        per[m.name] = {"us": round(a * 1e6, 3), "GB/s": round(m.bytes() / a / 1e9, 1)}
    out["per_matrix_fused"] = per
    log("extra 2B layer M=1: %s" % out)
    del mats
    torch.cuda.empty_cache()
    return out


def run_cfg1(torch, bl, datagen, dev):
    """One BitLinear, M = 1, K = N = 2560, latents N(0, 0.02^2), plain absmax input
    (fused call), rotating weight copies."""
    N = K = 2560
    C = n_copies(N * K // 4)
    w = datagen.gaussian_weights_torch(N, K, datagen.stream_id(1, 0, 0, 0), dev)
    packed, gamma = bl.bitlinear_pack_weights(w)
    del w
    copies = [packed] + [packed.clone() for _ in range(C - 1)]
    x = datagen.outlier_acts_torch(1, K, datagen.stream_id(1, 0, 0, 1), dev)
    y = torch.empty((1, N), dtype=torch.float32, device=dev)
    t = time_kernel(torch, lambda c: bl.bitlinear_forward_f32(x, copies[c], gamma, y=y), C, 400)
    b = layer_bytes(N, K, 1, "plain")
    out = {"us": round(t * 1e6, 3), "GB/s": round(b / t / 1e9, 1), "frac_hbm": round(b / t / 1e9 / HBM_PEAK_GBS, 4),
           "algorithmic_bytes": b}
    log("extra cfg1 single BitLinear: %s" % out)
    return out


def run_peaks(torch, dev):
    """Achievable peaks on this GPU, for context next to the specs: a streaming-read kernel
    (libbitlinear_peaks.so; back-to-back launches in a graph over rotating copies, best of
    grid sizes and loads in flight) at the packed sizes of the 2B and 100B matrices, a pure
    int8 matrix-core instruction loop, a streaming copy (torch), and the vendor int8 GEMM
    (torch._int_mm, int8 x int8 -> int32, hipBLASLt on ROCm) on the 2B prefill shapes at
    M = 2048 (dense int8 weights: 4x the bytes of the packed ternary ones)."""
    import ctypes
    from ternary_weight_linear_w1_amd import _build
    if not _build.up_to_date():
        _build.build()
    P = ctypes.CDLL(_build.PEAKS_LIB)
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    P.bl_peak_stream_read.argtypes = [vp, i64, ci, ci, vp, vp]
    P.bl_peak_mfma_i8.argtypes = [ci, ci, vp, vp]
    P.bl_peak_empty.argtypes = [ci, vp, vp]
    P.bl_peak_mfma_valu.argtypes = [ci, ci, ci, vp, vp]
    P.bl_peak_lds_read.argtypes = [ci, ci, vp, vp]
    out = {}
    sink = torch.zeros((4096 * 256,), dtype=torch.int32, device=dev)

    def cur():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    reads = {}
    for name, nbytes in (("2B up/down 4.42 MB", 4423680), ("100B O 16.78 MB", 16777216),
                         ("100B QKV 20.97 MB", 20971520), ("100B up/down 58.72 MB", 58720256)):
        copies = max(2, min(64, (1200 << 20) // nbytes))
        buf = torch.empty((copies * nbytes,), dtype=torch.uint8, device=dev)
        base = buf.data_ptr()
        best = None
        for blocks in (256, 512, 1024, 2048):
            for unroll in (4, 8):
                t = time_kernel(torch, lambda c, b=blocks, u=unroll: P.bl_peak_stream_read(
                    ctypes.c_void_p(base + c * nbytes), nbytes, b, u, ctypes.c_void_p(sink.data_ptr()), cur()),
                    copies, 40)
                if best is None or t < best[0]:
                    best = (t, blocks, unroll)
        reads[name] = {"us": round(best[0] * 1e6, 2), "GB/s": round(nbytes / best[0] / 1e9, 1),
                       "frac_hbm": round(nbytes / best[0] / 1e9 / HBM_PEAK_GBS, 4),
                       "blocks": best[1], "loads_in_flight": best[2]}
        del buf
        torch.cuda.empty_cache()
    out["stream_read (per launch, back to back)"] = reads
    # the floor of a kernel boundary: launches with no work, back to back in a graph
    empty = {}
    for blocks in (256, 1024):
        t = time_kernel(torch, lambda c, b=blocks: P.bl_peak_empty(b, ctypes.c_void_p(sink.data_ptr()), cur()), 2, 200)
        empty["%d blocks" % blocks] = round(t * 1e6, 2)
    out["empty_launch_us (graph, back to back)"] = empty
    blocks, iters = 2 * 256, 4000
    t = time_kernel(torch, lambda c: P.bl_peak_mfma_i8(iters, blocks, ctypes.c_void_p(sink.data_ptr()), cur()), 1, 5)
    ops = blocks * 4 * iters * 4 * 65536.0
    out["mfma_i8_loop"] = {"POPS": round(ops / t / 1e15, 3), "frac_int8_peak": round(ops / t / 1e15 / 5.0, 4),
                           "us": round(t * 1e6, 1)}
    # how much vector work the other wave of a SIMD can issue while the matrix core runs
    # (one matrix-core wave and one vector wave per SIMD, one 512-thread block per CU)
    co = {}
    blocks, iters = 256, 4000
    for nv in (0, 2, 4, 6, 8, 12):
        t = time_kernel(torch, lambda c, n=nv: P.bl_peak_mfma_valu(n, iters, blocks, ctypes.c_void_p(sink.data_ptr()),
                                                                    cur()), 1, 5)
        co["%d valu per mfma" % nv] = round(blocks * 4 * iters * 4 * 65536.0 / t / 1e15, 3)
    out["mfma_i8_POPS_with_valu_on_other_wave"] = co
    # LDS read rate (ds_read_b128, conflict-free, 1024-thread blocks, one and four per CU)
    lds = {}
    for blocks in (256, 1024):
        t = time_kernel(torch, lambda c, b=blocks: P.bl_peak_lds_read(2000, b, ctypes.c_void_p(sink.data_ptr()), cur()),
                        1, 5)
        lds["%d blocks" % blocks] = round(blocks * 1024 * 2000 * 4 * 16.0 / t / 1e12, 1)
    out["lds_read_TB/s (all CUs)"] = lds
    x = torch.ones((1 << 28,), dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    t = time_kernel(torch, lambda c: y.copy_(x), 1, 10)
    out["stream_copy_GB/s (read + write, torch)"] = round(2 * x.numel() * 4 / t / 1e9, 1)
    del x, y
    torch.cuda.empty_cache()
    gemm = {}
    try:
        for name, N, K, _ in LAYER_2B:
            M = 2048
            a = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev)
            b = torch.randint(-1, 2, (N, K), dtype=torch.int8, device=dev).t()   # [K][N], column-major
            t = time_kernel(torch, lambda c: torch._int_mm(a, b), 1, 10)
            gemm[name] = {"us": round(t * 1e6, 1), "TOPS": round(2.0 * M * N * K / t / 1e12, 2)}
            del a, b
    except Exception as e:   # not every torch build has the int8 GEMM on this GPU
        gemm = {"unavailable": str(e)[:200]}
    out["torch_int_mm_M2048"] = gemm
    log("extra measured peaks: %s" % out)
    return out


def run_tp8(torch, bl, datagen, dev):
    """The 100B slice at M = 1 on one GPU's share of an 8-way tensor-parallel split: the
    fused call and the product on pre-quantized codes (weights rotating through HBM)."""
    r = {}
    for i, (name, N, K, mode) in enumerate(LAYER_100B_TP8):
        C = n_copies(N * K // 4)
        m = Mat(torch, bl, datagen, 6, i, name, N, K, mode, 1, C, dev)
        a = time_kernel(torch, lambda c, m=m: m.fused(bl, c), C, 100)
        b = m.bytes()
        m.prequant(bl)
        f = time_kernel(torch, lambda c, m=m: m.forward(bl, c), C, 100)
        fb = m.bytes(fused=False)
        r[name] = {"N": N, "K": K, "fused_us": round(a * 1e6, 2), "fused_GB/s": round(b / a / 1e9, 1),
                   "forward_us": round(f * 1e6, 2), "forward_GB/s": round(fb / f / 1e9, 1)}
        del m
        torch.cuda.empty_cache()
    log("extra 100B TP8 shard M=1: %s" % r)
    return r


def run_few(torch, bl, datagen, dev):
    """A few tokens: the 2B layer at M = 4 and 8 (fused call, product on pre-quantized codes,
    quantization launch alone) and the 100B slice's product at M = 8, weights rotating
    through HBM as at M = 1."""
    res = {}
    for M in (4, 8):
        r = {}
        for i, (name, N, K, mode) in enumerate(LAYER_2B):
            C = n_copies(N * K // 4)
            m = Mat(torch, bl, datagen, 2, 8 + i, name, N, K, mode, M, C, dev)
            f = time_kernel(torch, lambda c, m=m: m.fused(bl, c), C, 200)
            m.prequant(bl)
            a = time_kernel(torch, lambda c, m=m: m.forward(bl, c), C, 200)
            q = time_kernel(torch, lambda c, m=m: m.prequant(bl), 1, 200)
            b, fb = m.bytes(fused=False), m.bytes()
            r[name] = {"fused_us": round(f * 1e6, 3), "fused_GB/s": round(fb / f / 1e9, 1),
                       "forward_us": round(a * 1e6, 3), "forward_GB/s": round(b / a / 1e9, 1),
                       "quantize_us": round(q * 1e6, 3)}
            del m
            torch.cuda.empty_cache()
        res["2B_M%d" % M] = r
        log("extra 2B M=%d: %s" % (M, r))
    M, r = 8, {}
    for i, (name, N, K, mode) in enumerate(LAYER_100B):
        C = n_copies(N * K // 4)
        m = Mat(torch, bl, datagen, 5, 8 + i, name, N, K, mode, M, C, dev)
        m.prequant(bl)
        need = bl.bitlinear_forward_workspace_bytes(M, N, K)
        ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
        a = time_kernel(torch, lambda c, m=m: m.forward(bl, c, ws), C, 100)
        b = m.bytes(fused=False)
        r[name] = {"us": round(a * 1e6, 2), "GB/s": round(b / a / 1e9, 1),
                   "frac_hbm": round(b / a / 1e9 / HBM_PEAK_GBS, 4)}
        if need:
            r[name]["k_slices"] = need // (4 * M * N)
        del m, ws
        torch.cuda.empty_cache()
    res["100B_M8"] = r
    log("extra 100B M=8: %s" % r)
    return res


def run_extra(torch, bl, datagen, dev):
    res = {}
    res["2B_layer_M1_step"] = run_2b_layer(torch, bl, datagen, dev)
    res["cfg1_single_M1"] = run_cfg1(torch, bl, datagen, dev)
    res["measured_peaks"] = run_peaks(torch, dev)
    torch.cuda.empty_cache()
    res.update(run_few(torch, bl, datagen, dev))
    torch.cuda.empty_cache()
    # ---- 100B-shaped slice at M = 1 (fused), M = 32 and 64 (pre-quantized; at 32 tokens the
    #      down projection's K is split across blocks, timed beside the unsplit product)
    for M in (1, 32, 64):
        r = {}
        for i, (name, N, K, mode) in enumerate(LAYER_100B):
            C = n_copies(N * K // 4)
            m = Mat(torch, bl, datagen, 5, i + 4 * (M > 1), name, N, K, mode, M, C, dev)
            ops = 2.0 * M * N * K
            if M == 1:
                # fused call, then the two-call path: the product on pre-quantized codes
                # (the HBM-bound kernel) and the quantization launch on its own
                a = time_kernel(torch, lambda c, m=m: m.fused(bl, c), C, 100)
                b = m.bytes()
                m.prequant(bl)
                f = time_kernel(torch, lambda c, m=m: m.forward(bl, c), C, 100)
                fb = m.bytes(fused=False)
                q = time_kernel(torch, lambda c, m=m: m.prequant(bl), 1, 100)
                r[name] = {"fused_us": round(a * 1e6, 2), "fused_GB/s": round(b / a / 1e9, 1),
                           "forward_us": round(f * 1e6, 2), "forward_GB/s": round(fb / f / 1e9, 1),
                           "forward_frac_hbm": round(fb / f / 1e9 / HBM_PEAK_GBS, 4),
                           "quantize_us": round(q * 1e6, 2), "TOPS_forward": round(ops / f / 1e12, 2)}
            else:
                m.prequant(bl)
                need = bl.bitlinear_forward_workspace_bytes(M, N, K)
                ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
                a = time_kernel(torch, lambda c, m=m: m.forward(bl, c, ws), C, 100)
                b = m.bytes(fused=False)
                r[name] = {"us": round(a * 1e6, 2), "GB/s": round(b / a / 1e9, 1), "TOPS": round(ops / a / 1e12, 2)}
                if need:
                    u = time_kernel(torch, lambda c, m=m: m.forward(bl, c, split=False), C, 100)
                    r[name].update({"k_slices": need // (4 * M * N), "unsplit_us": round(u * 1e6, 2)})
                del ws
            del m
            torch.cuda.empty_cache()
        res["100B_M%d" % M] = r
        log("extra 100B M=%d: %s" % (M, r))
    # ---- one GPU's share of the 100B slice under 8-way tensor parallelism, M = 1
    res["100B_TP8_shard_M1"] = run_tp8(torch, bl, datagen, dev)
    # ---- prefill on the 2B shapes (pre-quantized forward), int8 TOPS
    for M in (512, 2048):
        res["2B_prefill_M%d" % M] = run_prefill(torch, bl, datagen, dev, M)
    # ---- five codes per byte (1.6 bits per weight) against the 2-bit fields, pre-quantized
    res["trits5_vs_2bit"] = run_trits5(torch, bl, datagen, dev)
    torch.cuda.empty_cache()
    # ---- decode attention over a bf16 key/value cache at real context length
    res["attention_decode"] = run_attention(torch, bl, dev)
    torch.cuda.empty_cache()
    # ---- decode stack: 30 layers of the 2B shapes at M = 1, plain and gated FFN, attending
    #      over 1 and over 4096 cached positions
    for gated in (False, True):
        for ctx in (1, 4096):
            key = "2B_stack30_M1_ctx%d" % ctx + ("_gated" if gated else "")
            res[key] = run_stack(torch, bl, datagen, dev, gated, ctx=ctx)
            torch.cuda.empty_cache()
    # ---- packing rate (100B up projection)
    N, K = 28672, 8192
    w = datagen.gg_weights_torch(N, K, datagen.stream_id(5, 9, 0, 0), dev)
    packed = torch.empty((N, K // 4), dtype=torch.uint8, device=dev)
    gamma = torch.empty((1,), dtype=torch.float32, device=dev)
    ws = torch.empty((bl.bitlinear_pack_workspace_bytes(N, K),), dtype=torch.uint8, device=dev)
    a = time_kernel(torch, lambda c: bl.bitlinear_pack_weights(w, packed, gamma, ws), 1, 5)
    res["pack_100B_up"] = {"ms": round(a * 1e3, 3), "GB/s (2 reads of W + packed write)":
                           round((2 * 4 * N * K + N * K // 4) / a / 1e9, 1)}
    del w, packed, ws
    torch.cuda.empty_cache()
    return res


def run_prefill(torch, bl, datagen, dev, M):
    """The pre-quantized product on the 2B shapes at M tokens (int8 MFMA GEMM): time per
    launch (graph of 10, two weight copies) and int8 TOPS against the 5 POPS dense peak; the
    quantization launch on its own (GB/s of its algorithmic bytes against 8 TB/s; the fp32
    input is one buffer, so it may come from the 256 MB MALL) and the fused call with a
    workspace (quantization, then the product)."""
    r = {}
    for i, (name, N, K, mode) in enumerate(LAYER_2B):
        m = Mat(torch, bl, datagen, 4, i + 4 * (M > 512), name, N, K, mode, M, 2, dev)
        m.x = datagen.heavy_channel_acts_torch(M, K, datagen.stream_id(4, 1, i, 1), dev)
        m.prequant(bl)
        a = time_kernel(torch, lambda c, m=m: m.forward(bl, c), 2, 10)
        q = time_kernel(torch, lambda c, m=m: m.prequant(bl), 1, 10)
        ws = torch.empty((bl.bitlinear_forward_f32_workspace_bytes(M, N, K),), dtype=torch.uint8, device=dev)
        f = time_kernel(torch, lambda c, m=m: bl.bitlinear_forward_f32(m.x, m.copies[c], m.gamma, m.gain, EPS,
                                                                       m.relu2, y=m.y, workspace=ws), 2, 10)
        ops = 2.0 * M * N * K
        qb = 4 * M * K + (4 * K if m.gain is not None else 0) + M * K + 4 * M
        r[name] = {"us": round(a * 1e6, 1), "TOPS": round(ops / a / 1e12, 2),
                   "frac_int8_peak": round(ops / a / 1e12 / INT8_PEAK_TOPS, 4),
                   "quantize_us": round(q * 1e6, 1), "quantize_GB/s": round(qb / q / 1e9, 1),
                   "quantize_frac_hbm": round(qb / q / 1e9 / HBM_PEAK_GBS, 4), "fused_us": round(f * 1e6, 1)}
        del m, ws
    log("extra prefill M=%d: %s" % (M, r))
    return r


def summarize_mfma(counter_csv, out):
    """Matrix-core busy fraction of each GEMM launch shape from one rocprofv3 --pmc pass
    over `bench.py --prefill-only`. SQ_VALU_MFMA_BUSY_CYCLES sums the busy cycles of every
    MFMA (32 per v_mfma_i32_32x32x32_i8) over the 1024 SIMDs; SQ_CYCLES sums the launch's
    cycles over the 32 shader engines (8 XCDs x 4), so the launch spans SQ_CYCLES / 32
    cycles and the fraction is BUSY / (1024 * SQ_CYCLES / 32)."""
    import csv
    import statistics
    vals = {}
    with open(counter_csv) as f:
        for r in csv.DictReader(f):
            if "bl::gemm_" not in r["Kernel_Name"] or "reduce" in r["Kernel_Name"]:
                continue
            wg = int(r.get("Workgroup_Size", 256) or 256)
            key = (r["Kernel_Name"].replace("void ", "").split("(")[0], int(r["Grid_Size"]) // wg)
            d = vals.setdefault(key, {}).setdefault(int(r["Dispatch_Id"]), {})
            d[r["Counter_Name"]] = float(r["Counter_Value"])
    with open(out, "w") as f:
        f.write("# int8 matrix-core busy fraction of the prefill GEMM (2B shapes, M = 2048)\n")
        f.write("# commands (GPU box, repository root in $R):\n")
        f.write("#   cd /tmp && rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_INSTS_VALU_MFMA_I8 "
                "SQ_INSTS_VALU SQ_CYCLES SQ_BUSY_CU_CYCLES SQ_LDS_BANK_CONFLICT SQ_WAIT_ANY -d $R/gpurun_out/pmc_mfma "
                "-o mfma --output-format csv -- python3 $R/bench.py --prefill-only\n")
        f.write("#   python3 bench.py --summarize-mfma <mfma_counter_collection.csv> <this file>\n")
        f.write("# busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs * SQ_CYCLES / 32 shader engines); valu/mfma = "
                "SQ_INSTS_VALU / SQ_INSTS_VALU_MFMA_I8 (the VALU count includes the MFMAs);\n")
        f.write("# coexec = SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES (VALU issued while the matrix core "
                "runs); medians over the launches of each shape\n#\n")
        f.write("# %-44s %6s %6s %8s %9s %8s %10s\n" % ("kernel", "WGs", "calls", "busy", "valu/mfma", "coexec",
                                                     "bank_confl"))
        for key in sorted(vals):
            rows = [d for d in vals[key].values() if "SQ_VALU_MFMA_BUSY_CYCLES" in d and d.get("SQ_CYCLES")]
            if not rows:
                continue
            busy = statistics.median(d["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024.0 * d["SQ_CYCLES"] / 32.0) for d in rows)
            vpm = statistics.median(d["SQ_INSTS_VALU"] / max(d["SQ_INSTS_VALU_MFMA_I8"], 1.0) for d in rows)
            co = statistics.median(d["SQ_VALU_MFMA_COEXEC_CYCLES"] / max(d["SQ_VALU_MFMA_BUSY_CYCLES"], 1.0)
                                   for d in rows)
            bc = statistics.median(d.get("SQ_LDS_BANK_CONFLICT", 0.0) for d in rows)
            f.write("  %-44s %6d %6d %7.1f%% %9.2f %7.1f%% %10.0f\n" % (key[0][:44], key[1], len(rows), 100 * busy, vpm,
                                                                  100 * co, bc))
    log("wrote %s" % out)


def run_trits5(torch, bl, datagen, dev):
    """bitlinear_forward5 (five codes per byte) next to bitlinear_forward on the same
    weights and codes, M = 1 and 8, 2B and 100B shapes, rotating weight copies."""
    out = {}
    for tag, N, K in (("2B_up", 6912, 2560), ("2B_down", 2560, 6912), ("100B_up", 28672, 8192),
                      ("100B_down", 8192, 28672)):
        w = datagen.gg_weights_torch(N, K, datagen.stream_id(7, 0, 0, 0), dev)
        packed, gamma = bl.bitlinear_pack_weights(w)
        del w
        p5 = bl.bitlinear_repack5(packed)
        C = n_copies(N * K // 4)
        c2 = [packed] + [packed.clone() for _ in range(C - 1)]
        c5 = [p5] + [p5.clone() for _ in range(C - 1)]
        for M in (1, 8):
            x = datagen.outlier_acts_torch(M, K, datagen.stream_id(7, 1, M, 1), dev)
            xq, s = bl.bitlinear_quantize_act(x)
            y = torch.empty((M, N), dtype=torch.float32, device=dev)
            t2 = time_kernel(torch, lambda c: bl.bitlinear_forward(xq, s, c2[c], gamma, y=y), C, 100)
            t5 = time_kernel(torch, lambda c: bl.bitlinear_forward5(xq, s, c5[c], gamma, y=y), C, 100)
            out["%s_M%d" % (tag, M)] = {"us_2bit": round(t2 * 1e6, 2), "us_1.6bit": round(t5 * 1e6, 2),
                                        "MB_2bit": round(N * K / 4 / 1e6, 2), "MB_1.6bit": round(p5.numel() / 1e6, 2),
                                        "speedup_1.6bit": round(t2 / t5, 3)}
        del c2, c5
        torch.cuda.empty_cache()
    log("extra trits5: %s" % out)
    return out


STACK_DIMS = dict(hidden=2560, heads=20, kv_heads=5, head_dim=128, ffn=6912)


def attention_bytes(M, heads, kv_heads, ctx, d=128):
    """Algorithmic HBM bytes of one decode-attention call with every sequence at position
    ctx - 1: cached keys and values read (ctx - 1 rows each, bf16), the new key and value
    appended, the qkv vector read and the output written (fp32)."""
    return M * (2 * kv_heads * (ctx - 1) * d * 2 + 2 * kv_heads * d * 2 + (heads + 2 * kv_heads) * d * 4
                + heads * d * 4)


def run_attention(torch, bl, dev):
    """bitlinear_attention_decode at the 2B (20 query / 5 KV heads) and 100B (64 / 8) head
    shapes, every sequence at position ctx - 1, rotating cache copies (>= 1 GB) so that the
    keys and values stream from HBM."""
    out = {}
    for tag, H, KVH, ctx, M in (("2B", 20, 5, 4096, 1), ("2B", 20, 5, 4096, 8), ("2B", 20, 5, 32768, 1),
                                ("100B", 64, 8, 4096, 1)):
        shape = (M, KVH, ctx, 128)
        cache_bytes = 2 * M * KVH * ctx * 128 * 2
        C = n_copies(cache_bytes)
        gen = torch.Generator(device=dev)
        gen.manual_seed(ctx + H)
        kcs = [torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16) for _ in range(C)]
        vcs = [torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16) for _ in range(C)]
        qkv = torch.randn((M, (H + 2 * KVH) * 128), generator=gen, device=dev)
        pos = torch.full((M,), ctx - 1, dtype=torch.int32, device=dev)
        o = torch.empty((M, H * 128), dtype=torch.float32, device=dev)
        ws = torch.empty((bl.bitlinear_attention_workspace_bytes(M, H, ctx),), dtype=torch.uint8, device=dev)
        t = time_kernel(torch, lambda c: bl.bitlinear_attention_decode(qkv, kcs[c], vcs[c], pos, H, KVH, out=o,
                                                                       workspace=ws), C, 100)
        b = attention_bytes(M, H, KVH, ctx)
        out["%s_ctx%d_M%d" % (tag, ctx, M)] = {"us": round(t * 1e6, 2), "GB/s": round(b / t / 1e9, 1),
                                               "frac_hbm": round(b / t / 1e9 / HBM_PEAK_GBS, 4),
                                               "algorithmic_MB": round(b / 1e6, 2), "finite": bool(torch.isfinite(o).all())}
        del kcs, vcs
        torch.cuda.empty_cache()
    log("extra attention: %s" % out)
    return out


def run_stack(torch, bl, datagen, dev, gated, ctx=1, n_layers=30, copies=2, replays=20):
    """Per-token latency of a 30-layer decode stack (one launch per BitLinear plus the two
    attention launches) at position ctx - 1 (attending over ctx cached positions), as a HIP
    graph over `copies` weight copies of the stack so that each pass streams its weights
    (and caches) from HBM (>= 776 MB against 256 MB of MALL)."""
    from ternary_weight_linear_w1_amd.decode_stack import DecodeStack, LayerWeights
    d = STACK_DIMS
    H, F = d["hidden"], d["ffn"]
    nqkv = (d["heads"] + 2 * d["kv_heads"]) * d["head_dim"]
    shapes = [("qkv", nqkv, H, "norm", False), ("o", H, H, "norm", True),
              ("up", (2 if gated else 1) * F, H, "norm", False),
              ("down", H, F, "gatednorm" if gated else "relu2norm", True)]
    base = []
    for li in range(n_layers):
        mats = {}
        for mi, (name, N, K, mode, _) in enumerate(shapes):
            w = datagen.gg_weights_torch(N, K, datagen.stream_id(3, li, mi, 0), dev)
            mats[name] = bl.bitlinear_pack_weights(w)
            del w
        gains = {g: datagen.gains_torch(F if g == "g_ffn" else H, datagen.stream_id(3, li, 4 + j, 2), dev)
                 for j, g in enumerate(("g_in", "g_attn", "g_post", "g_ffn"))}
        base.append((mats, gains))
    stacks = []
    for c in range(copies):
        layers = [LayerWeights(*[(m[n][0] if c == 0 else m[n][0].clone(), m[n][1]) for n in ("qkv", "o", "up", "down")],
                               **g) for m, g in base]
        st = DecodeStack(layers, H, d["heads"], d["kv_heads"], d["head_dim"], F, gated, M=1, eps=EPS, device=dev,
                         capacity=max(ctx, 64))
        st.h.copy_(datagen.outlier_acts_torch(1, H, datagen.stream_id(3, 200, c, 1), dev))
        st.pos.fill_(ctx - 1)
        for li in range(n_layers):      # prior context: keys and values of unit scale
            st.k_cache[li].normal_()
            st.v_cache[li].normal_()
        stacks.append(st)
    for st in stacks:
        st.step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for st in stacks:
            st.step(stream=torch.cuda.current_stream())
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    per_token = e0.elapsed_time(e1) * 1e-3 / (replays * copies)
    finite = all(bool(torch.isfinite(st.h).all()) for st in stacks)
    nbytes = n_layers * (sum(layer_bytes(N, K, 1, mode, residual=res) for _, N, K, mode, res in shapes)
                         + attention_bytes(1, d["heads"], d["kv_heads"], ctx))
    packed = n_layers * sum(N * K // 4 for _, N, K, _, _ in shapes)
    out = {"us_per_token": round(per_token * 1e6, 1), "GB/s": round(nbytes / per_token / 1e9, 1),
           "frac_hbm": round(nbytes / per_token / 1e9 / HBM_PEAK_GBS, 4), "packed_MB": round(packed / 1e6, 1),
           "algorithmic_MB": round(nbytes / 1e6, 1), "launches_per_token": 6 * n_layers, "context": ctx,
           "ideal_us_at_8TBs": round(nbytes / HBM_PEAK_GBS / 1e3, 1), "h_finite": finite}
    log("extra stack%s ctx %d: %s" % (" gated" if gated else "", ctx, out))
    del g, stacks, base
    return out


if __name__ == "__main__":
    sys.exit(main())
