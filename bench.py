#!/usr/bin/env python3
"""Throughput of the block-scaled FP4 quantisation hot path on one MI355X.

Metric: quantize GB/s -- algorithmic HBM bytes (source read + every output
written, the error-feedback residual read and rewritten) per second -- and its
fraction of MI355X's 8 TB/s HBM peak.

Headline (the largest single-GPU workload): the grouped MoE step -- 32 expert
weights of 2880 x 2880 bf16 stacked along rows, NVFP4 with one 2D 64 x 64 FP32
outer scale per tile and expert, per-16 E4M3 inner scales, stochastic
rounding, an in-place FP32 error-feedback residual, rowwise and columnwise
packed codes.  One step = one fp4_cast_transpose_grouped call (the tile pass
and the gather pass that writes whole cache lines); the residual carries over
from step to step as in training.  Steps are replayed from a HIP graph.  After
the timed steps one more step is checked against the CPU oracle, buffer by
buffer, and that oracle run is the CPU baseline (all host cores; one expert on
one core).

Also reported (not part of `value`): the other workloads -- NVFP4 2D-outer
cast-transpose 4096^2, MXFP4 fake-quant 8192^2, AMD-FP4 1D-outer SR
cast-transpose 16384x2880, NVFP4 tensorwise QDQ 256^2, 16x16 inner tiles,
the MXFP4 projection with FP8 re-encodings, FP32 fake-quant, the MXFP4 GEMM.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra]
                       [--no-cpu-baseline] [--copy-probe] [--only KEY]
"""
import argparse
import ctypes as ct
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
STAGED = os.environ.get("FP4Q_BENCH_DIRECT", "0") != "1"   # direct-store path for comparison
FP4_MFMA_PEAK_TFLOPS = 10100.0   # MI355X dense FP4 / FP6 matrix peak
METRIC = "quantize GB/s (HBM bytes read+written) and fraction of MI355X HBM peak"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 256 MiB device copy (counter calibration) and exit")
    ap.add_argument("--only", default=None, help="time a single workload (nv_tensorwise_qdq_256, nv_2d_cast_transpose_4096, mx_fake_quant_8192, amd_1d_sr_cast_transpose_16384x2880, nv_grouped_sr_ef_32x2880, nv_2d_inner16_cast_transpose_4096, mx_project_fp8_8192, mx_fake_quant_fp32_8192, mx_gemm_8192) and exit")
    ap.add_argument("--eager", action="store_true", help="launch every step from the host (no graph replay)")
    ap.add_argument("--pmc-summary", nargs=5, metavar=("KEY", "FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    default=None,
                    help="write profiles/traffic_counters.json[KEY] from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE "
                         "output directories of `--only KEY --eager` and of `--copy-probe`, then exit (no GPU)")
    return ap.parse_args()


# ---------------------------------------------------------------------- helpers
# kernels of one step of each workload (a step's traffic is the sum of their per-dispatch averages)
STEP_KERNELS = {"nv_tensorwise_qdq_256": ("k_nv_rows",),
                "nv_2d_cast_transpose_4096": ("k_tile",), "mx_fake_quant_8192": ("k_mx_qdq<",),
                "amd_1d_sr_cast_transpose_16384x2880": ("k_tile",),
                "nv_grouped_sr_ef_32x2880": ("k_tile", "k_gather"),
                "nv_2d_inner16_cast_transpose_4096": ("k_tile",), "mx_project_fp8_8192": ("k_mx_fp8",),
                "mx_fake_quant_fp32_8192": ("k_mx_qdq_f32",), "mx_gemm_8192": ("k_mx_gemm",)}
COPY_PROBE_BYTES = 256 << 20


def _pmc_rows(directory, counter):
    """(kernel name, value) of every dispatch in a rocprofv3 --pmc csv directory."""
    import csv
    out = []
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return out


def pmc_summary(key, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    """HBM bytes per launch of the workload's kernel, each counter scaled by
    what it reads for a plain copy of known size (the copy probe moves
    COPY_PROBE_BYTES each way per launch)."""
    def per_dispatch(directory, counter, match):
        vals = [v for n, v in _pmc_rows(directory, counter) if match(n)]
        if not vals:
            raise SystemExit("no %s rows for the kernel in %s" % (counter, directory))
        return sum(vals) / len(vals), len(vals)
    def copy_kernel(directory, counter):
        # the copy itself is the kernel with 20 dispatches (the fill before it runs once)
        names = {}
        for n, _ in _pmc_rows(directory, counter):
            names[n] = names.get(n, 0) + 1
        best = max(names, key=lambda n: names[n])
        return per_dispatch(directory, counter, lambda n: n == best)[0]
    cf = copy_kernel(copy_fetch_dir, "FETCH_SIZE")
    cw = copy_kernel(copy_write_dir, "WRITE_SIZE")
    fetch_scale = COPY_PROBE_BYTES / (cf * 1024.0)
    write_scale = COPY_PROBE_BYTES / (cw * 1024.0)
    kf = kw = 0.0
    nf = nw = 0
    for k in STEP_KERNELS[key]:
        ours = lambda n, k=k: ("::" + k) in n
        if not any(ours(n) for n, _ in _pmc_rows(fetch_dir, "FETCH_SIZE")):
            continue
        f, n1 = per_dispatch(fetch_dir, "FETCH_SIZE", ours)
        w_, n2 = per_dispatch(write_dir, "WRITE_SIZE", ours)
        kf, kw, nf, nw = kf + f, kw + w_, nf + n1, nw + n2
    if nf == 0:
        raise SystemExit("no dispatches of %s in %s" % (STEP_KERNELS[key], fetch_dir))
    read_b = kf * 1024.0 * fetch_scale
    write_b = kw * 1024.0 * write_scale
    path = os.path.join(ROOT, "profiles", "traffic_counters.json")
    data = {}
    if os.path.exists(path):
        with open(path) as fh:
            data = json.load(fh)
    data[key] = {"bytes_per_launch": int(round(read_b + write_b)), "read_bytes": int(round(read_b)),
                 "write_bytes": int(round(write_b)), "fetch_kib_per_dispatch": kf, "write_kib_per_dispatch": kw,
                 "dispatches": [nf, nw], "fetch_scale": fetch_scale, "write_scale": write_scale,
                 "sources_sha": kernel_sources_hash()}
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
    print(json.dumps({key: data[key]}))

def kernel_sources_hash():
    files = sorted(glob.glob(os.path.join(ROOT, "block_scaled_fp4_amax_amd", "csrc", "*")))
    h = hashlib.sha256()
    for f in files:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key):
    """HBM bytes per launch from the committed counter summary, or None when the
    kernels changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    entry = data.get(kernel_key)
    if not entry or entry.get("sources_sha") != kernel_sources_hash():
        return None
    return entry.get("bytes_per_launch")


class Timed:
    """A workload: rotating buffer sets and a launch closure per set."""

    def __init__(self, name, desc, bytes_per_step, sets, launch, kernel, elements=0, flops=0, graph=True):
        self.name, self.desc, self.bytes, self.sets, self.launch, self.kernel = name, desc, bytes_per_step, sets, launch, kernel
        self.elements = elements
        self.flops = flops          # MFMA-bound workloads: algorithmic flops per launch
        self.graph = graph


def run_timed(torch, w, steps, warmup, graph=True):
    """Warm up, then time exactly `steps` launches bracketed by synchronisation;
    events are recorded on the stream the launches use (torch's current stream)."""
    n = len(w.sets)
    for i in range(warmup):
        w.launch(w.sets[i % n])
    torch.cuda.synchronize()
    # one graph replays the buffer sets in turn, at least 32 launches long so
    # that host-side replay calls do not separate short launches
    per_graph = n * max(1, -(-32 // n))
    reps, rem = divmod(steps, per_graph)
    g = None
    if graph and reps > 0:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(per_graph):
                w.launch(w.sets[i % n])
        g.replay()
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    if g is not None:
        for _ in range(reps):
            g.replay()
        for i in range(rem):
            w.launch(w.sets[i % n])
    else:
        for i in range(steps):
            w.launch(w.sets[i % n])
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    return ms


def n_sets_for(bytes_per_set, min_total=1 << 30, cap=64):
    return max(2, min(cap, -(-min_total // max(bytes_per_set, 1))))


# ---------------------------------------------------------------------- workloads
def make_cast_transpose_2d(torch, fq, W, inner_2d=False):
    R = C = 4096
    x = W.weight_4096_outlier_cols()
    cfg = fq.make_cfg(format="nvfp4", two_level="outer_block", outer_block_size=64, outer_2d=True, inner_2d=inner_2d)
    alg = R * C * 2 + 2 * (R * C // 2) + 2 * (R * C // 16) + (R // 64) * (C // 64) * 4
    nset = n_sets_for(alg)
    src = torch.from_numpy(x.view("int16")).cuda()
    sets = []
    for _ in range(nset):
        s = dict(x=src.clone(), rc=torch.empty(R * C // 2, dtype=torch.uint8, device="cuda"),
                 rs=torch.empty(R * C // 16, dtype=torch.uint8, device="cuda"),
                 cc=torch.empty(R * C // 2, dtype=torch.uint8, device="cuda"),
                 cs=torch.empty(R * C // 16, dtype=torch.uint8, device="cuda"),
                 ro=torch.empty((R // 64) * (C // 64), dtype=torch.float32, device="cuda"))
        sets.append(s)
    L = fq.lib()

    def launch(s):
        st = L.fp4_cast_transpose(ct.byref(cfg), s["x"].data_ptr(), R, C, C, s["rc"].data_ptr(), s["rs"].data_ptr(),
                                  s["ro"].data_ptr(), s["cc"].data_ptr(), s["cs"].data_ptr(), None, None, None, 0,
                                  torch.cuda.current_stream().cuda_stream)
        if st:
            raise fq.Fp4Error(st, "fp4_cast_transpose")
    if inner_2d:
        return Timed("nv_2d_inner16_cast_transpose_4096",
                     "NVFP4 2D 64x64 outer, E4M3 16x16 inner tiles, RTNE, fused cast-transpose 4096x4096 bf16", alg,
                     sets, launch, "k_tile", R * C)
    return Timed("nv_2d_cast_transpose_4096", "NVFP4 2D 64x64 outer, E4M3/16, RTNE, fused cast-transpose 4096x4096 bf16", alg, sets, launch,
                 "k_tile", R * C)


def make_cast_transpose_2d_inner16(torch, fq, W):
    return make_cast_transpose_2d(torch, fq, W, inner_2d=True)


def make_mx_fake_quant(torch, fq, W):
    R = C = 8192
    x = W.mx_weight_8192_edges()
    cfg = fq.make_cfg(format="mxfp4")
    alg = R * C * 2 * 2
    nset = n_sets_for(alg, cap=8)
    src = torch.from_numpy(x.view("int16")).cuda()
    sets = [dict(x=src.clone(), y=torch.empty(R * C, dtype=torch.int16, device="cuda")) for _ in range(nset)]
    L = fq.lib()

    def launch(s):
        st = L.fp4_qdq(ct.byref(cfg), s["x"].data_ptr(), R, C, C, s["y"].data_ptr(), None, None, None, None, None, 0,
                       torch.cuda.current_stream().cuda_stream)
        if st:
            raise fq.Fp4Error(st, "fp4_qdq")
    return Timed("mx_fake_quant_8192", "MXFP4 1x32 fake-quant 8192x8192 bf16 -> bf16", alg, sets, launch, "k_mx_qdq",
                 R * C)


def make_mx_project_fp8(torch, fq, W):
    R = C = 8192
    x = W.mx_weight_8192_edges()
    cfg = fq.make_cfg(format="mxfp4")
    n = R * C
    # read bf16; write bf16 y, MXFP8 row and column payloads + UE8M0 scales,
    # 128x128 payload and its transpose, one FP32 scale per tile
    alg = n * 2 + n * 2 + 2 * (n + n // 32) + 2 * n + 4 * (n // (128 * 128))
    nset = n_sets_for(alg, cap=4)
    src = torch.from_numpy(x.view("int16")).cuda()

    def outs():
        u8 = lambda m: torch.empty(m, dtype=torch.uint8, device="cuda")
        return dict(x=src.clone(), y=torch.empty(n, dtype=torch.int16, device="cuda"), r=u8(n), rs=u8(n // 32),
                    c=u8(n), cs=u8(n // 32), b=u8(n), bt=u8(n),
                    bs=torch.empty(n // (128 * 128), dtype=torch.float32, device="cuda"))
    sets = [outs() for _ in range(nset)]
    L = fq.lib()

    def launch(s):
        st = L.fp4_mx_project_fp8(ct.byref(cfg), s["x"].data_ptr(), R, C, C, s["y"].data_ptr(), s["r"].data_ptr(),
                                  s["rs"].data_ptr(), s["c"].data_ptr(), s["cs"].data_ptr(), s["b"].data_ptr(),
                                  s["bt"].data_ptr(), s["bs"].data_ptr(), torch.cuda.current_stream().cuda_stream)
        if st:
            raise fq.Fp4Error(st, "fp4_mx_project_fp8")
    return Timed("mx_project_fp8_8192", "MXFP4 projection 8192x8192 bf16 -> bf16 y + MXFP8 1x32 / 32x1 + FP8 128x128 (+T)",
                 alg, sets, launch, "k_mx_fp8", n)


def make_mx_fake_quant_fp32(torch, fq, W):
    R = C = 8192
    x = W.from_bf16(W.mx_weight_8192_edges())
    cfg = fq.make_cfg(format="mxfp4", input_dtype="fp32", output_dtype="fp32")
    alg = R * C * 4 * 2
    nset = n_sets_for(alg, cap=4)
    src = torch.from_numpy(x.copy()).cuda()
    sets = [dict(x=src.clone(), y=torch.empty(R * C, dtype=torch.float32, device="cuda")) for _ in range(nset)]
    L = fq.lib()

    def launch(s):
        st = L.fp4_qdq(ct.byref(cfg), s["x"].data_ptr(), R, C, C, s["y"].data_ptr(), None, None, None, None, None, 0,
                       torch.cuda.current_stream().cuda_stream)
        if st:
            raise fq.Fp4Error(st, "fp4_qdq")
    return Timed("mx_fake_quant_fp32_8192", "MXFP4 1x32 fake-quant 8192x8192 fp32 -> fp32", alg, sets, launch,
                 "k_mx_qdq_f32", R * C)


def make_mx_gemm(torch, fq, W):
    """C = A . B^T, 8192^3, MXFP4 operands (quantised from seeded bf16 with the
    library's MXFP4 quantiser), GEMM-ready tiled scales, bf16 C."""
    import numpy as np
    M = N = K = 8192
    cfg = fq.make_cfg(format="mxfp4")
    sets = []
    for k in range(2):
        rng = np.random.default_rng(60 + k)
        xa = torch.from_numpy(W.to_bf16(rng.standard_normal((M, K), dtype=np.float32)).view("int16")).cuda()
        xb = torch.from_numpy(W.to_bf16(rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)).view("int16")).cuda()
        qa, qb = fq.fp4_quantize(xa, cfg), fq.fp4_quantize(xb, cfg)
        del xa, xb
        sets.append(dict(a=qa["codes"], at=fq.fp4_mx_scales_tiled(qa["scales"], K), b=qb["codes"],
                         bt=fq.fp4_mx_scales_tiled(qb["scales"], K), c=torch.empty((M, N), dtype=torch.bfloat16,
                                                                                     device="cuda")))
    torch.cuda.synchronize()
    L = fq.lib()

    def launch(s):
        st = L.fp4_mm(ct.byref(cfg), s["a"].data_ptr(), s["at"].data_ptr(), s["b"].data_ptr(), s["bt"].data_ptr(),
                      M, N, K, 1, s["c"].data_ptr(), N, torch.cuda.current_stream().cuda_stream)
        if st:
            raise fq.Fp4Error(st, "fp4_mm")
    alg = M * K // 2 * 2 + 2 * 8 * ((M + 255) // 256) * ((K + 255) // 256) * 256 + M * N * 2
    return Timed("mx_gemm_8192", "MXFP4 GEMM C = A.B^T 8192x8192x8192, tiled scales, bf16 C", alg, sets, launch,
                 "k_mx_gemm_lds", M * N, flops=2 * M * N * K, graph=False)


def make_cast_transpose_1d_sr(torch, fq, W):
    R, C = 16384, 2880
    x = W.activations_16384x2880()
    cfg = fq.make_cfg(format="amdfp4", two_level="outer_block", outer_block_size=64, rounding="stochastic", seed=7,
                      step=3)
    alg = R * C * 2 + 2 * (R * C // 2) + 2 * (R * C // 16) + (R * (C // 64) + C * (R // 64)) * 4
    nset = n_sets_for(alg, cap=16)
    src = torch.from_numpy(x.view("int16")).cuda()
    sets = []
    for _ in range(nset):
        sets.append(dict(x=src.clone(), rc=torch.empty(R * C // 2, dtype=torch.uint8, device="cuda"),
                         rs=torch.empty(R * C // 16, dtype=torch.uint8, device="cuda"),
                         cc=torch.empty(R * C // 2, dtype=torch.uint8, device="cuda"),
                         cs=torch.empty(R * C // 16, dtype=torch.uint8, device="cuda"),
                         ro=torch.empty(R * (C // 64), dtype=torch.float32, device="cuda"),
                         co=torch.empty(C * (R // 64), dtype=torch.float32, device="cuda")))
    wsb = fq.fp4q_cast_transpose_workspace_bytes(cfg, [R], C) if STAGED else 0
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    L = fq.lib()

    def launch(s):
        st = L.fp4_cast_transpose(ct.byref(cfg), s["x"].data_ptr(), R, C, C, s["rc"].data_ptr(), s["rs"].data_ptr(),
                                  s["ro"].data_ptr(), s["cc"].data_ptr(), s["cs"].data_ptr(), s["co"].data_ptr(), None,
                                  ws.data_ptr(), wsb, torch.cuda.current_stream().cuda_stream)
        if st:
            raise fq.Fp4Error(st, "fp4_cast_transpose")
    return Timed("amd_1d_sr_cast_transpose_16384x2880", "AMD-FP4 1D 1x64 outer, UE5M3/16, SR, cast-transpose 16384x2880 bf16", alg, sets, launch,
                 "k_tile", R * C)


def make_grouped_sr_ef(torch, fq, W):
    E, R, C = 32, 2880, 2880
    w = W.experts_32x2880()
    cfg = fq.make_cfg(format="nvfp4", two_level="outer_block", outer_block_size=64, outer_2d=True,
                      rounding="stochastic", seed=5, step=0)
    n = E * R * C
    alg = n * 2 + n * 4 * 2 + 2 * (n // 2) + 2 * (n // 16) + E * (R // 64) * (C // 64) * 4
    s = dict(x=torch.from_numpy(w.view("int16")).cuda(), z=torch.zeros(n, dtype=torch.float32, device="cuda"),
             rc=torch.empty(n // 2, dtype=torch.uint8, device="cuda"), rs=torch.empty(n // 16, dtype=torch.uint8, device="cuda"),
             cc=torch.empty(n // 2, dtype=torch.uint8, device="cuda"), cs=torch.empty(n // 16, dtype=torch.uint8, device="cuda"),
             ro=torch.empty(E * (R // 64) * (C // 64), dtype=torch.float32, device="cuda"))
    rows = (ct.c_int64 * E)(*([R] * E))
    wsb = fq.fp4q_cast_transpose_workspace_bytes(cfg, [R] * E, C, with_residual=True) if STAGED else 0
    s["ws"] = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    L = fq.lib()

    def launch(s):
        st = L.fp4_cast_transpose_grouped(ct.byref(cfg), E, rows, C, s["x"].data_ptr(), C, s["rc"].data_ptr(),
                                          s["rs"].data_ptr(), s["ro"].data_ptr(), s["cc"].data_ptr(), s["cs"].data_ptr(),
                                          None, s["z"].data_ptr(), s["ws"].data_ptr(), wsb,
                                          torch.cuda.current_stream().cuda_stream)
        if st:
            raise fq.Fp4Error(st, "fp4_cast_transpose_grouped")
    # the working set (~3 GB per step) is far beyond the last-level cache: one set
    t = Timed("nv_grouped_sr_ef_32x2880", "grouped NVFP4 2D 64x64 outer, E4M3/16, SR + in-place EF residual, 32 x 2880x2880",
              alg, [s], launch, "k_tile + k_gather" if STAGED else "k_tile", n)
    t.source = w
    return t


def make_tensorwise_qdq(torch, fq, W):
    R = C = 256
    x = W.tensorwise_input_256()
    cfg = fq.make_cfg(format="nvfp4", two_level="tensorwise")
    alg = R * C * 2 + R * C // 2 + R * C // 16 + 4 + R * C * 2
    ws = torch.empty(fq.fp4q_workspace_bytes(cfg, R, C), dtype=torch.uint8, device="cuda")
    s = dict(x=torch.from_numpy(x.view("int16")).cuda(), y=torch.empty(R * C, dtype=torch.int16, device="cuda"),
             c=torch.empty(R * C // 2, dtype=torch.uint8, device="cuda"),
             sc=torch.empty(R * C // 16, dtype=torch.uint8, device="cuda"),
             o=torch.empty(1, dtype=torch.float32, device="cuda"))
    L = fq.lib()

    def launch(s):
        st = L.fp4_qdq(ct.byref(cfg), s["x"].data_ptr(), R, C, C, s["y"].data_ptr(), s["c"].data_ptr(),
                       s["sc"].data_ptr(), s["o"].data_ptr(), None, ws.data_ptr(), ws.numel(),
                       torch.cuda.current_stream().cuda_stream)
        if st:
            raise fq.Fp4Error(st, "fp4_qdq")
    return Timed("nv_tensorwise_qdq_256", "NVFP4 tensorwise QDQ 256x256 (one launch: each workgroup takes the tensor amax)", alg, [s], launch,
                 "k_nv_rows", R * C)


# ---------------------------------------------------------------------- CPU baseline
def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def check_and_cpu_baseline(torch, fq, W, w):
    """One more step of the headline workload, from a snapshot of its residual,
    checked buffer by buffer against the oracle; that oracle run (all host
    cores, the whole step) is the CPU baseline, and one expert is timed on one
    core.  Returns (bit-exact verdicts, cpu_baseline record)."""
    import numpy as np
    from oracle import ref
    s = w.sets[0]
    E, R, C = 32, 2880, 2880
    z0 = s["z"].detach().cpu().numpy().reshape(E * R, C).copy()
    w.launch(s)
    torch.cuda.synchronize()
    got = {k: s[k].detach().cpu().numpy() for k in ("rc", "rs", "cc", "cs", "ro", "z")}
    x = w.source
    zo = z0.copy()
    cores = ref.threads()
    kw = dict(two_level="outer", obs=64, outer_2d=True, stochastic=True, seed=5, step=0)
    t0 = time.perf_counter()
    want = ref.nv_quantize_grouped(x, [R] * E, residual=zo, **kw)
    el_total = time.perf_counter() - t0
    # the baseline sample: the same whole step again until about 10 s of oracle time
    runs = 1
    while el_total < 10.0 and runs < 8:
        zr = z0.copy()
        t0 = time.perf_counter()
        ref.nv_quantize_grouped(x, [R] * E, residual=zr, **kw)
        el_total += time.perf_counter() - t0
        runs += 1
    el = el_total / runs
    names = {"row_codes": ("rc", want["row_codes"]), "row_scales": ("rs", want["row_scales"]),
             "col_codes": ("cc", want["col_codes"]), "col_scales": ("cs", want["col_scales"]),
             "outer_fp32": ("ro", want["row_outer"]), "residual_fp32": ("z", zo)}
    verdict = {}
    for k, (gk, ref_arr) in names.items():
        a = got[gk].view(np.uint8).ravel()
        b = np.ascontiguousarray(ref_arr).view(np.uint8).ravel()
        verdict[k] = bool(a.size == b.size and np.array_equal(a, b))
    # two experts on one core
    ref.set_threads(1)
    n1 = 2
    t1 = time.perf_counter()
    for e in range(n1):
        z1 = z0[e * R:(e + 1) * R].copy()
        ref.nv_quantize(np.ascontiguousarray(x[e * R:(e + 1) * R]), two_level="outer", obs=64, outer_2d=True,
                        stochastic=True, seed=5, step=0, residual=z1, cols=True, want_y=False)
    el1 = (time.perf_counter() - t1) / n1
    ref.set_threads(cores)
    base = {"value": round(w.bytes / el / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": "the whole grouped step (32 experts of 2880x2880, both directions, residual update), %d runs, "
                      "%.1f s in all, %.2f s per step" % (runs, el_total, el),
            "single_thread_GB/s": round(w.bytes / E / el1 / 1e9, 4),
            "single_thread_sample": "%d experts (1/32 of the step each) on one core: %.2f s per expert" % (n1, el1),
            "cpu": cpu_model()}
    return verdict, base


def copy_ceiling(torch, total_bytes, steps=2000):
    """GB/s of a plain device copy moving the same number of bytes (half read,
    half written) as one headline launch, timed the same way: rotating buffers
    over >= 1 GiB, replayed from a graph."""
    n = total_bytes // 2
    sets = [(torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1), torch.empty(n, dtype=torch.uint8, device="cuda"))
            for _ in range(n_sets_for(total_bytes))]
    w = Timed("copy", "device copy", total_bytes, sets, lambda s: s[1].copy_(s[0]), "copy")
    ms = run_timed(torch, w, steps, 50)
    return round(total_bytes * steps / (ms * 1e-3) / 1e9, 2)


# ---------------------------------------------------------------------- main
def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the quantisation path has no cross-GPU step "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import block_scaled_fp4_amax_amd as fq
    from block_scaled_fp4_amax_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    if args.copy_probe:
        n = COPY_PROBE_BYTES
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        for _ in range(20):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 20}))
        return

    makers = {"nv_tensorwise_qdq_256": make_tensorwise_qdq, "nv_2d_cast_transpose_4096": make_cast_transpose_2d,
              "mx_fake_quant_8192": make_mx_fake_quant,
              "amd_1d_sr_cast_transpose_16384x2880": make_cast_transpose_1d_sr,
              "nv_grouped_sr_ef_32x2880": make_grouped_sr_ef,
              "nv_2d_inner16_cast_transpose_4096": make_cast_transpose_2d_inner16,
              "mx_project_fp8_8192": make_mx_project_fp8,
              "mx_fake_quant_fp32_8192": make_mx_fake_quant_fp32,
              "mx_gemm_8192": make_mx_gemm}
    if args.only:
        w = makers[args.only](torch, fq, W)
        ms = run_timed(torch, w, args.steps, args.warmup, graph=w.graph and not args.eager)
        per = ms / args.steps
        rec = {"workload": w.name, "desc": w.desc, "ms_per_launch": per,
               "GB/s": w.bytes / (per * 1e-3) / 1e9, "frac": w.bytes / (per * 1e-3) / 1e9 / HBM_PEAK_GBS}
        if w.flops:
            tf = w.flops / (per * 1e-3) / 1e12
            rec.update({"TFLOP/s": tf, "frac": tf / FP4_MFMA_PEAK_TFLOPS, "bound": "mfma"})
        print(json.dumps(rec))
        return

    key = "nv_grouped_sr_ef_32x2880"
    w = make_grouped_sr_ef(torch, fq, W)
    print("# headline %s: %d warmup + %d timed steps" % (w.name, args.warmup, args.steps), file=sys.stderr, flush=True)
    ms = run_timed(torch, w, args.steps, args.warmup, graph=not args.eager)
    per_ms = ms / args.steps
    gbs = w.bytes * args.steps / (ms * 1e-3) / 1e9
    traffic = measured_traffic(key)
    line = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(per_ms, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.desc, "experts": 32, "rows_per_expert": 2880, "cols": 2880, "source": "bf16",
                   "format": "nvfp4", "two_level": "outer_block 2D 64x64, one outer grid per expert",
                   "inner": "E4M3/16", "rounding": "stochastic (Philox4x32-10, seed 5)",
                   "error_feedback": "fp32 residual [92160, 2880], read and rewritten in place every step",
                   "outputs": "rowwise+columnwise codes and scales, shared 2D outer scales",
                   "algorithmic_bytes_per_step": w.bytes, "elements_per_step": w.elements,
                   "inputs_sha256": {"x_bf16_bits": hashlib.sha256(w.source.tobytes()).hexdigest(),
                                     "residual_start": "zeros"}},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     # measured HBM bytes per step (staging round trip included) over the same step time
                     "traffic_GB/s": round(traffic / (per_ms * 1e-3) / 1e9, 2) if traffic else None,
                     "kernel": "one step = k_tile (tile pass) + k_gather (whole-line gather), timed together",
                     "traffic_source": "profiles/traffic_counters.json[%s] (rocprofv3 FETCH_SIZE + WRITE_SIZE of "
                                       "both kernels per step, scaled by a plain copy)" % key},
        "elements_per_s": round(w.elements * args.steps / (ms * 1e-3), 1),
    }
    if not args.no_cpu_baseline:
        print("# oracle check of one more step + cpu baseline", file=sys.stderr, flush=True)
        verdict, base = check_and_cpu_baseline(torch, fq, W, w)
        line["bit_exact_vs_oracle"] = verdict
        line["cpu_baseline"] = base
    del w
    torch.cuda.empty_cache()
    if not args.no_extra:
        extra = {}
        for mk, steps in ((make_cast_transpose_2d, 2000), (make_mx_fake_quant, 400), (make_cast_transpose_1d_sr, 400),
                          (make_tensorwise_qdq, 2000), (make_cast_transpose_2d_inner16, 2000),
                          (make_mx_project_fp8, 200), (make_mx_fake_quant_fp32, 200), (make_mx_gemm, 50)):
            e = mk(torch, fq, W)
            print("# extra %s" % e.name, file=sys.stderr, flush=True)
            ems = run_timed(torch, e, steps, min(20, steps), graph=e.graph)
            per = ems / steps
            eg = e.bytes / (per * 1e-3) / 1e9
            extra[e.name] = {"desc": e.desc, "us_per_step": round(per * 1e3, 3), "GB/s": round(eg, 2),
                             "frac": round(eg / HBM_PEAK_GBS, 4), "algorithmic_bytes": e.bytes, "kernel": e.kernel,
                             "elements_per_s": round(e.elements / (per * 1e-3), 1)}
            if e.flops:
                tf = e.flops / (per * 1e-3) / 1e12
                extra[e.name].update({"bound": "mfma", "TFLOP/s": round(tf, 1), "peak_TFLOP/s": FP4_MFMA_PEAK_TFLOPS,
                                      "frac": round(tf / FP4_MFMA_PEAK_TFLOPS, 4), "flops": e.flops})
            t = measured_traffic(e.name)
            if t is not None:
                extra[e.name]["traffic"] = t
            del e
            torch.cuda.empty_cache()
        line["extra"] = extra
        cc = copy_ceiling(torch, 64 << 20)
        line["context"] = {"plain_copy_64MiB_GB/s": cc}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
