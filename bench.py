#!/usr/bin/env python3
"""Throughput of the tensor-parallel MLP shard path on one MI355X.

One step is one pass of the whole path over one batch: for every rank i of the
N-way split, the column-parallel GEMM with fused GeLU (Z_i = bf16(GeLU(X·A_i)))
and the row-parallel GEMM (Y_i = Z_i·B_i, fp32), then the on-device sum of the
N partials (Y = Σ_i Y_i). These are the same two launches tp_mlp_shard makes
per rank; the bench calls them separately so each kernel can be timed with HIP
events on the stream it runs on.

Default workload: 7b_tp8 - d = 4096, TP N = 8, X[8192x4096] (4 x 2048 tokens),
A_i[4096x2048], B_i[2048x4096]; all 8 ranks then the sum. Other workloads:
gpt2s_n1, 175b_tp8, 175b_tp8_e4m3 (fp8: col GEMM + GeLU + amax, requantise Z,
row GEMM; inputs quantised once, outside the timed region) and
175b_tp8_e4m3_delayed (fp8 with delayed scaling of Z: col GEMM + GeLU + e4m3
with the predicted scale + amax, row GEMM, amax history push) and 7b_tp8_bwd
(the backward of every rank's 7b_tp8 shard for an output gradient dY: one
tp_mlp_shard_backward call per rank, five GEMMs, then the sum of the ranks'
input gradients dX_i) and 7b_tp8_attn (the attention block: every rank's
QKV projection, causal attention of its 4 heads and output projection, then
the sum of the partials).

Prints one JSON line. `value` is TFLOP/s over the whole step (FLOPs =
4·M·d·F per rank shard forward, 10·M·d·F backward; GeLU, GeLU', scaling and
the sum are not counted).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def _host_cores() -> int:
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n)


HOST_CORES = _host_cores()
# the oracle's BLAS thread count is fixed when numpy loads
os.environ.setdefault("OPENBLAS_NUM_THREADS", str(HOST_CORES))

import numpy as np  # noqa: E402

METRIC = "TFLOP/s and % of MFMA peak per TP-rank MLP shard (GeLU(X·A_i)·B_i), 1 GPU"
METRIC_BWD = "TFLOP/s and % of MFMA peak per TP-rank MLP shard backward (dX_i, dA_i, dB_i), 1 GPU"
METRIC_ATTN = ("TFLOP/s and % of MFMA peak per TP-rank attention shard (QKV projection, causal "
               "attention, output projection), 1 GPU")
PEAK_TFLOPS = {"bf16": 2516.6, "e4m3": 5033.2}   # MI355X dense MFMA (256 CU x 2.4 GHz)
HBM_PEAK_GBS = 8000.0


def kernel_source_sha256() -> str:
    """Hash of every kernel source file; counter figures are tied to it."""
    d = os.path.join(ROOT, "megatron_tensor_transformer_shard_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        h.update(f.encode())
        with open(os.path.join(d, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


# The partial dtype the committed traffic profiles were taken with.
PROFILED_PARTIAL_DTYPE = "f32"


def measured_traffic(workload: str, kernel: str, partial_dtype: str = PROFILED_PARTIAL_DTYPE):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE passes (scaled by the copy calibration), or None when there are
    none for this workload, the kernels have changed since they were taken, or
    the run's partials differ in dtype from the profiled run's."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path) or partial_dtype != PROFILED_PARTIAL_DTYPE:
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_sha256") != kernel_source_sha256() or kernel not in t.get("kernels", {}):
        return None
    return int(round(t["kernels"][kernel]["bytes"]))


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="7b_tp8",
                   help="7b_tp8 (default), gpt2s_n1, 175b_tp8, 175b_tp8_e4m3, 175b_tp8_e4m3_delayed, "
                        "7b_tp8_bwd, 7b_tp8_bwd_fp8, 7b_tp8_attn, library_compare (the 7B-class column GEMM "
                        "against torch.matmul on the same data), "
                        "or copy (a "
                        "1-part tp_partial_sum over 256 MiB of fp32: the known-size copy that "
                        "calibrates rocprofv3's FETCH_SIZE / WRITE_SIZE)")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the timed oracle leg")
    p.add_argument("--no-cold", action="store_true",
                   help="skip the cold pass (for counter runs, whose per-dispatch averages it would mix)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="stop adding oracle row chunks once this much CPU time is spent")
    p.add_argument("--partial-dtype", choices=["f32", "bf16"], default="f32")
    p.add_argument("--eager", action="store_true",
                   help="time the steps' launches eagerly (default: one HIP graph of all K steps, replayed)")
    p.add_argument("--no-clock", action="store_true",
                   help="skip the pass that reads the shader clock inside the stamped kernels")
    p.add_argument("--weight-layout", choices=["math", "linear"], default="math",
                   help="bf16 forward only: weights as A [d, H], B [H, d] (math), or as the "
                        "linear layers store them, W1 [H, d], W2 [d, H] (linear)")
    return p.parse_args()


def dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


# spin cycles (shader clock) queued before each step of an event-timed pass:
# 2-5 ms at the clocks a loaded MI355X runs at
LEAD_CYCLES = 6_000_000


class KernelTimer:
    """HIP events recorded on the current stream around each launch."""

    def __init__(self):
        self.marks = {}

    def around(self, name, fn):
        import torch
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.marks.setdefault(name, []).append((a, b))

    def summary(self):
        out = {}
        for name, pairs in self.marks.items():
            ms = [a.elapsed_time(b) for a, b in pairs]
            out[name] = {"launches": len(ms), "avg_us": 1e3 * float(np.mean(ms)),
                         "median_us": 1e3 * float(np.median(ms)),
                         "min_us": 1e3 * float(np.min(ms)), "total_ms": float(np.sum(ms))}
        return out


class ColdTimer(KernelTimer):
    """KernelTimer with a 512 MiB write before every timed launch (outside the
    events), which evicts L2 and the 256 MB Infinity Cache: each launch then
    starts from HBM."""

    def __init__(self):
        import torch
        super().__init__()
        self.scratch = torch.empty(128 << 20, dtype=torch.float32, device="cuda")

    def around(self, name, fn):
        self.scratch.fill_(1.0)
        super().around(name, fn)


class ClockSampler:
    """Samples the engine clock the driver reports as current (the line it
    marks in pp_dpm_sclk) every few milliseconds from a thread while a pass
    runs. Only when the box shows exactly one such GPU (else no samples)."""

    def __init__(self, period_s=0.003):
        import glob
        paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = paths[0] if len(paths) == 1 else None
        self.period = period_s
        self.samples = []
        self._stop = None
        self._thread = None

    def _read(self):
        try:
            with open(self.path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        return float(line.split(":")[1].strip().split("M")[0])
        except (OSError, ValueError, IndexError):
            return None
        return None

    def __enter__(self):
        import threading
        if self.path is None:
            return self
        self._stop = threading.Event()

        def run():
            while not self._stop.wait(self.period):
                v = self._read()
                if v is not None:
                    self.samples.append(v)
        self._thread = threading.Thread(target=run, daemon=True)
        self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        return False

    def summary(self):
        if not self.samples:
            return None
        v = np.array(self.samples)
        return {"samples": int(v.size), "median_mhz": float(np.median(v)), "mean_mhz": round(float(v.mean()), 1),
                "min_mhz": float(v.min()), "max_mhz": float(v.max())}


def device_peak(tpm_peak_key):
    """The dense MFMA peak recomputed from the device's own figures: CUs and
    peak engine clock from hipDeviceGetAttribute (the clock torch does not
    expose on ROCm), times 4096 (bf16) or 8192 (fp8) flops per CU per clock."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        dev = ctypes.c_int()
        if hip.hipGetDevice(ctypes.byref(dev)) != 0:
            return None
        vals = {}
        # hipDeviceAttributeClockRate, ...MultiprocessorCount, ...ClockInstructionRate
        # (the rate HIP states for the device-side clock counters), ...WallClockRate
        for name, attr in (("clock_khz", 5), ("cus", 63), ("clock_instruction_rate_khz", 10000),
                           ("wall_clock_rate_khz", 10017)):
            v = ctypes.c_int()
            if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, dev) != 0:
                return None
            vals[name] = v.value
    except OSError:
        return None
    per_clk = 8192 if tpm_peak_key == "e4m3" else 4096
    vals["peak_tflops"] = vals["cus"] * vals["clock_khz"] * 1e3 * per_clk / 1e12
    return vals


def wall_clock_hz():
    """Rate of the constant counter the kernels' clock stamps read
    (hipDeviceAttributeWallClockRate, kHz), or None."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        dev, v = ctypes.c_int(), ctypes.c_int()
        if hip.hipGetDevice(ctypes.byref(dev)) != 0:
            return None
        if hip.hipDeviceGetAttribute(ctypes.byref(v), 10017, dev) != 0 or v.value <= 0:
            return None
        return v.value * 1e3
    except OSError:
        return None


def clock_pass(tpm, step, reps=5):
    """The shader clock inside the stamped kernels under the benchmark's own
    sustained load: `reps` ordinary steps back to back, with no
    synchronisation between them, in which one rank's launches carry clock
    stamps (the same kernels given a stamps array). For each workgroup, its
    shader-clock cycles over its constant-counter time; per kernel, the median
    over workgroups and launches, and the span from the first workgroup's start
    to the last one's end (the in-kernel duration, without the launch overhead
    that HIP events include)."""
    import torch
    shapes = getattr(step, "stamp_shapes", None)
    hz = wall_clock_hz()
    if not shapes or hz is None:
        return None
    bufs = [{k: torch.zeros(tpm.tp_clock_stamp_count(*mn), dtype=torch.int64, device="cuda")
             for k, mn in shapes.items()} for _ in range(reps)]
    torch.cuda.synchronize()
    for b in bufs:
        step(stamp=b)
    torch.cuda.synchronize()
    out = {}
    for name in shapes:
        clocks, spans = [], []
        for b in bufs:
            q = b[name].cpu().numpy().view(np.uint64).reshape(-1, 4)
            q = q[np.any(q != 0, axis=1)].astype(np.float64)
            if len(q) == 0:
                return None
            clocks.append((q[:, 2] - q[:, 0]) / ((q[:, 3] - q[:, 1]) / hz))
            spans.append((q[:, 3].max() - q[:, 1].min()) / hz)
        c = np.concatenate(clocks)
        out[name] = {"workgroups": int(len(clocks[0])), "launches": reps,
                     "clock_ghz_median": round(float(np.median(c)) / 1e9, 4),
                     "clock_ghz_min": round(float(c.min()) / 1e9, 4),
                     "clock_ghz_max": round(float(c.max()) / 1e9, 4),
                     "span_us_median": round(1e6 * float(np.median(spans)), 2),
                     "wall_clock_hz": hz}
    return out


def build_bf16_step(tpm, wl, partial_dtype, weight_layout="math"):
    """The forward of every rank's shard, then the sum of the partials. With
    the linear layout the weights are stored [out, in] (W1 = Aᵀ, W2 = Bᵀ,
    transposed once outside the timed region) and the rank's shards are a row
    block of W1 and a column block of W2."""
    import torch
    X, A, B = __import__("workloads").make_inputs(wl)
    Xd, Ad, Bd = dev_bf16(X), dev_bf16(A), dev_bf16(B)
    M, d, H, N, F = wl.M, wl.d, wl.H, wl.N, wl.F
    pdt = torch.float32 if partial_dtype == "f32" else torch.bfloat16
    Z = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    parts = [torch.empty((M, d), dtype=pdt, device="cuda") for _ in range(N)]
    Y = torch.empty((M, d), dtype=torch.float32, device="cuda")
    if weight_layout == "linear":
        W1, W2 = Ad.t().contiguous(), Bd.t().contiguous()
        del Ad, Bd
        views = [(W1[r * F:(r + 1) * F], W2[:, r * F:(r + 1) * F]) for r in range(N)]
        col, row, kc, kr = tpm.tp_mlp_col_gelu_wt, tpm.tp_mlp_row_partial_wt, "col_gelu_wt", "row_partial_wt"
    else:
        views = [(Ad[:, r * F:(r + 1) * F], Bd[r * F:(r + 1) * F, :]) for r in range(N)]
        col, row, kc, kr = tpm.tp_mlp_col_gelu, tpm.tp_mlp_row_partial, "col_gelu", "row_partial"

    def step(timer=None, stamp=None):
        for r in range(N):
            A_i, B_i = views[r]
            # one middle rank's launches with clock stamps (rank 0's follow the
            # previous step's partial sum and its 134 MB of fresh writes)
            if stamp is not None and r == N // 2:
                tpm.tp_mlp_col_gelu_stamped(Xd, A_i, stamp[kc], Z)
                tpm.tp_mlp_row_partial_stamped(Z, B_i, stamp[kr], parts[r])
            elif timer is None:
                col(Xd, A_i, Z)
                row(Z, B_i, parts[r])
            else:
                timer.around(kc, lambda: col(Xd, A_i, Z))
                timer.around(kr, lambda: row(Z, B_i, parts[r]))
        if N > 1:
            if timer is None:
                tpm.tp_partial_sum(parts, Y=Y)
            else:
                timer.around("partial_sum", lambda: tpm.tp_partial_sum(parts, Y=Y))

    if weight_layout != "linear":
        # output shapes of the launches step(stamp=...) runs with clock stamps
        step.stamp_shapes = {kc: (M, F), kr: (M, d)}
    kern_flops = {kc: 2 * M * d * F, kr: 2 * M * d * F}
    # algorithmic bytes: each operand read once, each output written once
    kern_bytes = {kc: (M * d + d * F) * 2 + M * F * 2,
                  kr: (M * F + F * d) * 2 + M * d * parts[0].element_size()}
    psum_bytes = (N * parts[0].element_size() + Y.element_size()) * M * d
    out = Y if N > 1 else parts[0]
    return step, kern_flops, kern_bytes, psum_bytes, (X, A, B), out


def build_bwd_step(tpm, wl):
    """Backward of every rank's shard: one tp_mlp_shard_backward call per rank
    (S recomputed, dS with GeLU', dX_i, dB_i, dA_i), or its fp8 form (the
    operands quantised inside the call), then Σ_i dX_i."""
    import torch
    from workloads import make_inputs, make_output_grad
    X, A, B = make_inputs(wl)
    dY = make_output_grad(wl.M, wl.d, wl.seed, wl.grad_sigma)
    Xd, Ad, Bd, dYd = dev_bf16(X), dev_bf16(A), dev_bf16(B), dev_bf16(dY)
    M, d, H, N, F = wl.M, wl.d, wl.H, wl.N, wl.F
    fn = tpm.tp_mlp_shard_backward_fp8 if wl.fp8 else tpm.tp_mlp_shard_backward
    size = (tpm.tp_mlp_shard_backward_fp8_workspace_size if wl.fp8
            else tpm.tp_mlp_shard_backward_workspace_size)
    ws = torch.empty(size(M, d, H, N), dtype=torch.uint8, device="cuda")
    dXs = [torch.empty((M, d), dtype=torch.float32, device="cuda") for _ in range(N)]
    dA = torch.empty((d, F), dtype=torch.float32, device="cuda")
    dB = torch.empty((F, d), dtype=torch.float32, device="cuda")
    dX = torch.empty((M, d), dtype=torch.float32, device="cuda")

    # fp8: the weights' whole-tensor amaxes, once per step for every rank (as
    # a real rank would all-reduce the amax of its own shard), inside the step
    wam = torch.empty(2, dtype=torch.float32, device="cuda")
    extra = {"w_amax": wam} if wl.fp8 else {}

    def weight_amax():
        tpm.tp_amax_bf16(Ad, amax=wam[0:1])
        tpm.tp_amax_bf16(Bd, amax=wam[1:2])

    def step(timer=None):
        if wl.fp8:
            if timer is None:
                weight_amax()
            else:
                timer.around("weight_amax", weight_amax)
        for r in range(N):
            def call(r=r):
                fn(Xd, Ad, Bd, dYd, N, r, dX_i=dXs[r], dA_i=dA, dB_i=dB, workspace=ws, **extra)
            if timer is None:
                call()
            else:
                timer.around("shard_backward", call)
        if N > 1:
            if timer is None:
                tpm.tp_partial_sum(dXs, Y=dX)
            else:
                timer.around("partial_sum", lambda: tpm.tp_partial_sum(dXs, Y=dX))

    kern_flops = {"shard_backward": 10 * M * d * F}
    # algorithmic bytes of one call: X, dY, A_i, B_i read once; dX_i, dA_i,
    # dB_i written once (the S, dS, Z intermediates and, for fp8, the
    # quantised copies are not counted)
    kern_bytes = {"shard_backward": (2 * M * d + 2 * d * F) * 2 + (M * d + 2 * d * F) * 4}
    psum_bytes = (N + 1) * 4 * M * d
    return step, kern_flops, kern_bytes, psum_bytes, (X, A, B, dY), (dX if N > 1 else dXs[0])


def build_attn_step(tpm, wl):
    """Attention block of every rank: QKV projection, per-head attention,
    output projection (the three launches tp_attn_shard makes), then Σ_i Y_i."""
    import torch
    from workloads import make_attn_inputs
    X, Wqkv, Wo = make_attn_inputs(wl)
    Xd, Wd, Wod = dev_bf16(X), dev_bf16(Wqkv), dev_bf16(Wo)
    M, d, N, F, B, S = wl.M, wl.d, wl.N, wl.F, wl.B, wl.S
    hr = wl.heads // N
    QKV = torch.empty((M, 3 * F), dtype=torch.bfloat16, device="cuda")
    O = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    parts = [torch.empty((M, d), dtype=torch.float32, device="cuda") for _ in range(N)]
    Y = torch.empty((M, d), dtype=torch.float32, device="cuda")
    views = [(Wd[:, r * 3 * F:(r + 1) * 3 * F], Wod[r * F:(r + 1) * F, :]) for r in range(N)]

    def step(timer=None):
        for r in range(N):
            W_i, Wo_i = views[r]
            calls = [("qkv_proj", lambda: tpm.tp_attn_qkv(Xd, W_i, QKV)),
                     ("attention", lambda: tpm.tp_attn_heads(QKV, B, S, hr, wl.causal, O)),
                     ("out_proj", lambda: tpm.tp_mlp_row_partial(O, Wo_i, parts[r]))]
            for name, fn in calls:
                if timer is None:
                    fn()
                else:
                    timer.around(name, fn)
        if N > 1:
            if timer is None:
                tpm.tp_partial_sum(parts, Y=Y)
            else:
                timer.around("partial_sum", lambda: tpm.tp_partial_sum(parts, Y=Y))

    att = 4 * S * S * wl.dh * hr * B // (2 if wl.causal else 1)
    kern_flops = {"qkv_proj": 2 * M * d * 3 * F, "attention": att, "out_proj": 2 * M * F * d}
    kern_bytes = {"qkv_proj": (M * d + d * 3 * F) * 2 + M * 3 * F * 2,
                  "attention": M * 3 * F * 2 + M * F * 2,
                  "out_proj": (M * F + F * d) * 2 + M * d * 4}
    psum_bytes = (N + 1) * 4 * M * d
    return step, kern_flops, kern_bytes, psum_bytes, (X, Wqkv, Wo), (Y if N > 1 else parts[0])


def build_e4m3_step(tpm, wl):
    import torch
    X, A, B = __import__("workloads").make_inputs(wl)
    M, d, F = wl.M, wl.d, wl.F

    def quant(bits):
        T = dev_bf16(bits)
        amax = tpm.tp_amax_bf16(T)
        return tpm.tp_quant_e4m3(T, amax)
    (Xq, sX), (Aq, sA), (Bq, sB) = quant(X), quant(A), quant(B)
    torch.cuda.synchronize()
    Z = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    Zq = torch.empty((M, F), dtype=torch.uint8, device="cuda")
    za = torch.empty(1, dtype=torch.float32, device="cuda")
    sZ = torch.empty(1, dtype=torch.float32, device="cuda")
    Y = torch.empty((M, d), dtype=torch.bfloat16, device="cuda")
    kern_flops = {"col_gelu_e4m3": 2 * M * d * F, "row_partial_e4m3": 2 * M * d * F}
    kern_bytes = {"col_gelu_e4m3": M * d + d * F + M * F * 2,
                  "row_partial_e4m3": M * F + F * d + M * d * 2}

    if "delayed" in wl.tags:
        # delayed scaling of Z: the column GEMM quantises Z with the scale
        # predicted from the amax history; the step ends by recording its amax
        hist = tpm.AmaxHistory(1024, initial_scale=1.0)

        def step(timer=None, stamp=None):
            st = None if stamp is None else stamp["row_partial_e4m3"]
            calls = [("col_gelu_e4m3_delayed",
                      lambda: tpm.tp_mlp_col_gelu_e4m3_delayed(Xq, sX, Aq, sA, hist.scale, Zq, za)),
                     ("row_partial_e4m3",
                      lambda: tpm.tp_mlp_row_partial_e4m3(Zq, hist.scale, Bq, sB, Y, stamps=st)),
                     ("amax_history_push", lambda: hist.push(za))]
            for name, fn in calls:
                if timer is None:
                    fn()
                else:
                    timer.around(name, fn)

        step.stamp_shapes = {"row_partial_e4m3": (M, d)}
        kern_flops = {"col_gelu_e4m3_delayed": 2 * M * d * F, "row_partial_e4m3": 2 * M * d * F}
        kern_bytes = {"col_gelu_e4m3_delayed": M * d + d * F + M * F,
                      "row_partial_e4m3": M * F + F * d + M * d * 2}
        return step, kern_flops, kern_bytes, 0, (X, A, B), Y

    def step(timer=None, stamp=None):
        st = None if stamp is None else stamp["row_partial_e4m3"]
        calls = [("col_gelu_e4m3", lambda: tpm.tp_mlp_col_gelu_e4m3(Xq, sX, Aq, sA, Z, za)),
                 ("quant_z", lambda: tpm.tp_quant_e4m3(Z, za, Zq, sZ)),
                 ("row_partial_e4m3",
                  lambda: tpm.tp_mlp_row_partial_e4m3(Zq, sZ, Bq, sB, Y, stamps=st))]
        for name, fn in calls:
            if timer is None:
                fn()
            else:
                timer.around(name, fn)

    step.stamp_shapes = {"row_partial_e4m3": (M, d)}
    return step, kern_flops, kern_bytes, 0, (X, A, B), Y


def cpu_baseline_attn(wl, inputs, budget_s):
    """Time the oracle's attention shard on whole sequences (all ranks + sum)
    until the budget is spent; FLOPs counted as the GPU's are."""
    import oracle
    from oracle import attention as oat
    X, Wqkv, Wo = inputs
    done = 0
    t_total = 0.0
    while done < wl.B and t_total < budget_s:
        rows = slice(done * wl.S, (done + 1) * wl.S)
        t0 = time.perf_counter()
        parts = [oat.attn_shard(X[rows], Wqkv, Wo, wl.N, r, 1, wl.S, wl.heads, wl.causal)
                 for r in range(wl.N)]
        if wl.N > 1:
            oracle.partial_sum(parts)
        t_total += time.perf_counter() - t0
        done += 1
    flops = wl.N * wl.flops_per_shard() * done // wl.B
    what = (f"sequences [0, {done}) of {wl.B} of the {wl.name} step (all {wl.N} ranks + sum), "
            f"float64 numpy/OpenBLAS oracle, {t_total:.2f} s")
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": HOST_CORES,
            "kind": "oracle", "sample": what, "seconds": t_total}


def cpu_baseline(wl, inputs, budget_s):
    """Time the oracle as it stands on row chunks of the same step until the budget is spent."""
    import oracle
    if hasattr(wl, "heads"):
        return cpu_baseline_attn(wl, inputs, budget_s)
    X, A, B = inputs[:3]
    chunk = max(1, min(wl.M, 1024))
    if wl.fp8 and wl.backward:   # one rank's whole fp8 backward (quantisation included)
        t0 = time.perf_counter()
        oracle.mlp_shard_backward_fp8(X, A, B, inputs[3], wl.N, 0)
        t = time.perf_counter() - t0
        return {"value": wl.flops_per_shard() / t / 1e12, "unit": "TFLOP/s", "cores": HOST_CORES,
                "kind": "oracle",
                "sample": f"rank 0 of {wl.N}: the whole fp8 backward of {wl.name} (all {wl.M} "
                          f"rows, quantisation included), float64 numpy/OpenBLAS oracle, {t:.2f} s",
                "seconds": t}
    if wl.fp8:   # input quantisation is preparation (outside the GPU's timed step too)
        Xq, sX = oracle.quantize_inputs_e4m3(X)
        Aq, sA = oracle.quantize_inputs_e4m3(A)
        Bq, sB = oracle.quantize_inputs_e4m3(B)
    done = 0
    t_total = 0.0
    while done < wl.M and t_total < budget_s:
        rows = slice(done, min(wl.M, done + chunk))
        t0 = time.perf_counter()
        if wl.backward:   # every row costs the five GEMMs' 10·d·F flops per rank
            parts = [oracle.mlp_shard_backward(X[rows], A, B, inputs[3][rows], wl.N, r)["dX"]
                     for r in range(wl.N)]
            if wl.N > 1:
                oracle.partial_sum(parts)
        elif wl.fp8 and "delayed" in wl.tags:
            oracle.mlp_shard_e4m3_delayed(Xq[rows], sX, Aq, sA, Bq, sB, np.float32(1.0))
        elif wl.fp8:
            oracle.mlp_shard_e4m3(Xq[rows], sX, Aq, sA, Bq, sB)
        else:
            parts = [oracle.mlp_shard(X[rows], A, B, wl.N, r) for r in range(wl.N)]
            if wl.N > 1:
                oracle.partial_sum(parts)
        t_total += time.perf_counter() - t0
        done = rows.stop
    flops = wl.N * (10 if wl.backward else 4) * done * wl.d * wl.F
    what = (f"rows [0, {done}) of {wl.M} of the {wl.name} step"
            + (f" (all {wl.N} ranks + partial sum)" if wl.N > 1 else "")
            + f", float64 numpy/OpenBLAS oracle, {t_total:.2f} s")
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": HOST_CORES,
            "kind": "oracle", "sample": what, "seconds": t_total}


def sampled_check(wl, inputs, out, nrows=8):
    import torch
    import oracle
    from workloads import sample_rows
    if hasattr(wl, "heads"):   # causal: a prefix of sequence 0 depends on nothing after it
        from oracle import attention as oat
        X, Wqkv, Wo = inputs
        T = min(wl.S, 256)
        rows = sample_rows(T, nrows)
        got = out[torch.from_numpy(rows).cuda()].double().cpu().numpy()
        ref = oat.attn_unsharded(X[:T], Wqkv, Wo, 1, T, wl.heads, wl.causal)[rows]
        if not wl.causal:
            return None
        return float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
    X, A, B = inputs[:3]
    rows = sample_rows(wl.M, nrows)
    got = out[torch.from_numpy(rows).cuda()].double().cpu().numpy()
    if wl.fp8 and not wl.backward:
        return None
    if wl.fp8:        # Σ_i dX_i against the unsharded bf16 input gradient: the fp8 error
        ref = oracle.mlp_shard_backward(X[rows], A, B, inputs[3][rows], 1, 0)["dX"]
    elif wl.backward:   # Σ_i dX_i is the unsharded block's input gradient
        ref = oracle.mlp_shard_backward(X[rows], A, B, inputs[3][rows], 1, 0)["dX"]
    elif wl.N > 1:
        ref = oracle.mlp_unsharded(X[rows], A, B)
    else:
        ref = oracle.mlp_shard(X[rows], A, B, 1, 0)
    return float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))


def library_compare(tpm, args):
    """The 7B-class column GEMM (X[8192x4096] · A_i[4096x2048], bf16) and row GEMM
    (Z[8192x2048] · B_i[2048x4096]) against the vendor library on the same data:
    tp_mlp_col_gelu (fused GeLU) and tp_mlp_row_partial (fp32 and bf16 partials) beside
    torch's GEMM with the weight N-contiguous (NN, the math layout) and K-contiguous (NT,
    stored transposed), bf16 output, and for the row GEMM also fp32 output where torch
    offers it (torch.mm with out_dtype). No library call has an activation. Prints one
    JSON line of HIP-event averages; a counter profile of this run compares the kernels'
    instruction mixes."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(0)
    out = {}
    for label, (M, K, N) in (("col", (8192, 4096, 2048)), ("row", (8192, 2048, 4096))):
        a = torch.randn(M, K, device="cuda", dtype=torch.bfloat16, generator=g)
        b = (torch.randn(K, N, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
        bt = b.t().contiguous().t()
        calls = {f"{label}_library_nt": lambda a=a, bt=bt: a @ bt,
                 f"{label}_library_nn": lambda a=a, b=b: a @ b}
        if label == "col":
            z = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
            calls["col_gelu"] = lambda a=a, b=b, z=z: tpm.tp_mlp_col_gelu(a, b, z)
        else:
            y32 = torch.empty(M, N, device="cuda", dtype=torch.float32)
            y16 = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
            calls["row_partial_f32"] = lambda a=a, b=b, y=y32: tpm.tp_mlp_row_partial(a, b, y)
            calls["row_partial_bf16"] = lambda a=a, b=b, y=y16: tpm.tp_mlp_row_partial(
                a, b, y, out_dtype=torch.bfloat16)
            try:
                torch.mm(a, b, out_dtype=torch.float32)
                calls["row_library_nn_f32"] = lambda a=a, b=b: torch.mm(a, b, out_dtype=torch.float32)
                calls["row_library_nt_f32"] = lambda a=a, bt=bt: torch.mm(a, bt, out_dtype=torch.float32)
            except (RuntimeError, NotImplementedError, TypeError) as e:
                log(f"library_compare: no fp32-output library GEMM ({type(e).__name__})")
        for _ in range(args.warmup):
            for fn in calls.values():
                fn()
        torch.cuda.synchronize()
        timer = KernelTimer()
        for _ in range(args.steps):
            torch.cuda._sleep(LEAD_CYCLES)
            for name, fn in calls.items():
                timer.around(name, fn)
        torch.cuda.synchronize()
        fl = 2 * M * N * K
        for k, v in timer.summary().items():
            out[k] = {"shape": [M, K, N], "avg_us": round(v["avg_us"], 2),
                      "tflops": round(fl / (v["avg_us"] * 1e-6) / 1e12, 1)}
    print(json.dumps({"workload": "library_compare", "kernels": out}), flush=True)


def copy_calibration(tpm, args):
    """Y = parts[0] over 64 Mi fp32 elements: 256 MiB read, 256 MiB written per launch."""
    import torch
    n = 64 << 20
    src = torch.arange(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        tpm.tp_partial_sum([src], Y=dst)
    torch.cuda.synchronize()
    timer = KernelTimer()
    for _ in range(args.steps):
        torch.cuda._sleep(LEAD_CYCLES)
        timer.around("copy", lambda: tpm.tp_partial_sum([src], Y=dst))
    torch.cuda.synchronize()
    st = timer.summary()["copy"]
    nbytes = 2 * n * 4
    print(json.dumps({"workload": "copy", "bytes_read": n * 4, "bytes_written": n * 4,
                      "avg_us": st["avg_us"], "GBps": nbytes / (st["avg_us"] * 1e-6) / 1e9}),
          flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the path; --gpus {args.gpus} is not "
              "supported (the N tensor-parallel ranks run one after another on one GPU).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import megatron_tensor_transformer_shard_amd as tpm
    from workloads import WORKLOADS
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.workload == "copy":
        copy_calibration(tpm, args)
        return
    if args.workload == "library_compare":
        library_compare(tpm, args)
        return
    from workloads import ATTN_WORKLOADS
    wl = WORKLOADS[args.workload] if args.workload in WORKLOADS else ATTN_WORKLOADS[args.workload]
    attn = args.workload in ATTN_WORKLOADS
    dtype = "e4m3" if getattr(wl, "fp8", False) else "bf16"
    log(f"bench: workload {wl.name}: {wl.description}")
    if attn:
        step, kern_flops, kern_bytes, psum_bytes, inputs, out = build_attn_step(tpm, wl)
    elif wl.backward:
        step, kern_flops, kern_bytes, psum_bytes, inputs, out = build_bwd_step(tpm, wl)
    elif wl.fp8:
        step, kern_flops, kern_bytes, psum_bytes, inputs, out = build_e4m3_step(tpm, wl)
    else:
        step, kern_flops, kern_bytes, psum_bytes, inputs, out = build_bf16_step(
            tpm, wl, args.partial_dtype, args.weight_layout)
    # only the bf16 forward takes --partial-dtype; every other step's partials are fixed
    pdt = args.partial_dtype if not (attn or wl.backward or wl.fp8) else PROFILED_PARTIAL_DTYPE
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"bench: warmup {args.warmup} steps done")

    # whole-step timing: exactly K steps between two synchronisations. By
    # default the launches of K steps are captured in one HIP graph, replayed
    # once untimed and once timed, so that neither the host's launch calls nor
    # a graph launch per step leaves gaps between kernels (every entry point
    # only enqueues kernels on the caller's stream, and every step here
    # replays to the eager bits: tests/test_gpu_graph.py); the same K steps
    # launched eagerly are timed beside it.
    graph = None
    if not args.eager:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(args.steps):
                step()
        graph.replay()
        torch.cuda.synchronize()

    def timed_steps(replay):
        t0 = time.perf_counter()
        if replay:
            graph.replay()
        else:
            for _ in range(args.steps):
                step()
        torch.cuda.synchronize()
        return 1e3 * (time.perf_counter() - t0) / max(1, args.steps)

    ms_eager = timed_steps(False)
    ms_per_step = timed_steps(True) if graph is not None else ms_eager
    flops_step = wl.N * wl.flops_per_shard()
    value = flops_step / (ms_per_step * 1e-3) / 1e12
    log(f"bench: {args.steps} steps, {ms_per_step:.3f} ms/step"
        f"{' (graph replay)' if graph is not None else ''}, {value:.1f} TFLOP/s; "
        f"eager launches {ms_eager:.3f} ms/step")

    # per-kernel timing with events on the launch stream (separate pass), with
    # the engine clock sampled meanwhile. Before each step a spin kernel of a
    # few milliseconds (outside every event pair) lets the host queue the
    # step's launches ahead of the GPU: an event pair around a launch that the
    # host has not yet queued would also time the host's delay.
    timer = KernelTimer()
    with ClockSampler() as clock:
        for _ in range(args.steps):
            torch.cuda._sleep(LEAD_CYCLES)
            step(timer)
        torch.cuda.synchronize()
    kstats = timer.summary()
    peak = PEAK_TFLOPS[dtype]
    for name, fl in kern_flops.items():
        kstats[name]["tflops"] = fl / (kstats[name]["avg_us"] * 1e-6) / 1e12
        kstats[name]["frac_of_peak"] = kstats[name]["tflops"] / peak
        kstats[name]["algorithmic_bytes"] = kern_bytes[name]
        kstats[name]["traffic"] = measured_traffic(wl.name, name, pdt)
    if "weight_amax" in kstats:   # reads the whole of A and B once per step
        wbytes = 2 * 2 * wl.d * wl.H
        kstats["weight_amax"]["GBps"] = wbytes / (kstats["weight_amax"]["avg_us"] * 1e-6) / 1e9
        kstats["weight_amax"]["algorithmic_bytes"] = wbytes
    if "partial_sum" in kstats:
        kstats["partial_sum"]["GBps"] = psum_bytes / (kstats["partial_sum"]["avg_us"] * 1e-6) / 1e9
        kstats["partial_sum"]["algorithmic_bytes"] = psum_bytes
        kstats["partial_sum"]["traffic"] = measured_traffic(wl.name, "partial_sum", pdt)
    dom = max(kern_flops, key=lambda k: kstats[k]["total_ms"])
    ach = kstats[dom]["tflops"]
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(ach / peak, 4),
                "traffic": measured_traffic(wl.name, dom, pdt),
                "flops_per_launch": kern_flops[dom], "algorithmic_bytes": kern_bytes[dom],
                "avg_launch_us": round(kstats[dom]["avg_us"], 2),
                "median_launch_us": round(kstats[dom]["median_us"], 2),
                "clock_ghz_in_kernel": None, "frac_at_measured_clock": None}

    # the shader clock inside the kernels, from the same kernels with clock
    # stamps (a separate pass, outside every timed region): the MFMA peak
    # scales with it, 4096 (bf16) or 8192 (fp8) flops per CU per clock
    clocks = None if args.no_clock else clock_pass(tpm, step)
    per_clk = 8192 if dtype == "e4m3" else 4096
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for name, c in (clocks or {}).items():
        peak_at = cus * per_clk * c["clock_ghz_median"] * 1e9 / 1e12
        c["peak_at_clock_tflops"] = round(peak_at, 1)
        if name in kstats:
            kstats[name]["clock_ghz_in_kernel"] = c["clock_ghz_median"]
            kstats[name]["frac_at_measured_clock"] = round(kstats[name]["tflops"] / peak_at, 4)
            kstats[name]["tflops_over_in_kernel_span"] = round(
                kern_flops[name] / (c["span_us_median"] * 1e-6) / 1e12, 1)
    if clocks and dom in clocks:
        roofline["clock_ghz_in_kernel"] = clocks[dom]["clock_ghz_median"]
        roofline["frac_at_measured_clock"] = kstats[dom]["frac_at_measured_clock"]

    # cold mode: the same launches, each after a 512 MiB write that evicts L2
    # and the Infinity Cache (a separate, shorter pass; context beside the
    # warm figures above, which are the primary ones)
    cold = None if args.no_cold else {}
    cold_timer = None if args.no_cold else ColdTimer()
    for _ in range(0 if args.no_cold else min(args.steps, 5)):
        torch.cuda._sleep(LEAD_CYCLES)
        step(cold_timer)
    torch.cuda.synchronize()
    for name, st in ({} if args.no_cold else cold_timer.summary()).items():
        c = {"launches": st["launches"], "avg_us": round(st["avg_us"], 2),
             "median_us": round(st["median_us"], 2), "min_us": round(st["min_us"], 2)}
        if name in kern_flops:
            c["tflops"] = round(kern_flops[name] / (st["median_us"] * 1e-6) / 1e12, 1)
        cold[name] = c
    del cold_timer

    check = sampled_check(wl, inputs, out)
    if hasattr(wl, "heads"):
        check_ref = "unsharded attention block, float64 oracle, sampled rows of a causal prefix"
    elif wl.fp8 and wl.backward:
        check_ref = ("unsharded bf16 input gradient, float64 oracle: the fp8 quantisation error "
                     "itself (parity with the fp8 oracle is a GPU test)")
    elif wl.backward:
        check_ref = "unsharded input gradient, float64 oracle"
    else:
        check_ref = "unsharded GeLU(X·A)·B, float64 oracle"
    props = torch.cuda.get_device_properties(0)
    device = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
              "cus": props.multi_processor_count}
    dp = device_peak(dtype)
    if dp is not None:
        device["clock_khz"] = dp["clock_khz"]
        device["clock_instruction_rate_khz"] = dp["clock_instruction_rate_khz"]
        device["wall_clock_rate_khz"] = dp["wall_clock_rate_khz"]
        device["peak_from_props_tflops"] = round(dp["peak_tflops"], 1)
    sclk = clock.summary()
    if sclk is not None:   # the driver's figure, not the shader clock itself (it reads lower)
        device["driver_reported_sclk_during_kernel_pass"] = sclk

    result = {
        "metric": (METRIC_ATTN if attn else METRIC_BWD if getattr(wl, "backward", False)
                   else METRIC),
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "step_timing": ("one HIP graph of all K steps, replayed" if graph is not None
                        else "eager launches"),
        "ms_per_step_eager_launches": round(ms_eager, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic: seeded X~N(0,1), weights~N(0,sigma^2), bf16 (no trained weights)",
        "config": ({"workload": wl.name, "B": wl.B, "S": wl.S, "d": wl.d, "heads": wl.heads,
                    "head_dim": wl.dh, "causal": wl.causal, "tp_ranks": wl.N,
                    "partial_dtype": "f32",
                    "parallelism": f"tp{wl.N} ranks sequentially on 1 GPU"} if attn else
                   {"workload": wl.name, "M": wl.M, "d": wl.d, "F": wl.F, "tp_ranks": wl.N,
                    "partial_dtype": "f32" if wl.backward else ("bf16" if wl.fp8
                                                                else args.partial_dtype),
                    "weight_layout": ("linear [out, in]" if args.weight_layout == "linear"
                                      and not (wl.backward or wl.fp8) else "math [in, out]"),
                    "parallelism": f"tp{wl.N} ranks sequentially on 1 GPU" if wl.N > 1 else "none"}),
        "pct_of_peak": round(100 * value / peak, 2),
        # one rank's shard (the event-timed averages of its flop-bearing launches
        # added) and the sum of the partials, once per step
        "per_rank_us": round(sum(kstats[k]["avg_us"] for k in kern_flops), 2),
        "partial_sum_us": round(kstats["partial_sum"]["avg_us"], 2) if "partial_sum" in kstats else None,
        "roofline": roofline,
        "kernels": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kstats.items()},
        "cold": cold,
        "check_max_err_ratio_8rows": check,
        "check_against": None if check is None else check_ref,
        "device": device,
        "clock_in_kernels": clocks,
    }
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(wl, inputs, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
