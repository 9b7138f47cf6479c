#!/usr/bin/env python3
"""Benchmark of the fp32 GEMM + GEMV hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one pass of the whole path on resident synthetic inputs:
  * GEMM  C = A B at the transformer-projection shape M = 8192 tokens, K = 4096,
    N = 14336 (A ~ N(0, 1), B ~ N(0, 1/K));
  * GEMV  y = A x for the fully-connected layer, 4096 inputs x 4096 outputs
    (A, x ~ U[-1, 1)).
W untimed steps, then K timed steps between two device synchronisations. The JSON
line's `value` is the step's FLOP rate (the GEMM is more than 99.9% of it); the
`gemm` and `gemv` objects give each kernel's own rate from HIP events recorded on
the launch stream around every launch in the timed region. After the timed steps
a burst of GEMV launches over 8 rotating 64 MiB matrices (more than the 256 MB
Infinity Cache) gives the GEMV's HBM rate. A clock phase follows (--clock-seconds,
default 2.5 s: the GEMM again, untimed, while amdsmi reports the graphics clock),
for the fp32 peak at the clock the kernel ran at. Results are then verified against the
CPU oracle (64+ sampled GEMM rows in full, every GEMV output) and the oracle's
own time on a bounded sample of the same work is reported as `cpu_baseline`.

Profiling helpers (same script, for rocprofv3 runs): --only gemm | gemv | copy | h16 |
conv | conv7x7 | split | gemm1024 | ragged | gemvt | narrow | h16_1024 | torch_gemm runs just that kernel `--steps` times with no oracle;
`copy` is a plain device-to-device copy of known size used to calibrate HBM counters;
`h16` is the bf16-input GEMM at the projection shape; `conv` the 3x3 convolution layer
(N=32, C=K=128, 28x28), `conv7x7` the 7x7 stride-2 first layer (N=32, C=3, 224x224, K=64); `split` the FC layer on a batch of 128 through both K splits;
`gemm1024` and `ragged` the fp32 GEMM at 1024^3 and 1000 x 1531 x 777; `gemvt` the
transposed GEMV with a workspace (row blocks, then the sum) on the GEMV workload's matrices;
`narrow` the FC layer on a batch of 64 (4096 x 64 x 4096) through mm_gemm_f32, A rotating
over 8 matrices; `h16_1024` the bf16-input GEMM at 1024^3; `torch_gemm` torch.mm (TF32 off)
on the GEMM workload's inputs, a reference point.

Sweeps (tables, not the benchmark line): --sweep conv times every convolution tile
configuration on the layer workloads; --sweep gemm times every GEMM tile
configuration on the workload shapes and a few others; --sweep gemv times the GEMV
at N = 4096 for growing M, which separates its per-launch fixed cost from its
streaming rate. Both time a run of back-to-back launches between two events on
the launch stream (for the GEMV this agrees with rocprofv3's kernel durations;
kernels much shorter than ~5 us are bounded by the host's launch rate instead).
--sweep lib times torch's library routines (torch.mm, torch.mv, conv2d) beside this
library's kernels on the same shapes; the benchmark line's `library_reference` does the
same for its own GEMM and GEMV.
"""
import argparse
import hashlib
import json
import statistics
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402
from tiled_gemm_gemv_amd import roofline as rl  # noqa: E402

METRIC = "fp32 GEMM TFLOP/s & % MFMA peak; GEMV GB/s & % HBM peak (1 MI355X)"
GEMV_SETS = 8
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
CSRC = os.path.join(ROOT, "tiled_gemm_gemv_amd", "csrc")
# the sources of each kernel whose HBM traffic profiles/hbm_traffic.txt records
GEMM_SRC = [os.path.join(CSRC, "mm_gemm.hip"), os.path.join(CSRC, "mm_gemm_tile.h"),
            os.path.join(CSRC, "mm_gemm_direct.hip"), os.path.join(CSRC, "mm_direct.h")]
GEMV_SRC = [os.path.join(CSRC, "mm_gemv.hip")]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_digest(paths):
    """First 16 hex digits of the sha256 of the files' bytes, concatenated in order."""
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic():
    """Per-dispatch HBM bytes measured with rocprofv3 counters, if they were taken on
    the current kernel sources (profiles/hbm_traffic.txt, `key: value` lines)."""
    if not os.path.exists(TRAFFIC_FILE):
        return {}
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.lstrip().startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    out = {}
    for kern, src in (("gemm", GEMM_SRC), ("gemv", GEMV_SRC)):
        if vals.get(f"{kern}_source_sha256") == source_digest(src):
            try:
                out[kern] = float(vals[f"{kern}_hbm_bytes_per_dispatch"])
            except (KeyError, ValueError):
                pass
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


# A GPU host shares its cores among its GPUs; one GPU's share is 16 threads, whatever
# the affinity mask of the process shows. The oracle runs on the smaller of the two, and
# the bench line states both.
HOST_SHARE = 16


def affinity_cpus():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def host_threads():
    return max(1, min(affinity_cpus(), HOST_SHARE))


class ClockProbe:
    """Graphics clock of the benchmark GPU as its power-management firmware reports
    it (amdsmi GPU metrics: the current clock of each XCD, averaged over the XCDs).
    The matrix peaks (157.3 TFLOP/s fp32, 2.5 PFLOP/s 16-bit) are quoted at 2.4 GHz and
    scale with the clock, so the clock seen while a kernel runs gives the peak at that
    clock. Reading it is optional: without the amdsmi module or a matching device the
    probe reports why."""

    def __init__(self, torch, dev):
        self.handle, self.why, self.samples, self.inited = None, None, [], False
        try:
            import amdsmi
        except ImportError as e:
            self.why = f"amdsmi not importable ({e})"
            return
        self.amdsmi = amdsmi
        try:
            amdsmi.amdsmi_init()
            self.inited = True
            p = torch.cuda.get_device_properties(dev)
            want = f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}."
            for h in amdsmi.amdsmi_get_processor_handles():
                if amdsmi.amdsmi_get_gpu_device_bdf(h).lower().startswith(want):
                    self.handle = h
            if self.handle is None:
                self.why = f"no amdsmi device at PCI {want}"
            elif self.read() is None:
                self.handle, self.why = None, "GPU metrics carry no graphics clock"
        except Exception as e:  # noqa: BLE001 - any amdsmi failure only drops the clock
            self.handle, self.why = None, "amdsmi: " + " ".join(str(e).split())

    def read(self):
        """Current graphics clock in MHz (mean over the XCDs that report one), or None."""
        m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.handle)
        per_xcd = m.get("current_gfxclks")
        if isinstance(per_xcd, list):
            vals = [v for v in per_xcd if isinstance(v, (int, float)) and v > 0]
            if vals:
                return float(np.mean(vals))
        v = m.get("current_gfxclk")
        return float(v) if isinstance(v, (int, float)) and v > 0 else None

    def measure(self, torch, stream, launch, seconds, launch_s):
        """Run `launch` back to back for about `seconds` and sample the clock every
        20 ms meanwhile. The firmware's metrics are cached by the driver for a few
        hundred milliseconds (an idle reading was still returned 0.3 s into a
        sustained load), so only samples from the second half of the run are kept:
        by then every reading was taken while the kernel was running."""
        if self.handle is None or seconds <= 0:
            return
        n = max(1, min(2000, int(np.ceil(seconds / max(launch_s, 1e-6)))))
        done = torch.cuda.Event()
        t0 = time.perf_counter()
        for _ in range(n):
            launch()
        done.record(stream)
        timed = []
        while not done.query():
            v = self.read()
            if v is not None:
                timed.append((time.perf_counter() - t0, v))
            time.sleep(0.02)
        total = time.perf_counter() - t0
        self.seconds = total
        self.samples = [v for t, v in timed if t >= total / 2]

    def summary(self, tflops, peak_tflops_at_max):
        """The clock readings and the peak they imply; with a measured rate `tflops`
        (None: no rate was timed), also that rate's share of the peak at this clock."""
        if not self.samples:
            return {"gfxclk_mhz": None, "why": self.why or "no sample taken"}
        f = float(np.median(self.samples))
        peak = peak_tflops_at_max * (f * 1e6 / rl.MI355X_PEAK_SCLK_HZ)
        out = {"gfxclk_mhz": round(f, 1), "gfxclk_mhz_min": round(min(self.samples), 1),
               "gfxclk_mhz_max": round(max(self.samples), 1), "samples": len(self.samples),
               "source": f"amdsmi GPU metrics (current clock of each XCD, averaged), sampled "
                         f"in the second half of {self.seconds:.1f} s of the same kernel run "
                         f"back to back after the timed steps",
               "peak_at_clock": round(peak, 2)}
        if tflops is not None:
            out["frac_at_clock"] = round(tflops / peak, 4)
        return out

    def close(self):
        if self.inited:
            self.inited = False
            try:
                self.amdsmi.amdsmi_shut_down()
            except Exception:  # noqa: BLE001
                pass


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--gemv-reps", type=int, default=400)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target length of the oracle's timed sample")
    ap.add_argument("--only", choices=["gemm", "gemv", "copy", "h16", "conv", "split", "gemm1024", "ragged",
                                           "gemvt", "narrow", "h16_1024", "conv7x7", "torch_gemm"],
                    default=None,
                    help="profiling helper: launch only this kernel --steps times")
    ap.add_argument("--clock-seconds", type=float, default=None,
                    help="length of the clock phase (default 2.5 s after the timed steps; "
                         "with --only h16 none unless given; 0: no clock reading)")
    ap.add_argument("--sweep", choices=["gemm", "gemv", "h16", "conv", "lib"], default=None,
                    help="print a timing table instead of the benchmark line")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported. "
              "Across GPUs the GEMM would split B and C by columns (A replicated) and the GEMV "
              "A by rows (x broadcast), with no exchange of results.", file=sys.stderr)
        sys.exit(2)

    import torch
    import tiled_gemm_gemv_amd as mm

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    mm.load()
    stream = torch.cuda.current_stream()

    if args.sweep:
        sweep(args.sweep, torch, mm, dev)
        return

    wg = wl.WORKLOADS["gemm_proj"]
    wv = wl.WORKLOADS["gemv4096"]
    M, N, K = wg.M, wg.N, wg.K
    VM, VN = wv.M, wv.N

    if args.only == "copy":
        # plain copy of 256 MiB: reads and writes 268,435,456 bytes per launch
        src = torch.empty(64 << 20, dtype=torch.float32, device=dev).uniform_()
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy: {args.steps} x {src.numel() * 4} bytes")
        return

    if args.only == "h16":
        # bf16 inputs at the projection shape (values from the same distributions)
        A16 = (torch.randn(M, K, device=dev)).to(torch.bfloat16)
        B16 = (torch.randn(K, N, device=dev) / 64.0).to(torch.bfloat16)
        C = torch.empty((M, N), dtype=torch.float32, device=dev)
        for _ in range(args.steps):
            mm.mm_gemm_bf16(M, N, K, A16, K, B16, N, C, N, stream)
        torch.cuda.synchronize()
        log(f"h16: {args.steps} bf16 launches")
        if args.clock_seconds:
            clock = ClockProbe(torch, dev)
            clock.measure(torch, stream, lambda: mm.mm_gemm_bf16(M, N, K, A16, K, B16, N, C, N, stream),
                          args.clock_seconds, 1e-3)
            torch.cuda.synchronize()
            c = clock.summary(None, rl.MI355X_16BIT_MFMA_PEAK / 1e12)  # no rate timed here
            clock.close()
            log(f"h16 clock: {json.dumps(c)}")
        return

    if args.only == "h16_1024":
        # bf16 inputs at 1024^3 (A ~ U[-1, 1), B ~ U[-1, 1)), in the configuration
        # mm_gemm_bf16 chooses
        S = 1024
        A16 = (torch.rand(S, S, device=dev) * 2 - 1).to(torch.bfloat16)
        B16 = (torch.rand(S, S, device=dev) * 2 - 1).to(torch.bfloat16)
        C = torch.empty((S, S), dtype=torch.float32, device=dev)
        for _ in range(args.steps):
            mm.mm_gemm_bf16(S, S, S, A16, S, B16, S, C, S, stream)
        torch.cuda.synchronize()
        log(f"h16_1024: {args.steps} bf16 launches at {S}^3, config "
            f"{mm.mm_gemm_h16_config_name(mm.mm_gemm_h16_select(S, S, S))}")
        return

    if args.only == "split":
        # the fully-connected layer on a batch of 128 (4096 x 128 x 4096): mm_gemm_f32 (two K
        # halves added into a zeroed C) and mm_gemm_f32_ws (4 chunks, then the sum)
        SM, SN, SK = 4096, 128, 4096
        A = torch.randn(SM, SK, device=dev)
        B = torch.randn(SK, SN, device=dev) / 64.0
        C = torch.empty((SM, SN), dtype=torch.float32, device=dev)
        ws = mm.gemm_workspace(SM, SN, SK, dev)
        for _ in range(args.steps):
            mm.mm_gemm_f32(SM, SN, SK, A, SK, B, SN, C, SN, stream)
        for _ in range(args.steps):
            mm.mm_gemm_f32_ws(SM, SN, SK, A, SK, B, SN, C, SN, ws, ws.numel(), stream)
        torch.cuda.synchronize()
        log(f"split: {args.steps} mm_gemm_f32 and {args.steps} mm_gemm_f32_ws calls at {SM}x{SN}x{SK}")
        return

    if args.only == "narrow":
        # the fully-connected layer on a batch of 64 (4096 x 64 x 4096) through mm_gemm_f32
        # (narrow C), A rotating over 8 matrices so that every call reads its A from HBM
        SM, SN, SK = 4096, 64, 4096
        As = [torch.randn(SM, SK, device=dev) for _ in range(GEMV_SETS)]
        B = torch.randn(SK, SN, device=dev) / 64.0
        C = torch.empty((SM, SN), dtype=torch.float32, device=dev)
        for i in range(args.steps):
            mm.mm_gemm_f32(SM, SN, SK, As[i % GEMV_SETS], SK, B, SN, C, SN, stream)
        torch.cuda.synchronize()
        log(f"narrow: {args.steps} mm_gemm_f32 calls at {SM}x{SN}x{SK}, config "
            f"{mm.mm_gemm_f32_config_name(mm.mm_gemm_f32_select(SM, SN, SK))}")
        return

    if args.only in ("gemm1024", "ragged"):
        # the report-only GEMM workloads, in the configuration mm_gemm_f32 chooses
        w = wl.WORKLOADS["gemm1024" if args.only == "gemm1024" else "gemm_ragged"]
        Ah, Bh = wl.gemm_inputs(w)
        A = torch.from_numpy(Ah).to(dev)
        B = torch.from_numpy(Bh).to(dev)
        C = torch.empty((w.M, w.N), dtype=torch.float32, device=dev)
        for _ in range(args.steps):
            mm.mm_gemm_f32(w.M, w.N, w.K, A, w.K, B, w.N, C, w.N, stream)
        torch.cuda.synchronize()
        log(f"{args.only}: {args.steps} launches of {w.describe()}, config "
            f"{mm.mm_gemm_f32_config_name(mm.mm_gemm_f32_select(w.M, w.N, w.K))}")
        return

    if args.only in ("conv", "conv7x7"):
        # the 3x3 middle layer (or the 7x7 stride-2 first layer), in the configuration
        # mm_conv2d_f32 chooses
        cw = wl.CONV_WORKLOADS["conv3x3" if args.only == "conv" else "conv7x7_s2"]
        x, f, y = conv_tensors(torch, cw, dev)
        for _ in range(args.steps):
            launch_conv(mm, cw, x, f, y, stream)
        torch.cuda.synchronize()
        log(f"conv: {args.steps} launches of {cw.describe()}")
        return

    log(f"generating inputs: {wg.describe()}, {wv.describe()}")
    A_h, B_h = wl.gemm_inputs(wg)
    Av_h, xv_h = wl.gemv_inputs(wv)
    A = torch.from_numpy(A_h).to(dev)
    B = torch.from_numpy(B_h).to(dev)
    C = torch.empty((M, N), dtype=torch.float32, device=dev)
    # GEMV sets: set 0 holds the workload's inputs, sets 1..7 the same values moved
    # to other addresses (so every launch reads its matrix from HBM).
    Avs = [torch.from_numpy(Av_h).to(dev) for _ in range(GEMV_SETS)]
    xvs = [torch.from_numpy(xv_h).to(dev) for _ in range(GEMV_SETS)]
    yvs = [torch.empty(VM, dtype=torch.float32, device=dev) for _ in range(GEMV_SETS)]
    torch.cuda.synchronize()

    def gemm():
        mm.mm_gemm_f32(M, N, K, A, K, B, N, C, N, stream)

    def gemv(i):
        mm.mm_gemv_f32(VM, VN, Avs[i], xvs[i], yvs[i], stream)

    if args.only == "gemm":
        for _ in range(args.steps):
            gemm()
        torch.cuda.synchronize()
        log(f"gemm: {args.steps} launches")
        return
    if args.only == "torch_gemm":
        # torch's own fp32 GEMM (rocBLAS / hipBLASLt) on the same resident inputs: a
        # reference point for profiles, not part of the path
        torch.backends.cuda.matmul.allow_tf32 = False
        for _ in range(args.steps):
            torch.mm(A, B, out=C)
        torch.cuda.synchronize()
        log(f"torch_gemm: {args.steps} launches")
        return
    if args.only == "gemv":
        for i in range(args.steps):
            gemv(i % GEMV_SETS)
        torch.cuda.synchronize()
        log(f"gemv: {args.steps} launches")
        return
    if args.only == "gemvt":
        # y = A^T x over the same rotating matrices (x has VM entries, y VN)
        nbytes = mm.mm_gemv_t_f32_workspace_bytes(VM, VN)
        ws = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=dev)
        xt = torch.randn(VM, device=dev)
        yt = torch.empty(VN, device=dev)
        for i in range(args.steps):
            mm.mm_gemv_t_f32_ws(VM, VN, Avs[i % GEMV_SETS], xt, yt, ws, nbytes, stream)
        torch.cuda.synchronize()
        log(f"gemvt: {args.steps} launches of {VM} x {VN}, workspace {nbytes} bytes")
        return

    clock = ClockProbe(torch, dev)

    # ---------------------------------------------------------------- warm-up
    log(f"warm-up: {args.warmup} steps")
    for s in range(args.warmup):
        gemm()
        gemv(s % GEMV_SETS)
    torch.cuda.synchronize()

    # ------------------------------------------------------------- timed steps
    steps = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    log(f"timed: {steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        ev[s][0].record(stream)
        gemm()
        ev[s][1].record(stream)
        gemv(0)
        ev[s][2].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    gemm_ms = [ev[s][0].elapsed_time(ev[s][1]) for s in range(steps)]
    gemv_step_ms = [ev[s][1].elapsed_time(ev[s][2]) for s in range(steps)]

    # ------------------------------------------------- GEMV burst, rotating sets
    # Back-to-back launches between two events: the average includes the short
    # gaps between dispatches but no event overhead per launch.
    reps = args.gemv_reps
    b0 = torch.cuda.Event(enable_timing=True)
    b1 = torch.cuda.Event(enable_timing=True)
    for i in range(GEMV_SETS):
        gemv(i)
    torch.cuda.synchronize()
    b0.record(stream)
    for i in range(reps):
        gemv(i % GEMV_SETS)
    b1.record(stream)
    torch.cuda.synchronize()
    burst_ms = b0.elapsed_time(b1) / reps

    # --------------------------------------------------------------- accounting
    gemm_flop = rl.gemm_flops(M, N, K)
    gemv_flop = rl.gemv_flops(VM, VN)
    gemm_avg_s = float(np.mean(gemm_ms)) / 1e3
    gemm_tflops = gemm_flop / gemm_avg_s / 1e12
    gemv_bytes = rl.gemv_algorithmic_bytes(VM, VN)
    gemv_gbs = gemv_bytes / (burst_ms / 1e3) / 1e9
    step_tflops = steps * (gemm_flop + gemv_flop) / elapsed / 1e12
    traffic = read_traffic()

    # ------------------- clock phase: the same GEMM again, untimed, clock sampled
    clock.measure(torch, stream, gemm, 2.5 if args.clock_seconds is None else args.clock_seconds,
                  gemm_avg_s)
    torch.cuda.synchronize()

    # ---- library reference: torch's own GEMM (rocBLAS / hipBLASLt, TF32 off) and GEMV on
    # the same resident inputs, timed the same way, into separate outputs (C and y are
    # verified below as this library computed them). A reference point, not the path.
    torch.backends.cuda.matmul.allow_tf32 = False
    Ct = torch.empty_like(C)
    yts = [torch.empty_like(y) for y in yvs]
    lib_reps = min(10, max(2, steps))
    for _ in range(2):
        torch.mm(A, B, out=Ct)
    for i in range(GEMV_SETS):
        torch.mv(Avs[i], xvs[i], out=yts[i])
    torch.cuda.synchronize()
    l0, l1, l2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    l0.record(stream)
    for _ in range(lib_reps):
        torch.mm(A, B, out=Ct)
    l1.record(stream)
    for i in range(reps):
        torch.mv(Avs[i % GEMV_SETS], xvs[i % GEMV_SETS], out=yts[i % GEMV_SETS])
    l2.record(stream)
    torch.cuda.synchronize()
    lib_gemm_tflops = gemm_flop / (l0.elapsed_time(l1) / lib_reps / 1e3) / 1e12
    lib_gemv_gbs = gemv_bytes / (l1.elapsed_time(l2) / reps / 1e3) / 1e9
    del Ct, yts

    # ------------------------------------------- verification + CPU baseline leg
    import oracle
    from oracle import verify

    threads = host_threads()
    rows64 = wl.sample_rows(wg, 64)
    tc = time.perf_counter()
    C64, S64 = oracle.gemm(A_h, B_h, rows=rows64, threads=threads)
    t64 = time.perf_counter() - tc
    rows = rows64
    n_more = int(64 * args.cpu_seconds / max(t64, 1e-3)) if t64 > 0 else 64
    n_more = max(64, min(n_more, M))
    if n_more > 64:
        rows = wl.sample_rows(wg, n_more)
        log(f"oracle: timing {len(rows)} rows of the projection on {threads} threads")
        tc = time.perf_counter()
        C64, S64 = oracle.gemm(A_h, B_h, rows=rows, threads=threads)
        t_cpu = time.perf_counter() - tc
    else:
        t_cpu = t64
    got = C[torch.from_numpy(rows).to(dev)].cpu().numpy()
    gemm_check = verify.within_tol(got, C64, S64, 1e-5)
    tv = time.perf_counter()
    y64, s64 = oracle.gemv(Av_h, xv_h, threads=threads)
    tv = time.perf_counter() - tv
    gemv_ok = True
    for i in range(GEMV_SETS):
        r = verify.within_tol(yvs[i].cpu().numpy(), y64, s64, 1e-5)
        gemv_ok = gemv_ok and bool(r)
    cpu_tflops = rl.gemm_flops(len(rows), N, K) / t_cpu / 1e12
    # the oracle on one thread: the small GEMM (128^3, best of 5) and the full GEMV
    w1 = wl.WORKLOADS["gemm128"]
    A1, B1 = wl.gemm_inputs(w1)
    t1g = []
    for _ in range(5):
        tc = time.perf_counter()
        oracle.gemm(A1, B1, threads=1)
        t1g.append(time.perf_counter() - tc)
    tc = time.perf_counter()
    oracle.gemv(Av_h, xv_h, threads=1)
    t1v = time.perf_counter() - tc

    result = {
        "metric": METRIC,
        "value": round(step_tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "fp32 GEMM M=8192 K=4096 N=14336 (A~N(0,1), B~N(0,1/K)) + fp32 GEMV "
                        "4096x4096 (U[-1,1)) per step",
            "gemm_config": mm.mm_gemm_f32_config_name(mm.mm_gemm_f32_select(M, N, K)),
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(gemm_tflops, 3),
            "peak": rl.MI355X_FP32_MFMA_PEAK / 1e12,
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops / (rl.MI355X_FP32_MFMA_PEAK / 1e12), 4),
            "traffic": traffic.get("gemm"),
        },
        "gemm": {
            "kernel_ms_mean": round(float(np.mean(gemm_ms)), 4),
            "kernel_ms_min": round(float(np.min(gemm_ms)), 4),
            "kernel_ms_median": round(float(np.median(gemm_ms)), 4),
            "tflops": round(gemm_tflops, 3),
            "frac_fp32_mfma_peak": round(gemm_tflops / (rl.MI355X_FP32_MFMA_PEAK / 1e12), 4),
            "algorithmic_bytes": rl.gemm_algorithmic_bytes(M, N, K),
            "verified_rows": int(len(rows)),
            "verify": str(gemm_check),
            "clock": clock.summary(gemm_tflops, rl.MI355X_FP32_MFMA_PEAK / 1e12),
        },
        "gemv": {
            "value": round(gemv_gbs, 1),
            "unit": "GB/s",
            "kernel_us_burst_mean": round(burst_ms * 1e3, 3),
            "us_in_step_with_events": round(float(np.mean(gemv_step_ms)) * 1e3, 3),
            "rotating_sets": GEMV_SETS,
            "roofline": {
                "bound": "hbm",
                "achieved": round(gemv_gbs, 1),
                "peak": rl.MI355X_HBM_PEAK / 1e9,
                "unit": "GB/s",
                "frac": round(gemv_gbs / (rl.MI355X_HBM_PEAK / 1e9), 4),
                "traffic": traffic.get("gemv"),
            },
            "verified": gemv_ok,
            "cpu_baseline": {
                "value": round(gemv_bytes / tv / 1e9, 3), "unit": "GB/s", "cores": threads,
                "kind": "oracle", "sample": "the full 4096x4096 GEMV, fp64 accumulation"},
        },
        "cpu_baseline": {
            "value": round(cpu_tflops, 5),
            "unit": "TFLOP/s",
            "cores": threads,
            "affinity_cpus": affinity_cpus(),
            "threads_rule": f"min(len(os.sched_getaffinity(0)), {HOST_SHARE}): the host's per-GPU share",
            "kind": "oracle",
            "sample": f"{len(rows)} sampled rows (all 14336 columns, K=4096) of the projection "
                      f"GEMM, fp64 accumulation, {t_cpu:.2f} s on {cpu_model()}",
            "full_matrix_s_extrapolated": round(t_cpu * M / len(rows), 1),
        },
        "library_reference": {
            "gemm": {"value": round(lib_gemm_tflops, 3), "unit": "TFLOP/s",
                     "this_over_library": round(gemm_tflops / lib_gemm_tflops, 4),
                     "how": f"torch.mm (TF32 off) on the same A and B, {lib_reps} launches between two events"},
            "gemv": {"value": round(lib_gemv_gbs, 1), "unit": "GB/s",
                     "this_over_library": round(gemv_gbs / lib_gemv_gbs, 4),
                     "how": f"torch.mv over the same {GEMV_SETS} rotating matrices, {reps} launches between two events"},
            "note": "torch's own routines on this GPU, as a reference point; not part of the path"},
        "cpu_single_thread": {
            "gemm128": {"value": round(rl.gemm_flops(128, 128, 128) / min(t1g) / 1e9, 3), "unit": "GFLOP/s",
                        "ms": round(min(t1g) * 1e3, 3)},
            "gemv4096": {"value": round(gemv_bytes / t1v / 1e9, 3), "unit": "GB/s", "ms": round(t1v * 1e3, 3)},
            "kind": "oracle", "cores": 1,
        },
        "verified": bool(gemm_check) and gemv_ok,
    }
    clock.close()
    print(json.dumps(result), flush=True)
    if not result["verified"]:
        log(f"VERIFICATION FAILED: gemm {gemm_check}; gemv ok={gemv_ok}")
        sys.exit(1)


def burst_time_ms(torch, launch, reps):
    """Average time per launch over `reps` back-to-back launches on the current
    stream, between two events, after one untimed pass."""
    stream = torch.cuda.current_stream()
    for i in range(reps):
        launch(i, stream)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps):
        launch(i, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def median_graph_ms(torch, launch, reps, runs=3):
    """Median over `runs` graph-replayed timings (graph_time_ms) of the same launches."""
    return statistics.median(graph_time_ms(torch, launch, reps) for _ in range(runs))


def graph_time_ms(torch, launch, reps):
    """Average time per launch over `reps` launches captured in one HIP graph and replayed
    between two events: the kernels' own time on the GPU, without the host's launch rate
    (which bounds back-to-back launches from Python at about 4 us each)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(2):
            launch(i, s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(reps):
            launch(i, s)
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    cur = torch.cuda.current_stream()
    e0.record(cur)
    g.replay()
    e1.record(cur)
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / reps


def conv_tensors(torch, cw, dev):
    """Device x, filters, y for a convolution workload (values from its distributions)."""
    x_h, f_h = wl.conv_inputs(cw)
    P, Q = cw.out_hw()
    x = torch.from_numpy(x_h).to(dev)
    f = torch.from_numpy(f_h).to(dev)
    y = torch.empty((cw.N, cw.K, P, Q), dtype=torch.float32, device=dev)
    return x, f, y


def launch_conv(mm, cw, x, f, y, stream, cfg=None):
    geo = cw.geometry()
    if cfg is None:
        mm.mm_conv2d_f32(*geo, x, f, y, stream)
    else:
        mm.mm_conv2d_f32_config(cfg, *geo, x, f, y, stream)


def sweep_conv(torch, mm, dev):
    nc = mm.mm_conv2d_f32_num_configs()
    peak = rl.MI355X_FP32_MFMA_PEAK
    print("# fp32 convolution (implicit GEMM), TFLOP/s per tile configuration (launches captured "
          "in a HIP graph and replayed between two events, median of 3 replays)")
    for c in range(nc):
        print(f"#   cfg {c}: {mm.mm_conv2d_f32_config_name(c)}")
    print("#   default = mm_conv2d_f32's own choice (* marks it among the configs; 1x1 layers on "
          "large maps run the batched GEMM with that tile)")
    print("#   dense = mm_gemm_f32 on the same M x N x K with the im2col matrix already in "
          "memory (what the gather costs, not counting writing that matrix)")
    print("#   bound = min(fp32 MFMA peak, algorithmic FLOP/byte x 8 TB/s); % = default / bound")
    print(f"{'workload':>12s} {'GEMM M':>7s} {'GEMM N':>8s} {'GEMM K':>7s} {'GFLOP':>7s}  " +
          " ".join(f"{'cfg' + str(c):>7s}" for c in range(nc)) +
          f" {'default':>8s} {'dense':>7s} {'bound':>7s} {'%':>6s}")
    for cw in wl.CONV_WORKLOADS.values():
        x, f, y = conv_tensors(torch, cw, dev)
        P, Q = cw.out_hw()
        flop = rl.conv_flops(cw.N, cw.C, cw.K, cw.R, cw.S, P, Q)
        by = rl.conv_algorithmic_bytes(cw.N, cw.C, cw.H, cw.W, cw.K, cw.R, cw.S, P, Q)
        bound = min(peak, flop / by * rl.MI355X_HBM_PEAK)
        reps = max(3, min(200, int(2e11 / flop)))
        sel = mm.mm_conv2d_f32_select(*cw.geometry())
        cells = []
        for c in range(nc):
            def launch(i, st, c=c):
                launch_conv(mm, cw, x, f, y, st, c)
            tf = flop / median_graph_ms(torch, launch, reps) / 1e9
            cells.append(f"{tf:6.1f}" + ("*" if c == sel else " "))

        def launch_default(i, st):
            launch_conv(mm, cw, x, f, y, st)
        td = flop / median_graph_ms(torch, launch_default, reps) / 1e9
        del x, y
        GM, GN, GK = cw.K, cw.N * P * Q, cw.C * cw.R * cw.S
        Bd = torch.randn(GK, GN, device=dev)
        Cd = torch.empty(GM, GN, device=dev)

        def launch_dense(i, st):
            mm.mm_gemm_f32(GM, GN, GK, f, GK, Bd, GN, Cd, GN, st)
        tdense = flop / median_graph_ms(torch, launch_dense, reps) / 1e9
        print(f"{cw.name:>12s} {GM:7d} {GN:8d} {GK:7d} "
              f"{flop / 1e9:7.2f}  " + " ".join(cells) +
              f" {td:8.1f} {tdense:7.1f} {bound / 1e12:7.1f} {100 * td * 1e12 / bound:6.1f}",
              flush=True)
        del f, Bd, Cd


def sweep_lib(torch, mm, dev):
    """The framework's own library routines on the same shapes and timing: rocBLAS /
    hipBLASLt behind torch.mm and torch.mv, MIOpen behind conv2d. A reference point for
    each kernel, not part of the path."""
    torch.backends.cuda.matmul.allow_tf32 = False
    torch.backends.cudnn.allow_tf32 = False
    print("# this library's kernels against torch's library routines on the same shapes (MI355X, "
          "one GPU); GEMMs: launches captured in a HIP graph and replayed between two events, "
          "median of 3 replays; GEMV: back-to-back launches rotating over >= 512 MiB of matrices "
          "(cold); convolution: back-to-back launches")
    print("#   fp32 GEMM: torch.mm with TF32 off; 16-bit GEMM: torch.mm writes a bf16 C, "
          "mm_gemm_bf16 an fp32 C; transposed GEMV: torch.mv on A.t()")
    print(f"{'op':>22s} {'shape':>22s} {'this library':>14s} {'torch':>14s} {'ratio':>6s}")

    def row(op, shape, ours, lib, unit):
        print(f"{op:>22s} {shape:>22s} {ours:9.1f} {unit:>4s} {lib:9.1f} {unit:>4s} "
              f"{ours / lib:6.2f}", flush=True)
    for dt, name in ((torch.float32, "fp32 GEMM"), (torch.bfloat16, "bf16 GEMM")):
        shapes = ([(8192, 14336, 4096), (8192, 4096, 14336), (4096, 4096, 4096), (2048, 2048, 2048),
                   (1024, 1024, 1024), (1000, 1531, 777), (4096, 64, 4096), (4096, 32, 4096),
                   (4096, 16, 4096)] if dt == torch.float32 else
                  [(8192, 14336, 4096), (4096, 4096, 4096), (1024, 1024, 1024), (1000, 1531, 777)])
        for M, N, K in shapes:
            A = torch.randn(M, K, device=dev).to(dt)
            B = (torch.randn(K, N, device=dev) / K ** 0.5).to(dt)
            C = torch.empty(M, N, device=dev)
            Ct = torch.empty(M, N, device=dev, dtype=dt)
            flop = rl.gemm_flops(M, N, K)
            reps = max(3, min(200, int((2e11 if dt == torch.float32 else 2e12) / flop)))
            if dt == torch.float32:
                def ours(i, st):
                    mm.mm_gemm_f32(M, N, K, A, K, B, N, C, N, st)
            else:
                def ours(i, st):
                    mm.mm_gemm_bf16(M, N, K, A, K, B, N, C, N, st)

            def lib(i, st):
                torch.mm(A, B, out=Ct)
            t_ours = flop / median_graph_ms(torch, ours, reps) / 1e9
            t_lib = flop / median_graph_ms(torch, lib, reps) / 1e9
            row(name, f"{M}x{N}x{K}", t_ours, t_lib, "TF/s")
            del A, B, C, Ct
    for TM, TN, trans in ((4096, 4096, False), (8192, 8192, False), (4096, 4096, True),
                          (8192, 8192, True), (4096, 16384, True)):
        sets = max(2, min(16, (512 << 20) // (TM * TN * 4)))
        As = [torch.rand(TM, TN, device=dev) for _ in range(sets)]
        xs = [torch.rand(TM if trans else TN, device=dev) for _ in range(sets)]
        ys = [torch.empty(TN if trans else TM, device=dev) for _ in range(sets)]
        if trans:
            def ours(i, st):
                k = i % sets
                mm.mm_gemv_t_f32(TM, TN, As[k], xs[k], ys[k], st)

            def lib(i, st):
                k = i % sets
                torch.mv(As[k].t(), xs[k], out=ys[k])
        else:
            def ours(i, st):
                k = i % sets
                mm.mm_gemv_f32(TM, TN, As[k], xs[k], ys[k], st)

            def lib(i, st):
                k = i % sets
                torch.mv(As[k], xs[k], out=ys[k])
        by = rl.FP32 * (TM * TN + TM + TN)
        t_ours = by / burst_time_ms(torch, ours, 8 * sets) / 1e6
        t_lib = by / burst_time_ms(torch, lib, 8 * sets) / 1e6
        row("transposed GEMV" if trans else "GEMV", f"{TM}x{TN}", t_ours, t_lib, "GB/s")
        del As, xs, ys
    for cw in wl.CONV_WORKLOADS.values():
        x, f, y = conv_tensors(torch, cw, dev)
        P, Q = cw.out_hw()
        flop = rl.conv_flops(cw.N, cw.C, cw.K, cw.R, cw.S, P, Q)

        def ours(i, st):
            launch_conv(mm, cw, x, f, y, st)

        def lib(i, st):
            torch.nn.functional.conv2d(x, f, stride=cw.stride, padding=cw.pad, dilation=cw.dilation)
        reps = max(3, min(100, int(2e11 / flop)))
        t_ours = flop / burst_time_ms(torch, ours, reps) / 1e9
        t_lib = flop / burst_time_ms(torch, lib, reps) / 1e9
        row("fp32 convolution", cw.name, t_ours, t_lib, "TF/s")
        del x, f, y


def sweep(kind, torch, mm, dev):
    if kind == "lib":
        sweep_lib(torch, mm, dev)
    elif kind == "conv":
        sweep_conv(torch, mm, dev)
    elif kind == "gemm":
        shapes = [(w.M, w.N, w.K, w.name) for w in wl.WORKLOADS.values() if w.op == "gemm"]
        shapes += [(1000, 1532, 784, "ragged M, aligned rows (N, K multiples of 4 and 16)"),
                   (512, 512, 512, ""), (1536, 1536, 1536, ""), (2048, 2048, 2048, ""),
                   (3072, 3072, 3072, ""), (4096, 4096, 4096, ""), (1024, 4096, 4096, ""),
                   (8192, 1792, 4096, "projection, 1/8 of N"),
                   (4096, 128, 4096, "128 tiles of 64 x 64: K in two halves"),
                   (1024, 512, 8192, "K in two halves"), (2048, 512, 8192, "K in two halves")]
        shapes += [(4096, n, 4096, f"FC layer 4096x4096, batch of {n}") for n in (1, 2, 4, 8, 16, 32, 64)]
        nc = mm.mm_gemm_f32_num_configs()
        print("# fp32 GEMM, TFLOP/s per tile configuration (launches captured in a HIP graph and "
              "replayed between two events, median of 3 replays; inputs N(0,1))")
        for c in range(nc):
            print(f"#   cfg {c}: {mm.mm_gemm_f32_config_name(c)}")
        print("#   * = the configuration mm_gemm_f32 selects for the shape; default = mm_gemm_f32 itself "
              "(differs from the starred column where it runs K as two halves); cold (FC layer rows "
              "only) = mm_gemm_f32 with A rotating over 8 copies, so that each call reads A from HBM")
        print(f"{'M':>6s} {'N':>6s} {'K':>6s}  " + " ".join(f"{'cfg' + str(c):>8s}" for c in range(nc))
              + f" {'default':>8s} {'cold':>8s}  workload")
        for M, N, K, name in shapes:
            A = torch.randn(M, K, device=dev)
            B = torch.randn(K, N, device=dev)
            C = torch.empty(M, N, device=dev)
            flop = rl.gemm_flops(M, N, K)
            reps = max(3, min(200, int(2e11 / flop)))
            sel = mm.mm_gemm_f32_select(M, N, K)
            cells = []
            for c in range(nc):
                def launch(i, st, c=c):
                    mm.mm_gemm_f32_config(c, M, N, K, A, K, B, N, C, N, st)
                ms = median_graph_ms(torch, launch, reps)
                cells.append(f"{flop / ms / 1e9:7.1f}" + ("*" if c == sel else " "))

            def default(i, st):
                mm.mm_gemm_f32(M, N, K, A, K, B, N, C, N, st)
            cells.append(f"{flop / median_graph_ms(torch, default, reps) / 1e9:8.1f}")
            if N <= 64 and M * K * 4 >= 32 << 20:
                # the FC layer with A read from HBM: calls rotate over 8 copies of A (more
                # than the 256 MB Infinity Cache)
                As = [A] + [torch.randn(M, K, device=dev) for _ in range(GEMV_SETS - 1)]

                def cold(i, st):
                    mm.mm_gemm_f32(M, N, K, As[i % GEMV_SETS], K, B, N, C, N, st)
                cells.append(f"{flop / median_graph_ms(torch, cold, 64) / 1e9:8.1f}")
                del As
            else:
                cells.append(f"{'':8s}")
            print(f"{M:6d} {N:6d} {K:6d}  " + " ".join(cells) + f"  {name}", flush=True)
            del A, B, C
        print("# strided batched GEMM (one mm_gemm_f32_batched launch) vs the same problems as "
              "separate mm_gemm_f32 calls, TFLOP/s")
        print(f"{'batch':>6s} {'M':>6s} {'N':>6s} {'K':>6s} {'batched':>9s} {'separate':>9s}")
        for batch, M, N, K in ((64, 512, 512, 512), (16, 1024, 1024, 1024), (256, 256, 256, 256),
                               (32, 128, 4096, 128)):
            A = torch.randn(batch, M, K, device=dev)
            B = torch.randn(batch, K, N, device=dev)
            C = torch.empty(batch, M, N, device=dev)
            flop = batch * rl.gemm_flops(M, N, K)
            reps = max(3, min(100, int(2e11 / flop)))

            def batched(i, st):
                mm.mm_gemm_f32_batched(batch, M, N, K, A, K, M * K, B, N, K * N, C, N, M * N, st)

            def separate(i, st):
                for b in range(batch):
                    mm.mm_gemm_f32(M, N, K, A[b], K, B[b], N, C[b], N, st)
            tb = median_graph_ms(torch, batched, reps)
            ts = median_graph_ms(torch, separate, max(1, reps // 4))
            print(f"{batch:6d} {M:6d} {N:6d} {K:6d} {flop / tb / 1e9:9.1f} {flop / ts / 1e9:9.1f}",
                  flush=True)
            del A, B, C
        print("# few output tiles: mm_gemm_f32 vs mm_gemm_f32_ws (K split over 2-8 chunks of the "
              "64 x 64 tile, partial products in a workspace, then a sum kernel), TFLOP/s")
        print(f"{'M':>6s} {'N':>6s} {'K':>6s} {'chunks':>7s} {'gemm':>9s} {'gemm_ws':>9s}")
        for M, N, K in ((4096, 32, 4096), (4096, 48, 4096), (4096, 64, 4096), (4096, 128, 4096),
                        (4096, 256, 4096), (1024, 128, 4096), (8192, 64, 8192), (1024, 64, 8192),
                        (4096, 45, 4096), (4096, 99, 4096), (4096, 127, 4096)):
            A = torch.randn(M, K, device=dev)
            B = torch.randn(K, N, device=dev)
            C = torch.empty(M, N, device=dev)
            ws = mm.gemm_workspace(M, N, K, dev)
            wsb = 0 if ws is None else ws.numel()
            N4 = -(-N // 4) * 4       # slices of N rounded up to 4, then B padded to N4 if N % 4
            chunks = (wsb // 4 - (K * N4 if N4 != N else 0)) // (M * N4) if wsb else 0
            flop = rl.gemm_flops(M, N, K)
            reps = max(3, min(200, int(2e11 / flop)))

            def plain(i, st):
                mm.mm_gemm_f32(M, N, K, A, K, B, N, C, N, st)

            def split(i, st):
                mm.mm_gemm_f32_ws(M, N, K, A, K, B, N, C, N, ws, wsb, st)
            tp = median_graph_ms(torch, plain, reps)
            tw = median_graph_ms(torch, split, reps)
            print(f"{M:6d} {N:6d} {K:6d} {chunks:7d} {flop / tp / 1e9:9.1f} {flop / tw / 1e9:9.1f}",
                  flush=True)
            del A, B, C, ws
    elif kind == "h16":
        shapes = [(w.M, w.N, w.K, w.name) for w in wl.WORKLOADS.values() if w.op == "gemm"]
        shapes += [(1536, 1536, 1536, ""), (2048, 2048, 2048, ""), (3072, 3072, 3072, ""),
                   (4096, 4096, 1024, ""), (4096, 4096, 4096, ""), (8192, 8192, 8192, ""),
                   (4096, 1024, 4096, ""), (1000, 4000, 3000, "")]
        nc = mm.mm_gemm_h16_num_configs()
        peak = rl.MI355X_16BIT_MFMA_PEAK / 1e12
        print("# 16-bit-input GEMM (fp32 accumulate, fp32 C), TFLOP/s per tile configuration "
              f"(launches captured in a HIP graph and replayed between two events, so that the "
              f"host's launch rate does not bound short kernels; dense 16-bit peak {peak:.0f} TFLOP/s)")
        for c in range(nc):
            print(f"#   cfg {c}: {mm.mm_gemm_h16_config_name(c)}")
        print("#   * = the configuration mm_gemm_bf16 / mm_gemm_f16 select for the shape")
        print(f"{'M':>6s} {'N':>6s} {'K':>6s}  fmt   " +
              " ".join(f"{'cfg' + str(c):>8s}" for c in range(nc)) + "  best % of peak  workload")
        for M, N, K, name in shapes:
            for fmt, dt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
                A = torch.randn(M, K, device=dev).to(dt)
                B = (torch.randn(K, N, device=dev) / K ** 0.5).to(dt)
                C = torch.empty(M, N, device=dev)
                flop = rl.gemm_flops(M, N, K)
                reps = max(3, min(200, int(2e12 / flop)))
                sel = mm.mm_gemm_h16_select(M, N, K)
                fn = mm.mm_gemm_bf16_config if fmt == "bf16" else mm.mm_gemm_f16_config
                cells, best = [], 0.0
                for c in range(nc):
                    def launch(i, st, c=c):
                        fn(c, M, N, K, A, K, B, N, C, N, st)
                    tf = flop / graph_time_ms(torch, launch, reps) / 1e9
                    best = max(best, tf)
                    cells.append(f"{tf:7.1f}" + ("*" if c == sel else " "))
                print(f"{M:6d} {N:6d} {K:6d}  {fmt:5s} " + " ".join(cells) +
                      f"  {100 * best / peak:13.1f}  {name}", flush=True)
                del A, B, C
    else:
        VN = 4096
        # The per-launch floor: kernels with next to no work, launched back to back (host
        # rate) and replayed from a HIP graph (the GPU's own dispatch-to-completion time).
        one = torch.empty(1, device=dev)
        xa = torch.rand(64, device=dev)
        ya = torch.empty(1, device=dev)

        def fill(i, st):
            one.zero_()

        def tiny_gemv(i, st):
            mm.mm_gemv_f32(1, 64, xa, xa, ya, st)
        floor_rows = []
        for name, fn in (("torch fill of 1 float", fill), ("mm_gemv_f32 1 x 64", tiny_gemv)):
            floor_rows.append((name, burst_time_ms(torch, fn, 500), graph_time_ms(torch, fn, 500)))
        floor_graph = min(r[2] for r in floor_rows)
        print("# per-launch floor (kernels with next to no work, 500 launches):")
        for name, tb, tg in floor_rows:
            print(f"#   {name:24s} back-to-back {tb * 1e3:6.2f} us   replayed from a HIP graph "
                  f"{tg * 1e3:6.2f} us")
        print("# fp32 GEMV y = A x, N = 4096: time per launch vs M (back-to-back launches "
              "between two events; graph: the same launches replayed from a HIP graph)")
        print("#   cold: the launches rotate over matrices totalling >= 512 MiB (more than the "
              "256 MB Infinity Cache); warm: one matrix, launched repeatedly")
        print(f"{'M':>7s} {'MiB':>7s} {'cold_us':>9s} {'cold_GB/s':>10s} {'warm_us':>9s} "
              f"{'warm_GB/s':>10s} {'graph_cold_us':>14s}")
        rows = []
        for VM in (256, 512, 1024, 2048, 4096, 8192, 16384, 32768):
            sets = max(2, min(16, (512 << 20) // (VM * VN * 4)))
            As = [torch.rand(VM, VN, device=dev) for _ in range(sets)]
            xs = [torch.rand(VN, device=dev) for _ in range(sets)]
            ys = [torch.empty(VM, device=dev) for _ in range(sets)]
            reps = 8 * sets if VM >= 4096 else 200

            def cold(i, st):
                k = i % sets
                mm.mm_gemv_f32(VM, VN, As[k], xs[k], ys[k], st)

            def warm(i, st):
                mm.mm_gemv_f32(VM, VN, As[0], xs[0], ys[0], st)
            by = rl.gemv_algorithmic_bytes(VM, VN)
            tc = burst_time_ms(torch, cold, reps)
            tw = burst_time_ms(torch, warm, reps)
            tg = graph_time_ms(torch, cold, reps)
            rows.append((VM, by, tc))
            print(f"{VM:7d} {VM * VN * 4 / 2**20:7.0f} {tc * 1e3:9.2f} {by / tc / 1e6:10.0f} "
                  f"{tw * 1e3:9.2f} {by / tw / 1e6:10.0f} {tg * 1e3:14.2f}", flush=True)
            del As, xs, ys
        # least-squares line t = t0 + bytes / rate over the cold points with M >= 2048
        pts = [(b, t) for (m, b, t) in rows if m >= 2048]
        n = len(pts)
        mb = sum(b for b, _ in pts) / n
        mt = sum(t for _, t in pts) / n
        slope = sum((b - mb) * (t - mt) for b, t in pts) / sum((b - mb) ** 2 for b, _ in pts)
        t0 = mt - slope * mb                    # ms
        rate = 1e3 / slope                      # bytes per second
        print(f"# cold fit over M >= 2048: fixed {t0 * 1e3:.2f} us per launch + streaming at "
              f"{rate / 1e9:.0f} GB/s ({100 * rate / rl.MI355X_HBM_PEAK:.1f}% of 8 TB/s)")
        by = rl.gemv_algorithmic_bytes(4096, VN)
        best = by / (floor_graph * 1e-3 + by / rl.MI355X_HBM_PEAK)
        print(f"# single-launch ceiling for the 4096 x 4096 GEMV: even streaming at the full 8 TB/s, "
              f"one launch takes at least the graph-replayed floor {floor_graph * 1e3:.2f} us + "
              f"{by / rl.MI355X_HBM_PEAK * 1e6:.2f} us, i.e. at most {best / 1e9:.0f} GB/s = "
              f"{100 * best / rl.MI355X_HBM_PEAK:.1f}% of 8 TB/s; at the fitted streaming rate, "
              f"{t0 * 1e3 + by / rate * 1e6:.2f} us = {100 * by / (t0 * 1e-3 + by / rate) / rl.MI355X_HBM_PEAK:.1f}%; "
              f"80% needs {by / (0.8 * rl.MI355X_HBM_PEAK) * 1e6:.2f} us")
        # What another implementation's single cold launch over the same bytes reaches: the
        # framework's row-sum reduction reads a 4096 x 4096 matrix once and writes 4096
        # floats, the GEMV's traffic without x (not part of the path, a reference point).
        sets = (512 << 20) // (4096 * VN * 4)
        As = [torch.rand(4096, VN, device=dev) for _ in range(sets)]
        ys = [torch.empty(4096, device=dev) for _ in range(sets)]

        def rowsum(i, st):
            torch.sum(As[i % sets], dim=1, out=ys[i % sets])
        tr = burst_time_ms(torch, rowsum, 8 * sets)
        rb = 4 * 4096 * (VN + 1)
        print(f"# reference read, cold, same rotation: torch.sum(A, dim=1) over 4096 x {VN}: "
              f"{tr * 1e3:.2f} us, {rb / tr / 1e6:.0f} GB/s ({100 * rb / (tr * 1e-3) / rl.MI355X_HBM_PEAK:.1f}% of 8 TB/s)",
              flush=True)
        del As, ys
        print("# transposed GEMV y = A^T x, same timing, cold: mm_gemv_t_f32 (column strips: 16 columns for N <= 6144, 32 for N <= 12288, else 64) and "
              "mm_gemv_t_f32_ws (row blocks, partial sums in a workspace, two launches)")
        for TM, TN in ((4096, 4096), (8192, 8192), (16384, 4096), (4096, 16384)):
            sets = max(2, min(16, (512 << 20) // (TM * TN * 4)))
            As = [torch.rand(TM, TN, device=dev) for _ in range(sets)]
            xs = [torch.rand(TM, device=dev) for _ in range(sets)]
            ys = [torch.empty(TN, device=dev) for _ in range(sets)]
            ws = mm.gemv_t_workspace(TM, TN, dev)
            wsb = 0 if ws is None else ws.numel()

            def cold_t(i, st):
                k = i % sets
                mm.mm_gemv_t_f32(TM, TN, As[k], xs[k], ys[k], st)

            def cold_ws(i, st):
                k = i % sets
                mm.mm_gemv_t_f32_ws(TM, TN, As[k], xs[k], ys[k], ws, wsb, st)
            by = rl.FP32 * (TM * TN + TM + TN)
            cells = []
            for fn in (cold_t, cold_ws):
                tc = burst_time_ms(torch, fn, 8 * sets)
                cells.append(f"{tc * 1e3:8.2f} us {by / tc / 1e6:6.0f} GB/s "
                             f"({100 * by * 1e3 / tc / rl.MI355X_HBM_PEAK:.1f}%)")
            print(f"#   M={TM:6d} N={TN:6d}: strips {cells[0]}   workspace {cells[1]}", flush=True)
            del As, xs, ys, ws


if __name__ == "__main__":
    main()
