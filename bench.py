#!/usr/bin/env python3
"""Benchmark of the block-scaled MXFP4 linear-layer hot path on one MI355X.

One step = one forward + backward pass of the LLaMA-1B FFN up-projection
layer (X bf16 8192x2048, W bf16 2048x5632, dY bf16 8192x5632, MXFP4 block 32)
through every kernel of the path:

  forward   Q2(X): ROW (forward operand) + COL (dW operand), RNE, one pass
            Q2(W): COL (forward operand) + ROW (dX operand), RNE, one pass
            Y = GEMM 8192x5632x2048 -> bf16;  DQ(Q(X)) -> bf16 (the QDQ output)
  backward  Q2(dY): ROW + COL, stochastic (one random stream, seed 1234)
            dX = GEMM 8192x2048x5632 -> bf16
            dW' = GEMM 2048x5632x8192 -> fp32 with DGE(W, col blocks, k=5,
                  clamp 3) applied in its epilogue (one kernel; the unfused
                  GEMM + DGE pair is timed aside)
  The quantisers of W and dY, dequantize and the backward GEMMs are launched
  any-order (each depends only on kernels that a plain launch before it has
  waited for); --sequential launches everything plainly.

The other workloads (the tiny case, the activation sweep, the 13B-shaped
outlier layer with its hot-channel residual, the outlier-compensation
fidelity) are measured in the same default run; --skip-configs leaves them
out.

`value` = FP4 GEMM flops of the step / step time (TFLOPS), i.e. whole-step
throughput over the timed steps.  The roofline object reports the forward
GEMM (the dominant kernel) against the dense FP4 MFMA peak, its launch time
taken from HIP events that its own dispatch records inside the timed region
(fp4q_set_next_launch; on the stream the kernels run on, created without a
system-scope fence), and its HBM traffic from rocprofv3 counter passes this
run starts as child processes after everything else is measured (or,
failing those, from the committed counter record while the GEMM source
matches it).  A
second pass, every launch plain, times each kernel by its own dispatch
events for the per-kernel table.  The CPU baseline times the
single-threaded oracle on a bounded sample.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

PEAK_FP4_TFLOPS = 10100.0   # MI355X dense MXFP4 MFMA
SR_SEED = 1234              # the gradient's stochastic rounding, both orientations
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--settle-s", type=float, default=0.3,
                   help="run whole steps for at least this many seconds before the warm-up "
                        "steps: an idle MI355X takes tens of milliseconds of load to reach its "
                        "steady clocks, and steps timed before that run up to 15%% slower")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-budget-s", type=float, default=20.0)
    p.add_argument("--hcp", action="store_true",
                   help="(kept for compatibility: the 13B-shaped layer is part of the default run)")
    p.add_argument("--skip-configs", action="store_true",
                   help="skip the activation-sweep and 13B-shaped outlier-layer measurements")
    p.add_argument("--profile-op", default=None,
                   help="run only this step kernel (or 'copy', a plain 256 MiB device copy, "
                        "or 'hcp_residual', the 13B layer's D-mode residual) --reps times "
                        "and exit: the target of rocprofv3 counter runs")
    p.add_argument("--hot-channels", type=int, default=None,
                   help="with --profile-op hcp_residual: use only the first N hot channels")
    p.add_argument("--reps", type=int, default=10)
    p.add_argument("--traffic", choices=("live", "record", "off"), default="live",
                   help="the roofline's HBM traffic: 'live' runs four short rocprofv3 counter "
                        "passes as child processes (falling back to the committed record), "
                        "'record' reads the committed record only")
    p.add_argument("--sequential", action="store_true",
                   help="launch every step kernel behind a barrier (no any-order launches)")
    return p.parse_args()


TRAFFIC_FILE = os.path.join(HERE, "profiles", "gemm_fwd_traffic.json")
KERNEL_SRC = os.path.join(HERE, "mxfp4_block_scaled_fp4q_amd", "csrc", "gemm_fp4.hip")


def counter_median(files, kname, counter, min_value, min_dispatches=3):
    """Median over dispatches of one counter in rocprofv3 CSV counter files
    (`--output-format csv`): rows of kernels whose name contains kname are
    summed per Dispatch_Id (a counter may come in several rows per
    dispatch); dispatches below min_value (a kernel of the same name on a
    tiny buffer) are left out; None with fewer than min_dispatches."""
    import csv
    per = {}
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if kname in row["Kernel_Name"] and row["Counter_Name"] == counter:
                    k = row["Dispatch_Id"]
                    per[k] = per.get(k, 0.0) + float(row["Counter_Value"])
    vals = [v for v in per.values() if v >= min_value]
    return float(np.median(vals)) if len(vals) >= min_dispatches else None


def live_traffic(budget_s=120.0, pass_s=60.0):
    """HBM bytes per forward-GEMM launch measured by this run: four rocprofv3
    counter passes, each a child process (this script with --profile-op, five
    launches): FETCH_SIZE and WRITE_SIZE of the GEMM, each scaled by what the
    same counter reads for a plain 256 MiB device copy (FETCH_SIZE counts a
    128-byte read as 64 bytes).  A pass takes a few seconds; each is cut at
    pass_s and all four at budget_s, and the first pass without a result
    ends the measurement.  Returns (bytes, details) or (None, reason)."""
    import glob
    import shutil
    import signal
    import subprocess
    import tempfile
    if any(k.startswith("ROCP") for k in os.environ) or "rocprof" in os.environ.get(
            "LD_PRELOAD", ""):
        return None, "running under a profiler: no nested counter passes"
    prof = shutil.which("rocprofv3") or "/opt/rocm/bin/rocprofv3"
    if not os.path.exists(prof):
        return None, "rocprofv3 not found"
    tmp = tempfile.mkdtemp(prefix="fp4q_traffic_")
    env = dict(os.environ, TMPDIR=tempfile.gettempdir())
    deadline = time.perf_counter() + budget_s

    def one_pass(counter, op, kname, min_kib):
        left = min(pass_s, deadline - time.perf_counter())
        if left <= 1.0:
            return None
        d = os.path.join(tmp, op + "_" + counter)
        cmd = [prof, "--pmc", counter, "-d", d, "-o", "p", "--output-format", "csv", "--",
               sys.executable, os.path.abspath(__file__), "--profile-op", op, "--reps", "5"]
        child = subprocess.Popen(cmd, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL,
                                 env=env, cwd=HERE, start_new_session=True)
        try:
            child.wait(timeout=left)
        except subprocess.TimeoutExpired:
            os.killpg(child.pid, signal.SIGKILL)
            child.wait()
            return None
        # the profiler may exit non-zero after the program ended with its
        # results whole: the counter file decides
        files = glob.glob(os.path.join(d, "**", "p_counter_collection.csv"), recursive=True)
        return counter_median(files, kname, counter, min_kib)

    gk = "gemm_fp4_persistent_kernel<1, 0, 0>"
    passes = (("gemm_fetch_kib", "FETCH_SIZE", "gemm_fwd", gk, 1.0),
              ("gemm_write_kib", "WRITE_SIZE", "gemm_fwd", gk, 1.0),
              ("copy_fetch_kib", "FETCH_SIZE", "copy", "copyBuffer", 1024.0),
              ("copy_write_kib", "WRITE_SIZE", "copy", "copyBuffer", 1024.0))
    got = dict((p[0], None) for p in passes)
    try:
        for key, counter, op, kname, min_kib in passes:
            got[key] = one_pass(counter, op, kname, min_kib)
            if got[key] is None:
                break
    except OSError as e:
        return None, "could not run rocprofv3: " + str(e)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    for key, counter, op, _, _ in passes:
        if got[key] is None:
            return None, "the %s pass of --profile-op %s gave no result" % (counter, op)
    copy_kib = 256.0 * 1024  # 64 Mi floats read and written
    fs, ws = copy_kib / got["copy_fetch_kib"], copy_kib / got["copy_write_kib"]
    if not (0.5 < fs < 4.0 and 0.5 < ws < 4.0):
        return None, "implausible copy calibration %.3f / %.3f" % (fs, ws)
    traffic = int(round(got["gemm_fetch_kib"] * 1024 * fs + got["gemm_write_kib"] * 1024 * ws))
    got.update(fetch_scale=round(fs, 4), write_scale=round(ws, 4))
    return traffic, got


def measured_traffic():
    """HBM bytes per forward-GEMM launch from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE runs, scaled by a plain copy's counters -- only while
    the GEMM source is the one those counters were taken on (else None)."""
    import hashlib
    import json as _json
    try:
        rec = _json.load(open(TRAFFIC_FILE))
        src = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != src:
        return None
    return rec.get("traffic_bytes_per_launch")


# asides timed by event records around the call rather than by the
# dispatch's own events: not a single library kernel
MARKER_TIMED = {"copy_dy", "occ_quantize_x"}


class HipEvents:
    """HIP events created with hipEventDisableSystemFence, recorded on the
    stream the kernels run on: a plain event's record releases to system
    scope, which writes the L2 back and charges that to the kernel before
    it (several microseconds after a GEMM that leaves its output in L2)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, torch):
        import ctypes
        self.ct = ctypes
        self.L = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        self.made = []

    def _check(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def create(self):
        ev = self.ct.c_void_p()
        self._check(self.L.hipEventCreateWithFlags(self.ct.byref(ev), self.DISABLE_SYSTEM_FENCE),
                    "hipEventCreateWithFlags")
        self.made.append(ev)
        return ev

    def record(self, ev):
        self._check(self.L.hipEventRecord(ev, self.stream), "hipEventRecord")

    def elapsed_us(self, a, b):
        ms = self.ct.c_float()
        self._check(self.L.hipEventElapsedTime(self.ct.byref(ms), a, b), "hipEventElapsedTime")
        return ms.value * 1e3

    def close(self):
        for ev in self.made:
            self.L.hipEventDestroy(ev)
        self.made = []


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    import mxfp4_block_scaled_fp4q_amd as fq
    from mxfp4_block_scaled_fp4q_amd import inputs

    fq.lib()  # fails loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    M, K, N = 8192, 2048, 5632
    f = inputs.ffn_forward(M, K, N)
    b = inputs.ffn_backward_grad(M, N)

    def to_bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    X, W, dY = to_bf16(f["X"]), to_bf16(f["W"]), to_bf16(b["dY"])
    u8 = dict(dtype=torch.uint8, device=dev)
    bufs = {
        "xr": (torch.empty((M, K // 2), **u8), torch.empty((M, K // 32), **u8)),
        "wc": (torch.empty((N, K // 2), **u8), torch.empty((N, K // 32), **u8)),
        "dyr": (torch.empty((M, N // 2), **u8), torch.empty((M, N // 32), **u8)),
        "wr": (torch.empty((K, N // 2), **u8), torch.empty((K, N // 32), **u8)),
        "xc": (torch.empty((K, M // 2), **u8), torch.empty((K, M // 32), **u8)),
        "dyc": (torch.empty((N, M // 2), **u8), torch.empty((N, M // 32), **u8)),
    }
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    Xdq = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dW = torch.empty((K, N), dtype=torch.float32, device=dev)
    dWo = torch.empty((K, N), dtype=torch.float32, device=dev)
    dYg = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    dXg = torch.empty((M, K), dtype=torch.bfloat16, device=dev)

    # (name, callable, algorithmic bytes, algorithmic flops)
    qb = 2 + 0.5 + 1 / 32  # bf16 in, codes + E8M0 bytes out, per element
    qb2 = 2 + 2 * (0.5 + 1 / 32)  # one read, both orientations written
    dual = lambda t, rr, sr, rc, sc, a, b: fq.quantize_dual(
        t, 32, rr, sr, rc, sc, out=(bufs[a][0], bufs[a][1], bufs[b][0], bufs[b][1]))
    ops = [
        # X: ROW for the forward GEMM, COL (X^T) for dW
        ("quant_x_dual", lambda: dual(X, fq.RNE, 0, fq.RNE, 0, "xr", "xc"), M * K * qb2, 0),
        # W: COL (W^T, K-major) for the forward GEMM, ROW for dX
        ("quant_w_dual", lambda: dual(W, fq.RNE, 0, fq.RNE, 0, "wr", "wc"), K * N * qb2, 0),
        # dY: ROW for dX, COL (dY^T) for dW, stochastic, one random stream
        ("quant_dy_dual_sr", lambda: dual(dY, fq.SR, SR_SEED, fq.SR, SR_SEED, "dyr", "dyc"),
         M * N * qb2, 0),
        ("gemm_fwd", lambda: fq.gemm(*bufs["xr"], *bufs["wc"], c=Y),
         (M + N) * K * (0.5 + 1 / 32) + M * N * 2, 2.0 * M * N * K),
        ("dequant_x", lambda: fq.dequantize(*bufs["xr"], 32, out=Xdq), M * K * qb, 0),
        ("gemm_dx", lambda: fq.gemm(*bufs["dyr"], *bufs["wr"], c=dX),
         (M + K) * N * (0.5 + 1 / 32) + M * K * 2, 2.0 * M * K * N),
        # dW = X^T dY with W's DGE derivative applied in the GEMM's epilogue
        # (the same bits as the GEMM into fp32 followed by fp4q_grad_estimate)
        ("gemm_dw_dge", lambda: fq.gemm_dge(*bufs["xc"], *bufs["dyc"], W, 5.0, 3.0, out=dWo),
         (K + N) * M * (0.5 + 1 / 32) + K * N * (2 + 4), 2.0 * K * N * M),
    ]
    yq = (torch.empty((M, N // 2), **u8), torch.empty((M, N // 32), **u8))
    w2d = (torch.empty((K, N // 2), **u8), torch.empty((K, N // 32), **u8),
           torch.empty((N, K // 2), **u8), torch.empty((N, K // 32), **u8))
    # one sign mask over the token axis for both weight-gradient operands
    gsm = torch.Generator().manual_seed(7)
    msk = torch.randint(-2 ** 31, 2 ** 31 - 1, ((M + 31) // 32,), generator=gsm,
                        dtype=torch.int64).to(torch.int32).to(dev)
    xrht = (torch.empty((K, M // 2), **u8), torch.empty((K, M // 32), **u8))
    # outlier clamping and compensation of X (1% clamped): buffers sized by
    # the bound, the residual's product added into an fp32 output
    occ_cap = fq.occ_max_nnz(M, K, 0.99)
    occ = dict(codes=torch.empty((M, K // 2), **u8), scales=torch.empty((M, K // 32), **u8),
               rp=torch.empty((M + 1,), dtype=torch.int64, device=dev),
               ci=torch.empty((occ_cap,), dtype=torch.int32, device=dev),
               v=torch.empty((occ_cap,), dtype=torch.float32, device=dev),
               thr=torch.empty((8,), dtype=torch.int16, device=dev),
               ws=torch.empty(fq.lib().fp4q_occ_workspace_bytes(M, K), **u8),
               y=torch.zeros((M, N), dtype=torch.float32, device=dev))

    def occ_quant():
        fq._check(fq.lib().fp4q_occ_quantize(
            fq._ptr(X), M, K, K, 0.99, fq.RNE, 0, 0, fq._ptr(occ["codes"]), fq._ptr(occ["scales"]),
            fq._ptr(occ["rp"]), fq._ptr(occ["ci"]), fq._ptr(occ["v"]), occ_cap,
            fq._ptr(occ["thr"]), fq._ptr(occ["ws"]), occ["ws"].numel(), fq._stream(None)))

    dyrht = (torch.empty((N, M // 2), **u8), torch.empty((N, M // 32), **u8))
    # timed aside: the unfused dW GEMM and DGE (the DGE kernel's own HBM
    # rate), and the forward GEMM that also quantises Y for a next layer
    # against the same GEMM followed by the ROW quantiser
    aside_ops = [
        ("gemm_fwd_quant_y", lambda: fq.gemm_quant(*bufs["xr"], *bufs["wc"], c=Y, out=yq),
         (M + N) * K * (0.5 + 1 / 32) + M * N * (2 + 0.5 + 1 / 32), 2.0 * M * N * K),
        ("quant_y_row", lambda: fq.quantize(Y, 32, fq.ROW, codes=yq[0], scales=yq[1]),
         M * N * qb, 0),
        # the quantiser headline's stochastic case on its own: dY, ROW blocks
        # of 32, Philox seed 1234
        ("quant_dy_row_sr", lambda: fq.quantize(dY, 32, fq.ROW, fq.SR, SR_SEED, codes=yq[0],
                                                scales=yq[1]), M * N * qb, 0),
        ("gemm_dw", lambda: fq.gemm(*bufs["xc"], *bufs["dyc"], c=dW),
         (K + N) * M * (0.5 + 1 / 32) + K * N * 4, 2.0 * K * N * M),
        ("dge_dw", lambda: fq.grad_estimate(fq.DGE, W, dW, 32, fq.COL, 5.0, 3.0, out=dWo),
         K * N * (2 + 4 + 4), 0),
        # W with one scale per 32 x 32 square: both layouts from one pass,
        # one set of values for the forward and the data-gradient GEMM
        ("quant_w_2d", lambda: fq.quantize_2d(W, fq.RNE, 0, 0, out=w2d), K * N * qb2, 0),
        # the weight-gradient operands with the random Hadamard transform
        # along the token axis (COL groups), X nearest-even and dY stochastic
        ("quant_x_col_rht", lambda: fq.quantize_rht(X, msk, fq.COL, fq.RNE, 0, 0, codes=xrht[0],
                                                    scales=xrht[1]), M * K * qb, 0),
        ("quant_dy_col_rht_sr", lambda: fq.quantize_rht(dY, msk, fq.COL, fq.SR, SR_SEED, 0,
                                                        codes=dyrht[0], scales=dyrht[1]),
         M * N * qb, 0),
        # six launches: histogram, threshold, clamp + quantise, scan, CSR fill
        ("occ_quantize_x", occ_quant, M * K * qb, 0),
        # Y[M, N] += R W: reads and writes the fp32 rows that hold outliers
        ("occ_spmm", lambda: fq.occ_spmm(occ["rp"], occ["ci"], occ["v"], W, occ["y"]),
         M * N * 8, 0),
        # the straight-through estimator on a gradient of dY's size (bf16 in,
        # bf16 out, 4 B per element), and torch's device copy of the same
        # tensor as the attainable rate for that traffic
        ("ste_dy", lambda: fq.grad_estimate(fq.STE, None, dY, 32, fq.ROW, out=dYg), M * N * 4, 0),
        ("copy_dy", lambda: dYg.copy_(dY), M * N * 4, 0),
        # the activation quantiser's DGE backward at the layer's size: X's ROW
        # blocks (scales recomputed from X), applied to the data gradient dX
        # (bf16 x, g and out, 6 B per element)
        ("dge_x", lambda: fq.grad_estimate(fq.DGE, X, dX, 32, fq.ROW, 5.0, 3.0, out=dXg),
         M * K * 6, 0),
    ]
    step_flops = sum(o[3] for o in ops)

    if args.profile_op == "hcp_residual":
        profile_hcp_residual(torch, fq, inputs, dev, args.reps, args.hot_channels)
        return
    if args.profile_op is not None:
        if args.profile_op == "copy":
            n = 64 << 20
            a = torch.ones(n, dtype=torch.float32, device=dev)
            b = torch.empty_like(a)
            fn = lambda: b.copy_(a)
        else:
            fn = dict((o[0], o[1]) for o in ops + aside_ops)[args.profile_op]
        for _ in range(args.reps):
            fn()
        torch.cuda.synchronize()
        return

    i_fwd = [o[0] for o in ops].index("gemm_fwd")
    # Launches that may start before the stream's earlier kernels finish
    # (fp4q_set_next_launch any-order): each reads only what a kernel behind
    # a barrier has already finished (the step's first kernel and the forward
    # GEMM are plain launches, so they wait for everything before them).
    # The three quantisers overlap each other's ramp-up and tail; dequantize
    # and the backward GEMMs fill compute units as the forward GEMM's
    # workgroups finish.
    any_order = {"quant_w_dual", "quant_dy_dual_sr", "dequant_x", "gemm_dx", "gemm_dw_dge"}
    ao = [o[0] in any_order and not args.sequential for o in ops]

    hev = HipEvents(torch)

    def run_step(evs=None, fwd_evs=None):
        # evs: a start/stop pair per kernel, recorded by each kernel's own
        # dispatch (the per-kernel pass, every launch plain)
        for i, (_, fn, _, _) in enumerate(ops):
            if evs is not None:
                fq.set_next_launch(evs[2 * i], evs[2 * i + 1])
            elif fwd_evs is not None and i == i_fwd:
                fq.set_next_launch(fwd_evs[0], fwd_evs[1])
            elif ao[i]:
                fq.set_next_launch(any_order=True)
            fn()

    # Clock settling, then the warm-up steps: the device runs whole steps
    # until it has been busy for settle_s seconds (an idle GPU's clocks ramp
    # up over the first tens of milliseconds of load; measured on MI355X, 5
    # warm-up steps left the timed steps 16% slower than 200 did), so the
    # timed steps see the steady state a continuous training job runs in.
    settle_steps = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_s:
        for _ in range(10):
            run_step()
        torch.cuda.synchronize()
        settle_steps += 10
    settle_s = time.perf_counter() - t_settle
    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()

    # Timed region: exactly `steps` steps, synchronised on both sides.  The
    # only events inside it are the forward GEMM's (the roofline kernel),
    # recorded by that kernel's own dispatch on the stream every kernel is
    # launched on (fp4q_set_next_launch), so no marker packets sit between
    # the step's kernels and the events span the kernel alone.
    fwd_events = [[hev.create() for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        run_step(fwd_evs=fwd_events[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    fwd_us = [hev.elapsed_us(e[0], e[1]) for e in fwd_events]

    # Per-kernel breakdown: the same steps again, every launch plain, each
    # kernel's duration from the events its own dispatch records.
    events = [[hev.create() for _ in range(2 * len(ops))] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        run_step(events[s])
    torch.cuda.synchronize()

    def op_stats(ts, nbytes, nflops):
        us = float(np.mean(ts))
        d = {"us": round(us, 2), "us_min": round(float(np.min(ts)), 2),
             "us_median": round(float(np.median(ts)), 2),
             "us_p10": round(float(np.percentile(ts, 10)), 2)}
        if nflops:
            d["TFLOPS"] = round(nflops / (us * 1e-6) / 1e12, 1)
            d["frac_fp4_peak"] = round(d["TFLOPS"] / PEAK_FP4_TFLOPS, 4)
        d["GBps"] = round(nbytes / (us * 1e-6) / 1e9, 1)
        d["frac_hbm_peak"] = round(d["GBps"] / PEAK_HBM_GBPS, 4)
        return d

    per_op = {}
    for i, (name, _, nbytes, nflops) in enumerate(ops):
        ts = [hev.elapsed_us(events[s][2 * i], events[s][2 * i + 1]) for s in range(args.steps)]
        per_op[name] = op_stats(ts, nbytes, nflops)

    # asides, each timed alone: one library kernel by its own dispatch's
    # events; torch's copy and the six-kernel outlier quantisation by event
    # records around the call (which add the queue's turnaround to them)
    aside = {}
    for name, fn, nbytes, nflops in aside_ops:
        fn()
        torch.cuda.synchronize()
        evs = [hev.create() for _ in range(2 * args.steps)]
        for s_ in range(args.steps):
            if name in MARKER_TIMED:
                hev.record(evs[2 * s_])
                fn()
                hev.record(evs[2 * s_ + 1])
            else:
                fq.set_next_launch(evs[2 * s_], evs[2 * s_ + 1])
                fn()
        torch.cuda.synchronize()
        ts = [hev.elapsed_us(evs[2 * s_], evs[2 * s_ + 1]) for s_ in range(args.steps)]
        aside[name] = op_stats(ts, nbytes, nflops)

    qhead = quantize_headline(torch, fq, hev, dY, M, N, bufs, qb, args.steps)
    hev.close()
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    fwd_flops = 2.0 * M * N * K
    fwd_mean_us = float(np.mean(fwd_us))
    achieved = fwd_flops / (fwd_mean_us * 1e-6) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_FP4_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP4_TFLOPS, 4),
                "traffic": None,
                "kernel": "gemm_fp4_persistent_kernel<1, 0, 0> 8192x5632x2048 bf16 out",
                "per_launch_flops": fwd_flops, "launch_us_mean": round(fwd_mean_us, 2),
                "launch_us_min": round(float(np.min(fwd_us)), 2),
                "launch_us_median": round(float(np.median(fwd_us)), 2),
                "launch_us_p10": round(float(np.percentile(fwd_us, 10)), 2)}
    q = per_op["quant_dy_dual_sr"]
    qr = per_op["quant_x_dual"]
    quant = {"quant_bf16_dual_rne_GBps": qr["GBps"], "quant_bf16_dual_rne_frac": qr["frac_hbm_peak"],
             "quant_bf16_dual_sr_GBps": q["GBps"], "quant_bf16_dual_sr_frac": q["frac_hbm_peak"],
             "quant_dual_bytes_per_elem": qb2}
    quant.update(qhead)

    extra = {"copy_ceiling_GBps": copy_ceiling(torch, dev)}
    if not args.skip_configs:
        # the other workloads: the tiny reference case, the activation sweep
        # (every block size, both roundings, dequantize, STE and DGE) and the
        # 13B-shaped outlier layer
        extra["tiny_ref"] = bench_tiny_ref(torch, fq, inputs, dev)
        extra["activation_sweep"] = bench_activation_sweep(torch, fq, inputs, dev)
        extra["occ_fidelity"] = bench_occ_fidelity(torch, fq, inputs, dev)
        extra["outlier_layer"] = bench_outlier_layer(torch, fq, inputs, dev)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(f, b, step_flops, args.cpu_budget_s)

    # the counter passes last: they leave the GPU idle for several seconds
    if args.traffic == "live":
        traffic, info = live_traffic()
        if traffic is not None:
            roofline["traffic"] = traffic
            roofline["traffic_source"] = ("this run: rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE "
                                          "passes of the kernel, scaled by a 256 MiB copy")
            roofline["traffic_counters"] = info
        else:
            roofline["traffic_live_error"] = info
    if roofline["traffic"] is None and args.traffic != "off":
        roofline["traffic"] = measured_traffic()
        if roofline["traffic"] is not None:
            roofline["traffic_source"] = "committed record " + os.path.relpath(TRAFFIC_FILE, HERE)

    out = {
        "metric": "MXFP4 quantize GB/s + FP4 GEMM TFLOPS (8192x5632x2048), % of roofline",
        "value": round(value, 1),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"seconds": round(settle_s, 3), "steps": settle_steps},
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": "LLaMA-1B FFN up-proj layer, forward + backward: X bf16 8192x2048 "
                               "N(0,1), W bf16 2048x5632 N(0,0.02), dY bf16 8192x5632 N(0,1e-3); "
                               "MXFP4 block 32, E2M1 codes, E8M0 scales, fp32 accumulate",
                   "global_batch": M, "parallelism": "none (1 GPU)",
                   "step_fp4_gflop": round(step_flops / 1e9, 2),
                   "launches": "sequential" if args.sequential else
                               "any-order where independent: " + ", ".join(
                                   o[0] for o, a in zip(ops, ao) if a)},
        "roofline": roofline,
        "quantize": quant,
        "kernels": per_op,
        "unfused_aside": aside,
        **extra,
    }
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


def quantize_headline(torch, fq, hev, dY, M, N, bufs, qb, reps):
    """The quantiser on dY (8192x5632 bf16, ROW blocks of 32, RNE and SR) one
    launch at a time, cold: before each launch a 1 GiB buffer is read (a sum),
    which evicts dY from the L2s and the 256 MB Infinity Cache without leaving
    dirty lines behind; the launch's own dispatch records its events."""
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dY.device)
    out = {}
    for name, rnd in (("rne", fq.RNE), ("sr", fq.SR)):
        fn = lambda: fq.quantize(dY, 32, fq.ROW, rnd, 1234, codes=bufs["dyr"][0],
                                 scales=bufs["dyr"][1])
        fn()
        torch.cuda.synchronize()
        evs = [hev.create() for _ in range(2 * reps)]
        for r in range(reps):
            flush.sum()
            fq.set_next_launch(evs[2 * r], evs[2 * r + 1])
            fn()
        torch.cuda.synchronize()
        us = float(np.mean([hev.elapsed_us(evs[2 * r], evs[2 * r + 1]) for r in range(reps)]))
        gbps = M * N * qb / (us * 1e-6) / 1e9
        out[f"quant_dY_row_{name}_cold_us"] = round(us, 2)
        out[f"quant_dY_row_{name}_cold_GBps"] = round(gbps, 1)
        out[f"quant_dY_row_{name}_cold_frac"] = round(gbps / PEAK_HBM_GBPS, 4)
    del flush
    # The same quantiser streaming over six copies of dY back to back, one
    # pair of events around all the launches: each launch reads a copy that
    # the five launches before it (461 MB of inputs and 122 MB of outputs)
    # have pushed out of the 256 MB Infinity Cache, so its input comes from
    # HBM, and no per-launch event turnaround is counted.
    nc = 6
    copies = [dY] + [dY.clone() for _ in range(nc - 1)]
    outs = [(torch.empty_like(bufs["dyr"][0]), torch.empty_like(bufs["dyr"][1]))
            for _ in range(nc)]
    n = 8 * nc
    for name, rnd in (("rne", fq.RNE), ("sr", fq.SR)):
        run = lambda i: fq.quantize(copies[i % nc], 32, fq.ROW, rnd, 1234, codes=outs[i % nc][0],
                                    scales=outs[i % nc][1])
        for i in range(nc):
            run(i)
        torch.cuda.synchronize()
        e0, e1 = hev.create(), hev.create()
        hev.record(e0)
        for i in range(n):
            run(i)
        hev.record(e1)
        torch.cuda.synchronize()
        us = hev.elapsed_us(e0, e1) / n
        gbps = M * N * qb / (us * 1e-6) / 1e9
        out[f"quant_dY_row_{name}_stream_us"] = round(us, 2)
        out[f"quant_dY_row_{name}_stream_GBps"] = round(gbps, 1)
        out[f"quant_dY_row_{name}_stream_frac"] = round(gbps / PEAK_HBM_GBPS, 4)
    del copies, outs
    return out


def copy_ceiling(torch, dev):
    """Attainable HBM bandwidth of a plain device copy (torch's copy kernel),
    1 GiB read + 1 GiB written, the reference point for the streaming kernels."""
    n = 1 << 28
    a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    secs = e0.elapsed_time(e1) * 1e-3 / reps
    del a, b
    return round(2 * 4 * n / secs / 1e9, 1)


def _stream_us(torch, fn, n=50):
    """Mean time per launch of n back-to-back launches between one pair of
    events (the per-launch event turnaround is not counted)."""
    fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def _graph_us(torch, fns, replays=5):
    """Mean time per launch of the launches fns[0](), fns[1](), ... captured
    in order in one HIP graph, the graph replayed `replays` times (no
    host-side launch cost between kernels)."""
    for f in fns:
        f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e3 / (len(fns) * replays)


def _rate(nbytes, us, us_graph=None):
    """Rates by the graph-replay time when given (else the stream time)."""
    t = us_graph if us_graph is not None else us
    gbps = nbytes / (t * 1e-6) / 1e9
    d = {"us": round(us, 2)}
    if us_graph is not None:
        d["us_graph"] = round(us_graph, 2)
    d.update({"GBps": round(gbps, 1), "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4)})
    return d


def bench_occ_fidelity(torch, fq, inputs, dev):
    """Context for the outlier pages' fidelity figures (cosine, MSE, SNR of
    the quantised activation against the original): the activation workload
    (Student-t(3) x 0.5, bf16 4096 x 2048) quantised directly (ROW blocks of
    32, nearest-even) and with outlier clamping and compensation (values
    beyond the 99th percentile of |x| clamped before quantisation, their
    excess kept in the sparse residual).  Every step runs in the library's
    kernels: the reconstruction of the compensated path is the dequantised
    clamped codes plus R I, R's product with a bf16 identity through
    fp4q_occ_spmm; only the three metrics are torch reductions."""
    d = inputs.activation_sweep()
    x = torch.from_numpy(d["X"].view(np.int16)).view(torch.bfloat16).to(dev)
    R, K = x.shape
    ref = x.float().double()

    def metrics(xh):
        e = xh.double() - ref
        cos = float((xh.double() * ref).sum() / (xh.double().norm() * ref.norm()))
        mse = float((e * e).mean())
        snr = float(10.0 * torch.log10((ref * ref).sum() / (e * e).sum()))
        return {"cosine": round(cos, 6), "mse": mse, "snr_db": round(snr, 3)}

    direct = fq.dequantize(*fq.quantize(x, 32), 32, torch.float32)
    codes, scales, rp, ci, v, _ = fq.occ_quantize(x, 0.99)
    comp = fq.dequantize(codes, scales, 32, torch.float32)
    eye = torch.eye(K, dtype=torch.bfloat16, device=dev)
    fq.occ_spmm(rp, ci, v, eye, comp)
    torch.cuda.synchronize()
    nnz = int(rp[-1].item())
    return {"input": f"bf16 {R}x{K} Student-t(3) x 0.5 (the activation workload)",
            "quantile": 0.99, "outliers": nnz,
            "direct": metrics(direct), "clamp_and_compensate": metrics(comp)}


def bench_activation_sweep(torch, fq, inputs, dev, ncopies=32):
    """Activation sweep: bf16 4096x2048 = 0.5 * Student-t(3), ROW blocks of
    16/32/64/128, nearest-even and stochastic (seed 1234); dequantize of each
    back to bf16; STE and DGE(k=5, clamp 3, blocks of 32) on a bf16 N(0,1)
    gradient.  `us`: one launch on one set of buffers, 50 times back to back
    (the 16.8 MB tensors stay in the caches).  `us_graph`, which the rates
    use: one launch on each of `ncopies` copies of the inputs and outputs
    (about 0.7 GB in all, so each launch finds its data evicted from the 256 MB
    Infinity Cache by the others), captured in one HIP graph and replayed:
    no host launch cost between kernels, inputs from HBM; a launch lasts a
    few microseconds, so its ramp-up and drain are still counted."""
    d = inputs.activation_sweep()
    R, C = d["X"].shape

    def to_bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    X, G = to_bf16(d["X"]), to_bf16(d["G"])
    Xs = [X] + [X.clone() for _ in range(ncopies - 1)]
    Gs = [G] + [G.clone() for _ in range(ncopies - 1)]
    ys = [torch.empty((R, C), dtype=torch.bfloat16, device=dev) for _ in range(ncopies)]
    cs = [torch.empty((R, C // 2), dtype=torch.uint8, device=dev) for _ in range(ncopies)]
    n = R * C
    out = {"shape": [R, C], "copies": ncopies}
    seed = d["sr_seed"]
    for b in (16, 32, 64, 128):
        ss = [torch.empty((R, C // b), dtype=torch.uint8, device=dev) for _ in range(ncopies)]
        qbytes = n * (2 + 0.5 + 1.0 / b)
        for name, rnd in (("rne", fq.RNE), ("sr", fq.SR)):
            fns = [lambda i=i: fq.quantize(Xs[i], b, fq.ROW, rnd, seed, codes=cs[i], scales=ss[i])
                   for i in range(ncopies)]
            out[f"quant_b{b}_{name}"] = _rate(qbytes, _stream_us(torch, fns[0]),
                                              _graph_us(torch, fns))
        fns = [lambda i=i: fq.dequantize(cs[i], ss[i], b, out=ys[i]) for i in range(ncopies)]
        out[f"dequant_b{b}"] = _rate(qbytes, _stream_us(torch, fns[0]), _graph_us(torch, fns))
        del ss
    # the attainable rate at this size: torch's device copy of one bf16
    # tensor to another (16.8 MB read, 16.8 MB written), timed the same way
    fns = [lambda i=i: ys[i].copy_(Gs[i]) for i in range(ncopies)]
    out["copy_same_size"] = _rate(n * 4, _stream_us(torch, fns[0]), _graph_us(torch, fns))
    fns = [lambda i=i: fq.grad_estimate(fq.STE, None, Gs[i], 32, fq.ROW, out=ys[i])
           for i in range(ncopies)]
    out["ste"] = _rate(n * 4, _stream_us(torch, fns[0]), _graph_us(torch, fns))
    fns = [lambda i=i: fq.grad_estimate(fq.DGE, Xs[i], Gs[i], 32, fq.ROW, 5.0, 3.0, out=ys[i])
           for i in range(ncopies)]
    out["dge"] = _rate(n * 6, _stream_us(torch, fns[0]), _graph_us(torch, fns))
    del Xs, Gs, ys, cs
    return out


def profile_hcp_residual(torch, fq, inputs, dev, reps, n_hot=None):
    """The 13B layer's D-mode residual (fp4q_hcp_residual_add) `reps` times on
    a zero fp32 Y, with the first n_hot of its hot channels (all 461 by
    default): the target of counter and trace runs."""
    d = inputs.outlier_layer()

    def to_bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    X, W = to_bf16(d["X"]), to_bf16(d["W"])
    hot = torch.from_numpy(d["hot"]).to(dev)
    if n_hot is not None:
        hot = hot[:n_hot].contiguous()
    M, K = X.shape
    N = W.shape[1]
    xq = fq.quantize(X, 32, fq.ROW)
    wq = fq.quantize(W, 32, fq.COL)
    y = torch.zeros((M, N), dtype=torch.float32, device=dev)
    ws = torch.empty(fq.hcp_workspace_bytes(M, N, hot.numel()), dtype=torch.uint8, device=dev)
    for _ in range(reps):
        fq.hcp_residual_add(X, xq[0], xq[1], W, wq[0], wq[1], hot, y, workspace=ws)
    torch.cuda.synchronize()


def bench_tiny_ref(torch, fq, inputs, dev):
    """Tiny reference case: fp32 256x256 N(0,1) with 1% of entries x50, ROW
    blocks of 32, nearest-even; dequantize; DGE(k=5, clamp 3) backward on an
    N(0,1) gradient; the FP4 GEMM 256x256x256 of two such quantised
    matrices into fp32.  Each launch is a few microseconds of launch-bound
    work: timed as 20 launches captured in a HIP graph and replayed."""
    d = inputs.tiny_ref()
    A = torch.from_numpy(d["A"]).to(dev)
    B = torch.from_numpy(d["B"]).to(dev)
    G = torch.from_numpy(d["G"]).to(dev)
    aq = fq.quantize(A, 32)
    bq = fq.quantize(B, 32)
    y = torch.empty_like(A)
    c = torch.empty((256, 256), dtype=torch.float32, device=dev)
    out = {"shape": [256, 256, 256]}
    rep = 20
    ops = (("quant_row_rne", lambda: fq.quantize(A, 32, codes=aq[0], scales=aq[1]),
            256 * 256 * (4 + 0.5 + 1 / 32), 0),
           ("dequant", lambda: fq.dequantize(aq[0], aq[1], 32, out=y),
            256 * 256 * (4 + 0.5 + 1 / 32), 0),
           ("dge", lambda: fq.grad_estimate(fq.DGE, A, G, 32, fq.ROW, 5.0, 3.0, out=y),
            256 * 256 * 12, 0),
           ("gemm", lambda: fq.gemm(aq[0], aq[1], bq[0], bq[1], c=c),
            2 * 256 * 256 * (0.5 + 1 / 32) + 256 * 256 * 4, 2.0 * 256 ** 3))
    for name, fn, nbytes, nflops in ops:
        us = _graph_us(torch, [fn] * rep)
        d_ = {"us_graph": round(us, 2), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1)}
        if nflops:
            d_["TFLOPS"] = round(nflops / (us * 1e-6) / 1e12, 2)
        out[name] = d_
    return out


def bench_outlier_layer(torch, fq, inputs, dev):
    """13B-shaped outlier layer (X 16384x5120 with 461 hot channels x100, W
    5120x13824): X ROW and W COL quantisation, the fp32 base GEMM, the
    dual-kernel hot-channel residual, the single-kernel and split forms and
    the on-device hot-channel choice; 5 back-to-back launches each between
    one pair of events."""
    d = inputs.outlier_layer()
    M, K = d["X"].shape
    N = d["W"].shape[1]

    def to_bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    X, W = to_bf16(d["X"]), to_bf16(d["W"])
    hot = torch.from_numpy(d["hot"]).to(dev)
    xq = fq.quantize(X, 32, fq.ROW)
    wq = fq.quantize(W, 32, fq.COL)
    Y = torch.empty((M, N), dtype=torch.float32, device=dev)
    Y2 = torch.empty((M, N), dtype=torch.float32, device=dev)
    hmask = torch.empty(((K + 31) // 32,), dtype=torch.int32, device=dev)
    xs = (torch.empty_like(xq[0]), torch.empty_like(xq[1]))
    wsq = (torch.empty_like(wq[0]), torch.empty_like(wq[1]))
    ws = torch.empty(fq.hcp_workspace_bytes(M, N, hot.numel()), dtype=torch.uint8, device=dev)
    hsel = torch.empty_like(hot)
    hws = torch.empty(fq.hot_channels_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
    res = {}
    for name, fn in (("quant_x_row", lambda: fq.quantize(X, 32, fq.ROW, codes=xq[0], scales=xq[1])),
                     ("quant_w_col", lambda: fq.quantize(W, 32, fq.COL, codes=wq[0], scales=wq[1])),
                     ("gemm_fp32", lambda: fq.gemm(xq[0], xq[1], wq[0], wq[1], c=Y)),
                     ("hcp_residual", lambda: fq.hcp_residual_add(X, xq[0], xq[1], W, wq[0], wq[1],
                                                                  hot, Y, ws)),
                     ("gemm_hcp_single", lambda: fq.gemm_hcp(X, xq[0], xq[1], W, wq[0], wq[1], hot,
                                                             y=Y2, workspace=ws)),
                     ("hcp_split_masks_quant", lambda: (
                         fq.channel_mask(hot, K, out=hmask),
                         fq.quantize_masked(X, hmask, 32, fq.ROW, codes=xs[0], scales=xs[1]),
                         fq.quantize_masked(W, hmask, 32, fq.COL, codes=wsq[0], scales=wsq[1]))),
                     ("gemm_hcp_split", lambda: fq.gemm_hcp_split(X, xs[0], xs[1], W, wsq[0], wsq[1],
                                                                 hot, y=Y2, workspace=ws)),
                     ("hot_channels", lambda: fq.hot_channels(X, hot.numel(), hot_idx=hsel,
                                                              workspace=hws)),
                     # the floor of the residual's C traffic: a plain
                     # elementwise read-modify-write of the same fp32 Y
                     ("y_plain_rmw", lambda: Y2.add_(1.0))):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        reps = 5
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name + "_us"] = round(e0.elapsed_time(e1) * 1e3 / reps, 1)
    res["gemm_TFLOPS"] = round(2.0 * M * N * K / (res["gemm_fp32_us"] * 1e-6) / 1e12, 1)
    res["gemm_frac_fp4_peak"] = round(res["gemm_TFLOPS"] / PEAK_FP4_TFLOPS, 4)
    qb = 2.53125
    res["quant_x_row_GBps"] = round(M * K * qb / (res["quant_x_row_us"] * 1e-6) / 1e9, 1)
    res["quant_w_col_GBps"] = round(K * N * qb / (res["quant_w_col_us"] * 1e-6) / 1e9, 1)
    res["quant_x_row_frac_hbm_peak"] = round(res["quant_x_row_GBps"] / PEAK_HBM_GBPS, 4)
    res["quant_w_col_frac_hbm_peak"] = round(res["quant_w_col_GBps"] / PEAK_HBM_GBPS, 4)
    res["hcp_n_hot"] = int(hot.numel())
    # the choice reads X once (bf16); the partial-sum rows are small beside it
    res["hot_channels_GBps"] = round(2.0 * M * K / (res["hot_channels_us"] * 1e-6) / 1e9, 1)
    res["hot_channels_match_planted"] = bool(torch.equal(hsel, hot))
    # D mode: the residual's floor is the fp32 read-modify-write of Y (8 B per
    # output) plus the gathered operands written and read once
    kp = (2 * int(hot.numel()) + 31) // 32 * 32
    hcp_bytes = 8.0 * M * N + 2.0 * 2.0 * (M + N) * kp
    res["hcp_residual_GBps"] = round(hcp_bytes / (res["hcp_residual_us"] * 1e-6) / 1e9, 1)
    res["hcp_residual_frac_hbm_peak"] = round(res["hcp_residual_GBps"] / PEAK_HBM_GBPS, 4)
    res["hcp_y_rmw_GBps"] = round(8.0 * M * N / (res["hcp_residual_us"] * 1e-6) / 1e9, 1)
    res["y_plain_rmw_GBps"] = round(8.0 * M * N / (res["y_plain_rmw_us"] * 1e-6) / 1e9, 1)
    # dual-kernel mode (base GEMM, then the residual's read-modify-write of Y)
    # against the single kernel that writes Y once
    res["hcp_two_kernel_total_us"] = round(res["gemm_fp32_us"] + res["hcp_residual_us"], 1)
    res["gemm_hcp_single_flops"] = 2.0 * M * N * K + 2.0 * M * N * kp
    res["gemm_hcp_single_TFLOPS"] = round(res["gemm_hcp_single_flops"] /
                                          (res["gemm_hcp_single_us"] * 1e-6) / 1e12, 1)
    return res


def cpu_baseline(f, b, step_flops, budget_s):
    """The CPU oracle (single-threaded, untuned) on a bounded sample of the
    same step: every quantize/dequantize/DGE on a row slab, each GEMM on a
    row slab of its output, all extrapolated linearly to the full step."""
    import oracle as orc
    M, K = f["X"].shape
    N = f["W"].shape[1]
    X, W, dY = f["X"], f["W"], b["dY"]
    rows = max(8, int(64 * budget_s / 20.0))
    t = {}

    def timed(key, scale, fn):
        t0 = time.perf_counter()
        r = fn()
        t[key] = (time.perf_counter() - t0) * scale
        return r

    xs, dys = X[:rows], dY[:rows]
    xr = timed("quant_x_row", M / rows, lambda: orc.quantize(xs, 32))
    wc = timed("quant_w_col", 1.0, lambda: orc.quantize(W, 32, axis=orc.COL))
    timed("dequant_x", M / rows, lambda: orc.dequantize(xr[0], xr[1], 32))
    dyr = timed("quant_dy_row_sr", M / rows, lambda: orc.quantize(dys, 32, round=orc.SR,
                                                                   seed=SR_SEED))
    wr = timed("quant_w_row", 1.0, lambda: orc.quantize(W, 32))
    # column quantisation of a 32-row slab of the transposed operands' sources
    timed("quant_x_col", M / 32, lambda: orc.quantize(X[:32], 32, axis=orc.COL))
    timed("quant_dy_col_sr", M / 32, lambda: orc.quantize(dY[:32], 32, axis=orc.COL,
                                                          round=orc.SR, seed=SR_SEED))
    g = 4
    timed("gemm_fwd", M / g, lambda: orc.gemm(xr[0][:g], xr[1][:g], wc[0], wc[1]))
    timed("gemm_dx", M / g, lambda: orc.gemm(dyr[0][:g], dyr[1][:g], wr[0], wr[1]))
    xc32 = orc.quantize(np.ascontiguousarray(X[:, :g]), 32, axis=orc.COL)
    dyc = orc.quantize(dY[:, :256], 32, axis=orc.COL, round=orc.SR, seed=SR_SEED)
    timed("gemm_dw", (K / g) * (N / 256), lambda: orc.gemm(xc32[0], xc32[1], dyc[0], dyc[1]))
    gw = np.zeros((32, N), np.float32)
    timed("dge_dw", K / 32, lambda: orc.grad_estimate(orc.DGE, W[:32], gw, 32, orc.COL))
    total = sum(t.values())
    return {"value": round(step_flops / total / 1e12, 6), "unit": "TFLOPS", "cores": 1,
            "kind": "oracle",
            "sample": f"single-threaded C oracle (double precision) on row slabs of the step's "
                      f"tensors ({rows} rows for row ops, 32 rows for column ops, {g} output "
                      f"rows/cols per GEMM), extrapolated linearly to one full step; "
                      f"est. step {total:.1f} s",
            "est_step_s": round(total, 2),
            "per_kernel_est_s": {k: round(v, 3) for k, v in t.items()},
            "host_cpus": os.cpu_count()}


if __name__ == "__main__":
    main()
