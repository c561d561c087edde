#!/usr/bin/env python3
"""Benchmark of the dynamic mixed-precision quantized linear layer on one MI355X.

One step is one pass of the whole hot path over a CogVideoX-5B-like batch
(17776 tokens, hidden 3072, FFN 12288) of four DiT blocks:
  1. the Purified Delta Refresh outlier count of every block input (kappa=4;
     the synthetic inputs have a ratio near 0.7%, below rho=1%, so no block is
     forced to BF16), one device->host copy of it and of every block's Gamma
     sums, then the host router.  The Gamma sums S1, S2 of a block's input and
     output at the previous step are what that step's TDC refresh computed
     (--gamma standalone adds a dmpq_gamma_sums call per block instead).  The
     router computes
     E = alpha*Gamma+beta (alpha=1, beta=0, tau=0.2; the synthetic blocks have
     Gamma ~ 0.05, 0.40, 0.05, 0.40, so two blocks route to INT8 and two to
     NVFP4) and the PDR decision;
  2. per block, per linear (qkv 9216x3072, out 3072x3072, ffn_up 12288x3072,
     ffn_down 3072x12288): Hadamard + activation quant at the routed
     precision, then the quantized GEMM against the offline NVFP4 weights
     (with the GEMM workspace, so the last partial wave of tiles is split
     along K);
     an INT8-routed linear first converts its NVFP4 weight to INT8 into one
     shared scratch buffer (only the 4.5-bit weights are kept);
     with --fuse-ffn on, ffn_down consumes ffn_up's output instead: the
     ffn_up GEMM applies GELU in its epilogue and, when ffn_down is routed to
     NVFP4, also leaves the per-tile Hadamard amax that lets ffn_down's
     quantizer skip its amax pass (this adds the GELU's work to the step);
  3. per block, the Temporal Delta Cache refresh (delta, four L1 sums).
Inputs are synthetic (seeded, drawn on the device) and resident in HBM
before timing; weights are prepared once, outside the timed region.

Prints one JSON line.  value = qGEMM tera-ops per second of the whole step
(all GEMM ops of the step / step wall time).  Inside the timed region HIP
events on the launch stream bracket the calls of the GEMM with the most time
in the warmup steps (the dominant kernel), which give its per-launch duration
(the roofline); the per-kernel table comes from as many further steps with
events around every call.  An event record leaves the GPU idle for a few
microseconds, so the timed region keeps them few and uses events without the
system-scope fence.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_GBPS = 8000.0          # MI355X HBM3E peak
PEAK_INT8_TOPS = 5000.0    # dense int8 MFMA
PEAK_FP4_TFLOPS = 10100.0  # dense fp4 MFMA
PEAK_BF16_TFLOPS = 2500.0  # dense bf16 MFMA (the pipe the exact NVFP4 GEMM runs on)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--out-dtype", choices=["bf16", "f32"], default="bf16",
                   help="GEMM output type (bf16 feeds the next layer; f32 is the parity contract)")
    p.add_argument("--int8-weights", choices=["convert", "stored"], default="convert",
                   help="convert: only NVFP4 weights are kept and an INT8-routed linear converts its "
                        "weight into one scratch buffer right before its GEMM (the method's weight "
                        "handling); stored: use INT8 weights prepared offline")
    p.add_argument("--pdr", default="4,0.01", metavar="KAPPA,RHO",
                   help="Purified Delta Refresh check of every block input ('off' to skip it); "
                        "a block above rho runs its linears as BF16 GEMMs")
    p.add_argument("--gamma", choices=["refresh", "standalone"], default="refresh",
                   help="where the router's Gamma sums S1, S2 come from: the previous step's TDC "
                        "refresh of the block, which computes them over the same tensors "
                        "(default; the first step finds Gamma missing and routes INT8), or a "
                        "dmpq_gamma_sums call per block at the step start")
    p.add_argument("--fuse-ffn", choices=["on", "off"], default="off",
                   help="on: ffn_down's input is ffn_up's output, GELU and the next NVFP4 amax are "
                        "fused into ffn_up's GEMM epilogue (needs --out-dtype bf16); off: every "
                        "linear reads its own synthetic input (the linears alone)")
    p.add_argument("--tail-split", choices=["on", "off"], default="on",
                   help="on: the GEMMs get the full workspace, so the last partial wave of tiles is "
                        "split along K; off: a workspace with room for the fused-amax maxima only")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--events", choices=["nofence", "torch"], default="nofence",
                   help="timing events: HIP events without the system-scope fence (default), "
                        "or default torch.cuda events")
    p.add_argument("--cpu-rows", type=int, default=512,
                   help="rows of the qkv linear the oracle runs for the CPU baseline")
    p.add_argument("--calibrate-mib", type=int, default=0,
                   help="before warmup, run the TDC skip kernel (a plain streaming kernel: two "
                        "reads and one write per element) 3 times over buffers of this many MiB, "
                        "the known-size reference for the HBM byte counters")
    p.add_argument("--summarize-stats", nargs=2, metavar=("KERNEL_STATS_CSV", "OUT_MD"),
                   help="(no GPU) write the markdown summary of a rocprofv3 --stats run")
    p.add_argument("--summarize-traffic", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_JSON"),
                   help="(no GPU) turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of "
                        "'bench.py --calibrate-mib N' into per-launch HBM bytes of the GEMMs")
    p.add_argument("--command", default="",
                   help="the command that produced the csv, recorded in the summary")
    return p.parse_args()


class HipTimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence:
    recording it skips the system-scope cache writeback and invalidation that
    a default event performs, which otherwise leaves the GPU idle for several
    microseconds at every record.  Same record / elapsed_time interface as
    torch.cuda.Event; recorded on torch's current stream.  Reading a time
    needs a device synchronization first (the bench synchronizes before it
    reads any)."""
    DISABLE_SYSTEM_FENCE = 0x20000000
    _hip = None

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import ctypes as C
            # the HIP runtime this process already uses (torch's), not a second copy
            path = None
            with open("/proc/self/maps") as f:
                for line in f:
                    if "libamdhip64.so" in line:
                        path = line.split()[-1]
                        break
            if path is None:
                raise RuntimeError("libamdhip64 is not loaded in this process")
            h = C.CDLL(path)
            h.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
            h.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
            h.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
            h.hipEventDestroy.argtypes = [C.c_void_p]
            cls._hip = h
        return cls._hip

    def __init__(self, torch):
        import ctypes as C
        self.torch = torch
        self.ev = C.c_void_p()
        if self._lib().hipEventCreateWithFlags(C.byref(self.ev), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self):
        if self._lib().hipEventRecord(self.ev, self.torch.cuda.current_stream().cuda_stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end) -> float:
        import ctypes as C
        ms = C.c_float()
        if self._lib().hipEventElapsedTime(C.byref(ms), self.ev, end.ev) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.ev:
            self._hip.hipEventDestroy(self.ev)


class KernelTimer:
    """HIP events around library calls on the current stream.  The events are
    created before timing starts (prepare), so a timed call costs only its two
    event records; `only` restricts the events to the named calls (None: every
    call).  Event records are not free, so the timed region brackets only the
    GEMM calls and a separate pass times every call.  kind "nofence": timing
    events without the system-scope fence (HipTimingEvent); "torch": default
    torch.cuda events."""

    def __init__(self, torch, kind="nofence"):
        self.torch = torch
        self.kind = kind
        self.rec = {}
        self.on = False
        self.only = None
        self.calls = 0          # calls that would be timed, counted while off
        self.pool = []

    def _event(self):
        if self.kind == "torch":
            return self.torch.cuda.Event(enable_timing=True)
        return HipTimingEvent(self.torch)

    def prepare(self, n):
        self.pool = [(self._event(), self._event()) for _ in range(n)]
        self.pool.reverse()
        self.rec = {}

    def __call__(self, name, work, fn, *a, _shape=None, **kw):
        timed = self.only is None or name in self.only
        if not self.on or not timed:
            self.calls += timed
            fn(*a, **kw)
            return
        if self.pool:
            s, e = self.pool.pop()
        else:
            s, e = self._event(), self._event()
        s.record()
        fn(*a, **kw)
        e.record()
        self.rec.setdefault(name, []).append((s, e, work, _shape))

    def summary(self, steps, by_shape=False):
        groups = {}
        for name, lst in self.rec.items():
            for rec in lst:
                key = (name, rec[3]) if by_shape else name
                groups.setdefault(key, []).append(rec)
        out = {}
        for key, lst in groups.items():
            ms = [s.elapsed_time(e) for s, e, _, _ in lst]
            work = sum(w for _, _, w, _ in lst)
            out[key] = dict(calls_per_step=len(lst) / steps, total_ms=sum(ms),
                            avg_us=1e3 * sum(ms) / len(ms),
                            median_us=1e3 * sorted(ms)[len(ms) // 2], work=work)
        return out


def main():
    args = parse()
    if args.summarize_stats:
        summarize_stats(*args.summarize_stats, args.command)
        return
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, args.command)
        return
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} requested, but the benchmark runs on one GPU only "
              "(the hot path is token-parallel; sharding it over GPUs is not implemented)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import dynamic_mixed_precision_amd as dm
    import workloads as wl

    dm.lib()
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    cfg = wl.COGVIDEOX_5B
    M, H = cfg.M, cfg.hidden
    out_dtype = dm.OUT_BF16 if args.out_dtype == "bf16" else dm.OUT_F32
    ydt = torch.bfloat16 if out_dtype == dm.OUT_BF16 else torch.float32
    n_blocks = len(wl.GAMMA_TARGETS_5B)
    alpha = np.full(len(cfg.linears), wl.ROUTER_5B["alpha"])
    beta = np.full(len(cfg.linears), wl.ROUTER_5B["beta"])
    tau = wl.ROUTER_5B["tau"]

    pdr = None if args.pdr == "off" else tuple(float(v) for v in args.pdr.split(","))

    # ---- inputs and offline weight prep (untimed) -----------------------------
    t0 = time.time()
    blocks = []
    ws_prep = dm.new_workspace(dm.OP_PREP_WEIGHT)
    for b in range(n_blocks):
        gen = wl.device_generator(cfg.seeds[b])
        x_in = wl.activations_device(gen, M, H)
        x_out = wl.perturbed_output_device(gen, x_in, wl.GAMMA_TARGETS_5B[b])
        lins = []
        for lin in cfg.linears:
            x = wl.activations_device(gen, M, lin.K)
            w = wl.weight_device(gen, lin.N, lin.K)
            pw = dict(cw=torch.empty((lin.N, lin.K // 2), dtype=torch.uint8, device="cuda"),
                      sw=torch.empty((lin.N, lin.K // 16), dtype=torch.uint8, device="cuda"),
                      gw=torch.zeros(1, device="cuda"),
                      qw=torch.empty((lin.N, lin.K), dtype=torch.int8, device="cuda"),
                      swr=torch.empty(lin.N, device="cuda"))
            dm.prep_weight(w, pw["cw"], pw["sw"], pw["gw"], pw["qw"], pw["swr"], ws_prep)
            pw["w"] = w.view(torch.int16) if pdr is not None else None
            del w
            lins.append(dict(lin=lin, x=x, **pw))
        blocks.append(dict(x_in=x_in, x_out=x_out, lins=lins,
                           delta=torch.empty_like(x_in), delta_valid=False))
    ks = sorted({lin.K for lin in cfg.linears})
    qbuf = {K: dict(q=torch.empty((M, K), dtype=torch.int8, device="cuda"),
                    s=torch.empty(M, device="cuda"),
                    c=torch.empty((M, K // 2), dtype=torch.uint8, device="cuda"),
                    sc=torch.empty((M, K // 16), dtype=torch.uint8, device="cuda"),
                    g=torch.zeros(1, device="cuda")) for K in ks}
    ybuf = {lin.name: torch.empty((M, lin.N), dtype=ydt, device="cuda") for lin in cfg.linears}
    big = max(lin.N * lin.K for lin in cfg.linears)
    w8_scratch = torch.empty(big, dtype=torch.int8, device="cuda")
    s8_scratch = torch.empty(max(lin.N for lin in cfg.linears), device="cuda")
    ws = dm.new_workspace(dm.OP_TDC)
    # per block, one 64-byte row (every device pointer stays 16-byte aligned):
    # [0:4] the TDC refresh's S1..S4, [4:6] the standalone Gamma sums S1, S2,
    # [6] the PDR outlier count.  One device-to-host copy per step.
    sums = torch.zeros((n_blocks, 8), dtype=torch.float64, device="cuda")
    sums_host = torch.zeros((n_blocks, 8), dtype=torch.float64).pin_memory()
    sums_np = sums_host.numpy()  # the same pinned memory: numpy indexing costs far less on the host
    refreshed = [False] * n_blocks  # the block's refresh sums are from the previous step
    ws_out = dm.new_workspace(dm.OP_OUTLIER)
    fuse = args.fuse_ffn == "on"
    if fuse and out_dtype != dm.OUT_BF16:
        print("bench.py: --fuse-ffn on needs --out-dtype bf16", file=sys.stderr)
        sys.exit(2)
    names = [lin.name for lin in cfg.linears]
    i_up, i_down = names.index("ffn_up"), names.index("ffn_down")
    # the GEMMs' workspace: fused-amax maxima, then the split area of the
    # last partial wave of tiles (sized for the widest output)
    ws_gemm = dm.new_workspace(dm.OP_GEMM if args.tail_split == "on" else dm.OP_GEMM_AMAX, "cuda", M,
                               max(lin.N for lin in cfg.linears))
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    kt = KernelTimer(torch, args.events)
    pdr_ratio = [None] * n_blocks
    gemm_ops_step = 0
    routes_seen = []

    def step():
        nonlocal gemm_ops_step
        # 1. Gamma predictor + router: one device->host boundary per step.
        # Gamma's sums are the previous step's (the refresh computed them), or
        # with --gamma standalone a dmpq_gamma_sums call per block.
        for b, blk in enumerate(blocks):
            if args.gamma == "standalone":
                kt("gamma_sums", 4.0 * M * H, dm.gamma_sums, blk["x_in"], blk["x_out"], sums[b, 4:6], ws,
                   _shape=f"{M}x{H}")
            if pdr is not None:
                kt("outlier_count", 2.0 * M * H, dm.outlier_count, blk["x_in"].view(M, H), pdr[0],
                   sums[b, 6:7], ws_out, _shape=f"{M}x{H}")
        sums_host.copy_(sums, non_blocking=True)
        torch.cuda.current_stream().synchronize()
        if args.gamma == "standalone":
            routes = [dm.gate_and_route(sums_np[b, 4:6], alpha, beta, tau)[2] for b in range(n_blocks)]
        else:
            routes = [dm.gate_and_route(sums_np[b, 0:2] if refreshed[b] else None, alpha, beta, tau)[2]
                      for b in range(n_blocks)]
        if pdr is not None:
            for b in range(n_blocks):
                if dm.pdr_decide(float(sums_np[b, 6]), M * H, pdr[1]):
                    routes[b] = np.full(len(routes[b]), dm.ROUTE_BF16, np.uint8)
                pdr_ratio[b] = float(sums_np[b, 6]) / (M * H)
        ops = 0
        # 2. quantized linears at the routed precision
        for b, blk in enumerate(blocks):
            for li, L in enumerate(blk["lins"]):
                lin = L["lin"]
                qb = qbuf[lin.K]
                flops = 2.0 * M * lin.N * lin.K
                ops += flops
                route = routes[b][li]
                gshape = f"{M}x{lin.N}x{lin.K}"
                x, epi, qflags, qws = L["x"], 0, 0, ws
                if fuse and li == i_up:
                    epi = dm.EPI_GELU
                    if routes[b][i_down] == dm.ROUTE_NVFP4:
                        epi |= dm.EPI_NVFP4_AMAX
                if fuse and li == i_down:
                    x = ybuf[names[i_up]].view(torch.int16)
                    if route == dm.ROUTE_NVFP4:
                        qflags, qws = dm.AMAX_GIVEN, ws_gemm
                if route == dm.ROUTE_BF16:
                    kt("gemm_bf16", flops, dm.gemm_bf16_ex, x.view(M, lin.K), L["w"], ybuf[lin.name],
                       epi, ws_gemm, out_dtype, _shape=gshape)
                elif route == dm.ROUTE_INT8:
                    kt("hadamard_quant_int8", 3.0 * M * lin.K + 4.0 * M,
                       dm.hadamard_quant_int8, x, qb["q"], qb["s"], _shape=f"{M}x{lin.K}")
                    qw, swr = L["qw"], L["swr"]
                    if args.int8_weights == "convert":
                        qw = w8_scratch[:lin.N * lin.K].view(lin.N, lin.K)
                        swr = s8_scratch[:lin.N]
                        kt("weight_int8_from_nvfp4", (0.5 + 1.0 / 16 + 1.0) * lin.N * lin.K + 8.0 * lin.N,
                           dm.weight_int8_from_nvfp4, L["cw"], L["sw"], L["gw"], qw, swr,
                           _shape=f"{lin.N}x{lin.K}")
                    kt("qgemm_int8", flops, dm.qgemm_int8_ex, qb["q"], qb["s"], qw, swr,
                       ybuf[lin.name], epi, ws_gemm, out_dtype, _shape=gshape)
                else:
                    kt("hadamard_quant_nvfp4_given" if qflags else "hadamard_quant_nvfp4",
                       (2.0 + 0.5 + 1.0 / 16) * M * lin.K + 4.0,
                       dm.hadamard_quant_nvfp4, x, qb["c"], qb["sc"], qb["g"], qws, qflags,
                       _shape=f"{M}x{lin.K}")
                    kt("qgemm_nvfp4", flops, dm.qgemm_nvfp4_ex, qb["c"], qb["sc"], qb["g"], L["cw"],
                       L["sw"], L["gw"], ybuf[lin.name], epi, ws_gemm, out_dtype, _shape=gshape)
            # 3. Temporal Delta Cache refresh of the block
            kt("tdc_step_refresh", 8.0 * M * H, dm.tdc_step, dm.TDC_REFRESH, blk["x_in"],
               blk["x_out"], blk["delta"], blk["delta_valid"], sums[b, 0:4], ws, _shape=f"{M}x{H}")
            blk["delta_valid"] = True
            refreshed[b] = True
        gemm_ops_step = ops
        routes_seen.append([r.tolist() for r in routes])  # bookkeeping, off the sync-to-launch path

    calib = None
    if args.calibrate_mib > 0:
        n = args.calibrate_mib * (1 << 20) // 2
        cx = torch.zeros(n, dtype=torch.int16, device="cuda")
        cd = torch.zeros(n, dtype=torch.int16, device="cuda")
        co = torch.empty(n, dtype=torch.int16, device="cuda")
        for _ in range(3):
            dm.tdc_step(dm.TDC_SKIP, cx, co, cd, True)
        torch.cuda.synchronize()
        del cx, cd, co
        calib = dict(kernel=CALIB_KERNEL, elements=n, read_bytes=4 * n, write_bytes=2 * n)

    # After the warmup steps, one more step brackets the GEMM calls (the
    # dominant-kernel candidates) with events; the timed region then
    # brackets only the calls of the one with the most time in that step,
    # since every event record leaves the GPU idle for a few microseconds.
    # (The first step routes every block to INT8, Gamma being missing, so
    # the choice is made once the routes have settled.)  Every other call
    # runs without events.
    for _ in range(args.warmup):
        step()
    kt.only = GEMM_CALLS
    kt.on = True
    step()
    torch.cuda.synchronize()
    kt.on = False
    warm = kt.summary(1)
    if warm:
        kt.only = {max(warm, key=lambda n: warm[n]["total_ms"])}
    kt.calls = 0
    step()  # counts the calls to bracket per step (one more untimed step)
    kt.prepare(kt.calls * args.steps)
    torch.cuda.synchronize()
    kt.on = True
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    kt.on = False
    ms_per_step = 1e3 * elapsed / args.steps
    value = gemm_ops_step / (elapsed / args.steps) / 1e12
    ktimed = kt.summary(args.steps)

    # ---- per-kernel figures: events on every call, in as many extra steps -----
    kt.only = None
    kt.calls = 0
    step()
    kt.prepare(kt.calls * args.steps)
    torch.cuda.synchronize()
    kt.on = True
    for _ in range(args.steps):
        step()
    if args.gamma == "refresh":
        # the standalone Gamma sums, outside the step (the refresh provides
        # them there), timed per block for the per-kernel table
        for _ in range(args.steps):
            for b, blk in enumerate(blocks):
                kt("gamma_sums_standalone", 4.0 * M * H, dm.gamma_sums, blk["x_in"], blk["x_out"],
                   sums[b, 4:6], ws, _shape=f"{M}x{H}")
    torch.cuda.synchronize()
    kt.on = False
    ksum = kt.summary(args.steps)
    kshape = kt.summary(args.steps, by_shape=True)
    peaks = {"hadamard_quant_int8": ("hbm", HBM_GBPS, "GB/s"),
             "weight_int8_from_nvfp4": ("hbm", HBM_GBPS, "GB/s"),
             "outlier_count": ("hbm", HBM_GBPS, "GB/s"),
             "gemm_bf16": ("mfma", PEAK_BF16_TFLOPS, "TFLOP/s"),
             "hadamard_quant_nvfp4": ("hbm", HBM_GBPS, "GB/s"),
             "hadamard_quant_nvfp4_given": ("hbm", HBM_GBPS, "GB/s"),
             "gamma_sums": ("hbm", HBM_GBPS, "GB/s"),
             "gamma_sums_standalone": ("hbm", HBM_GBPS, "GB/s"),
             "tdc_step_refresh": ("hbm", HBM_GBPS, "GB/s"),
             "qgemm_int8": ("mfma", PEAK_INT8_TOPS, "TOPS"),
             "qgemm_nvfp4": ("mfma", PEAK_FP4_TFLOPS, "TFLOP/s")}
    kernels = {}
    for name, s in ksum.items():
        bound, peak, unit = peaks[name]
        scale = 1e-9 if unit == "GB/s" else 1e-12
        achieved = s["work"] * scale / (s["total_ms"] * 1e-3)
        kernels[name] = dict(calls_per_step=s["calls_per_step"], avg_us=round(s["avg_us"], 2),
                             median_us=round(s["median_us"], 2), achieved=round(achieved, 2), unit=unit,
                             bound=bound, peak=peak, frac=round(achieved / peak, 4))
        if name == "qgemm_nvfp4":
            kernels[name]["frac_of_bf16_pipe"] = round(achieved / PEAK_BF16_TFLOPS, 4)
    by_shape = {}
    for (name, shape), s in sorted(kshape.items()):
        bound, peak, unit = peaks[name]
        achieved = s["work"] * (1e-9 if unit == "GB/s" else 1e-12) / (s["total_ms"] * 1e-3)
        by_shape[f"{name} {shape}"] = dict(calls_per_step=s["calls_per_step"], median_us=round(s["median_us"], 2),
                                           achieved=round(achieved, 2), unit=unit,
                                           frac=round(achieved / peak, 4))
    dom = max(ksum, key=lambda n: ksum[n]["total_ms"])
    d = kernels[dom]
    if dom in ktimed:  # the dominant kernel as timed inside the timed region
        t = ktimed[dom]
        ach = t["work"] * (1e-9 if d["unit"] == "GB/s" else 1e-12) / (t["total_ms"] * 1e-3)
        d = dict(d, achieved=round(ach, 2), frac=round(ach / d["peak"], 4), avg_us=round(t["avg_us"], 2))
    roofline = dict(kernel=dom, bound=d["bound"], achieved=d["achieved"], peak=d["peak"],
                    unit=d["unit"], frac=d["frac"], traffic=None, avg_us_per_call=d["avg_us"],
                    timed_in="timed region" if dom in ktimed else "per-kernel pass")
    if dom == "qgemm_nvfp4":  # exact NVFP4 runs on the fp16 pipe: its share of that peak too
        roofline["frac_of_fp16_pipe"] = round(d["achieved"] / PEAK_BF16_TFLOPS, 4)
    roofline.update(measured_traffic(dom))
    q_bytes = sum(ksum[n]["work"] for n in ksum if n.startswith("hadamard_quant"))
    q_ms = sum(ksum[n]["total_ms"] for n in ksum if n.startswith("hadamard_quant"))

    result = {
        "metric": "qGEMM TOPS (INT8/NVFP4) + act-quant GB/s at 17.8k-token×3072 DiT shapes",
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+nvfp4",
        "data": "synthetic",
        "config": {"workload": "cogvideox5b-like: 4 DiT blocks x 4 routed linears "
                               "(qkv 9216x3072, out 3072x3072, ffn_up 12288x3072, "
                               "ffn_down 3072x12288), 17776 tokens, hidden 3072",
                   "tokens": M, "hidden": H, "blocks": n_blocks,
                   "routes_per_block": [{0: "NVFP4", 1: "INT8", 2: "BF16"}[r[0]] for r in routes_seen[-1]],
                   "pdr": None if pdr is None else {"kappa": pdr[0], "rho": pdr[1],
                                                    "outlier_ratio_per_block": [round(v, 5) for v in pdr_ratio]},
                   "gemm_out": args.out_dtype,
                   "int8_weights": args.int8_weights,
                   "gamma_sums": ("the previous step's TDC refresh" if args.gamma == "refresh"
                                  else "dmpq_gamma_sums at the step start"),
                   "ffn_fused": fuse,
                   "tail_split": args.tail_split == "on",
                   "gemm_tera_ops_per_step": round(gemm_ops_step / 1e12, 3)},
        "act_quant_GBps": round(q_bytes * 1e-9 / (q_ms * 1e-3), 1),
        "kernels": kernels,
        "kernels_note": ("per-call HIP events on every call, in as many untimed steps after the timed "
                         "region; gamma_sums_standalone is timed beside those steps, not in them"),
        "timing_events": ("HIP events without the system-scope fence" if args.events == "nofence"
                          else "torch.cuda events"),
        "kernels_by_shape": by_shape,
        "roofline": roofline,
        "setup_s": round(setup_s, 1),
    }
    if calib is not None:
        result["copy_calibration"] = calib
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.cpu_rows)
    print(json.dumps(result), flush=True)


def cpu_baseline(rows: int) -> dict:
    """The oracle (plain C, OpenMP over rows) on a bounded sample: Hadamard +
    quant and the GEMM for `rows` tokens of the qkv linear (9216 x 3072), on
    both routes (the step's ops are half INT8, half NVFP4)."""
    import numpy as np

    import oracle as orc
    import workloads as wl

    rng = np.random.default_rng(6)
    N, K = 9216, 3072
    x = wl.activations(rng, rows, K)
    w = wl.weight(rng, N, K)
    p = orc.prep_weight(w)
    t = time.perf_counter()
    qa, sa = orc.quant_int8(x)
    orc.gemm_int8(qa, sa, p["qw"], p["sw_row"])
    ca, sca, ga = orc.quant_nvfp4(x)
    orc.gemm_nvfp4(ca, sca, ga, p["cw"], p["sw"], p["gw"])
    dt = time.perf_counter() - t
    ops = 2 * (2.0 * rows * N * K)
    return {"value": round(ops / dt / 1e12, 6), "unit": "TOPS", "cores": orc.max_threads(),
            "kind": "oracle",
            "sample": f"{rows} tokens of the qkv linear ({N}x{K}), INT8 and NVFP4 routes, "
                      f"quant + GEMM, {dt:.1f} s"}


# ---- HBM byte counters and profile summaries ---------------------------------
# The kernels behind each timed entry point and the sources they are built from:
# a stored traffic figure is used only while these sources are unchanged.
# The kernels of one GEMM call (bf16 output, every epilogue; '*' matches a
# template argument): the whole-tile DMA kernel, which every call of the
# step runs once, and the split and fixup kernels of its tail.
# library calls bracketed by events inside the timed region
GEMM_CALLS = ("qgemm_nvfp4", "qgemm_int8", "gemm_bf16")

GEMM_KERNELS = {"qgemm_nvfp4": ["dmpq::gemm_fp4_dma_kernel<1, *>", "dmpq::gemm_fp4_split_kernel",
                                "dmpq::gemm_f32_fixup_kernel<1, *, *>"],
                "qgemm_int8": ["dmpq::gemm_i8_dma_kernel<1, *>", "dmpq::gemm_i8_split_kernel",
                               "dmpq::gemm_i8_fixup_kernel<1, *, *>"]}
GEMM_SOURCES = {"qgemm_nvfp4": ["gemm_nvfp4.hip", "gemm_bf16.hip", "gemm_common.hpp", "device.hpp",
                                "internal.hpp"],
                "qgemm_int8": ["gemm_int8.hip", "gemm_dma.hpp", "gemm_common.hpp", "device.hpp",
                               "internal.hpp"]}
CALIB_KERNEL = "dmpq::tdc_skip_kernel"
HERE = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_JSON = os.path.join(HERE, "profiles", "traffic_qgemm_cogvideox5b.json")


def sources_sha256(api: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES[api]:
        with open(os.path.join(HERE, "dynamic_mixed_precision_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def gemm_algorithmic_bytes(api: str) -> float:
    """Average compulsory bytes of one GEMM launch of the step: operands once
    (codes + scales) and the bf16 output once, over the four linear shapes."""
    import workloads as wl
    cfg = wl.COGVIDEOX_5B
    M = cfg.M
    tot = 0.0
    for lin in cfg.linears:
        N, K = lin.N, lin.K
        if api == "qgemm_nvfp4":
            tot += (M + N) * (K / 2 + K / 16) + 8
        else:
            tot += (M + N) * (K + 4)
        tot += 2.0 * M * N
    return tot / len(cfg.linears)


def measured_traffic(api: str) -> dict:
    """traffic = counter-measured HBM bytes per launch (calibrated), or None
    when no measurement exists or the kernel's sources changed since."""
    out = {"traffic_unit": "bytes/launch"}
    if api not in GEMM_KERNELS:
        return out
    out["algorithmic_bytes_per_launch"] = round(gemm_algorithmic_bytes(api))
    if not os.path.exists(TRAFFIC_JSON):
        return out
    with open(TRAFFIC_JSON) as f:
        rec = json.load(f).get(api)
    if rec is None or rec["sources_sha256"] != sources_sha256(api):
        out["traffic_note"] = "kernel changed since the counters were taken"
        return out
    out["traffic"] = rec["bytes_per_launch"]
    out["traffic_over_algorithmic"] = round(rec["bytes_per_launch"] / out["algorithmic_bytes_per_launch"], 3)
    return out


def _counter_rows(path: str, counter: str):
    import csv
    with open(path) as f:
        return [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]


def _kernel_re(kernel: str):
    import re
    return re.compile(re.escape(kernel).replace(r"\*", r"\d+") + r"\(")


def _per_kernel_kib(rows, kernel: str):
    """Counter value (KiB) of every dispatch of `kernel`, in dispatch order."""
    pat = _kernel_re(kernel)
    sel = {}
    for r in rows:
        if pat.search(r["Kernel_Name"]):
            sel[int(r["Dispatch_Id"])] = sel.get(int(r["Dispatch_Id"]), 0.0) + float(r["Counter_Value"])
    return [sel[k] for k in sorted(sel)]


def summarize_traffic(fetch_csv: str, write_csv: str, out_json: str, command: str) -> None:
    fr, wr = _counter_rows(fetch_csv, "FETCH_SIZE"), _counter_rows(write_csv, "WRITE_SIZE")
    cf, cw = _per_kernel_kib(fr, CALIB_KERNEL), _per_kernel_kib(wr, CALIB_KERNEL)
    if len(cf) != 3 or len(cw) != 3:
        raise SystemExit(f"expected 3 calibration dispatches, got {len(cf)}, {len(cw)}")
    # the calibration buffers' size is recorded in the command (--calibrate-mib N)
    mib = int(command.split("--calibrate-mib")[1].split()[0])
    n = mib * (1 << 20) // 2
    f_read = 4.0 * n / (1024.0 * sum(cf) / 3)
    f_write = 2.0 * n / (1024.0 * sum(cw) / 3)
    rec = {"command": command, "calibration": {
        "kernel": CALIB_KERNEL, "elements": n, "read_bytes": 4 * n, "write_bytes": 2 * n,
        "fetch_kib_per_dispatch": cf, "write_kib_per_dispatch": cw,
        "fetch_factor": round(f_read, 5), "write_factor": round(f_write, 5)}}
    for api, knames in GEMM_KERNELS.items():
        calls = len(_per_kernel_kib(fr, knames[0]))  # one whole-tile dispatch per call
        f = [v for k in knames for v in _per_kernel_kib(fr, k)]
        w = [v for k in knames for v in _per_kernel_kib(wr, k)]
        if not calls or len(f) != len(w):
            continue
        fb = 1024.0 * f_read * sum(f) / calls
        wb = 1024.0 * f_write * sum(w) / calls
        alg = gemm_algorithmic_bytes(api)
        rec[api] = {"kernels": knames, "calls": calls, "dispatches": len(f),
                    "sources_sha256": sources_sha256(api),
                    "fetch_kib_per_call_raw": round(sum(f) / calls, 1),
                    "write_kib_per_call_raw": round(sum(w) / calls, 1),
                    "fetch_bytes_per_launch": round(fb), "write_bytes_per_launch": round(wb),
                    "bytes_per_launch": round(fb + wb),
                    "algorithmic_bytes_per_launch": round(alg),
                    "traffic_over_algorithmic": round((fb + wb) / alg, 3)}
    with open(out_json, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


def summarize_stats(stats_csv: str, out_md: str, command: str) -> None:
    import csv
    import re
    with open(stats_csv) as f:
        rows = list(csv.DictReader(f))
    lines = ["# rocprofv3 kernel stats: bench.py step, CogVideoX-5B-like batch "
             "(17776 tokens, 4 blocks x 4 linears, 2 INT8 + 2 NVFP4 blocks)", "",
             "Command (run from /tmp, repository at $GRAFT_REPO_ROOT):", "", "```", command, "```", "",
             "| kernel | calls | avg us | min us | max us | share of GPU time |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        if "dmpq" not in r["Name"]:
            continue
        name = re.sub(r"\(.*", "", r["Name"]).replace("void ", "")
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f}% |")
    other = sum(float(r["Percentage"]) for r in rows if "dmpq" not in r["Name"])
    lines += ["", f"Other kernels (torch input generation, setup): {other:.1f}% of GPU time.", "",
              "Per GEMM call (whole-tile kernel, plus the split and fixup kernels of the tail; the",
              "bench's HIP events time the same span):", "",
              "| call | calls | kernels | us per call |", "|---|---|---|---|"]
    for api, knames in GEMM_KERNELS.items():
        pats = [_kernel_re(k) for k in knames]
        sel = [r for r in rows if any(p.search(r["Name"]) for p in pats)]
        calls = sum(int(r["Calls"]) for r in sel if pats[0].search(r["Name"]))
        if calls:
            tot = sum(int(r["Calls"]) * float(r["AverageNs"]) for r in sel) / 1e3
            lines.append(f"| {api} | {calls} | {len(sel)} | {tot / calls:.1f} |")
    lines.append("")
    with open(out_md, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


if __name__ == "__main__":
    main()
