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
     every linear reads its own synthetic input (the linears alone); with
     --fuse-ffn on, ffn_down reads GELU of ffn_up's output, as in a DiT FFN:
     the ffn_up GEMM applies GELU in its epilogue and, when ffn_down is
     routed to NVFP4, also leaves the per-tile Hadamard amax that lets
     ffn_down's quantizer skip its amax pass; --fuse-ffn separate runs that
     FFN with GELU as its own kernel and the two-pass quantizer (both forms
     are measured as extra keys);
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
import gc
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
    p.add_argument("--int8-weights", choices=["convert", "convert-separate", "stored"], default="convert",
                   help="convert: only NVFP4 weights are kept and an INT8-routed linear converts its "
                        "weight into one scratch buffer right before its GEMM (the method's weight "
                        "handling), in the same launch as its activation quantization; "
                        "convert-separate: the same conversion as a launch of its own; stored: use "
                        "INT8 weights prepared offline")
    p.add_argument("--pdr", default="4,0.01", metavar="KAPPA,RHO",
                   help="Purified Delta Refresh check of every block input ('off' to skip it); "
                        "a block above rho runs its linears as BF16 GEMMs")
    p.add_argument("--gamma", choices=["refresh", "standalone"], default="refresh",
                   help="where the router's Gamma sums S1, S2 come from: the previous step's TDC "
                        "refresh of the block, which computes them over the same tensors "
                        "(default; the first step finds Gamma missing and routes INT8), or a "
                        "dmpq_gamma_sums call per block at the step start")
    p.add_argument("--fuse-ffn", choices=["on", "separate", "off"], default="off",
                   help="on: ffn_down's input is GELU(ffn_up's output), with GELU and the next "
                        "NVFP4 tensor amax fused into ffn_up's GEMM epilogue, so an NVFP4-routed "
                        "ffn_down quantizes with the given amax and reads its input once (needs "
                        "--out-dtype bf16); separate: the same FFN with GELU as a separate kernel after "
                        "ffn_up and ffn_down's two-pass quantizer (the like-for-like unfused form); "
                        "off (default): every linear reads its own synthetic input (the linears alone)")
    p.add_argument("--tail-split", choices=["on", "off"], default="on",
                   help="on: the GEMMs get the full workspace, so the last partial wave of tiles is "
                        "split along K; off: a workspace with room for the fused-amax maxima only")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--extras", choices=["on", "off"], default="on",
                   help="on: after the headline, also measure the other workloads as labelled "
                        "extra keys (2B-like linears, 1080p-like all-INT8 and all-NVFP4 steps, the "
                        "42-block x 50-step TDC schedule), the headline kernels with the MALL "
                        "flushed before every call, and the oracle's 1-thread quantizers")
    p.add_argument("--extra-steps", type=int, default=3,
                   help="timed steps of each extra linear workload (after one warmup step)")
    p.add_argument("--graph", choices=["off", "on"], default="off",
                   help="on: after the host decisions, each step replays a HIP graph of its linears and "
                        "refreshes (captured once per routing); the timed region then carries no "
                        "per-call events and the roofline uses the per-kernel pass")
    p.add_argument("--host-sync", choices=["spin", "block"], default="spin",
                   help="the step's one wait for the device (the Gamma/PDR sums): poll an event "
                        "(spin) or a blocking stream synchronize (block)")
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
    p.add_argument("--summarize-counters", nargs="+", metavar="CSV_OR_OUT_MD",
                   help="(no GPU) OUT_MD then one or more rocprofv3 --pmc counter_collection CSVs of the "
                        "same bench command: per-kernel MFMA busy share, clock, VALU and LDS figures")
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
        self.flush = None       # called before each timed call (evicts the MALL)

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
        if self.flush is not None:
            self.flush()
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
    if args.summarize_counters:
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1:], args.command)
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
    from dynamic_mixed_precision_amd.schedule import spin_sync

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
    skip_out = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
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
    separate = args.fuse_ffn == "separate"
    if (fuse or separate) and out_dtype != dm.OUT_BF16:
        print("bench.py: --fuse-ffn on/separate needs --out-dtype bf16", file=sys.stderr)
        sys.exit(2)
    names = [lin.name for lin in cfg.linears]
    i_up, i_down = names.index("ffn_up"), names.index("ffn_down")
    gelu_buf = (torch.empty((M, cfg.linears[i_up].N), dtype=torch.bfloat16, device="cuda")
                if separate else None)
    # the GEMMs' workspace: fused-amax maxima, then the split area of the
    # last partial wave of tiles (sized for the widest output)
    ws_gemm = dm.new_workspace(dm.OP_GEMM if args.tail_split == "on" else dm.OP_GEMM_AMAX, "cuda", M,
                               max(lin.N for lin in cfg.linears))
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    kt = KernelTimer(torch, args.events)
    host_t = {"wait": 0.0, "decide": 0.0}  # host seconds in the per-step wait and the decisions after it
    pdr_ratio = [None] * n_blocks
    gemm_ops_step = 0
    routes_seen = []

    def step(eager=False):
        # eager: issue per call even in graph mode (a step that counts the
        # timer's calls must go through them)
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
        t_wait = time.perf_counter()
        if args.host_sync == "spin":
            spin_sync()
        else:
            torch.cuda.current_stream().synchronize()
        t_decide = time.perf_counter()
        host_t["wait"] += t_decide - t_wait
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
        host_t["decide"] += time.perf_counter() - t_decide
        if args.graph == "on" and not kt.on and not eager:
            # the issue below, captured once per routing (after one eager
            # pass, which does the library's one-time set-up) and replayed
            key = (tuple(tuple(r.tolist()) for r in routes), tuple(blk["delta_valid"] for blk in blocks))
            if key in graphs:
                g, ops = graphs[key]
                g.replay()
            elif key in seen_eager:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    ops = issue(routes)
                graphs[key] = (g, ops)
                g.replay()  # capture only records the work
            else:
                ops = issue(routes)
                seen_eager.add(key)
        else:
            ops = issue(routes)
        gemm_ops_step = ops
        routes_seen.append([r.tolist() for r in routes])  # bookkeeping, off the sync-to-launch path

    graphs, seen_eager = {}, set()

    def issue(routes):
        """Everything after the step's host decisions: the routed linears and
        the TDC refresh of every block; returns the step's GEMM ops."""
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
                if separate and li == i_down:
                    # GELU as its own kernel (torch, exact erf form, bf16 in and out)
                    yu = ybuf[names[i_up]]
                    kt("gelu_separate", 4.0 * yu.numel(), torch.ops.aten.gelu.out, yu, approximate="none",
                       out=gelu_buf, _shape=f"{M}x{yu.shape[1]}")
                    x = gelu_buf.view(torch.int16)
                if route == dm.ROUTE_BF16:
                    kt("gemm_bf16", flops, dm.gemm_bf16_ex, x.view(M, lin.K), L["w"], ybuf[lin.name],
                       epi, ws_gemm, out_dtype, _shape=gshape)
                elif route == dm.ROUTE_INT8:
                    qw, swr = L["qw"], L["swr"]
                    w8_bytes = (0.5 + 1.0 / 16 + 1.0) * lin.N * lin.K + 8.0 * lin.N
                    if args.int8_weights == "convert":
                        qw = w8_scratch[:lin.N * lin.K].view(lin.N, lin.K)
                        swr = s8_scratch[:lin.N]
                        kt("hadamard_quant_int8_w8", 3.0 * M * lin.K + 4.0 * M + w8_bytes,
                           dm.hadamard_quant_int8_w8, x, qb["q"], qb["s"], L["cw"], L["sw"], L["gw"], qw, swr,
                           _shape=f"{M}x{lin.K}+{lin.N}x{lin.K}")
                    else:
                        kt("hadamard_quant_int8", 3.0 * M * lin.K + 4.0 * M,
                           dm.hadamard_quant_int8, x, qb["q"], qb["s"], _shape=f"{M}x{lin.K}")
                    if args.int8_weights == "convert-separate":
                        qw = w8_scratch[:lin.N * lin.K].view(lin.N, lin.K)
                        swr = s8_scratch[:lin.N]
                        kt("weight_int8_from_nvfp4", w8_bytes,
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
        return ops

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
        # the GEMMs' own load path (global_load_lds DMA into LDS) on a known
        # size: one 256 x 256 output tile over K = 65536, so every operand byte
        # is fetched exactly once (no other tile could share it)
        kc = DMA_CALIB_K
        y1 = torch.empty((256, 256), dtype=torch.bfloat16, device="cuda")
        qa1 = torch.ones((256, kc), dtype=torch.int8, device="cuda")
        s1 = torch.ones(256, device="cuda")
        for _ in range(3):
            dm.qgemm_int8(qa1, s1, qa1, s1, y1, dm.OUT_BF16)
        c1 = torch.full((256, kc // 2), 0x22, dtype=torch.uint8, device="cuda")
        e1 = torch.full((256, kc // 16), 0x38, dtype=torch.uint8, device="cuda")
        g1 = torch.ones(1, device="cuda")
        for _ in range(3):
            dm.qgemm_nvfp4(c1, e1, g1, c1, e1, g1, y1, dm.OUT_BF16)
        torch.cuda.synchronize()
        del y1, qa1, s1, c1, e1, g1
        calib["dma_gemm_tile"] = {k: dict(kernel=v[0], read_bytes=v[1], write_bytes=v[2])
                                  for k, v in DMA_CALIB.items()}

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
    if args.graph == "on":
        for _ in range(2):  # the settled routing's graph is captured before the timed region
            step()
    kt.prepare(kt.calls * args.steps)
    gc.collect()  # the heap's collection before, not inside, the timed steps
    torch.cuda.synchronize()
    kt.on = args.graph == "off"
    host_t["wait"] = host_t["decide"] = 0.0
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    t_issued = time.perf_counter()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    host_timing = {"sync": args.host_sync,
                   "wait_ms_per_step": round(1e3 * host_t["wait"] / args.steps, 3),
                   "enqueue_ms_per_step": round(1e3 * (t_issued - t_start - host_t["wait"]) / args.steps, 3),
                   "decide_ms_per_step": round(1e3 * host_t["decide"] / args.steps, 3)}
    kt.on = False
    ms_per_step = 1e3 * elapsed / args.steps
    value = gemm_ops_step / (elapsed / args.steps) / 1e12
    ktimed = kt.summary(args.steps)

    # ---- per-kernel figures: events on every call, in as many extra steps -----
    kt.only = None
    kt.calls = 0
    step(eager=True)
    kt.prepare(kt.calls * args.steps)
    gc.collect()
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
        # the TDC skip (a block reusing its cached delta), timed the same way
        # into a scratch output
        for _ in range(args.steps):
            for b, blk in enumerate(blocks):
                kt("tdc_step_skip_standalone", 6.0 * M * H, dm.tdc_step, dm.TDC_SKIP, blk["x_in"],
                   skip_out, blk["delta"], True, _shape=f"{M}x{H}")
    torch.cuda.synchronize()
    kt.on = False
    ksum = kt.summary(args.steps)
    kshape = kt.summary(args.steps, by_shape=True)
    kernels, by_shape = kernel_tables(ksum, kshape)

    # ---- the same per-kernel pass with the memory-side cache flushed ---------
    # (a 1 GiB read-modify-write before every call evicts the 256 MB MALL:
    # every operand then comes from HBM, the cold-cache figure)
    cold = None
    if args.extras == "on":
        flush = torch.zeros(1 << 28, dtype=torch.int32, device="cuda")
        kt.flush = lambda: flush.add_(1)
        cold_steps = min(args.steps, 5)
        kt.only = None
        kt.calls = 0
        kt.on = False
        step(eager=True)
        kt.prepare(kt.calls * cold_steps)
        torch.cuda.synchronize()
        kt.on = True
        for _ in range(cold_steps):
            step()
        torch.cuda.synchronize()
        kt.on = False
        kt.flush = None
        del flush
        ck, cs = kernel_tables(kt.summary(cold_steps), kt.summary(cold_steps, by_shape=True))
        cold = {"note": ("every call preceded by a 1 GiB read-modify-write that evicts the 256 MB "
                         "memory-side cache; medians over %d steps" % cold_steps),
                "kernels": ck, "kernels_by_shape": cs}
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
                   "ffn": {"on": "ffn_down reads GELU(ffn_up); GELU and the NVFP4 amax fused into ffn_up's "
                                 "epilogue",
                           "separate": "ffn_down reads GELU(ffn_up); GELU as a separate kernel",
                           "off": "every linear on its own input"}[args.fuse_ffn],
                   "tail_split": args.tail_split == "on",
                   "issue": "HIP graph replay after the host decisions" if args.graph == "on" else "per-call launches",
                   "gemm_tera_ops_per_step": round(gemm_ops_step / 1e12, 3)},
        "act_quant_GBps": round(q_bytes * 1e-9 / (q_ms * 1e-3), 1),
        "kernels": kernels,
        "kernels_note": ("per-call HIP events on every call, in as many untimed steps after the timed "
                         "region; gamma_sums_standalone is timed beside those steps, not in them"),
        "host": host_timing,
        "timing_events": ("HIP events without the system-scope fence" if args.events == "nofence"
                          else "torch.cuda events"),
        "kernels_by_shape": by_shape,
        "roofline": roofline,
        "setup_s": round(setup_s, 1),
    }
    if calib is not None:
        result["copy_calibration"] = calib
    if cold is not None:
        result["kernels_cold"] = cold
    if args.extras == "on":
        # free the headline's tensors first: the extra workloads bring their own
        del blocks, qbuf, ybuf, w8_scratch, skip_out, ws_gemm
        torch.cuda.empty_cache()
        result["extras"] = run_extras(args)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.cpu_rows)
        if args.extras == "on":
            result["cpu_baseline"]["oracle_quant_1thread"] = oracle_quant_1thread()
    print(json.dumps(result), flush=True)


PEAKS = {"hadamard_quant_int8": ("hbm", HBM_GBPS, "GB/s"),
         "hadamard_quant_int8_w8": ("hbm", HBM_GBPS, "GB/s"),
         "weight_int8_from_nvfp4": ("hbm", HBM_GBPS, "GB/s"),
         "outlier_count": ("hbm", HBM_GBPS, "GB/s"),
         "gemm_bf16": ("mfma", PEAK_BF16_TFLOPS, "TFLOP/s"),
         "hadamard_quant_nvfp4": ("hbm", HBM_GBPS, "GB/s"),
         "hadamard_quant_nvfp4_given": ("hbm", HBM_GBPS, "GB/s"),
         "gamma_sums": ("hbm", HBM_GBPS, "GB/s"),
         "gamma_sums_standalone": ("hbm", HBM_GBPS, "GB/s"),
         "tdc_step_refresh": ("hbm", HBM_GBPS, "GB/s"),
         "tdc_step_skip": ("hbm", HBM_GBPS, "GB/s"),
         "tdc_step_skip_standalone": ("hbm", HBM_GBPS, "GB/s"),
         "gelu_separate": ("hbm", HBM_GBPS, "GB/s"),
         "qgemm_int8": ("mfma", PEAK_INT8_TOPS, "TOPS"),
         "qgemm_nvfp4": ("mfma", PEAK_FP4_TFLOPS, "TFLOP/s")}


def kernel_tables(ksum: dict, kshape: dict):
    """Per-kernel and per-(kernel, shape) figures from KernelTimer summaries:
    achieved rate (algorithmic work / event-timed duration) against the
    MI355X peak of the kernel's bound."""
    kernels = {}
    for name, s in ksum.items():
        bound, peak, unit = PEAKS[name]
        scale = 1e-9 if unit == "GB/s" else 1e-12
        achieved = s["work"] * scale / (s["total_ms"] * 1e-3)
        kernels[name] = dict(calls_per_step=s["calls_per_step"], avg_us=round(s["avg_us"], 2),
                             median_us=round(s["median_us"], 2), achieved=round(achieved, 2), unit=unit,
                             bound=bound, peak=peak, frac=round(achieved / peak, 4))
        if name == "qgemm_nvfp4":
            kernels[name]["frac_of_bf16_pipe"] = round(achieved / PEAK_BF16_TFLOPS, 4)
        if name == "hadamard_quant_nvfp4":
            # the two-pass form moves 2 + 2 + 0.5625 B per element against the
            # 2.5625 algorithmic ones: its own bound is that share of the peak
            kernels[name]["frac_of_two_read_bound"] = round(achieved / (peak * 2.5625 / 4.5625), 4)
    by_shape = {}
    for (name, shape), s in sorted(kshape.items()):
        bound, peak, unit = PEAKS[name]
        achieved = s["work"] * (1e-9 if unit == "GB/s" else 1e-12) / (s["total_ms"] * 1e-3)
        by_shape[f"{name} {shape}"] = dict(calls_per_step=s["calls_per_step"], median_us=round(s["median_us"], 2),
                                           achieved=round(achieved, 2), unit=unit,
                                           frac=round(achieved / peak, 4))
    return kernels, by_shape


# ---- the other workloads, measured after the headline ------------------------

def _gemm_call(dm, kt, route, x, qb, L, y, ws_q, ws_gemm, w8, s8, epi=0):
    """One routed linear as the headline step runs it: Hadamard + quant and,
    on the INT8 route in the same launch, the NVFP4 -> INT8 weight conversion
    into the shared scratch; then the quantized GEMM with the full GEMM
    workspace, bf16 output."""
    M, K = x.shape
    N = L["N"]
    flops = 2.0 * M * N * K
    gshape = f"{M}x{N}x{K}"
    if route == dm.ROUTE_INT8:
        qw = w8[:N * K].view(N, K)
        sw = s8[:N]
        kt("hadamard_quant_int8_w8", 3.0 * M * K + 4.0 * M + (0.5 + 1.0 / 16 + 1.0) * N * K + 8.0 * N,
           dm.hadamard_quant_int8_w8, x, qb["q"], qb["s"], L["cw"], L["sw"], L["gw"], qw, sw,
           _shape=f"{M}x{K}+{N}x{K}")
        kt("qgemm_int8", flops, dm.qgemm_int8_ex, qb["q"], qb["s"], qw, sw, y, epi, ws_gemm, dm.OUT_BF16,
           _shape=gshape)
    else:
        kt("hadamard_quant_nvfp4", (2.0 + 0.5 + 1.0 / 16) * M * K + 4.0, dm.hadamard_quant_nvfp4, x,
           qb["c"], qb["sc"], qb["g"], ws_q, _shape=f"{M}x{K}")
        kt("qgemm_nvfp4", flops, dm.qgemm_nvfp4_ex, qb["c"], qb["sc"], qb["g"], L["cw"], L["sw"], L["gw"], y,
           epi, ws_gemm, dm.OUT_BF16, _shape=gshape)
    return flops


def _nvfp4_weight(torch, dm, w, ws_prep):
    N, K = w.shape
    L = dict(N=N, cw=torch.empty((N, K // 2), dtype=torch.uint8, device="cuda"),
             sw=torch.empty((N, K // 16), dtype=torch.uint8, device="cuda"),
             gw=torch.zeros(1, device="cuda"))
    qw = torch.empty((N, K), dtype=torch.int8, device="cuda")   # prep's INT8 output, not kept
    swr = torch.empty(N, device="cuda")
    dm.prep_weight(w, L["cw"], L["sw"], L["gw"], qw, swr, ws_prep)
    return L


def _quant_buffers(torch, M, K):
    return dict(q=torch.empty((M, K), dtype=torch.int8, device="cuda"), s=torch.empty(M, device="cuda"),
                c=torch.empty((M, K // 2), dtype=torch.uint8, device="cuda"),
                sc=torch.empty((M, K // 16), dtype=torch.uint8, device="cuda"),
                g=torch.zeros(1, device="cuda"))


def run_linears_workload(torch, dm, wl, cfg, steps: int, events: str) -> dict:
    """Every linear of a config on one route per step (all INT8, then all
    NVFP4), each on its own synthetic input, launched as in the headline
    step.  Wall time per step without events, then the per-kernel figures
    from as many steps with events around every call."""
    M = cfg.M
    gen = wl.device_generator(cfg.seeds[0])
    ws_prep = dm.new_workspace(dm.OP_PREP_WEIGHT)
    lins = []
    for lin in cfg.linears:
        x = wl.activations_device(gen, M, lin.K)
        L = _nvfp4_weight(torch, dm, wl.weight_device(gen, lin.N, lin.K), ws_prep)
        lins.append(dict(L, x=x, name=lin.name, K=lin.K))
    qbuf = {K: _quant_buffers(torch, M, K) for K in sorted({lin.K for lin in cfg.linears})}
    nmax = max(lin.N for lin in cfg.linears)
    ybuf = torch.empty(M * nmax, dtype=torch.bfloat16, device="cuda")
    w8 = torch.empty(max(lin.N * lin.K for lin in cfg.linears), dtype=torch.int8, device="cuda")
    s8 = torch.empty(nmax, device="cuda")
    ws_q = dm.new_workspace(dm.OP_QUANT_NVFP4)
    ws_gemm = dm.new_workspace(dm.OP_GEMM, "cuda", M, nmax)
    kt = KernelTimer(torch, events)

    def step(route):
        ops = 0.0
        for L in lins:
            y = ybuf[:M * L["N"]].view(M, L["N"])
            ops += _gemm_call(dm, kt, route, L["x"], qbuf[L["K"]], L, y, ws_q, ws_gemm, w8, s8)
        return ops

    out = {}
    for route, rname in ((dm.ROUTE_INT8, "all_int8"), (dm.ROUTE_NVFP4, "all_nvfp4")):
        step(route)                           # warmup
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            ops = step(route)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / steps
        kt.rec = {}
        kt.on = True
        for _ in range(steps):
            step(route)
        torch.cuda.synchronize()
        kt.on = False
        kernels, by_shape = kernel_tables(kt.summary(steps), kt.summary(steps, by_shape=True))
        out[rname] = {"ms_per_step": round(1e3 * dt, 3), "gemm_tera_ops_per_step": round(ops / 1e12, 3),
                      "value_TOPS": round(ops / dt / 1e12, 2), "kernels": kernels,
                      "kernels_by_shape": by_shape}
    return out


def run_schedule_workload(torch, dm, wl, events: str, T: int = 50, NB: int = 42) -> dict:
    """The full TDC schedule on a proxy DiT: NB residual blocks
    x + W2 GELU(W1 x) (hidden 1920 -> 1920 -> 1920, W1 ~ N(0, 1/H),
    W2 ~ N(0, 0.3^2/H)) at 17776 tokens over T timesteps of a drifting latent
    z_t = z_{t-1} + 0.02 N(0, 1).  Per block and timestep the library's
    TdcScheduler decides skip or refresh; a refresh routes both linears by
    the block's Gamma (INT8 when it is missing) and runs them with the GELU
    fused into the first GEMM's epilogue; the residual add is torch glue.
    Thresholds from three always-refresh steps (tau = median Gamma,
    eps_sim = median d, delta_acc = 2.5 median d).  Runs the schedule three
    times from the same state: without events (the wall time), with events
    around every library call (per-kernel time; its decisions must equal the
    first run's), and with every block refreshed (the no-TDC reference).
    A fourth run uses a fitted router: over CAL always-refresh steps every
    linear's NVFP4 error against its BF16 output (ErrorProbe) is paired with
    the Gamma the router saw, alpha_l and beta_l are fitted by least squares
    (fit_router) and tau is the median predicted error of those samples."""
    import numpy as np

    from dynamic_mixed_precision_amd.calibrate import ErrorProbe, fit_router
    from dynamic_mixed_precision_amd.schedule import TdcScheduler
    CAL = 6
    cfg = wl.PROXY_DIT
    M, H = cfg.M, cfg.hidden
    gen = wl.device_generator(cfg.seeds[0])
    ws_prep = dm.new_workspace(dm.OP_PREP_WEIGHT)
    blocks, blocks_bf16 = [], []
    for _ in range(NB):
        w1 = wl.weight_device(gen, H, H)
        w2 = (wl.weight_device(gen, H, H).float() * 0.3).to(torch.bfloat16)
        blocks.append((_nvfp4_weight(torch, dm, w1, ws_prep), _nvfp4_weight(torch, dm, w2, ws_prep)))
        blocks_bf16.append((w1, w2))
    z = [wl.activations_device(gen, M, H)]
    for _ in range(T - 1):                    # the drifting latents, resident before timing
        n = torch.randn((M, H), generator=gen, device="cuda", dtype=torch.float32)
        z.append((z[-1].float() + 0.02 * n).to(torch.bfloat16))
    del n
    qb = _quant_buffers(torch, M, H)
    h = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    act = [torch.empty((M, H), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    w8 = torch.empty(H * H, dtype=torch.int8, device="cuda")
    s8 = torch.empty(H, device="cuda")
    ws_q = dm.new_workspace(dm.OP_QUANT_NVFP4)
    ws_gemm = dm.new_workspace(dm.OP_GEMM, "cuda", M, H)
    alpha, beta = np.ones(2), np.zeros(2)

    def run(steps, tau, eps, dacc, kt, force_refresh=False, router=(alpha, beta), probe=None):
        sched = TdcScheduler(NB, M * H, router[0], router[1], tau, eps, dacc)
        log = []
        ops = 0.0
        for t in range(steps):
            sched.begin_step()
            x = z[t]
            for i in range(NB):
                out = act[i % 2]
                if not force_refresh and sched.decide(i):
                    b = sched.blocks[i]
                    kt("tdc_step_skip", 6.0 * M * H, dm.tdc_step, dm.TDC_SKIP, x.view(-1), out.view(-1),
                       b.delta, True, _shape=f"{M}x{H}")
                    dm.tdc_commit(b.state, dm.TDC_SKIP)
                    log.append((t, i, "skip"))
                else:
                    g_seen, _, r = sched.routes(i)
                    l1, l2 = blocks[i]
                    ops += _gemm_call(dm, kt, int(r[0]), x, qb, l1, h, ws_q, ws_gemm, w8, s8, dm.EPI_GELU)
                    if probe is not None and sched.blocks[i].state.gamma_valid:
                        probe(g_seen, (x, l1, blocks_bf16[i][0]), (h, l2, blocks_bf16[i][1]))
                    ops += _gemm_call(dm, kt, int(r[1]), h, qb, l2, y, ws_q, ws_gemm, w8, s8)
                    torch.add(x, y, out=out)
                    b = sched.blocks[i]
                    kt("tdc_step_refresh", 8.0 * M * H, dm.tdc_step, dm.TDC_REFRESH, x.view(-1), out.view(-1),
                       b.delta, bool(b.state.delta_valid), b.sums, sched.ws, _shape=f"{M}x{H}")
                    b.sums_host.copy_(b.sums, non_blocking=True)
                    b.pending = True
                    log.append((t, i, tuple(int(v) for v in r)))
                x = out
        sched.begin_step()
        return sched, log, ops

    off = KernelTimer(torch, events)
    cal, _, _ = run(3, float("inf"), 0.0, 0.0, off)          # always refresh, routes NVFP4
    gam = [b.state.gamma for b in cal.blocks]
    ds = [b.state.d for b in cal.blocks]
    tau, eps = float(np.median(gam)), float(np.median(ds))
    dacc = 2.5 * eps
    del cal
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    _, log, ops = run(T, tau, eps, dacc, off)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kt = KernelTimer(torch, events)
    kt.on = True
    _, log_ev, _ = run(T, tau, eps, dacc, kt)
    torch.cuda.synchronize()
    kt.on = False
    kernels, by_shape = kernel_tables(kt.summary(T), kt.summary(T, by_shape=True))
    lib_ms = sum(v["total_ms"] for v in kt.summary(T).values())
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    _, _, ops_all = run(T, tau, eps, dacc, off, force_refresh=True)
    torch.cuda.synchronize()
    wall_all = time.perf_counter() - t0

    # fitted router: (Gamma seen, NVFP4 error of each linear) over CAL steps
    ep = ErrorProbe(M, H, H)
    samples = []

    def probe(g_seen, *lins):
        samples.append((g_seen, [ep(xi, wb, L["cw"], L["sw"], L["gw"]) for xi, L, wb in lins]))

    run(CAL, float("inf"), 0.0, 0.0, off, probe=probe)       # always refresh, routes NVFP4
    gs = np.array([smp[0] for smp in samples])
    errs = np.array([smp[1] for smp in samples])
    a_fit, b_fit, rms = fit_router(gs, errs)
    tau_fit = float(np.median(a_fit[None, :] * gs[:, None] + b_fit[None, :]))
    del ep
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    _, log_fit, _ = run(T, tau_fit, eps, dacc, off, router=(a_fit, b_fit))
    torch.cuda.synchronize()
    wall_fit = time.perf_counter() - t0

    bits = {dm.ROUTE_INT8: 8.0, dm.ROUTE_NVFP4: 4.5}

    def mix(lg):
        calls = [r for e in lg if e[2] != "skip" for r in e[2]]
        return (sum(1 for e in lg if e[2] == "skip"), sum(1 for r in calls if r == dm.ROUTE_INT8),
                sum(1 for r in calls if r == dm.ROUTE_NVFP4),
                round(sum(bits[r] for r in calls) / max(len(calls), 1), 3))

    skips, n8, n4, avg_bits = mix(log)
    fs, f8, f4, fbits = mix(log_fit)
    return {
        "workload": (f"proxy DiT, {NB} blocks x + W2 GELU(W1 x) (hidden {H}), {M} tokens, {T} timesteps of "
                     "a drifting latent; TDC skip/refresh + Gamma router, GELU fused into W1's GEMM"),
        "thresholds": {"tau": tau, "eps_sim": eps, "delta_acc": dacc, "alpha": 1.0, "beta": 0.0},
        "block_steps": NB * T, "skips": skips, "skip_rate": round(skips / (NB * T), 4),
        "linear_calls": {"INT8": n8, "NVFP4": n4},
        "avg_activation_bits": avg_bits,
        "ms_per_timestep": round(1e3 * wall / T, 3),
        "ms_per_timestep_all_refresh": round(1e3 * wall_all / T, 3),
        "tdc_speedup": round(wall_all / wall, 3),
        "gemm_tera_ops": round(ops / 1e12, 3), "gemm_tera_ops_all_refresh": round(ops_all / 1e12, 3),
        "library_kernel_ms_per_timestep": round(lib_ms / T, 3),
        "decisions_equal_across_runs": log == log_ev,
        "kernels": kernels, "kernels_by_shape": by_shape,
        "router_fitted": {
            "fit": (f"{CAL} always-refresh steps, {len(samples)} block refreshes with Gamma; E = relative L1 "
                    "error of each linear's NVFP4 output against its BF16 output (W1 before GELU)"),
            "alpha": [round(float(v), 5) for v in a_fit], "beta": [round(float(v), 5) for v in b_fit],
            "rms_residual": [round(float(v), 5) for v in rms],
            "error_range": [round(float(errs.min()), 5), round(float(errs.max()), 5)],
            "gamma_range": [round(float(gs.min()), 5), round(float(gs.max()), 5)],
            "tau": round(tau_fit, 5), "skip_rate": round(fs / (NB * T), 4),
            "linear_calls": {"INT8": f8, "NVFP4": f4}, "avg_activation_bits": fbits,
            "ms_per_timestep": round(1e3 * wall_fit / T, 3),
        },
    }


def run_extras(args) -> dict:
    import torch

    import dynamic_mixed_precision_amd as dm
    import workloads as wl
    out = {}
    for key, cfg in (("cogvideox2b_linears", wl.COGVIDEOX_2B), ("video1080p_linears", wl.VIDEO_1080P)):
        out[key] = dict(workload=f"{cfg.name}: {', '.join(f'{l.name} {l.N}x{l.K}' for l in cfg.linears)}, "
                                 f"{cfg.M} tokens, each on its own synthetic input; all-INT8 step, "
                                 "then all-NVFP4 step",
                        **run_linears_workload(torch, dm, wl, cfg, args.extra_steps, args.events))
        torch.cuda.empty_cache()
    out["proxy_dit_tdc_schedule"] = run_schedule_workload(torch, dm, wl, args.events)
    torch.cuda.empty_cache()
    out["int8_weight_forms_5b"] = run_int8_weight_forms(torch, dm, wl, 5, args.events)
    # the step with a real DiT FFN (ffn_down reads GELU(ffn_up)), each form in
    # a child process (the same command with another --fuse-ffn): GELU and
    # the NVFP4 amax fused into ffn_up's epilogue, and like-for-like with
    # GELU as a separate kernel and the two-pass quantizer
    for mode in ("on", "separate"):
        out[f"headline_step_ffn_{mode}"] = child_bench(
            ["--fuse-ffn", mode, "--extras", "off", "--no-cpu-baseline", "--steps", str(min(args.steps, 10)),
             "--warmup", str(min(args.warmup, 3)), "--events", args.events])
    # the headline step with its linears and refreshes replayed from a HIP
    # graph after the host decisions: what the per-call launches cost
    out["headline_step_graph"] = child_bench(
        ["--graph", "on", "--extras", "off", "--no-cpu-baseline", "--steps", str(min(args.steps, 10)),
         "--warmup", str(min(args.warmup, 3)), "--events", args.events])
    return out


def run_int8_weight_forms(torch, dm, wl, reps: int, events: str) -> dict:
    """The INT8 route's two exact forms of the NVFP4 weight on the 5B-like
    linears (17776 tokens): the separate conversion into a scratch INT8
    weight followed by the INT8 GEMM (the headline step's form), and the
    INT8 GEMM that converts the weight inside its tile load.  Per-call HIP
    event times over `reps` calls of each, and whether the two outputs agree
    bit for bit."""
    cfg = wl.COGVIDEOX_5B
    M = cfg.M
    gen = wl.device_generator(cfg.seeds[0] + 100)
    ws_prep = dm.new_workspace(dm.OP_PREP_WEIGHT)
    kt = KernelTimer(torch, events)
    out = {}
    for lin in cfg.linears:
        N, K = lin.N, lin.K
        x = wl.activations_device(gen, M, K)
        L = _nvfp4_weight(torch, dm, wl.weight_device(gen, N, K), ws_prep)
        qa = torch.empty((M, K), dtype=torch.int8, device="cuda")
        sa = torch.empty(M, device="cuda")
        dm.hadamard_quant_int8(x, qa, sa)
        qw = torch.empty((N, K), dtype=torch.int8, device="cuda")
        swr = torch.empty(N, device="cuda")
        y1 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        y2 = torch.empty_like(y1)
        ws_gemm = dm.new_workspace(dm.OP_GEMM, "cuda", M, N)
        ws_w4 = dm.new_workspace(dm.OP_GEMM_W4, "cuda", M, N)
        conv = (dm.weight_int8_from_nvfp4, L["cw"], L["sw"], L["gw"], qw, swr)
        quant = (dm.hadamard_quant_int8, x, qa, sa)
        quant_w8 = (dm.hadamard_quant_int8_w8, x, qa, sa, L["cw"], L["sw"], L["gw"], qw, swr)
        gemm = (dm.qgemm_int8_ex, qa, sa, qw, swr, y1, 0, ws_gemm, dm.OUT_BF16)
        fused = (dm.qgemm_int8_from_nvfp4, qa, sa, L["cw"], L["sw"], L["gw"], y2, ws_w4, 0, dm.OUT_BF16)
        for f in (conv, gemm, fused, quant, quant_w8):  # warmup
            f[0](*f[1:])
        torch.cuda.synchronize()
        kt.rec = {}
        kt.on = True
        for _ in range(reps):
            kt("quant", 0.0, *quant)
            kt("convert", 0.0, *conv)
            kt("quant_w8", 0.0, *quant_w8)
            kt("int8_gemm", 0.0, *gemm)
            kt("fused", 0.0, *fused)
        torch.cuda.synchronize()
        kt.on = False
        t = {k: v["avg_us"] for k, v in kt.summary(reps).items()}
        flops = 2.0 * M * N * K
        out[f"{lin.name} {M}x{N}x{K}"] = {
            "act_quant_us": round(t["quant"], 1), "act_quant_and_convert_one_launch_us": round(t["quant_w8"], 1),
            "convert_us": round(t["convert"], 1), "int8_gemm_us": round(t["int8_gemm"], 1),
            "convert_then_gemm_us": round(t["convert"] + t["int8_gemm"], 1), "fused_us": round(t["fused"], 1),
            "fused_TOPS": round(flops / t["fused"] / 1e6, 1),
            "bit_identical": bool(torch.equal(y1.view(torch.int16), y2.view(torch.int16)))}
        del x, L, qa, qw, y1, y2, ws_gemm, ws_w4
        torch.cuda.empty_cache()
    return out


def child_bench(extra_args: list) -> dict:
    """Run bench.py with extra_args in a child process and keep the figures
    that compare step forms."""
    import subprocess
    r = subprocess.run([sys.executable, os.path.abspath(__file__), *extra_args], capture_output=True, text=True,
                       timeout=600)
    if r.returncode != 0:
        return {"error": f"exit {r.returncode}: {r.stderr.strip()[-300:]}"}
    d = json.loads(r.stdout.strip().splitlines()[-1])
    keep = ("hadamard_quant_nvfp4", "hadamard_quant_nvfp4_given", "gelu_separate", "qgemm_nvfp4", "qgemm_int8")
    return {"args": " ".join(extra_args), "value_TOPS": d["value"], "ms_per_step": d["ms_per_step"],
            "act_quant_GBps": d["act_quant_GBps"], "ffn": d["config"]["ffn"], "host": d.get("host"),
            "kernels": {k: v for k, v in d["kernels"].items() if k in keep}}


def cpu_info() -> dict:
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "logical_cpus": os.cpu_count(),
            "cpus_available": len(os.sched_getaffinity(0))}


def oracle_quant_1thread() -> dict:
    """The oracle's two quantizers on one host thread: the tiny config
    (256 x 256) and a 1024-token slice of the 2B-like hidden (1920)."""
    import numpy as np

    import oracle as orc
    import workloads as wl
    before = orc.max_threads()
    orc.set_threads(1)
    out = {}
    try:
        for name, (M, K) in (("tiny_256x256", (256, 256)), ("2b_hidden_1024x1920", (1024, 1920))):
            x = wl.activations(np.random.default_rng(M + K), M, K)
            t = time.perf_counter()
            orc.quant_int8(x)
            t8 = time.perf_counter() - t
            t = time.perf_counter()
            orc.quant_nvfp4(x)
            t4 = time.perf_counter() - t
            out[name] = {"int8_GBps": round((3.0 * M * K + 4 * M) / t8 / 1e9, 4),
                         "nvfp4_GBps": round((2.5625 * M * K + 4) / t4 / 1e9, 4),
                         "int8_s": round(t8, 4), "nvfp4_s": round(t4, 4)}
    finally:
        orc.set_threads(before)
    return dict(threads=1, **out)


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
            "kind": "oracle", **cpu_info(),
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
CALIB_KERNEL = "dmpq::tdc_skip_kernel<2>"  # the skip kernel at the calibration size (64 M chunks)
# Known-size calibration of the DMA load path: one 256 x 256 tile over K =
# DMA_CALIB_K (a one-workgroup launch, so its dispatches are told apart from
# the step's by their grid of 256 work-items); bytes each operand moves once.
DMA_CALIB_K = 65536
DMA_CALIB = {"qgemm_int8": ("dmpq::gemm_i8_dma_kernel<1, *>", 2 * 256 * DMA_CALIB_K + 2 * 256 * 4,
                            256 * 256 * 2),
             "qgemm_nvfp4": ("dmpq::gemm_fp4_dma_kernel<1, *>",
                             2 * 256 * (DMA_CALIB_K // 2 + DMA_CALIB_K // 16) + 8, 256 * 256 * 2)}
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


def gemm_operand_bytes(api: str) -> float:
    """Average compulsory operand bytes (codes + scales of A and W) of one GEMM
    launch of the step."""
    import workloads as wl
    cfg = wl.COGVIDEOX_5B
    tot = 0.0
    for lin in cfg.linears:
        per = (lin.K / 2 + lin.K / 16) if api == "qgemm_nvfp4" else (lin.K + 4)
        tot += (cfg.M + lin.N) * per
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
    if "fetch_factor_used" in rec:
        out["traffic_note"] = ("FETCH_SIZE and WRITE_SIZE of L2 misses (the memory-side cache serves part "
                               "of them), scaled by factors %.3g / %.3g measured on a one-tile launch of "
                               "the same DMA load path" % (rec["fetch_factor_used"], rec["write_factor_used"]))
    return out


def _counter_rows(path: str, counter: str):
    import csv
    with open(path) as f:
        return [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]


def _kernel_re(kernel: str):
    import re
    return re.compile(re.escape(kernel).replace(r"\*", r"\d+") + r"\(")


def _per_kernel_kib(rows, kernel: str, grid=None, not_grid=None):
    """Counter value (KiB) of every dispatch of `kernel`, in dispatch order;
    `grid` / `not_grid`: keep only dispatches with / without that many work-items."""
    pat = _kernel_re(kernel)
    sel = {}
    for r in rows:
        if not pat.search(r["Kernel_Name"]):
            continue
        g = int(r.get("Grid_Size", 0) or 0)
        if (grid is not None and g != grid) or (not_grid is not None and g == not_grid):
            continue
        sel[int(r["Dispatch_Id"])] = sel.get(int(r["Dispatch_Id"]), 0.0) + float(r["Counter_Value"])
    return [sel[k] for k in sorted(sel)]


def summarize_traffic(fetch_csv: str, write_csv: str, out_json: str, command: str) -> None:
    fr, wr = _counter_rows(fetch_csv, "FETCH_SIZE"), _counter_rows(write_csv, "WRITE_SIZE")
    # the calibration's three dispatches come before the warmup steps (which
    # may run the same kernel again)
    cf, cw = _per_kernel_kib(fr, CALIB_KERNEL)[:3], _per_kernel_kib(wr, CALIB_KERNEL)[:3]
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
    # the DMA load path of each GEMM on its known-size one-tile launch; its
    # factors (not the streaming kernel's) scale that GEMM's counts
    dma = {}
    for api, (kname, rbytes, wbytes) in DMA_CALIB.items():
        df = _per_kernel_kib(fr, kname, grid=256)
        dw = _per_kernel_kib(wr, kname, grid=256)
        if len(df) != 3 or len(dw) != 3:
            raise SystemExit(f"expected 3 one-tile dispatches of {kname}, got {len(df)}, {len(dw)}")
        dma[api] = {"kernel": kname, "read_bytes": rbytes, "write_bytes": wbytes,
                    "fetch_kib_per_dispatch": df, "write_kib_per_dispatch": dw,
                    "fetch_factor": round(rbytes / (1024.0 * sum(df) / 3), 5),
                    "write_factor": round(wbytes / (1024.0 * sum(dw) / 3), 5)}
    rec["calibration_dma"] = dma
    for api, knames in GEMM_KERNELS.items():
        # one whole-tile dispatch per call (the one-tile calibration launches excluded)
        calls = len(_per_kernel_kib(fr, knames[0], not_grid=256))
        f = [v for k in knames for v in _per_kernel_kib(fr, k, not_grid=256)]
        w = [v for k in knames for v in _per_kernel_kib(wr, k, not_grid=256)]
        if not calls or len(f) != len(w):
            continue
        ff, fw = dma[api]["fetch_factor"], dma[api]["write_factor"]
        fb = 1024.0 * ff * sum(f) / calls
        wb = 1024.0 * fw * sum(w) / calls
        alg = gemm_algorithmic_bytes(api)
        rec[api] = {"kernels": knames, "calls": calls, "dispatches": len(f),
                    "sources_sha256": sources_sha256(api),
                    "fetch_factor_used": ff, "write_factor_used": fw,
                    "fetch_kib_per_call_raw": round(sum(f) / calls, 1),
                    "write_kib_per_call_raw": round(sum(w) / calls, 1),
                    "fetch_bytes_per_launch": round(fb), "write_bytes_per_launch": round(wb),
                    "bytes_per_launch": round(fb + wb),
                    "algorithmic_bytes_per_launch": round(alg),
                    "traffic_over_algorithmic": round((fb + wb) / alg, 3),
                    "fetch_over_operand_bytes": round(fb / gemm_operand_bytes(api), 3)}
    with open(out_json, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


def summarize_counters(out_md: str, csvs: list, command: str, n_xcd: int = 8, n_cu: int = 256) -> dict:
    """Per-kernel counter figures from rocprofv3 --pmc runs of one command
    (one-workgroup calibration dispatches excluded).  Each dispatch's counters
    are summed over the chip; GRBM_GUI_ACTIVE counts each XCD's cycles, so
    cycles = GRBM_GUI_ACTIVE / n_xcd, clock = cycles / duration, and the MFMA
    busy share = SQ_VALU_MFMA_BUSY_CYCLES / (cycles * CUs * 4 SIMDs)."""
    import csv
    import re
    per = {}   # kernel -> counter -> list of (value, duration_ns) per dispatch
    ndisp = {}  # kernel -> most dispatches in one file
    for path in csvs:
        disp = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if "dmpq" not in r["Kernel_Name"] or int(r.get("Grid_Size", 0) or 0) == 256:
                    continue
                key = (int(r["Dispatch_Id"]), r["Counter_Name"])
                name = re.sub(r"\(.*", "", r["Kernel_Name"]).replace("void ", "")
                dur = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
                v = disp.get(key, (name, 0.0, dur))
                disp[key] = (name, v[1] + float(r["Counter_Value"]), dur)
        seen = {}
        for (d, counter), (name, val, dur) in disp.items():
            per.setdefault(name, {}).setdefault(counter, []).append((val, dur))
            seen.setdefault(name, set()).add(d)
        for name, ds in seen.items():
            ndisp[name] = max(ndisp.get(name, 0), len(ds))

    def mean(name, c):
        xs = per[name].get(c)
        return None if not xs else sum(v for v, _ in xs) / len(xs)

    res = {}
    for name, cs in per.items():
        g = cs.get("GRBM_GUI_ACTIVE")
        row = {"dispatches": ndisp[name]}
        if g:
            cyc = [v / n_xcd for v, _ in g]
            row["avg_us"] = sum(d for _, d in g) / len(g) / 1e3
            row["clock_GHz"] = sum(c / d for c, (_, d) in zip(cyc, g)) / len(g)
            mb = mean(name, "SQ_VALU_MFMA_BUSY_CYCLES")
            if mb is not None:
                row["mfma_busy"] = mb / (sum(cyc) / len(cyc) * n_cu * 4)
        vi, mi = mean(name, "SQ_INSTS_VALU"), mean(name, "SQ_INSTS_MFMA")
        if vi is not None and mi:
            row["valu_per_mfma"] = vi / mi
        wa, wc = mean(name, "SQ_WAIT_INST_ANY"), mean(name, "SQ_WAVE_CYCLES")
        if wa is not None and wc:
            row["wait_share"] = wa / wc
        bc = mean(name, "SQ_LDS_BANK_CONFLICT")
        if bc is not None:
            row["lds_bank_conflict_cycles"] = bc
            la = mean(name, "SQ_ACTIVE_INST_LDS")
            if la:
                row["lds_conflict_per_active"] = bc / la
        res[name] = row

    def fmt(v, f):
        return "-" if v is None else f.format(v)

    lines = ["# rocprofv3 counters per kernel: bench.py step, CogVideoX-5B-like batch", "",
             "Commands (each counter set is its own run, from /tmp, $REPO is the repository root):", "",
             "```", command, "```", "",
             f"Cycles = GRBM_GUI_ACTIVE / {n_xcd} XCDs; clock = cycles / dispatch duration; MFMA busy = "
             f"SQ_VALU_MFMA_BUSY_CYCLES / (cycles x {n_cu} CUs x 4 SIMDs); wait share = SQ_WAIT_INST_ANY / "
             "SQ_WAVE_CYCLES; LDS conflict = SQ_LDS_BANK_CONFLICT cycles per dispatch (and per "
             "SQ_ACTIVE_INST_LDS cycle).  Durations are those of the counter runs (dispatches serialized); "
             "for kernels shorter than about 100 us the GRBM window exceeds the dispatch timestamps, so their "
             "clock column overstates.  SQ_INSTS_VALU counts the MFMA instructions too.",
             "", "| kernel | dispatches | avg us | clock GHz | MFMA busy | VALU / MFMA insts | wait share | "
             "LDS conflict cycles | conflict / LDS active |", "|---|---|---|---|---|---|---|---|---|"]
    for name in sorted(res, key=lambda n: -res[n].get("avg_us", 0) * res[n]["dispatches"]):
        r = res[name]
        lines.append(f"| `{name}` | {r['dispatches']} | {fmt(r.get('avg_us'), '{:.1f}')} | "
                     f"{fmt(r.get('clock_GHz'), '{:.2f}')} | {fmt(r.get('mfma_busy'), '{:.1%}')} | "
                     f"{fmt(r.get('valu_per_mfma'), '{:.2f}')} | {fmt(r.get('wait_share'), '{:.1%}')} | "
                     f"{fmt(r.get('lds_bank_conflict_cycles'), '{:.3g}')} | "
                     f"{fmt(r.get('lds_conflict_per_active'), '{:.3f}')} |")
    lines.append("")
    with open(out_md, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))
    return res


def summarize_stats(stats_csv: str, out_md: str, command: str) -> None:
    import csv
    import re
    with open(stats_csv) as f:
        rows = list(csv.DictReader(f))
    lines = ["# rocprofv3 kernel stats: bench.py step, CogVideoX-5B-like batch "
             "(17776 tokens, 4 blocks x 4 linears, 2 INT8 + 2 NVFP4 blocks)", "",
             "Command (run from /tmp, $REPO is the repository root):", "", "```", command, "```", "",
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
