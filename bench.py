#!/usr/bin/env python3
"""Benchmark of the fine-grained FP8 Linear hot path on one MI355X.

One step = the whole path over one batch of synthetic input already resident in HBM.  The default workload
is the largest one that fits one GPU, the MoE layer: 8192 tokens x 7168 quantized 1x128, routed top-8 of 64
experts into 128-padded expert segments, the 64 expert weights [2048, 7168] quantized 128x128, and the
grouped block-scaled FP8 GEMM reading the routed token rows in place (bf16 out); the token quantization and
the routing run on a second stream, overlapping the weight quantization, and the GEMM waits for both.  Their
per-kernel durations are therefore taken while the weight quantizer runs beside them.  The dense workloads run
1x128 activation quantization -> 128x128 weight quantization -> block-scaled FP8 GEMM; decode starts from
pre-quantized weights, so its step has no weight quantization.  With the MoE headline, the dense up and down
projections and decode are measured after it the same way and reported under `other_workloads` (--also).

Prints ONE JSON line.  `value` is the step's GEMM work divided by the whole step time (TFLOP/s), so the
quantizers' and the routing's time counts against it; the timed region is K back-to-back steps between two
synchronizations, after an untimed settle phase (the step repeated for --settle-ms, reported as
settle_steps) and W warmup steps.
The GEMM's own duration is measured inside that region with a HIP event pair around each of its launches,
recorded on the stream the kernels are launched on; the quantizers' durations come from a second pass of K
steps with an event pair around every launch.  `roofline` describes the dominant kernel (the GEMM) against
MI355X's published peaks; its `traffic` (HBM bytes per launch) is read from the committed rocprofv3
summary of that kernel and workload under profiles/, and is null when the kernel sources have changed since
the counters were taken (the summary records their SHA-256).  `cpu_baseline` times the CPU oracle on a
bounded sample of the same workload.  Each kernel's entry gives the mean (the rates use it), median and
minimum of its K launch durations; the 1x128 and 128x128 quantizers' entries add `torch_cast_floor`, the median
duration of torch's own elementwise bf16 -> FP8 cast over the same input (the same bytes read and written,
without max-abs or scales), a same-size floor for that quantizer on this GPU.  `gpu_clock` is the graphics clock of each XCD while the steps ran (the
device's metrics table through amdsmi, about one refresh a second, hence the 2.5 s settle), and MFMA-bound
lines add the FP8 peak at that clock.

The decode workload's weight (132 MB) would fit in the 256 MB Infinity Cache, so the bench keeps four
copies and rotates them step by step: every step streams its weight from HBM, as a model with many layers
would.  The other workloads move more than 256 MB per step by themselves.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "block-scaled FP8 GEMM TFLOP/s (% FP8 MFMA peak) + 1x128 quant GB/s"
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E

DESCRIPTIONS = {
    "up": "dense FFN up-projection: A bf16 [4096,7168] ~N(0,1) with 72 (1%) outlier channels x20, W bf16 "
          "[18432,7168] ~N(0,0.02); 1x128 act quant + 128x128 weight quant + block-scaled FP8 GEMM -> bf16 "
          "[4096,18432]",
    "down": "dense FFN down-projection: gate x, up y bf16 [4096,18432] ~N(0,1), W bf16 [7168,18432] ~N(0,0.02); "
            "fused SwiGLU + 1x128 act quant of A = bf16(SiLU(x)*y) + 128x128 weight quant + block-scaled FP8 "
            "GEMM -> bf16 [4096,7168]",
    "moe": "MoE layer: 8192 tokens x 7168 bf16 ~N(0,1), router logits [8192,64] ~N(0,1), expert W bf16 "
           "[64][2048,7168] ~N(0,0.02); 1x128 act quant of the tokens + top-8 routing into 128-padded expert "
           "segments + 128x128 weight quant + grouped block-scaled FP8 GEMM reading the routed token rows "
           "directly (FP8 dispatch folded in) -> bf16",
    "decode": "decode-shaped small M: A bf16 [64,7168], W pre-quantized E4M3 [18432,7168] with 128x128 fp32 "
              "scales; 1x128 act quant + block-scaled FP8 GEMM -> bf16 [64,18432]",
    "tiny": "tiny: A bf16 [128,512] with 4 outlier channels x50, W bf16 [256,512]; full path -> bf16 [128,256]",
    "dequant": "FP8 -> BF16 weight conversion with 128x128 scales: E4M3 [18432,7168] (uniform finite codes), "
               "scales [144,56] ~U(1e-4,1e-2) -> bf16 [18432,7168]",
    "fp4": "FP4 (E2M1) quantization of the up projection's operands: A bf16 [4096,7168] ~N(0,1) with 72 outlier "
           "channels x20 (1x128 groups), W bf16 [18432,7168] ~N(0,0.02) (128x128 blocks) -> two codes a byte",
    "e5m6": "E5M6 1x128 quantization of the up projection's input: A bf16 [4096,7168] ~N(0,1) with 72 outlier "
            "channels x20 -> 12-bit codes, two per 3 bytes, + 1x128 fp32 scales",
    "per_channel": "per-channel FP8 quantization of the up projection's weight: W bf16 [18432,7168] ~N(0,0.02) "
                   "-> E4M3 [18432,7168] + one fp32 scale per output channel",
    "dual": "forward and backward FP8 copies of the up projection's input: A bf16 [4096,7168] ~N(0,1) with 72 "
            "outlier channels x20 -> 1x128 codes [4096,7168] + codes of A^T [7168,4096] (per channel, 128 tokens)",
}
DEQUANT_METRIC = "FP8 -> BF16 128x128 block dequantization GB/s (% HBM peak)"
DUAL_METRIC = "one-pass forward (1x128) + backward (1x128 of x^T) FP8 copies of a Linear input GB/s (% HBM peak)"
FP4_METRIC = "FP4 (E2M1) 1x128 activation + 128x128 weight quantization GB/s (% HBM peak)"
PER_CHANNEL_METRIC = "per-channel FP8 weight quantization GB/s (% HBM peak)"
E5M6_METRIC = "E5M6 1x128 activation quantization GB/s (% HBM peak)"
BANDWIDTH_METRICS = {"dequant": DEQUANT_METRIC, "dual": DUAL_METRIC, "fp4": FP4_METRIC,
                     "per_channel": PER_CHANNEL_METRIC, "e5m6": E5M6_METRIC}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def act_bytes(M, K):
    return 2 * M * K + M * K + 4 * M * (K // 128)


def w_bytes(N, K):
    return 2 * N * K + N * K + 4 * (N // 128) * (K // 128)


def gemm_bytes(M, N, K, out_bytes=2):
    return M * K + N * K + 4 * M * (K // 128) + 4 * (N // 128) * (K // 128) + out_bytes * M * N


class Workload:
    """Device-resident inputs and outputs, plus the list of kernels one step launches."""

    def __init__(self, name):
        import torch

        import fine_grained_quantization_amd as fq
        import workloads as wl

        self.name = name
        self.side, self.side_kernels = None, ()
        self.cast_floor = {}  # quantizer name -> its bf16 input, for the same-traffic torch cast floor
        dev = "cuda"
        t0 = time.time()
        d = wl.WORKLOADS[name]()
        log(f"[bench] generated {name} inputs in {time.time() - t0:.1f}s")
        self.host = d

        def bf16(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

        M, N, K = d["M"], d["N"], d["K"]
        self.M, self.N, self.K = M, N, K
        self.step_count = 0
        if name == "fp4":
            self.a, self.w = bf16(d["a"]), bf16(d["w"])
            self.flops = 0.0
            ab = 2 * M * K + M * K // 2 + 4 * (K // 128) * M
            wbytes = 2 * N * K + N * K // 2 + 4 * (N // 128) * (K // 128)
            self.bytes = ab + wbytes
            self.qa, self.sa = fq.fp8q_quant_act_fp4_1x128(self.a)      # output buffers, reused every step
            self.qw, self.sw = fq.fp8q_quant_w_fp4_128x128(self.w)
            self.kernels = [("quant_act_fp4_1x128", lambda: fq.fp8q_quant_act_fp4_1x128(self.a, self.qa, self.sa),
                             {"bytes": ab}),
                            ("quant_w_fp4_128x128", lambda: fq.fp8q_quant_w_fp4_128x128(self.w, self.qw, self.sw),
                             {"bytes": wbytes})]
            torch.cuda.synchronize()
            return
        if name == "e5m6":
            self.a = bf16(d["a"])
            self.flops = 0.0
            self.bytes = 2 * M * K + M * K // 2 * 3 + 4 * (K // 128) * M
            self.qa, self.sa = fq.fp8q_quant_act_e5m6_1x128(self.a)
            self.kernels = [("quant_act_e5m6_1x128", lambda: fq.fp8q_quant_act_e5m6_1x128(self.a, self.qa, self.sa),
                             {"bytes": self.bytes})]
            torch.cuda.synchronize()
            return
        if name == "per_channel":
            self.w = bf16(d["w"])
            self.flops = 0.0
            self.bytes = 3 * N * K + 4 * N
            self.qw, self.sw = fq.fp8q_quant_w_per_channel(self.w)
            self.kernels = [("quant_w_per_channel", lambda: fq.fp8q_quant_w_per_channel(self.w, self.qw, self.sw),
                             {"bytes": self.bytes})]
            torch.cuda.synchronize()
            return
        if name == "dual":
            self.a = bf16(d["a"])
            self.flops = 0.0
            self.bytes = 4 * M * K + 4 * (K // 128) * M + 4 * (M // 128) * K
            self.outs = fq.fp8q_quant_act_dual(self.a)
            self.kernels = [("quant_act_dual", lambda: fq.fp8q_quant_act_dual(self.a, *self.outs),
                             {"bytes": self.bytes})]
            torch.cuda.synchronize()
            return
        if name == "dequant":
            self.qw = torch.from_numpy(d["wq"]).to(dev)
            self.sw = torch.from_numpy(d["sw"]).to(dev)
            self.w = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
            self.flops = 0.0
            self.bytes = 3 * N * K + 4 * (N // 128) * (K // 128)
            self.kernels = [("dequant_w_128x128", lambda: fq.fp8q_dequant_w_128x128(self.qw, self.sw, w=self.w),
                             {"bytes": self.bytes})]
            torch.cuda.synchronize()
            return
        if name == "moe":
            self._init_moe(d, bf16, dev)
            return
        self.qa = torch.empty((M, K), dtype=torch.uint8, device=dev)
        self.sa = torch.empty((K // 128, M), dtype=torch.float32, device=dev)
        if name == "down":   # the activation is SwiGLU(gate, up), quantized by the fused kernel
            self.x, self.y = bf16(d["x"]), bf16(d["y"])
            kernels = [("swiglu_quant_act_1x128",
                        lambda: fq.fp8q_swiglu_quant_act_1x128(self.x, self.y, self.qa, self.sa),
                        {"bytes": act_bytes(M, K) + 2 * M * K})]
        else:
            self.a = bf16(d["a"])
            kernels = [("quant_act_1x128", lambda: fq.fp8q_quant_act_1x128(self.a, self.qa, self.sa),
                        {"bytes": act_bytes(M, K)})]
        if name == "decode":
            wq = torch.from_numpy(d["wq"]).to(dev)
            self.qw_copies = [wq] + [wq.clone() for _ in range(3)]
            self.qw = wq
            self.sw = torch.from_numpy(d["sw"]).to(dev)
        else:
            self.w = bf16(d["w"])
            self.qw = torch.empty(d["w"].shape, dtype=torch.uint8, device=dev)
            lead = tuple(d["w"].shape[:-2])
            self.sw = torch.empty(lead + (N // 128, K // 128), dtype=torch.float32, device=dev)
            wrows = int(np.prod(d["w"].shape[:-1]))
            kernels.append(("quant_w_128x128", lambda: fq.fp8q_quant_w_128x128(self.w, self.qw, self.sw),
                            {"bytes": w_bytes(wrows, K)}))
        self.c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        self.cast_floor = {"quant_act_1x128": self.a} if name != "down" else {}
        if name != "decode":
            self.cast_floor["quant_w_128x128"] = self.w
        self.flops = 2.0 * M * N * K
        kernels.append(("gemm_blockscaled",
                        lambda: fq.fp8q_gemm_blockscaled(self.qa, self.sa, self.qw, self.sw, c=self.c),
                        {"flops": self.flops, "bytes": gemm_bytes(M, N, K)}))
        self.step_count = 0
        self.kernels = kernels
        torch.cuda.synchronize()

    def _init_moe(self, d, bf16, dev):
        """Tokens are quantized once and routed on the GPU; the grouped GEMM reads each row of the
        expert-sorted, 128-padded layout straight from the quantized tokens (the FP8 dispatch gather folded into
        the GEMM; the layout is sized to the routing capacity, so nothing is read back to the host inside a
        step)."""
        import torch

        import fine_grained_quantization_amd as fq

        T, E, k, N, K = d["T"], d["E"], d["topk"], d["N"], d["K"]
        rows = fq.fp8q_moe_route_capacity(T, E, k)
        self.M = rows
        self.tokens = bf16(d["tokens"])
        self.logits = torch.from_numpy(d["logits"]).to(dev)
        self.qt = torch.empty((T, K), dtype=torch.uint8, device=dev)
        self.st = torch.empty((K // 128, T), dtype=torch.float32, device=dev)
        self.route_out = (torch.empty((T, k), dtype=torch.int32, device=dev),
                          torch.empty(E + 1, dtype=torch.int32, device=dev),
                          torch.empty((T, k), dtype=torch.int32, device=dev),
                          torch.empty(rows, dtype=torch.int32, device=dev))
        self.route_ws = torch.empty(fq.load_library().fp8q_moe_route_workspace_bytes(T, E), dtype=torch.uint8,
                                    device=dev)
        self.w = bf16(d["w"])
        self.qw = torch.empty(d["w"].shape, dtype=torch.uint8, device=dev)
        self.sw = torch.empty((E, N // 128, K // 128), dtype=torch.float32, device=dev)
        self.c = torch.empty((rows, N), dtype=torch.bfloat16, device=dev)
        # rows in use (for the byte counts only): one routing outside the timed region
        fq.fp8q_moe_route_topk(self.logits, k, workspace=self.route_ws, out=self.route_out)
        used = int(self.route_out[1][-1].item())
        self.rows_used = used
        off = self.route_out[1]
        self.flops = 2.0 * T * k * N * K       # routed (token, expert) rows only; padding rows are not work
        KB = K // 128
        route_bytes = 4 * T * E + 4 * 3 * T * k + 4 * rows + 4 * (E + 1)
        gb = used * K + E * N * K + 4 * used * KB + 4 * E * (N // 128) * KB + 2 * used * N
        self.kernels = [
            ("quant_act_1x128", lambda: fq.fp8q_quant_act_1x128(self.tokens, self.qt, self.st),
             {"bytes": act_bytes(T, K)}),
            ("moe_route_topk", lambda: fq.fp8q_moe_route_topk(self.logits, k, workspace=self.route_ws,
                                                              out=self.route_out), {"bytes": route_bytes}),
            ("quant_w_128x128", lambda: fq.fp8q_quant_w_128x128(self.w, self.qw, self.sw),
             {"bytes": w_bytes(E * N, K)}),
            ("grouped_gemm_blockscaled_gather",
             lambda: fq.fp8q_grouped_gemm_blockscaled_gather(self.qt, self.st, self.route_out[3], self.qw, self.sw,
                                                             off, c=self.c),
             {"flops": self.flops, "bytes": gb}),
        ]
        self.cast_floor = {"quant_act_1x128": self.tokens, "quant_w_128x128": self.w}
        # token quantization and routing (kernels 0 and 1) overlap the weight quantization (kernel 2)
        self.side, self.side_kernels = torch.cuda.Stream(), (0, 1)
        self.step_count = 0
        torch.cuda.synchronize()

    def step(self, events=None):
        if self.name == "decode":  # rotate weight copies so each step reads its weight from HBM
            self.qw = self.qw_copies[self.step_count % len(self.qw_copies)]
        self.step_count += 1
        if self.side is not None:
            return self._step_two_streams(events)
        for i, (_, fn, _) in enumerate(self.kernels):
            ev = events[i] if events is not None else None
            if ev is not None:
                ev[0].record()
            fn()
            if ev is not None:
                ev[1].record()

    def _step_two_streams(self, events):
        """The MoE step on two streams: the token quantization and the routing (a chain of short, latency-bound
        launches) run on a side stream while the expert weights are quantized on the main stream; the grouped
        GEMM, which needs all three, waits for the side stream. The side stream first waits for the main one,
        so a step's token quantization never overwrites tokens the previous step's GEMM still reads."""
        import torch

        main = torch.cuda.current_stream()
        self.side.wait_stream(main)
        for i, (_, fn, _) in enumerate(self.kernels):
            ev = events[i] if events is not None else None
            on_side = i in self.side_kernels
            if not on_side and i == len(self.kernels) - 1:
                main.wait_stream(self.side)   # the GEMM needs the quantized tokens and the routing
            with torch.cuda.stream(self.side if on_side else main):
                if ev is not None:
                    ev[0].record()
                fn()
                if ev is not None:
                    ev[1].record()


def measured_copy_gbs(mib: int = 1024, reps: int = 5) -> float:
    """Device-to-device copy bandwidth (bytes read + written per second) of a plain torch copy over `mib` MiB,
    the best of `reps` runs: the practical streaming rate of this GPU, beside the datasheet's 8 TB/s."""
    import torch

    src = torch.ones(mib << 18, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    best = float("inf")
    for _ in range(reps + 1):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b))
    del src, dst
    return 2 * (mib << 20) / (best * 1e-3) / 1e9


def cast_floor_us(src, reps: int) -> float:
    """Median duration of torch's own elementwise bf16 -> float8_e4m3fn cast of `src` into a preallocated
    tensor: it reads 2 and writes 1 byte per element, the traffic of a quantizer minus its scales (no max-abs,
    no scale, one conversion per element), so it is a same-size floor for that quantizer on this GPU."""
    import torch

    dst = torch.empty(src.shape, dtype=torch.float8_e4m3fn, device=src.device)
    each = []
    for i in range(reps + 2):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        if i >= 2:
            each.append(1e3 * a.elapsed_time(b))
    del dst
    return float(np.median(each))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class ClockSampler:
    """The GPU's graphics clocks while the steps run, from the device's metrics table (amdsmi), which the
    firmware refreshes about once a second with the clock of each XCD averaged over that second.  A host
    thread polls the table every `period_s` between start() and stop() and keeps each refresh once.  Reading
    it needs no GPU work.  Where amdsmi is missing or refuses (no permission, no matching device), the record
    says why and holds no windows."""

    def __init__(self, period_s: float = 0.02):
        import threading

        self.period_s = period_s
        self.windows: list[tuple[float, list[int]]] = []   # (host time first seen, per-XCD MHz)
        self.error = None
        self._stop = threading.Event()
        self._thread = None

    def _open(self):
        """amdsmi's metrics reader for torch's device 0 (on the sampler thread, so that the benchmark never
        waits on amdsmi)."""
        import amdsmi

        amdsmi.amdsmi_init()
        handle = self._match(amdsmi, amdsmi.amdsmi_get_processor_handles())
        return lambda: amdsmi.amdsmi_get_gpu_metrics_info(handle)

    @staticmethod
    def _match(amdsmi, handles):
        """The amdsmi handle of torch's device 0: the only GPU, or the one whose PCI address matches."""
        if len(handles) == 1:
            return handles[0]
        import torch

        p = torch.cuda.get_device_properties(0)
        want = (getattr(p, "pci_domain_id", None), getattr(p, "pci_bus_id", None),
                getattr(p, "pci_device_id", None))
        if None not in want:
            for h in handles:
                d, b, rest = amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")
                if (int(d, 16), int(b, 16), int(rest.split(".")[0], 16)) == want:
                    return h
        raise RuntimeError(f"{len(handles)} GPUs and none matched to torch's device 0")

    def _run(self):
        try:
            metrics = self._open()
        except Exception as e:  # the benchmark runs on without the clock record
            self.error = f"{type(e).__name__}: {' '.join(str(e).split())}"
            return
        last = None
        while not self._stop.is_set():
            try:
                m = metrics()
            except Exception as e:
                self.error = f"{type(e).__name__}: {' '.join(str(e).split())}"
                return
            stamp = m.get("system_clock_counter")
            xcd = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, int)] \
                if isinstance(m.get("current_gfxclks"), list) else []
            if stamp != last and xcd:
                self.windows.append((time.perf_counter(), xcd))
                last = stamp
            self._stop.wait(self.period_s)

    def start(self):
        import threading

        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()

    def stop(self):
        self._stop.set()
        if self._thread is not None:
            self._thread.join(timeout=1.0)
            if self._thread.is_alive() and self.error is None:
                self.error = "amdsmi did not answer within 1 s of the end of the timed region"

    def record(self, busy_from: float, busy_to: float, window_s: float = 1.05):
        """Clocks over the refreshes whose whole averaging window (about a second before each) lies in
        [busy_from, busy_to] (host perf_counter seconds): the mean over XCDs and windows, and the slowest and
        fastest XCD."""
        v = [x for t, x in self.windows if busy_from + window_s <= t <= busy_to]
        out = {"source": "amdsmi metrics table, per-XCD GFX clock averaged over each ~1 s refresh",
               "windows": len(v)}
        if v:
            flat = [c for x in v for c in x]
            out.update(MHz_mean=round(float(np.mean(flat)), 1), MHz_min_xcd=min(flat), MHz_max_xcd=max(flat),
                       xcds=len(v[0]))
        if self.error:
            out["error"] = self.error
        return out


def cpu_baseline(wk: Workload, target_s: float = 12.0):
    """Time the CPU oracle (as it stands) on a bounded sample of the same workload: the 1x128 quantization
    of `rows` activation rows, the 128x128 quantization of the weight blocks those rows need, and the
    rows x N output elements of the GEMM.  Reported in the metric's unit (TFLOP/s of GEMM work)."""
    import oracle

    d = wk.host
    N, K = wk.N, wk.K
    lib = oracle.load()
    if wk.name == "fp4":
        # calibrate on 128 weight rows, then about target_s seconds' worth of weight rows and token rows
        t0 = time.perf_counter()
        oracle.quant_w_fp4_128x128(d["w"][:128], lib=lib)
        oracle.quant_act_fp4_1x128(d["a"][:128], lib=lib)
        per = time.perf_counter() - t0
        nb = int(max(1, min(wk.M // 128, target_s / max(per, 1e-6))))
        t1 = time.perf_counter()
        oracle.quant_w_fp4_128x128(d["w"][:128 * nb], lib=lib)
        oracle.quant_act_fp4_1x128(d["a"][:128 * nb], lib=lib)
        t = time.perf_counter() - t1
        byts = nb * 128 * (2.5 * K) * 2
        return {"value": byts / t / 1e9, "unit": "GB/s", "cores": oracle.num_threads(lib), "kind": "oracle",
                "sample": f"{128 * nb} weight rows and {128 * nb} token rows (K={K}); {t:.1f} s"}
    if wk.name == "e5m6":
        # calibrate on 128 token rows, then about target_s seconds' worth of rows
        t0 = time.perf_counter()
        oracle.quant_act_e5m6_1x128(d["a"][:128], lib=lib)
        per = time.perf_counter() - t0
        nb = int(max(1, min(wk.M // 128, target_s / max(per, 1e-6))))
        t1 = time.perf_counter()
        oracle.quant_act_e5m6_1x128(d["a"][:128 * nb], lib=lib)
        t = time.perf_counter() - t1
        byts = wk.bytes * nb * 128 / wk.M
        return {"value": byts / t / 1e9, "unit": "GB/s", "cores": oracle.num_threads(lib), "kind": "oracle",
                "sample": f"{128 * nb} of the {wk.M} token rows (K={K}); {t:.1f} s"}
    if wk.name == "per_channel":
        # calibrate on 128 weight rows, then about target_s seconds' worth of rows
        t0 = time.perf_counter()
        oracle.quant_w_per_channel(d["w"][:128], lib=lib)
        per = time.perf_counter() - t0
        nb = int(max(1, min(N // 128, target_s / max(per, 1e-6))))
        t1 = time.perf_counter()
        oracle.quant_w_per_channel(d["w"][:128 * nb], lib=lib)
        t = time.perf_counter() - t1
        byts = wk.bytes * nb * 128 / N
        return {"value": byts / t / 1e9, "unit": "GB/s", "cores": oracle.num_threads(lib), "kind": "oracle",
                "sample": f"{128 * nb} of the {N} weight rows (K={K}); {t:.1f} s"}
    if wk.name == "dual":
        # calibrate on one 128-token block, then about target_s seconds' worth of blocks
        t0 = time.perf_counter()
        oracle.quant_act_1x128(d["a"][:128], lib=lib)
        oracle.quant_act_backward_copy(d["a"][:128], lib=lib)
        per = time.perf_counter() - t0
        nb = int(max(1, min(wk.M // 128, target_s / max(per, 1e-6))))
        t1 = time.perf_counter()
        oracle.quant_act_1x128(d["a"][:128 * nb], lib=lib)
        oracle.quant_act_backward_copy(d["a"][:128 * nb], lib=lib)
        t = time.perf_counter() - t1
        byts = wk.bytes * nb * 128 / wk.M
        return {"value": byts / t / 1e9, "unit": "GB/s", "cores": oracle.num_threads(lib), "kind": "oracle",
                "sample": f"{128 * nb} of the {wk.M} tokens (K={K}), both copies; {t:.1f} s"}
    if wk.name == "dequant":
        # calibrate on one 128-row block row, then convert about target_s seconds' worth of block rows
        t0 = time.perf_counter()
        oracle.dequant_w_128x128(d["wq"][:128], d["sw"][:1], lib=lib)
        per = time.perf_counter() - t0
        nb = int(max(1, min(N // 128, target_s / max(per, 1e-6))))
        t1 = time.perf_counter()
        oracle.dequant_w_128x128(d["wq"][:128 * nb], d["sw"][:nb], lib=lib)
        t = time.perf_counter() - t1
        byts = 3 * 128 * nb * K + 4 * nb * (K // 128)
        return {"value": byts / t / 1e9, "unit": "GB/s", "cores": oracle.num_threads(lib), "kind": "oracle",
                "sample": f"{128 * nb} of the {N} weight rows (K={K}) converted; {t:.1f} s"}
    if wk.name == "moe":
        e = 0   # expert 0's routed tokens against its weight (routing by the oracle)
        r = oracle.moe_route_topk(d["logits"], d["topk"], lib=lib)
        seg = r.row_token[r.offsets[e]:r.offsets[e + 1]]
        w_bits, a_src = d["w"][e], d["tokens"][seg[seg >= 0]]
    elif wk.name == "decode":
        w_bits, a_src = None, d["a"]
    elif wk.name == "down":
        w_bits, a_src = d["w"], None   # rows of SiLU(x) * y, made below by the oracle inside the timing
    else:
        w_bits, a_src = d["w"], d["a"]

    def act(r):
        if a_src is not None:
            return oracle.quant_act_1x128(a_src[:r], lib=lib)
        return oracle.swiglu_quant_1x128(d["x"][:r], d["y"][:r], lib=lib)
    t0 = time.perf_counter()
    if w_bits is not None:
        qw, sw = oracle.quant_w_128x128(w_bits, lib=lib)
    else:
        qw, sw = d["wq"], d["sw"]
    t_w = time.perf_counter() - t0
    # calibrate the GEMM rate on a few rows (one row overstates it: the call's fixed cost), then size the
    # sample to about `target_s` seconds in total
    n_src = a_src.shape[0] if a_src is not None else d["x"].shape[0]
    n_cal = min(8, n_src)
    qa, sa = act(n_cal)
    t1 = time.perf_counter()
    oracle.gemm_blockscaled(qa, sa, qw, sw, rows=np.arange(n_cal), lib=lib)
    per_row = (time.perf_counter() - t1) / n_cal
    rows = int(max(1, min(n_src, (target_s - t_w) / max(per_row, 1e-6))))
    t2 = time.perf_counter()
    qa, sa = act(rows)
    oracle.gemm_blockscaled(qa, sa, qw, sw, rows=np.arange(rows), lib=lib)
    t_rows = time.perf_counter() - t2
    total = t_w + t_rows
    flops = 2.0 * rows * N * K
    what = "expert 0's weights" if wk.name == "moe" else ("pre-quantized weights" if wk.name == "decode" else
                                                         "all weights")
    return {"value": flops / total / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(lib), "kind": "oracle",
            "sample": f"{rows} token rows x all {N} outputs (K={K}): their "
                      f"{'SwiGLU and ' if wk.name == 'down' else ''}1x128 quantization, 128x128 "
                      f"quantization of {what}, and the double-precision GEMM of those rows; {total:.1f} s"}


class HipEvents:
    """Timing events of the HIP runtime the process already uses (found in /proc/self/maps), created with
    hipEventDisableSystemFence: recording one does not add a system-scope release, which keeps the gap
    between an event and the kernel after it small."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes

        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64.so" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded")
        self.ct = ctypes
        self.hip = ctypes.CDLL(path)
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = self.ct.c_void_p()
        if self.hip.hipEventCreateWithFlags(self.ct.byref(ev), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return ev

    def record(self, ev, stream):
        if self.hip.hipEventRecord(ev, self.ct.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, ev):
        self.hip.hipEventDestroy(ev)


class _Rec:
    """Event pair endpoint with the torch.cuda.Event record() interface, on the current stream."""

    def __init__(self, he, ev):
        self.he, self.ev = he, ev

    def record(self):
        import torch

        self.he.record(self.ev, torch.cuda.current_stream().cuda_stream)


GEMM_SOURCES = ("fine_grained_quantization_amd/csrc/fp8q_gemm.hip", "fine_grained_quantization_amd/csrc/fp8q_device.h")
QUANT_SOURCES = ("fine_grained_quantization_amd/csrc/fp8q_quant.hip", "fine_grained_quantization_amd/csrc/fp8q_device.h")
# The sources each reported kernel is built from (its recorded traffic is stale once they change).
KERNEL_SOURCES = {"gemm_blockscaled": GEMM_SOURCES, "grouped_gemm_blockscaled": GEMM_SOURCES,
                  "grouped_gemm_blockscaled_gather": GEMM_SOURCES,
                  "dequant_w_128x128": QUANT_SOURCES, "quant_act_dual": QUANT_SOURCES,
                  "quant_w_fp4_128x128": QUANT_SOURCES, "quant_w_per_channel": QUANT_SOURCES,
                  "quant_act_e5m6_1x128": QUANT_SOURCES}


def sources_sha256(paths=GEMM_SOURCES):
    import hashlib

    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profiled_traffic(kname, workload):
    """HBM bytes per launch of `kname` on `workload` from its committed rocprofv3 summary, or None when
    there is none or the kernel sources differ from the ones it was taken with."""
    path = os.path.join(ROOT, "profiles", f"{kname}_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.strip().startswith(("source_sha256", "traffic_bytes_per_launch")):
                k, v = line.strip().strip("`").split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    srcs = KERNEL_SOURCES.get(kname, GEMM_SOURCES)
    if fields.get("source_sha256") != sources_sha256(srcs) or "traffic_bytes_per_launch" not in fields:
        return None
    return int(fields["traffic_bytes_per_launch"])


def measure(name, args, he, copy_gbs):
    """Settle, warm up and time `args.steps` steps of workload `name`; returns its part of the JSON line (without
    the CPU baseline) and the Workload."""
    import torch

    wk = Workload(name)
    if args.pmc_copy_mb:
        src = torch.ones(args.pmc_copy_mb << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    # Settle: a few milliseconds of warmup leave the GPU below its sustained clock (measured: the up GEMM
    # runs at 568 us after 5 steps, 490 us after 100), so repeat the step, untimed, for settle_ms first.
    clock = ClockSampler()
    clock.start()
    settle_steps = 0
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(4):
            wk.step()
        settle_steps += 4
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        wk.step()
    torch.cuda.synchronize()

    # Timed region: exactly K steps, back to back, between two synchronizations; an event pair brackets
    # every launch of the step's last (dominant) kernel in it.
    nk = len(wk.kernels)
    gemm_raw = [(he.create(), he.create()) for _ in range(args.steps)]
    gemm_ev = [[_Rec(he, a), _Rec(he, b)] for a, b in gemm_raw]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for s in range(args.steps):
        wk.step([None] * (nk - 1) + [gemm_ev[s]])
    end.record()
    torch.cuda.synchronize()
    wall1 = time.perf_counter()
    wall = wall1 - wall0
    clock.stop()
    ms_step = start.elapsed_time(end) / args.steps
    gemm_all = [1e3 * he.elapsed_ms(a, b) for a, b in gemm_raw]
    for a, b in gemm_raw:
        he.destroy(a)
        he.destroy(b)

    # The other kernels' durations: K more steps with an event pair around every launch.
    raw = [[(he.create(), he.create()) for _ in range(nk)] for _ in range(args.steps)]
    for s in range(args.steps):
        wk.step([[_Rec(he, a), _Rec(he, b)] for a, b in raw[s]])
    torch.cuda.synchronize()

    kernels = {}
    for i, (kname, _, work) in enumerate(wk.kernels):  # (all event pairs are destroyed below)
        if i == nk - 1:
            each = gemm_all  # measured in the timed region
        else:
            each = [1e3 * he.elapsed_ms(*raw[s][i]) for s in range(args.steps)]
        us = float(np.mean(each))
        # mean (used for the rates below), median and minimum over the K launches
        info = {"us": round(us, 2), "us_median": round(float(np.median(each)), 2), "us_min": round(min(each), 2)}
        if "flops" in work:
            info["TFLOP/s"] = round(work["flops"] / us / 1e6, 1)
            info["frac_fp8_peak"] = round(work["flops"] / us / 1e6 / PEAK_FP8_TFLOPS, 4)
        info["GB/s"] = round(work["bytes"] / us / 1e3, 1)
        info["frac_hbm"] = round(work["bytes"] / us / 1e3 / PEAK_HBM_GBS, 4)
        info["frac_of_measured_copy"] = round(work["bytes"] / us / 1e3 / copy_gbs, 4)
        if i in wk.side_kernels:
            info["beside_weight_quant"] = True  # its duration includes waiting for CUs the weight quantizer holds
        if kname in wk.cast_floor:
            src = wk.cast_floor[kname]
            fl = cast_floor_us(src, args.steps)
            info["torch_cast_floor"] = {"us_median": round(fl, 2), "GB/s": round(3 * src.numel() / fl / 1e3, 1),
                                        "frac_of_floor": round(fl / info["us_median"], 4)}
        kernels[kname] = info

    for pairs in raw:
        for a, b in pairs:
            he.destroy(a)
            he.destroy(b)
    gname, _, gwork = wk.kernels[-1]
    g = kernels[gname]
    traffic = profiled_traffic(gname, name)
    if name in BANDWIDTH_METRICS or name == "decode":
        roof = {"kernel": gname, "bound": "hbm", "achieved": g["GB/s"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(g["GB/s"] / PEAK_HBM_GBS, 4), "traffic": traffic}
    else:
        roof = {"kernel": gname, "bound": "mfma", "achieved": g["TFLOP/s"], "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": round(g["TFLOP/s"] / PEAK_FP8_TFLOPS, 4), "traffic": traffic}
    roof["algorithmic_bytes"] = int(gwork["bytes"])
    roof["measured_copy_GBs"] = round(copy_gbs, 1)
    if roof["bound"] == "hbm":
        roof["frac_of_measured_copy"] = round(roof["achieved"] / copy_gbs, 4)
    # The clock while the steps ran: the metrics windows that lie inside the settle phase and the timed
    # region (the timed region alone is far shorter than one window).
    clk = clock.record(t_settle, wall1)
    if roof["bound"] == "mfma" and "MHz_mean" in clk:
        # 256 CUs x 4 SIMDs x 2048 FP8 flop per clock (a 16x16x128 MFMA every 32 cycles)
        at_clock = 256 * 8192 * clk["MHz_mean"] * 1e6 / 1e12
        roof["peak_at_measured_clock"] = round(at_clock, 1)
        roof["frac_at_measured_clock"] = round(roof["achieved"] / at_clock, 4)

    dq = name in BANDWIDTH_METRICS
    part = {
        "value": round(wk.bytes / (ms_step * 1e-3) / 1e9, 1) if dq else round(wk.flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "GB/s" if dq else "TFLOP/s",
        "settle_steps": settle_steps,
        "ms_per_step": round(ms_step, 4),
        "config": {"workload": DESCRIPTIONS[name], "name": name, "M": wk.M, "N": wk.N, "K": wk.K, "out": "bf16",
                   "parallelism": "single GPU"},
        "kernels": kernels,
        "roofline": roof,
        "wall_s_timed": round(wall, 3),
        "gpu_clock": clk,
    }
    if name == "moe":
        part["config"]["rows_used"] = wk.rows_used   # M is the routing capacity the buffers are sized to
    return part, wk


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="moe", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--also", default=None,
                    help="comma-separated workloads measured after the headline one, each reported under "
                         "other_workloads with its own step time, kernels and roofline (default: up,down,decode "
                         "with the moe headline, none otherwise; 'none' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=2500.0,
                    help="before the warmup steps, repeat the step for this long (untimed) so that the GPU's "
                         "clocks reach their sustained state; the count is reported as settle_steps")
    ap.add_argument("--pmc-copy-mb", type=int, default=0,
                    help="before warmup, run one plain elementwise copy (torch.neg) of this many MiB; its "
                         "FETCH_SIZE / WRITE_SIZE under rocprofv3 calibrate the traffic counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path is built and measured for a "
              f"single MI355X.", file=sys.stderr)
        sys.exit(2)
    if args.also is None:
        also = ["up", "down", "decode"] if args.workload == "moe" else []
    else:
        also = [] if args.also in ("", "none") else args.also.split(",")
    for a in also:
        if a not in DESCRIPTIONS or a == args.workload:
            print(f"--also: {a!r} is not another workload", file=sys.stderr)
            sys.exit(2)

    import torch

    import fine_grained_quantization_amd as fq

    fq.load_library()  # fails loudly when the HIP library is missing
    torch.cuda.set_device(0)
    he = HipEvents()
    copy_gbs = measured_copy_gbs()
    part, wk = measure(args.workload, args, he, copy_gbs)
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(wk)
        cpu["cpu_model"] = cpu_model()
    del wk
    others = {}
    for a in also:
        torch.cuda.empty_cache()
        p, w = measure(a, args, he, copy_gbs)
        del w
        others[a] = {k: p[k] for k in ("value", "unit", "ms_per_step", "settle_steps", "config", "kernels",
                                       "roofline", "gpu_clock")}
        log(f"[bench] {a}: {p['ms_per_step']} ms per step")

    dq = args.workload in BANDWIDTH_METRICS
    out = {
        "metric": BANDWIDTH_METRICS[args.workload] if dq else METRIC,
        "value": part["value"],
        "unit": part["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": part["settle_steps"],
        "ms_per_step": part["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"dequant": "fp8_e4m3 -> bf16", "dual": "bf16 -> fp8_e4m3", "fp4": "bf16 -> fp4_e2m1",
                  "per_channel": "bf16 -> fp8_e4m3", "e5m6": "bf16 -> e5m6"}.get(
            args.workload, "fp8_e4m3"),
        "data": "synthetic",
        "config": part["config"],
        "kernels": part["kernels"],
        "roofline": part["roofline"],
        "wall_s_timed": part["wall_s_timed"],
        "gpu_clock": part["gpu_clock"],
    }
    if others:
        out["other_workloads"] = others
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
