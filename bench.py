#!/usr/bin/env python3
"""Benchmark of the MXFP4 mixture-of-experts layer on one MI355X.

One step = one call of the whole layer (router, top-k + softmax, permutation,
gate_up GEMM + SwiGLU, down GEMM, combine) on one batch of synthetic tokens whose
inputs are already resident in HBM. The headline workload is the GPT-OSS-20B
shaped single-token decode (T=1, H=I=2880, E=32, top-4); the skewed 64-token batched
decode, the 4096-token prefill of the same layer and the 2048-token prefill of the
120B-shaped layer (E=128) are measured in the same run (``other_workloads``).

Timing: W untimed warmup steps, then exactly K steps bracketed by torch.cuda.synchronize()
and HIP events on the stream the kernels run on; the K steps are timed 5 times and the
median is reported. The weights are replicated R times (and x drawn R times) and the steps
rotate over the replicas so that the 256 MB last-level cache cannot serve a step's weights
from the previous step. By default the steps are replayed from two HIP graphs, one captured
over a whole rotation and one over the first K mod R replicas (--mode eager launches every
call from Python instead). One cold call (after a 512 MiB write has evicted the caches) is
timed on its own.

Also reported, in the same JSON line, per workload:
* roofline: the dominant kernel's average duration, measured with the start / end HIP
  events each kernel of a moe_mxfp4_forward_timed call records around itself, turned into
  achieved GB/s and TFLOP/s from its algorithmic bytes and flops per launch, against
  MI355X's published peaks (the binding one in `frac`); `traffic` comes from the committed
  rocprofv3 counter summary for that kernel when its source has not changed since;
* cpu_baseline: the CPU oracle (expert-major mode) timed on this host on the same inputs.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--mode graph|eager]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s, 20B shape, decode & 4k prefill; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA
LLC_BYTES = 256 << 20            # MI355X Infinity Cache
KERNEL_SOURCES = {               # kernel -> files whose text defines it
    "route": ["route.hip", "device_common.h", "rms.h", "mx_mfma.h", "topk.h", "lds_dma.h"],
    "permute": ["permute.hip", "device_common.h"],
    "logits": ["route.hip", "device_common.h", "rms.h", "mx_mfma.h", "topk.h", "lds_dma.h"],
    "up_decode": ["gemm_decode.hip", "device_common.h", "weight_tiles.h", "routing.h", "topk.h", "mx_mfma.h",
                  "lds_dma.h"],
    "down_decode": ["gemm_decode.hip", "device_common.h", "weight_tiles.h", "routing.h", "topk.h", "mx_mfma.h",
                    "lds_dma.h"],
    "up_stream": ["gemm_stream.hip", "device_common.h", "weight_tiles.h", "routing.h", "lds_dma.h", "mx_mfma.h"],
    "down_stream": ["gemm_stream.hip", "device_common.h", "weight_tiles.h", "routing.h", "lds_dma.h", "mx_mfma.h"],
    "up_grouped": ["gemm_grouped.hip", "device_common.h", "lds_dma.h", "mx_mfma.h"],
    "down_grouped": ["gemm_grouped.hip", "device_common.h", "lds_dma.h", "mx_mfma.h"],
    "combine": ["gemm_grouped.hip", "device_common.h", "lds_dma.h"],
    "combine_decode": ["gemm_decode.hip", "device_common.h"],
    "rmsnorm": ["norm.hip", "device_common.h", "rms.h"],
    "up_bank": ["gemm_bank.hip", "device_common.h"],
    "down_bank": ["gemm_bank.hip", "device_common.h"],
}
FEW_STAGES = ["logits", "up_decode", "down_decode"]                       # T < 4
STREAM_STAGES = ["route", "up_stream", "down_stream", "combine_decode"]     # 4 <= T <= 64
PREFILL_STAGES = ["route", "permute", "up_grouped", "down_grouped", "combine"]


BANK_STAGES = ["route", "permute", "up_bank", "down_bank", "combine"]


def stages_of(T: int, variant: str = "layer"):
    """Kernels of one call (GPT-OSS shapes). In the pre-norm block the decode routers
    normalize the rows themselves; the prefill sequence starts with an RMSNorm kernel. The
    dequantized-bank variant takes the grouped sequence at every T."""
    if variant == "dequantized":
        return BANK_STAGES
    st = FEW_STAGES if T < 4 else (STREAM_STAGES if T <= 64 else PREFILL_STAGES)
    return (["rmsnorm"] if variant == "prenorm" and T > 64 else []) + st


def code_only(text: str) -> str:
    """The source without its comments and with whitespace runs collapsed: a comment edit does
    not change the kernel, so it does not make a profile of it stale. (The kernel sources hold
    no string literal containing a comment marker.)"""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_sha(kernel: str, read=None) -> str:
    """sha256 (16 hex digits) of the kernel's sources, code only; `read(name)` supplies a
    source's text (default: the file under csrc/)."""
    if read is None:
        def read(f):
            with open(os.path.join(ROOT, "mxfp4_mixture_experts_router_amd", "csrc", f)) as fh:
                return fh.read()
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update(code_only(read(f)).encode())
    return h.hexdigest()[:16]


OTHER_WORKLOADS = "batched_decode_20b,prefill_20b,prefill_120b"
DEFAULT_STEPS = {"decode_20b": 2000, "batched_decode_20b": 500, "prefill_20b": 100, "prefill_120b": 100,
                 "decode_20b_tp8": 2000, "batched_decode_20b_tp8": 500, "prefill_20b_ep8": 100}
REPEATS = 5


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps of the headline workload (default: 2000); the other workloads "
                         "time min(K, their default) steps")
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="decode_20b")
    ap.add_argument("--also", "--secondary", dest="also", default=OTHER_WORKLOADS,
                    help="comma-separated other workloads measured in the same run ('' to skip)")
    ap.add_argument("--repeats", type=int, default=REPEATS, help="timed repetitions (median reported)")
    ap.add_argument("--mode", choices=["graph", "eager"], default="graph")
    ap.add_argument("--replicas", type=int, default=0, help="0 = enough to defeat the LLC")
    ap.add_argument("--timed-steps", type=int, default=200, help="steps of the per-kernel timing run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold single-call timing")
    ap.add_argument("--prenorm", action="store_true",
                    help="time the pre-norm block y = x + layer(rmsnorm(x)) instead of the layer")
    ap.add_argument("--dequantized-bank", action="store_true",
                    help="time the layer on the bank dequantized once to bf16 (an ablation)")
    return ap.parse_args()


class Hip:
    """The HIP runtime already loaded in this process (the one torch and the library use)."""

    def __init__(self):
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                m = re.search(r"(/\S*libamdhip64\.so\S*)", line)
                if m:
                    path = m.group(1)
                    break
        self.lib = ctypes.CDLL(path or "libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]

    def event(self):
        ev = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(ev)) == 0
        return ev.value

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return ms.value

    def destroy(self, ev):
        self.lib.hipEventDestroy(ctypes.c_void_p(ev))


class Workload:
    """R replicas of one layer's weights and R batches of tokens, resident on the GPU."""

    WEIGHTS = ("router_w", "router_b", "gu_blocks", "gu_scales", "gu_bias", "dn_blocks",
               "dn_scales", "dn_bias")

    NORM_EPS = 1e-5

    @classmethod
    def create(cls, name: str, replicas: int, variant: str = "layer"):
        import numpy as np
        import torch
        import mxfp4_mixture_experts_router_amd as moe
        from workloads import CONFIGS, make_inputs

        self = cls()
        cfg = CONFIGS[name]
        self.name, self.cfg = name, cfg
        dev = torch.device("cuda:0")

        def up(a):
            if a.dtype == np.uint16:
                return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

        self.variant = variant
        self.prenorm = variant == "prenorm"
        self.bank = variant == "dequantized"
        self.label = name + ("" if variant == "layer" else "+" + variant)
        host_w = make_inputs(cfg, seed=0, parts=self.WEIGHTS + (("norm_w",) if self.prenorm else ()))
        self.host_weights = host_w
        layer_bytes = sum(v.nbytes for v in host_w.values())
        if self.bank:   # bf16 weights: 4 bytes per packed byte
            layer_bytes = 4 * (host_w["gu_blocks"].nbytes + host_w["dn_blocks"].nbytes)
        if replicas <= 0:
            touched = self.touched_weight_bytes_estimate(cfg, layer_bytes)
            replicas = max(2, min(16, -(-2 * LLC_BYTES // max(touched, 1)) + 1))
        self.R = replicas
        base = {k: up(v) for k, v in host_w.items()}
        self.weights = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(replicas - 1)]
        self.bank_dequant_ms = None
        if self.bank:
            # the one-off expansion, timed on the first replica
            for r, wt in enumerate(self.weights):
                E_, I2_, Hh_ = wt["gu_blocks"].shape
                outs = (torch.empty((E_, I2_, 2 * Hh_), dtype=torch.bfloat16, device=dev),
                        torch.empty((E_, Hh_ * 2, I2_ // 2), dtype=torch.bfloat16, device=dev))
                torch.cuda.synchronize()
                start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                start.record()
                wt["gu_w"], wt["dn_w"] = moe.dequantize_bank(wt["gu_blocks"], wt["gu_scales"], wt["dn_blocks"],
                                                             wt["dn_scales"], out=outs)
                end.record()
                torch.cuda.synchronize()
                if r == 0:
                    self.bank_dequant_ms = start.elapsed_time(end)
                for key in ("gu_blocks", "gu_scales", "dn_blocks", "dn_scales"):
                    del wt[key]
        self.host_x = [make_inputs(cfg, seed=r, parts=("x",))["x"] for r in range(replicas)]
        self.x = [up(x) for x in self.host_x]
        T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
        self.shape = moe._shape(T, H, I, E, k, cfg.alpha, cfg.limit)
        self.y = [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in range(replicas)]
        self.idx = [torch.empty((T, k), dtype=torch.int32, device=dev) for _ in range(replicas)]
        self.w = [torch.empty((T, k), dtype=torch.float32, device=dev) for _ in range(replicas)]
        nbytes = (moe.workspace_bytes_dequantized if self.bank else moe.workspace_bytes)(T, H, I, E, k)
        self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        self.lib = moe.load_library()
        self.layer_bytes = layer_bytes
        return self

    @staticmethod
    def touched_weight_bytes_estimate(cfg, layer_bytes):
        per_expert = layer_bytes / cfg.E
        return int(min(cfg.E, cfg.T * cfg.k) * per_expert)

    def args(self, r: int, stream_ptr: int):
        w = self.weights[r]
        P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        if self.bank:
            return (ctypes.byref(self.shape), P(self.x[r]), P(w["router_w"]), P(w["router_b"]), P(w["gu_w"]),
                    P(w["gu_bias"]), P(w["dn_w"]), P(w["dn_bias"]), P(self.y[r]), P(self.idx[r]), P(self.w[r]),
                    P(self.ws), self.ws.numel(), ctypes.c_void_p(stream_ptr))
        norm = (P(w["norm_w"]), ctypes.c_double(self.NORM_EPS)) if self.prenorm else ()
        return (ctypes.byref(self.shape), P(self.x[r]), *norm, P(w["router_w"]), P(w["router_b"]),
                P(w["gu_blocks"]), P(w["gu_scales"]), P(w["gu_bias"]), P(w["dn_blocks"]),
                P(w["dn_scales"]), P(w["dn_bias"]), P(self.y[r]), P(self.idx[r]), P(self.w[r]),
                P(self.ws), self.ws.numel(), ctypes.c_void_p(stream_ptr))

    def step(self, r: int, stream_ptr: int):
        fn = {"layer": self.lib.moe_mxfp4_forward, "prenorm": self.lib.moe_mxfp4_forward_prenorm,
              "dequantized": self.lib.moe_mxfp4_forward_dequantized}[self.variant]
        st = fn(*self.args(r, stream_ptr))
        if st != 0:
            raise RuntimeError(self.lib.moe_mxfp4_last_error().decode())


def _capture(wl: Workload, replicas):
    """A HIP graph of one call per replica in `replicas`, checked bit for bit against eager
    launches of the same calls over three replays."""
    import torch
    stream = torch.cuda.current_stream()
    ref = {r: wl.y[r].clone() for r in replicas}
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for r in replicas:
            wl.step(r, side.cuda_stream)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap = torch.cuda.current_stream()
        for r in replicas:
            wl.step(r, cap.cuda_stream)
    for _ in range(3):
        for r in replicas:
            wl.y[r].zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for r in replicas:
            if not torch.equal(wl.y[r].view(torch.int16), ref[r].view(torch.int16)):
                raise RuntimeError("graph replay differs from eager launches")
    return graph


def run_timed(wl: Workload, steps: int, warmup: int, mode: str, repeats: int):
    """Whole-layer time per step: exactly `steps` steps (rotating over the replicas), timed
    `repeats` times. Returns (median ms/step, all ms/step, wall ms/step of the median run)."""
    import torch
    stream = torch.cuda.current_stream()
    for i in range(max(warmup, wl.R)):
        wl.step(i % wl.R, stream.cuda_stream)
    torch.cuda.synchronize()
    full, rest = divmod(steps, wl.R)
    graphs = []
    if mode == "graph":
        g_all = _capture(wl, list(range(wl.R)))
        g_rest = _capture(wl, list(range(rest))) if rest else None
        graphs = [g_all] * full + ([g_rest] if g_rest is not None else [])
        for g in graphs[:2]:
            g.replay()
    torch.cuda.synchronize()
    times, walls = [], []
    for _ in range(repeats):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record(stream)
        if graphs:
            for g in graphs:
                g.replay()
        else:
            sp = stream.cuda_stream
            for i in range(steps):
                wl.step(i % wl.R, sp)
        end.record(stream)
        torch.cuda.synchronize()
        walls.append((time.perf_counter() - t0) * 1e3 / steps)
        times.append(start.elapsed_time(end) / steps)
    order = sorted(range(repeats), key=lambda i: times[i])
    med = order[repeats // 2]
    return times[med], times, walls[med]


def run_cold(wl: Workload):
    """One call after a 512 MiB write has pushed every weight byte out of the L2s and the
    last-level cache: GPU time between events recorded around the call on its stream (host
    launch included), and host wall time until it has finished."""
    import torch
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    best = None
    for _ in range(3):
        flush.fill_(1)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record(stream)
        wl.step(0, stream.cuda_stream)
        end.record(stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3
        gpu = start.elapsed_time(end)
        if best is None or gpu < best[0]:
            best = (gpu, wall)
    del flush
    return {"gpu_ms": round(best[0], 4), "wall_ms": round(best[1], 4), "runs": 3, "reported": "fastest"}


def run_per_kernel(wl: Workload, steps: int, hip: Hip):
    """Average duration of each kernel of the layer, from the start / end events each kernel
    records around its own execution (moe_mxfp4_forward_timed), on the stream it runs on."""
    import torch
    import mxfp4_mixture_experts_router_amd as moe
    lib = wl.lib
    stream = torch.cuda.current_stream()
    n_ev = 2 * moe.MAX_LAUNCHES
    events = [[hip.event() for _ in range(n_ev)] for _ in range(steps)]
    arrays = [(ctypes.c_void_p * n_ev)(*evs) for evs in events]
    n_launch = ctypes.c_int(0)
    torch.cuda.synchronize()
    fn = {"layer": lib.moe_mxfp4_forward_timed, "prenorm": lib.moe_mxfp4_forward_prenorm_timed,
          "dequantized": lib.moe_mxfp4_forward_dequantized_timed}[wl.variant]
    for i in range(steps):
        st = fn(*wl.args(i % wl.R, stream.cuda_stream), arrays[i], n_ev, ctypes.byref(n_launch))
        if st != 0:
            raise RuntimeError(lib.moe_mxfp4_last_error().decode())
    torch.cuda.synchronize()
    n = n_launch.value
    sums = [0.0] * n
    for evs in events:
        for j in range(n):
            sums[j] += hip.elapsed_ms(evs[2 * j], evs[2 * j + 1])
    for evs in events:
        for ev in evs:
            hip.destroy(ev)
    return [s / steps * 1e3 for s in sums]   # microseconds


def distinct_experts(wl: Workload):
    import numpy as np
    return float(np.mean([len(np.unique(i.cpu().numpy())) for i in wl.idx]))


def kernel_work(wl: Workload, kernel: str, D: float):
    """Algorithmic bytes and flops of one launch of `kernel` (what the method must move or
    compute; D = distinct routed experts)."""
    c = wl.cfg
    T, H, I, E, k = c.T, c.H, c.I, c.E, c.k
    N = T * k
    gu_expert = 2 * I * (H // 2) + 2 * I * (H // 32) + 2 * I * 2      # packed + scales + bias
    dn_expert = H * (I // 2) + H * (I // 32) + H * 2
    res = T * H * 2 if wl.prenorm else 0      # the residual the last kernel adds
    if kernel == "rmsnorm":
        return 2 * T * H * 2 + H * 2, 0
    gam = H * 2 if wl.prenorm and T <= 64 else 0    # the decode routers also read the norm weights
    if kernel == "route":
        return T * H * 2 + E * H * 2 + E * 2 + N * 8 + gam, 2 * T * E * H
    if kernel == "logits":
        return T * H * 2 + E * H * 2 + E * 2 + T * E * 8 + gam, 2 * T * E * H
    if kernel == "permute":
        return N * 8 + (E + 1) * 4 + N * 12, 0
    if kernel in ("up_decode", "up_stream"):
        return D * gu_expert + T * H * 2 + N * 8 + N * I * 2, 2 * N * 2 * I * H
    if kernel == "down_decode":      # y directly
        return D * dn_expert + N * I * 2 + N * 8 + T * H * 2 + res, 2 * N * H * I
    if kernel == "down_stream":      # per-slot partial rows
        return D * dn_expert + N * I * 2 + N * 8 + N * H * 4, 2 * N * H * I
    if kernel == "up_bank":          # bf16 weights and bias of the routed experts
        return D * (2 * I * H * 2 + 2 * I * 2) + T * H * 2 + N * 4 + N * I * 2, 2 * N * 2 * I * H
    if kernel == "down_bank":
        return D * (H * I * 2 + H * 2) + N * I * 2 + N * 8 + N * H * 4, 2 * N * H * I
    if kernel == "up_grouped":
        return D * gu_expert + T * H * 2 + N * 4 + N * I * 2, 2 * N * 2 * I * H
    if kernel == "down_grouped":
        return D * dn_expert + N * I * 2 + N * 4 + N * H * 4, 2 * N * H * I
    if kernel == "combine":
        return N * H * 4 + N * 4 + T * H * 2 + res, 0
    if kernel == "combine_decode":
        return N * H * 4 + T * H * 2 + res, 0
    raise KeyError(kernel)


def load_traffic(workload: str, kernel: str):
    if "+" in workload:
        return None
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        line = line.strip()
        if line.startswith("{"):
            rec = json.loads(line)
            if rec.get("source_sha") == kernel_source_sha(kernel):
                return rec.get("traffic_bytes")
    return None


def roofline_for(wl: Workload, stages, kernel_us, D):
    entries = []
    for name, us in zip(stages, kernel_us):
        nbytes, flops = kernel_work(wl, name, D)
        gbs = nbytes / (us * 1e-6) / 1e9
        tfs = flops / (us * 1e-6) / 1e12
        entries.append({"kernel": name, "avg_us": round(us, 3), "alg_bytes": int(nbytes),
                        "alg_flops": int(flops), "GB/s": round(gbs, 1), "TFLOP/s": round(tfs, 2)})
    dom = max(range(len(entries)), key=lambda i: entries[i]["avg_us"])
    e = entries[dom]
    # bound: arithmetic intensity against the bf16 ridge point
    intensity = e["alg_flops"] / max(e["alg_bytes"], 1)
    if intensity > BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": e["TFLOP/s"], "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(e["TFLOP/s"] / BF16_PEAK_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": e["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(e["GB/s"] / HBM_PEAK_GBS, 4)}
    roof["hbm_frac"] = round(e["GB/s"] / HBM_PEAK_GBS, 4)
    roof["mfma_frac"] = round(e["TFLOP/s"] / BF16_PEAK_TFLOPS, 4)
    roof["kernel"] = e["kernel"]
    roof["alg_bytes_per_launch"] = e["alg_bytes"]
    roof["alg_flops_per_launch"] = e["alg_flops"]
    roof["avg_us"] = e["avg_us"]
    roof["traffic"] = load_traffic(wl.label, e["kernel"])
    return roof, entries


def measure(name, steps, warmup, mode, replicas, timed_steps, hip, variant="layer", repeats=REPEATS,
            cold=True):
    wl = Workload.create(name, replicas, variant)
    ms, all_ms, wall_ms = run_timed(wl, steps, warmup, mode, repeats)
    D = distinct_experts(wl)
    stages = stages_of(wl.cfg.T, variant)
    kus = run_per_kernel(wl, timed_steps, hip)
    roof, kernels = roofline_for(wl, stages, kus, D)
    layer_bytes = sum(kernel_work(wl, s, D)[0] for s in stages)
    layer_flops = sum(kernel_work(wl, s, D)[1] for s in stages)
    return wl, {
        "ms_per_step": ms, "ms_per_step_repeats": [round(t, 6) for t in all_ms],
        "wall_ms_per_step": wall_ms, "steps": steps, "mode": mode,
        "value": wl.cfg.T / (ms * 1e-3), "distinct_experts": D, "roofline": roof,
        "kernels": kernels, "bank_dequant_ms": wl.bank_dequant_ms,
        "cold_call": run_cold(wl) if cold else None,
        "layer": {"alg_bytes": int(layer_bytes), "alg_flops": int(layer_flops),
                  "hbm_frac": round(layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                  "mfma_frac": round(layer_flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
    }


def cpu_threads():
    """Threads the oracle uses: OpenMP's (its C loops) and the BLAS library's (its matrix
    products)."""
    import oracle
    omp = oracle.max_threads()
    blas = None
    try:
        import threadpoolctl
        blas = max((p["num_threads"] for p in threadpoolctl.threadpool_info() if p.get("user_api") == "blas"),
                   default=None)
    except Exception:   # threadpoolctl missing or unreadable: report OpenMP's count only
        blas = None
    return omp, blas


def cpu_baseline(wl: Workload):
    """The oracle's expert-major mode on the same inputs as replica 0 (all T tokens): the median
    of 3 runs up to 64 tokens, one run above."""
    import numpy as np
    import oracle
    inp = dict(wl.host_weights)
    inp["x"] = wl.host_x[0]
    runs = 3 if wl.cfg.T <= 64 else 1
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        if wl.prenorm:
            oracle.forward_prenorm_expert_major(inp, wl.cfg.k, alpha=wl.cfg.alpha, limit=wl.cfg.limit,
                                                eps=wl.NORM_EPS)
        else:
            oracle.forward_expert_major(inp, wl.cfg.k, alpha=wl.cfg.alpha, limit=wl.cfg.limit)
        ts.append(time.perf_counter() - t0)
    dt = float(np.median(ts))
    omp, blas = cpu_threads()
    return {"value": round(wl.cfg.T / dt, 4), "unit": "tokens/s", "cores": max(omp, blas or 0),
            "kind": "oracle",
            "sample": f"the whole {wl.label} workload ({wl.cfg.T} tokens, same weights and x as the GPU's "
                      f"replica 0), oracle expert-major mode (fp64: C dequantization and SwiGLU with OpenMP, "
                      f"float64 BLAS matrix products), {'median of 3 runs' if runs > 1 else 'one run'}, "
                      f"{dt:.2f} s per run",
            "omp_threads": omp, "blas_threads": blas}


def host_info():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    git = None
    try:
        import subprocess
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True, timeout=5)
        git = r.stdout.strip() or None if r.returncode == 0 else None
    except Exception:   # no git, or not a checkout (the source hash below still identifies the code)
        git = None
    h = hashlib.sha256()
    for sub in ("include", os.path.join("mxfp4_mixture_experts_router_amd", "csrc")):
        d = os.path.join(ROOT, sub)
        for f in sorted(os.listdir(d)):
            with open(os.path.join(d, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    lib_sha = h.hexdigest()[:16]
    with open(os.path.abspath(__file__), "rb") as fh:
        h.update(fh.read())
    # what the library was built from (written by the build next to it): the commit, when this
    # run's tree has no history, and whether the library matches the sources in this tree
    build = None
    try:
        with open(os.path.join(ROOT, "mxfp4_mixture_experts_router_amd", "build_info.json")) as f:
            info = json.load(f)
        build = {"git_sha": info.get("git_sha"), "sources_dirty": info.get("sources_dirty"),
                 "library_matches_sources": info.get("sources_sha16") == lib_sha}
        if git is None:
            git = info.get("git_sha")
    except (OSError, ValueError):
        pass
    return {"cpu_model": model, "host_cores": len(os.sched_getaffinity(0)), "git_sha": git,
            "source_sha16": h.hexdigest()[:16], "build": build}


def hbm_probe():
    """Bandwidth of this GPU's HBM with plain library kernels, as context for the roofline's
    published 8 TB/s: a 1 GiB device-to-device copy (bytes read + written) and a reduction over
    2 GiB of fp32 (bytes read), best of 5 each."""
    import torch

    def best_ms(fn):
        fn()
        torch.cuda.synchronize()
        best = None
        for _ in range(5):
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            start.record()
            fn()
            end.record()
            torch.cuda.synchronize()
            ms = start.elapsed_time(end)
            best = ms if best is None else min(best, ms)
        return best

    a = torch.ones(1 << 29, dtype=torch.float32, device="cuda")
    read = 4 * (1 << 29) / (best_ms(lambda: a.sum()) * 1e-3) / 1e9
    src = a[: 1 << 28]
    dst = torch.empty_like(src)
    copy = 2 * 4 * (1 << 28) / (best_ms(lambda: dst.copy_(src)) * 1e-3) / 1e9
    del a, dst
    return {"copy_GBps": round(copy, 1), "sum_read_GBps": round(read, 1),
            "method": "torch copy of 1 GiB (read + write bytes) and torch.sum over 2 GiB fp32, best of 5"}


def clock_probe():
    """The shader clock under a full-chip ALU load (the library's clock probe: 1024 workgroups
    timing a dependent multiply-add chain with the shader cycle counter against the constant
    100 MHz counter), as context for the peak rates, which assume 2.4 GHz; median of 5."""
    import torch
    import mxfp4_mixture_experts_router_amd as moe
    lib = moe.load_library()
    blocks = 1024
    buf = torch.zeros(2 * blocks, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    mhz = []
    for _ in range(6):
        st = lib.moe_mxfp4_clock_probe(ctypes.c_void_p(buf.data_ptr()), blocks, 200000, ctypes.c_void_p(stream))
        if st != 0:
            raise RuntimeError(lib.moe_mxfp4_last_error().decode())
        torch.cuda.synchronize()
        c = buf.view(blocks, 2).cpu()
        mhz.append(100.0 * float(c[:, 0].sum()) / float(c[:, 1].sum()))
    mhz = sorted(mhz[1:])
    return {"sclk_MHz": round(mhz[len(mhz) // 2], 1), "method": "library clock probe: shader cycles / 100 MHz "
            "ticks over a dependent FMA chain on 1024 workgroups, median of 5"}


def record(wl, res, cpu):
    cfg = wl.cfg
    out = {
        "workload": wl.label, "T": cfg.T, "H": cfg.H, "I": cfg.I, "E": cfg.E, "k": cfg.k,
        "value": round(res["value"], 2), "unit": "tokens/s",
        "ms_per_step": round(res["ms_per_step"], 6), "ms_per_step_repeats": res["ms_per_step_repeats"],
        "steps": res["steps"], "replicas": wl.R, "mode": res["mode"],
        "distinct_experts_per_step": res["distinct_experts"],
        "roofline": res["roofline"], "layer_roofline": res["layer"], "kernels": res["kernels"],
        "wall_ms_per_step": round(res["wall_ms_per_step"], 6), "cold_call": res["cold_call"],
    }
    if res["bank_dequant_ms"]:
        out["bank_dequant_ms"] = round(res["bank_dequant_ms"], 4)
    if cpu is not None:
        out["cpu_baseline"] = cpu
    return out


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer's multi-GPU sharding is described, not implemented; the per-GPU shard "
              "shapes run as the workloads decode_20b_tp8, batched_decode_20b_tp8 and prefill_20b_ep8).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import mxfp4_mixture_experts_router_amd as moe
    if not os.path.exists(moe.library_path()):
        from mxfp4_mixture_experts_router_amd import build
        build.build()
    moe.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    hip = Hip()
    if args.prenorm and args.dequantized_bank:
        print("--prenorm and --dequantized-bank are separate variants", file=sys.stderr)
        sys.exit(2)
    variant = "prenorm" if args.prenorm else ("dequantized" if args.dequantized_bank else "layer")
    steps = args.steps if args.steps is not None else DEFAULT_STEPS.get(args.workload, 100)
    wl, main_res = measure(args.workload, steps, args.warmup, args.mode, args.replicas,
                           args.timed_steps, hip, variant, args.repeats, not args.no_cold)
    cfg = wl.cfg
    out = {
        "metric": METRIC,
        "value": round(main_res["value"], 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": main_res["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.label, "T": cfg.T, "H": cfg.H, "I": cfg.I, "E": cfg.E, "k": cfg.k,
                   "experts": "mxfp4 e2m1 + e8m0 per 32", "replicas": wl.R, "mode": main_res["mode"],
                   "distinct_experts_per_step": main_res["distinct_experts"]},
        "roofline": main_res["roofline"],
        "layer_roofline": main_res["layer"],
        "timing": {"repeats": args.repeats, "reported": "median", "ms_per_step_repeats":
                   main_res["ms_per_step_repeats"]},
        "cold_call": main_res["cold_call"],
        "wall_ms_per_step": round(main_res["wall_ms_per_step"], 6),
        "kernels": main_res["kernels"],
        **({"bank_dequant_ms": round(main_res["bank_dequant_ms"], 4)} if main_res["bank_dequant_ms"] else {}),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl)
    del wl
    torch.cuda.empty_cache()
    others = []
    for name in [n for n in args.also.split(",") if n and n != args.workload]:
        st = min(steps, DEFAULT_STEPS.get(name, 100)) if args.steps is not None else DEFAULT_STEPS.get(name, 100)
        wl2, res2 = measure(name, st, min(args.warmup, 10), args.mode, 0, min(args.timed_steps, 50), hip,
                            variant, args.repeats, not args.no_cold)
        cpu2 = None if args.no_cpu_baseline else cpu_baseline(wl2)
        others.append(record(wl2, res2, cpu2))
        del wl2
        torch.cuda.empty_cache()
    if others:
        out["other_workloads"] = others
    out["host"] = host_info()
    out["hbm_probe"] = hbm_probe()
    out["clock_probe"] = clock_probe()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
