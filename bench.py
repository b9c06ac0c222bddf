#!/usr/bin/env python3
"""Benchmark of the any-precision MoE expert layer on one MI355X.

Default run (the suite): every GPU workload of the layer, measured in one process.
  - headline: the Mixtral-8x7B-shaped expert set of 32 layers resident in HBM
    (45 GB of planes), a decode batch of 32 tokens through all 32 MoE layers under
    q map A (mean 6 bits); then map B (mean 4 bits) committed at a launch boundary.
    One step = the 32 layers, one apmoe_moe_forward call each.
  - sub-records: the Mixtral-8x7B decode layer (16 tokens), the Zipf-skewed
    Mixtral-8x22B decode layer (256 tokens), the Mixtral-8x7B prefill layer (4096
    tokens).  One step = one layer (route, gate_up with the activation, down,
    combine); two weight copies alternate between steps for the single-layer decode
    workloads, so no step reads weights the last one left in the caches.
Inputs are seeded and synthetic (no trained weights), resident before timing.

Timing, per workload: warm-up of at least --warmup steps, continued until the
per-step times settle (the GPU clock ramps up over the first ~0.1-1 s of load);
then exactly --steps steps timed as one loop between two HIP events (the mean,
ms_per_step); then a second pass of --steps steps with an event between steps for
the median and p10/p90; then a third pass with events around the two product calls
(the kernel timings of the roofline).  The roofline's dominant kernel is the gate_up
product call (with the activation in its epilogue): algorithmic bytes (or FLOPs, on
the prefill layer) per call over its mean duration.

Prints one JSON line.  --workload NAME runs a single workload instead (studies and
profiles).
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import statistics
import sys
import time

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X published dense fp16 matrix peak
ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "any_precision_weight_amd", "csrc")
KERNEL_SOURCES = ["gemm.hip", "gemm_tile.hip", "device.h", "internal.h"]
METRIC = "decode tokens/s + achieved HBM GB/s (% peak), fused any-precision MoE layer"
HEADLINE = "mixtral8x7b_32layer_decode_t32"
SUBRECORDS = ["mixtral8x7b_decode_t16", "mixtral8x22b_decode_t256_zipf", "mixtral8x7b_prefill_t4096_zipf"]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_sha256(names):
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profiled_traffic(workload):
    """HBM bytes per gate_up product call from the committed counter summary
    profiles/gemm_gate_up_<workload>_counters.md (FETCH_SIZE + WRITE_SIZE, scaled by
    a plain copy of known size), or None when there is none or the kernel sources
    have changed since it was taken."""
    path = os.path.join(PROFILES, f"gemm_gate_up_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.strip().startswith("- "):
                k, v = line.strip()[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel sources sha256") != source_sha256(KERNEL_SOURCES):
        return None
    try:
        return int(fields["traffic bytes per launch"])
    except (KeyError, ValueError):
        return None


def weight_bytes(cfg, counts, qmap, kind):
    """Eq. 3 bytes of the active blocks of one kind: planes 0..q-1 and LUT level q."""
    N, K = cfg.block_shape(kind)
    return sum(N * int(qmap[e, kind]) * K // 8 + N * (1 << int(qmap[e, kind])) * 2
               for e, c in enumerate(counts) if c)


def product_bytes(cfg, counts, qmap, kind):
    """Bytes one product call must move: the active blocks' Eq. 3 bytes, the input
    rows it reads and the output rows it writes (gate_up writes the activation a,
    fp16 [rows][F]; down writes y, fp32 [rows][H])."""
    N, K = cfg.block_shape(kind)
    rows = int(sum(counts))
    in_bytes = cfg.tokens * K * 2 if kind == 0 else rows * K * 2  # x [T][H] once; a [rows][F]
    out_bytes = rows * (N // 2) * 2 if kind == 0 else rows * N * 4
    return weight_bytes(cfg, counts, qmap, kind) + in_bytes + out_bytes


def layer_bytes(cfg, counts, qmap):
    """Whole-layer algorithmic bytes: active weights + x + router + out + routing metadata."""
    T, H, E, k = cfg.tokens, cfg.hidden, cfg.experts, cfg.assign
    w = weight_bytes(cfg, counts, qmap, 0) + weight_bytes(cfg, counts, qmap, 1)
    return w + 2 * T * H + 2 * E * H + 2 * T * H + 12 * T * k


def layer_flops(cfg):
    return 2 * cfg.tokens * cfg.assign * 3 * cfg.hidden * cfg.ffn + 2 * cfg.tokens * cfg.experts * cfg.hidden


def pct(xs, p):
    s = sorted(xs)
    i = min(len(s) - 1, max(0, int(round(p / 100.0 * (len(s) - 1)))))
    return s[i]


def host_info():
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "host_cores": len(os.sched_getaffinity(0))}


# ----------------------------------------------------------------------------- timing

class Timer:
    """Warm-up until settled, the timed loop, the per-step distribution and the
    per-kernel pass, all on the current torch stream."""

    def __init__(self, args):
        self.args = args

    def settle(self, step):
        import torch
        ev = lambda: torch.cuda.Event(enable_timing=True)
        times = []
        t0 = time.perf_counter()
        n = 0
        while True:
            a, b = ev(), ev()
            a.record()
            step(n)
            b.record()
            b.synchronize()
            times.append(a.elapsed_time(b))
            n += 1
            el = time.perf_counter() - t0
            if n >= self.args.warmup and el >= self.args.settle_min_s and len(times) >= 6:
                last = times[-5:]
                if max(last) <= 1.03 * min(last) or el >= self.args.settle_max_s:
                    break
        return n, times

    def loop(self, step, start):
        import torch
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(self.args.steps):
            step(start + i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / self.args.steps

    def distribution(self, step, start):
        import torch
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(self.args.steps + 1)]
        torch.cuda.synchronize()
        evs[0].record()
        for i in range(self.args.steps):
            step(start + i)
            evs[i + 1].record()
        torch.cuda.synchronize()
        d = [evs[i].elapsed_time(evs[i + 1]) for i in range(self.args.steps)]
        return {"median_ms": round(statistics.median(d), 5), "p10_ms": round(pct(d, 10), 5),
                "p90_ms": round(pct(d, 90), 5)}

    def kernels(self, step_split, start):
        """step_split(i, evs) runs step i with events around the product calls;
        returns mean ms per step of gate_up and down."""
        import torch
        tot = {"gate_up": 0.0, "down": 0.0}
        torch.cuda.synchronize()
        marks = [step_split(start + i) for i in range(self.args.steps)]
        torch.cuda.synchronize()
        for m in marks:
            for name, pairs in m.items():
                tot[name] += sum(p[0].elapsed_time(p[1]) for p in pairs)
        return {k: v / self.args.steps for k, v in tot.items()}


def new_event_pair():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


# ----------------------------------------------------------------------------- workloads

class SingleLayer:
    """One MoE layer of a workload resident on the GPU (copies alternate by step)."""

    def __init__(self, cfg, copies, uniform_q=0):
        import numpy as np
        import torch

        import any_precision_weight_amd as apw
        import synth
        import synth.gpu
        from any_precision_weight_amd.resident import ResidentWeights

        self.np, self.torch, self.apw = np, torch, apw
        self.cfg = cfg
        self.ctx = apw.Context(0)
        self.copies = copies
        E = cfg.weight_experts
        self.q = synth.gen_qmap(cfg, 0)
        if uniform_q:
            self.q[:] = uniform_q
        self.rw = ResidentWeights(self.ctx, copies, E)
        for e in range(E):
            for u in (0, 1):
                P, L8 = synth.gpu.planes(cfg, 0, e, u), synth.gpu.parent_lut(cfg, 0, e, u)
                for c in range(copies):
                    self.rw.add_block(c, e, u, P, L8, int(self.q[e, u]))
                del P, L8
        self.rw.commit()
        self.x = synth.gen_x(cfg, 0)
        self.wr = synth.gen_router(cfg, 0)
        self.bias = synth.gen_bias(cfg, 0)
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        self.x_d, self.wr_d = dev(self.x), dev(self.wr)
        self.bias_d = None if self.bias is None else dev(self.bias)
        T, k, H, F = cfg.tokens, cfg.assign, cfg.hidden, cfg.ffn
        R = T * k
        z = lambda shape, dt: torch.empty(shape, dtype=dt, device="cuda")
        self.b = dict(ids=z((T, k), torch.int32), w=z((T, k), torch.float32), counts=z(E, torch.int32),
                      offsets=z(E + 1, torch.int32), perm=z(R, torch.int32), inv=z(R, torch.int32),
                      a=z((R, F), torch.float16), y=z((R, H), torch.float32), out=z((T, H), torch.float16))
        self.nbytes = apw.moe_workspace(self.rw.table, 0, T, cfg.topk, cfg.shared)
        self.ws = z(self.nbytes, torch.uint8)

    def step(self, i):
        """One layer through apmoe_moe_forward (the timed form)."""
        cfg = self.cfg
        self.apw.moe_forward(self.ctx, self.rw.table, i % self.copies, self.x_d, self.wr_d, self.bias_d, cfg.tokens,
                             cfg.topk, cfg.renormalize, self.ws, self.nbytes, self.b["out"], n_shared=cfg.shared)

    def step_split(self, i):
        """The same four steps as separate calls, with events around the products."""
        apw, b, cfg, c = self.apw, self.b, self.cfg, self.ctx
        T, k, H, E = cfg.tokens, cfg.assign, cfg.hidden, cfg.experts
        slot = i % self.copies
        apw.route(c, self.x_d, self.wr_d, self.bias_d, T, H, E, cfg.topk, cfg.renormalize, b["ids"], b["w"],
                  b["counts"], b["offsets"], b["perm"], b["inv"], n_shared=cfg.shared)
        gu, dn = new_event_pair(), new_event_pair()
        gu[0].record()
        apw.gemm_act(c, self.rw.table, slot, self.x_d, True, b["perm"], b["offsets"], T, k, b["a"])
        gu[1].record()
        dn[0].record()
        apw.gemm(c, self.rw.table, slot, apw.DOWN, b["a"], False, b["perm"], b["offsets"], T, k, b["y"], apw.F32)
        dn[1].record()
        apw.combine(c, b["y"], apw.F32, b["w"], b["inv"], T, k, H, b["out"])
        return {"gate_up": [gu], "down": [dn]}

    def counts(self):
        return [self.np.asarray(self.b["counts"].cpu())]

    def qmaps(self):
        return [self.q]

    def close(self):
        self.rw.close()
        self.ctx.close()


class StackedLayers:
    """Every layer of a multi-layer workload resident at once (planes generated on
    the device); one step = the whole stack, one apmoe_moe_forward per layer."""

    def __init__(self, cfg):
        import numpy as np
        import torch

        import any_precision_weight_amd as apw
        import synth
        import synth.gpu
        from any_precision_weight_amd.resident import ResidentWeights

        self.np, self.torch, self.apw = np, torch, apw
        self.cfg = cfg
        Ln, E, T, H = cfg.layers, cfg.weight_experts, cfg.tokens, cfg.hidden
        self.ctx = apw.Context(0)
        self.rw = ResidentWeights(self.ctx, Ln, E)
        self.qa = [synth.gen_qmap(cfg, l, 0) for l in range(Ln)]
        self.qb = [synth.gen_qmap(cfg, l, 1) for l in range(Ln)]
        for l in range(Ln):
            for e in range(E):
                for u in (0, 1):
                    self.rw.add_block(l, e, u, synth.gpu.planes(cfg, l, e, u), synth.gpu.parent_lut(cfg, l, e, u),
                                      int(self.qa[l][e, u]))
            if l % 8 == 7:
                log(f"{cfg.name}: {l + 1} of {Ln} layers resident")
        self.rw.commit()
        self.q = self.qa
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        self.xs = [dev(synth.gen_x(cfg, l)) for l in range(Ln)]
        self.wrs = [dev(synth.gen_router(cfg, l)) for l in range(Ln)]
        self.nbytes = apw.moe_workspace(self.rw.table, 0, T, cfg.topk, cfg.shared)
        self.ws = torch.empty(self.nbytes, dtype=torch.uint8, device="cuda")
        self.outs = [torch.empty((T, H), dtype=torch.float16, device="cuda") for _ in range(Ln)]
        k, Et = cfg.assign, E
        z = lambda n, dt: torch.empty(n, dtype=dt, device="cuda")
        self.b = dict(ids=z(T * k, torch.int32), w=z(T * k, torch.float32), counts=z(Et, torch.int32),
                      offsets=z(Et + 1, torch.int32), perm=z(T * k, torch.int32), inv=z(T * k, torch.int32),
                      a=z((T * k, cfg.ffn), torch.float16), y=z((T * k, H), torch.float32))
        # per-layer routed counts (the same inputs route the same way under either map)
        self._counts = []
        for l in range(Ln):
            apw.route(self.ctx, self.xs[l], self.wrs[l], None, T, H, cfg.experts, cfg.topk, cfg.renormalize,
                      self.b["ids"], self.b["w"], self.b["counts"], self.b["offsets"], self.b["perm"], self.b["inv"],
                      n_shared=cfg.shared)
            self._counts.append(np.asarray(self.b["counts"].cpu()))

    def use_map(self, which):
        """Stage q map A or B for every layer and commit it on the current stream."""
        maps = self.qa if which == "A" else self.qb
        for l in range(self.cfg.layers):
            self.rw.stage_qmap(l, maps[l])
        self.rw.commit()
        self.q = maps

    def step(self, i):
        cfg, apw = self.cfg, self.apw
        for l in range(cfg.layers):
            apw.moe_forward(self.ctx, self.rw.table, l, self.xs[l], self.wrs[l], None, cfg.tokens, cfg.topk,
                            cfg.renormalize, self.ws, self.nbytes, self.outs[l], n_shared=cfg.shared)

    def step_split(self, i):
        apw, b, cfg, c = self.apw, self.b, self.cfg, self.ctx
        T, k, H, E = cfg.tokens, cfg.assign, cfg.hidden, cfg.experts
        marks = {"gate_up": [], "down": []}
        for l in range(cfg.layers):
            apw.route(c, self.xs[l], self.wrs[l], None, T, H, E, cfg.topk, cfg.renormalize, b["ids"], b["w"],
                      b["counts"], b["offsets"], b["perm"], b["inv"], n_shared=cfg.shared)
            gu, dn = new_event_pair(), new_event_pair()
            gu[0].record()
            apw.gemm_act(c, self.rw.table, l, self.xs[l], True, b["perm"], b["offsets"], T, k, b["a"])
            gu[1].record()
            dn[0].record()
            apw.gemm(c, self.rw.table, l, apw.DOWN, b["a"], False, b["perm"], b["offsets"], T, k, b["y"], apw.F32)
            dn[1].record()
            apw.combine(c, b["y"], apw.F32, b["w"], b["inv"], T, k, H, self.outs[l])
            marks["gate_up"].append(gu)
            marks["down"].append(dn)
        return marks

    def counts(self):
        return self._counts

    def qmaps(self):
        return self.q

    def close(self):
        self.rw.close()
        self.ctx.close()


def measure(timer, wl, label):
    """Settle, time, distribution, kernels; returns the record of one workload."""
    cfg = wl.cfg
    n_w, wt = timer.settle(wl.step)
    log(f"{label}: warm-up {n_w} steps, first {wt[0]:.3f} ms, last {wt[-1]:.3f} ms")
    ms = timer.loop(wl.step, n_w)
    dist = timer.distribution(wl.step, n_w + timer.args.steps)
    kern = timer.kernels(wl.step_split, n_w + 2 * timer.args.steps)
    counts, qmaps = wl.counts(), wl.qmaps()
    L = len(counts)
    lb = sum(layer_bytes(cfg, counts[l], qmaps[l]) for l in range(L))
    gu_b = sum(product_bytes(cfg, counts[l], qmaps[l], 0) for l in range(L))
    dn_b = sum(product_bytes(cfg, counts[l], qmaps[l], 1) for l in range(L))
    flops = layer_flops(cfg) * L
    gu_flops = 2 * cfg.tokens * cfg.assign * 2 * cfg.ffn * cfg.hidden * L
    gbs = lb / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    gu_ms, dn_ms = kern["gate_up"], kern["down"]
    gu_gbs = gu_b / (gu_ms * 1e-3) / 1e9
    dn_gbs = dn_b / (dn_ms * 1e-3) / 1e9
    gu_tf = gu_flops / (gu_ms * 1e-3) / 1e12
    rec = {
        "workload": cfg.name, "layers": L, "tokens": cfg.tokens, "hidden": cfg.hidden, "ffn": cfg.ffn,
        "experts": cfg.experts, "topk": cfg.topk,
        "mean_bits": round(float(sum(q.mean() for q in qmaps) / L), 3),
        "tokens_per_s": round(cfg.tokens / (ms * 1e-3), 1),
        "ms_per_step": round(ms, 5), **dist,
        "warmup_steps_run": n_w,
        "layer_gbps": round(gbs, 1), "layer_hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "layer_tflops": round(tflops, 2), "layer_mfma_frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
        "algorithmic_bytes_per_step": lb, "algorithmic_flops_per_step": flops,
        "kernels_us_per_step": {"gate_up": round(gu_ms * 1e3, 2), "down": round(dn_ms * 1e3, 2)},
        "down": {"achieved_gbps": round(dn_gbs, 1), "hbm_frac": round(dn_gbs / HBM_PEAK_GBS, 4)},
    }
    if L == 1:
        rec["counts"] = [int(c) for c in counts[0]]
    # the gate_up product call is the dominant kernel; HBM-bound below the ridge point
    # (peak FLOP/s over peak bytes/s), MFMA-bound above it
    if gu_flops / gu_b > MFMA_F16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        rec["roofline"] = {"kernel": "apmoe_gemm_act (gate_up product + activation)", "bound": "mfma",
                           "achieved": round(gu_tf, 1), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(gu_tf / MFMA_F16_PEAK_TFLOPS, 4), "algorithmic_flops": gu_flops // L,
                           "traffic": profiled_traffic(cfg.name),
                           "hbm_achieved_gbps": round(gu_gbs, 1)}
    else:
        rec["roofline"] = {"kernel": "apmoe_gemm_act (gate_up product + activation)", "bound": "hbm",
                           "achieved": round(gu_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(gu_gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": gu_b // L,
                           "traffic": profiled_traffic(cfg.name),
                           "mfma_achieved_tflops": round(gu_tf, 1)}
    log(f"{label}: step {ms * 1e3:.1f} us (median {dist['median_ms'] * 1e3:.1f}, p10 {dist['p10_ms'] * 1e3:.1f}, "
        f"p90 {dist['p90_ms'] * 1e3:.1f})  {gbs:.0f} GB/s  {tflops:.1f} TFLOP/s  gate_up {gu_ms * 1e3:.1f} us "
        f"({gu_gbs:.0f} GB/s, {gu_tf:.0f} TFLOP/s)  down {dn_ms * 1e3:.1f} us ({dn_gbs:.0f} GB/s)")
    return rec


def stream_ceiling():
    """Practical HBM rates of this GPU over 2 GiB (beyond the 256 MB last-level
    cache), best of 10: a plain read stream (libhbmprobe.so: 16-byte non-temporal
    loads, 4096 workgroups) and a device copy (PyTorch)."""
    import ctypes

    import torch
    n = 2 << 30
    a = torch.empty(n // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    probe = ctypes.CDLL(os.path.join(ROOT, "any_precision_weight_amd", "libhbmprobe.so"))
    probe.hbm_read_probe.restype = ctypes.c_int
    probe.hbm_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    blocks = 4096
    sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")

    def read():
        rc = probe.hbm_read_probe(a.data_ptr(), n, sink.data_ptr(), blocks, torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"hbm_read_probe: hipError {rc}")

    res = {}
    for name, fn, nbytes in (("read_gbps", read, n), ("copy_gbps", lambda: b.copy_(a), 2 * n)):
        for _ in range(3):
            fn()
        best = 1e30
        for _ in range(10):
            e0, e1 = new_event_pair()
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            best = min(best, e0.elapsed_time(e1))
        res[name] = round(nbytes / (best * 1e-3) / 1e9, 1)
    del a, b, sink
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- CPU baseline

def oracle_layer_time(cfg, layer, qmap, threads=None):
    """Wall time of the fp64 oracle on one layer (all tokens), generation excluded."""
    import oracle
    import synth
    E = cfg.weight_experts
    x, wr, bias = synth.gen_x(cfg, layer), synth.gen_router(cfg, layer), synth.gen_bias(cfg, layer)
    pg = [synth.gen_planes(cfg, layer, e, 0) for e in range(E)]
    pd = [synth.gen_planes(cfg, layer, e, 1) for e in range(E)]
    lg = [synth.gen_parent_lut(cfg, layer, e, 0) for e in range(E)]
    ld = [synth.gen_parent_lut(cfg, layer, e, 1) for e in range(E)]
    prev = oracle.num_threads()
    if threads:
        oracle.set_num_threads(threads)
    try:
        t0 = time.perf_counter()
        oracle.moe_forward(x, wr, bias, cfg.topk, pg, lg, qmap[:, 0], pd, ld, qmap[:, 1], renormalize=cfg.renormalize,
                           n_shared=cfg.shared)
        return time.perf_counter() - t0
    finally:
        oracle.set_num_threads(prev)


def cpu_baseline(headline_cfg, qmaps):
    """The oracle as it stands on the host cores: a bounded sample of the headline
    workload (layers of the 32-layer stack under map A, each a full layer of 32
    tokens), scaled to tokens/s of the whole stack; plus 1-thread times of the tiny
    and the Mixtral-8x7B decode layers."""
    import oracle
    import synth
    cores = oracle.num_threads()
    per, n = [], 0
    t_all = time.perf_counter()
    while n < 4 and (n < 2 or time.perf_counter() - t_all < 20.0):
        per.append(oracle_layer_time(headline_cfg, n, qmaps[n]))
        n += 1
    t_layer = statistics.mean(per)
    value = headline_cfg.tokens / (t_layer * headline_cfg.layers)
    tiny = synth.config_by_name("tiny")
    dec = synth.config_by_name("mixtral8x7b_decode_t16")
    one = {"tiny_s": round(oracle_layer_time(tiny, 0, synth.gen_qmap(tiny, 0), threads=1), 4),
           "mixtral8x7b_decode_t16_s": round(oracle_layer_time(dec, 0, synth.gen_qmap(dec, 0), threads=1), 3)}
    return {"value": round(value, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} of the {headline_cfg.layers} layers under map A (layers 0..{n - 1}), each a whole layer "
                      f"of {headline_cfg.tokens} tokens in fp64, {statistics.mean(per):.2f} s per layer; tokens/s "
                      f"= {headline_cfg.tokens} / ({headline_cfg.layers} x mean layer time); input generation "
                      f"excluded",
            "one_thread_layer_seconds": one}


# ----------------------------------------------------------------------------- main

def copy_calibration(mib):
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()


def base_record(args, wl_name, rec):
    return {
        "metric": METRIC,
        "value": rec["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "dtype_detail": "fp16 weights (LUT centroids) and activations, fp32 accumulation, fp64 router logits",
        "data": "synthetic (seeded bit-planes, sorted N(0,0.02) fp16 LUTs, N(0,1) fp16 activations; no trained "
                "weights)",
        "config": {"workload": wl_name},
        "timing": {"median_ms": rec["median_ms"], "p10_ms": rec["p10_ms"], "p90_ms": rec["p90_ms"],
                   "warmup_policy": f"at least --warmup steps, continued until the last 5 step times agree within "
                                    f"3% and at least {args.settle_min_s} s of load have run (GPU clock ramp); "
                                    f"{rec['warmup_steps_run']} warm-up steps ran"},
        "roofline": rec["roofline"],
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-min-s", type=float, default=1.0, help="warm-up seconds at least")
    ap.add_argument("--settle-max-s", type=float, default=8.0, help="warm-up seconds at most")
    ap.add_argument("--copies", type=int, default=2, help="resident weight copies of a single-layer decode workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layer-kernel", action="store_true",
                    help="small decode batches: gate_up and down in one launch (APMOE_LAYER_KERNEL=1)")
    ap.add_argument("--uniform-q", type=int, default=0, metavar="Q",
                    help="single-layer workload: every block at bitwidth Q (per-q study)")
    ap.add_argument("--workload", default="suite",
                    help="'suite' (default: the 32-layer headline plus the single-layer workloads) or one workload")
    ap.add_argument("--map", default="AB", choices=["A", "B", "AB"], help="multi-layer workload: q maps to run")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run one plain device copy of MIB MiB (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (--gpus {args.gpus} requested); "
              "the layer's multi-GPU sharding is a design, not a measured path.", file=sys.stderr)
        return 2
    if args.layer_kernel:
        os.environ["APMOE_LAYER_KERNEL"] = "1"  # read when the contexts are created

    import torch

    import synth
    timer = Timer(args)
    stream = torch.cuda.Stream()  # default priority
    with torch.cuda.stream(stream):
        if args.copy_calibration:
            copy_calibration(args.copy_calibration)
        if args.workload != "suite":
            cfg = synth.config_by_name(args.workload)
            if cfg.layers > 1:
                log(f"generating and uploading {cfg.name} ({cfg.layers} layers)")
                wl = StackedLayers(cfg)
                recs = {}
                for m in args.map:
                    wl.use_map(m)
                    recs[m] = measure(timer, wl, f"{cfg.name} map {m}")
                rec = recs[args.map[0]]
                out = base_record(args, cfg.name, rec)
                out["config"].update({k: rec[k] for k in ("layers", "tokens", "hidden", "ffn", "experts", "topk",
                                                          "mean_bits")})
                out["maps"] = recs
            else:
                copies = args.copies if cfg.tokens <= 256 else 1
                log(f"generating and uploading {cfg.name} ({copies} weight copies)")
                wl = SingleLayer(cfg, copies, args.uniform_q)
                rec = measure(timer, wl, cfg.name)
                out = base_record(args, cfg.name, rec)
                out["config"].update({k: rec[k] for k in ("tokens", "hidden", "ffn", "experts", "topk", "mean_bits",
                                                          "counts")})
                out["record"] = rec
            wl.close()
            print(json.dumps(out), flush=True)
            return 0

        # ---- the suite
        hinfo = host_info()
        ceil = stream_ceiling()
        log(f"stream ceiling: read {ceil['read_gbps']:.0f} GB/s, copy {ceil['copy_gbps']:.0f} GB/s")
        cfg4 = synth.config_by_name(HEADLINE)
        log(f"generating and uploading {cfg4.name} ({cfg4.layers} layers)")
        wl = StackedLayers(cfg4)
        wl.use_map("A")
        rec_a = measure(timer, wl, f"{cfg4.name} map A")
        wl.use_map("B")
        rec_b = measure(timer, wl, f"{cfg4.name} map B (committed at a launch boundary)")
        qa = wl.qa
        wl.close()
        del wl
        torch.cuda.empty_cache()
        subs = {}
        for name in SUBRECORDS:
            cfg = synth.config_by_name(name)
            copies = args.copies if cfg.tokens <= 256 else 1
            log(f"generating and uploading {name} ({copies} weight copies)")
            w1 = SingleLayer(cfg, copies)
            subs[name] = measure(timer, w1, name)
            w1.close()
            del w1
            torch.cuda.empty_cache()
    out = base_record(args, HEADLINE, rec_a)
    out["config"].update({"layers": cfg4.layers, "tokens": cfg4.tokens, "hidden": cfg4.hidden, "ffn": cfg4.ffn,
                          "experts": cfg4.experts, "topk": cfg4.topk, "q_map": "A", "mean_bits": rec_a["mean_bits"]})
    out["headline"] = rec_a
    out["map_b"] = rec_b
    out["workloads"] = subs
    out["hbm_ceiling_measured"] = ceil
    out["host"] = hinfo
    if not args.no_cpu_baseline:
        log("timing the fp64 CPU oracle (sample of the headline workload; 1-thread layers)")
        out["cpu_baseline"] = cpu_baseline(cfg4, qa)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
