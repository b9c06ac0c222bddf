#!/usr/bin/env python3
"""Benchmark of the any-precision MoE expert layer on one MI355X.

One step = one pass of the whole layer (route, gate_up product, SiLU*up, down
product, combine) over one decode batch of the Mixtral-8x7B-shaped workload:
hidden 4096, ffn 14336, 8 experts, top-2, 16 tokens, per-block bitwidths drawn
uniformly from 3..8 (synthetic, seeded; no trained weights).  Weights are
resident in HBM before timing; two copies alternate between steps so that no
step reads weights the previous one left in the last-level cache.

Prints one JSON line: tokens/s of the layer, the gate_up product kernel against
the HBM roofline (algorithmic bytes per launch / average launch time from HIP
events on its stream), and the fp64 CPU oracle timed on the host as a baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X published dense fp16 matrix peak
ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "any_precision_weight_amd", "csrc")


def source_sha256(names):
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profiled_traffic(workload, sources):
    """HBM bytes per launch of the gate_up product from the committed counter summary
    profiles/gemm_gate_up_<workload>_counters.md (FETCH_SIZE + WRITE_SIZE, scaled by a
    plain copy of known size), or None when there is none or the kernel sources have
    changed since it was taken."""
    path = os.path.join(PROFILES, f"gemm_gate_up_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.strip().startswith("- "):
                k, v = line.strip()[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel sources sha256") != source_sha256(sources):
        return None
    try:
        return int(fields["traffic bytes per launch"])
    except (KeyError, ValueError):
        return None


def algorithmic_bytes(cfg, counts, qmap, kind):
    """Bytes one product launch must move: the q needed planes and LUT level q of
    every active expert (Eq. 3 of the paper), the input rows it reads and the
    output rows it writes (gate_up writes the activation a, fp16 [rows][F])."""
    N, K = cfg.block_shape(kind)
    w = 0
    rows = 0
    for e, c in enumerate(counts):
        if c == 0:
            continue
        q = int(qmap[e, kind])
        w += N * q * K // 8 + N * (1 << q) * 2
        rows += int(c)
    in_bytes = rows * K * 2
    out_bytes = rows * (N // 2) * 2 if kind == 0 else rows * N * 4
    return w + in_bytes + out_bytes, w


def layer_bytes(cfg, counts, qmap):
    """Whole-layer algorithmic bytes: active weights + x + router + out + routing metadata."""
    T, H, E, k = cfg.tokens, cfg.hidden, cfg.experts, cfg.assign
    w = 0
    for kind in (0, 1):
        N, K = cfg.block_shape(kind)
        for e, c in enumerate(counts):
            if c:
                q = int(qmap[e, kind])
                w += N * q * K // 8 + N * (1 << q) * 2
    return w + 2 * T * H + 2 * E * H + 2 * T * H + 12 * T * k


def cpu_baseline(cfg, layer, min_seconds=10.0):
    """The fp64 oracle on the benchmark's own layer, repeated until about ten seconds
    of host work have run (bounded to keep the default run short)."""
    import oracle
    runs, t0 = 0, time.perf_counter()
    while True:
        layer.oracle()
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or runs >= 50:
            break
    per = dt / runs
    return {"value": cfg.tokens / per, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"whole layer, all {cfg.tokens} tokens of the benchmark batch, fp64, input generation "
                      f"excluded; {runs} runs in {dt:.1f} s"}


class BenchLayer:
    def __init__(self, cfg, copies, device_gen=False, uniform_q=0):
        import numpy as np
        import torch

        import any_precision_weight_amd as apw
        import synth
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
        self.planes, self.parent = {}, {}
        for e in range(E):
            for u in (0, 1):
                if device_gen:  # bit-identical device generator; no host copies (no CPU baseline)
                    import synth.gpu
                    P, L8 = synth.gpu.planes(cfg, 0, e, u), synth.gpu.parent_lut(cfg, 0, e, u)
                else:
                    P = synth.gen_planes(cfg, 0, e, u)
                    L8 = synth.gen_parent_lut(cfg, 0, e, u)
                    self.planes[(e, u)], self.parent[(e, u)] = P, L8
                for c in range(copies):
                    self.rw.add_block(c, e, u, P, L8, int(self.q[e, u]))
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
                      a=z((R, F), torch.float16), y=z((R, H), torch.float32),
                      out=z((T, H), torch.float16))

    def step(self, slot, ev=None):
        apw, b, cfg, c = self.apw, self.b, self.cfg, self.ctx
        T, k, H, F, E = cfg.tokens, cfg.assign, cfg.hidden, cfg.ffn, cfg.experts
        apw.route(c, self.x_d, self.wr_d, self.bias_d, T, H, E, cfg.topk, cfg.renormalize, b["ids"], b["w"],
                  b["counts"], b["offsets"], b["perm"], b["inv"], n_shared=cfg.shared)
        if ev:
            ev[0].record()
        # gate_up with SiLU(gate) * up in its epilogue: a [R][F] directly
        apw.gemm_act(c, self.rw.table, slot, self.x_d, True, b["perm"], b["offsets"], T, k, b["a"])
        if ev:
            ev[1].record()
            ev[2].record()
        apw.gemm(c, self.rw.table, slot, apw.DOWN, b["a"], False, b["perm"], b["offsets"], T, k, b["y"], apw.F32)
        if ev:
            ev[3].record()
        apw.combine(c, b["y"], apw.F32, b["w"], b["inv"], T, k, H, b["out"])

    def oracle(self):
        import oracle
        E = self.cfg.weight_experts
        return oracle.moe_forward(self.x, self.wr, self.bias, self.cfg.topk,
                                  [self.planes[(e, 0)] for e in range(E)], [self.parent[(e, 0)] for e in range(E)],
                                  self.q[:, 0], [self.planes[(e, 1)] for e in range(E)],
                                  [self.parent[(e, 1)] for e in range(E)], self.q[:, 1],
                                  renormalize=self.cfg.renormalize, n_shared=self.cfg.shared)


def bench_layers(args, cfg) -> int:
    """Every layer of a multi-layer workload resident at once (planes generated on the
    device); one step = the whole stack, one apmoe_moe_forward per layer, under q map
    A, then again after map B is committed at a launch boundary."""
    import numpy as np
    import torch

    import any_precision_weight_amd as apw
    import synth
    import synth.gpu
    from any_precision_weight_amd.resident import ResidentWeights

    Ln, E, T, H = cfg.layers, cfg.weight_experts, cfg.tokens, cfg.hidden
    print(f"[bench] generating and uploading {cfg.name} ({Ln} layers)", file=sys.stderr, flush=True)
    ctx = apw.Context(0)
    rw = ResidentWeights(ctx, Ln, E)
    qa = [synth.gen_qmap(cfg, l, 0) for l in range(Ln)]
    qb = [synth.gen_qmap(cfg, l, 1) for l in range(Ln)]
    for l in range(Ln):
        for e in range(E):
            for u in (0, 1):
                rw.add_block(l, e, u, synth.gpu.planes(cfg, l, e, u), synth.gpu.parent_lut(cfg, l, e, u),
                             int(qa[l][e, u]))
    rw.commit()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    xs = [dev(synth.gen_x(cfg, l)) for l in range(Ln)]
    wrs = [dev(synth.gen_router(cfg, l)) for l in range(Ln)]
    nbytes = apw.moe_workspace(rw.table, 0, T, cfg.topk, cfg.shared)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    outs = [torch.empty((T, H), dtype=torch.float16, device="cuda") for _ in range(Ln)]
    # per-layer routed counts (the same inputs route the same way under either map)
    counts = []
    for l in range(Ln):
        kt, Et = cfg.assign, E
        o = [torch.empty(n, dtype=dt, device="cuda") for n, dt in
             ((T * kt, torch.int32), (T * kt, torch.float32), (Et, torch.int32), (Et + 1, torch.int32),
              (T * kt, torch.int32), (T * kt, torch.int32))]
        apw.route(ctx, xs[l], wrs[l], None, T, H, cfg.experts, cfg.topk, cfg.renormalize, *o, n_shared=cfg.shared)
        counts.append(o[2].cpu().numpy())

    def step():
        for l in range(Ln):
            apw.moe_forward(ctx, rw.table, l, xs[l], wrs[l], None, T, cfg.topk, cfg.renormalize, ws, nbytes, outs[l],
                            n_shared=cfg.shared)

    def timed(qmaps):
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(args.steps):
            step()
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / args.steps
        nb = sum(layer_bytes(cfg, counts[l], qmaps[l]) for l in range(Ln))
        return ms, nb, float(np.mean([q.mean() for q in qmaps]))

    ms_a, nb_a, bits_a = timed(qa)
    for l in range(Ln):
        rw.stage_qmap(l, qb[l])
    rw.commit()
    ms_b, nb_b, bits_b = timed(qb)
    gbs_a, gbs_b = nb_a / (ms_a * 1e-3) / 1e9, nb_b / (ms_b * 1e-3) / 1e9
    print(f"[bench] {cfg.name}: map A ({bits_a:.2f} bits) step {ms_a * 1e3:.0f} us {gbs_a:.0f} GB/s; "
          f"map B ({bits_b:.2f} bits) step {ms_b * 1e3:.0f} us {gbs_b:.0f} GB/s", file=sys.stderr, flush=True)
    result = {
        "metric": "decode tokens/s + achieved HBM GB/s (% peak), fused any-precision MoE layer",
        "value": round(T / (ms_a * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_a, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 (fp32 accumulate; fp64 router)",
        "data": "synthetic (seeded bit-planes generated on the device, sorted N(0,0.02) fp16 LUTs, N(0,1) activations)",
        "config": {"workload": cfg.name, "layers": Ln, "tokens": T, "hidden": H, "ffn": cfg.ffn,
                   "experts": cfg.experts, "topk": cfg.topk, "map_a_mean_bits": round(bits_a, 3),
                   "map_b_mean_bits": round(bits_b, 3)},
        "roofline": {"kernel": "whole layer stack (map A)", "bound": "hbm", "achieved": round(gbs_a, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs_a / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes": nb_a, "traffic": None},
        "map_b": {"ms_per_step": round(ms_b, 5), "tokens_per_s": round(T / (ms_b * 1e-3), 1),
                  "achieved_gbps": round(gbs_b, 1), "frac": round(gbs_b / HBM_PEAK_GBS, 4),
                  "algorithmic_bytes": nb_b},
    }
    print(json.dumps(result), flush=True)
    rw.close()
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=2, help="resident weight copies rotated between steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--uniform-q", type=int, default=0, metavar="Q",
                    help="commit every block at bitwidth Q instead of the workload's map (per-q study)")
    ap.add_argument("--workload", default="mixtral8x7b_decode_t16",
                    help="synthetic workload (default: the Mixtral-8x7B decode layer the metric is quoted on)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run one plain device copy of MIB MiB (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (--gpus {args.gpus} requested); "
              "the layer's multi-GPU sharding is a design, not a measured path.", file=sys.stderr)
        return 2

    import torch

    import synth
    cfg = synth.config_by_name(args.workload)
    if cfg.layers != 1:
        return bench_layers(args, cfg)
    big = cfg.tokens * cfg.hidden > 16 * 4096 or cfg.hidden > 4096
    print(f"[bench] generating and uploading {cfg.name} ({args.copies} weight copies)", file=sys.stderr, flush=True)
    L = BenchLayer(cfg, args.copies, device_gen=big, uniform_q=args.uniform_q)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            L.step(i % args.copies)
        torch.cuda.synchronize()
        counts = L.b["counts"].cpu().numpy()
        if args.copy_calibration:
            n = args.copy_calibration << 20
            src = torch.empty(n, dtype=torch.uint8, device="cuda")
            dst = torch.empty_like(src)
            dst.copy_(src)
            torch.cuda.synchronize()
            del src, dst
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_start.record()
        for i in range(args.steps):
            L.step(i % args.copies, evs[i])
        t_end.record()
        torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms = total_ms / args.steps
    gu_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    dn_ms = sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps
    gu_bytes, gu_w = algorithmic_bytes(cfg, counts, L.q, 0)
    dn_bytes, dn_w = algorithmic_bytes(cfg, counts, L.q, 1)
    lb = layer_bytes(cfg, counts, L.q)
    gu_gbs = gu_bytes / (gu_ms * 1e-3) / 1e9
    tokens_per_s = cfg.tokens / (ms * 1e-3)
    flops = 2 * cfg.tokens * cfg.assign * 3 * cfg.hidden * cfg.ffn + 2 * cfg.tokens * cfg.experts * cfg.hidden
    tflops = flops / (ms * 1e-3) / 1e12
    print(f"[bench] {cfg.name}: {tflops:.1f} TFLOP/s  "
          f"step {ms * 1e3:.1f} us  gate_up {gu_ms * 1e3:.1f} us ({gu_gbs:.0f} GB/s)  "
          f"down {dn_ms * 1e3:.1f} us ({dn_bytes / (dn_ms * 1e-3) / 1e9:.0f} GB/s)  "
          f"layer {lb / (ms * 1e-3) / 1e9:.0f} GB/s", file=sys.stderr, flush=True)

    result = {
        "metric": "decode tokens/s + achieved HBM GB/s (% peak), fused any-precision MoE layer",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 (fp32 accumulate; fp64 router)",
        "data": "synthetic (seeded bit-planes, sorted N(0,0.02) fp16 LUTs, N(0,1) fp16 activations)",
        "config": {"workload": cfg.name, "tokens": cfg.tokens, "hidden": cfg.hidden, "ffn": cfg.ffn,
                   "experts": cfg.experts, "shared_experts": cfg.shared, "topk": cfg.topk,
                   "qmap_mean_bits": float(L.q.mean()), "counts": [int(c) for c in counts],
                   "weight_copies": args.copies},
        "layer_gbps": round(lb / (ms * 1e-3) / 1e9, 1),
        "layer_hbm_frac": round(lb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "kernels_us": {"gate_up": round(gu_ms * 1e3, 2), "down": round(dn_ms * 1e3, 2)},
        "layer_tflops": round(tflops, 2),
        "layer_mfma_frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
    }
    # the gate_up product is the dominant kernel; it is HBM-bound below the ridge point
    # (peak FLOP/s over peak bytes/s) and MFMA-bound above it
    gu_flops = 2 * cfg.tokens * cfg.assign * 2 * cfg.ffn * cfg.hidden
    sources = ["gemm.hip", "gemm_tile.hip"]
    if gu_flops / gu_bytes > MFMA_F16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        tf = gu_flops / (gu_ms * 1e-3) / 1e12
        result["roofline"] = {"kernel": "apmoe gemm (gate_up)", "bound": "mfma", "achieved": round(tf, 1),
                              "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                              "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4), "algorithmic_flops": gu_flops,
                              "traffic": profiled_traffic(cfg.name, sources)}
    else:
        result["roofline"] = {"kernel": "apmoe gemm (gate_up)", "bound": "hbm", "achieved": round(gu_gbs, 1),
                              "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gu_gbs / HBM_PEAK_GBS, 4),
                              "algorithmic_bytes": gu_bytes, "traffic": profiled_traffic(cfg.name, sources)}
    if not args.no_cpu_baseline and L.planes:
        print("[bench] timing the fp64 CPU oracle on the same layer", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, L)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
