"""Helpers of the GPU parity tests: upload a synthetic workload, run the layer
through the C ABI step by step, and compare with the fp64 oracle."""
from __future__ import annotations

import numpy as np
import torch

import any_precision_weight_amd as apw
import oracle
import synth
from any_precision_weight_amd.resident import ResidentWeights

_CTX = None


def ctx() -> apw.Context:
    global _CTX
    if _CTX is None:
        _CTX = apw.Context(0)
    return _CTX


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def ulp16(v: np.ndarray) -> np.ndarray:
    """Spacing of fp16 numbers at |v| (normal range), 2^-24 below it."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return np.exp2(e - 10)


class Layer:
    """One MoE layer of a config, resident on the GPU, with host copies for the oracle."""

    def __init__(self, cfg: synth.MoEConfig, layer: int = 0, qmap: np.ndarray | None = None,
                 T: int | None = None, resident: ResidentWeights | None = None, slot: int = 0):
        """Data of generator layer `layer`, stored in table layer `slot` of `resident`
        (a fresh one-layer table when None)."""
        self.cfg = cfg
        self.T = cfg.tokens if T is None else T
        self.x = synth.gen_x(cfg, layer, self.T)
        self.wr = synth.gen_router(cfg, layer)
        self.bias = synth.gen_bias(cfg, layer)
        self.q = synth.gen_qmap(cfg, layer) if qmap is None else np.asarray(qmap, np.int32)
        E = cfg.weight_experts
        self.planes = {}
        self.parent = {}
        own = resident is None
        self.rw = ResidentWeights(ctx(), 1, E) if own else resident
        self.layer = 0 if own else slot
        for e in range(E):
            for u in (0, 1):
                P = synth.gen_planes(cfg, layer, e, u)
                L8 = synth.gen_parent_lut(cfg, layer, e, u)
                self.planes[(e, u)] = P
                self.parent[(e, u)] = L8
                self.rw.add_block(self.layer, e, u, P, L8, int(self.q[e, u]))
        if own:
            self.rw.commit()
        self.x_d = dev(self.x)
        self.wr_d = dev(self.wr)
        self.bias_d = None if self.bias is None else dev(self.bias)

    # ------------------------------------------------------------------ GPU run
    def run(self, stream=None) -> dict:
        """Route, gate_up (fp16 h), act, down (fp32 y), combine -- each via the C ABI."""
        cfg, T, k, kt = self.cfg, self.T, self.cfg.topk, self.cfg.assign
        H, F, E, Et = cfg.hidden, cfg.ffn, cfg.experts, cfg.weight_experts
        R = T * kt
        o = dict(
            ids=torch.empty((T, kt), dtype=torch.int32, device="cuda"),
            w=torch.empty((T, kt), dtype=torch.float32, device="cuda"),
            counts=torch.empty(Et, dtype=torch.int32, device="cuda"),
            offsets=torch.empty(Et + 1, dtype=torch.int32, device="cuda"),
            perm=torch.empty(R, dtype=torch.int32, device="cuda"),
            inv_perm=torch.empty(R, dtype=torch.int32, device="cuda"),
            h=torch.empty((R, 2 * F), dtype=torch.float16, device="cuda"),
            a=torch.empty((R, F), dtype=torch.float16, device="cuda"),
            y=torch.empty((R, H), dtype=torch.float32, device="cuda"),
            out=torch.empty((T, H), dtype=torch.float16, device="cuda"),
        )
        c = ctx()
        apw.route(c, self.x_d, self.wr_d, self.bias_d, T, H, E, k, cfg.renormalize, o["ids"], o["w"], o["counts"],
                  o["offsets"], o["perm"], o["inv_perm"], stream, n_shared=cfg.shared)
        apw.gemm(c, self.rw.table, self.layer, apw.GATE_UP, self.x_d, True, o["perm"], o["offsets"], T, kt, o["h"],
                 apw.F16, stream)
        apw.act(c, o["h"], R, F, o["a"], stream)
        apw.gemm(c, self.rw.table, self.layer, apw.DOWN, o["a"], False, o["perm"], o["offsets"], T, kt, o["y"],
                 apw.F32, stream)
        apw.combine(c, o["y"], apw.F32, o["w"], o["inv_perm"], T, kt, H, o["out"], stream)
        return o

    def run_fused_call(self, stream=None) -> torch.Tensor:
        """The same layer through apmoe_moe_forward."""
        cfg = self.cfg
        nbytes = apw.moe_workspace(self.rw.table, self.layer, self.T, cfg.topk, cfg.shared)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        out = torch.empty((self.T, cfg.hidden), dtype=torch.float16, device="cuda")
        apw.moe_forward(ctx(), self.rw.table, self.layer, self.x_d, self.wr_d, self.bias_d, self.T, cfg.topk,
                        cfg.renormalize, ws, nbytes, out, stream, n_shared=cfg.shared)
        return out

    # ------------------------------------------------------------------ oracle
    def oracle(self, eval_tokens=None, intermediates=False, qmap=None) -> dict:
        E = self.cfg.weight_experts
        q = self.q if qmap is None else qmap
        return oracle.moe_forward(
            self.x, self.wr, self.bias, self.cfg.topk,
            [self.planes[(e, 0)] for e in range(E)], [self.parent[(e, 0)] for e in range(E)], q[:, 0],
            [self.planes[(e, 1)] for e in range(E)], [self.parent[(e, 1)] for e in range(E)], q[:, 1],
            renormalize=self.cfg.renormalize, eval_tokens=eval_tokens, intermediates=intermediates,
            n_shared=self.cfg.shared)


def check_route(o_gpu: dict, r: dict) -> None:
    assert np.array_equal(host(o_gpu["ids"]), r["ids"])
    assert np.array_equal(host(o_gpu["counts"]), r["counts"])
    assert np.array_equal(host(o_gpu["offsets"]), r["offsets"])
    assert np.array_equal(host(o_gpu["perm"]), r["perm"])
    assert np.array_equal(host(o_gpu["inv_perm"]), r["inv_perm"])
    dw = np.abs(host(o_gpu["w"]).astype(np.float64) - r["w32"].astype(np.float64))
    assert dw.size == 0 or dw.max() <= 1e-6, dw.max()


def check_out(out_gpu: np.ndarray, out_ref: np.ndarray, max_abs=1e-2, rel_l2=2e-3) -> tuple[float, float]:
    """Spec bar for fp16 outputs of the layer."""
    g = np.asarray(out_gpu, np.float64)
    d = g - out_ref
    ma = float(np.abs(d).max()) if d.size else 0.0
    rl = float(np.linalg.norm(d) / max(np.linalg.norm(out_ref), 1e-300)) if d.size else 0.0
    assert np.all(np.isfinite(g))
    assert ma <= max_abs, (ma, rl)
    assert rl <= rel_l2, (ma, rl)
    return ma, rl


def topk_margin_ok(x, wr, bias, k: int) -> bool:
    """Every token's k-th and (k+1)-th logits differ by more than the worst fp64
    rounding of both logits: each is a sum of H+1 exact terms, so any summation
    order is within gamma_H * sum|terms| of the exact value (Higham, Accuracy and
    Stability of Numerical Algorithms, eq. 4.6).  Then the GPU's summation order
    cannot change the selection."""
    r = oracle.route(x, wr, bias, k, want_absdot=True)
    H = x.shape[1]
    z = r["logits"]
    if z.shape[1] <= k:
        return True
    u = 2.0 ** -53
    gamma = H * u / (1 - H * u)
    order = np.argsort(-z, axis=1, kind="stable")
    rows = np.arange(z.shape[0])
    zk, zk1 = z[rows, order[:, k - 1]], z[rows, order[:, k]]
    slack = gamma * 2 * (r["absdot"][rows, order[:, k - 1]] + r["absdot"][rows, order[:, k]])
    return bool(np.all(zk - zk1 > slack))
