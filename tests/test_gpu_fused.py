"""The fused launches against the separate ones (calls go through the C ABI).

Two fusions of the layer's steps (PagedWeight, Section 3.3: routing, the expert
computation and the output accumulation in the fused kernel's launches):
  - route in one launch: every token's selection, then the expert grouping by the
    workgroup that finishes last (small batches);
  - the output accumulation in the down product's epilogue, when every expert of the
    call takes the decode product (at most 32 tokens).
A context created with APMOE_UNFUSED=1 runs every step in its own launches.  The bar
is identical bits for every output of the route and of the layer, call after call
(the completion counters must be back at zero after each launch), and the oracle's
layer bound on one case.
"""
import os

import numpy as np
import pytest
import torch

import any_precision_weight_amd as apw
import synth
from gpu_util import Layer, check_out, ctx, dev, host

pytestmark = pytest.mark.gpu

_UNFUSED = None


def unfused_ctx() -> apw.Context:
    global _UNFUSED
    if _UNFUSED is None:
        old = os.environ.get("APMOE_UNFUSED")
        os.environ["APMOE_UNFUSED"] = "1"
        try:
            _UNFUSED = apw.Context(0)
        finally:
            if old is None:
                del os.environ["APMOE_UNFUSED"]
            else:
                os.environ["APMOE_UNFUSED"] = old
    return _UNFUSED


def _route(c, x_d, wr_d, bias_d, T, H, E, k, ns, renorm):
    kt, Et, R = k + ns, E + ns, T * (k + ns)
    o = dict(ids=torch.full((T, kt), -7, dtype=torch.int32, device="cuda"),
             w=torch.full((T, kt), -7.0, dtype=torch.float32, device="cuda"),
             counts=torch.full((Et,), -7, dtype=torch.int32, device="cuda"),
             offsets=torch.full((Et + 1,), -7, dtype=torch.int32, device="cuda"),
             perm=torch.full((R,), -7, dtype=torch.int32, device="cuda"),
             inv_perm=torch.full((R,), -7, dtype=torch.int32, device="cuda"))
    apw.route(c, x_d, wr_d, bias_d, T, H, E, k, renorm, o["ids"], o["w"], o["counts"], o["offsets"], o["perm"],
              o["inv_perm"], n_shared=ns)
    torch.cuda.synchronize()
    return {n: host(t) for n, t in o.items()}


# (T, H, E, k, n_shared, bias, renorm): one token; the Mixtral decode batches; shared-
# expert layers; 256 assignments (the largest fused route, twice) and 258, 512 and 2050
# (the two launches)
ROUTE_CASES = [
    (1, 4096, 8, 2, 0, False, True),
    (16, 4096, 8, 2, 0, False, True),
    (32, 4096, 8, 2, 0, True, True),
    (16, 2048, 60, 4, 4, False, True),
    (28, 256, 128, 8, 1, True, False),
    (32, 1024, 60, 4, 4, True, True),
    (128, 512, 8, 2, 0, False, True),
    (129, 512, 8, 2, 0, True, True),
    (64, 2048, 60, 4, 4, False, True),
    (1025, 256, 8, 2, 0, False, True),
]


@pytest.mark.parametrize("case", ROUTE_CASES, ids=lambda c: f"T{c[0]}E{c[2]}k{c[3]}s{c[4]}")
def test_route_fused_matches_separate(case):
    T, H, E, k, ns, use_bias, renorm = case
    seed = 500 + T
    x = synth.fp16_normal(seed, 1, T * H, 1.0).reshape(T, H)
    wr = synth.fp16_normal(seed, 2, E * H, 0.02).reshape(E, H)
    bias = synth.fp16_normal(seed, 3, E, 1.0).astype(np.float32) if use_bias else None
    x_d, wr_d = dev(x), dev(wr)
    bias_d = None if bias is None else dev(bias)
    ref = _route(unfused_ctx(), x_d, wr_d, bias_d, T, H, E, k, ns, renorm)
    for rep in range(3):  # the completion counter must be back at zero after every launch
        got = _route(ctx(), x_d, wr_d, bias_d, T, H, E, k, ns, renorm)
        for name in ref:
            np.testing.assert_array_equal(got[name].view(np.uint32) if got[name].dtype == np.float32 else got[name],
                                          ref[name].view(np.uint32) if ref[name].dtype == np.float32 else ref[name],
                                          err_msg=f"{name} (call {rep})")


def _forward(c, L: Layer, T: int):
    cfg = L.cfg
    x_d = dev(synth.gen_x(cfg, 0, T))
    nbytes = apw.moe_workspace(L.rw.table, L.layer, T, cfg.topk, cfg.shared)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    out = torch.full((T, cfg.hidden), float("nan"), dtype=torch.float16, device="cuda")
    apw.moe_forward(c, L.rw.table, L.layer, x_d, L.wr_d, L.bias_d, T, cfg.topk, cfg.renormalize, ws, nbytes, out,
                    n_shared=cfg.shared)
    torch.cuda.synchronize()
    return host(out)


_LAYERS = {}


def _layer(name: str) -> Layer:
    if name not in _LAYERS:  # x of the layer object: 32 tokens (the oracle case below)
        _LAYERS[name] = Layer(synth.config_by_name(name), T=32)
    return _LAYERS[name]


# token counts called in this order on one context: fused accumulation up to 32 tokens,
# the separate launch above; small counts after large ones reuse the counters
LAYER_CASES = [
    ("tiny", [8, 1, 32, 3, 33, 8]),
    ("mixtral8x7b_decode_t16", [16, 32, 1, 33, 16]),
    ("qwen_60r4s_top4_decode_t64", [16, 32, 64, 7]),
    ("gemma_128r1s_top8_decode_t64", [32, 5, 64]),
]


@pytest.mark.parametrize("name,Ts", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
def test_layer_fused_matches_separate(name, Ts):
    L = _layer(name)
    for T in Ts:
        ref = _forward(unfused_ctx(), L, T)
        got = _forward(ctx(), L, T)
        assert not np.isnan(got.astype(np.float32)).any(), f"T={T}: an output left unwritten"
        np.testing.assert_array_equal(got.view(np.uint16), ref.view(np.uint16), err_msg=f"{name} T={T}")


def test_layer_fused_against_oracle():
    """The fused layer at 32 Mixtral tokens against the fp64 oracle (eight tokens)."""
    L = _layer("mixtral8x7b_decode_t16")
    got = _forward(ctx(), L, 32)
    ev = [0, 3, 9, 14, 17, 22, 28, 31]
    ref = L.oracle(eval_tokens=ev)
    check_out(got[ev], ref["out"])


def test_two_contexts_on_two_streams():
    """Each context owns its completion counters: two contexts running fused layers on
    two streams at the same time (calls interleaved, no synchronisation between them)
    give the bits of the separate launches."""
    L = _layer("mixtral8x7b_decode_t16")
    cfg = L.cfg
    Ts = [16, 32, 7, 32, 24, 1]
    refs = [_forward(unfused_ctx(), L, T) for T in Ts]
    c2 = apw.Context(0)
    try:
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        jobs = []
        for i, T in enumerate(Ts):
            c, s = (ctx(), s1) if i % 2 == 0 else (c2, s2)
            x_d = dev(synth.gen_x(cfg, 0, T))
            nbytes = apw.moe_workspace(L.rw.table, L.layer, T, cfg.topk, cfg.shared)
            ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
            out = torch.full((T, cfg.hidden), float("nan"), dtype=torch.float16, device="cuda")
            torch.cuda.synchronize()  # inputs ready before either stream starts
            jobs.append((T, x_d, ws, out))
        for i, (T, x_d, ws, out) in enumerate(jobs):
            c, s = (ctx(), s1) if i % 2 == 0 else (c2, s2)
            apw.moe_forward(c, L.rw.table, L.layer, x_d, L.wr_d, L.bias_d, T, cfg.topk, cfg.renormalize, ws,
                            ws.numel(), out, s, n_shared=cfg.shared)
        torch.cuda.synchronize()
        for (T, _, _, out), ref in zip(jobs, refs):
            np.testing.assert_array_equal(host(out).view(np.uint16), ref.view(np.uint16), err_msg=f"T={T}")
    finally:
        c2.close()



def _env_ctx(var: str) -> apw.Context:
    old = os.environ.get(var)
    os.environ[var] = "1"
    try:
        return apw.Context(0)
    finally:
        if old is None:
            del os.environ[var]
        else:
            os.environ[var] = old


_ONE = None


def layer_kernel_ctx() -> apw.Context:
    """A context that runs a small batch's gate_up and down in one launch."""
    global _ONE
    if _ONE is None:
        _ONE = _env_ctx("APMOE_LAYER_KERNEL")
    return _ONE


def test_layer_kernel_matches_two_launches():
    """The one-launch decode layer (gate_up and down in one launch, the down blocks of an
    expert started once its gate_up blocks are stored) against gate_up and down as two
    launches: identical bits call after call (the launch leaves its counters at zero),
    with one and two tokens (experts without rows), and no fault flag."""
    name = "mixtral8x7b_decode_t16"
    L = _layer(name)
    for T in [32, 16, 1, 2, 32, 9, 31, 17, 16]:
        ref = _forward(ctx(), L, T)
        got = _forward(layer_kernel_ctx(), L, T)
        assert not np.isnan(got.astype(np.float32)).any(), f"T={T}: an output left unwritten"
        np.testing.assert_array_equal(got.view(np.uint16), ref.view(np.uint16), err_msg=f"{name} T={T}")
    assert layer_kernel_ctx().faults() == 0


def test_layer_kernel_two_contexts_on_two_streams():
    """Two one-launch layers at once on two streams (each context its own work list and
    counters; each launch gets only part of the GPU, so its down blocks wait for gate_up
    blocks that start late): the bits of the separate launches, no fault flag."""
    L = _layer("mixtral8x7b_decode_t16")
    cfg = L.cfg
    Ts = [32, 32, 16, 32, 24, 1]
    refs = [_forward(ctx(), L, T) for T in Ts]
    c2 = _env_ctx("APMOE_LAYER_KERNEL")
    try:
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        jobs = []
        for T in Ts:
            x_d = dev(synth.gen_x(cfg, 0, T))
            nbytes = apw.moe_workspace(L.rw.table, L.layer, T, cfg.topk, cfg.shared)
            ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
            out = torch.full((T, cfg.hidden), float("nan"), dtype=torch.float16, device="cuda")
            jobs.append((T, x_d, ws, out))
        torch.cuda.synchronize()  # inputs ready before either stream starts
        for i, (T, x_d, ws, out) in enumerate(jobs):
            c, s = (layer_kernel_ctx(), s1) if i % 2 == 0 else (c2, s2)
            apw.moe_forward(c, L.rw.table, L.layer, x_d, L.wr_d, L.bias_d, T, cfg.topk, cfg.renormalize, ws,
                            ws.numel(), out, s, n_shared=cfg.shared)
        torch.cuda.synchronize()
        for (T, _, _, out), ref in zip(jobs, refs):
            np.testing.assert_array_equal(host(out).view(np.uint16), ref.view(np.uint16), err_msg=f"T={T}")
        assert layer_kernel_ctx().faults() == 0 and c2.faults() == 0
    finally:
        c2.close()
