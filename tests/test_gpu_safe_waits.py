"""The build with every counted vector-memory wait drained to zero gives the same bits.

The product kernels end their pipeline steps with counted waits (s_waitcnt with a
vmcnt above zero): they wait for the token copies that must have landed and leave
the plane requests issued after them in flight, which is right only as long as the
requests go out in the order the counts assume.  libapmoe_safe.so is the same
source built with APMOE_SAFE_WAITS, where every such wait drains all outstanding
requests: slower, never early.  If a compiler or schedule change made a counted
wait too short, a barrier would pass before a copy landed and the default build's
outputs would change; here both builds run the same layers on the same resident
weights (the safe build's table points at the same device planes and LUTs) and
every output must match bit for bit: routing, the gate_up product to fp16, the
fused activation, the down product to fp32, the layer output.

Workloads: the tiny layer; the Mixtral-8x7B decode layer (16 tokens: the decode
product); the Zipf-skewed Mixtral-8x22B decode layer (256 tokens: decode, mid and
tile products, the tile launch on the side stream); the Mixtral-8x7B prefill layer
(4096 tokens: the tile product).
"""
import numpy as np
import pytest
import torch

import any_precision_weight_amd as apw
import synth
import synth.gpu
from any_precision_weight_amd.resident import ResidentWeights
from gpu_util import ctx, dev, host

pytestmark = pytest.mark.gpu

_SAFE = None


def safe_ctx() -> apw.Context:
    global _SAFE
    if _SAFE is None:
        _SAFE = apw.Context(0, library=apw.load_library(apw.SAFE_LIB_PATH))
    return _SAFE


def _layer_outputs(c, table, cfg, x_d, wr_d, bias_d):
    T, k, H, F, E, Et = cfg.tokens, cfg.assign, cfg.hidden, cfg.ffn, cfg.experts, cfg.weight_experts
    R = T * k
    z = lambda shape, dt: torch.full(shape, -1, dtype=dt, device="cuda")
    o = dict(ids=z((T, k), torch.int32), w=z((T, k), torch.float32), counts=z((Et,), torch.int32),
             offsets=z((Et + 1,), torch.int32), perm=z((R,), torch.int32), inv_perm=z((R,), torch.int32),
             h=z((R, 2 * F), torch.float16), a=z((R, F), torch.float16), a_fused=z((R, F), torch.float16),
             y=z((R, H), torch.float32), out=z((T, H), torch.float16))
    apw.route(c, x_d, wr_d, bias_d, T, H, E, cfg.topk, cfg.renormalize, o["ids"], o["w"], o["counts"],
              o["offsets"], o["perm"], o["inv_perm"], n_shared=cfg.shared)
    apw.gemm(c, table, 0, apw.GATE_UP, x_d, True, o["perm"], o["offsets"], T, k, o["h"], apw.F16)
    apw.act(c, o["h"], R, F, o["a"])
    apw.gemm_act(c, table, 0, x_d, True, o["perm"], o["offsets"], T, k, o["a_fused"])
    apw.gemm(c, table, 0, apw.DOWN, o["a"], False, o["perm"], o["offsets"], T, k, o["y"], apw.F32)
    apw.combine(c, o["y"], apw.F32, o["w"], o["inv_perm"], T, k, H, o["out"])
    torch.cuda.synchronize()
    return {n: host(t) for n, t in o.items()}


@pytest.mark.parametrize("name", ["tiny", "mixtral8x7b_decode_t16", "mixtral8x22b_decode_t256_zipf",
                                  "mixtral8x7b_prefill_t4096_zipf"])
def test_safe_wait_build_gives_identical_bits(name):
    cfg = synth.config_by_name(name)
    q = synth.gen_qmap(cfg)
    rw = ResidentWeights(ctx(), 1, cfg.weight_experts)
    for e in range(cfg.weight_experts):
        for u in (0, 1):
            rw.add_block(0, e, u, synth.gpu.planes(cfg, 0, e, u), synth.gpu.parent_lut(cfg, 0, e, u), int(q[e, u]))
    rw.commit()
    tbl_safe = rw.mirror_table(safe_ctx())
    x, wr, bias = synth.gen_x(cfg), synth.gen_router(cfg), synth.gen_bias(cfg)
    x_d, wr_d = dev(x), dev(wr)
    bias_d = None if bias is None else dev(bias)
    print(f"{name}: default build", flush=True)
    a = _layer_outputs(ctx(), rw.table, cfg, x_d, wr_d, bias_d)
    print(f"{name}: safe-wait build", flush=True)
    b = _layer_outputs(safe_ctx(), tbl_safe, cfg, x_d, wr_d, bias_d)
    for n in a:
        assert np.array_equal(a[n].view(np.uint8), b[n].view(np.uint8)), n
    assert np.array_equal(a["a"].view(np.uint16), a["a_fused"].view(np.uint16))
    print(f"{name}: counts {a['counts'].tolist()}: identical", flush=True)
    tbl_safe.close()
    rw.close()
