"""Full-size workloads on the GPU, checked against the fp64 oracle on sampled tokens.

- Mixtral-8x22B-shaped decode layer (256 tokens, Zipf 1.2 router bias, hot/cold q).
- Mixtral-8x7B-shaped prefill layer (4096 tokens, Zipf 0.8).
- 32 Mixtral-8x7B layers resident (45 GB of planes), decode batch 32, with the q map
  switched between two committed maps at a launch boundary (PagedWeight, Section 3.3:
  commits only at safe boundaries).
- Many small experts plus shared experts (the fine-grained models of Table 1: 60
  routed + 4 shared top-4, 128 routed + 1 shared top-8; hidden and FFN sizes chosen),
  decode and prefill.

Bars: routing bit-exact for all tokens; the outputs of the evaluated tokens within
max-abs 1e-2 and relative L2 2e-3 of the oracle.  The evaluated tokens are chosen
from the routing so that every expert's first and last row is among them, and for
experts on the tile product (more than 64 rows) the first and last row of every
256-row token tile, so every product and every partial tile is compared at full
size; 32 seeded random tokens are added.  At the prefill size one complete tile
expert is also compared row by row on both products against the block product of
the oracle, within the fp32 accumulation bound.
"""
import numpy as np
import pytest
import torch

import any_precision_weight_amd as apw
import oracle
import synth
import synth.gpu
from any_precision_weight_amd.resident import ResidentWeights
from gpu_util import check_out, check_route, ctx, dev, host, topk_margin_ok, ulp16

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _run_layer(rw, layer, x_d, wr_d, bias_d, cfg, T):
    k, H, F, E, Et = cfg.assign, cfg.hidden, cfg.ffn, cfg.experts, cfg.weight_experts
    R = T * k
    o = dict(ids=torch.empty((T, k), dtype=torch.int32, device="cuda"),
             w=torch.empty((T, k), dtype=torch.float32, device="cuda"),
             counts=torch.empty(Et, dtype=torch.int32, device="cuda"),
             offsets=torch.empty(Et + 1, dtype=torch.int32, device="cuda"),
             perm=torch.empty(R, dtype=torch.int32, device="cuda"),
             inv_perm=torch.empty(R, dtype=torch.int32, device="cuda"),
             h=torch.empty((R, 2 * F), dtype=torch.float16, device="cuda"),
             a=torch.empty((R, F), dtype=torch.float16, device="cuda"),
             y=torch.empty((R, H), dtype=torch.float32, device="cuda"),
             out=torch.empty((T, H), dtype=torch.float16, device="cuda"))
    c = ctx()
    apw.route(c, x_d, wr_d, bias_d, T, H, E, cfg.topk, cfg.renormalize, o["ids"], o["w"], o["counts"],
              o["offsets"], o["perm"], o["inv_perm"], n_shared=cfg.shared)
    apw.gemm(c, rw.table, layer, apw.GATE_UP, x_d, True, o["perm"], o["offsets"], T, k, o["h"], apw.F16)
    apw.act(c, o["h"], R, F, o["a"])
    apw.gemm(c, rw.table, layer, apw.DOWN, o["a"], False, o["perm"], o["offsets"], T, k, o["y"], apw.F32)
    apw.combine(c, o["y"], apw.F32, o["w"], o["inv_perm"], T, k, H, o["out"])
    return o


def _upload_layer_gpu(rw, cfg, gen_layer, slot, q):
    """Blocks generated on the device (bit-identical to synth.gen), tiled, LUT levels built."""
    for e in range(cfg.weight_experts):
        for u in (0, 1):
            rw.add_block(slot, e, u, synth.gpu.planes(cfg, gen_layer, e, u), synth.gpu.parent_lut(cfg, gen_layer, e, u),
                         int(q[e, u]))


def _oracle_layer(cfg, layer, q, eval_tokens):
    E = cfg.weight_experts
    x, wr, bias = synth.gen_x(cfg, layer), synth.gen_router(cfg, layer), synth.gen_bias(cfg, layer)
    pg = [synth.gen_planes(cfg, layer, e, 0) for e in range(E)]
    pd = [synth.gen_planes(cfg, layer, e, 1) for e in range(E)]
    lg = [synth.gen_parent_lut(cfg, layer, e, 0) for e in range(E)]
    ld = [synth.gen_parent_lut(cfg, layer, e, 1) for e in range(E)]
    r = oracle.moe_forward(x, wr, bias, cfg.topk, pg, lg, q[:, 0], pd, ld, q[:, 1], eval_tokens=eval_tokens,
                           renormalize=cfg.renormalize, n_shared=cfg.shared)
    return r, x, wr, bias


def coverage_tokens(route, kt, T, n_random=32, seed=0):
    """Tokens whose rows include, for every expert, its first and last row and, for
    experts with more than 64 rows (the tile product, 256-row token tiles), the first
    and last row of every token tile; plus n_random seeded random tokens."""
    offsets, perm = route["offsets"], route["perm"]
    rows = set()
    for e in range(offsets.size - 1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        rows.update((r0, r1 - 1))
        if r1 - r0 > 64:
            for t0 in range(r0, r1, 256):
                rows.update((t0, min(t0 + 255, r1 - 1)))
    toks = {int(perm[r]) // kt for r in rows}
    rng = np.random.default_rng(seed)
    toks.update(int(t) for t in rng.choice(T, size=min(n_random, T), replace=False))
    return sorted(toks)


def _single_layer_case(cfg, eval_tokens=None):
    """eval_tokens None: coverage_tokens of the layer's routing; "all": every token."""
    q = synth.gen_qmap(cfg)
    rw = ResidentWeights(ctx(), 1, cfg.weight_experts)
    _upload_layer_gpu(rw, cfg, 0, 0, q)
    rw.commit()
    x, wr, bias = synth.gen_x(cfg), synth.gen_router(cfg), synth.gen_bias(cfg)
    assert topk_margin_ok(x, wr, bias, cfg.topk)
    if eval_tokens is None:
        route = oracle.route(x, wr, bias, cfg.topk, cfg.renormalize, n_shared=cfg.shared)
        eval_tokens = coverage_tokens(route, cfg.assign, cfg.tokens)
    elif eval_tokens == "all":
        eval_tokens = list(range(cfg.tokens))
    print(f"{cfg.name}: evaluating {len(eval_tokens)} tokens", flush=True)
    o = _run_layer(rw, 0, dev(x), dev(wr), None if bias is None else dev(bias), cfg, cfg.tokens)
    torch.cuda.synchronize()
    r, *_ = _oracle_layer(cfg, 0, q, np.array(eval_tokens, np.int32))
    check_route(o, r)
    ma, rl = check_out(host(o["out"])[eval_tokens], r["out"])
    print(f"{cfg.name}: {len(eval_tokens)} tokens: max-abs {ma:.3e} rel-L2 {rl:.3e}", flush=True)
    rw.close()
    return r, q


def test_mixtral8x22b_decode_skewed():
    cfg = synth.config_by_name("mixtral8x22b_decode_t256_zipf")
    r, q = _single_layer_case(cfg)
    # the generator's hot experts (Zipf ranks 1 and 2) are the top-2 by Eq. 1 routing mass
    mass = oracle.routing_mass(r["ids"], r["w64"], cfg.experts)
    assert sorted(np.argsort(-mass, kind="stable")[:2].tolist()) == synth.hot_experts(cfg)
    assert all(q[e, u] >= 6 for e in synth.hot_experts(cfg) for u in (0, 1))


def test_mixtral8x7b_prefill():
    cfg = synth.config_by_name("mixtral8x7b_prefill_t4096_zipf")
    _single_layer_case(cfg)


def test_mixtral8x7b_prefill_complete_tile_expert():
    """Every row of one tile expert at the full prefill size (the expert with the
    fewest rows: two or more 256-row token tiles, the last one partial): gate_up to
    fp16 h and down to fp32 y, each against the oracle's block product of the GPU's
    own input rows, within half an fp16 ulp plus the fp32 accumulation bound
    K * 2^-24 * sum |x| |W|."""
    cfg = synth.config_by_name("mixtral8x7b_prefill_t4096_zipf")
    q = synth.gen_qmap(cfg)
    rw = ResidentWeights(ctx(), 1, cfg.weight_experts)
    _upload_layer_gpu(rw, cfg, 0, 0, q)
    rw.commit()
    x, wr, bias = synth.gen_x(cfg), synth.gen_router(cfg), synth.gen_bias(cfg)
    o = _run_layer(rw, 0, dev(x), dev(wr), None if bias is None else dev(bias), cfg, cfg.tokens)
    torch.cuda.synchronize()
    counts, offsets, perm = host(o["counts"]), host(o["offsets"]), host(o["perm"])
    e = int(np.argmin(np.where(counts > 64, counts, 1 << 30)))
    r0, r1 = int(offsets[e]), int(offsets[e + 1])
    assert r1 - r0 > 256 and (r1 - r0) % 256 != 0, counts
    print(f"complete tile expert {e}: {r1 - r0} rows, q gate_up {q[e, 0]} down {q[e, 1]}", flush=True)
    H, F, kt = cfg.hidden, cfg.ffn, cfg.assign

    def check(kind, inp, got, out_f16):
        P = synth.gen_planes(cfg, 0, e, kind)
        lut = oracle.lut_level(synth.gen_parent_lut(cfg, 0, e, kind), int(q[e, kind]))
        ref = oracle.block_gemm(P, lut, int(q[e, kind]), inp)
        S = oracle.block_gemm(P, np.abs(lut.astype(np.float64)), int(q[e, kind]), np.abs(inp))
        acc = inp.shape[1] * 2.0 ** -24 * S
        tol = acc + (0.5 * ulp16(np.abs(ref) + acc) if out_f16 else 0.0)
        d = np.abs(got - ref)
        assert np.all(d <= tol), (kind, float((d - tol).max()))
        return float(d.max())

    xin = x[perm[r0:r1] // kt].astype(np.float64)
    dg = check(0, xin, host(o["h"][r0:r1]).astype(np.float64), True)
    dd = check(1, host(o["a"][r0:r1]).astype(np.float64), host(o["y"][r0:r1]).astype(np.float64), False)
    print(f"complete tile expert {e}: gate_up max |d| {dg:.3e}, down max |d| {dd:.3e}", flush=True)
    rw.close()


def test_mixtral8x7b_prefill_fused_activation():
    """At full prefill size (tile product), gate_up with the activation fused gives
    the bits of gate_up to fp16 h plus the activation launch."""
    cfg = synth.config_by_name("mixtral8x7b_prefill_t4096_zipf")
    q = synth.gen_qmap(cfg)
    rw = ResidentWeights(ctx(), 1, cfg.weight_experts)
    _upload_layer_gpu(rw, cfg, 0, 0, q)
    rw.commit()
    x, wr, bias = synth.gen_x(cfg), synth.gen_router(cfg), synth.gen_bias(cfg)
    x_d = dev(x)
    o = _run_layer(rw, 0, x_d, dev(wr), None if bias is None else dev(bias), cfg, cfg.tokens)
    a = torch.empty_like(o["a"])
    apw.gemm_act(ctx(), rw.table, 0, x_d, True, o["perm"], o["offsets"], cfg.tokens, cfg.assign, a)
    torch.cuda.synchronize()
    assert np.array_equal(host(a).view(np.uint16), host(o["a"]).view(np.uint16))
    rw.close()


def test_32_layers_resident_with_map_switch():
    cfg = synth.config_by_name("mixtral8x7b_32layer_decode_t32")
    L, E, T = cfg.layers, cfg.experts, cfg.tokens
    qa = [synth.gen_qmap(cfg, l, 0) for l in range(L)]
    qb = [synth.gen_qmap(cfg, l, 1) for l in range(L)]
    rw = ResidentWeights(ctx(), L, E)
    for l in range(L):
        _upload_layer_gpu(rw, cfg, l, l, qa[l])
    rw.commit()
    xs = [dev(synth.gen_x(cfg, l)) for l in range(L)]
    wrs = [dev(synth.gen_router(cfg, l)) for l in range(L)]
    # map A for every layer, then map B committed at a launch boundary, no host sync
    outs_a = [_run_layer(rw, l, xs[l], wrs[l], None, cfg, T) for l in range(L)]
    for l in range(L):
        rw.stage_qmap(l, qb[l])
    rw.commit()
    outs_b = [_run_layer(rw, l, xs[l], wrs[l], None, cfg, T) for l in range(L)]
    torch.cuda.synchronize()
    mean_a = float(np.mean([qa[l].mean() for l in range(L)]))
    mean_b = float(np.mean([qb[l].mean() for l in range(L)]))
    print(f"32 layers: realised mean bits map A {mean_a:.3f}, map B {mean_b:.3f}", flush=True)
    assert 5.8 < mean_a < 6.2 and 3.8 < mean_b < 4.2
    ev = np.arange(T, dtype=np.int32)  # every token of the batch
    for layer in (5, 31):
        for q, outs in ((qa[layer], outs_a), (qb[layer], outs_b)):
            r, x, wr, _ = _oracle_layer(cfg, layer, q, ev)
            check_route(outs[layer], r)
            ma, rl = check_out(host(outs[layer]["out"])[ev], r["out"])
            print(f"layer {layer} mean q {q.mean():.2f}: max-abs {ma:.3e} rel-L2 {rl:.3e}", flush=True)
    rw.close()


@pytest.mark.parametrize("name,tokens", [("qwen_60r4s_top4_decode_t64", "all"),
                                         ("gemma_128r1s_top8_decode_t64", "all"),
                                         ("qwen_60r4s_top4_prefill_t2048", None)])
def test_shared_expert_workloads(name, tokens):
    cfg = synth.config_by_name(name)
    r, q = _single_layer_case(cfg, tokens)
    T, k, E = cfg.tokens, cfg.topk, cfg.experts
    # every token's row ends with the shared experts at weight 1; each holds all T rows
    assert np.array_equal(r["ids"][:, k:], np.tile(np.arange(E, E + cfg.shared, dtype=np.int32), (T, 1)))
    assert np.all(r["counts"][E:] == T)
