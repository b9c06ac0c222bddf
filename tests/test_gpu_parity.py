"""GPU parity of libapmoe against the fp64 oracle (calls go through the C ABI).

Bars: route ids, counts, offsets, perm, inv_perm bit-exact; routing weights
within 1e-6; identity-LUT products (integers, fp32 out) bit-exact; fp16 products
within half an fp16 ulp plus the fp32 accumulation bound; layer outputs within
max-abs 1e-2 and relative L2 2e-3 of the fp64 oracle.

Paper: PagedWeight (arXiv:2607.16184), Section 2.1 (router, Eq. 1), Section 3 /
Figure 3 caption (bit-planes + LUT), Section 3.1 (page table, q_i only over
resident planes), Section 3.3 (safe-boundary commits; fused MoE layer).
"""
import numpy as np
import pytest
import torch

import any_precision_weight_amd as apw
import oracle
import synth
from gpu_util import Layer, check_out, check_route, ctx, dev, host, topk_margin_ok, ulp16

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(2024)


# --------------------------------------------------------------------------- route

ROUTE_CASES = [
    # (T, H, E, k, bias, renorm, seed)
    (8, 256, 4, 2, False, True, 0),
    (1, 4096, 8, 2, False, True, 1),
    (13, 4096, 8, 2, True, True, 2),
    (300, 512, 60, 4, False, True, 3),
    (37, 256, 128, 8, True, True, 4),
    (50, 256, 8, 2, True, False, 5),
    (1500, 128, 8, 2, True, True, 6),
    (0, 256, 8, 2, False, True, 7),
]


@pytest.mark.parametrize("case", ROUTE_CASES, ids=lambda c: f"T{c[0]}H{c[1]}E{c[2]}k{c[3]}")
def test_route_parity(case):
    T, H, E, k, use_bias, renorm, seed = case
    x = synth.fp16_normal(100 + seed, 1, T * H, 1.0).reshape(T, H)
    wr = synth.fp16_normal(100 + seed, 2, E * H, 0.02).reshape(E, H)
    bias = synth.fp16_normal(100 + seed, 3, E, 1.0).astype(np.float32) if use_bias else None
    if T > 0:
        assert topk_margin_ok(x, wr, bias, k)
    r = oracle.route(x, wr, bias, k, renorm)
    R = T * k
    o = dict(ids=torch.empty((T, k), dtype=torch.int32, device="cuda"),
             w=torch.empty((T, k), dtype=torch.float32, device="cuda"),
             counts=torch.full((E,), -1, dtype=torch.int32, device="cuda"),
             offsets=torch.full((E + 1,), -1, dtype=torch.int32, device="cuda"),
             perm=torch.empty(R, dtype=torch.int32, device="cuda"),
             inv_perm=torch.empty(R, dtype=torch.int32, device="cuda"))
    xd = dev(x) if T > 0 else torch.empty((1, H), dtype=torch.float16, device="cuda")
    apw.route(ctx(), xd, dev(wr), None if bias is None else dev(bias), T, H, E, k, renorm, o["ids"], o["w"],
              o["counts"], o["offsets"], o["perm"], o["inv_perm"])
    torch.cuda.synchronize()
    check_route(o, r)


@pytest.mark.parametrize("case", ROUTE_CASES[:3], ids=lambda c: f"T{c[0]}H{c[1]}E{c[2]}k{c[3]}")
def test_route_stats_accumulate(case):
    """Eq. 1 terms accumulated over two calls: selection counts exact; with dyadic
    weights every fp64 sum is exact whatever the order, so the masses match bit for
    bit; with the router's own weights they match within the fp64 summation bound."""
    T, H, E, k, use_bias, renorm, seed = case
    x = synth.fp16_normal(100 + seed, 1, T * H, 1.0).reshape(T, H)
    wr = synth.fp16_normal(100 + seed, 2, E * H, 0.02).reshape(E, H)
    R = T * k
    o = dict(ids=torch.empty((T, k), dtype=torch.int32, device="cuda"),
             w=torch.empty((T, k), dtype=torch.float32, device="cuda"),
             counts=torch.empty(E, dtype=torch.int32, device="cuda"),
             offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
             perm=torch.empty(max(R, 1), dtype=torch.int32, device="cuda"),
             inv_perm=torch.empty(max(R, 1), dtype=torch.int32, device="cuda"))
    apw.route(ctx(), dev(x), dev(wr), None, T, H, E, k, renorm, o["ids"], o["w"], o["counts"], o["offsets"],
              o["perm"], o["inv_perm"])
    mass = torch.zeros(E, dtype=torch.float64, device="cuda")
    total = torch.zeros(1, dtype=torch.float64, device="cuda")
    sel = torch.zeros(E, dtype=torch.int64, device="cuda")
    for _ in range(2):
        apw.route_stats(ctx(), o["w"], o["perm"], o["offsets"], T, k, E, mass, total, sel)
    torch.cuda.synchronize()
    ids, w = host(o["ids"]), host(o["w"])
    num, cnt, den = oracle.route_stats(ids, w, E)
    assert np.array_equal(host(sel), 2 * cnt)
    bound = 2 * R * 2.0 ** -52 * (2 * den) + 1e-300
    assert np.all(np.abs(host(mass) - 2 * num) <= bound)
    assert abs(float(host(total)[0]) - 2 * den) <= bound
    # dyadic weights: exact in any summation order
    wd = (RNG.integers(1, 1024, (T, k)) / 1024.0).astype(np.float32)
    mass.zero_(), total.zero_(), sel.zero_()
    apw.route_stats(ctx(), dev(wd), o["perm"], o["offsets"], T, k, E, mass, total, sel)
    torch.cuda.synchronize()
    num, cnt, den = oracle.route_stats(ids, wd, E)
    assert np.array_equal(host(mass), num) and float(host(total)[0]) == den
    assert np.array_equal(host(sel), cnt)


SHARED_ROUTE_CASES = [
    # T, H, E routed, k, shared, bias, renormalize, seed
    (37, 256, 12, 3, 2, False, True, 11),
    (64, 512, 60, 4, 4, True, False, 12),
    (5, 256, 128, 8, 1, False, True, 13),
    (16, 256, 248, 8, 8, False, True, 14),  # E + shared = 256 experts, the most shared experts
    (0, 256, 8, 2, 3, False, True, 15),
    (9, 256, 4, 4, 2, False, False, 16),  # every routed expert chosen
]


@pytest.mark.parametrize("case", SHARED_ROUTE_CASES, ids=lambda c: f"T{c[0]}E{c[2]}k{c[3]}s{c[4]}")
def test_route_shared_parity(case):
    """Shared experts: each token's row is its top-k routed experts, then the shared
    ones at weight 1; the sort groups all E + shared experts."""
    T, H, E, k, S, use_bias, renorm, seed = case
    x = synth.fp16_normal(200 + seed, 1, T * H, 1.0).reshape(T, H)
    wr = synth.fp16_normal(200 + seed, 2, E * H, 0.02).reshape(E, H)
    bias = synth.fp16_normal(200 + seed, 3, E, 1.0).astype(np.float32) if use_bias else None
    if T > 0:
        assert topk_margin_ok(x, wr, bias, k)
    r = oracle.route(x, wr, bias, k, renorm, n_shared=S)
    kt, R = k + S, T * (k + S)
    o = dict(ids=torch.empty((T, kt), dtype=torch.int32, device="cuda"),
             w=torch.empty((T, kt), dtype=torch.float32, device="cuda"),
             counts=torch.full((E + S,), -1, dtype=torch.int32, device="cuda"),
             offsets=torch.full((E + S + 1,), -1, dtype=torch.int32, device="cuda"),
             perm=torch.empty(max(R, 1), dtype=torch.int32, device="cuda"),
             inv_perm=torch.empty(max(R, 1), dtype=torch.int32, device="cuda"))
    xd = dev(x) if T > 0 else torch.empty((1, H), dtype=torch.float16, device="cuda")
    apw.route(ctx(), xd, dev(wr), None if bias is None else dev(bias), T, H, E, k, renorm, o["ids"], o["w"],
              o["counts"], o["offsets"], o["perm"], o["inv_perm"], n_shared=S)
    torch.cuda.synchronize()
    o["perm"], o["inv_perm"] = o["perm"][:R], o["inv_perm"][:R]
    check_route(o, r)
    assert np.all(host(o["counts"])[E:] == T)
    if T == 0:
        return
    # Eq. 1 statistics over the routed choices only: routed E, row stride k + shared
    mass = torch.zeros(E, dtype=torch.float64, device="cuda")
    total = torch.zeros(1, dtype=torch.float64, device="cuda")
    sel = torch.zeros(E, dtype=torch.int64, device="cuda")
    apw.route_stats(ctx(), o["w"], o["perm"], o["offsets"], T, kt, E, mass, total, sel)
    torch.cuda.synchronize()
    num, cnt, den = oracle.route_stats(r["ids"][:, :k], r["w32"][:, :k], E)
    assert np.array_equal(host(sel), cnt)
    bound = R * 2.0 ** -52 * den + 1e-300
    assert np.all(np.abs(host(mass) - num) <= bound)
    assert abs(float(host(total)[0]) - den) <= bound


def test_route_shared_rejected():
    H, E = 256, 250
    x = dev(synth.fp16_normal(7, 1, 4 * H, 1.0).reshape(4, H))
    wr = dev(synth.fp16_normal(7, 2, E * H, 0.02).reshape(E, H))
    buf = torch.empty(4096, dtype=torch.int32, device="cuda")
    wbuf = torch.empty(4096, dtype=torch.float32, device="cuda")
    for S in (-1, 7, 9):  # 7: E + S above 256 experts; 9: above the shared-expert limit
        with pytest.raises(apw.ApmoeError) as ex:
            apw.route(ctx(), x, wr, None, 4, H, E, 2, True, buf, wbuf, buf, buf, buf, buf, n_shared=S)
        assert ex.value.status == apw.INVALID_ARG


def test_route_ties_lower_index():
    T, H, E, k = 40, 256, 8, 2
    x = synth.fp16_normal(9, 1, T * H, 1.0).reshape(T, H)
    wr = synth.fp16_normal(9, 2, E * H, 0.02).reshape(E, H)
    wr[5] = wr[2]
    wr[7] = wr[2]
    r = oracle.route(x, wr, None, k)
    o = dict(ids=torch.empty((T, k), dtype=torch.int32, device="cuda"),
             w=torch.empty((T, k), dtype=torch.float32, device="cuda"),
             counts=torch.empty(E, dtype=torch.int32, device="cuda"),
             offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
             perm=torch.empty(T * k, dtype=torch.int32, device="cuda"),
             inv_perm=torch.empty(T * k, dtype=torch.int32, device="cuda"))
    apw.route(ctx(), dev(x), dev(wr), None, T, H, E, k, True, o["ids"], o["w"], o["counts"], o["offsets"],
              o["perm"], o["inv_perm"])
    torch.cuda.synchronize()
    check_route(o, r)
    assert np.any(np.isin(r["ids"], [2, 5, 7]))


# --------------------------------------------------------------------------- format tools

def test_lut_build_parity():
    n = 300
    # random finite fp16 patterns (subnormals, large magnitudes, exact ties) and a real parent
    bits = RNG.integers(0, 0x7C00, (n // 2, 256)).astype(np.uint16)
    bits |= (RNG.integers(0, 2, bits.shape).astype(np.uint16) << 15)
    parent = np.concatenate([bits.view(np.float16), synth.gen_parent_lut_shape(5, 0, 0, 0, n - n // 2)])
    pd = dev(parent)
    levels = {b: torch.empty((n, 1 << b), dtype=torch.float16, device="cuda") for b in range(3, 8)}
    apw.lut_build(ctx(), pd, n, levels)
    torch.cuda.synchronize()
    for b in range(3, 8):
        ref = oracle.lut_level(parent, b).view(np.uint16)
        got = host(levels[b]).view(np.uint16)
        assert np.array_equal(got, ref), b


def _tiled_numpy(P):
    """The documented tiled layout, written independently with numpy reshapes:
    tiles of 32 rows x 128 columns; slot L = 32g + i holds row i, 2 words for
    columns 64g..64g+63."""
    _, N, W = P.shape
    RT, KT = (N + 31) // 32, W // 4
    pad = np.zeros((8, RT * 32, W), np.uint32)
    pad[:, :N] = P
    t = pad.reshape(8, RT, 32, KT, 2, 2)          # plane, rt, i, kt, g, word
    t = t.transpose(0, 1, 3, 4, 2, 5)             # plane, rt, kt, g, i, word
    return t.reshape(8, RT * KT * 128)


@pytest.mark.parametrize("NK", [(77, 384), (64, 128), (200, 1024)])
def test_tile_planes_layout(NK):
    N, K = NK
    P = synth.gen_planes_shape(13, 0, 0, 0, N, K)
    out = torch.full((8, apw.tiled_plane_words(N, K)), -1, dtype=torch.int32, device="cuda")
    apw.tile_planes(ctx(), dev(P), N, K, out)
    torch.cuda.synchronize()
    assert np.array_equal(host(out).view(np.uint32), _tiled_numpy(P))


def test_pack_planes_parity():
    n, k = 77, 384
    codes = RNG.integers(0, 256, (n, k)).astype(np.uint8)
    planes = torch.empty((8, n, k // 32), dtype=torch.int32, device="cuda")
    apw.pack_planes(ctx(), dev(codes), n, k, planes)
    torch.cuda.synchronize()
    assert np.array_equal(host(planes).view(np.uint32), oracle.pack_planes(codes))


# --------------------------------------------------------------------------- expert product

def _gemm_setup(qs, counts, N, K, identity, seed):
    """One layer, E = len(qs) experts, gate_up kind, given per-expert token counts."""
    E = len(qs)
    tbl = apw.Table(1, E)
    keep = []
    planes_np, luts_np = [], []
    for e, q in enumerate(qs):
        P = synth.gen_planes_shape(seed, 0, e, 0, N, K)
        Pd = torch.empty((8, apw.tiled_plane_words(N, K)), dtype=torch.int32, device="cuda")
        apw.tile_planes(ctx(), dev(P), N, K, Pd)
        if identity:
            lut = np.tile(np.arange(1 << q, dtype=np.float16), (N, 1))
        else:
            lut = oracle.lut_level(synth.gen_parent_lut_shape(seed, 0, e, 0, N), q)
        Ld = dev(lut)
        keep += [Pd, Ld]
        planes_np.append(P)
        luts_np.append(lut)
        tbl.set_block(0, e, 0, N, K, q, [Pd[p] for p in range(8)], {q: Ld})
        # the down slot must be present for a complete layer; reuse the same block
        tbl.set_block(0, e, 1, N, K, q, [Pd[p] for p in range(8)], {q: Ld})
    tbl.commit(ctx())
    R = int(sum(counts))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = R  # gather: topk = 1, a random permutation of tokens
    perm = RNG.permutation(R).astype(np.int32)
    return tbl, keep, planes_np, luts_np, offsets, perm, T


def _gemm_run(tbl, x, offsets, perm, T, N, out_dtype, gather=True):
    R = int(offsets[-1])
    out = torch.full((R, N), float("nan"), dtype=torch.float32 if out_dtype == apw.F32 else torch.float16,
                     device="cuda")
    apw.gemm(ctx(), tbl, 0, apw.GATE_UP, dev(x), gather, dev(perm), dev(offsets), T, 1, out, out_dtype)
    torch.cuda.synchronize()
    return host(out)


GEMM_QS = [3, 4, 5, 6, 7, 8]
GEMM_COUNTS = [0, 1, 33, 70, 5, 31]


@pytest.mark.parametrize("NK", [(136, 384), (64, 256), (200, 1024), (96, 128), (112, 128), (40, 640)])
def test_gemm_identity_lut_exact(NK):
    """Identity LUT + integer activations: every partial sum is an integer below
    2^24, so the fp32 result must equal the integer matmul exactly.  Shapes include
    K = 128 (one 128-column step: the second column half of a workgroup has none),
    an odd number of steps, and N % 64 of 8, 32 and 48 (a partly valid row tile)."""
    N, K = NK
    tbl, keep, P, L, offsets, perm, T = _gemm_setup(GEMM_QS, GEMM_COUNTS, N, K, True, 41)
    x = RNG.integers(-2, 3, (T, K)).astype(np.float16)
    got = _gemm_run(tbl, x, offsets, perm, T, N, apw.F32)
    for e, q in enumerate(GEMM_QS):
        rows = perm[offsets[e]:offsets[e + 1]]
        codes = oracle.unpack_codes(P[e], q).astype(np.int64)
        ref = x[rows].astype(np.int64) @ codes.T
        assert np.array_equal(got[offsets[e]:offsets[e + 1]], ref.astype(np.float32)), (e, q)
    tbl.close()


@pytest.mark.parametrize("counts", [[9, 1, 0, 3, 2, 1], [0, 1, 20, 3, 5, 3], [0, 0, 32, 0, 0, 0]])
def test_gemm_decode_multipass_exact(counts):
    """The decode product's token buffers hold 8 rows (batches up to 16 tokens) or 16
    rows: an expert with more rows takes a second pass over its weights (9 rows of 16
    tokens; 20 and 32 rows of 32 tokens)."""
    N, K = 136, 384
    tbl, keep, P, L, offsets, perm, T = _gemm_setup(GEMM_QS, counts, N, K, True, 50)
    x = RNG.integers(-2, 3, (T, K)).astype(np.float16)
    got = _gemm_run(tbl, x, offsets, perm, T, N, apw.F32)
    for e, q in enumerate(GEMM_QS):
        rows = perm[offsets[e]:offsets[e + 1]]
        codes = oracle.unpack_codes(P[e], q).astype(np.int64)
        ref = x[rows].astype(np.int64) @ codes.T
        assert np.array_equal(got[offsets[e]:offsets[e + 1]], ref.astype(np.float32)), (e, q, counts[e])
    tbl.close()


@pytest.mark.parametrize("counts", [[2, 5, 0, 9, 4, 12], [17, 1, 3, 0, 0, 11]])
def test_gemm_decode_two_parts_exact(counts):
    """32 tokens with 16-row token buffers and two column parts (N/64 row blocks per
    expert, more than 1024 in all, the headline's launch shape), every q, one expert
    with 17 rows (two passes): every expert's rows exact against the integer matmul
    (identity LUTs), and the fused activation equals gate_up to fp16 followed by the
    activation launch."""
    N, K = 11264, 256
    tbl, keep, P, L, offsets, perm, T = _gemm_setup(GEMM_QS, counts, N, K, True, 53)
    assert 16 < T <= 32 and N // 64 * len(GEMM_QS) > 1024
    x = RNG.integers(-2, 3, (T, K)).astype(np.float16)
    got = _gemm_run(tbl, x, offsets, perm, T, N, apw.F32)
    for e, q in enumerate(GEMM_QS):
        rows = perm[offsets[e]:offsets[e + 1]]
        codes = oracle.unpack_codes(P[e], q).astype(np.int64)
        ref = x[rows].astype(np.int64) @ codes.T
        assert np.array_equal(got[offsets[e]:offsets[e + 1]], ref.astype(np.float32)), (e, q, counts[e])
    R = int(offsets[-1])
    h = torch.empty((R, N), dtype=torch.float16, device="cuda")
    a2 = torch.empty((R, N // 2), dtype=torch.float16, device="cuda")
    a1 = torch.full((R, N // 2), float("nan"), dtype=torch.float16, device="cuda")
    xd, pd, od = dev(x), dev(perm), dev(offsets)
    apw.gemm(ctx(), tbl, 0, apw.GATE_UP, xd, True, pd, od, T, 1, h, apw.F16)
    apw.act(ctx(), h, R, N // 2, a2)
    apw.gemm_act(ctx(), tbl, 0, xd, True, pd, od, T, 1, a1)
    torch.cuda.synchronize()
    assert np.array_equal(host(a1).view(np.uint16), host(a2).view(np.uint16))
    tbl.close()


def test_gemm_many_experts_exact():
    """Above 16 experts the decode and mid products start the experts in the host's
    order of the committed q map (a scheduling hint): 40 experts, q cycling 3..8,
    rows 0..70 (decode, mid and tile products in one call), identity LUTs, exact."""
    E = 40
    qs = [3 + (e * 5) % 6 for e in range(E)]
    counts = [(e * 37) % 71 for e in range(E)]
    N, K = 136, 256
    tbl, keep, P, L, offsets, perm, T = _gemm_setup(qs, counts, N, K, True, 52)
    x = RNG.integers(-2, 3, (T, K)).astype(np.float16)
    got = _gemm_run(tbl, x, offsets, perm, T, N, apw.F32)
    for e, q in enumerate(qs):
        rows = perm[offsets[e]:offsets[e + 1]]
        codes = oracle.unpack_codes(P[e], q).astype(np.int64)
        ref = x[rows].astype(np.int64) @ codes.T
        assert np.array_equal(got[offsets[e]:offsets[e + 1]], ref.astype(np.float32)), (e, q, counts[e])
    tbl.close()


@pytest.mark.parametrize("out_dtype", [apw.F16, apw.F32])
def test_gemm_random_lut(out_dtype):
    N, K = 136, 384
    tbl, keep, P, L, offsets, perm, T = _gemm_setup(GEMM_QS, GEMM_COUNTS, N, K, False, 42)
    x = synth.gen_aux_fp16(42, 0, T * K).reshape(T, K)
    got = _gemm_run(tbl, x, offsets, perm, T, N, out_dtype).astype(np.float64)
    for e, q in enumerate(GEMM_QS):
        rows = perm[offsets[e]:offsets[e + 1]]
        if rows.size == 0:
            continue
        xin = x[rows].astype(np.float64)
        ref = oracle.block_gemm(P[e], L[e], q, xin)
        S = oracle.block_gemm(P[e], np.abs(L[e]), q, np.abs(xin))
        acc = K * 2.0 ** -24 * S
        tol = acc + (0.5 * ulp16(np.abs(ref) + acc) if out_dtype == apw.F16 else 0.0)
        d = np.abs(got[offsets[e]:offsets[e + 1]] - ref)
        assert np.all(d <= tol), (e, q, float((d - tol).max()))
    tbl.close()


def test_gemm_non_gather_rows():
    N, K = 64, 256
    tbl, keep, P, L, offsets, perm, T = _gemm_setup(GEMM_QS, GEMM_COUNTS, N, K, True, 43)
    R = int(offsets[-1])
    a = RNG.integers(-2, 3, (R, K)).astype(np.float16)
    got = _gemm_run(tbl, a, offsets, perm, R, N, apw.F32, gather=False)
    for e, q in enumerate(GEMM_QS):
        codes = oracle.unpack_codes(P[e], q).astype(np.int64)
        ref = a[offsets[e]:offsets[e + 1]].astype(np.int64) @ codes.T
        assert np.array_equal(got[offsets[e]:offsets[e + 1]], ref.astype(np.float32))
    tbl.close()


# Experts above 64 rows take the MFMA tile product (128 weight rows x 256 rows per
# tile): several token tiles per expert with ragged tails, a weight-row tail, and
# more than one group of 8 weight-row tiles.  The smaller counts in these cases take
# the decode and mid products in the same call.
TILE_CASES = [
    (200, 384, [300, 0, 257, 33, 600, 64]),
    (112, 128, [40, 300, 0, 33, 1, 90]),  # K = 128: one step; N % 128 = 112
    (1280, 256, [40, 300, 1, 31, 500, 32]),
    (64, 1024, [256, 512, 3, 0, 129, 70]),
]


@pytest.mark.parametrize("case", TILE_CASES)
def test_gemm_tile_identity_lut_exact(case):
    N, K, counts = case
    tbl, keep, P, L, offsets, perm, T = _gemm_setup(GEMM_QS, counts, N, K, True, 44)
    x = RNG.integers(-2, 3, (T, K)).astype(np.float16)
    got = _gemm_run(tbl, x, offsets, perm, T, N, apw.F32)
    for e, q in enumerate(GEMM_QS):
        rows = perm[offsets[e]:offsets[e + 1]]
        codes = oracle.unpack_codes(P[e], q).astype(np.int64)
        ref = x[rows].astype(np.int64) @ codes.T
        assert np.array_equal(got[offsets[e]:offsets[e + 1]], ref.astype(np.float32)), (e, q, counts[e])
    tbl.close()


@pytest.mark.parametrize("out_dtype", [apw.F16, apw.F32])
def test_gemm_tile_random_lut(out_dtype):
    N, K, counts = 200, 384, [300, 0, 257, 33, 600, 64]
    tbl, keep, P, L, offsets, perm, T = _gemm_setup(GEMM_QS, counts, N, K, False, 45)
    x = synth.gen_aux_fp16(45, 0, T * K).reshape(T, K)
    got = _gemm_run(tbl, x, offsets, perm, T, N, out_dtype).astype(np.float64)
    for e, q in enumerate(GEMM_QS):
        rows = perm[offsets[e]:offsets[e + 1]]
        if rows.size == 0:
            continue
        xin = x[rows].astype(np.float64)
        ref = oracle.block_gemm(P[e], L[e], q, xin)
        S = oracle.block_gemm(P[e], np.abs(L[e]), q, np.abs(xin))
        acc = K * 2.0 ** -24 * S
        tol = acc + (0.5 * ulp16(np.abs(ref) + acc) if out_dtype == apw.F16 else 0.0)
        d = np.abs(got[offsets[e]:offsets[e + 1]] - ref)
        assert np.all(d <= tol), (e, q, float((d - tol).max()))
    tbl.close()


def test_gemm_tile_non_gather_rows():
    N, K, counts = 136, 256, [70, 300, 0, 33, 1, 260]
    tbl, keep, P, L, offsets, perm, T = _gemm_setup(GEMM_QS, counts, N, K, True, 46)
    R = int(offsets[-1])
    a = RNG.integers(-2, 3, (R, K)).astype(np.float16)
    got = _gemm_run(tbl, a, offsets, perm, R, N, apw.F16, gather=False)
    for e, q in enumerate(GEMM_QS):
        codes = oracle.unpack_codes(P[e], q).astype(np.int64)
        ref = a[offsets[e]:offsets[e + 1]].astype(np.int64) @ codes.T
        assert np.array_equal(got[offsets[e]:offsets[e + 1]].astype(np.float64), ref.astype(np.float16).astype(np.float64))
    tbl.close()


# Experts with 33..64 rows take the mid product (128 weight rows per workgroup, each
# weight decoded once for two 32-token tiles): the boundaries 32 / 33 and 64 / 65
# between the three products, weight-row tails (N % 128 of 72, 8 and 40), K = 128
# (one step) and odd numbers of steps; the other counts take the decode product (one
# or two passes) and the tile product (one to three token tiles) in the same call.
# Blocks at q = 8 (the last expert) take a launch of their own (64 KB LUT region)
# when the launch has many row blocks.
MID_CASES = [
    (200, 384, [32, 64, 65, 16, 17, 33]),
    (136, 128, [128, 33, 0, 100, 1, 65]),
    (40, 640, [64, 127, 17, 96, 16, 50]),
    (256, 1152, [90, 33, 128, 0, 64, 20]),
    (168, 384, [129, 128, 65, 64, 300, 97]),
]


@pytest.mark.parametrize("case", MID_CASES)
def test_gemm_mid_identity_lut_exact(case):
    N, K, counts = case
    tbl, keep, P, L, offsets, perm, T = _gemm_setup(GEMM_QS, counts, N, K, True, 47)
    x = RNG.integers(-2, 3, (T, K)).astype(np.float16)
    got = _gemm_run(tbl, x, offsets, perm, T, N, apw.F32)
    for e, q in enumerate(GEMM_QS):
        rows = perm[offsets[e]:offsets[e + 1]]
        codes = oracle.unpack_codes(P[e], q).astype(np.int64)
        ref = x[rows].astype(np.int64) @ codes.T
        assert np.array_equal(got[offsets[e]:offsets[e + 1]], ref.astype(np.float32)), (e, q, counts[e])
    tbl.close()


def test_gemm_mid_wide_launch_exact():
    """A launch with at least 128 row blocks of 128 rows runs the mid product as two
    launches: blocks at q <= 7 with two workgroups per CU, then the blocks at q = 8
    (here the expert with 50 rows)."""
    N, K, counts = 16384, 256, [33, 64, 40, 0, 5, 50]
    tbl, keep, P, L, offsets, perm, T = _gemm_setup(GEMM_QS, counts, N, K, True, 51)
    x = RNG.integers(-2, 3, (T, K)).astype(np.float16)
    got = _gemm_run(tbl, x, offsets, perm, T, N, apw.F32)
    for e, q in enumerate(GEMM_QS):
        rows = perm[offsets[e]:offsets[e + 1]]
        codes = oracle.unpack_codes(P[e], q).astype(np.int64)
        ref = x[rows].astype(np.int64) @ codes.T
        assert np.array_equal(got[offsets[e]:offsets[e + 1]], ref.astype(np.float32)), (e, q, counts[e])
    tbl.close()


@pytest.mark.parametrize("out_dtype", [apw.F16, apw.F32])
def test_gemm_mid_random_lut(out_dtype):
    N, K, counts = 200, 640, [33, 64, 65, 128, 100, 40]
    tbl, keep, P, L, offsets, perm, T = _gemm_setup(GEMM_QS, counts, N, K, False, 48)
    x = synth.gen_aux_fp16(48, 0, T * K).reshape(T, K)
    got = _gemm_run(tbl, x, offsets, perm, T, N, out_dtype).astype(np.float64)
    for e, q in enumerate(GEMM_QS):
        rows = perm[offsets[e]:offsets[e + 1]]
        xin = x[rows].astype(np.float64)
        ref = oracle.block_gemm(P[e], L[e], q, xin)
        S = oracle.block_gemm(P[e], np.abs(L[e]), q, np.abs(xin))
        acc = K * 2.0 ** -24 * S
        tol = acc + (0.5 * ulp16(np.abs(ref) + acc) if out_dtype == apw.F16 else 0.0)
        d = np.abs(got[offsets[e]:offsets[e + 1]] - ref)
        assert np.all(d <= tol), (e, q, float((d - tol).max()))
    tbl.close()


def test_gemm_mid_non_gather_rows():
    N, K, counts = 136, 256, [70, 128, 0, 33, 1, 64]
    tbl, keep, P, L, offsets, perm, T = _gemm_setup(GEMM_QS, counts, N, K, True, 49)
    R = int(offsets[-1])
    a = RNG.integers(-2, 3, (R, K)).astype(np.float16)
    got = _gemm_run(tbl, a, offsets, perm, R, N, apw.F16, gather=False)
    for e, q in enumerate(GEMM_QS):
        codes = oracle.unpack_codes(P[e], q).astype(np.int64)
        ref = a[offsets[e]:offsets[e + 1]].astype(np.int64) @ codes.T
        assert np.array_equal(got[offsets[e]:offsets[e + 1]].astype(np.float64), ref.astype(np.float16).astype(np.float64))
    tbl.close()


# --------------------------------------------------------------------------- act / combine

def test_act_parity():
    R, F = 37, 1024
    h = synth.gen_aux_fp16(7, 1, R * 2 * F, 2.0).reshape(R, 2 * F)
    a = torch.empty((R, F), dtype=torch.float16, device="cuda")
    apw.act(ctx(), dev(h), R, F, a)
    torch.cuda.synchronize()
    ref = oracle.act(h.astype(np.float64))
    got = host(a).astype(np.float64)
    # fp32 SiLU (relative error well below 1e-5) then one fp16 rounding
    tol = 0.5 * ulp16(np.abs(ref) * (1 + 1e-5)) + 1e-5 * np.abs(ref) + 1e-7
    assert np.all(np.abs(got - ref) <= tol)


@pytest.mark.parametrize("y_dtype", [apw.F32, apw.F16])
def test_combine_parity(y_dtype):
    T, k, H = 19, 3, 512
    R = T * k
    y = synth.gen_aux_fp16(8, 2, R * H, 1.5).reshape(R, H)
    yin = y.astype(np.float32) if y_dtype == apw.F32 else y
    w = RNG.dirichlet(np.ones(k), T).astype(np.float32)
    inv = RNG.permutation(R).astype(np.int32)
    out = torch.empty((T, H), dtype=torch.float16, device="cuda")
    apw.combine(ctx(), dev(yin), y_dtype, dev(w), dev(inv), T, k, H, out)
    torch.cuda.synchronize()
    ref = oracle.combine(y.astype(np.float64), w.astype(np.float64), inv, k)
    got = host(out).astype(np.float64)
    acc = k * 2.0 ** -24 * (np.abs(w).astype(np.float64)[:, :, None] *
                             np.abs(y.astype(np.float64))[inv.reshape(T, k)]).sum(axis=1)
    tol = 0.5 * ulp16(np.abs(ref) + acc) + acc
    assert np.all(np.abs(got - ref) <= tol)


# --------------------------------------------------------------------------- whole layer

def test_layer_tiny_parity():
    cfg = synth.CONFIGS[0]
    assert topk_margin_ok(synth.gen_x(cfg), synth.gen_router(cfg), synth.gen_bias(cfg), cfg.topk)
    L = Layer(cfg)
    o = L.run()
    fused = L.run_fused_call()
    torch.cuda.synchronize()
    r = L.oracle(intermediates=True)
    check_route(o, r)
    check_out(host(o["out"]), r["out"])
    assert np.array_equal(host(fused).view(np.uint16), host(o["out"]).view(np.uint16))
    # h: fp16 rounding of an fp32 accumulation of the exact products
    H = cfg.hidden
    h = host(o["h"]).astype(np.float64)
    for e in range(cfg.experts):
        s, t = r["offsets"][e], r["offsets"][e + 1]
        if s == t:
            continue
        q = int(L.q[e, 0])
        lut = oracle.lut_level(L.parent[(e, 0)], q)
        xin = np.abs(L.x[r["perm"][s:t] // cfg.topk].astype(np.float64))
        S = oracle.block_gemm(L.planes[(e, 0)], np.abs(lut), q, xin)
        acc = H * 2.0 ** -24 * S
        tol = 0.5 * ulp16(np.abs(r["h"][s:t]) + acc) + acc
        assert np.all(np.abs(h[s:t] - r["h"][s:t]) <= tol), e


TINY_SHARED = synth.MoEConfig("tiny_shared", tokens=48, hidden=256, ffn=384, experts=12, topk=3, seed=21,
                              shared=2, note="12 routed + 2 shared experts, top-3")


@pytest.mark.parametrize("T,renorm", [(48, True), (48, False), (7, True), (150, False)])
def test_layer_shared_experts(T, renorm):
    """Shared experts run every token (T rows each: the tile product once T > 32,
    the decode product below); routed ones get few rows.  Step-by-step calls and
    the one-call layer agree bit for bit, both within the bar of the oracle."""
    import dataclasses
    cfg = dataclasses.replace(TINY_SHARED, renormalize=renorm)
    L = Layer(cfg, T=T)
    assert topk_margin_ok(L.x, L.wr, L.bias, cfg.topk)
    o = L.run()
    fused = L.run_fused_call()
    torch.cuda.synchronize()
    r = L.oracle()
    check_route(o, r)
    assert np.all(r["counts"][cfg.experts:] == T)
    check_out(host(o["out"]), r["out"])
    assert np.array_equal(host(fused).view(np.uint16), host(o["out"]).view(np.uint16))


@pytest.mark.parametrize("q", [3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("T", [8, 100, 220, 600])
def test_gemm_act_matches_two_steps(T, q):
    """The activation fused into the gate_up epilogue (decode product at T = 8, mid
    product for experts of 33..64 rows at T = 100, tile product above 64 rows at
    T = 220 (one token tile) and T = 600 (two)) gives exactly the bits of gate_up to
    fp16 h followed by the activation launch."""
    cfg = synth.CONFIGS[0]
    L = Layer(cfg, T=T, qmap=np.full((cfg.weight_experts, 2), q, np.int32))
    o = L.run()
    a = torch.full_like(o["a"], float("nan"))
    apw.gemm_act(ctx(), L.rw.table, L.layer, L.x_d, True, o["perm"], o["offsets"], T, cfg.assign, a)
    torch.cuda.synchronize()
    assert np.array_equal(host(a).view(np.uint16), host(o["a"]).view(np.uint16))


def test_gemm_act_shared_experts_and_rejects_odd_f():
    cfg = TINY_SHARED
    L = Layer(cfg, T=48)
    o = L.run()
    a = torch.empty_like(o["a"])
    apw.gemm_act(ctx(), L.rw.table, L.layer, L.x_d, True, o["perm"], o["offsets"], 48, cfg.assign, a)
    torch.cuda.synchronize()
    assert np.array_equal(host(a).view(np.uint16), host(o["a"]).view(np.uint16))
    # a gate_up block of 96 rows (F = 48, not a multiple of 64) cannot pair gate and up rows
    N, K = 96, 128
    tbl = apw.Table(1, 1)
    P = synth.gen_planes_shape(71, 0, 0, 0, N, K)
    Pd = torch.empty((8, apw.tiled_plane_words(N, K)), dtype=torch.int32, device="cuda")
    apw.tile_planes(ctx(), dev(P), N, K, Pd)
    luts = {b: dev(np.tile(np.arange(1 << b, dtype=np.float16), (N, 1))) for b in range(3, 9)}
    tbl.set_block(0, 0, apw.GATE_UP, N, K, 8, [Pd[p] for p in range(8)], luts)
    tbl.commit(ctx())
    x = torch.zeros((4, K), dtype=torch.float16, device="cuda")
    offs = torch.tensor([0, 4], dtype=torch.int32, device="cuda")
    perm = torch.arange(4, dtype=torch.int32, device="cuda")
    out = torch.zeros((4, N // 2), dtype=torch.float16, device="cuda")
    with pytest.raises(apw.ApmoeError) as ex:
        apw.gemm_act(ctx(), tbl, 0, x, True, perm, offs, 4, 1, out)
    assert ex.value.status == apw.INVALID_ARG
    torch.cuda.synchronize()
    tbl.close()


@pytest.mark.parametrize("T", [1, 5, 13])
def test_layer_tiny_ragged_tokens(T):
    cfg = synth.CONFIGS[0]
    L = Layer(cfg, T=T)
    o = L.run()
    torch.cuda.synchronize()
    r = L.oracle()
    check_route(o, r)
    check_out(host(o["out"]), r["out"])


def test_layer_zero_tokens():
    cfg = synth.CONFIGS[0]
    L = Layer(cfg, T=0)
    out = L.run_fused_call()
    torch.cuda.synchronize()
    assert out.shape == (0, cfg.hidden)


def test_deterministic_and_uniform_q():
    """Two runs give identical bits; a uniform q map (the paper's uniform
    APL-style baseline, Section 4) is the special case all blocks equal."""
    cfg = synth.CONFIGS[0]
    L = Layer(cfg, qmap=np.full((cfg.experts, 2), 4, np.int32))
    a = host(L.run()["out"])
    b = host(L.run()["out"])
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    check_out(a, L.oracle()["out"])


def test_commit_between_launches():
    """Section 3.3: q changes only at safe boundaries.  Launches enqueued before a
    commit use the old q map, launches after it the new one, with no host sync."""
    cfg = synth.CONFIGS[0]
    qa = synth.gen_qmap(cfg)
    qb = 11 - qa  # 3..8 -> 8..3
    L = Layer(cfg, qmap=qa)
    s = torch.cuda.current_stream()
    o1 = L.run(s)
    L.rw.stage_qmap(0, qb)
    L.rw.commit(s)
    o2 = L.run(s)
    L.rw.stage_qmap(0, qa)
    L.rw.commit(s)
    o3 = L.run(s)
    torch.cuda.synchronize()
    check_out(host(o1["out"]), L.oracle(qmap=qa)["out"])
    check_out(host(o2["out"]), L.oracle(qmap=qb)["out"])
    assert np.array_equal(host(o1["out"]).view(np.uint16), host(o3["out"]).view(np.uint16))
    assert not np.array_equal(host(o1["out"]).view(np.uint16), host(o2["out"]).view(np.uint16))
    assert L.rw.table.committed_bits(0, 0, 0) == qa[0, 0]


def test_planes_above_q_are_never_read():
    """Section 3.1: after an offload lowers q, planes p >= q may leave the GPU.
    Poisoned or absent planes above q must not change a single output bit."""
    cfg = synth.CONFIGS[0]
    L = Layer(cfg)
    ref = host(L.run()["out"])
    for (_, e, u), pt in L.rw.planes.items():
        q = int(L.q[e, u])
        if q < 8:
            pt[q:].fill_(-1)
    poisoned = host(L.run()["out"])
    for (_, e, u) in list(L.rw.planes):
        q = int(L.q[e, u])
        for p in range(q, 8):
            L.rw.table.set_plane(0, e, u, p, None, False)
    L.rw.commit()
    absent = host(L.run()["out"])
    torch.cuda.synchronize()
    assert np.array_equal(poisoned.view(np.uint16), ref.view(np.uint16))
    assert np.array_equal(absent.view(np.uint16), ref.view(np.uint16))


def test_gemm_rejects_uncommitted_and_bad_args():
    cfg = synth.CONFIGS[0]
    tbl = apw.Table(1, cfg.experts)
    x = torch.zeros((4, cfg.hidden), dtype=torch.float16, device="cuda")
    out = torch.zeros((8, 2 * cfg.ffn), dtype=torch.float16, device="cuda")
    offs = torch.zeros(cfg.experts + 1, dtype=torch.int32, device="cuda")
    with pytest.raises(apw.ApmoeError) as ex:
        apw.gemm(ctx(), tbl, 0, apw.GATE_UP, x, True, offs, offs, 4, 2, out, apw.F16)
    assert ex.value.status == apw.NOT_RESIDENT
    L = Layer(cfg)
    with pytest.raises(apw.ApmoeError) as ex:
        apw.gemm(ctx(), L.rw.table, 0, apw.GATE_UP, x, True, offs, offs, 4, 2, out, 7)
    assert ex.value.status == apw.UNSUPPORTED
    with pytest.raises(apw.ApmoeError) as ex:
        apw.gemm(ctx(), L.rw.table, 1, apw.GATE_UP, x, True, offs, offs, 4, 2, out, apw.F16)
    assert ex.value.status == apw.INVALID_ARG
    tbl.close()


@pytest.mark.slow
def test_layer_mixtral_decode_full_size():
    """Mixtral-8x7B-shaped decode layer (T = 16), the benchmark's workload and
    launch configuration; oracle on every token."""
    cfg = synth.CONFIGS[1]
    assert topk_margin_ok(synth.gen_x(cfg), synth.gen_router(cfg), None, cfg.topk)
    L = Layer(cfg)
    o = L.run()
    fused = L.run_fused_call()
    torch.cuda.synchronize()
    r = L.oracle()
    check_route(o, r)
    ma, rl = check_out(host(o["out"]), r["out"])
    print(f"mixtral decode T=16: max-abs {ma:.3e} rel-L2 {rl:.3e}", flush=True)
    assert np.array_equal(host(fused).view(np.uint16), host(o["out"]).view(np.uint16))
