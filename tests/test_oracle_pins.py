"""Pins of the fp64 oracle against facts fixed by the paper and by mathematics.

Each test ties one oracle function to something other than itself: a closed
form, an invariant of the format, a library routine (numpy / scipy), or a brute
force written independently here.  Citations are to PagedWeight
(arXiv:2607.16184): Section 2.1 (router top-K, Eq. 1), Section 3 / Figure 3
caption (bit-planes + LUT), Section 3.1 Eq. 3, Section 3.3 (fused layer).
"""
import itertools
import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle
import synth

RNG = np.random.default_rng(12345)


# ---------------------------------------------------------------- fp16 --------

def test_h2d_all_bit_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.h2d(bits.view(np.float16))
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zero kept
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_d2h_matches_numpy_rne():
    # random magnitudes across the whole fp16 range, subnormals, overflow, exact ties
    v = np.concatenate([
        RNG.normal(0, 1, 20000),
        RNG.normal(0, 0.02, 20000),
        RNG.uniform(-70000, 70000, 5000),
        RNG.uniform(-2 ** -13, 2 ** -13, 20000),
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, -65520.0, 2 ** -25, 2 ** -25 * 3, 2 ** -24 * 1.5,
                  np.inf, -np.inf, 1 + 2 ** -11, 1 + 3 * 2 ** -11, 2 ** -14 - 2 ** -25]),
    ])
    # midpoints between consecutive fp16 values (exact ties)
    h = RNG.integers(0, 0x7BFF, 5000).astype(np.uint16).view(np.float16).astype(np.float64)
    h2 = (RNG.integers(0, 0x7BFF, 5000).astype(np.uint16) + 1).astype(np.uint16).view(np.float16)
    v = np.concatenate([v, (h + h2.astype(np.float64)) / 2])
    got = oracle.d2h(v).view(np.uint16)
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- format ------

def _planes_one_bit(N, K, p, n, c):
    P = np.zeros((8, N, K // 32), np.uint32)
    P[p, n, c // 32] = np.uint32(1) << np.uint32(c % 32)
    return P


@pytest.mark.parametrize("q", [3, 4, 5, 6, 7, 8])
def test_one_hot_bit_probe(q):
    """Plane p carries code bit (q-1-p) of a q-bit weight (plane 0 = MSB, Figure 3
    draws b7 first); bit j of word w is column 32w + j.  A single set bit must
    show up in exactly one code, with exactly this value."""
    N, K = 3, 128
    for p in range(8):
        for (n, c) in [(0, 0), (1, 31), (2, 32), (1, 127), (0, 77)]:
            codes = oracle.unpack_codes(_planes_one_bit(N, K, p, n, c), q)
            expect = np.zeros((N, K), np.uint8)
            if p < q:
                expect[n, c] = 1 << (q - 1 - p)
            assert np.array_equal(codes, expect), (q, p, n, c)


def _codes8_numpy(planes):
    """Independent unpack: numpy's little-endian unpackbits, then weights 2^(7-p)."""
    _, N, W = planes.shape
    bits = np.unpackbits(planes.view(np.uint8).reshape(8, N, W * 4), axis=2, bitorder="little")
    return sum(bits[p].astype(np.uint16) << (7 - p) for p in range(8)).astype(np.uint8)


def test_unpack_matches_unpackbits():
    P = synth.gen_planes_shape(7, 0, 0, 0, 33, 256)
    assert np.array_equal(oracle.unpack_codes(P, 8), _codes8_numpy(P))


def test_code_b_is_top_bits_of_parent():
    """A b-bit weight is the subset of the top b planes of the 8-bit parent, so
    code_b = code_8 >> (8 - b) for every b in 3..8."""
    c = synth.CONFIGS[0]
    for kind in (0, 1):
        P = synth.gen_planes(c, 0, 1, kind)
        c8 = _codes8_numpy(P)
        for b in range(3, 9):
            assert np.array_equal(oracle.unpack_codes(P, b), c8 >> (8 - b)), (kind, b)


def test_pack_unpack_round_trip():
    N, K = 5, 128
    cases = [RNG.integers(0, 256, (N, K)).astype(np.uint8), np.zeros((N, K), np.uint8),
             np.full((N, K), 0xFF, np.uint8)]
    for k in (0, 31, 32, K - 1):
        z = np.zeros((N, K), np.uint8)
        z[2, k] = 0x81
        cases.append(z)
    for c8 in cases:
        P = oracle.pack_planes(c8)
        assert np.array_equal(oracle.unpack_codes(P, 8), c8)
        assert np.array_equal(oracle.pack_planes(oracle.unpack_codes(P, 8)), P)
    P = synth.gen_planes_shape(3, 0, 0, 1, 7, 96)
    assert np.array_equal(oracle.pack_planes(oracle.unpack_codes(P, 8)), P)


# ---------------------------------------------------------------- LUT ---------

def test_lut_levels_pairwise_mean_and_order():
    parent = synth.gen_parent_lut_shape(11, 0, 0, 0, 64)
    prev = parent
    for b in range(7, 2, -1):
        lv = oracle.lut_level(parent, b)
        # numpy: exact fp64 mean of two fp16 values, numpy RNE cast back to fp16
        ref = ((prev[:, 0::2].astype(np.float64) + prev[:, 1::2].astype(np.float64)) / 2).astype(np.float16)
        assert np.array_equal(lv.view(np.uint16), ref.view(np.uint16)), b
        # ordering invariants: sorted, and each centroid between its two children
        f = lv.astype(np.float64)
        assert np.all(np.diff(f, axis=1) >= 0)
        assert np.all(f >= prev[:, 0::2].astype(np.float64)) and np.all(f <= prev[:, 1::2].astype(np.float64))
        prev = lv
    assert np.array_equal(oracle.lut_level(parent, 8), parent)


def test_eq3_block_bytes():
    """Eq. 3: M_i^b counts the b bit-planes and the b-bit LUT of the block."""
    for (N, K) in [(1024, 256), (28672, 4096), (4096, 14336)]:
        for b in range(3, 9):
            planes = np.zeros((b, N, K // 32), np.uint32)
            lut = np.zeros((N, 1 << b), np.float16)
            assert oracle.block_bytes(N, K, b) == planes.nbytes + lut.nbytes
            if b > 3:
                delta = oracle.block_bytes(N, K, b) - oracle.block_bytes(N, K, b - 1)
                assert delta == N * K // 8 + N * 2 * (1 << (b - 1))


# ---------------------------------------------------------------- GEMM --------

@pytest.mark.parametrize("q", [3, 5, 8])
def test_identity_lut_is_integer_matmul(q):
    """With LUT_q[n][c] = c and integer activations the product is an exact
    integer matmul x . (code_8 >> (8-q))^T."""
    N, K, M = 40, 256, 6
    P = synth.gen_planes_shape(5, 0, q, 0, N, K)
    lut = np.tile(np.arange(1 << q, dtype=np.float16), (N, 1))
    x = RNG.integers(-2, 3, (M, K))
    got = oracle.block_gemm(P, lut, q, x.astype(np.float64))
    ref = x.astype(np.int64) @ (_codes8_numpy(P).astype(np.int64) >> (8 - q)).T
    assert np.array_equal(got, ref.astype(np.float64))


def test_constant_lut_closed_form():
    N, K, q = 16, 128, 6
    P = synth.gen_planes_shape(6, 0, 0, 0, N, K)
    v = np.float16(0.1234)
    lut = np.full((N, 1 << q), v, np.float16)
    x = RNG.normal(0, 1, (3, K))
    got = oracle.block_gemm(P, lut, q, x)
    ref = np.float64(v) * x.sum(axis=1)
    assert np.allclose(got, ref[:, None], rtol=1e-13, atol=0)


def test_one_hot_activation_reads_one_centroid():
    N, K = 24, 128
    P = synth.gen_planes_shape(8, 0, 0, 0, N, K)
    parent = synth.gen_parent_lut_shape(8, 0, 0, 0, N)
    c8 = _codes8_numpy(P)
    for q in (3, 7, 8):
        lut = oracle.lut_level(parent, q)
        for c in (0, 31, 64, 127):
            x = np.zeros((1, K))
            x[0, c] = 1.0
            got = oracle.block_gemm(P, lut, q, x)[0]
            ref = lut.astype(np.float64)[np.arange(N), c8[:, c] >> (8 - q)]
            assert np.array_equal(got, ref)


# ---------------------------------------------------------------- act, combine --

def test_act_matches_scipy_logistic():
    """Expert activation (Section 3.3): a = SiLU(gate) * up with SiLU(z) = z * sigmoid(z),
    gate = columns [0, F) and up = columns [F, 2F) of h.  Checked against scipy's
    logistic function on random values (a swapped gate/up or a dropped factor fails),
    plus the exact zeros of a zero gate or a zero up."""
    from scipy.special import expit
    F = 7
    h = RNG.normal(0, 3, size=(5, 2 * F))
    h[0, :F] = 0.0
    h[1, F:] = 0.0
    a = oracle.act(h)
    g, u = h[:, :F], h[:, F:]
    assert np.allclose(a, g * expit(g) * u, rtol=1e-14, atol=0)
    assert np.all(a[0] == 0.0) and np.all(a[1] == 0.0)


def test_combine_hand_example():
    """Output accumulation (Section 3.3): out[t] = sum_j w[t][j] * y[inv_perm[t*k + j]].
    Two tokens, top-2, dyadic weights and values, so every sum is exact; the expected
    rows are worked out by hand."""
    y = np.array([[1.0, -2.0, 4.0],
                  [8.0, 0.5, -1.0],
                  [-3.0, 6.0, 2.0],
                  [0.25, 1.0, -8.0]])
    w = np.array([[0.75, 0.25], [0.5, 0.5]])
    inv_perm = np.array([2, 0, 3, 1], np.int32)  # token 0 -> rows 2, 0; token 1 -> rows 3, 1
    out = oracle.combine(y, w, inv_perm, 2)
    # token 0: 0.75 * [-3, 6, 2] + 0.25 * [1, -2, 4]
    # token 1: 0.5 * [0.25, 1, -8] + 0.5 * [8, 0.5, -1]
    assert np.array_equal(out, np.array([[-2.0, 4.0, 2.5], [4.125, 0.75, -4.5]]))


def test_combine_single_choice_is_a_gather():
    """With top-1 and routing weight 1 the accumulation is the row gather y[inv_perm[t]]."""
    y = RNG.normal(0, 1, size=(6, 5))
    inv_perm = np.array([4, 0, 5, 1, 3, 2], np.int32)
    out = oracle.combine(y, np.ones((6, 1)), inv_perm, 1)
    assert np.array_equal(out, y[inv_perm])


def test_combine_equals_layer_accumulation():
    """The combine of the tiny layer's own y, weights and inv_perm gives the layer
    output bit for bit (the same slot order); the layer is pinned by brute force."""
    cfg, x, wr, pg, pd, lg, ld, q = _tiny_layer()
    r = oracle.moe_forward(x, wr, None, cfg.topk, pg, lg, q[:, 0], pd, ld, q[:, 1], intermediates=True)
    out = oracle.combine(r["y"], r["w64"], r["inv_perm"], cfg.topk)
    assert np.array_equal(out, r["out"])


# ---------------------------------------------------------------- route -------

def _route_case(T, H, E, seed, bias=True):
    x = synth.fp16_normal(seed, 1, T * H, 1.0).reshape(T, H)
    wr = synth.fp16_normal(seed, 2, E * H, 0.02).reshape(E, H)
    b = synth.fp16_normal(seed, 3, E, 1.0).astype(np.float32) if bias else None
    return x, wr, b


@pytest.mark.parametrize("renorm", [True, False])
def test_route_brute_force(renorm):
    T, H, E, k = 13, 96, 6, 3
    x, wr, b = _route_case(T, H, E, 21)
    r = oracle.route(x, wr, b, k, renorm)
    z_ref = x.astype(np.float64) @ wr.astype(np.float64).T + b.astype(np.float64)
    assert np.allclose(r["logits"], z_ref, rtol=0, atol=1e-12)
    z = r["logits"]
    for t in range(T):
        # brute force over all k-subsets: the chosen set has the largest logit sum
        best = max(itertools.combinations(range(E), k), key=lambda s: (sum(z[t, list(s)]), [-e for e in s]))
        assert sorted(r["ids"][t]) == sorted(best)
        # within the selection: descending logit order
        assert all(z[t, r["ids"][t][j]] >= z[t, r["ids"][t][j + 1]] for j in range(k - 1))
        sel = z[t, r["ids"][t]]
        w_ref = softmax(sel) if renorm else softmax(z[t])[r["ids"][t]]
        assert np.allclose(r["w64"][t], w_ref, rtol=1e-14, atol=1e-16)
        assert np.array_equal(r["w32"][t], r["w64"][t].astype(np.float32))


def test_route_ties_go_to_lower_expert():
    T, H, E, k = 4, 64, 5, 2
    x, wr, _ = _route_case(T, H, E, 22, bias=False)
    wr[3] = wr[1]  # experts 1 and 3 always tie
    wr[4] = wr[1]
    r = oracle.route(x, wr, None, k)
    z = r["logits"]
    for t in range(T):
        assert z[t, 1] == z[t, 3] == z[t, 4]
        ids = list(r["ids"][t])
        if 3 in ids or 4 in ids:
            assert 1 in ids
        if 4 in ids:
            assert 3 in ids


def test_permutation_invariants():
    T, H, E, k = 37, 64, 7, 2
    x, wr, b = _route_case(T, H, E, 23)
    r = oracle.route(x, wr, b, k)
    R = T * k
    ids = r["ids"].reshape(-1)
    assert r["counts"].sum() == R
    assert np.array_equal(r["counts"], np.bincount(ids, minlength=E))
    assert r["offsets"][0] == 0 and r["offsets"][-1] == R
    assert np.array_equal(np.diff(r["offsets"]), r["counts"])
    assert np.array_equal(np.sort(r["perm"]), np.arange(R))
    assert np.array_equal(r["inv_perm"][r["perm"]], np.arange(R))
    for e in range(E):
        seg = r["perm"][r["offsets"][e]:r["offsets"][e + 1]]
        assert np.all(ids[seg] == e)
        assert np.all(np.diff(seg) > 0)  # stable: ascending assignment (token) order
    assert np.allclose(r["w64"].sum(axis=1), 1.0, rtol=0, atol=1e-15)


def test_routing_mass_eq1():
    """Eq. 1: routing mass sums to one; with renormalised weights every token
    contributes exactly 1/T in total."""
    T, H, E, k = 50, 64, 8, 2
    x, wr, b = _route_case(T, H, E, 24)
    r = oracle.route(x, wr, b, k)
    m = oracle.routing_mass(r["ids"], r["w64"], E)
    assert math.isclose(m.sum(), 1.0, rel_tol=1e-14)
    brute = np.zeros(E)
    for t in range(T):
        for j in range(k):
            brute[r["ids"][t, j]] += r["w64"][t, j] / T
    assert np.allclose(m, brute, rtol=1e-13, atol=1e-16)


def test_route_stats_eq1_terms():
    """Eq. 1 numerator, selection count and denominator on a hand example whose
    weights are dyadic (every sum exact): experts 0, 1, 2 receive 0.75+0.125,
    0.5 and 0.25+0.5+0.875 of a total 3."""
    ids = np.array([[0, 2], [2, 1], [0, 2]], np.int32)
    w = np.array([[0.75, 0.25], [0.5, 0.5], [0.125, 0.875]], np.float32)
    num, cnt, den = oracle.route_stats(ids, w, 4)
    assert num.tolist() == [0.875, 0.5, 1.625, 0.0]
    assert cnt.tolist() == [2, 1, 3, 0]
    assert den == 3.0
    # and the normalised form is the routing mass of Eq. 1
    assert np.array_equal(num / den, oracle.routing_mass(ids, w, 4))


# ---------------------------------------------------------------- layer -------

def _tiny_layer(T=5, H=64, F=64, E=4, k=2, seed=31, qs=None):
    cfg = synth.MoEConfig("pin", tokens=T, hidden=H, ffn=F, experts=E, topk=k, seed=seed)
    x = synth.gen_x(cfg)
    wr = synth.gen_router(cfg) * np.float16(20)  # wider logits: well separated top-k
    pg = [synth.gen_planes(cfg, 0, e, 0) for e in range(E)]
    pd = [synth.gen_planes(cfg, 0, e, 1) for e in range(E)]
    lg = [synth.gen_parent_lut(cfg, 0, e, 0) for e in range(E)]
    ld = [synth.gen_parent_lut(cfg, 0, e, 1) for e in range(E)]
    q = synth.gen_qmap(cfg) if qs is None else np.asarray(qs, np.int32)
    return cfg, x, wr, pg, pd, lg, ld, q


def _brute_layer(x, wr, k, pg, pd, lg, ld, q):
    """Independent pure-Python forward: bit-by-bit codes from Python ints,
    numpy-built LUT levels, Python-float loops."""
    T, H = x.shape
    E = wr.shape[0]
    F = pd[0].shape[2] * 32

    def level(parent, b):
        cur = parent
        for _ in range(8 - b):
            cur = ((cur[:, 0::2].astype(np.float64) + cur[:, 1::2].astype(np.float64)) / 2).astype(np.float16)
        return cur.astype(np.float64)

    def weight_matrix(P, parent, b):
        _, N, W = P.shape
        L = level(parent, b)
        Wm = [[0.0] * (W * 32) for _ in range(N)]
        for n in range(N):
            for c in range(W * 32):
                code = 0
                for p in range(b):
                    bit = (int(P[p, n, c // 32]) >> (c % 32)) & 1
                    code = code * 2 + bit
                Wm[n][c] = float(L[n, code])
        return Wm

    xs = x.astype(np.float64).tolist()
    out = [[0.0] * H for _ in range(T)]
    for t in range(T):
        z = [sum(xs[t][h] * float(wr[e, h]) for h in range(H)) for e in range(E)]
        order = sorted(range(E), key=lambda e: (-z[e], e))[:k]
        zs = [z[e] for e in order]
        den = sum(math.exp(v - zs[0]) for v in zs)
        for j, e in enumerate(order):
            w = math.exp(zs[j] - zs[0]) / den
            Wg = weight_matrix(pg[e], lg[e], int(q[e, 0]))
            Wd = weight_matrix(pd[e], ld[e], int(q[e, 1]))
            hh = [sum(xs[t][c] * Wg[n][c] for c in range(H)) for n in range(2 * F)]
            a = [hh[f] / (1 + math.exp(-hh[f])) * hh[F + f] for f in range(F)]
            for n in range(H):
                out[t][n] += w * sum(a[f] * Wd[n][f] for f in range(F))
    return np.array(out)


def test_tiny_layer_brute_force():
    cfg, x, wr, pg, pd, lg, ld, q = _tiny_layer()
    r = oracle.moe_forward(x, wr, None, cfg.topk, pg, lg, q[:, 0], pd, ld, q[:, 1])
    ref = _brute_layer(x, wr, cfg.topk, pg, pd, lg, ld, q)
    assert np.allclose(r["out"], ref, rtol=1e-10, atol=1e-13)


def test_eval_token_subset_matches_full():
    cfg, x, wr, pg, pd, lg, ld, q = _tiny_layer(T=9)
    full = oracle.moe_forward(x, wr, None, cfg.topk, pg, lg, q[:, 0], pd, ld, q[:, 1])
    ev = np.array([7, 0, 3], np.int32)
    sub = oracle.moe_forward(x, wr, None, cfg.topk, pg, lg, q[:, 0], pd, ld, q[:, 1], eval_tokens=ev)
    assert np.array_equal(sub["out"], full["out"][ev])


def test_single_expert_q8_is_dense_ffn():
    """E = 1, k = 1, q = 8 reduces to a dense SwiGLU FFN on the dequantised
    matrices (routing weight exactly 1)."""
    cfg, x, wr, pg, pd, lg, ld, _ = _tiny_layer(T=6, E=1, k=1)
    q = np.array([[8, 8]], np.int32)
    r = oracle.moe_forward(x, wr, None, 1, pg, lg, q[:, 0], pd, ld, q[:, 1])
    assert np.all(r["w64"] == 1.0)
    Wg = lg[0].astype(np.float64)[np.arange(2 * cfg.ffn)[:, None], _codes8_numpy(pg[0])]
    Wd = ld[0].astype(np.float64)[np.arange(cfg.hidden)[:, None], _codes8_numpy(pd[0])]
    h = x.astype(np.float64) @ Wg.T
    g, u = h[:, :cfg.ffn], h[:, cfg.ffn:]
    ref = (g / (1 + np.exp(-g)) * u) @ Wd.T
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-15)


def test_uniform_q_is_apl_style_baseline():
    """A uniform bitwidth (the paper's uniform APL-style baseline, Section 4) is
    the special case where every block takes the same q: the layer must equal
    the mixed-q layer evaluated with that constant map."""
    cfg, x, wr, pg, pd, lg, ld, _ = _tiny_layer(T=4)
    for b in (3, 6):
        q = np.full((cfg.experts, 2), b, np.int32)
        r = oracle.moe_forward(x, wr, None, cfg.topk, pg, lg, q[:, 0], pd, ld, q[:, 1])
        ref = _brute_layer(x, wr, cfg.topk, pg, pd, lg, ld, q)
        assert np.allclose(r["out"], ref, rtol=1e-10, atol=1e-13)


def test_shared_experts_add_their_ffn():
    """Shared experts (the "+4" / "+1" experts of Table 1): every token visits
    them with weight 1 after its routed top-k, so the layer equals the routed-only
    layer plus each shared expert's FFN of x, computed here from the block product
    and the activation directly."""
    T, H, F, E, k, S = 6, 64, 64, 4, 2, 2
    cfg, x, wr, pg, pd, lg, ld, q = _tiny_layer(T=T, H=H, F=F, E=E + S, k=k, seed=37)
    wr_routed = wr[:E]
    with_shared = oracle.moe_forward(x, wr_routed, None, k, pg, lg, q[:, 0], pd, ld, q[:, 1], n_shared=S)
    routed = oracle.moe_forward(x, wr_routed, None, k, pg[:E], lg[:E], q[:E, 0], pd[:E], ld[:E], q[:E, 1])
    ref = routed["out"].copy()
    xin = x.astype(np.float64)
    for s_ in range(S):
        e = E + s_
        h = oracle.block_gemm(pg[e], oracle.lut_level(lg[e], int(q[e, 0])), int(q[e, 0]), xin)
        a = oracle.act(h)
        ref += oracle.block_gemm(pd[e], oracle.lut_level(ld[e], int(q[e, 1])), int(q[e, 1]), a)
    assert np.allclose(with_shared["out"], ref, rtol=1e-12, atol=1e-12)
    # routing: the shared experts follow the routed ones in every row, weight 1
    assert np.array_equal(with_shared["ids"][:, :k], routed["ids"])
    assert np.all(with_shared["ids"][:, k:] == np.arange(E, E + S))
    assert np.all(with_shared["w64"][:, k:] == 1.0)
    assert with_shared["counts"][E:].tolist() == [T] * S

