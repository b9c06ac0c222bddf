"""Page movement on the GPU (PagedWeight, Section 3.1: planes are pages, dropping the
top planes lowers a block's bitwidth; Section 3.3 / Figure 4: asynchronous page
movement, q lowered before offload and raised after reload, commits at launch
boundaries).

Identity LUTs and small-integer activations make every product an exact integer
matmul with the top-q codes, so each output is checked bit for bit:
- q 8 -> 5 by page-out: the next launch (no host sync) already uses 5-bit codes;
- after done_event the released device planes are overwritten: outputs unchanged;
- the host buffers hold exactly the released plane bytes;
- page-in to 8 from those buffers into fresh device planes: the next launch is
  bit-identical to the original q = 8 output;
- invalid requests are rejected and change nothing.
"""
import numpy as np
import pytest
import torch

import any_precision_weight_amd as apw
import oracle
import synth
from gpu_util import ctx, dev, host

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(2024)


def _identity_luts(N):
    return {b: dev(np.tile(np.arange(1 << b, dtype=np.float16), (N, 1))) for b in range(3, 9)}


def _setup(E, N, K, counts, seed):
    tbl = apw.Table(1, E)
    keep, planes_np, dplanes = [], [], []
    luts = _identity_luts(N)
    keep.append(luts)
    for e in range(E):
        for u in (0, 1):  # each kind owns its planes, so paging one kind leaves the other intact
            P = synth.gen_planes_shape(seed, 0, e, u, N, K)
            Pd = torch.empty((8, apw.tiled_plane_words(N, K)), dtype=torch.int32, device="cuda")
            apw.tile_planes(ctx(), dev(P), N, K, Pd)
            keep.append(Pd)
            if u == 0:
                planes_np.append(P)
                dplanes.append(Pd)
            tbl.set_block(0, e, u, N, K, 8, [Pd[p] for p in range(8)], luts)
    tbl.commit(ctx())
    R = int(sum(counts))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    perm = RNG.permutation(R).astype(np.int32)
    return tbl, keep, planes_np, dplanes, offsets, perm, R


def _run(tbl, x_d, off_d, perm_d, T, N, stream):
    out = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")
    apw.gemm(ctx(), tbl, 0, apw.GATE_UP, x_d, True, perm_d, off_d, T, 1, out, apw.F32, stream)
    return out


def _ref(x, perm, offsets, planes_np, q):
    out = np.zeros((x.shape[0], planes_np[0].shape[1]), np.float64)
    for e, P in enumerate(planes_np):
        rows = perm[offsets[e]:offsets[e + 1]]
        codes = oracle.unpack_codes(P, q).astype(np.int64)
        out[offsets[e]:offsets[e + 1]] = x[rows].astype(np.int64) @ codes.T
    return out


def test_page_out_then_in_round_trip():
    E, N, K = 3, 200, 384
    counts = [7, 40, 300]  # decode and tile products both run
    tbl, keep, planes_np, dplanes, offsets, perm, T = _setup(E, N, K, counts, 61)
    x = RNG.integers(-2, 3, (T, K)).astype(np.float16)
    x_d, off_d, perm_d = dev(x), dev(offsets), dev(perm)
    stream = torch.cuda.current_stream()
    copy_stream = torch.cuda.Stream()
    words = apw.tiled_plane_words(N, K)

    out8 = host(_run(tbl, x_d, off_d, perm_d, T, N, stream))
    assert np.array_equal(out8, _ref(x, perm, offsets, planes_np, 8).astype(np.float32))
    original = [host(Pd).copy() for Pd in dplanes]

    # page-out 8 -> 5 for every gate_up block; the launch right after it uses q = 5
    host_bufs, dones = [], []
    for e in range(E):
        hb = [None] * 5 + [torch.empty(words, dtype=torch.int32).pin_memory() for _ in range(3)]
        done = torch.cuda.Event()
        apw.page_out(ctx(), tbl, 0, e, apw.GATE_UP, 5, hb, stream, copy_stream, done)
        host_bufs.append(hb)
        dones.append(done)
    out5 = host(_run(tbl, x_d, off_d, perm_d, T, N, stream))
    ref5 = _ref(x, perm, offsets, planes_np, 5).astype(np.float32)
    assert np.array_equal(out5, ref5)
    assert all(tbl.committed_bits(0, e, apw.GATE_UP) == 5 for e in range(E))

    # after done the released planes are free: overwrite them; outputs must not move
    for e in range(E):
        dones[e].synchronize()
        for p in range(5, 8):
            assert np.array_equal(host_bufs[e][p].numpy(), original[e][p]), (e, p)
        dplanes[e][5:].fill_(-1)
    out5b = host(_run(tbl, x_d, off_d, perm_d, T, N, stream))
    assert np.array_equal(out5b, out5)

    # page-in 5 -> 8 into fresh device planes; the launch right after it uses q = 8
    fresh = []
    for e in range(E):
        dp = [None] * 5 + [torch.empty(words, dtype=torch.int32, device="cuda") for _ in range(3)]
        fresh.append(dp)
        apw.page_in(ctx(), tbl, 0, e, apw.GATE_UP, 8, host_bufs[e], dp, stream, copy_stream, torch.cuda.Event())
    out8b = host(_run(tbl, x_d, off_d, perm_d, T, N, stream))
    assert np.array_equal(out8b, out8)
    assert all(tbl.committed_bits(0, e, apw.GATE_UP) == 8 for e in range(E))
    torch.cuda.synchronize()
    tbl.close()


def test_page_requests_rejected():
    E, N, K = 1, 64, 128
    tbl, keep, planes_np, dplanes, offsets, perm, T = _setup(E, N, K, [4], 62)
    stream, cs = torch.cuda.current_stream(), torch.cuda.Stream()
    words = apw.tiled_plane_words(N, K)
    hb = [torch.empty(words, dtype=torch.int32).pin_memory() for _ in range(8)]
    with pytest.raises(apw.ApmoeError):  # not lower
        apw.page_out(ctx(), tbl, 0, 0, apw.GATE_UP, 8, hb, stream, cs, torch.cuda.Event())
    with pytest.raises(apw.ApmoeError):  # below 3
        apw.page_out(ctx(), tbl, 0, 0, apw.GATE_UP, 2, hb, stream, cs, torch.cuda.Event())
    with pytest.raises(apw.ApmoeError):  # missing host buffer for plane 6
        apw.page_out(ctx(), tbl, 0, 0, apw.GATE_UP, 5, hb[:6] + [None, hb[7]], stream, cs, torch.cuda.Event())
    assert tbl.committed_bits(0, 0, apw.GATE_UP) == 8  # nothing changed
    with pytest.raises(apw.ApmoeError):  # page-in must raise q
        apw.page_in(ctx(), tbl, 0, 0, apw.GATE_UP, 8, hb, [dplanes[0][p] for p in range(8)], stream, cs,
                    torch.cuda.Event())
    done = torch.cuda.Event()
    apw.page_out(ctx(), tbl, 0, 0, apw.GATE_UP, 4, [None] * 4 + hb[4:], stream, cs, done)
    done.synchronize()
    with pytest.raises(apw.ApmoeError):  # a device plane missing for 4..6
        apw.page_in(ctx(), tbl, 0, 0, apw.GATE_UP, 7, hb, [None] * 8, stream, cs, torch.cuda.Event())
    assert tbl.committed_bits(0, 0, apw.GATE_UP) == 4
    torch.cuda.synchronize()
    tbl.close()
