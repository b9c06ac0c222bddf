"""apmoe_moe_forward_noalloc: the whole layer with the library's static scratch as
its workspace, for callers that cannot allocate device memory.  Through the C ABI,
two calls in a row on the same device -- the Mixtral-8x7B decode layer at 16 tokens,
then the same layer at 3 tokens -- each give the bits of apmoe_moe_forward with a
caller-owned workspace on the same inputs (the same launches).  A layer whose
workspace exceeds the static array is refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import any_precision_weight_amd as apw
import synth
import synth.gpu
from any_precision_weight_amd.resident import ResidentWeights
from gpu_util import ctx, dev, host

pytestmark = pytest.mark.gpu


def test_noalloc_matches_workspace_entry_point():
    cfg = synth.config_by_name("mixtral8x7b_decode_t16")
    q = synth.gen_qmap(cfg)
    rw = ResidentWeights(ctx(), 1, cfg.weight_experts)
    for e in range(cfg.weight_experts):
        for u in (0, 1):
            rw.add_block(0, e, u, synth.gpu.planes(cfg, 0, e, u), synth.gpu.parent_lut(cfg, 0, e, u), int(q[e, u]))
    rw.commit()
    x, wr = synth.gen_x(cfg), synth.gen_router(cfg)
    wr_d = dev(wr)
    for T in (16, 3):  # the second call is smaller: it must not depend on what the first left behind
        x_d = dev(x[:T])
        nbytes = apw.moe_workspace(rw.table, 0, T, cfg.topk)
        assert nbytes <= apw.NOALLOC_SCRATCH_BYTES
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        ref = torch.full((T, cfg.hidden), float("nan"), dtype=torch.float16, device="cuda")
        got = torch.full((T, cfg.hidden), float("nan"), dtype=torch.float16, device="cuda")
        apw.moe_forward(ctx(), rw.table, 0, x_d, wr_d, None, T, cfg.topk, True, ws, nbytes, ref)
        apw.moe_forward_noalloc(ctx(), rw.table, 0, x_d, wr_d, None, T, cfg.topk, True, got)
        torch.cuda.synchronize()
        r, g = host(ref), host(got)
        assert np.all(np.isfinite(g)), T
        assert np.array_equal(r.view(np.uint16), g.view(np.uint16)), T
        print(f"T={T}: allocation-free layer equals the workspace layer bit for bit", flush=True)
        del ws
    # a batch whose workspace exceeds the static array is refused, nothing enqueued
    big = 4096
    assert apw.moe_workspace(rw.table, 0, big, cfg.topk) > apw.NOALLOC_SCRATCH_BYTES
    xb = torch.zeros((big, cfg.hidden), dtype=torch.float16, device="cuda")
    ob = torch.full((big, cfg.hidden), 7.0, dtype=torch.float16, device="cuda")
    with pytest.raises(apw.ApmoeError) as ei:
        apw.moe_forward_noalloc(ctx(), rw.table, 0, xb, wr_d, None, big, cfg.topk, True, ob)
    assert ei.value.status == apw.INVALID_ARG and "static scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert bool(torch.all(ob == 7.0))
    rw.close()
