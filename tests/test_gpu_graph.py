"""The layer captured in a HIP graph and replayed (calls through the C ABI).

apmoe_moe_forward enqueues only kernel launches on the caller's stream, plus an event
fork and join onto the context's side stream when a short tile launch runs beside the
others: no allocation, no memset, no host synchronisation.  So one call can be
captured and replayed.  The fused launches' completion counters are reset by the
kernels themselves, so every replay finds them at zero.

Each case captures one call and replays it six times. Between replays new token rows
are written into the captured input buffer, the output is poisoned, and the program
runs eager work of its own and synchronises. Every replay must give the bits of an
eager call on the same data. The allocation-free entry point, whose audience includes
code under graph capture, is captured the same way.
"""
import numpy as np
import pytest
import torch

import any_precision_weight_amd as apw
import synth
from gpu_util import Layer, ctx, dev, host

pytestmark = pytest.mark.gpu

# (config, tokens): the 16-token Mixtral layer (one-launch route, output accumulation
# in the down product); the tiny layer at 48 tokens (decode and mid products, separate
# combine) and at 300 tokens (tile launches beside the others on the side stream)
CASES = [("mixtral8x7b_decode_t16", 16), ("tiny", 48), ("tiny", 300)]


@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
@pytest.mark.parametrize("name,T", CASES, ids=[f"{n}-T{t}" for n, t in CASES])
def test_layer_graph_replays(name, T, noalloc):
    cfg = synth.config_by_name(name)
    L = Layer(cfg, T=T)
    c = ctx()
    xs = [synth.gen_x(cfg, layer, T) for layer in range(3)]  # three different batches of token rows
    nbytes = apw.moe_workspace(L.rw.table, L.layer, T, cfg.topk, cfg.shared)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    x_d = dev(xs[0])
    out = torch.empty((T, cfg.hidden), dtype=torch.float16, device="cuda")

    def forward(stream):
        if noalloc:
            apw.moe_forward_noalloc(c, L.rw.table, L.layer, x_d, L.wr_d, L.bias_d, T, cfg.topk, cfg.renormalize, out,
                                    stream, n_shared=cfg.shared)
        else:
            apw.moe_forward(c, L.rw.table, L.layer, x_d, L.wr_d, L.bias_d, T, cfg.topk, cfg.renormalize, ws, nbytes,
                            out, stream, n_shared=cfg.shared)

    refs = []
    for x in xs:  # eager references on the default stream
        x_d.copy_(dev(x))
        out.fill_(float("nan"))
        forward(torch.cuda.current_stream())
        torch.cuda.synchronize()
        refs.append(host(out).copy())
    assert not any(np.isnan(r.astype(np.float32)).any() for r in refs)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        forward(s)  # one eager call on the capture stream first
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        forward(s)
    torch.cuda.synchronize()

    other = torch.randn(256, 256, device="cuda")
    for rep in range(6):
        i = rep % len(xs)
        x_d.copy_(dev(xs[i]))
        out.fill_(float("nan"))
        other = torch.tanh(other @ other.T / 256.0)  # the program's own work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(out).view(np.uint16), refs[i].view(np.uint16),
                                      err_msg=f"{name} T={T} replay {rep}")
    del g
