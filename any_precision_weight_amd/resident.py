"""Device-resident any-precision expert weights and their block table.

``ResidentWeights`` owns, for every linear-block (layer, expert, kind), one
device tensor of the 8 bit-planes (uint32 [8][N][K/32], plane p = code bit 7-p)
and the six LUT levels b = 3..8 (fp16 [N][2^b]).  Level 8 is the parent LUT the
caller supplies; levels 3..7 are built on the device by ``apmoe_lut_build``
(PagedWeight, Figure 3 caption: one LUT of bitwidth-specific centroids per
quantised tensor; read here as one LUT row per output row).

The committed bitwidths live in an :class:`any_precision_weight_amd.Table`;
``commit(qmap)`` stages q for every block and publishes it on the stream
(Section 3.1 / 3.3: q changes only at a launch boundary).
"""
from __future__ import annotations

import numpy as np
import torch

from . import DOWN, GATE_UP, Context, Table, lut_build, tile_planes, tiled_plane_words


class ResidentWeights:
    def __init__(self, ctx: Context, n_layers: int, n_experts: int, device: str = "cuda"):
        self.ctx = ctx
        self.L, self.E = n_layers, n_experts
        self.device = device
        self.table = Table(n_layers, n_experts, library=ctx.L)
        self.planes: dict[tuple[int, int, int], torch.Tensor] = {}
        self.luts: dict[tuple[int, int, int], dict[int, torch.Tensor]] = {}
        self.shape: dict[tuple[int, int, int], tuple[int, int]] = {}

    # -- upload -----------------------------------------------------------------
    def add_block(self, layer: int, expert: int, kind: int, planes: np.ndarray | torch.Tensor,
                  parent_lut: np.ndarray | torch.Tensor, q: int) -> None:
        """planes: canonical uint32 [8][N][K/32] (host or device) -- rearranged on the
        device into the tiled layout the kernels read; parent LUT fp16 [N][256]."""
        if isinstance(planes, np.ndarray):
            canon = torch.from_numpy(np.ascontiguousarray(planes).view(np.int32)).to(self.device)
        else:
            canon = planes.to(self.device).contiguous()
        _, N, W = canon.shape
        K = W * 32
        pt = torch.empty((8, tiled_plane_words(N, K)), dtype=torch.int32, device=self.device)
        tile_planes(self.ctx, canon, N, K, pt)
        del canon
        if isinstance(parent_lut, np.ndarray):
            l8 = torch.from_numpy(np.ascontiguousarray(parent_lut, dtype=np.float16)).to(self.device)
        else:
            l8 = parent_lut.to(self.device).contiguous()
        assert l8.shape == (N, 256)
        levels = {b: torch.empty((N, 1 << b), dtype=torch.float16, device=self.device) for b in range(3, 8)}
        lut_build(self.ctx, l8, N, levels)
        levels[8] = l8
        key = (layer, expert, kind)
        self.planes[key] = pt
        self.luts[key] = levels
        self.shape[key] = (N, K)
        self.table.set_block(layer, expert, kind, N, K, q, [pt[p] for p in range(8)], levels)

    def set_q(self, layer: int, expert: int, kind: int, q: int) -> None:
        self.table.set_bits(layer, expert, kind, q)

    def stage_qmap(self, layer: int, qmap: np.ndarray) -> None:
        """qmap int [E][2] (column 0 gate_up, 1 down)."""
        for e in range(self.E):
            self.table.set_bits(layer, e, GATE_UP, int(qmap[e, 0]))
            self.table.set_bits(layer, e, DOWN, int(qmap[e, 1]))

    def commit(self, stream=None) -> None:
        self.table.commit(self.ctx, stream)

    def mirror_table(self, ctx: Context, stream=None) -> Table:
        """A table of ctx's library build over the same device planes and LUTs, with
        this table's committed bitwidths, committed on `stream`.  The caller closes it
        before these weights."""
        t = Table(self.L, self.E, library=ctx.L)
        for (layer, expert, kind), pt in self.planes.items():
            N, K = self.shape[(layer, expert, kind)]
            q = self.table.committed_bits(layer, expert, kind)
            t.set_block(layer, expert, kind, N, K, q, [pt[p] for p in range(8)], self.luts[(layer, expert, kind)])
        t.commit(ctx, stream)
        return t

    def plane_bytes(self, layer: int, expert: int, kind: int, q: int) -> int:
        N, K = self.shape[(layer, expert, kind)]
        return N * q * K // 8

    def close(self) -> None:
        self.table.close()
        self.planes.clear()
        self.luts.clear()
