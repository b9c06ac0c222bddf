"""Counter-based generators and the workload table.

All arithmetic here is random-number plumbing: SplitMix64 outputs, uniform and
approximately normal variates, RNE rounding to fp16 (numpy's float64 -> float16
cast), sorting of the parent LUT rows, and the Zipf prior used as a router bias.
synth/synth_gpu.hip implements the same definitions for bulk generation on the
device; both produce identical bits.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

GOLDEN = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_MASK = (1 << 64) - 1


def _mix_int(z: int) -> int:
    """SplitMix64 output function on a Python int (mod 2^64)."""
    z &= _MASK
    z = ((z ^ (z >> 30)) * _M1) & _MASK
    z = ((z ^ (z >> 27)) * _M2) & _MASK
    return z ^ (z >> 31)


def _mix_np(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(_M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(_M2)
        return z ^ (z >> np.uint64(31))


def stream_key(seed: int, tid: int) -> int:
    """Key of the stream (seed, tensor id): mix(mix(seed + GOLDEN) ^ tid)."""
    return _mix_int(_mix_int(seed + GOLDEN) ^ (tid & _MASK))


def u64(seed: int, tid: int, idx) -> np.ndarray:
    """Element ``idx`` of stream (seed, tid): the (idx+1)-th SplitMix64 output
    of a generator whose state starts at ``stream_key(seed, tid)``."""
    key = np.uint64(stream_key(seed, tid))
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = key + (idx + np.uint64(1)) * np.uint64(GOLDEN)
    return _mix_np(z)


def uniform01(u: np.ndarray) -> np.ndarray:
    """Map uint64 to a double in the open interval (0, 1): ((u>>11)+0.5)*2^-53."""
    return ((u >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def normal(seed: int, tid: int, idx) -> np.ndarray:
    """Approximately standard normal variate number ``idx``: the Irwin-Hall sum of
    twelve 16-bit uniforms minus 6 (stream elements 3*idx .. 3*idx+2, each split into
    four 16-bit chunks).  Mean 0, variance 1 - 2^-32, support [-6, 6], resolution
    2^-16.  The sum is exact integer arithmetic and the scaling by 2^-16 is exact, so
    a device implementation of the same definition reproduces the bits."""
    idx = np.asarray(idx, dtype=np.uint64)
    acc = np.zeros(idx.shape, dtype=np.int64)
    base = idx * np.uint64(3)
    m16 = np.uint64(0xFFFF)
    for i in range(3):
        u = u64(seed, tid, base + np.uint64(i))
        for sh in (0, 16, 32, 48):
            acc += ((u >> np.uint64(sh)) & m16).astype(np.int64)
    return (acc - 393210).astype(np.float64) * (2.0 ** -16)  # 393210 = 12 * 65535 / 2


def fp16_normal(seed: int, tid: int, n: int, std: float, offset: int = 0) -> np.ndarray:
    """``n`` consecutive normal(0, std^2) values: fp64 product normal*std (one
    correctly rounded multiply), then rounded to fp16 (round to nearest even)."""
    out = np.empty(n, dtype=np.float16)
    step = 1 << 22
    for s in range(0, n, step):
        e = min(n, s + step)
        v = normal(seed, tid, np.arange(offset + s, offset + e, dtype=np.uint64)) * std
        out[s:e] = v.astype(np.float16)
    return out


class TID:
    """Tensor kinds of the stream table (combined with layer/expert/kind)."""
    X = 1
    ROUTER = 2
    ZIPF_PERM = 3
    PLANES = 4
    LUT = 5
    QMAP = 6
    AUX = 7  # auxiliary test tensors (h, y, ... fed to single-stage tests)


def tensor_id(kind: int, layer: int = 0, expert: int = 0, sub: int = 0) -> int:
    return (((kind * 4096 + layer) * 4096 + expert) * 16 + sub) & _MASK


@dataclass(frozen=True)
class MoEConfig:
    """One synthetic workload.

    qmode: "u38"  per-block q uniform over {3..8}
           "hot"  hot experts (Zipf ranks 1 and 2) uniform over {6,7,8}, others {3,4,5}
           "maps" two maps per block: A uniform over {4..8}, B uniform over {3,4,5}
    """
    name: str
    tokens: int
    hidden: int
    ffn: int
    experts: int
    topk: int
    seed: int
    layers: int = 1
    zipf_s: float | None = None
    qmode: str = "u38"
    renormalize: bool = True
    shared: int = 0
    note: str = field(default="", compare=False)

    @property
    def assign(self) -> int:
        """Expert rows per token: the topk routed ones, then every shared expert."""
        return self.topk + self.shared

    @property
    def weight_experts(self) -> int:
        """Experts holding weights: the `experts` routed ones, then the shared ones."""
        return self.experts + self.shared

    @property
    def rows(self) -> int:
        return self.tokens * self.assign

    def block_shape(self, kind: int) -> tuple[int, int]:
        """(N, K) of a linear-block: gate_up is [2F x H], down is [H x F]."""
        return (2 * self.ffn, self.hidden) if kind == 0 else (self.hidden, self.ffn)


CONFIGS = [
    MoEConfig("tiny", tokens=8, hidden=256, ffn=512, experts=4, topk=2, seed=0,
              note="tiny MoE layer, CPU-seconds scale"),
    MoEConfig("mixtral8x7b_decode_t16", tokens=16, hidden=4096, ffn=14336, experts=8, topk=2,
              seed=1, note="Mixtral-8x7B-shaped single MoE layer, decode batch 16"),
    MoEConfig("mixtral8x22b_decode_t256_zipf", tokens=256, hidden=6144, ffn=16384, experts=8,
              topk=2, seed=2, zipf_s=1.2, qmode="hot",
              note="Mixtral-8x22B-shaped single MoE layer, decode batch 256, Zipf(1.2) router bias"),
    MoEConfig("mixtral8x7b_prefill_t4096_zipf", tokens=4096, hidden=4096, ffn=14336, experts=8,
              topk=2, seed=3, zipf_s=0.8,
              note="Mixtral-8x7B-shaped MoE layer, prefill 4096 tokens, Zipf(0.8) router bias"),
    MoEConfig("mixtral8x7b_32layer_decode_t32", tokens=32, hidden=4096, ffn=14336, experts=8,
              topk=2, seed=4, layers=32, qmode="maps",
              note="32 layers x 8 experts resident, decode batch 32, q map switch"),
    # Many small experts plus shared experts.  The expert counts and top-k are the
    # two fine-grained models the paper evaluates; their hidden and expert FFN sizes
    # are not given there, so the ones below are chosen (fine-grained scale).
    MoEConfig("qwen_60r4s_top4_decode_t64", tokens=64, hidden=2048, ffn=1408, experts=60, topk=4,
              seed=5, shared=4, renormalize=False,
              note="60 routed + 4 shared experts, top-4, decode batch 64; H=2048, F=1408 chosen"),
    MoEConfig("gemma_128r1s_top8_decode_t64", tokens=64, hidden=2048, ffn=768, experts=128, topk=8,
              seed=6, shared=1,
              note="128 routed + 1 shared expert, top-8, decode batch 64; H=2048, F=768 chosen"),
    MoEConfig("qwen_60r4s_top4_prefill_t2048", tokens=2048, hidden=2048, ffn=1408, experts=60, topk=4,
              seed=7, shared=4, renormalize=False,
              note="60 routed + 4 shared experts, top-4, prefill 2048 tokens; H=2048, F=1408 chosen"),
]


def config_by_name(name: str) -> MoEConfig:
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)


# ----------------------------------------------------------------------------
# tensors
# ----------------------------------------------------------------------------

def gen_x(cfg: MoEConfig, layer: int = 0, tokens: int | None = None) -> np.ndarray:
    """Activations [T][H] fp16, N(0,1).  Each layer has its own input."""
    T = cfg.tokens if tokens is None else tokens
    return fp16_normal(cfg.seed, tensor_id(TID.X, layer), T * cfg.hidden, 1.0).reshape(T, cfg.hidden)


def gen_router(cfg: MoEConfig, layer: int = 0) -> np.ndarray:
    """Router weights [E][H] fp16, N(0, 0.02^2)."""
    return fp16_normal(cfg.seed, tensor_id(TID.ROUTER, layer), cfg.experts * cfg.hidden,
                       0.02).reshape(cfg.experts, cfg.hidden)


def zipf_probs(E: int, s: float) -> np.ndarray:
    r = np.arange(1, E + 1, dtype=np.float64)
    p = r ** (-s)
    return p / p.sum()


def zipf_ranks(cfg: MoEConfig, layer: int = 0) -> np.ndarray:
    """rank[e] in 1..E: a seeded permutation assigning Zipf ranks to experts."""
    keys = u64(cfg.seed, tensor_id(TID.ZIPF_PERM, layer), np.arange(cfg.experts))
    order = np.argsort(keys, kind="stable")
    rank = np.empty(cfg.experts, dtype=np.int64)
    rank[order] = np.arange(1, cfg.experts + 1)
    return rank


def gen_bias(cfg: MoEConfig, layer: int = 0) -> np.ndarray | None:
    """Router bias [E] fp32: ln of the Zipf(s) prior of each expert's rank, or None."""
    if cfg.zipf_s is None:
        return None
    p = zipf_probs(cfg.experts, cfg.zipf_s)
    rank = zipf_ranks(cfg, layer)
    return np.log(p[rank - 1]).astype(np.float32)


def hot_experts(cfg: MoEConfig, layer: int = 0) -> list[int]:
    """Experts holding Zipf ranks 1 and 2 (the two largest prior routing masses)."""
    rank = zipf_ranks(cfg, layer)
    return sorted(int(e) for e in np.nonzero(rank <= 2)[0])


def gen_planes(cfg: MoEConfig, layer: int, expert: int, kind: int) -> np.ndarray:
    """Bit-plane words uint32 [8][N][K/32] of one linear-block.

    Uniform random words: every parent 8-bit code of every weight is equally
    likely and independent, which is the same distribution as packing i.i.d.
    uniform parent codes.  Word j uses half j%2 (low first) of stream element j//2.
    """
    N, K = cfg.block_shape(kind)
    return gen_planes_shape(cfg.seed, layer, expert, kind, N, K)


def gen_planes_shape(seed: int, layer: int, expert: int, kind: int, N: int, K: int) -> np.ndarray:
    assert K % 32 == 0
    nwords = 8 * N * (K // 32)
    tid = tensor_id(TID.PLANES, layer, expert, kind)
    out = np.empty(nwords // 2, dtype=np.uint64)
    step = 1 << 24
    for s in range(0, nwords // 2, step):
        e = min(nwords // 2, s + step)
        out[s:e] = u64(seed, tid, np.arange(s, e, dtype=np.uint64))
    return out.view(np.uint32).reshape(8, N, K // 32)


def gen_parent_lut(cfg: MoEConfig, layer: int, expert: int, kind: int) -> np.ndarray:
    """Parent (8-bit) LUT [N][256] fp16: per row, 256 N(0, 0.02^2) values rounded
    to fp16 (signed zeros made +0) and sorted ascending."""
    N, _ = cfg.block_shape(kind)
    return gen_parent_lut_shape(cfg.seed, layer, expert, kind, N)


def gen_parent_lut_shape(seed: int, layer: int, expert: int, kind: int, N: int) -> np.ndarray:
    tid = tensor_id(TID.LUT, layer, expert, kind)
    v = fp16_normal(seed, tid, N * 256, 0.02).reshape(N, 256)
    v[v == 0] = np.float16(0.0)
    return np.sort(v, axis=1)


def gen_qmap(cfg: MoEConfig, layer: int = 0, which: int = 0) -> np.ndarray:
    """Committed bitwidths q[e][kind] (kind 0 gate_up, 1 down) of one layer, for
    the routed experts followed by the shared ones.

    which selects map A (0) or map B (1) for the "maps" workload.
    """
    E = cfg.weight_experts
    u = u64(cfg.seed, tensor_id(TID.QMAP, layer, 0, which), np.arange(2 * E)).reshape(E, 2)
    if cfg.qmode == "u38":
        return (3 + (u % np.uint64(6))).astype(np.int32)
    if cfg.qmode == "hot":
        hot = set(hot_experts(cfg, layer))
        q = np.empty((E, 2), dtype=np.int32)
        for e in range(E):
            base = 6 if e in hot else 3
            q[e] = base + (u[e] % np.uint64(3)).astype(np.int32)
        return q
    if cfg.qmode == "maps":
        if which == 0:
            return (4 + (u % np.uint64(5))).astype(np.int32)
        return (3 + (u % np.uint64(3))).astype(np.int32)
    raise ValueError(cfg.qmode)


def gen_aux_fp16(seed: int, sub: int, n: int, std: float = 1.0) -> np.ndarray:
    """Auxiliary fp16 N(0, std^2) vector for single-stage tests."""
    return fp16_normal(seed, tensor_id(TID.AUX, 0, 0, sub), n, std)


def gen_aux_u64(seed: int, sub: int, n: int) -> np.ndarray:
    return u64(seed, tensor_id(TID.AUX, 1, 0, sub), np.arange(n))
