"""fp64 CPU oracle of the any-precision MoE expert layer -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It is a ctypes wrapper over ``oracle.c`` (plain C, fp64, OpenMP),
built with gcc into ``liboracle.so`` next to this file.  It shares no code with
the HIP library.

Source of each function: PagedWeight (arXiv:2607.16184), Section 2.1 (router,
top-K experts, routing weights; Eq. 1 routing mass), Section 3 and the Figure 3
caption (overlaid bit-planes, per-bitwidth centroid LUT), Section 3.1 Eq. 3
(memory of a block at b bits), Section 3.3 (gate_up / activation / down /
output accumulation with a bitwidth per linear-block).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
               "-fPIC", "-shared", "-Wall", "-Wno-unknown-pragmas", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = ctypes.CDLL(_LIB)
        _declare(_lib)
    return _lib


P = ctypes.c_void_p
I64 = ctypes.c_int64
I32 = ctypes.c_int


def _declare(L):
    L.apo_h2d.restype = ctypes.c_double
    L.apo_h2d.argtypes = [ctypes.c_uint16]
    L.apo_d2h.restype = ctypes.c_uint16
    L.apo_d2h.argtypes = [ctypes.c_double]
    L.apo_h2d_array.argtypes = [P, I64, P]
    L.apo_d2h_array.argtypes = [P, I64, P]
    L.apo_unpack_codes.argtypes = [P, I64, I64, I32, P]
    L.apo_pack_planes.argtypes = [P, I64, I64, P]
    L.apo_lut_level.argtypes = [P, I64, I32, P]
    L.apo_block_bytes.restype = I64
    L.apo_block_bytes.argtypes = [I64, I64, I32]
    L.apo_route.argtypes = [P, P, P, I32, I32, I32, I32, I32, I32, P, P, P, P, P, P, P, P, P]
    L.apo_block_gemm.argtypes = [P, P, I32, I64, I64, P, I64, P]
    L.apo_act.argtypes = [P, I64, I64, P]
    L.apo_combine.argtypes = [P, P, P, I32, I32, I64, P]
    L.apo_moe_forward.restype = I32
    L.apo_moe_forward.argtypes = [P, P, P, I32, I32, I32, I32, I32, I32, I32,
                                  P, P, P, P, P, P, P, I32,
                                  P, P, P, P, P, P, P, P, P, P, P, P]
    L.apo_num_threads.restype = I32
    L.apo_set_num_threads.argtypes = [I32]


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return lib().apo_num_threads()


def set_num_threads(n: int) -> None:
    lib().apo_set_num_threads(n)


# -- fp16 ---------------------------------------------------------------------

def h2d(h: np.ndarray) -> np.ndarray:
    h = _c(h, np.float16).view(np.uint16)
    out = np.empty(h.shape, np.float64)
    lib().apo_h2d_array(_p(h), h.size, _p(out))
    return out


def d2h(d: np.ndarray) -> np.ndarray:
    d = _c(d, np.float64)
    out = np.empty(d.shape, np.uint16)
    lib().apo_d2h_array(_p(d), d.size, _p(out))
    return out.view(np.float16)


# -- format -------------------------------------------------------------------

def unpack_codes(planes: np.ndarray, q: int) -> np.ndarray:
    """Codes [N][K] (uint8) of a block at q bits from planes uint32 [8][N][K/32]."""
    planes = _c(planes, np.uint32)
    _, N, W = planes.shape
    K = W * 32
    out = np.empty((N, K), np.uint8)
    lib().apo_unpack_codes(_p(planes), N, K, q, _p(out))
    return out


def pack_planes(codes8: np.ndarray) -> np.ndarray:
    codes8 = _c(codes8, np.uint8)
    N, K = codes8.shape
    assert K % 32 == 0
    out = np.empty((8, N, K // 32), np.uint32)
    lib().apo_pack_planes(_p(codes8), N, K, _p(out))
    return out


def lut_level(parent: np.ndarray, b: int) -> np.ndarray:
    """LUT level b [N][2^b] fp16 from the parent [N][256] (pairwise means)."""
    parent = _c(parent, np.float16).view(np.uint16)
    N = parent.shape[0]
    assert parent.shape[1] == 256 and 3 <= b <= 8
    out = np.empty((N, 1 << b), np.uint16)
    lib().apo_lut_level(_p(parent), N, b, _p(out))
    return out.view(np.float16)


def block_bytes(N: int, K: int, b: int) -> int:
    return int(lib().apo_block_bytes(N, K, b))


# -- route ------------------------------------------------------------------

def route(x, wr, bias, topk: int, renormalize: bool = True, want_absdot: bool = False, n_shared: int = 0):
    """Router of Section 2.1 (see apo_route); with n_shared > 0 the shared experts
    E .. E+n_shared-1 follow the topk routed ones in every token's row, weight 1."""
    x = _c(x, np.float16).view(np.uint16)
    wr = _c(wr, np.float16).view(np.uint16)
    T, H = x.shape
    E = wr.shape[0]
    assert E <= 1024 and 1 <= topk <= E and n_shared >= 0
    b = None if bias is None else _c(bias, np.float32)
    kt, Et = topk + n_shared, E + n_shared
    R = T * kt
    out = dict(
        logits=np.empty((T, E), np.float64),
        ids=np.empty((T, kt), np.int32),
        w64=np.empty((T, kt), np.float64),
        w32=np.empty((T, kt), np.float32),
        counts=np.empty(Et, np.int32),
        offsets=np.empty(Et + 1, np.int32),
        perm=np.empty(R, np.int32),
        inv_perm=np.empty(R, np.int32),
    )
    absdot = np.empty((T, E), np.float64) if want_absdot else None
    lib().apo_route(_p(x), _p(wr), _p(b), T, H, E, topk, n_shared, int(renormalize), _p(out["logits"]),
                    _p(out["ids"]),
                    _p(out["w64"]), _p(out["w32"]), _p(out["counts"]), _p(out["offsets"]), _p(out["perm"]),
                    _p(out["inv_perm"]), _p(absdot))
    if want_absdot:
        out["absdot"] = absdot
    return out


# -- block product ----------------------------------------------------------

def block_gemm(planes, lut_q, q: int, inp: np.ndarray) -> np.ndarray:
    """out[m][n] = sum_c inp[m][c] * LUT_q[n][code_q(n,c)]  (fp64)."""
    planes = _c(planes, np.uint32)
    lut_q = _c(lut_q, np.float16).view(np.uint16)
    _, N, W = planes.shape
    K = W * 32
    assert lut_q.shape == (N, 1 << q)
    inp = _c(inp, np.float64)
    M = inp.shape[0]
    assert inp.shape[1] == K
    out = np.empty((M, N), np.float64)
    lib().apo_block_gemm(_p(planes), _p(lut_q), q, N, K, _p(inp), M, _p(out))
    return out


def act(h: np.ndarray) -> np.ndarray:
    h = _c(h, np.float64)
    M, F2 = h.shape
    F = F2 // 2
    out = np.empty((M, F), np.float64)
    lib().apo_act(_p(h), M, F, _p(out))
    return out


def combine(y: np.ndarray, w: np.ndarray, inv_perm: np.ndarray, topk: int) -> np.ndarray:
    y = _c(y, np.float64)
    w = _c(w, np.float64)
    inv_perm = _c(inv_perm, np.int32)
    R, H = y.shape
    T = inv_perm.size // topk
    out = np.empty((T, H), np.float64)
    lib().apo_combine(_p(y), _p(w), _p(inv_perm), T, topk, H, _p(out))
    return out


# -- whole layer --------------------------------------------------------------

def moe_forward(x, wr, bias, topk: int, planes_gu, lutp_gu, q_gu, planes_dn, lutp_dn, q_dn,
                renormalize: bool = True, eval_tokens=None, intermediates: bool = False, n_shared: int = 0):
    """One MoE layer in fp64.  planes_* / lutp_* are lists over experts of uint32
    [8][N][K/32] planes and fp16 [N][256] parent LUTs; q_* are int arrays.  The
    lists cover the E routed experts (router rows) followed by n_shared shared
    experts."""
    x = _c(x, np.float16).view(np.uint16)
    wr = _c(wr, np.float16).view(np.uint16)
    T, H = x.shape
    Er = wr.shape[0]
    E = Er + n_shared  # experts with weights
    assert len(planes_gu) == E
    F = planes_dn[0].shape[2] * 32
    b = None if bias is None else _c(bias, np.float32)
    keep = []

    def ptr_array(arrs, dtype):
        cs = [_c(a, dtype) for a in arrs]
        keep.extend(cs)
        return (ctypes.c_void_p * E)(*[a.ctypes.data for a in cs])

    pg = ptr_array(planes_gu, np.uint32)
    lg = ptr_array([np.asarray(a, np.float16).view(np.uint16) for a in lutp_gu], np.uint16)
    pd = ptr_array(planes_dn, np.uint32)
    ld = ptr_array([np.asarray(a, np.float16).view(np.uint16) for a in lutp_dn], np.uint16)
    qg = _c(q_gu, np.int32)
    qd = _c(q_dn, np.int32)
    kt = topk + n_shared
    R = T * kt
    ev = None if eval_tokens is None else _c(eval_tokens, np.int32)
    n_eval = T if ev is None else ev.size
    res = dict(
        ids=np.empty((T, kt), np.int32), w64=np.empty((T, kt), np.float64),
        w32=np.empty((T, kt), np.float32), counts=np.empty(E, np.int32),
        offsets=np.empty(E + 1, np.int32), perm=np.empty(R, np.int32), inv_perm=np.empty(R, np.int32),
        logits=np.empty((T, Er), np.float64), out=np.empty((n_eval, H), np.float64),
    )
    h = a = y = None
    if intermediates:
        assert ev is None
        h = np.zeros((R, 2 * F), np.float64)
        a = np.zeros((R, F), np.float64)
        y = np.zeros((R, H), np.float64)
    rc = lib().apo_moe_forward(
        _p(x), _p(wr), _p(b), T, H, F, Er, topk, n_shared, int(renormalize),
        ctypes.cast(pg, P), ctypes.cast(lg, P), _p(qg), ctypes.cast(pd, P), ctypes.cast(ld, P), _p(qd),
        _p(ev), n_eval, _p(res["ids"]), _p(res["w64"]), _p(res["w32"]), _p(res["counts"]),
        _p(res["offsets"]), _p(res["perm"]), _p(res["inv_perm"]), _p(res["logits"]), _p(res["out"]),
        _p(h), _p(a), _p(y))
    if rc != 0:
        raise MemoryError("oracle forward failed to allocate")
    if intermediates:
        res.update(h=h, a=a, y=y)
    return res


def route_stats(ids: np.ndarray, w: np.ndarray, E: int):
    """Eq. 1 (Section 2.1) terms of one batch, in fp64: for every expert e the sum of
    the routing weights r_tk of the selections z_tk = e (numerator), the number of
    those selections, and the sum of all routing weights (denominator).  Plain loops
    over tokens t and choices k, in that order."""
    ids = np.asarray(ids)
    w = np.asarray(w)
    num = np.zeros(E, np.float64)
    cnt = np.zeros(E, np.int64)
    den = 0.0
    T, K = ids.shape
    for t in range(T):
        for k in range(K):
            e = int(ids[t, k])
            r = float(w[t, k])
            num[e] += r
            cnt[e] += 1
            den += r
    return num, cnt, den


def routing_mass(ids: np.ndarray, w: np.ndarray, E: int) -> np.ndarray:
    """Eq. 1 (Section 2.1): m_e = sum_t sum_k r_tk [z_tk = e] / sum_t sum_k r_tk."""
    ids = np.asarray(ids)
    w = np.asarray(w, np.float64)
    m = np.zeros(E, np.float64)
    for e in range(E):
        m[e] = w[ids == e].sum()
    return m / w.sum()
