"""Python binding of libapmoe (ctypes), the any-precision MoE expert layer for
MI355X (gfx950).

Argument marshalling only: every step runs in the HIP kernels of
``libapmoe.so``.  Tensors are torch device tensors (PyTorch provides device
memory and streams); they are passed to the C ABI as raw pointers.  There is
no fallback: if the library is missing, importing the functions raises.

Function names and argument order follow ``include/apmoe.h``.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libapmoe.so")
# the same library built with every counted vector-memory wait drained to zero
SAFE_LIB_PATH = os.path.join(_HERE, "libapmoe_safe.so")

OK, INVALID_ARG, UNSUPPORTED, NOT_RESIDENT, HIP_ERROR, OUT_OF_MEMORY = range(6)
GATE_UP, DOWN = 0, 1
F16, F32 = 0, 1
MIN_BITS, MAX_BITS, PLANES = 3, 8, 8

EXPORTED = [
    "apmoe_status_string", "apmoe_last_error", "apmoe_version", "apmoe_create", "apmoe_destroy", "apmoe_ctx_faults",
    "apmoe_block_bytes", "apmoe_table_create", "apmoe_table_destroy", "apmoe_table_set_block",
    "apmoe_table_set_bits", "apmoe_table_set_plane", "apmoe_table_validate", "apmoe_table_committed_bits",
    "apmoe_table_commit", "apmoe_lut_build", "apmoe_tiled_plane_words", "apmoe_tile_planes", "apmoe_pack_planes", "apmoe_route", "apmoe_route_workspace", "apmoe_route_stats", "apmoe_gemm",
    "apmoe_gemm_act", "apmoe_act",
    "apmoe_combine", "apmoe_moe_workspace", "apmoe_moe_forward", "apmoe_page_out", "apmoe_page_in",
    "apmoe_moe_forward_noalloc",
]


class ApmoeError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        self.status = status
        super().__init__(f"{fn}: status {status} ({_status_text(status)}): {detail}")


class BlockDesc(ctypes.Structure):
    _fields_ = [
        ("n", ctypes.c_int32), ("k", ctypes.c_int32), ("q", ctypes.c_int32), ("d", ctypes.c_int32),
        ("resident_mask", ctypes.c_uint32),
        ("plane", ctypes.c_void_p * PLANES),
        ("lut", ctypes.c_void_p * (MAX_BITS + 1)),
    ]


_lib = None


def _status_text(s: int) -> str:
    try:
        return lib().apmoe_status_string(s).decode()
    except Exception:  # pragma: no cover - library missing
        return "?"


_loaded: dict[str, ctypes.CDLL] = {}


def load_library(path: str) -> ctypes.CDLL:
    """Load a libapmoe build (once per path; raises if it has not been built).
    Contexts and tables remember the library that made them, so two builds can be
    used side by side in one process."""
    if path not in _loaded:
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with `python -m any_precision_weight_amd.build`")
        L = ctypes.CDLL(path)
        _declare(L)
        _loaded[path] = L
    return _loaded[path]


def lib() -> ctypes.CDLL:
    """The default build, libapmoe.so."""
    global _lib
    if _lib is None:
        _lib = load_library(LIB_PATH)
    return _lib


def _declare(L):
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    S = ctypes.c_int32
    sig = {
        "apmoe_status_string": (ctypes.c_char_p, [S]),
        "apmoe_last_error": (ctypes.c_char_p, []),
        "apmoe_version": (I32, []),
        "apmoe_create": (S, [ctypes.POINTER(P), ctypes.c_int]),
        "apmoe_destroy": (S, [P]),
        "apmoe_ctx_faults": (S, [P, ctypes.POINTER(I32)]),
        "apmoe_block_bytes": (I64, [I32, I32, I32]),
        "apmoe_table_create": (S, [I32, I32, ctypes.POINTER(P)]),
        "apmoe_table_destroy": (S, [P]),
        "apmoe_table_set_block": (S, [P, I32, I32, I32, ctypes.POINTER(BlockDesc)]),
        "apmoe_table_set_bits": (S, [P, I32, I32, I32, I32]),
        "apmoe_table_set_plane": (S, [P, I32, I32, I32, I32, P, I32]),
        "apmoe_table_validate": (S, [P]),
        "apmoe_table_committed_bits": (S, [P, I32, I32, I32, ctypes.POINTER(I32)]),
        "apmoe_table_commit": (S, [P, P, P]),
        "apmoe_lut_build": (S, [P, P, I32, P, P]),
        "apmoe_tiled_plane_words": (I64, [I32, I32]),
        "apmoe_tile_planes": (S, [P, P, I32, I32, P, P]),
        "apmoe_pack_planes": (S, [P, P, I32, I32, P, P]),
        "apmoe_route": (S, [P, P, P, P, I32, I32, I32, I32, I32, I32, P, P, P, P, P, P, P]),
        "apmoe_route_workspace": (S, [P, I32, I32, I32, I32, ctypes.POINTER(SZ)]),
        "apmoe_route_stats": (S, [P, P, P, P, I32, I32, I32, P, P, P, P]),
        "apmoe_gemm": (S, [P, P, I32, I32, P, I32, P, P, I32, I32, P, I32, P]),
        "apmoe_gemm_act": (S, [P, P, I32, P, I32, P, P, I32, I32, P, P]),
        "apmoe_act": (S, [P, P, I32, I32, P, P]),
        "apmoe_combine": (S, [P, P, I32, P, P, I32, I32, I32, P, P]),
        "apmoe_moe_workspace": (S, [P, I32, I32, I32, I32, ctypes.POINTER(SZ)]),
        "apmoe_moe_forward": (S, [P, P, I32, P, P, P, I32, I32, I32, I32, P, SZ, P, P]),
        "apmoe_moe_forward_noalloc": (S, [P, P, I32, P, P, P, I32, I32, I32, I32, P, P]),
        "apmoe_page_out": (S, [P, P, I32, I32, I32, I32, ctypes.POINTER(P), P, P, P]),
        "apmoe_page_in": (S, [P, P, I32, I32, I32, I32, ctypes.POINTER(P), ctypes.POINTER(P), P, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args


def _check(status: int, fn: str, L: ctypes.CDLL | None = None) -> None:
    if status != OK:
        raise ApmoeError(status, fn, (L or lib()).apmoe_last_error().decode())


def ptr(t) -> int | None:
    """Raw pointer of a torch tensor / int / None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def stream_handle(stream=None) -> int | None:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream or None


# --------------------------------------------------------------------------- API

def version() -> int:
    return lib().apmoe_version()


def block_bytes(n: int, k: int, b: int) -> int:
    return int(lib().apmoe_block_bytes(n, k, b))


class Context:
    """apmoe_create / apmoe_destroy.  A context owns a side stream and the completion
    counters of the fused launches: calls on one context that may run at the same time
    must be ordered by the caller (or use a context each).  APMOE_UNFUSED=1 in the
    environment when the context is created gives one that runs every layer step in
    its own launches; APMOE_LAYER_KERNEL=1 one that runs a small batch's gate_up and
    down in one launch (the one-launch decode layer) instead of two."""

    def __init__(self, device: int = 0, library: ctypes.CDLL | None = None):
        self.L = lib() if library is None else library
        h = ctypes.c_void_p()
        _check(self.L.apmoe_create(ctypes.byref(h), device), "apmoe_create", self.L)
        self.handle = h.value
        self.device = device

    def faults(self) -> int:
        """apmoe_ctx_faults: the context's sticky fault flags (0 = none; synchronises)."""
        v = ctypes.c_int32()
        _check(self.L.apmoe_ctx_faults(self.handle, ctypes.byref(v)), "apmoe_ctx_faults", self.L)
        return v.value

    def close(self):
        if self.handle:
            self.L.apmoe_destroy(self.handle)
            self.handle = None

    def __del__(self):  # pragma: no cover
        try:
            self.close()
        except Exception:
            pass


class Table:
    """apmoe_table_* : staging, validation and stream-ordered commit."""

    def __init__(self, n_layers: int, n_experts: int, library: ctypes.CDLL | None = None):
        self.L = lib() if library is None else library
        h = ctypes.c_void_p()
        _check(self.L.apmoe_table_create(n_layers, n_experts, ctypes.byref(h)), "apmoe_table_create", self.L)
        self.handle = h.value
        self.n_layers, self.n_experts = n_layers, n_experts

    def set_block(self, layer: int, expert: int, kind: int, n: int, k: int, q: int, planes, luts,
                  d: int | None = None, resident_mask: int | None = None) -> None:
        """planes: 8 device pointers/tensors (None = not resident);
        luts: dict {b: tensor/pointer} for b in 3..8."""
        desc = BlockDesc()
        desc.n, desc.k, desc.q = n, k, q
        desc.d = q if d is None else d
        mask = 0
        for p in range(PLANES):
            pp = ptr(planes[p]) if p < len(planes) else None
            desc.plane[p] = pp
            if pp:
                mask |= 1 << p
        desc.resident_mask = mask if resident_mask is None else resident_mask
        for b in range(MAX_BITS + 1):
            desc.lut[b] = ptr(luts.get(b)) if b in luts else None
        _check(self.L.apmoe_table_set_block(self.handle, layer, expert, kind, ctypes.byref(desc)),
               "apmoe_table_set_block", self.L)

    def set_bits(self, layer: int, expert: int, kind: int, q: int) -> None:
        _check(self.L.apmoe_table_set_bits(self.handle, layer, expert, kind, q), "apmoe_table_set_bits", self.L)

    def set_plane(self, layer: int, expert: int, kind: int, p: int, plane, resident: bool) -> None:
        _check(self.L.apmoe_table_set_plane(self.handle, layer, expert, kind, p, ptr(plane), int(resident)),
               "apmoe_table_set_plane", self.L)

    def validate(self) -> int:
        """Status apmoe_table_commit would return (no exception)."""
        return int(self.L.apmoe_table_validate(self.handle))

    def committed_bits(self, layer: int, expert: int, kind: int) -> int:
        q = ctypes.c_int32()
        _check(self.L.apmoe_table_committed_bits(self.handle, layer, expert, kind, ctypes.byref(q)),
               "apmoe_table_committed_bits", self.L)
        return q.value

    def commit(self, ctx: Context, stream=None) -> None:
        _check(self.L.apmoe_table_commit(ctx.handle, self.handle, stream_handle(stream)), "apmoe_table_commit", self.L)

    def close(self):
        if self.handle:
            self.L.apmoe_table_destroy(self.handle)
            self.handle = None

    def __del__(self):  # pragma: no cover
        try:
            self.close()
        except Exception:
            pass


def lut_build(ctx: Context, parent, n: int, levels: dict, stream=None) -> None:
    arr = (ctypes.c_void_p * (MAX_BITS + 1))(*[ptr(levels.get(b)) for b in range(MAX_BITS + 1)])
    _check(ctx.L.apmoe_lut_build(ctx.handle, ptr(parent), n, ctypes.cast(arr, ctypes.c_void_p),
                                 stream_handle(stream)), "apmoe_lut_build", ctx.L)


def tiled_plane_words(n: int, k: int) -> int:
    return int(lib().apmoe_tiled_plane_words(n, k))


def tile_planes(ctx: Context, canonical, n: int, k: int, tiled, stream=None) -> None:
    _check(ctx.L.apmoe_tile_planes(ctx.handle, ptr(canonical), n, k, ptr(tiled), stream_handle(stream)),
           "apmoe_tile_planes", ctx.L)


def pack_planes(ctx: Context, codes, n: int, k: int, planes, stream=None) -> None:
    _check(ctx.L.apmoe_pack_planes(ctx.handle, ptr(codes), n, k, ptr(planes), stream_handle(stream)),
           "apmoe_pack_planes", ctx.L)


def route(ctx: Context, x, w_router, bias, T: int, H: int, E: int, topk: int, renormalize: bool, topk_ids,
          topk_w, counts, offsets, perm, inv_perm, stream=None, n_shared: int = 0) -> None:
    """Top-k routing over E routed experts; with n_shared > 0 each token's row of
    topk_ids / topk_w (stride topk + n_shared) ends with the shared experts
    E .. E + n_shared - 1 at weight 1, and counts / offsets cover E + n_shared experts."""
    _check(ctx.L.apmoe_route(ctx.handle, ptr(x), ptr(w_router), ptr(bias), T, H, E, topk, n_shared, int(renormalize),
                             ptr(topk_ids), ptr(topk_w), ptr(counts), ptr(offsets), ptr(perm), ptr(inv_perm),
                             stream_handle(stream)), "apmoe_route", ctx.L)


def route_workspace(ctx: Context, T: int, E: int, topk: int, n_shared: int = 0) -> int:
    n = ctypes.c_size_t()
    _check(ctx.L.apmoe_route_workspace(ctx.handle, T, E, topk, n_shared, ctypes.byref(n)), "apmoe_route_workspace",
           ctx.L)
    return n.value


def route_stats(ctx: Context, topk_w, perm, offsets, T: int, topk: int, E: int, mass, total, selections,
                stream=None) -> None:
    """Add one routed batch to the routing-statistics accumulators (Eq. 1):
    mass[E] fp64, total[1] fp64, selections[E] int64, all device memory."""
    _check(ctx.L.apmoe_route_stats(ctx.handle, ptr(topk_w), ptr(perm), ptr(offsets), T, topk, E, ptr(mass),
                                   ptr(total), ptr(selections), stream_handle(stream)), "apmoe_route_stats", ctx.L)


def gemm(ctx: Context, table: Table, layer: int, kind: int, inp, gather: bool, perm, offsets, T: int, topk: int,
         out, out_dtype: int, stream=None) -> None:
    _check(ctx.L.apmoe_gemm(ctx.handle, table.handle, layer, kind, ptr(inp), int(gather), ptr(perm), ptr(offsets),
                            T, topk, ptr(out), out_dtype, stream_handle(stream)), "apmoe_gemm", ctx.L)


def gemm_act(ctx: Context, table: Table, layer: int, x, gather: bool, perm, offsets, T: int, topk: int, a,
             stream=None) -> None:
    """gate_up product with SiLU(gate) * up in its epilogue: fp16 a [T*topk][F]."""
    _check(ctx.L.apmoe_gemm_act(ctx.handle, table.handle, layer, ptr(x), int(gather), ptr(perm), ptr(offsets), T,
                                topk, ptr(a), stream_handle(stream)), "apmoe_gemm_act", ctx.L)


def act(ctx: Context, h, R: int, F: int, a, stream=None) -> None:
    _check(ctx.L.apmoe_act(ctx.handle, ptr(h), R, F, ptr(a), stream_handle(stream)), "apmoe_act", ctx.L)


def combine(ctx: Context, y, y_dtype: int, topk_w, inv_perm, T: int, topk: int, H: int, out, stream=None) -> None:
    _check(ctx.L.apmoe_combine(ctx.handle, ptr(y), y_dtype, ptr(topk_w), ptr(inv_perm), T, topk, H, ptr(out),
                               stream_handle(stream)), "apmoe_combine", ctx.L)


def moe_workspace(table: Table, layer: int, T: int, topk: int, n_shared: int = 0) -> int:
    n = ctypes.c_size_t()
    _check(table.L.apmoe_moe_workspace(table.handle, layer, T, topk, n_shared, ctypes.byref(n)), "apmoe_moe_workspace",
           table.L)
    return n.value


def moe_forward(ctx: Context, table: Table, layer: int, x, w_router, bias, T: int, topk: int, renormalize: bool,
                ws, ws_bytes: int, out, stream=None, n_shared: int = 0) -> None:
    """Whole layer; the table's last n_shared experts of the layer are shared ones."""
    _check(ctx.L.apmoe_moe_forward(ctx.handle, table.handle, layer, ptr(x), ptr(w_router), ptr(bias), T, topk,
                                   n_shared,
                                   int(renormalize), ptr(ws), ws_bytes, ptr(out), stream_handle(stream)),
           "apmoe_moe_forward", ctx.L)


NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_forward_noalloc(ctx: Context, table: Table, layer: int, x, w_router, bias, T: int, topk: int,
                        renormalize: bool, out, stream=None, n_shared: int = 0) -> None:
    """The whole layer with the library's static scratch as its workspace (no device
    allocation by the call)."""
    _check(ctx.L.apmoe_moe_forward_noalloc(ctx.handle, table.handle, layer, ptr(x), ptr(w_router), ptr(bias), T,
                                           topk, n_shared, int(renormalize), ptr(out), stream_handle(stream)),
           "apmoe_moe_forward_noalloc", ctx.L)


# --------------------------------------------------------------------------- page movement

def _plane_array(planes):
    arr = (ctypes.c_void_p * PLANES)()
    for p, t in enumerate(planes if planes is not None else []):
        if p < PLANES:
            arr[p] = ptr(t)
    return arr


def _event_handle(ev, stream) -> int:
    """Raw hipEvent_t of a torch.cuda.Event (recorded once on `stream` so that the
    handle exists; the library records it again)."""
    ev.record(stream)
    return ev.cuda_event


def page_out(ctx: Context, table: Table, layer: int, expert: int, kind: int, q_new: int, host_planes,
             stream, copy_stream, done_event) -> None:
    """Lower (layer, expert, kind) to q_new and copy planes q_new.. to host_planes[p]
    (8-entry list; pinned tensors).  done_event (torch.cuda.Event) completes once the
    device planes may be freed."""
    _check(ctx.L.apmoe_page_out(ctx.handle, table.handle, layer, expert, kind, q_new, _plane_array(host_planes),
                                stream_handle(stream), stream_handle(copy_stream),
                                _event_handle(done_event, copy_stream)), "apmoe_page_out", ctx.L)


def page_in(ctx: Context, table: Table, layer: int, expert: int, kind: int, q_new: int, host_planes, dev_planes,
            stream, copy_stream, copied_event) -> None:
    """Copy host_planes[p] to dev_planes[p] for the planes above the current bitwidth,
    then raise (layer, expert, kind) to q_new with a commit on `stream` that waits for
    the copies."""
    _check(ctx.L.apmoe_page_in(ctx.handle, table.handle, layer, expert, kind, q_new, _plane_array(host_planes),
                               _plane_array(dev_planes), stream_handle(stream), stream_handle(copy_stream),
                               _event_handle(copied_event, copy_stream)), "apmoe_page_in", ctx.L)
