"""Device-side generation of the same synthetic tensors as synth.gen (bit-identical),
for workloads too large to generate on the host.  Built into libsynth.so next to
this file (hipcc, gfx950)."""
from __future__ import annotations

import ctypes
import os
import subprocess

from .gen import TID, MoEConfig, stream_key, tensor_id

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth_gpu.hip")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None


def build() -> str:
    tmp = _LIB + ".tmp"
    # the fp64 -> fp16 rounding is the library's own header (one definition)
    inc = os.path.join(os.path.dirname(_HERE), "any_precision_weight_amd", "csrc")
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", inc, _SRC, "-o", tmp]
    subprocess.run(cmd, check=True, capture_output=True)
    os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            raise ImportError(f"{_LIB} is missing: run synth.gpu.build()")
        L = ctypes.CDLL(_LIB)
        P, U64 = ctypes.c_void_p, ctypes.c_uint64
        L.synth_gpu_planes.argtypes = [U64, U64, P, P]
        L.synth_gpu_fp16_normal.argtypes = [U64, U64, ctypes.c_double, P, P]
        L.synth_gpu_parent_lut.argtypes = [U64, ctypes.c_int, ctypes.c_double, P, P]
        for f in (L.synth_gpu_planes, L.synth_gpu_fp16_normal, L.synth_gpu_parent_lut):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream or None


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what}: hip error {rc}")


def planes_shape(seed: int, layer: int, expert: int, kind: int, N: int, K: int):
    """Canonical planes uint32 [8][N][K/32] as an int32 torch tensor on the device."""
    import torch
    out = torch.empty((8, N, K // 32), dtype=torch.int32, device="cuda")
    key = stream_key(seed, tensor_id(TID.PLANES, layer, expert, kind))
    _check(lib().synth_gpu_planes(key, out.numel(), out.data_ptr(), _stream()), "synth_gpu_planes")
    return out


def parent_lut_shape(seed: int, layer: int, expert: int, kind: int, N: int):
    import torch
    out = torch.empty((N, 256), dtype=torch.float16, device="cuda")
    key = stream_key(seed, tensor_id(TID.LUT, layer, expert, kind))
    _check(lib().synth_gpu_parent_lut(key, N, 0.02, out.data_ptr(), _stream()), "synth_gpu_parent_lut")
    return out


def planes(cfg: MoEConfig, layer: int, expert: int, kind: int):
    N, K = cfg.block_shape(kind)
    return planes_shape(cfg.seed, layer, expert, kind, N, K)


def parent_lut(cfg: MoEConfig, layer: int, expert: int, kind: int):
    N, _ = cfg.block_shape(kind)
    return parent_lut_shape(cfg.seed, layer, expert, kind, N)


def fp16_normal(seed: int, tid: int, n: int, std: float):
    import torch
    out = torch.empty(n, dtype=torch.float16, device="cuda")
    _check(lib().synth_gpu_fp16_normal(stream_key(seed, tid), n, std, out.data_ptr(), _stream()),
           "synth_gpu_fp16_normal")
    return out
