"""Seeded synthetic inputs shared by the oracle checks, the GPU tests and the bench.

Only input bytes come from here (see gen.c); no scoring, selection or softmax.
The workloads mirror the pages' long-context decode setting: a fixed top-k
budget (2048 is the example budget in "Evolution of Sparse Attention in
Long-Context LLMs", section 4, and "Sparse Attention in LLM Inference", "The
Significance of Top-K"), contexts up to a million tokens, grouped KV heads,
block-mean and lightweight-indexer proxies ("Sparse Attention Landscape",
"Block Sparse Attention" and "Token Sparse Attention").
"""
from __future__ import annotations

import ctypes
import hashlib
import math
import os
import subprocess
from dataclasses import dataclass, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libfx.so")
_SRC = os.path.join(_HERE, "gen.c")

F32, BF16, E4M3 = 0, 1, 2
PLANT_NONE, PLANT_SCALE, PLANT_ALIGN, PLANT_BLOCK = 0, 1, 2, 3
MODE_EXACT, MODE_BLOCK, MODE_INDEXER = 0, 1, 2


def build(force: bool = False) -> str:
    """Compile gen.c into libfx.so (plain gcc, OpenMP, no fast-math)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


class _Spec(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("L", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("plant", ctypes.c_int32), ("n_plant", ctypes.c_int32), ("block", ctypes.c_int32),
                ("plant_param", ctypes.c_double), ("seed", ctypes.c_uint64)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        _lib.fx_make_attn.argtypes = [ctypes.POINTER(_Spec), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        _lib.fx_make_indexer.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        _lib.fx_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                   ctypes.c_int, ctypes.c_void_p]
        _lib.fx_encode.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
        _lib.fx_sample_distinct.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_void_p]
    return _lib


def _np_dtype(dt: int):
    return {F32: np.float32, BF16: np.uint16, E4M3: np.uint8}[dt]


@dataclass(frozen=True)
class Workload:
    """One decode-step workload: shapes, budget, scoring variant and input recipe."""
    name: str
    mode: int
    B: int
    Hq: int
    Hkv: int
    d: int
    L: int
    k: int
    dtype: int
    seed: int
    plant: int = PLANT_NONE
    n_plant: int = 0
    plant_param: float = 0.0
    block: int = 0          # block-mean variant: block size b
    HI: int = 0             # indexer variant: indexer heads
    dI: int = 0             # indexer variant: indexer dim

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def m(self) -> int:
        return (self.L + self.block - 1) // self.block if self.block else 0


def _plant_rows(frac: float, L: int) -> int:
    return int(round(frac * L))


def _workloads():
    w = {}
    w["C1"] = Workload("exact-f32-L1024-k64", MODE_EXACT, 1, 1, 1, 64, 1024, 64, F32, 1,
                       PLANT_SCALE, 16, 3.0)
    w["C2"] = Workload("gqa-exact-bf16-L32K-k2048", MODE_EXACT, 1, 32, 8, 128, 32768, 2048, BF16, 2,
                       PLANT_ALIGN, _plant_rows(0.01, 32768), 0.5)
    w["C3"] = Workload("batched-gqa-exact-bf16-L128K-k4096", MODE_EXACT, 16, 64, 8, 128, 131072, 4096, BF16, 3,
                       PLANT_ALIGN, _plant_rows(0.005, 131072), 0.5)
    m4 = 131072 // 64
    w["C4"] = Workload("block-mean-bf16-L128K-b64-top16", MODE_BLOCK, 4, 32, 8, 128, 131072, 16, BF16, 4,
                       PLANT_BLOCK, _plant_rows(0.02, m4), math.sqrt(128 / (3 * 64)), block=64)
    w["C5"] = Workload("indexer-e4m3-L1M-top2048", MODE_INDEXER, 1, 64, 8, 128, 1048576, 2048, BF16, 5,
                       HI=32, dI=64)
    return w


WORKLOADS = _workloads()


def shrink(w: Workload, L: int, B: int | None = None, Hq: int | None = None, Hkv: int | None = None,
           k: int | None = None, seed: int | None = None) -> Workload:
    """Same recipe at a size the oracle finishes in seconds (planting keeps its density)."""
    B = w.B if B is None else B
    Hq = w.Hq if Hq is None else Hq
    Hkv = w.Hkv if Hkv is None else Hkv
    if w.plant == PLANT_BLOCK:
        m = (L + w.block - 1) // w.block
        n_plant = max(1, int(round(0.02 * m)))
    elif w.plant == PLANT_ALIGN:
        n_plant = max(1, int(round(w.n_plant / w.L * L)))
    else:
        n_plant = min(w.n_plant, L)
    return replace(w, name=w.name + f"-shrunk-L{L}", B=B, Hq=Hq, Hkv=Hkv, L=L,
                   k=w.k if k is None else k, n_plant=n_plant, seed=w.seed if seed is None else seed)


def make_attn(w: Workload):
    """q [B,Hq,d], K and V [B,Hkv,L,d]; fp32 arrays or raw bf16 bit patterns (uint16)."""
    nd = _np_dtype(w.dtype)
    q = np.empty((w.B, w.Hq, w.d), nd)
    K = np.empty((w.B, w.Hkv, w.L, w.d), nd)
    V = np.empty((w.B, w.Hkv, w.L, w.d), nd)
    sp = _Spec(w.B, w.Hq, w.Hkv, w.d, w.L, w.dtype, w.plant, w.n_plant, w.block, w.plant_param, w.seed)
    rc = lib().fx_make_attn(ctypes.byref(sp), q.ctypes.data, K.ctypes.data, V.ctypes.data)
    if rc != 0:
        raise ValueError(f"fx_make_attn failed ({rc}) for {w}")
    return q, K, V


def make_indexer(w: Workload):
    """qI [B,HI,dI] and kI [B,L,dI] as E4M3FN bytes, w [B,HI] float32."""
    qI = np.empty((w.B, w.HI, w.dI), np.uint8)
    kI = np.empty((w.B, w.L, w.dI), np.uint8)
    wt = np.empty((w.B, w.HI), np.float32)
    rc = lib().fx_make_indexer(w.seed, w.B, w.HI, w.dI, w.L, qI.ctypes.data, kI.ctypes.data, wt.ctypes.data)
    if rc != 0:
        raise ValueError(f"fx_make_indexer failed ({rc})")
    return qI, kI, wt


def normal(seed: int, tensor: int, n: int, dtype: int = F32, offset: int = 0):
    out = np.empty(n, _np_dtype(dtype))
    lib().fx_normal(seed, tensor, offset, n, dtype, out.ctypes.data)
    return out


def encode(x, dtype: int):
    """fp32 -> bf16 (RNE) or E4M3FN (RNE, saturating) bit patterns."""
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(x.shape, _np_dtype(dtype))
    lib().fx_encode(x.ctypes.data, x.size, dtype, out.ctypes.data)
    return out


def sample_distinct(seed: int, stream: int, rng: int, n: int):
    out = np.empty(n, np.int64)
    if lib().fx_sample_distinct(seed, stream, rng, n, out.ctypes.data) != 0:
        raise ValueError("bad sample request")
    return out


def bf16_bits_to_f32(a):
    return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32)


def digest(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()
