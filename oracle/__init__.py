"""Python handle on the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's CPU
baseline may use it; the GPU library and its binding never import it.
It shares no code with the GPU path; the two only see the same input bytes
(from ``fixtures``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")

F32, BF16, E4M3 = 0, 1, 2
EXACT, BLOCK, INDEXER = 0, 1, 2


def build(force: bool = False) -> str:
    """Compile oracle.c (gcc, fp64, OpenMP, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


class Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("L", ctypes.c_int32), ("k", ctypes.c_int32),
                ("sb", ctypes.c_int64), ("sh", ctypes.c_int64), ("sl", ctypes.c_int64),
                ("dt", ctypes.c_int32), ("scale", ctypes.c_double), ("mode", ctypes.c_int32),
                ("block", ctypes.c_int32), ("HI", ctypes.c_int32), ("dI", ctypes.c_int32)]


_lib = None
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64


def lib():
    global _lib
    if _lib is None:
        L = ctypes.CDLL(build())
        P = ctypes.POINTER(Problem)
        L.orc_score.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp]
        L.orc_select_f64.argtypes = [_vp, _i64, _i64, _i64, _i64, _vp]
        L.orc_select_f32.argtypes = [_vp, _i64, _i64, _i64, _i64, _vp]
        L.orc_encode_e4m3.argtypes = [_vp, _i64, _vp]
        L.orc_block_means.argtypes = [P, _vp, _vp]
        L.orc_hisa_decode.argtypes = [P, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.orc_decode_mq.argtypes = [P, _i64, _vp, _vp, _vp, _vp, _vp]
        L.orc_select_adaptive_f32.argtypes = [_vp, _i64, _i64, _i64, ctypes.c_double, _i64, _i64, _vp, _vp, _vp]
        L.orc_select_adaptive_f64.argtypes = [_vp, _i64, _i64, _i64, ctypes.c_double, _i64, _i64, _vp, _vp, _vp]
        L.orc_attend.argtypes = [P, _vp, _vp, _vp, _vp, _i64, _i64, ctypes.c_int32, _vp, _i64, _vp]
        L.orc_decode.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp]
        L.orc_diag_exact.argtypes = [P, _vp, _vp, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp]
        L.orc_decode_buf.argtypes = [ctypes.c_int, _vp, _i64, _vp]
        L.orc_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def problem(mode, B, Hq, Hkv, d, L, k, dt, scale=0.0, block=0, HI=0, dI=0, strides=None) -> Problem:
    sb, sh, sl = strides if strides is not None else (Hkv * L * d, L * d, d)
    return Problem(B, Hq, Hkv, d, L, k, sb, sh, sl, dt, scale, mode, block, HI, dI)


def problem_for(w, scale=0.0) -> Problem:
    """Problem of a fixtures.Workload."""
    return problem(w.mode, w.B, w.Hq, w.Hkv, w.d, w.L, w.k, w.dtype, scale, w.block, w.HI, w.dI)


def score_len(p: Problem) -> int:
    if p.mode == BLOCK:
        return (p.L + p.block - 1) // p.block - 1
    return p.L


def _rows_arg(rows, p: Problem):
    if rows is None:
        n = p.B if p.mode == INDEXER else p.B * p.Hq
        return None, n
    rows = np.ascontiguousarray(rows, np.int64)
    return rows, len(rows)


def score(p: Problem, q=None, K=None, qI=None, kI=None, w=None, rows=None):
    """fp64 scores [n_rows, row_len] (rows = b*Hq+h, or b for the indexer)."""
    rows, n = _rows_arg(rows, p)
    out = np.empty((n, score_len(p)), np.float64)
    lib().orc_score(ctypes.byref(p), _ptr(q), _ptr(K), _ptr(qI), _ptr(kI), _ptr(w), _ptr(rows), n, _ptr(out))
    return out


def select(scores, k: int):
    """Exact top-k per row, ascending positions, -1 padded. fp32 input is compared as fp32."""
    s = np.ascontiguousarray(scores)
    if s.ndim == 1:
        s = s[None, :]
    n_rows, n = s.shape
    idx = np.empty((n_rows, k), np.int32)
    if s.dtype == np.float32:
        rc = lib().orc_select_f32(_ptr(s), n_rows, n, n, k, _ptr(idx))
    else:
        s = s.astype(np.float64)
        rc = lib().orc_select_f64(_ptr(s), n_rows, n, n, k, _ptr(idx))
    if rc != 0:
        raise ValueError("bad select arguments")
    return idx


def select_adaptive(scores, eps: float, k_min: int, k_max: int):
    """Certified top-k per row of logits: the smallest k whose top-k keeps >= 1 - eps of the
    softmax mass, clamped to [max(k_min, 1), min(k_max, len)]. Returns (idx [rows, k_max]
    ascending then -1, k [rows], tau [rows] = discarded mass of the final k). fp32 input is
    compared as fp32; masses in fp64."""
    s = np.ascontiguousarray(scores)
    if s.ndim == 1:
        s = s[None, :]
    n_rows, n = s.shape
    idx = np.empty((n_rows, k_max), np.int32)
    k = np.empty(n_rows, np.int32)
    tau = np.empty(n_rows, np.float64)
    if s.dtype == np.float32:
        rc = lib().orc_select_adaptive_f32(_ptr(s), n_rows, n, n, eps, k_min, k_max, _ptr(idx), _ptr(k), _ptr(tau))
    else:
        s = s.astype(np.float64)
        rc = lib().orc_select_adaptive_f64(_ptr(s), n_rows, n, n, eps, k_min, k_max, _ptr(idx), _ptr(k), _ptr(tau))
    if rc != 0:
        raise ValueError("bad adaptive select arguments")
    return idx, k, tau


def block_means(p: Problem, K):
    """fp64 block-mean keys [B, Hkv, ceil(L/b), d] of the block variant (partial last block included)."""
    m = (p.L + p.block - 1) // p.block
    out = np.empty((p.B, p.Hkv, m, p.d), np.float64)
    lib().orc_block_means(ctypes.byref(p), _ptr(K), _ptr(out))
    return out


def decode_mq(p: Problem, M: int, q, K, V):
    """M causal queries per sequence at positions L-M .. L-1 (q [B, M, Hq, d]). Returns (out [B*M*Hq, d],
    idx [B*M*Hq, k]); rows (b*M + t)*Hq + h, query t keeps the top min(k, L-M+t+1) of its visible keys."""
    n = p.B * M * p.Hq
    out = np.empty((n, p.d), np.float64)
    idx = np.empty((n, p.k), np.int32)
    rc = lib().orc_decode_mq(ctypes.byref(p), M, _ptr(q), _ptr(K), _ptr(V), _ptr(out), _ptr(idx))
    if rc != 0:
        raise ValueError("bad multi-query arguments")
    return out, idx


def hisa_decode(p: Problem, KB: int, q, K, V):
    """Two-level selection (top-KB blocks by <q, block mean>, then top-k tokens among their keys by the
    exact score) and attention over the kept tokens. Returns (out [B*Hq, d], idx [B*Hq, k] positions,
    blk [B*Hq, KB] block ids, block scores [B*Hq, m])."""
    m = (p.L + p.block - 1) // p.block
    n = p.B * p.Hq
    out = np.empty((n, p.d), np.float64)
    idx = np.empty((n, p.k), np.int32)
    blk = np.empty((n, KB), np.int32)
    bs = np.empty((n, m), np.float64)
    rc = lib().orc_hisa_decode(ctypes.byref(p), KB, _ptr(q), _ptr(K), _ptr(V), _ptr(out), _ptr(idx), _ptr(blk),
                               _ptr(bs))
    if rc != 0:
        raise ValueError("oracle two-level decode failed")
    return out, idx, blk, bs


def encode_e4m3(x):
    """fp32 values -> OCP E4M3FN codes (nearest, ties to even mantissa, saturating at +-448, NaN -> 0x7f)."""
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().orc_encode_e4m3(_ptr(x), x.size, _ptr(out))
    return out


def attend(p: Problem, q, K, V, idx, unit=0, list_mode=2, rows=None):
    """fp64 softmax attention over kept lists; out [n_rows, d].

    unit 0: lists hold token positions; unit b >= 1: lists hold block ids of b keys and the
    current block (ceil(L/b) - 1) is attended as well. -1 entries are ignored."""
    rows, n = _rows_arg(rows, p) if rows is not None else (None, p.B * p.Hq)
    idx = np.ascontiguousarray(idx, np.int32)
    n_idx = idx.shape[-1]
    out = np.empty((n, p.d), np.float64)
    rc = lib().orc_attend(ctypes.byref(p), _ptr(q), _ptr(K), _ptr(V), _ptr(idx), n_idx, unit, list_mode,
                          _ptr(rows), n, _ptr(out))
    if rc != 0:
        raise ValueError("a row had an empty kept set")
    return out


def decode(p: Problem, q, K, V, qI=None, kI=None, w=None, rows=None):
    """Whole step. Returns (out, idx); out [n_rows, d] or [n_b, Hq, d] for the indexer."""
    rows, n = _rows_arg(rows, p)
    idx = np.empty((n, p.k), np.int32)
    if p.mode == INDEXER:
        out = np.empty((n, p.Hq, p.d), np.float64)
    else:
        out = np.empty((n, p.d), np.float64)
    rc = lib().orc_decode(ctypes.byref(p), _ptr(q), _ptr(K), _ptr(V), _ptr(qI), _ptr(kI), _ptr(w),
                          _ptr(rows), n, _ptr(out), _ptr(idx))
    if rc != 0:
        raise ValueError("oracle decode failed")
    return out, idx


def diag_exact(p: Problem, q, K, V, row: int, kept):
    """Diagnostics of one exact row: dict with tau, tv, kl, entropy, gap, diam, o_full, mu_head, mu_tail."""
    kept = np.ascontiguousarray(kept, np.int32)
    res = np.empty(6, np.float64)
    of, mh, mt = (np.empty(p.d, np.float64) for _ in range(3))
    rc = lib().orc_diag_exact(ctypes.byref(p), _ptr(q), _ptr(K), _ptr(V), row, _ptr(kept), len(kept),
                              _ptr(res), _ptr(of), _ptr(mh), _ptr(mt))
    if rc != 0:
        raise MemoryError
    return dict(tau=res[0], tv=res[1], kl=res[2], entropy=res[3], gap=res[4], diam=res[5],
                o_full=of, mu_head=mh, mu_tail=mt)


def decode_values(dt: int, raw):
    raw = np.ascontiguousarray(raw)
    out = np.empty(raw.size, np.float64)
    lib().orc_decode_buf(dt, _ptr(raw), raw.size, _ptr(out))
    return out.reshape(raw.shape)


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().orc_threads())
