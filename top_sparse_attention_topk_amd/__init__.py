"""Python binding of libtka, the gfx950 top-k sparse decode-attention library.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
(include/tka.h). Tensors are torch device tensors; pointers and the current
HIP stream are handed to the library as integers. Importing this package
raises ImportError when libtka.so has not been built - there is no fallback.

The names match the C entry points: topk_attn_score,
topk_attn_score_threshold, topk_select, topk_select_adaptive,
sparse_attn_gather, topk_decode, topk_decode_adaptive, topk_hisa_decode,
topk_cache_append, topk_block_mean_build and the workspace-size queries
(topk_workspace_size and one per call).
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libtka.so")

TKA_OK, TKA_ERR_INVALID_ARG, TKA_ERR_UNSUPPORTED, TKA_ERR_WORKSPACE, TKA_ERR_ALIGNMENT, TKA_ERR_HIP = range(6)
TKA_F32, TKA_BF16, TKA_FP8_E4M3 = 0, 1, 2
EXACT, BLOCK_MEAN, INDEXER, HISA = 0, 1, 2, 3
TKA_PATH_AUTO, TKA_PATH_PREFILTER, TKA_PATH_DENSE = 0, 1, 2  # tka_problem.decode_path


class TkaError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        super().__init__(f"{fn}: status {status} ({detail})")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("seq_len", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("kv_stride_b", ctypes.c_int64), ("kv_stride_h", ctypes.c_int64), ("kv_stride_l", ctypes.c_int64),
                ("qkv_dtype", ctypes.c_int32), ("scale", ctypes.c_float), ("mode", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("n_idx_heads", ctypes.c_int32), ("idx_dim", ctypes.c_int32),
                ("idx_dtype", ctypes.c_int32), ("block_capacity", ctypes.c_int32), ("idx_capacity", ctypes.c_int32),
                ("top_blocks", ctypes.c_int32), ("n_queries", ctypes.c_int32), ("decode_path", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python top_sparse_attention_topk_amd/build.py`")
    # torch first: libtka then binds the HIP runtime torch already loaded (one runtime per
    # process, shared with the tensors whose pointers it receives)
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    P = ctypes.POINTER(Problem)
    sig = {
        "topk_attn_score": [P, vp, vp, vp, vp, vp],
        "topk_attn_score_threshold": [P, vp, vp, vp, vp, vp, vp, i32, vp],
        "topk_select": [vp, i64, i32, i64, i32, vp, vp, vp, sz, vp],
        "topk_select_workspace_size": [i64, i32, i32, ctypes.POINTER(sz)],
        "sparse_attn_gather": [P, vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, sz, vp],
        "sparse_attn_gather_workspace_size": [P, i32, i32, i32, ctypes.POINTER(sz)],
        "topk_decode": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "topk_decode_workspace_size": [P, ctypes.POINTER(sz)],
        "topk_block_mean_build": [P, vp, vp, vp],
        "topk_cache_append": [P, vp, vp, vp, vp, vp, vp, vp, vp],
        "topk_hisa_decode": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "topk_hisa_decode_workspace_size": [P, ctypes.POINTER(sz)],
        "topk_select_adaptive": [vp, i64, i32, i64, f32, i32, i32, vp, vp, vp, vp, vp, sz, vp],
        "topk_select_adaptive_workspace_size": [i64, i32, i32, ctypes.POINTER(sz)],
        "topk_decode_adaptive": [P, vp, vp, vp, f32, i32, vp, vp, vp, vp, vp, sz, vp],
        "topk_decode_adaptive_workspace_size": [P, ctypes.POINTER(sz)],
        "topk_workspace_size": [P, i32, ctypes.POINTER(sz)],
        "topk_decode_noalloc": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.tka_status_str.argtypes = [ctypes.c_int]
    lib.tka_status_str.restype = ctypes.c_char_p
    lib.tka_last_error.argtypes = []
    lib.tka_last_error.restype = ctypes.c_char_p
    lib.tka_abi_version.argtypes = []
    lib.tka_abi_version.restype = ctypes.c_int32
    return lib


LIB = _load()
EXPORTS = ["topk_attn_score", "topk_attn_score_threshold", "topk_select", "topk_select_workspace_size", "sparse_attn_gather",
           "sparse_attn_gather_workspace_size", "topk_decode", "topk_decode_workspace_size",
           "topk_block_mean_build", "topk_select_adaptive", "topk_select_adaptive_workspace_size",
           "topk_decode_adaptive", "topk_decode_adaptive_workspace_size", "topk_cache_append", "topk_hisa_decode",
           "topk_hisa_decode_workspace_size", "topk_workspace_size", "topk_decode_noalloc", "tka_status_str",
           "tka_last_error",
           "tka_abi_version"]


def _check(status: int, fn: str):
    if status != TKA_OK:
        raise TkaError(status, fn, LIB.tka_status_str(status).decode() + ": " + LIB.tka_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def problem(mode: int, batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, seq_len: int, top_k: int,
            dtype: int = TKA_BF16, scale: float = 0.0, block_size: int = 0, n_idx_heads: int = 0, idx_dim: int = 0,
            strides=None, block_capacity: int = 0, idx_capacity: int = 0, top_blocks: int = 0,
            n_queries: int = 0, decode_path: int = 0) -> Problem:
    """tka_problem; strides default to a contiguous [B, Hkv, L, d] cache."""
    sb, sh, sl = strides if strides is not None else (n_kv_heads * seq_len * head_dim, seq_len * head_dim, head_dim)
    return Problem(batch, n_q_heads, n_kv_heads, head_dim, seq_len, top_k, sb, sh, sl, dtype, scale, mode,
                   block_size, n_idx_heads, idx_dim, TKA_FP8_E4M3, block_capacity, idx_capacity, top_blocks,
                   n_queries, decode_path)


def score_shape(p: Problem):
    if p.mode == INDEXER:
        return (p.batch, p.seq_len)
    if p.mode in (BLOCK_MEAN, HISA):
        m = (p.seq_len + p.block_size - 1) // p.block_size
        return (p.batch, p.n_q_heads, m - 1 if p.mode == BLOCK_MEAN else m)
    if p.n_queries > 1:
        return (p.batch, p.n_queries, p.n_q_heads, p.seq_len)
    return (p.batch, p.n_q_heads, p.seq_len)


def _qrows(p: Problem):
    """Leading dims of q / out: (B, M, Hq) with several queries per sequence, else (B, Hq)."""
    return (p.batch, p.n_queries, p.n_q_heads) if p.n_queries > 1 else (p.batch, p.n_q_heads)


def _empty(shape, dtype, like):
    import torch
    return torch.empty(shape, dtype=dtype, device=like.device)


def _ws(nbytes: int, like):
    import torch
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=like.device)


def topk_attn_score(p: Problem, q, keys, idx_w=None, scores=None, stream=None):
    import torch
    if scores is None:
        scores = _empty(score_shape(p), torch.float32, keys)
    _check(LIB.topk_attn_score(ctypes.byref(p), _ptr(q), _ptr(keys), _ptr(idx_w), _ptr(scores), _stream(stream)),
           "topk_attn_score")
    return scores


def topk_attn_score_threshold(p: Problem, q, k_cache, thresholds, counts, cand_scores, cand_pos, stream=None):
    """Append (score, position) pairs ranking at or above thresholds[row]; see include/tka.h."""
    capacity = cand_scores.shape[-1]
    _check(LIB.topk_attn_score_threshold(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(thresholds), _ptr(counts),
                                         _ptr(cand_scores), _ptr(cand_pos), capacity, _stream(stream)),
           "topk_attn_score_threshold")
    return counts


def topk_select_workspace_size(n_rows: int, row_len: int, k: int) -> int:
    n = ctypes.c_size_t(0)
    _check(LIB.topk_select_workspace_size(n_rows, row_len, k, ctypes.byref(n)), "topk_select_workspace_size")
    return n.value


def topk_select(scores, k: int, row_len: int | None = None, row_stride: int | None = None, idx_out=None,
                sel_out=None, want_sel: bool = True, ws=None, stream=None):
    """scores [..., row_len] fp32 -> (idx [n_rows, k] int32, sel [n_rows, k] fp32 or None)."""
    import torch
    row_len = scores.shape[-1] if row_len is None else row_len
    row_stride = (scores.stride(-2) if scores.dim() > 1 else row_len) if row_stride is None else row_stride
    n_rows = 1
    for dim in scores.shape[:-1]:
        n_rows *= int(dim)
    if idx_out is None:
        idx_out = _empty((n_rows, k), torch.int32, scores)
    if sel_out is None and want_sel:
        sel_out = _empty((n_rows, k), torch.float32, scores)
    nbytes = topk_select_workspace_size(n_rows, row_len, k)
    if ws is None and nbytes:
        ws = _ws(nbytes, scores)
    _check(LIB.topk_select(_ptr(scores), n_rows, row_len, row_stride, k, _ptr(idx_out), _ptr(sel_out), _ptr(ws),
                           ws.numel() if ws is not None else 0, _stream(stream)), "topk_select")
    return idx_out, sel_out


def topk_select_adaptive_workspace_size(n_rows: int, row_len: int, k_max: int) -> int:
    n = ctypes.c_size_t(0)
    _check(LIB.topk_select_adaptive_workspace_size(n_rows, row_len, k_max, ctypes.byref(n)),
           "topk_select_adaptive_workspace_size")
    return n.value


def topk_select_adaptive(scores, eps: float, k_min: int, k_max: int, row_len: int | None = None,
                         row_stride: int | None = None, idx_out=None, k_out=None, tau_out=None, sel_out=None,
                         want_sel: bool = False, ws=None, stream=None):
    """Certified top-k of logit rows [..., row_len] fp32 -> (idx [n_rows, k_max], k [n_rows], tau [n_rows],
    sel [n_rows, k_max] or None)."""
    import torch
    row_len = scores.shape[-1] if row_len is None else row_len
    row_stride = (scores.stride(-2) if scores.dim() > 1 else row_len) if row_stride is None else row_stride
    n_rows = 1
    for dim in scores.shape[:-1]:
        n_rows *= int(dim)
    if idx_out is None:
        idx_out = _empty((n_rows, k_max), torch.int32, scores)
    if k_out is None:
        k_out = _empty((n_rows,), torch.int32, scores)
    if tau_out is None:
        tau_out = _empty((n_rows,), torch.float32, scores)
    if sel_out is None and want_sel:
        sel_out = _empty((n_rows, k_max), torch.float32, scores)
    if ws is None:
        ws = _ws(topk_select_adaptive_workspace_size(n_rows, row_len, k_max), scores)
    _check(LIB.topk_select_adaptive(_ptr(scores), n_rows, row_len, row_stride, eps, k_min, k_max, _ptr(idx_out),
                                    _ptr(k_out), _ptr(tau_out), _ptr(sel_out), _ptr(ws), ws.numel(),
                                    _stream(stream)), "topk_select_adaptive")
    return idx_out, k_out, tau_out, sel_out


def sparse_attn_gather_workspace_size(p: Problem, n_idx: int, idx_unit: int = 0, shared: bool = False) -> int:
    n = ctypes.c_size_t(0)
    _check(LIB.sparse_attn_gather_workspace_size(ctypes.byref(p), n_idx, idx_unit, int(shared), ctypes.byref(n)),
           "sparse_attn_gather_workspace_size")
    return n.value


def sparse_attn_gather(p: Problem, q, k_cache, v_cache, idx, idx_unit: int = 0, shared: bool = False,
                       sel_scores=None, out=None, ws=None, stream=None):
    import torch
    n_idx = idx.shape[-1]
    if out is None:
        out = _empty(_qrows(p) + (p.head_dim,), torch.float32, q)
    nbytes = sparse_attn_gather_workspace_size(p, n_idx, idx_unit, shared)
    if ws is None and nbytes:
        ws = _ws(nbytes, q)
    _check(LIB.sparse_attn_gather(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(idx), n_idx,
                                  idx_unit, int(shared), _ptr(sel_scores), _ptr(out), _ptr(ws),
                                  ws.numel() if ws is not None else 0, _stream(stream)), "sparse_attn_gather")
    return out


def topk_decode_workspace_size(p: Problem) -> int:
    n = ctypes.c_size_t(0)
    _check(LIB.topk_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)), "topk_decode_workspace_size")
    return n.value


def topk_decode(p: Problem, q, k_cache, v_cache, proxy_keys=None, q_idx=None, idx_w=None, out=None, idx_out=None,
                ws=None, want_idx: bool = True, stream=None):
    """One fused decode step. Returns (out [B,Hq,d] fp32 ([B,M,Hq,d] with several queries), idx or None)."""
    import torch
    if out is None:
        out = _empty(_qrows(p) + (p.head_dim,), torch.float32, q)
    if idx_out is None and want_idx:
        shape = (p.batch, p.top_k) if p.mode == INDEXER else _qrows(p) + (p.top_k,)
        idx_out = _empty(shape, torch.int32, q)
    if ws is None:
        ws = _ws(topk_decode_workspace_size(p), q)
    _check(LIB.topk_decode(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(proxy_keys), _ptr(q_idx),
                           _ptr(idx_w), _ptr(out), _ptr(idx_out), _ptr(ws), ws.numel(), _stream(stream)),
           "topk_decode")
    return out, idx_out


NOALLOC_SCRATCH_BYTES = 256 << 20


def topk_decode_noalloc(p: Problem, q, k_cache, v_cache, proxy_keys=None, q_idx=None, idx_w=None, out=None,
                        idx_out=None, want_idx: bool = True, stream=None):
    """topk_decode without a workspace (the library's per-GPU scratch array; see include/tka.h).
    Returns (out, idx or None); pass out / idx_out to allocate nothing here either."""
    import torch
    if out is None:
        out = _empty(_qrows(p) + (p.head_dim,), torch.float32, q)
    if idx_out is None and want_idx:
        shape = (p.batch, p.top_k) if p.mode == INDEXER else _qrows(p) + (p.top_k,)
        idx_out = _empty(shape, torch.int32, q)
    _check(LIB.topk_decode_noalloc(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(proxy_keys),
                                   _ptr(q_idx), _ptr(idx_w), _ptr(out), _ptr(idx_out), _stream(stream)),
           "topk_decode_noalloc")
    return out, idx_out


def topk_decode_adaptive_workspace_size(p: Problem) -> int:
    n = ctypes.c_size_t(0)
    _check(LIB.topk_decode_adaptive_workspace_size(ctypes.byref(p), ctypes.byref(n)),
           "topk_decode_adaptive_workspace_size")
    return n.value


def topk_decode_adaptive(p: Problem, q, k_cache, v_cache, eps: float, k_min: int = 1, out=None, idx_out=None,
                         k_out=None, tau_out=None, ws=None, stream=None):
    """Certified decode step (exact scores; k_max = p.top_k). Returns (out, idx, k, tau)."""
    import torch
    if out is None:
        out = _empty((p.batch, p.n_q_heads, p.head_dim), torch.float32, q)
    if idx_out is None:
        idx_out = _empty((p.batch, p.n_q_heads, p.top_k), torch.int32, q)
    if k_out is None:
        k_out = _empty((p.batch, p.n_q_heads), torch.int32, q)
    if tau_out is None:
        tau_out = _empty((p.batch, p.n_q_heads), torch.float32, q)
    if ws is None:
        ws = _ws(topk_decode_adaptive_workspace_size(p), q)
    _check(LIB.topk_decode_adaptive(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), eps, k_min, _ptr(out),
                                    _ptr(idx_out), _ptr(k_out), _ptr(tau_out), _ptr(ws), ws.numel(),
                                    _stream(stream)), "topk_decode_adaptive")
    return out, idx_out, k_out, tau_out


def topk_block_mean_build(p: Problem, k_cache, means=None, stream=None):
    import torch
    if means is None:
        m = p.block_capacity or (p.seq_len + p.block_size - 1) // p.block_size
        means = _empty((p.batch, p.n_kv_heads, m, p.head_dim), torch.float32, k_cache)
    _check(LIB.topk_block_mean_build(ctypes.byref(p), _ptr(k_cache), _ptr(means), _stream(stream)),
           "topk_block_mean_build")
    return means


def topk_cache_append(p: Problem, k_new=None, v_new=None, k_cache=None, v_cache=None, kI_new=None, kI_cache=None,
                      means=None, stream=None):
    """Append the step's new rows at position p.seq_len - 1 (and refresh the block mean / encode the indexer key)."""
    _check(LIB.topk_cache_append(ctypes.byref(p), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                 _ptr(kI_new), _ptr(kI_cache), _ptr(means), _stream(stream)), "topk_cache_append")


def topk_hisa_decode_workspace_size(p: Problem) -> int:
    n = ctypes.c_size_t(0)
    _check(LIB.topk_hisa_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)), "topk_hisa_decode_workspace_size")
    return n.value


def topk_hisa_decode(p: Problem, q, k_cache, v_cache, means, out=None, idx_out=None, want_parts: bool = False,
                     ws=None, stream=None):
    """Two-level step (mode HISA). Returns (out, idx) or, with want_parts, (out, idx, blk [B,Hq,K_B],
    block scores [B,Hq,m], candidate scores [B,Hq,K_B*b])."""
    import torch
    if out is None:
        out = _empty((p.batch, p.n_q_heads, p.head_dim), torch.float32, q)
    if idx_out is None:
        idx_out = _empty((p.batch, p.n_q_heads, p.top_k), torch.int32, q)
    blk = bs = cs = None
    if want_parts:
        m = (p.seq_len + p.block_size - 1) // p.block_size
        blk = _empty((p.batch, p.n_q_heads, p.top_blocks), torch.int32, q)
        bs = _empty((p.batch, p.n_q_heads, m), torch.float32, q)
        cs = _empty((p.batch, p.n_q_heads, p.top_blocks * p.block_size), torch.float32, q)
    if ws is None:
        ws = _ws(topk_hisa_decode_workspace_size(p), q)
    _check(LIB.topk_hisa_decode(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(means), _ptr(out),
                                _ptr(idx_out), _ptr(blk), _ptr(bs), _ptr(cs), _ptr(ws), ws.numel(), _stream(stream)),
           "topk_hisa_decode")
    return (out, idx_out, blk, bs, cs) if want_parts else (out, idx_out)


WS_SELECT, WS_GATHER, WS_DECODE, WS_DECODE_ADAPTIVE = range(4)


def topk_workspace_size(p: Problem, which: int) -> int:
    """Workspace bytes of one step of p: WS_SELECT, WS_GATHER, WS_DECODE or WS_DECODE_ADAPTIVE."""
    n = ctypes.c_size_t(0)
    _check(LIB.topk_workspace_size(ctypes.byref(p), which, ctypes.byref(n)), "topk_workspace_size")
    return n.value


def abi_version() -> int:
    return LIB.tka_abi_version()
