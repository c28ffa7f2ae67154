"""The C ABI without a GPU: the library loads, exports every function that
include/tka.h declares, and every argument check fails with its own status
before any launch (so these calls are safe on a machine without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tka.h")

# no skip: a missing libtka.so (build() not run, or a failed build) fails every test here
import top_sparse_attention_topk_amd as tka  # noqa: E402

LIB = tka.LIB

FAKE = 1 << 40  # aligned, never dereferenced: every call below fails its checks first


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?([a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_function():
    names = declared_functions()
    assert {"topk_attn_score", "topk_select", "sparse_attn_gather", "topk_decode"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", tka.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert LIB.tka_abi_version() == 3


def _status(code):
    return LIB.tka_status_str(code).decode()


def _p(**kw):
    base = dict(mode=tka.EXACT, batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, seq_len=1000, top_k=64,
                dtype=tka.TKA_BF16)
    base.update(kw)
    return tka.problem(**base)


def _score(p, q=FAKE, keys=FAKE * 2, w=None, scores=FAKE * 3):
    return LIB.topk_attn_score(ctypes.byref(p), q, keys, w, scores, None)


def test_status_strings():
    assert [_status(i) for i in range(6)] == ["TKA_OK", "TKA_ERR_INVALID_ARG", "TKA_ERR_UNSUPPORTED",
                                               "TKA_ERR_WORKSPACE", "TKA_ERR_ALIGNMENT", "TKA_ERR_HIP"]


@pytest.mark.parametrize("kw,status", [
    (dict(top_k=0), tka.TKA_ERR_INVALID_ARG),
    (dict(seq_len=0), tka.TKA_ERR_INVALID_ARG),
    (dict(batch=0), tka.TKA_ERR_INVALID_ARG),
    (dict(n_q_heads=6, n_kv_heads=4), tka.TKA_ERR_INVALID_ARG),
    (dict(head_dim=96), tka.TKA_ERR_UNSUPPORTED),
    (dict(dtype=tka.TKA_FP8_E4M3), tka.TKA_ERR_UNSUPPORTED),
    (dict(mode=tka.BLOCK_MEAN, block_size=0), tka.TKA_ERR_INVALID_ARG),
    (dict(mode=tka.INDEXER, n_idx_heads=32, idx_dim=96), tka.TKA_ERR_UNSUPPORTED),
    (dict(mode=tka.INDEXER, n_idx_heads=0, idx_dim=64), tka.TKA_ERR_INVALID_ARG),
    (dict(strides=(1000 * 2 * 128, 1000 * 128, 100)), tka.TKA_ERR_INVALID_ARG),
    (dict(strides=(1000 * 2 * 136, 1000 * 136, 132)), tka.TKA_ERR_ALIGNMENT),
])
def test_problem_checks(kw, status):
    p = _p(**kw)
    assert _score(p, w=FAKE * 4 if p.mode == tka.INDEXER else None) == status
    assert LIB.tka_last_error().decode() != ""


def test_score_pointer_checks():
    p = _p()
    assert _score(p, q=None) == tka.TKA_ERR_INVALID_ARG
    assert _score(p, q=FAKE + 8) == tka.TKA_ERR_ALIGNMENT
    assert _score(p, scores=None) == tka.TKA_ERR_INVALID_ARG
    assert _score(p, w=FAKE * 4) == tka.TKA_ERR_INVALID_ARG  # idx_w only for the indexer
    assert _score(p, scores=FAKE * 2 + 64) == tka.TKA_ERR_INVALID_ARG  # scores inside the K cache
    pi = _p(mode=tka.INDEXER, n_idx_heads=32, idx_dim=64)
    assert _score(pi, w=None) == tka.TKA_ERR_INVALID_ARG


def _select(scores=FAKE, n_rows=4, row_len=100, stride=100, k=10, idx=FAKE * 2, sel=None, ws=None, ws_bytes=0):
    return LIB.topk_select(scores, n_rows, row_len, stride, k, idx, sel, ws, ws_bytes, None)


def test_select_checks():
    assert _select(k=0) == tka.TKA_ERR_INVALID_ARG
    assert _select(stride=50) == tka.TKA_ERR_INVALID_ARG
    assert _select(idx=None) == tka.TKA_ERR_INVALID_ARG
    assert _select(scores=FAKE + 2) == tka.TKA_ERR_ALIGNMENT
    assert _select(idx=FAKE + 8) == tka.TKA_ERR_INVALID_ARG  # idx_out inside the scores
    assert _select(n_rows=-1) == tka.TKA_ERR_INVALID_ARG
    # few long rows need scratch
    need = tka.topk_select_workspace_size(2, 1 << 20, 2048)
    assert need > 0
    assert _select(n_rows=2, row_len=1 << 20, stride=1 << 20, k=2048, idx=FAKE * 4) == tka.TKA_ERR_WORKSPACE
    assert _select(n_rows=2, row_len=1 << 20, stride=1 << 20, k=2048, idx=FAKE * 4, ws=FAKE * 8,
                   ws_bytes=need - 1) == tka.TKA_ERR_WORKSPACE
    # many long rows: samples, thresholds, flags and candidate lists (3 k' pairs a row at most 12288)
    need = tka.topk_select_workspace_size(1024, 131072, 4096)
    assert 1024 * 12288 * 8 <= need < 1024 * 12288 * 8 + (16 << 20)
    assert _select(n_rows=1024, row_len=131072, stride=131072, k=4096, idx=FAKE * 64) == tka.TKA_ERR_WORKSPACE
    # short rows: one workgroup (or wave) per row, no scratch
    assert tka.topk_select_workspace_size(1024, 8192, 256) == 0
    assert tka.topk_select_workspace_size(1024, 131072, 32768) == 0  # k' > n/8: the row kernel
    # few rows split over workgroups: the finish's table of segment offsets bounds the row length
    far = 1 << 44
    assert _select(n_rows=2, row_len=20_000_000, stride=20_000_000, k=2048, idx=far) == tka.TKA_ERR_UNSUPPORTED
    assert _select(n_rows=2, row_len=12_000_000, stride=12_000_000, k=2048, idx=far) == tka.TKA_ERR_WORKSPACE


def _gather(p, q=FAKE, K=FAKE * 2, V=FAKE * 3, idx=FAKE * 4, n_idx=64, unit=0, shared=0, sel=None, out=FAKE * 5,
            ws=None, ws_bytes=0):
    return LIB.sparse_attn_gather(ctypes.byref(p), q, K, V, idx, n_idx, unit, shared, sel, out, ws, ws_bytes, None)


def test_gather_checks():
    p = _p()
    assert _gather(p, n_idx=0) == tka.TKA_ERR_INVALID_ARG
    assert _gather(p, unit=-1) == tka.TKA_ERR_INVALID_ARG
    assert _gather(p, V=None) == tka.TKA_ERR_INVALID_ARG
    assert _gather(p, out=FAKE * 2 + 256) == tka.TKA_ERR_INVALID_ARG  # out inside K
    assert _gather(p, shared=1, sel=FAKE * 6) == tka.TKA_ERR_INVALID_ARG
    assert _gather(p, unit=64, sel=FAKE * 6) == tka.TKA_ERR_INVALID_ARG
    assert _gather(_p(n_q_heads=6, n_kv_heads=2), shared=1) == tka.TKA_ERR_UNSUPPORTED
    # split work needs partials
    small = _p(batch=1, n_q_heads=4, n_kv_heads=1, seq_len=100000, top_k=4096)
    need = tka.sparse_attn_gather_workspace_size(small, 4096)
    assert need > 0 and _gather(small, n_idx=4096) == tka.TKA_ERR_WORKSPACE


def test_decode_checks_and_workspace():
    p = _p()
    need = tka.topk_decode_workspace_size(p)
    assert need >= 2 * 8 * 1000 * 4  # at least the score array
    call = lambda **kw: LIB.topk_decode(ctypes.byref(p), kw.get("q", FAKE), kw.get("K", FAKE * 2),
                                        kw.get("V", FAKE * 3), kw.get("proxy"), kw.get("qi"), kw.get("w"),
                                        kw.get("out", FAKE * 5), kw.get("idx"), kw.get("ws", FAKE * 8),
                                        kw.get("ws_bytes", need), None)
    assert call(ws_bytes=need - 1) == tka.TKA_ERR_WORKSPACE
    assert call(ws=None) == tka.TKA_ERR_WORKSPACE
    assert call(proxy=FAKE * 6) == tka.TKA_ERR_INVALID_ARG  # no proxy keys in the exact variant
    assert call(out=None) == tka.TKA_ERR_INVALID_ARG
    assert call(idx=FAKE * 5) == tka.TKA_ERR_INVALID_ARG  # idx_out overlapping out
    pb = _p(mode=tka.BLOCK_MEAN, block_size=64)
    assert LIB.topk_decode(ctypes.byref(pb), FAKE, FAKE * 2, FAKE * 3, None, None, None, FAKE * 5, None, FAKE * 8,
                           1 << 30, None) == tka.TKA_ERR_INVALID_ARG  # block means missing
    assert LIB.topk_block_mean_build(ctypes.byref(p), FAKE, FAKE * 2, None) == tka.TKA_ERR_INVALID_ARG


def test_decode_path_values():
    """decode_path takes auto, prefilter or dense; anything else fails before any launch. The
    automatic choice keeps the score array below 2^22 scores (it is in the workspace) and drops it
    above; forced paths size the workspace for their own path."""
    ok = tka.problem(tka.EXACT, 2, 8, 2, 128, 32768, 2048)
    for bad in (-1, 3):
        p = tka.problem(tka.EXACT, 2, 8, 2, 128, 32768, 2048, decode_path=bad)
        assert LIB.topk_attn_score(ctypes.byref(p), FAKE, FAKE * 2, None, FAKE * 3, None) == tka.TKA_ERR_INVALID_ARG
    scores = 2 * 8 * 32768 * 4
    assert tka.topk_decode_workspace_size(ok) >= scores  # 2^19 scores: dense
    pre = tka.problem(tka.EXACT, 2, 8, 2, 128, 32768, 2048, decode_path=tka.TKA_PATH_PREFILTER)
    assert tka.topk_decode_workspace_size(pre) != tka.topk_decode_workspace_size(ok)
    big = tka.problem(tka.EXACT, 16, 8, 2, 128, 32768, 2048)  # 2^22 scores: prefilter
    dense = tka.problem(tka.EXACT, 16, 8, 2, 128, 32768, 2048, decode_path=tka.TKA_PATH_DENSE)
    assert tka.topk_decode_workspace_size(dense) >= 16 * 8 * 32768 * 4
    assert tka.topk_decode_workspace_size(big) == tka.topk_decode_workspace_size(
        tka.problem(tka.EXACT, 16, 8, 2, 128, 32768, 2048, decode_path=tka.TKA_PATH_PREFILTER))


def test_workspace_sizes_scale_with_problem():
    c3 = tka.problem(tka.EXACT, 16, 64, 8, 128, 131072, 4096)
    n = tka.topk_decode_workspace_size(c3)
    # with the prefilter: candidate lists (3k per row, 8-byte pairs) + the repair's score slots
    # (64 MiB) + indices, kept scores and samples; no [B*Hq, L] score array
    cand = 16 * 64 * 3 * 4096 * 8
    assert cand + (64 << 20) <= n < cand + (64 << 20) + (48 << 20)
    # without it (k' > L/8) the full score array
    dense = tka.problem(tka.EXACT, 16, 64, 8, 128, 131072, 20000)
    assert tka.topk_decode_workspace_size(dense) >= 16 * 64 * 131072 * 4


def test_adaptive_checks():
    sel = lambda **kw: LIB.topk_select_adaptive(kw.get("scores", FAKE), kw.get("n_rows", 4), kw.get("row_len", 100),
                                                kw.get("stride", 100), kw.get("eps", 0.1), kw.get("k_min", 1),
                                                kw.get("k_max", 10), kw.get("idx", FAKE * 2), kw.get("k", FAKE * 3),
                                                kw.get("tau", FAKE * 4), kw.get("sel"), kw.get("ws", FAKE * 5),
                                                kw.get("ws_bytes", 1 << 20), None)
    assert sel(eps=float("nan")) == tka.TKA_ERR_INVALID_ARG
    assert sel(eps=-0.1) == tka.TKA_ERR_INVALID_ARG
    assert sel(eps=float("inf")) == tka.TKA_ERR_INVALID_ARG
    assert sel(k_max=0) == tka.TKA_ERR_INVALID_ARG
    assert sel(k_min=-1) == tka.TKA_ERR_INVALID_ARG
    assert sel(k=None) == tka.TKA_ERR_INVALID_ARG
    assert sel(tau=FAKE * 3 + 8) == tka.TKA_ERR_INVALID_ARG  # tau_out overlaps k_out
    assert sel(k=FAKE * 3 + 2) == tka.TKA_ERR_ALIGNMENT
    need = tka.topk_select_adaptive_workspace_size(4, 100, 10)
    assert need >= 4 * 12
    assert sel(ws_bytes=need - 1) == tka.TKA_ERR_WORKSPACE
    assert sel(ws=None) == tka.TKA_ERR_WORKSPACE
    # the certified step is defined on exact attention logits only
    pb = _p(mode=tka.BLOCK_MEAN, block_size=64)
    dec = lambda p, **kw: LIB.topk_decode_adaptive(ctypes.byref(p), FAKE, FAKE * 2, FAKE * 3, kw.get("eps", 0.1), 1,
                                                    FAKE * 5, None, None, None, kw.get("ws", FAKE * 8),
                                                    kw.get("ws_bytes", 1 << 30), None)
    assert dec(pb) == tka.TKA_ERR_INVALID_ARG
    p = _p()
    need = tka.topk_decode_adaptive_workspace_size(p)
    assert need >= 2 * 8 * 1000 * 4
    assert dec(p, ws_bytes=need - 1) == tka.TKA_ERR_WORKSPACE
    assert dec(p, eps=float("nan")) == tka.TKA_ERR_INVALID_ARG


def test_cache_append_checks():
    p = _p()
    app = lambda p, **kw: LIB.topk_cache_append(ctypes.byref(p), kw.get("kn", FAKE), kw.get("vn", FAKE * 2),
                                                kw.get("K", FAKE * 3), kw.get("V", FAKE * 4), kw.get("kin"),
                                                kw.get("kic"), kw.get("means"), None)
    assert app(p, vn=None) == tka.TKA_ERR_INVALID_ARG          # both new rows or neither
    assert app(p, K=None) == tka.TKA_ERR_INVALID_ARG
    assert app(p, kn=FAKE + 8) == tka.TKA_ERR_ALIGNMENT
    assert app(p, vn=FAKE * 3 + 256) == tka.TKA_ERR_INVALID_ARG  # v_new inside the K cache
    assert app(p, means=FAKE * 6) == tka.TKA_ERR_INVALID_ARG     # means only for the block variant
    assert app(p, kin=FAKE * 6, kic=FAKE * 7) == tka.TKA_ERR_INVALID_ARG  # indexer keys only for the indexer
    pb = _p(mode=tka.BLOCK_MEAN, block_size=64)
    assert app(pb, means=FAKE * 3 + 512) == tka.TKA_ERR_INVALID_ARG  # means overlapping the K cache
    pi = _p(mode=tka.INDEXER, n_idx_heads=32, idx_dim=64)
    assert app(pi, kin=FAKE * 6) == tka.TKA_ERR_INVALID_ARG      # kI_cache missing
    assert app(pi, kin=FAKE * 6 + 2, kic=FAKE * 7) == tka.TKA_ERR_ALIGNMENT
    # the block-mean capacity must hold every block
    small = _p(mode=tka.BLOCK_MEAN, block_size=64, seq_len=1000)
    small.block_capacity = 15  # ceil(1000 / 64) = 16
    assert _score(small) == tka.TKA_ERR_INVALID_ARG
    small.block_capacity = 16
    assert _score(small) != tka.TKA_ERR_INVALID_ARG or LIB.tka_last_error().decode().find("capacity") < 0


def test_hisa_checks():
    p = _p(mode=tka.HISA, block_size=64, top_blocks=8, top_k=100)
    call = lambda p, **kw: LIB.topk_hisa_decode(ctypes.byref(p), FAKE, FAKE * 2, FAKE * 3, kw.get("means", FAKE * 6),
                                                FAKE * 5, kw.get("idx"), kw.get("blk"), None, None,
                                                kw.get("ws", FAKE * 8), kw.get("ws_bytes", 1 << 30), None)
    need = tka.topk_hisa_decode_workspace_size(p)
    assert need > 0
    assert call(p, ws_bytes=need - 1) == tka.TKA_ERR_WORKSPACE
    assert call(p, means=None) == tka.TKA_ERR_INVALID_ARG
    assert call(p, idx=FAKE * 5 + 4) == tka.TKA_ERR_INVALID_ARG    # idx_out inside out
    assert call(p, blk=FAKE * 9, idx=FAKE * 9) == tka.TKA_ERR_INVALID_ARG  # two outputs overlapping
    assert call(_p(mode=tka.HISA, block_size=64, top_blocks=0)) == tka.TKA_ERR_INVALID_ARG
    assert call(_p(mode=tka.HISA, block_size=0, top_blocks=4)) == tka.TKA_ERR_INVALID_ARG
    assert call(_p(mode=tka.BLOCK_MEAN, block_size=64)) == tka.TKA_ERR_INVALID_ARG  # wrong mode
    # topk_decode leaves the two-level mode to topk_hisa_decode
    assert LIB.topk_decode(ctypes.byref(p), FAKE, FAKE * 2, FAKE * 3, FAKE * 6, None, None, FAKE * 5, None, FAKE * 8,
                           1 << 30, None) == tka.TKA_ERR_INVALID_ARG


def test_workspace_size_by_kind():
    """topk_workspace_size(p, which) reports what the per-call queries report."""
    c3 = tka.problem(tka.EXACT, 16, 64, 8, 128, 131072, 4096)
    assert tka.topk_workspace_size(c3, tka.WS_DECODE) == tka.topk_decode_workspace_size(c3)
    assert tka.topk_workspace_size(c3, tka.WS_SELECT) == tka.topk_select_workspace_size(16 * 64, 131072, 4096)
    assert tka.topk_workspace_size(c3, tka.WS_GATHER) == tka.sparse_attn_gather_workspace_size(c3, 4096)
    assert tka.topk_workspace_size(c3, tka.WS_DECODE_ADAPTIVE) == tka.topk_decode_adaptive_workspace_size(c3)
    c5 = tka.problem(tka.INDEXER, 1, 64, 8, 128, 1 << 20, 2048, n_idx_heads=32, idx_dim=64)
    assert tka.topk_workspace_size(c5, tka.WS_SELECT) == tka.topk_select_workspace_size(1, 1 << 20, 2048) > 0
    assert tka.topk_workspace_size(c5, tka.WS_GATHER) == tka.sparse_attn_gather_workspace_size(c5, 2048, 0, True)
    c4 = tka.problem(tka.BLOCK_MEAN, 4, 32, 8, 128, 131072, 16, block_size=64)
    assert tka.topk_workspace_size(c4, tka.WS_SELECT) == tka.topk_select_workspace_size(128, 2047, 16)
    assert tka.topk_workspace_size(c4, tka.WS_GATHER) == tka.sparse_attn_gather_workspace_size(c4, 16, 64)
    assert tka.topk_workspace_size(c4, tka.WS_DECODE) == tka.topk_decode_workspace_size(c4)
    hs = tka.problem(tka.HISA, 2, 8, 2, 128, 6400, 300, block_size=64, top_blocks=12)
    assert tka.topk_workspace_size(hs, tka.WS_DECODE) == tka.topk_hisa_decode_workspace_size(hs)
    n = ctypes.c_size_t(0)
    assert LIB.topk_workspace_size(ctypes.byref(c3), 7, ctypes.byref(n)) == tka.TKA_ERR_INVALID_ARG
    assert LIB.topk_workspace_size(ctypes.byref(c3), 0, None) == tka.TKA_ERR_INVALID_ARG
    bad = tka.problem(tka.EXACT, 0, 64, 8, 128, 131072, 4096)
    assert LIB.topk_workspace_size(ctypes.byref(bad), 2, ctypes.byref(n)) == tka.TKA_ERR_INVALID_ARG


def test_threshold_scan_checks():
    """The thresholded scan takes up to 4 queries per sequence, bf16, 2 <= G <= 16."""
    call = lambda p, cap=100: LIB.topk_attn_score_threshold(ctypes.byref(p), FAKE, FAKE * 2, FAKE * 3, FAKE * 4,
                                                            FAKE * 5, FAKE * 6, cap, None)
    assert call(_p(n_queries=5)) == tka.TKA_ERR_UNSUPPORTED
    assert call(_p(dtype=tka.TKA_F32)) == tka.TKA_ERR_UNSUPPORTED
    assert call(_p(n_q_heads=2, n_kv_heads=2)) == tka.TKA_ERR_UNSUPPORTED
    assert call(_p(), cap=0) == tka.TKA_ERR_INVALID_ARG
    assert call(_p(mode=tka.BLOCK_MEAN, block_size=64)) == tka.TKA_ERR_INVALID_ARG


def test_noalloc_refuses_steps_beyond_its_scratch():
    """topk_decode_noalloc runs topk_decode's checks, then refuses a step whose workspace exceeds the
    library's scratch array, before any GPU call."""
    call = lambda p, **kw: LIB.topk_decode_noalloc(ctypes.byref(p), kw.get("q", FAKE), FAKE * 2, FAKE * 3, None,
                                                   None, None, kw.get("out", FAKE * 5), None, None)
    big = tka.problem(tka.EXACT, 16, 64, 8, 128, 131072, 32768)  # k' > L/8: the full score array (512 MiB)
    assert tka.topk_decode_workspace_size(big) > tka.NOALLOC_SCRATCH_BYTES
    assert call(big) == tka.TKA_ERR_UNSUPPORTED
    assert "topk_decode_noalloc" in LIB.tka_last_error().decode()
    c3 = tka.problem(tka.EXACT, 16, 64, 8, 128, 131072, 4096)  # the prefilter step fits
    assert tka.topk_decode_workspace_size(c3) <= tka.NOALLOC_SCRATCH_BYTES
    assert call(c3, q=None) == tka.TKA_ERR_INVALID_ARG  # the same argument checks as topk_decode
    assert call(c3, out=FAKE * 2 + 64) == tka.TKA_ERR_INVALID_ARG


def test_bench_probe_library_checks():
    """The benchmark's probe library (not part of the decode ABI) loads, exports its two
    streaming probes, and rejects bad arguments before any launch."""
    probe = ctypes.CDLL(os.path.join(ROOT, "top_sparse_attention_topk_amd", "libtka_probe.so"))
    rd, rw = probe.tka_probe_stream_read, probe.tka_probe_stream_read_write
    rd.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    rw.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    assert rd(None, 4096, FAKE, 1, None) == 1 and rd(FAKE, 4100, FAKE, 1, None) == 1 and rd(FAKE, 4096, FAKE, 0, None) == 1
    assert rw(FAKE, 8192 * 3 + 16, FAKE, FAKE, 1, None) == 1  # not whole 8 KiB tiles
    assert rw(FAKE, 8192, None, FAKE, 1, None) == 1 and rw(FAKE, 8192, FAKE, FAKE, 0, None) == 1
