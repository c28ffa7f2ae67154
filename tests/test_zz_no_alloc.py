"""topk_decode_noalloc, the fused step for callers that cannot allocate device
memory, against topk_decode on the same inputs: outputs and indices bitwise
equal (the same kernels run on the library's per-GPU scratch array instead of
a caller workspace), on two calls in a row, the second with a smaller input
and another layout of the scratch, then the block-mean and indexer variants
on the same array."""
import numpy as np
import pytest
import torch

import fixtures as fx
import oracle as orc
from tests.gpu_common import dev, problem, say, tka, tol

pytestmark = pytest.mark.gpu


def _both(w, **kw):
    m = tka()
    q, K, V = fx.make_attn(w)
    qt, Kt, Vt = dev(q), dev(K), dev(V)
    p = problem(w)
    if w.mode == fx.MODE_BLOCK:
        kw = dict(proxy_keys=m.topk_block_mean_build(p, Kt))
    elif w.mode == fx.MODE_INDEXER:
        qI, kI, wt = fx.make_indexer(w)
        kw = dict(proxy_keys=dev(kI), q_idx=dev(qI), idx_w=dev(wt))
    need = m.topk_decode_workspace_size(p)
    assert need <= m.NOALLOC_SCRATCH_BYTES, need
    say(f"[no-alloc] {w.name}: B={w.B} L={w.L} k={w.k}, step scratch {need / 2**20:.1f} MiB")
    out_n, idx_n = m.topk_decode_noalloc(p, qt, Kt, Vt, **kw)
    out_w, idx_w = m.topk_decode(p, qt, Kt, Vt, **kw)
    torch.cuda.synchronize()
    assert torch.equal(idx_n, idx_w)
    assert torch.equal(out_n.view(torch.int32), out_w.view(torch.int32))
    return w, q, K, V, out_n, idx_n


def test_noalloc_two_calls_then_smaller():
    # 1: the candidate prefilter path (k' <= L/8): samples, candidate lists and repair slots in the scratch
    big = fx.Workload("noalloc-prefilter", fx.MODE_EXACT, 4, 64, 8, 128, 65536, 2048, fx.BF16, 61,
                      fx.PLANT_ALIGN, 328, 0.5)
    _both(big)
    # 2: smaller, the dense path (full score array, row select): another layout of the same scratch
    small = fx.shrink(fx.WORKLOADS["C3"], 6000, B=2, k=512)
    w, q, K, V, out, idx = _both(small)
    # and against the oracle: attention over the kept sets within tolerance
    gi = idx.cpu().numpy().reshape(-1, w.k)
    ref = orc.attend(orc.problem_for(w), q, K, V, gi, list_mode=0)
    assert np.abs(out.cpu().numpy().reshape(-1, w.d) - ref).max() <= tol(w)


def test_noalloc_block_mean_and_indexer():
    _both(fx.shrink(fx.WORKLOADS["C4"], 64 * 150 + 17, B=2))
    _both(fx.shrink(fx.WORKLOADS["C5"], 50001))
    # after the proxies, an exact step again on the same array
    _both(fx.shrink(fx.WORKLOADS["C2"], 9000, k=700))
