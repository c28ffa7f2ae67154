"""Helpers shared by the GPU parity tests (the oracle side and the library
side see the same fixture bytes; nothing here computes the method)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import fixtures as fx
import oracle as orc

BF16_TOL = 2e-3   # max abs error of outputs for bf16 inputs
F32_TOL = 1e-5    # max abs error of outputs for fp32 inputs


def tka():
    import top_sparse_attention_topk_amd as m
    return m


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(a).to("cuda")


def problem(w: fx.Workload, scale: float = 0.0, decode_path=None):
    """The workload's tka_problem. topk_decode takes the candidate prefilter wherever it applies
    (TKA_PATH_PREFILTER) unless decode_path says otherwise, so that the reduced test sizes exercise
    the path the full sizes take."""
    m = tka()
    dt = m.TKA_BF16 if w.dtype == fx.BF16 else m.TKA_F32
    path = m.TKA_PATH_PREFILTER if decode_path is None else decode_path
    return m.problem(w.mode, w.B, w.Hq, w.Hkv, w.d, w.L, w.k, dt, scale, w.block, w.HI, w.dI, decode_path=path)


def tol(w: fx.Workload) -> float:
    return BF16_TOL if w.dtype == fx.BF16 else F32_TOL


def as_f64(a: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == fx.BF16:
        return fx.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def exact_score_bound(w, q, K, rows):
    """Forward-error bound of an fp32 dot product of length d, scaled:
    d * 2^-23 * scale * sum_c |q_c k_c| (recursive summation bound with slack)."""
    qf, Kf = np.abs(as_f64(q, w.dtype)), np.abs(as_f64(K, w.dtype))
    G = w.Hq // w.Hkv
    out = []
    for r in rows:
        b, h = divmod(int(r), w.Hq)
        out.append(Kf[b, h // G] @ qf[b, h])
    scale = 1.0 / np.sqrt(w.d)
    return np.stack(out) * scale * w.d * 2.0 ** -23 + 1e-30


def block_score_bound(w, q, K):
    """Bound of an fp32 block score <q, mean of the block>: the mean sums up to b terms, the dot d terms;
    (d + b + 2) * 2^-23 * sum_c |q_c| * mean_i |K_ic|, rows b*Hq + h, the m - 1 competing blocks."""
    qa = np.abs(as_f64(q, w.dtype))
    Ka = np.abs(as_f64(K, w.dtype))
    m = w.m
    pad = m * w.block - w.L
    Kp = np.concatenate([Ka, np.zeros(Ka.shape[:2] + (pad, w.d))], 2) if pad else Ka
    sizes = np.minimum(w.block, w.L - np.arange(m) * w.block)
    mabs = Kp.reshape(w.B, w.Hkv, m, w.block, w.d).sum(3) / sizes[None, None, :, None]
    bound = np.stack([mabs[b, h // w.G, : m - 1] @ qa[b, h] for b in range(w.B) for h in range(w.Hq)])
    return bound * (w.d + w.block + 2) * 2.0 ** -23 + 1e-30


def indexer_score_bound(w, qI, kI, wt, b):
    qd = np.abs(orc.decode_values(orc.E4M3, qI[b]))
    kd = np.abs(orc.decode_values(orc.E4M3, kI[b]))
    s = (kd @ qd.T) @ wt[b].astype(np.float64)
    return s * (w.dI + w.HI + 2) * 2.0 ** -23 + 1e-30


def gpu_scores_np(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.float().cpu().numpy()
