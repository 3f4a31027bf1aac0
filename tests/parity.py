"""Helpers shared by the GPU parity tests: device upload, sampled rows, and the
comparison rules.

Tolerances (max-abs): 1e-4 for fp32 inputs, 2e-2 for bf16 inputs, 6e-2 for fp8
key/value caches.  fp32 side outputs (LSE, raw block scores) are compared at
1e-4 absolute in every precision: they are fp32 sums of exactly representable
products, so their error is a few fp32 ulps of the logits.

Index rule: for a row whose oracle scores (sorted descending) have a relative
gap (s_k - s_{k+1})/s_k >= 1e-4 between the k-th and (k+1)-th candidate, the
GPU index list must equal the oracle's exactly.  Inside the near-tie band the
GPU set must contain every candidate scoring above s_k(1+1e-4), nothing below
s_k(1-1e-4), be duplicate-free, ascending, -1 padded and of size min(k, #cand).
"""
from __future__ import annotations

import numpy as np
import torch

TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}
SIDE_TOL = 1e-4
REL_TIE = 1e-4


def dev(arr: np.ndarray, dtype: str | None = None) -> torch.Tensor:
    """Stored numpy array -> CUDA tensor of the storage dtype."""
    if dtype == "bf16" or arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def sample_rows(T: int, every: int = 61, head: int = 128, tail: int = 64) -> np.ndarray:
    rows = set(range(min(T, head)))
    rows |= set(range(max(0, T - tail), T))
    rows |= set(range(0, T, every))
    for b in range(64, T, 64 * max(1, T // 64 // 8)):
        rows |= {b - 1, b}
    return np.array(sorted(r for r in rows if 0 <= r < T))


def check_index_row(gpu_row, oracle_row, ranked, kb, rel=REL_TIE):
    """Returns (ok, near_tie) for one (row, group)."""
    gpu_row = np.asarray(gpu_row)
    valid = gpu_row[gpu_row >= 0]
    n = min(kb, len(ranked))
    structural = (len(valid) == n and np.all(gpu_row[n:] == -1)
                  and np.all(np.diff(valid) > 0))
    if len(ranked) <= kb:
        return structural and np.array_equal(gpu_row, oracle_row), False
    sk, sk1 = ranked[kb - 1], ranked[kb]
    if sk > 0 and (sk - sk1) / sk >= rel:
        return np.array_equal(gpu_row, oracle_row), False
    return structural, True


def check_index_set(gpu_row, Sg_row, cand, kb, ranked, rel=REL_TIE):
    """Near-tie rule for a row: must hold everything clearly above s_k and
    nothing clearly below, all ids being candidates."""
    valid = np.asarray(gpu_row)[np.asarray(gpu_row) >= 0]
    if not np.all(np.isin(valid, cand)):
        return False
    sk = ranked[kb - 1]
    must = cand[Sg_row[cand] > sk * (1 + rel)]
    banned = cand[Sg_row[cand] < sk * (1 - rel)]
    return np.all(np.isin(must, valid)) and not np.any(np.isin(banned, valid))


def compare_indices(gpu_idx, ora, pos, kb, include_diag=False, block=64):
    """gpu_idx [Hkv, R, kb] vs the oracle dict of hybrid_block_rows.
    Returns (n_rows, n_near_tie, list of failures)."""
    Hkv = gpu_idx.shape[0]
    fails, ties = [], 0
    for g in range(Hkv):
        for r, t in enumerate(pos):
            ranked = ora["ranked"][g, r]
            ok, tie = check_index_row(gpu_idx[g, r], ora["idx"][g, r], ranked, kb)
            if tie:
                ties += 1
                last = t // block
                cand = np.arange(last + 1 if include_diag else last)
                ok = ok and check_index_set(gpu_idx[g, r], ora["Sg"][g, r], cand, kb, ranked)
            if not ok:
                fails.append((g, int(t), list(gpu_idx[g, r]), list(ora["idx"][g, r])))
    return Hkv * len(pos), ties, fails
