"""Helpers for the parity tests: run the fp64 oracle per head and compare the
library's outputs with it under the stated tolerances.

Tolerances (fixed in the tests, not tuned):
  * block and micro lists identical, except members of the symmetric
    difference whose oracle score lies within TIE_BAND of the row's cut
    (top-k / top-m), or rows whose oracle cumulative mass at the cut lies
    within TIE_BAND of p (top-p);
  * O: max |err| <= 1e-2 and mean |err| <= 1e-3 (float32 output);
  * LSE: max |err| <= 1e-3.
A bf16 O is compared against the oracle rounded to bf16 with the same
bounds plus half a bf16 ulp of the oracle value per store that rounded it
(two for a result updated in place).
"""

from __future__ import annotations

import math

import numpy as np
import torch

from oracle import bsa_oracle as O

TIE_BAND = 1e-5
O_MAX, O_MEAN, LSE_MAX = 1e-2, 1e-3, 1e-3


def head64(X: torch.Tensor, b: int, h: int) -> np.ndarray:
    return X[b, h].to(torch.float64).numpy()


def oracle_scores(Q, K, b, h, block, scale):
    q, k = head64(Q, b, h), head64(K, b, h)
    Qb, Kb = O.pool_means(q, block), O.pool_means(k, block)
    return Qb, Kb, O.pooled_scores(Qb, Kb, scale)


def rows_to_csr(rows_all: list[list[int]]):
    """Flatten a list of rows (over all (b, h, i)) into int32 CSR arrays."""
    lens = np.array([len(r) for r in rows_all], dtype=np.int64)
    row_ptr = np.zeros(len(rows_all) + 1, dtype=np.int32)
    row_ptr[1:] = np.cumsum(lens)
    col = np.array([j for r in rows_all for j in r], dtype=np.int32)
    if col.size == 0:
        col = np.zeros(1, dtype=np.int32)
    return torch.from_numpy(row_ptr), torch.from_numpy(col)


def compare_topk_rows(gpu_rows, ora_rows, S, k, forced_rows=None):
    """Returns the number of exempt rows; asserts every other row matches."""
    exempt = 0
    for i, (g, o) in enumerate(zip(gpu_rows, ora_rows)):
        gs, os_ = set(g), set(o)
        assert list(g) == sorted(gs), f"row {i} not ascending/unique: {g}"
        if gs == os_:
            continue
        forced = set(forced_rows[i]) if forced_rows is not None else set()
        order = O.rank_desc(S[i])
        thr = S[i][order[min(k, len(order)) - 1]] if k > 0 else math.inf
        bad = [j for j in gs ^ os_ if j in forced or abs(S[i][j] - thr) > TIE_BAND]
        assert not bad, f"row {i}: gpu {sorted(gs)} vs oracle {sorted(os_)}; non-tie {bad}"
        exempt += 1
    return exempt


def compare_topp_rows(gpu_rows, ora_rows, S, sizes, p, k_min, k_cap, forced_rows=None):
    """Top-p rows: a differing row is exempt when the oracle's cumulative mass
    next to the cut lies within TIE_BAND of p and the library kept the
    adjacent prefix, or when every differing block's probability is within
    a relative TIE_BAND of the cut probability."""
    exempt = 0
    for i, (g, o) in enumerate(zip(gpu_rows, ora_rows)):
        gs, os_ = set(g), set(o)
        assert list(g) == sorted(gs), f"row {i} not ascending/unique"
        if gs == os_:
            continue
        F = set(forced_rows[i]) if forced_rows is not None else set()
        P = O.size_weighted_softmax(S[i], sizes)
        order = O.rank_desc(P)
        c = np.cumsum(P[order])
        n = len(P)
        Lc = min(max(O.topp_length(P, p), k_min), k_cap, n)
        cut_amb = any(0 <= t < n and abs(c[t] - p) <= TIE_BAND for t in (Lc - 2, Lc - 1))
        prefix_ok = any(gs == set(order[:Lx].tolist()) | F
                        for Lx in (Lc - 1, Lc + 1) if 0 <= Lx <= n)
        if not (cut_amb and prefix_ok):
            cutP = P[order[Lc - 1]]
            bad = [j for j in gs ^ os_ if j in F or abs(P[j] - cutP) > TIE_BAND * cutP]
            assert not bad, f"row {i}: gpu {sorted(gs)} vs oracle {sorted(os_)}; non-tie {bad}"
        exempt += 1
    return exempt


def compare_o_lse(O_gpu: torch.Tensor, L_gpu: torch.Tensor, O_ref: np.ndarray,
                  L_ref: np.ndarray, what: str, bf16: bool = False, roundings: int = 1):
    """``roundings``: how many times a bf16 O was rounded on its way out (a
    result updated in place, e.g. rectified or merged into a bf16 O, is
    rounded once per store; each store adds at most half a bf16 ulp)."""
    Og = O_gpu.to(torch.float64).cpu().numpy()
    Lg = L_gpu.to(torch.float64).cpu().numpy()
    ninf_ref = np.isneginf(L_ref)
    assert np.array_equal(np.isneginf(Lg), ninf_ref), f"{what}: -inf LSE pattern differs"
    if bf16:
        ref_b = torch.from_numpy(np.ascontiguousarray(O_ref)).to(torch.bfloat16).double().numpy()
        half_ulp = roundings * np.abs(ref_b) * 2.0 ** -8
        err = np.abs(Og - O_ref)
        assert np.all(err <= O_MAX + half_ulp), f"{what}: O max err {err.max()}"
        assert float(np.mean(np.maximum(err - half_ulp, 0))) <= O_MEAN, f"{what}: O mean err"
    else:
        err = np.abs(Og - O_ref)
        assert err.max() <= O_MAX, f"{what}: O max err {err.max():.3e}"
        assert err.mean() <= O_MEAN, f"{what}: O mean err {err.mean():.3e}"
    fin = ~ninf_ref
    if fin.any():
        lerr = np.abs(Lg[fin] - L_ref[fin])
        assert lerr.max() <= LSE_MAX, f"{what}: LSE max err {lerr.max():.3e}"
    zero_rows = Og[ninf_ref]
    assert np.all(zero_rows == 0), f"{what}: empty rows must give O = 0"
    return float(np.abs(Og - O_ref).max()), float(np.abs(Og - O_ref).mean())
