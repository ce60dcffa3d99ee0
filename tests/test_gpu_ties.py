"""GPU selection on inputs with exact ties, compared with the oracle with NO
tie band: equal values must be broken exactly as the oracle breaks them.

The rules: top-k keeps the k key blocks of highest score, equal scores to the
lower block index (and +0 equals -0); top-p takes the smallest heaviest
prefix (HyperVAttention, section 2, Eq. 3), equal probabilities in index
order, then clamps the length; micro selection keeps the top-m candidates
by (score descending, code 4 beta + a ascending); the Lowe subset keeps the
largest ratios, equal ratios to the lower token index (HyperVAttention,
section 4.2, Eq. 6).  Ties are planted so that both sides see bit-equal
values: the scores are passed in directly, or the tokens that produce them
are copies of each other.  Other values are kept far apart (the tests check
it), so that float32 and float64 order them alike."""

import math
import sys

import numpy as np
import pytest
import torch

from oracle import bsa_oracle as O
from synth import VideoSpec, gen_qkv
import parity as PT

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import block_sparse_attention_pool_amd as bsa
else:  # collected on CPU, skipped by the marker
    bsa = None

DEV = "cuda:0"


def say(*a):
    print("[gpu-ties]", *a, file=sys.stderr, flush=True)


def _shape_like(B, H, N, d=64):
    return torch.empty((B, H, N, d), dtype=torch.bfloat16, device=DEV)


def _rows_by_head(rp, ci, nnz, B, H, nB):
    rows = bsa.csr_rows(rp, ci, nnz)
    return {(b, h): rows[(b * H + h) * nB:(b * H + h + 1) * nB] for b in range(B) for h in range(H)}


# ------------------------------------------------------------------ top-k

# score levels with many repeats; +0.0 and -0.0 are equal values
LEVELS = np.array([-1.5, -0.0, 0.0, 0.25, 1.0, 2.0], dtype=np.float32)


@pytest.mark.parametrize("nB,k,diag", [(40, 7, False), (40, 13, True), (40, 1, True),
                                       (700, 150, False), (700, 333, True), (2000, 1000, False),
                                       (2000, 71, True)])
def test_topk_exact_ties(nB, k, diag):
    B, H = 1, 2
    N = 64 * nB
    rng = np.random.default_rng(nB * 131 + k)
    S = LEVELS[rng.integers(0, len(LEVELS), size=(B, H, nB, nB))]
    say("topk ties", nB, k, diag)
    Sd = torch.from_numpy(S).to(DEV)
    rp, ci, nnz = bsa.bsa_select_blocks(Sd, _shape_like(B, H, N), mode="topk", k=k,
                                        force_diag=diag)
    torch.cuda.synchronize()
    got = _rows_by_head(rp, ci, nnz, B, H, nB)
    n_cut_ties = 0
    for h in range(H):
        S64 = S[0, h].astype(np.float64)
        want = O.select_rows(S64, N, 64, "topk", k=k, force_diag=diag)
        assert got[(0, h)] == want, f"head {h}: lists differ"
        for i in range(nB):
            order = O.rank_desc(S64[i])
            cut = S64[i][order[k - 1]]
            n_cut_ties += int((S64[i] == cut).sum() > 1)
    assert n_cut_ties > 0  # the cut falls inside a group of equal scores


def test_topk_signed_zeros_tie():
    # a row of -0.0 and +0.0 only: every score equal, the k lowest indices win
    nB, k = 64, 10
    S = np.where(np.arange(nB) % 2 == 0, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
    S = np.broadcast_to(S, (1, 1, nB, nB)).copy()
    rp, ci, nnz = bsa.bsa_select_blocks(torch.from_numpy(S).to(DEV), _shape_like(1, 1, 64 * nB),
                                        mode="topk", k=k)
    torch.cuda.synchronize()
    got = bsa.csr_rows(rp, ci, nnz)
    assert all(r == list(range(k)) for r in got)


# ------------------------------------------------------------------ top-p

def _topp_rows(levels, counts, nB, rng):
    """Rows made of groups of equal scores, placed at random positions."""
    base = np.concatenate([np.full(c, v, np.float32) for v, c in zip(levels, counts)])
    assert base.size == nB
    return np.stack([base[rng.permutation(nB)] for _ in range(nB)])


@pytest.mark.parametrize("p,k_min,k_cap,want_len", [(0.8, 1, 1000, 18), (0.99, 1, 10, 10),
                                                    (0.5, 1, 1000, 7), (0.3, 6, 1000, 6)])
def test_topp_exact_ties(p, k_min, k_cap, want_len):
    # 4 blocks of score 2, 8 of score 1, 20 of score 0, equal sizes: the
    # softmax masses are 4 e^2, 8 e, 20 over 71.30; p = 0.8 cuts 6 blocks
    # into the zeros (cumulative 0.7896 after 5, 0.8037 after 6), p = 0.5
    # cuts 3 blocks into the ones, the cap of 10 and the floor of 6 cut into
    # ties too; the cumulative sums sit >= 3e-3 away from p
    nB = 32
    N = 64 * nB
    rng = np.random.default_rng(int(p * 1000) + k_cap)
    rows = [_topp_rows([2.0, 1.0, 0.0], [4, 8, 20], nB, rng) for _ in range(2)]
    S = np.stack(rows)[None]
    say("topp ties", p, k_min, k_cap)
    rp, ci, nnz = bsa.bsa_select_blocks(torch.from_numpy(S).to(DEV), _shape_like(1, 2, N),
                                        mode="topp", p=p, k_min=k_min, k_cap=k_cap)
    torch.cuda.synchronize()
    got = _rows_by_head(rp, ci, nnz, 1, 2, nB)
    sizes = O.block_sizes(N, 64)
    for h in range(2):
        S64 = S[0, h].astype(np.float64)
        want = O.select_rows(S64, N, 64, "topp", p=p, k_min=k_min, k_cap=k_cap)
        assert got[(0, h)] == want, f"head {h}: lists differ"
        assert all(len(r) == want_len for r in want)
        for i in range(nB):
            P = O.size_weighted_softmax(S64[i], sizes)
            c = np.cumsum(P[O.rank_desc(P)])
            assert np.abs(c - p).min() > 2e-3   # the cut itself is unambiguous


def test_topp_uniform_row_keeps_the_lowest_indices():
    # 16 equal blocks, p = 0.9: 15 of them (ceil(14.4)), blocks 0..14
    nB = 16
    S = np.zeros((1, 1, nB, nB), np.float32)
    rp, ci, nnz = bsa.bsa_select_blocks(torch.from_numpy(S).to(DEV), _shape_like(1, 1, 64 * nB),
                                        mode="topp", p=0.9)
    torch.cuda.synchronize()
    assert all(r == list(range(15)) for r in bsa.csr_rows(rp, ci, nnz))


# ------------------------------------------------------------------ micro

def _tiled(X, palette_idx, tile):
    """X [B, H, N, d]: token block t (of `tile` tokens) becomes a copy of
    palette block palette_idx[t] (taken from X itself)."""
    Y = X.clone()
    for t, src in enumerate(palette_idx):
        Y[:, :, tile * t:tile * (t + 1)] = X[:, :, tile * src:tile * (src + 1)]
    return Y


@pytest.mark.parametrize("grid,d,m", [((4, 16, 16), 64, 8), ((3, 8, 16), 128, 20),
                                      ((2, 8, 16), 128, 1000)])
def test_micro_exact_ties(grid, d, m):
    spec = VideoSpec(1, 2, d, grid, 160)
    Q, K, _ = gen_qkv(spec)
    B, H, N, _ = Q.shape
    nB, nT = O.n_blocks(N, 64), O.n_blocks(N, 16)
    rng = np.random.default_rng(161)
    # key tiles copies of 3 palette tiles, query sub-tiles copies of 2
    K = _tiled(K, rng.integers(0, 3, size=nT), 16)
    Q = _tiled(Q, rng.integers(0, 2, size=nT), 16)
    scale = 1 / math.sqrt(d)
    say("micro ties", grid, d, m)
    rows, mo = {}, {}
    for h in range(H):
        q, k = PT.head64(Q, 0, h), PT.head64(K, 0, h)
        S = O.pooled_scores(O.pool_means(q, 64), O.pool_means(k, 64), scale)
        rows[h] = O.select_rows(S, N, 64, "topk", k=1, force_diag=True)
        Qt, Kt = O.pool_means(q, 16), O.pool_means(k, 16)
        sig = sorted({scale * float(Qt[a] @ Kt[b]) for a in range(nT) for b in range(nT)})
        assert len(sig) <= 6 and np.min(np.diff(sig)) > 1e-3, "distinct scores too close"
        mo[h] = [O.micro_select_row(Qt, Kt, rows[h][i], i, N, 64, 16, scale, m)
                 for i in range(nB)]
    rp, ci = PT.rows_to_csr([r for h in range(H) for r in rows[h]])
    Qd, Kd = Q.to(DEV), K.to(DEV)
    sc = bsa.bsa_score_blocks(Qd, Kd, scores=False, micro=16)
    mrp, mci, mnnz = bsa.bsa_select_blocks(
        None, Qd, mode="micro",
        micro=dict(m=m, scale=scale, macro=(rp.to(DEV), ci.to(DEV)),
                   qpool16=sc["qpool16"], kpool16=sc["kpool16"]))
    torch.cuda.synchronize()
    got = _rows_by_head(mrp, mci, mnnz, 1, H, nB)
    for h in range(H):
        assert got[(0, h)] == mo[h], f"head {h}: micro lists differ"


# ------------------------------------------------------------- Lowe subset

@pytest.mark.parametrize("n_sub", [44, 17, 3, 61])
def test_lowe_subset_exact_ties(n_sub):
    # a 2 x 8 x 8 lattice in cells of 1 x 4 x 4 (8 cells of 16 tokens); every
    # token of a cell is a copy of one of two tokens, so 8 tokens share each
    # ratio, and a subset size that is not a multiple of 8 cuts into a group
    # of equal ratios: its lowest token indices must be taken
    thw, cell, window = (2, 8, 8), (1, 4, 4), (2, 2, 2)
    spec = VideoSpec(1, 1, 64, thw, 170)
    X, _, _ = gen_qkv(spec)
    N = spec.N
    T, Hg, W = thw
    src = np.zeros(N, dtype=np.int64)
    for t in range(T):
        for y in range(Hg):
            for x in range(W):
                n = (t * Hg + y) * W + x
                src[n] = (t * Hg + (y // 4) * 4) * W + (x // 4) * 4 + (x % 2)  # one of the cell's first two tokens
    X = X[:, :, torch.from_numpy(src)].contiguous()
    Xd = X.to(DEV)
    say("lowe ties", n_sub)
    _, mu, _ = bsa.bsa_local_window_cluster(Xd, thw, cell, window, 2)
    rho, sub = bsa.bsa_lowe_ratio_subset(Xd, mu, thw, cell, window, n_sub=n_sub)
    torch.cuda.synchronize()
    ro = O.lowe_ratios(X[0, 0].double().numpy(), thw, cell, window, mu[0, 0].double().cpu().numpy())
    levels = np.unique(ro)
    # float32 ratios carry about 1e-5 of error: distinct levels 3e-4 apart
    # are ordered alike on both sides
    assert len(levels) > 2 and np.min(np.diff(levels)) > 3e-4, "distinct ratios too close"
    rg = rho[0, 0].double().cpu().numpy()
    for lv in levels:  # equal ratios on the GPU too, bit for bit
        assert np.unique(rg[ro == lv]).size == 1
    want = O.lowe_subset(ro, n_sub)
    assert sub[0, 0].cpu().tolist() == want.tolist()
