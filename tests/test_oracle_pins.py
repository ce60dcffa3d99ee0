"""Pins of the fp64 oracle against facts that do not come from the oracle:
hand-worked fixtures, closed forms, invariants, library special cases and
brute force on tiny inputs.  CPU only."""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import bsa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# --------------------------------------------------------------- pooling / score

def test_golden_pooled_score():
    g = _load("pooled_score.json")
    Q, K = np.array(g["Q"], float), np.array(g["K"], float)
    Qb, Kb = O.pool_means(Q, g["b"]), O.pool_means(K, g["b"])
    np.testing.assert_array_equal(Qb, g["Qbar"])
    np.testing.assert_array_equal(Kb, g["Kbar"])
    np.testing.assert_array_equal(O.pooled_scores(Qb, Kb, g["scale"]), g["S"])


def test_pooled_score_is_mean_of_token_logits():
    # bilinearity: <mean q, mean k> = mean over all token pairs of <q, k>,
    # written out with explicit loops over tokens
    N, b, d, s = 150, 64, 8, 0.3
    Q, K = _rand(1, N, d), _rand(2, N, d)
    S = O.pooled_scores(O.pool_means(Q, b), O.pool_means(K, b), s)
    nB = O.n_blocks(N, b)
    for i in range(nB):
        for j in range(nB):
            ti = range(b * i, min(b * i + b, N))
            tj = range(b * j, min(b * j + b, N))
            acc = 0.0
            for t in ti:
                for tau in tj:
                    acc += s * sum(Q[t, c] * K[tau, c] for c in range(d))
            assert abs(S[i, j] - acc / (len(ti) * len(tj))) < 1e-12


def test_pool_constant_blocks_and_ragged_tail():
    N, b, d = 64 * 3 + 5, 64, 4
    X = np.zeros((N, d))
    for j in range(4):
        X[64 * j:64 * j + 64] = j + 0.5
    P = O.pool_means(X, b)
    np.testing.assert_array_equal(P[:, 0], [0.5, 1.5, 2.5, 3.5])
    # tail mean uses only the 5 valid tokens
    X2 = np.ones((N, d))
    X2[-5:] = 7.0
    assert O.pool_means(X2, b)[-1, 0] == 7.0
    np.testing.assert_array_equal(O.block_sizes(N, b), [64, 64, 64, 5])


# ------------------------------------------------------------------- top-k

def test_topk_is_best_subset_by_brute_force():
    rng = np.random.default_rng(3)
    for trial in range(30):
        n = int(rng.integers(2, 10))
        k = int(rng.integers(1, n + 1))
        row = rng.standard_normal(n)
        best = max(itertools.combinations(range(n), k),
                   key=lambda c: sum(row[j] for j in c))
        assert O.topk_set(row, k) == set(best)


def test_topk_ties_go_to_lower_index():
    row = np.array([1.0, 3.0, 3.0, 2.0, 3.0])
    assert O.topk_set(row, 1) == {1}
    assert O.topk_set(row, 2) == {1, 2}
    assert O.topk_set(row, 3) == {1, 2, 4}
    assert O.topk_set(row, 4) == {1, 2, 3, 4}
    assert O.topk_set(row, 0) == set()


def test_select_rows_topk_with_diagonal_union():
    S = np.array([[0.0, 5.0, 4.0], [9.0, 0.0, 1.0], [3.0, 2.0, 1.0]])
    rows = O.select_rows(S, 3 * 64, 64, "topk", k=1, force_diag=True)
    assert rows == [[0, 1], [0, 1], [0, 2]]


# ------------------------------------------------------------------- top-p

def test_golden_topp():
    g = _load("topp_size_weighted.json")
    for c in g["cases"]:
        P = O.size_weighted_softmax(np.array(c["scores"]), np.array(c["sizes"], float))
        np.testing.assert_allclose(P, c["P"], atol=c.get("P_tol", 1e-12))
        for p, want in c["by_p"].items():
            got = O.topp_set(np.array(c["scores"]), np.array(c["sizes"], float),
                             float(p), k_min=1)
            assert got == set(want), (c["note"], p)


def test_topp_matches_brute_force_smallest_set():
    # TopP = smallest set whose mass is at least p; among sets of that size the
    # heaviest (unique for distinct masses)
    rng = np.random.default_rng(4)
    for trial in range(40):
        n = int(rng.integers(1, 9))
        row = rng.standard_normal(n) * 2
        sizes = rng.integers(1, 65, size=n).astype(float)
        p = float(rng.uniform(0.05, 0.99))
        P = sizes * np.exp(row)
        P /= P.sum()
        best = None
        for L in range(1, n + 1):
            sets = [c for c in itertools.combinations(range(n), L)
                    if sum(P[j] for j in c) >= p]
            if sets:
                best = max(sets, key=lambda c: sum(P[j] for j in c))
                break
        assert O.topp_set(row, sizes, p) == set(best)


def test_topp_uniform_16_blocks_keeps_15():
    # 16 equal blocks at p = 0.9: 14 blocks hold 0.875 < 0.9, 15 hold 0.9375
    assert len(O.topp_set(np.zeros(16), np.full(16, 64.0), 0.9)) == 15


def test_topp_equal_sizes_is_plain_softmax():
    row = _rand(5, 40)
    np.testing.assert_allclose(O.size_weighted_softmax(row, np.full(40, 64.0)),
                               scipy.special.softmax(row), rtol=1e-13)


def test_topp_clamps_to_kmin_and_cap():
    row = np.array([10.0, 0.0, 0.0, 0.0, 0.0])
    sz = np.full(5, 64.0)
    assert O.topp_set(row, sz, 0.5) == {0}
    assert len(O.topp_set(row, sz, 0.5, k_min=3)) == 3
    flat = np.zeros(5)
    assert len(O.topp_set(flat, sz, 0.99, k_cap=2)) == 2


# ------------------------------------------------------------- static mask

def test_golden_static_window_anchor():
    g = _load("static_window_anchor.json")
    for c in g["cases"]:
        nB = O.n_blocks(c["N"], c["b"])
        rows = [sorted(O.window_anchor_set(
            c["N"], c["b"], i, c["frame_tokens"], c["window_frames"],
            c["n_anchors"], c["anchor_offset"])) for i in range(nB)]
        assert rows == c["rows"], c["note"]


def test_static_window_matches_token_level_brute_force():
    # window rule at block level == "some token pair within r frames"
    for (T, Hg, Wg, b, r) in [(5, 3, 5, 8, 1), (7, 2, 3, 16, 2), (4, 4, 4, 64, 0),
                              (6, 3, 7, 10, 1)]:
        N, ft = T * Hg * Wg, Hg * Wg
        nB = O.n_blocks(N, b)
        for i in range(nB):
            got = O.window_anchor_set(N, b, i, ft, r, 0, 0)
            want = set()
            for j in range(nB):
                for t in range(b * i, min(b * i + b, N)):
                    if any(abs(t // ft - tau // ft) <= r
                           for tau in range(b * j, min(b * j + b, N))):
                        want.add(j)
                        break
            assert got == want


def test_static_anchor_rotation_and_density_at_long_horizon():
    # 126 x 30 x 52 tokens, 64-blocks, 1-frame window, 4 anchors
    N, b, ft = 126 * 30 * 52, 64, 30 * 52
    nB = O.n_blocks(N, b)
    assert nB == 3072
    a0 = O.window_anchor_set(N, b, 1500, ft, 0, 4, 0) - \
        O.window_anchor_set(N, b, 1500, ft, 0, 0, 0)
    assert a0 <= {0, 768, 1536, 2304}
    anchors = {(5 + a * 768) % nB for a in range(4)}
    assert anchors <= O.window_anchor_set(N, b, 100, ft, 1, 4, 5)
    # average row length of the literal 1-frame window + 4 anchors
    tot = sum(len(O.window_anchor_set(N, b, i, ft, 1, 4, 5)) for i in range(0, nB, 7))
    avg = tot / len(range(0, nB, 7))
    assert 75 < avg < 82  # about 2.5% of 3072 blocks


# ------------------------------------------------ MOD patterns and block 128

def _basis_C(n):
    """The 2n-1 parallel-diagonal basis matrices: numpy's eye with a diagonal
    offset puts ones at (i, i + offset)."""
    return {k - n + 1: np.eye(n, k=k - n + 1, dtype=np.int64) for k in range(2 * n - 1)}


def test_parallel_diagonal_basis_partitions_the_block_map():
    n = 7
    C = _basis_C(n)
    assert len(C) == 2 * n - 1 and all(M.sum() > 0 for M in C.values())
    np.testing.assert_array_equal(sum(C.values()), np.ones((n, n), dtype=np.int64))


def test_pattern_set_equals_union_of_basis_matrices():
    rng = np.random.default_rng(40)
    for n in (1, 5, 13):
        C = _basis_C(n)
        for trial in range(6):
            diags = sorted(set(rng.integers(-(n + 1), n + 2, size=3).tolist()))
            cols = sorted(set(rng.integers(0, n, size=2).tolist()))
            M = np.zeros((n, n), dtype=np.int64)
            for dlt in diags:
                if dlt in C:
                    M |= C[dlt]
            for j in cols:
                D = np.zeros((n, n), dtype=np.int64)
                D[:, j] = 1          # vertical basis: one key column for every query
                M |= D
            for i in range(n):
                assert O.pattern_set(n, i, diags, cols) == set(np.nonzero(M[i])[0].tolist())
    with pytest.raises(ValueError):
        O.pattern_set(4, 0, (), (4,))


def test_pattern_pin_catches_a_flipped_offset(monkeypatch):
    real = O.pattern_set
    monkeypatch.setattr(O, "pattern_set",
                        lambda n, i, diagonals=(), columns=(): real(n, i, [-x for x in diagonals],
                                                                   columns))
    n, C = 6, _basis_C(6)
    assert any(O.pattern_set(n, i, [2], []) != set(np.nonzero(C[2][i])[0].tolist())
               for i in range(n))


def test_intra_frame_block_diagonal_matches_token_level_definition():
    # block (i, j) is in the block-diagonal support iff some query token of i
    # and key token of j share a frame: the window of radius 0, no anchors
    N, ft = 64 * 7 + 13, 150
    for b in (64, 128):
        nB = O.n_blocks(N, b)
        for i in range(nB):
            fi = {int(t) // ft for t in O.block_tokens(N, b, i)}
            want = {j for j in range(nB)
                    if fi & {int(t) // ft for t in O.block_tokens(N, b, j)}}
            assert O.window_anchor_set(N, b, i, ft, 0, 0, 0) == want


def test_select_rows_with_patterns_is_a_union():
    N, b, s = 64 * 9 + 7, 64, 0.3
    Q, K = _rand(41, N, 8), _rand(42, N, 8)
    S = O.pooled_scores(O.pool_means(Q, b), O.pool_means(K, b), s)
    pats = dict(diagonals=[-3, 0, 4], columns=[1, 9])
    base = O.select_rows(S, N, b, "topk", k=2)
    got = O.select_rows(S, N, b, "topk", k=2, patterns=pats)
    for i in range(len(base)):
        assert set(got[i]) == set(base[i]) | O.pattern_set(len(base), i, **pats)


def test_block128_expansion_keeps_the_token_support():
    N, d = 128 * 4 + 70, 8          # 5 blocks of 128 (tail 70), 10 blocks of 64 (tail 6)
    s = 1 / math.sqrt(d)
    Q, K, V = _rand(43, N, d), _rand(44, N, d), _rand(45, N, d)
    S = O.pooled_scores(O.pool_means(Q, 128), O.pool_means(K, 128), s)
    rows128 = O.select_rows(S, N, 128, "topk", k=2, patterns=dict(diagonals=[1]))
    rows64 = O.expand_rows(rows128, N, 128, 64)
    assert len(rows64) == O.n_blocks(N, 64) == 10
    # token-level supports are identical for every query token
    for t in range(N):
        sup128 = {int(x) for J in rows128[t // 128] for x in O.block_tokens(N, 128, J)}
        sup64 = {int(x) for j in rows64[t // 64] for x in O.block_tokens(N, 64, j)}
        assert sup128 == sup64
    Oa, La = O.block_sparse_attention(Q, K, V, rows128, 128, s)
    Ob, Lb = O.block_sparse_attention(Q, K, V, rows64, 64, s)
    np.testing.assert_allclose(Oa, Ob, atol=1e-12)
    np.testing.assert_allclose(La, Lb, atol=1e-12)


def test_pooled_score_at_block128_is_mean_of_token_logits():
    N, b, d, s = 128 * 2 + 33, 128, 6, 0.4
    Q, K = _rand(46, N, d), _rand(47, N, d)
    S = O.pooled_scores(O.pool_means(Q, b), O.pool_means(K, b), s)
    for i in range(O.n_blocks(N, b)):
        for j in range(O.n_blocks(N, b)):
            ti, tj = O.block_tokens(N, b, i), O.block_tokens(N, b, j)
            want = sum(s * float(Q[a] @ K[c]) for a in ti for c in tj) / (len(ti) * len(tj))
            assert abs(S[i, j] - want) < 1e-11


# --------------------------------------------------------------- attention

def test_golden_attention_two_keys():
    g = _load("attention_two_keys.json")
    Ov, L = O.attend(np.array(g["q"]), np.array(g["K"]), np.array(g["V"]), g["scale"])
    np.testing.assert_allclose(Ov, g["O"], atol=1e-12)
    np.testing.assert_allclose(L, g["LSE"], atol=1e-12)


def test_all_blocks_equals_torch_sdpa_fp64():
    N, d, b = 200, 16, 64
    s = 1 / math.sqrt(d)
    Q, K, V = _rand(6, N, d), _rand(7, N, d), _rand(8, N, d)
    rows = [list(range(O.n_blocks(N, b)))] * O.n_blocks(N, b)
    Ov, L = O.block_sparse_attention(Q, K, V, rows, b, s)
    tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (Q, K, V))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=s)
    np.testing.assert_allclose(Ov, ref[0, 0].numpy(), atol=1e-12)
    lse = torch.logsumexp(s * (tq[0, 0] @ tk[0, 0].T), dim=-1).numpy()
    np.testing.assert_allclose(L, lse, atol=1e-12)


def test_block_mask_equals_masked_dense_softmax():
    # restricted attention == softmax(sQK^T + M)V with M in {0,-inf}, built
    # by torch on the full matrix
    N, d, b = 150, 8, 64
    s = 0.37
    Q, K, V = _rand(9, N, d), _rand(10, N, d), _rand(11, N, d)
    rows = [[0, 2], [1], [0, 1, 2]]
    Ov, L = O.block_sparse_attention(Q, K, V, rows, b, s)
    M = torch.full((N, N), -math.inf, dtype=torch.float64)
    for i, sel in enumerate(rows):
        for j in sel:
            M[b * i:b * i + b, b * j:b * j + b] = 0.0
    logits = s * torch.from_numpy(Q) @ torch.from_numpy(K).T + M
    ref = torch.softmax(logits, -1) @ torch.from_numpy(V)
    np.testing.assert_allclose(Ov, ref.numpy(), atol=1e-12)
    np.testing.assert_allclose(L, torch.logsumexp(logits, -1).numpy(), atol=1e-12)


def test_zero_query_gives_mean_of_values():
    N, d, b = 130, 4, 64
    Q = np.zeros((N, d))
    K, V = _rand(12, N, d), _rand(13, N, d)
    rows = [[1, 2], [0], [2]]
    Ov, L = O.block_sparse_attention(Q, K, V, rows, b, 0.5)
    np.testing.assert_allclose(Ov[0], V[64:130].mean(0), atol=1e-13)
    np.testing.assert_allclose(L[0], math.log(66), atol=1e-13)
    np.testing.assert_allclose(Ov[129], V[128:130].mean(0), atol=1e-13)
    np.testing.assert_allclose(L[129], math.log(2), atol=1e-13)


def test_single_key_support():
    N, d, b = 65, 4, 64
    Q, K, V = _rand(14, N, d), _rand(15, N, d), _rand(16, N, d)
    Ov, L = O.block_sparse_attention(Q, K, V, [[1], [1]], b, 0.5)
    np.testing.assert_allclose(Ov, np.repeat(V[64:65], N, 0), atol=1e-14)
    np.testing.assert_allclose(L, 0.5 * Q @ K[64], atol=1e-13)


def test_empty_row_gives_zero_and_neg_inf():
    Q, K, V = _rand(17, 70, 4), _rand(18, 70, 4), _rand(19, 70, 4)
    Ov, L = O.block_sparse_attention(Q, K, V, [[], [0]], 64, 0.5)
    assert np.all(Ov[:64] == 0) and np.all(np.isneginf(L[:64]))
    assert np.all(np.isfinite(L[64:]))


# ------------------------------------------------------------------- merge

def test_merge_of_disjoint_supports_equals_union():
    rng = np.random.default_rng(20)
    N, d, s = 90, 6, 0.4
    Q, K, V = _rand(21, N, d), _rand(22, N, d), _rand(23, N, d)
    for trial in range(10):
        perm = rng.permutation(N)
        cut = int(rng.integers(1, N))
        S1, S2 = np.sort(perm[:cut]), np.sort(perm[cut:])
        O1, L1 = O.attend(Q, K[S1], V[S1], s)
        O2, L2 = O.attend(Q, K[S2], V[S2], s)
        Om, Lm = O.lse_merge(O1, L1, O2, L2)
        Ou, Lu = O.attend(Q, K, V, s)
        np.testing.assert_allclose(Om, Ou, atol=1e-12)
        np.testing.assert_allclose(Lm, Lu, atol=1e-12)


def test_merge_with_empty_parts():
    O1, L1 = _rand(24, 3, 4), np.array([0.3, -1.0, 2.0])
    Oe, Le = np.zeros((3, 4)), np.full(3, -math.inf)
    Om, Lm = O.lse_merge(O1, L1, Oe, Le)
    np.testing.assert_allclose(Om, O1, atol=1e-15)
    np.testing.assert_allclose(Lm, L1, atol=1e-15)
    Om, Lm = O.lse_merge(Oe, Le, O1, L1)
    np.testing.assert_allclose(Om, O1, atol=1e-15)
    Om, Lm = O.lse_merge(Oe, Le, Oe, Le)
    assert np.all(Om == 0) and np.all(np.isneginf(Lm))


# ------------------------------------------------------------------- micro

def test_micro_score_is_mean_of_tile_logits():
    N, b, u, d, s = 140, 64, 16, 4, 0.25
    Q, K = _rand(25, N, d), _rand(26, N, d)
    Qt, Kt = O.pool_means(Q, u), O.pool_means(K, u)
    cand = O.micro_candidates(Qt, Kt, [1], 0, N, b, u, s)
    codes = {c for _, c in cand}
    # omitted blocks are 0 and 2 -> key tiles 0..3 and 8 (tile 8 = tokens 128..139)
    assert {c // 4 for c in codes} == {0, 1, 2, 3, 8}
    assert {c % 4 for c in codes} == {0, 1, 2, 3}
    for sig, c in cand:
        a, beta = c % 4, c // 4
        qi = range(16 * a, 16 * a + 16)
        kj = range(16 * beta, min(16 * beta + 16, N))
        want = np.mean([s * Q[t] @ K[tau] for t in qi for tau in kj])
        assert abs(sig - want) < 1e-12


def test_micro_select_order_and_ties():
    Qt = np.ones((8, 1))
    Kt = np.array([[3.0], [1.0], [3.0], [2.0], [9.0], [9.0], [9.0], [9.0]])
    # macro keeps block 1 (tiles 4..7), so candidates are tiles 0..3
    got = O.micro_select_row(Qt, Kt, [1], 0, 128, 64, 16, 1.0, 3)
    # tiles 0 and 2 score 3 for every sub-tile a; ranked by code 4*beta+a:
    # (0,a=0)=0,(0,1)=1,(0,2)=2 win; output sorted by (a, beta)
    assert got == [0, 1, 2]
    got = O.micro_select_row(Qt, Kt, [1], 0, 128, 64, 16, 1.0, 6)
    assert got == [0, 8, 1, 9, 2, 3]


def test_macro_plus_all_micro_equals_full_attention():
    N, b, u, d = 64 * 4 + 20, 64, 16, 8
    s = 1 / math.sqrt(d)
    Q, K, V = _rand(27, N, d), _rand(28, N, d), _rand(29, N, d)
    S = O.pooled_scores(O.pool_means(Q, b), O.pool_means(K, b), s)
    rows = O.select_rows(S, N, b, "topk", k=2, force_diag=True)
    Qt, Kt = O.pool_means(Q, u), O.pool_means(K, u)
    mrows = [O.micro_select_row(Qt, Kt, rows[i], i, N, b, u, s, 10 ** 6)
             for i in range(len(rows))]
    Om, Lm = O.block_sparse_attention(Q, K, V, rows, b, s)
    Ou, Lu = O.micro_attention(Q, K, V, mrows, b, u, s)
    Of, Lf = O.lse_merge(Om, Lm, Ou, Lu)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x)[None, None] for x in (Q, K, V)), scale=s)[0, 0].numpy()
    np.testing.assert_allclose(Of, ref, atol=1e-12)
    np.testing.assert_allclose(
        Lf, scipy.special.logsumexp(s * Q @ K.T, axis=1), atol=1e-12)


# ------------------------------------------------------ local-window clustering

def _brute_force_clustering(X, thw, cell, window, iters):
    """Algorithm 2 with explicit loops over tokens, cells and dimensions."""
    T, H, W = thw
    K = [-(-thw[a] // cell[a]) for a in range(3)]
    w = [min(window[a], K[a]) for a in range(3)]
    ncell = K[0] * K[1] * K[2]
    mu = []
    for ut in range(K[0]):
        for uh in range(K[1]):
            for uw in range(K[2]):
                c = [min(u * cell[i] + cell[i] // 2, thw[i] - 1) for i, u in enumerate((ut, uh, uw))]
                mu.append(list(X[(c[0] * H + c[1]) * W + c[2]]))
    assign = [0] * (T * H * W)
    counts = [0] * ncell
    for _ in range(iters):
        for t in range(T):
            for h in range(H):
                for x in range(W):
                    g = (t // cell[0], h // cell[1], x // cell[2])
                    best, best_u = None, None
                    s0 = [min(max(g[i] - w[i] // 2, 0), K[i] - w[i]) for i in range(3)]
                    for vt in range(s0[0], s0[0] + w[0]):
                        for vh in range(s0[1], s0[1] + w[1]):
                            for vw in range(s0[2], s0[2] + w[2]):
                                u = (vt * K[1] + vh) * K[2] + vw
                                dd = sum((X[(t * H + h) * W + x][e] - mu[u][e]) ** 2
                                         for e in range(X.shape[1]))
                                if best is None or dd < best or (dd == best and u < best_u):
                                    best, best_u = dd, u
                    assign[(t * H + h) * W + x] = best_u
        counts = [0] * ncell
        sums = [[0.0] * X.shape[1] for _ in range(ncell)]
        for n, u in enumerate(assign):
            counts[u] += 1
            for e in range(X.shape[1]):
                sums[u][e] += X[n][e]
        for u in range(ncell):
            if counts[u]:
                mu[u] = [v / counts[u] for v in sums[u]]
    return np.array(assign), np.array(mu), np.array(counts)


@pytest.mark.parametrize("thw,cell,window,iters", [((3, 5, 7), (1, 2, 3), (2, 2, 2), 1),
                                                   ((4, 6, 5), (2, 2, 2), (3, 2, 3), 3),
                                                   ((2, 7, 9), (2, 3, 2), (1, 3, 3), 2)])
def test_clustering_matches_brute_force(thw, cell, window, iters):
    X = _rand(70, thw[0] * thw[1] * thw[2], 3)
    a, mu, c = O.local_window_clustering(X, thw, cell, window, iters)
    ab, mub, cb = _brute_force_clustering(X, thw, cell, window, iters)
    np.testing.assert_array_equal(a, ab)
    np.testing.assert_allclose(mu, mub, atol=1e-12)
    np.testing.assert_array_equal(c, cb)


def test_clustering_with_a_global_window_is_lloyd_kmeans():
    # a window covering the whole grid searches every centroid: Algorithm 2
    # is then plain k-means (Lloyd) from the cell-centre initialisation
    from sklearn.cluster import KMeans
    thw, cell, iters = (3, 8, 8), (3, 4, 4), 4
    X = _rand(71, 3 * 8 * 8, 5) + np.repeat(np.arange(3 * 8 * 8)[:, None] // 48, 5, axis=1)
    a, mu, c = O.local_window_clustering(X, thw, cell, (9, 9, 9), iters)
    init = np.stack([X[(min(ut * 3 + 1, 2) * 8 + (uh * 4 + 2)) * 8 + (uw * 4 + 2)]
                     for ut in range(1) for uh in range(2) for uw in range(2)])
    # no cluster empties on these inputs, so the library's relocation of
    # empty clusters never applies
    assert np.all(c > 0)
    km = KMeans(n_clusters=4, init=init, n_init=1, max_iter=iters, tol=0.0,
                algorithm="lloyd").fit(X)
    np.testing.assert_allclose(mu, km.cluster_centers_, atol=1e-10)


def test_clustering_cell_constant_tokens_stay_put():
    thw, cell = (4, 6, 6), (2, 3, 3)
    T, H, W = thw
    rng = np.random.default_rng(72)
    centres = rng.standard_normal((8, 4)) * 10
    X = np.zeros((T * H * W, 4))
    for t in range(T):
        for h in range(H):
            for x in range(W):
                X[(t * H + h) * W + x] = centres[((t // 2) * 2 + h // 3) * 2 + x // 3]
    a, mu, c = O.local_window_clustering(X, thw, cell, (2, 2, 2), 3)
    np.testing.assert_array_equal(a, [((t // 2) * 2 + h // 3) * 2 + x // 3
                                      for t in range(T) for h in range(H) for x in range(W)])
    np.testing.assert_allclose(mu, centres, atol=1e-12)
    np.testing.assert_array_equal(c, np.full(8, 18))


def test_cluster_permutation_properties():
    rng = np.random.default_rng(73)
    a = rng.integers(0, 9, size=200)
    a[a == 4] = 5                       # an empty cluster
    perm, off = O.cluster_permutation(a, 9)
    assert sorted(perm.tolist()) == list(range(200))           # a permutation
    assert off[0] == 0 and off[-1] == 200 and off[4] == off[5]
    for u in range(9):
        seg = perm[off[u]:off[u + 1]]
        assert np.all(a[seg] == u)                             # contiguous clusters
        assert np.all(np.diff(seg) > 0)                        # original order kept
        assert len(seg) == np.sum(a == u)


def test_cluster_topp_on_block_means_is_block_topp():
    # 64-token blocks are clusters whose centroids are the block means and
    # whose sizes are the valid counts: the cluster rule is the block rule
    N, d, s = 64 * 9 + 30, 8, 0.35
    Q, K = _rand(74, N, d), _rand(75, N, d)
    Qb, Kb = O.pool_means(Q, 64), O.pool_means(K, 64)
    S = O.pooled_scores(Qb, Kb, s)
    for p, kmin, kcap in ((0.9, 1, None), (0.5, 3, 6), (0.99, 1, 4)):
        rows = O.cluster_topp_rows(Qb, Kb, O.block_sizes(N, 64), s, p, kmin, kcap)
        assert rows == O.select_rows(S, N, 64, "topp", p=p, k_min=kmin, k_cap=kcap)


def test_cluster_topp_ignores_empty_clusters_unless_forced():
    mu_q = np.array([[1.0, 0.0]])
    mu_k = np.array([[1.0, 0.0], [5.0, 0.0], [0.0, 1.0]])
    sizes = np.array([10, 0, 10])          # key cluster 1 is empty
    rows = O.cluster_topp_rows(mu_q, mu_k, sizes, 1.0, 0.6)
    assert rows == [[0]]                   # e^1 * 10 of (e^1 + 1) * 10: 0.73 >= 0.6
    rows = O.cluster_topp_rows(mu_q, mu_k, sizes, 1.0, 0.6, k_min=3)
    assert rows == [[0, 1, 2]]


def test_cluster_attention_all_clusters_is_full_attention():
    N, d = 150, 8
    s = 1 / math.sqrt(d)
    Q, K, V = _rand(76, N, d), _rand(77, N, d), _rand(78, N, d)
    rng = np.random.default_rng(79)
    aq, ak = rng.integers(0, 7, N), rng.integers(0, 11, N)
    pq, oq = O.cluster_permutation(aq, 7)
    pk, ok = O.cluster_permutation(ak, 11)
    Oc, Lc = O.cluster_block_attention(Q, K, V, pq, oq, pk, ok, [list(range(11))] * 7, s)
    tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (Q, K, V))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=s)[0, 0].numpy()
    np.testing.assert_allclose(Oc, ref, atol=1e-12)
    np.testing.assert_allclose(Lc, scipy.special.logsumexp(s * Q @ K.T, axis=1), atol=1e-12)


def test_cluster_attention_on_block_clusters_is_block_sparse_attention():
    # clusters = 64-token blocks in order: Eq. 4 is block-sparse attention
    N, d, b = 64 * 4 + 17, 6, 64
    s = 0.4
    Q, K, V = _rand(80, N, d), _rand(81, N, d), _rand(82, N, d)
    a = np.arange(N) // b
    perm, off = O.cluster_permutation(a, 5)
    assert np.array_equal(perm, np.arange(N))
    rows = [[0, 2], [1], [], [0, 3, 4], [4]]
    Oc, Lc = O.cluster_block_attention(Q, K, V, perm, off, perm, off, rows, s)
    Ob, Lb = O.block_sparse_attention(Q, K, V, rows, b, s)
    np.testing.assert_allclose(Oc, Ob, atol=1e-13)
    np.testing.assert_array_equal(np.isneginf(Lc), np.isneginf(Lb))
    fin = ~np.isneginf(Lb)
    np.testing.assert_allclose(Lc[fin], Lb[fin], atol=1e-13)
    # tile work: query tiles x key tiles of the selected clusters
    assert O.cluster_tile_pairs(off, off, rows) == 1 * 2 + 1 * 1 + 0 + 1 * 3 + 1 * 1


def test_clustering_pin_catches_an_unclipped_window(monkeypatch):
    monkeypatch.setattr(O, "window_start", lambda g, w, K: max(g - w // 2, 0))
    thw, cell, window = (4, 6, 5), (2, 2, 2), (3, 2, 3)
    X = _rand(70, 4 * 6 * 5, 3)
    with pytest.raises(Exception):
        a, mu, c = O.local_window_clustering(X, thw, cell, window, 3)
        ab, mub, cb = _brute_force_clustering(X, thw, cell, window, 3)
        np.testing.assert_array_equal(a, ab)


# ------------------------------------------------------- pooled rectification

def _blockwise_constant_keys(seed, N, b, d):
    """Keys equal within every block (each block's keys are its first key)."""
    K = _rand(seed, N, d)
    for j in range(O.n_blocks(N, b)):
        t = O.block_tokens(N, b, j)
        K[t] = K[t[0]]
    return K


def test_rectification_is_exact_for_blockwise_constant_keys():
    # a block whose keys are all equal contributes exactly n_j e^{s q.k}
    # to the normaliser and n_j e^{s q.k} Vbar_j to the output, so the
    # rectified result is full attention (torch SDPA in fp64), whatever V is
    N, b, d = 64 * 5 + 21, 64, 8       # ragged tail of 21 tokens
    s = 1 / math.sqrt(d)
    Q, V = _rand(50, N, d), _rand(51, N, d)
    K = _blockwise_constant_keys(52, N, b, d)
    nB = O.n_blocks(N, b)
    rows = [[i] for i in range(nB)]
    rows[2] = []                           # an empty row: pooled keys only
    rows[4] = list(range(nB))              # nothing omitted: the sparse result
    Orc, Lrc = O.pooled_rectified_attention(Q, K, V, rows, b, s)
    tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (Q, K, V))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=s)[0, 0].numpy()
    np.testing.assert_allclose(Orc, ref, atol=1e-12)
    np.testing.assert_allclose(Lrc, scipy.special.logsumexp(s * Q @ K.T, axis=1), atol=1e-12)


def test_pooled_part_of_a_full_row_is_empty_and_merge_keeps_sparse():
    N, b, d = 64 * 3, 64, 4
    Q, K, V = _rand(53, N, d), _rand(54, N, d), _rand(55, N, d)
    rows = [[0, 1, 2], [1], [0, 2]]
    Op, Lp = O.pooled_omitted_attention(Q, K, V, rows, b, 0.5)
    assert np.all(np.isneginf(Lp[:64])) and np.all(Op[:64] == 0)
    Os, Ls = O.block_sparse_attention(Q, K, V, rows, b, 0.5)
    Orc, Lrc = O.pooled_rectified_attention(Q, K, V, rows, b, 0.5)
    np.testing.assert_allclose(Orc[:64], Os[:64], atol=1e-14)
    np.testing.assert_allclose(Lrc[:64], Ls[:64], atol=1e-14)


def test_pooled_part_is_a_size_weighted_mixture_of_block_means():
    # brute force from the definition with explicit loops: weights n_j
    # e^{s q.Kbar_j} over the omitted blocks, normalised; output the
    # weighted mean of the value means
    N, b, d, s = 64 * 2 + 10, 64, 3, 0.7
    Q, K, V = _rand(56, N, d), _rand(57, N, d), _rand(58, N, d)
    rows = [[0], [2], []]
    Op, Lp = O.pooled_omitted_attention(Q, K, V, rows, b, s)
    for t in (0, 63, 64, 130, N - 1):
        i = t // b
        num, den = np.zeros(d), 0.0
        for j in range(3):
            if j in rows[i]:
                continue
            toks = range(b * j, min(b * j + b, N))
            kb = sum(K[x] for x in toks) / len(toks)
            vb = sum(V[x] for x in toks) / len(toks)
            w = len(toks) * math.exp(s * float(Q[t] @ kb))
            num += w * vb
            den += w
        np.testing.assert_allclose(Op[t], num / den, atol=1e-13)
        assert abs(Lp[t] - math.log(den)) < 1e-13


def test_rectification_pin_catches_a_dropped_size_bias(monkeypatch):
    real_sizes = O.block_sizes
    monkeypatch.setattr(O, "block_sizes", lambda N_, b_: np.ones_like(real_sizes(N_, b_)))
    N, b, d = 64 * 3 + 5, 64, 4
    s = 0.5
    Q, V = _rand(59, N, d), _rand(60, N, d)
    K = _blockwise_constant_keys(61, N, b, d)
    Orc, _ = O.pooled_rectified_attention(Q, K, V, [[0], [1], [], [3]], b, s)
    tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (Q, K, V))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=s)[0, 0].numpy()
    assert not np.allclose(Orc, ref, atol=1e-6)


# ----------------------------------------------- gain-aware rectification

def _golden_lse(vals):
    return np.array([-np.inf if v == "-inf" else v for v in vals], float)


def test_golden_rectify_gate():
    g = _load("rectify_gate.json")
    Q, K, V = (np.array(g[x], float) for x in ("Q", "K", "V"))
    b, s = g["b"], g["scale"]
    np.testing.assert_allclose(O.block_key_spread(K, b), g["spread"], atol=1e-15)
    assert O.rectify_gate(Q, K, b, s).tolist() == g["gate"]
    for case in g["cases"]:
        Op, Lp = O.pooled_omitted_attention(Q, K, V, case["rows"], b, s, gate=True)
        want_L = _golden_lse(case["LSE"])
        assert np.array_equal(np.isneginf(Lp), np.isneginf(want_L))
        fin = ~np.isneginf(want_L)
        np.testing.assert_allclose(Lp[fin], want_L[fin], atol=1e-14)
        np.testing.assert_allclose(Op, case["O"], atol=1e-14)
        # no sparse part in these rows beyond the kept block: the rectified
        # result of a row with nothing kept is the pooled part itself
        Orc, Lrc = O.pooled_rectified_attention(Q, K, V, case["rows"], b, s, gate=True)
        np.testing.assert_allclose(Orc[2:], Op[2:], atol=1e-14)


@pytest.mark.parametrize("sigma2,passes", [(0.8 * math.log(4.0), True), (1.2 * math.log(4.0), False),
                                           (0.3, True), (3.0, False)])
def test_gate_threshold_is_where_the_measured_error_meets_the_gain(sigma2, passes):
    # keys of one large block drawn isotropic normal (per-coordinate variance
    # 1.5): the brute-force pooling error of the mass estimate, w - w_hat with
    # w = sum_tau e^{s q.k_tau} and w_hat = n e^{s q.Kbar}, exceeds the gain
    # w_hat exactly when the gate refuses the block
    d, n, s = 8, 400_000, 1 / math.sqrt(8)
    rng = np.random.default_rng(71)
    K = 0.3 + math.sqrt(1.5) * rng.standard_normal((n, d))
    u = rng.standard_normal(d)
    v = float(O.block_key_spread(K, n)[0])
    q = u / np.linalg.norm(u) * math.sqrt(sigma2 / (s * s * v))
    kbar = K.mean(axis=0)
    w_hat = n * math.exp(s * float(q @ kbar))
    w = float(np.exp(s * (K @ q)).sum())
    assert ((w - w_hat) < w_hat) == passes
    assert bool(O.rectify_gate(q[None, :], K, n, s)[0, 0]) == passes


def test_gate_passes_every_block_of_constant_keys():
    # zero spread: the estimate is exact (gain, no error), the gated result is
    # the ungated one and both equal full attention
    N, b, d = 64 * 4 + 9, 64, 8
    s = 1 / math.sqrt(d)
    Q, V = 3.0 * _rand(62, N, d), _rand(63, N, d)
    K = _blockwise_constant_keys(64, N, b, d)
    # (the mean of equal keys carries rounding: the spread is ~1e-30, not 0)
    assert np.all(O.block_key_spread(K, b) < 1e-25)
    assert O.rectify_gate(Q, K, b, s).all()
    rows = [[i] for i in range(O.n_blocks(N, b))]
    Og, Lg = O.pooled_rectified_attention(Q, K, V, rows, b, s, gate=True)
    Ou, Lu = O.pooled_rectified_attention(Q, K, V, rows, b, s)
    np.testing.assert_array_equal(Og, Ou)
    np.testing.assert_array_equal(Lg, Lu)


def test_gated_part_is_the_mixture_over_passing_blocks():
    # brute force with explicit loops: per token, the size-weighted mixture of
    # value means over the omitted blocks whose spread test passes
    N, b, d, s = 64 * 3 + 7, 64, 4, 0.45
    Q, K, V = _rand(65, N, d), _rand(66, N, d), _rand(67, N, d)
    Q[::3] *= 2.5                      # some tokens fail for some blocks
    rows = [[0], [], [1, 3], [2]]
    Op, Lp = O.pooled_omitted_attention(Q, K, V, rows, b, s, gate=True)
    n_pass = n_fail = 0
    for t in range(N):
        i = t // b
        num, den = np.zeros(d), 0.0
        for j in range(O.n_blocks(N, b)):
            if j in rows[i]:
                continue
            toks = range(b * j, min(b * j + b, N))
            kb = sum(K[x] for x in toks) / len(toks)
            vj = sum(float((K[x] - kb) @ (K[x] - kb)) for x in toks) / (len(toks) * d)
            if s * s * float(Q[t] @ Q[t]) * vj >= 2 * math.log(2):
                n_fail += 1
                continue
            n_pass += 1
            w = len(toks) * math.exp(s * float(Q[t] @ kb))
            num += w * sum(V[x] for x in toks) / len(toks)
            den += w
        if den == 0.0:
            assert np.isneginf(Lp[t]) and np.all(Op[t] == 0)
        else:
            np.testing.assert_allclose(Op[t], num / den, atol=1e-13)
            assert abs(Lp[t] - math.log(den)) < 1e-13
    assert n_pass > 50 and n_fail > 50


@pytest.mark.parametrize("mistake", ["threshold", "no_d", "norm_not_squared"])
def test_gate_pins_catch_planted_mistakes(mistake, monkeypatch):
    real_spread = O.block_key_spread
    if mistake == "threshold":
        monkeypatch.setattr(O, "GATE_SIGMA2", math.log(2.0))
    elif mistake == "no_d":
        monkeypatch.setattr(O, "block_key_spread",
                            lambda K_, b_: real_spread(K_, b_) * np.asarray(K_).shape[1])
    else:
        def bad_gate(Q_, K_, b_, s_):
            Q_ = np.asarray(Q_, np.float64)
            qn = np.sqrt((Q_ * Q_).sum(axis=1))
            return (s_ * s_) * qn[:, None] * real_spread(K_, b_)[None, :] < O.GATE_SIGMA2
        monkeypatch.setattr(O, "rectify_gate", bad_gate)
    with pytest.raises(AssertionError):
        test_golden_rectify_gate()


# ------------------------------------------------------------------ density

def test_density_counts_blocks_over_the_whole_map():
    # MOD-DiT, Metrics: computed B x B blocks over all blocks of every head's
    # map.  Two heads of a 3 x 3 block map: 1 + 2 + 3 and 3 + 1 + 0 kept
    # blocks, 10 of 18.
    rows = [[[0], [0, 1], [0, 1, 2]], [[0, 1, 2], [1], []]]
    assert O.density(rows, 3) == 10 / 18
    # closed forms: the diagonal alone is 1/nB, every block is 1, top-k rows
    # of length k are k/nB
    nB = 16
    assert O.density([[[i] for i in range(nB)]], nB) == 1 / nB
    assert O.density([[list(range(nB))] * nB] * 3, nB) == 1.0
    S = _rand(68, nB, nB)
    rows_k = O.select_rows(S, 64 * nB, 64, "topk", k=4)
    assert O.density([rows_k, rows_k], nB) == 4 / nB


def test_density_of_the_long_horizon_window():
    # the +-1-frame window with 4 anchors over 3072 blocks keeps about 2.55%
    N, b, ft = 126 * 30 * 52, 64, 30 * 52
    nB = O.n_blocks(N, b)
    rows = [sorted(O.window_anchor_set(N, b, i, ft, 1, 4, 5)) for i in range(nB)]
    dens = O.density([rows], nB)
    assert 0.0245 < dens < 0.0265
    # counted directly: every row's length over nB, averaged
    assert abs(dens - np.mean([len(r) / nB for r in rows])) < 1e-15


# ---------------------------------------------------- micro selection, all rows

@pytest.mark.parametrize("N,m,seed", [(64 * 5 + 23, 7, 81), (64 * 3, 1000, 82), (64 * 6 + 1, 0, 83),
                                      (64 * 4 + 40, 30, 84)])
def test_micro_select_rows_equals_the_per_row_definition(N, m, seed):
    b, u, d = 64, 16, 8
    s = 1 / math.sqrt(d)
    Q, K = _rand(seed, N, d), _rand(seed + 100, N, d)
    S = O.pooled_scores(O.pool_means(Q, b), O.pool_means(K, b), s)
    rows = O.select_rows(S, N, b, "topk", k=2, force_diag=True)
    rows[1] = []
    Qt, Kt = O.pool_means(Q, u), O.pool_means(K, u)
    got = O.micro_select_rows(Qt, Kt, rows, N, b, u, s, m)
    want = [O.micro_select_row(Qt, Kt, rows[i], i, N, b, u, s, m) for i in range(len(rows))]
    assert got == want


def test_micro_select_rows_breaks_exact_ties_by_code():
    # every key tile equal: all candidates tie, the lowest codes 4 beta + a win
    N, b, u = 64 * 3, 64, 16
    Qt = np.ones((12, 2))
    Kt = np.ones((12, 2))
    rows = [[0], [1], [2]]
    got = O.micro_select_rows(Qt, Kt, rows, N, b, u, 1.0, 5)
    # block 0 omits blocks 1, 2 (tiles 4..11): codes 16, 17, 18, 19, 20 win
    assert got[0] == [16, 20, 17, 18, 19]
    assert got[1] == [0, 4, 1, 2, 3]


# ------------------------------------------------------------ omission risk

def test_golden_omission_three_keys():
    g = _load("omission_three_keys.json")
    q, K = np.array(g["q"]), np.array(g["K"])
    w = O.softmax_mass_outside(q, K, np.array(g["support"]), g["scale"])
    np.testing.assert_allclose(w, [g["omitted"]], atol=1e-15)
    rep = np.array(g["support"] + g["repair"])
    w2 = O.softmax_mass_outside(q, K, rep, g["scale"])
    np.testing.assert_allclose(w[0] - w2[0], g["recovered"], atol=1e-15)
    wl, gl = O.risk_from_lse([g["LSE_sparse"]], [g["LSE_full"]], [g["LSE_repaired"]])
    np.testing.assert_allclose(wl, [g["omitted"]], atol=1e-15)
    np.testing.assert_allclose(gl, [g["recovered"]], atol=1e-15)


def _risk_instance(seed=30, N=64 * 5 + 23, d=8):
    s = 1 / math.sqrt(d)
    Q, K, V = _rand(seed, N, d), _rand(seed + 1, N, d), _rand(seed + 2, N, d)
    S = O.pooled_scores(O.pool_means(Q, 64), O.pool_means(K, 64), s)
    rows = O.select_rows(S, N, 64, "topk", k=2)
    rows[1] = []  # an empty row: everything omitted
    return Q, K, V, rows, s


def test_risk_from_lse_equals_mass_outside_the_support():
    # the LSE form (normalisers of the two supports) against the mass summed
    # key by key over the full-attention distribution
    Q, K, V, rows, s = _risk_instance()
    N = Q.shape[0]
    w_def = O.omitted_mass(Q, K, rows, 64, s)
    _, Ls = O.block_sparse_attention(Q, K, V, rows, 64, s)
    _, Lf = O.dense_attention(Q, K, V, s)
    w, g = O.risk_from_lse(Ls, Lf)
    np.testing.assert_allclose(w, w_def, atol=1e-13)
    assert np.all(g == 0)
    assert np.all(w[64:128] == 1.0) and np.all((w >= 0) & (w <= 1))
    # repair: the Micro residual over a few tiles of the omitted blocks
    Qt, Kt = O.pool_means(Q, 16), O.pool_means(K, 16)
    mrows = [O.micro_select_row(Qt, Kt, rows[i], i, N, 64, 16, s, 5)
             for i in range(len(rows))]
    _, Lu = O.micro_attention(Q, K, V, mrows, 64, 16, s)
    _, Lr = O.lse_merge(np.zeros((N, 8)), Ls, np.zeros((N, 8)), Lu)
    w, g = O.risk_from_lse(Ls, Lf, Lr)
    np.testing.assert_allclose(g, O.micro_mass(Q, K, mrows, 64, 16, s), atol=1e-13)
    assert np.all(g <= w + 1e-15) and np.any(g > 0)


def test_risk_zero_query_closed_form():
    # q = 0: every key weighs the same, so the omitted share of a token of
    # block i is 1 - (tokens of its support) / N
    N, b = 64 * 3 + 9, 64
    Q, K = np.zeros((N, 4)), _rand(31, N, 4)
    rows = [[0], [0, 2], [1, 3], [3]]
    w = O.omitted_mass(Q, K, rows, b, 0.7)
    sizes = O.block_sizes(N, b)
    for i, sel in enumerate(rows):
        want = 1 - sum(sizes[j] for j in sel) / N
        np.testing.assert_allclose(w[O.block_tokens(N, b, i)], want, atol=1e-14)
    Ls = np.array([math.log(sum(sizes[j] for j in rows[t // b])) for t in range(N)])
    wl, _ = O.risk_from_lse(Ls, np.full(N, math.log(N)))
    np.testing.assert_allclose(wl, w, atol=1e-14)


def test_risk_full_support_all_micro_and_edges():
    Q, K, V, rows, s = _risk_instance(seed=33)
    N, nB = Q.shape[0], O.n_blocks(Q.shape[0], 64)
    full = [list(range(nB))] * nB
    np.testing.assert_allclose(O.omitted_mass(Q, K, full, 64, s), 0.0, atol=1e-14)
    # every candidate tile as micro repair: the repair recovers all omitted mass
    Qt, Kt = O.pool_means(Q, 16), O.pool_means(K, 16)
    mrows = [O.micro_select_row(Qt, Kt, rows[i], i, N, 64, 16, s, 10 ** 6) for i in range(nB)]
    np.testing.assert_allclose(O.micro_mass(Q, K, mrows, 64, 16, s),
                               O.omitted_mass(Q, K, rows, 64, s), atol=1e-13)
    # -inf conventions: empty support omits all, no keys at all counts 0
    w, g = O.risk_from_lse([-math.inf, 0.5, -math.inf], [1.0, 0.5, -math.inf],
                           [0.0, 0.5, -math.inf])
    np.testing.assert_allclose(w, [1.0, 0.0, 0.0], atol=1e-15)
    np.testing.assert_allclose(g, [math.exp(-1.0), 0.0, 0.0], atol=1e-15)


def test_head_risk_and_heads_at_risk():
    assert O.head_risk(np.array([0.1, 0.4, 0.1]), np.array([0.0, 0.3, 0.0])) == \
        pytest.approx((0.2, 0.4, 0.1), abs=1e-15)
    assert O.head_risk(np.zeros(0), np.zeros(0)) == (0.0, 0.0, 0.0)
    risk = np.array([0.2, 0.5, 0.2, 0.9, 0.2])
    assert O.heads_at_risk(risk, 2) == [1, 3]
    assert O.heads_at_risk(risk, 3) == [0, 1, 3]   # tie at 0.2 -> lowest index
    assert O.heads_at_risk(risk, 0) == []
    assert O.heads_at_risk(risk, 9) == [0, 1, 2, 3, 4]


@pytest.mark.parametrize("mistake", ["swap", "tail", "plain_exp"])
def test_risk_pins_catch_planted_mistakes(mistake, monkeypatch):
    """Plausible slips in the risk functions fail the pins above."""
    g = _load("omission_three_keys.json")
    if mistake == "swap":
        real = O.risk_from_lse
        monkeypatch.setattr(O, "risk_from_lse", lambda a, b, c=None: real(b, a, c))
        w, _ = O.risk_from_lse([g["LSE_sparse"]], [g["LSE_full"]])
        assert abs(w[0] - g["omitted"]) > 1e-3
    elif mistake == "tail":
        monkeypatch.setattr(O, "block_tokens",
                            lambda N_, b_, j: np.arange(b_ * j, min(b_ * j + b_, N_ - 1)))
        N, b = 64 * 3 + 9, 64
        Q, K = np.zeros((N, 4)), _rand(31, N, 4)
        w = O.omitted_mass(Q, K, [[0], [0, 3], [1, 3], [3]], b, 0.7)
        assert abs(w[64] - (1 - (64 + 9) / N)) > 1e-3
    else:
        # mass from exp(z) without the normaliser of the full distribution
        monkeypatch.setattr(O, "softmax_mass_outside", lambda q, K, keys, sc: 1.0 - np.exp(
            sc * np.asarray(q) @ np.asarray(K)[np.asarray(keys, int)].T).sum(axis=1))
        w = O.softmax_mass_outside(np.array(g["q"]), np.array(g["K"]),
                                   np.array(g["support"]), g["scale"])
        assert abs(w[0] - g["omitted"]) > 1e-3


def test_flop_accounting():
    assert O.executed_flops(128, 64, 1) == 4 * 128 * 64 * 64
    assert O.dense_flops(1, 12, 32760, 128) == 4 * 12 * 32760 ** 2 * 128
    assert O.executed_flops(64, 64, 0, 16, 3) == 4 * 64 * 256 * 3


@pytest.mark.parametrize("mistake", ["scale", "tail"])
def test_pins_catch_planted_mistakes(mistake, monkeypatch):
    """A plausible slip in the oracle must fail a pin: plant it and check."""
    N, d, b = 200, 16, 64
    s = 1 / math.sqrt(d)
    Q, K, V = _rand(6, N, d), _rand(7, N, d), _rand(8, N, d)
    if mistake == "scale":
        real = O.attend
        monkeypatch.setattr(O, "attend", lambda q, k, v, sc: real(q, k, v, sc * 1.01))
    else:
        # a ragged tail "padded" by wrapping around to the first tokens
        monkeypatch.setattr(O, "block_tokens",
                            lambda N_, b_, j: np.arange(b_ * j, b_ * j + b_) % N_)
    rows = [list(range(O.n_blocks(N, b)))] * O.n_blocks(N, b)
    Ov, _ = O.block_sparse_attention(Q, K, V, rows, b, s)
    tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (Q, K, V))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=s)
    assert not np.allclose(Ov, ref[0, 0].numpy(), atol=1e-9)


# --------------------------------------------- HVA hardware cost and merging

def _group_state(members, rows, nk):
    chi = np.zeros(nk, dtype=bool)
    for i in members:
        chi[list(rows[i])] = True
    return chi


def test_golden_merge_cost():
    g = _load("hva_merge_rounds.json")
    for c in g["cost_cases"]:
        got = O.merge_cost(c["sq"], np.array(c["chi"], bool), c["sizes_k"], g["tau_q"],
                           g["tau_k"], c["g"])
        assert got == c["cost"], c["note"]


def test_golden_merge_rounds():
    g = _load("hva_merge_rounds.json")
    m = g["merge"]
    sq, sk, rows = m["sizes_q"], m["sizes_k"], m["rows"]
    nk = len(sk)
    for i, c in enumerate(m["singleton_costs"]):
        assert O.partition_cost([[i]], sq, rows, sk) == c

    def gain(a_members, b_members):
        return O.merge_gain(sum(sq[i] for i in a_members), _group_state(a_members, rows, nk),
                            sum(sq[i] for i in b_members), _group_state(b_members, rows, nk), sk)

    assert gain([1], [0]) == m["round1_gains"]["1->0"]
    assert gain([1], [3]) == m["round1_gains"]["1->3"]
    assert gain([2], [0]) == m["round1_gains"]["2->0"]
    assert gain([2], [3]) == m["round1_gains"]["2->3"]
    assert gain([0, 2], [1]) == m["round2_gains"]["0->1"]
    assert gain([0, 2], [3]) == m["round2_gains"]["0->3"]
    assert gain([3], [0, 1, 2]) == m["round3_gains"]["3->0"]
    for r, key in [(1, "round1_groups"), (2, "round2_groups"), (3, "final_groups")]:
        _, groups = O.agglomerative_merge(sq, rows, sk, m["sides"][:r])
        assert groups == m[key], key
    grp, groups = O.agglomerative_merge(sq, rows, sk, m["sides"])
    assert grp.tolist() == m["final_group_of"]
    assert O.partition_cost(groups, sq, rows, sk) == m["final_cost"]
    assert _best_partition_cost(sq, rows, sk) == m["optimal_cost"]


def _partitions(items):
    if not items:
        yield []
        return
    first, rest = items[0], items[1:]
    for p in _partitions(rest):
        for k in range(len(p)):
            yield p[:k] + [[first] + p[k]] + p[k + 1:]
        yield [[first]] + p


def _best_partition_cost(sq, rows, sk, g=1):
    """Eq. 9 solved exactly by enumerating every partition (tiny inputs)."""
    return min(O.partition_cost(p, sq, rows, sk, 64, 64, g) for p in _partitions(list(range(len(sq)))))


def _random_merge_instance(seed, nq, nk):
    rng = np.random.default_rng(seed)
    sq = rng.integers(0, 90, nq).tolist()
    sk = rng.integers(1, 70, nk).tolist()
    rows = [sorted(rng.choice(nk, int(rng.integers(0, nk + 1)), replace=False).tolist())
            for _ in range(nq)]
    sides = rng.integers(0, 2, (3, nq)).tolist()
    return sq, sk, rows, sides


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("g", [1, 16])
def test_merge_is_a_valid_partition_that_never_raises_the_cost(seed, g):
    sq, sk, rows, sides = _random_merge_instance(900 + seed, 6, 5)
    start = O.partition_cost([[i] for i in range(6)], sq, rows, sk, 64, 64, g)
    prev = start
    for r in range(1, 4):
        grp, groups = O.agglomerative_merge(sq, rows, sk, sides[:r], g=g)
        assert sorted(i for S in groups for i in S) == list(range(6))
        for S in groups:
            assert all(grp[i] == min(S) for i in S) and S == sorted(S)
        cost = O.partition_cost(groups, sq, rows, sk, 64, 64, g)
        assert cost <= prev          # every accepted merge has a negative gain
        prev = cost
    assert prev >= _best_partition_cost(sq, rows, sk, g)


@pytest.mark.parametrize("seed", range(20))
def test_merge_of_two_clusters_follows_the_sign_of_the_gain(seed):
    sq, sk, rows, _ = _random_merge_instance(950 + seed, 2, 4)
    grp, groups = O.agglomerative_merge(sq, rows, sk, [[0, 1]])
    together = O.partition_cost([[0, 1]], sq, rows, sk) < O.partition_cost([[0], [1]], sq, rows, sk)
    assert (groups == [[0, 1]]) == together


def test_merge_without_rounds_or_with_one_side_keeps_singletons():
    sq, sk, rows, _ = _random_merge_instance(990, 5, 4)
    for sides in ([], [[0] * 5], [[1] * 5]):
        grp, groups = O.agglomerative_merge(sq, rows, sk, sides)
        assert groups == [[i] for i in range(5)] and grp.tolist() == list(range(5))


def test_packed_pairs_and_group_rows():
    off_q = [0, 64, 128, 192]        # three query clusters of 64
    off_k = [0, 64, 192, 256]        # key clusters of 64, 128, 64
    rows = [[0], [1, 2], [2]]
    # tile-aligned clusters: packing changes nothing
    singles = [[0], [1], [2]]
    assert O.packed_tile_pairs(off_q, off_k, singles, O.group_rows(singles, rows)) == \
        O.cluster_tile_pairs(off_q, off_k, rows) == 1 + 3 + 1
    merged = [[0, 2], [1]]
    gr = O.group_rows(merged, rows)
    assert gr == [[0, 2], [1, 2], [0, 2]]
    assert O.packed_tile_pairs(off_q, off_k, merged, gr) == 2 * 2 + 1 * 3
    # 16-token grain: a key cluster of 20 takes 32 slots, packed with 40 -> 48
    off_k2 = [0, 20, 60]
    assert O.packed_tile_pairs([0, 10], off_k2, [[0]], [[0, 1]], g=16) == 2
    assert O.packed_tile_pairs([0, 10], off_k2, [[0]], [[0, 1]], g=1) == 1


def test_attention_over_merged_groups_is_masked_dense_softmax():
    """Every query of a merged group attends over the union of the group's
    key clusters: the token-level mask built directly, through SDPA in fp64."""
    rng = np.random.default_rng(77)
    N, d = 90, 16
    Q, K, V = _rand(71, N, d), _rand(72, N, d), _rand(73, N, d)
    aq = rng.integers(0, 5, N)
    ak = rng.integers(0, 4, N)
    rows = [[0], [1, 3], [2], [], [0, 2]]
    groups = [[0, 2], [1], [3, 4]]
    gr = O.group_rows(groups, rows)
    pq, oq = O.cluster_permutation(aq, 5)
    pk, ok = O.cluster_permutation(ak, 4)
    Oc, Lc = O.cluster_block_attention(Q, K, V, pq, oq, pk, ok, gr, 1 / math.sqrt(d))
    group_of = {i: gi for gi, S in enumerate(groups) for i in S}
    keys_of = [set().union(*[set(rows[i]) for i in S]) for S in groups]
    M = np.array([[ak[t] in keys_of[group_of[aq[s]]] for t in range(N)] for s in range(N)])
    tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (Q, K, V))
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=torch.from_numpy(M)[None, None], scale=1 / math.sqrt(d))[0, 0].numpy()
    has = M.any(axis=1)
    np.testing.assert_allclose(Oc[has], ref[has], atol=1e-12)
    assert np.all(Oc[~has] == 0) and np.all(np.isneginf(Lc[~has]))


@pytest.mark.parametrize("mistake", ["gain_sign", "first_chooser", "no_union", "no_query_ceil"])
def test_merge_pins_catch_planted_mistakes(mistake, monkeypatch):
    g = _load("hva_merge_rounds.json")
    m = g["merge"]
    if mistake == "gain_sign":
        real = O.merge_gain
        monkeypatch.setattr(O, "merge_gain", lambda *a, **k: -real(*a, **k))
    elif mistake == "first_chooser":
        def first(choice):
            out = {}
            for A in sorted(choice):
                gain, B = choice[A]
                if gain < 0 and B not in out:
                    out[B] = (gain, A)
            return out
        monkeypatch.setattr(O, "disjoint_merges", first)
    elif mistake == "no_union":
        real_cost = O.merge_cost

        def gain_a_only(sq_a, chi_a, sq_b, chi_b, sizes_k, tau_q=64, tau_k=64, gg=1):
            return (real_cost(sq_a + sq_b, chi_a, sizes_k, tau_q, tau_k, gg)
                    - real_cost(sq_a, chi_a, sizes_k, tau_q, tau_k, gg)
                    - real_cost(sq_b, chi_b, sizes_k, tau_q, tau_k, gg))
        monkeypatch.setattr(O, "merge_gain", gain_a_only)
    else:
        monkeypatch.setattr(O, "merge_cost", lambda sq, chi, sk, tq=64, tk=64, gg=1: int(sq) * (
            tk * (-(-int(sum(np.asarray(sk)[np.asarray(chi, bool)])) // tk))))
    with pytest.raises(AssertionError):
        test_golden_merge_cost()
        test_golden_merge_rounds()


# ------------------------------------------------------------ Lowe's ratio

def test_golden_lowe_ratio():
    g = _load("hva_lowe_ratio.json")
    rho = O.lowe_ratios(np.array(g["X"]), tuple(g["thw"]), tuple(g["cell"]), tuple(g["window"]),
                        np.array(g["mu"]))
    np.testing.assert_allclose(rho, g["rho"], rtol=0, atol=1e-15)
    assert O.lowe_subset(rho, 2).tolist() == g["subset_2"]
    assert O.lowe_subset(rho, 3).tolist() == g["subset_3"]


def test_lowe_ratio_with_a_global_window_is_cdist():
    """A window covering the whole grid: the two smallest Euclidean distances
    of scipy's cdist over every centroid."""
    import scipy.spatial.distance as sd
    thw, cell = (3, 6, 8), (1, 3, 4)
    X, mu = _rand(81, 3 * 6 * 8, 5), _rand(82, 3 * 2 * 2, 5)
    rho = O.lowe_ratios(X, thw, cell, (3, 2, 2), mu)
    dd = np.sort(sd.cdist(X, mu), axis=1)
    np.testing.assert_allclose(rho, dd[:, 0] / dd[:, 1], rtol=1e-14)


def test_lowe_ratio_special_cases():
    thw, cell = (1, 2, 2), (1, 1, 1)
    mu = np.array([[0.0, 0.0], [4.0, 0.0], [0.0, 4.0], [4.0, 4.0]])
    X = np.array([[0.0, 0.0], [2.0, 2.0], [1.0, 0.0], [4.0, 4.0]])
    rho = O.lowe_ratios(X, thw, cell, (1, 2, 2), mu)
    assert rho[0] == 0.0 and rho[3] == 0.0          # on a centroid
    assert rho[1] == 1.0                            # equidistant from all four
    assert abs(rho[2] - 1.0 / 3.0) < 1e-15          # 1 against 3
    # one candidate per token: no second centroid
    assert np.all(O.lowe_ratios(X, thw, cell, (1, 1, 1), mu) == 0.0)
    # two coincident centroids at distance 0 from the token
    assert O.lowe_ratios(np.zeros((2, 2)), (1, 1, 2), (1, 1, 1), (1, 1, 2), np.zeros((2, 2)))[0] == 1.0
    # rho = 1 exactly where the assignment margin is 0
    m = O.assignment_margins(X, thw, cell, (1, 2, 2), mu)
    assert np.array_equal(rho == 1.0, m == 0.0)


def test_lowe_subset_order_and_ties():
    rho = np.array([0.5, 0.9, 0.5, 0.1, 0.9, 0.5])
    assert O.lowe_subset(rho, 2).tolist() == [1, 4]
    assert O.lowe_subset(rho, 3).tolist() == [0, 1, 4]       # tie at 0.5 -> lowest index
    assert O.lowe_subset(rho, 4).tolist() == [0, 1, 2, 4]
    assert O.lowe_subset(rho, 0).tolist() == []
    assert O.lowe_subset(rho, 9).tolist() == list(range(6))


@pytest.mark.parametrize("mistake", ["inverted", "squared"])
def test_lowe_pins_catch_planted_mistakes(mistake, monkeypatch):
    real = O.lowe_ratios

    def wrong(X, thw, cell, window, mu):
        r = real(X, thw, cell, window, mu)
        if mistake == "inverted":
            return np.where(r > 0, 1.0 / np.where(r > 0, r, 1.0), 0.0)
        return r ** 2
    monkeypatch.setattr(O, "lowe_ratios", wrong)
    with pytest.raises(AssertionError):
        test_golden_lowe_ratio()


# ------------------------------------------------ HVA subset refinement (4.2)

def test_golden_subset_refinement():
    g = _load("hva_subset_refine.json")
    a, mu, n = O.subset_refinement(np.array(g["X"]), g["assign"], np.array(g["mu"]), g["subset"])
    assert a.tolist() == g["assign_out"]
    np.testing.assert_allclose(mu, g["mu_out"], atol=1e-15)
    assert n.tolist() == g["counts_out"]


def test_subset_refinement_of_every_token_is_one_lloyd_step():
    # with the whole lattice as the subset and centroids that are their
    # members' means, the update is one step of Lloyd's k-means: assign to
    # the nearest centroid, then move every centroid that changed members to
    # its members' mean (scikit-learn's single Lloyd iteration moves all of
    # them; the untouched ones are already their members' means)
    from sklearn.cluster import KMeans
    rng = np.random.default_rng(91)
    X = np.concatenate([rng.standard_normal((60, 5)) + 4 * rng.standard_normal(5) for _ in range(6)])
    a0 = rng.integers(0, 6, X.shape[0])
    mu0 = np.stack([X[a0 == c].mean(axis=0) for c in range(6)])
    a, mu, n = O.subset_refinement(X, a0, mu0, np.arange(X.shape[0]))
    km = KMeans(n_clusters=6, init=mu0, n_init=1, max_iter=1, algorithm="lloyd").fit(X)
    # scikit-learn's labels_ come from one more assignment after the update;
    # compare the centroids and recompute the first assignment directly
    np.testing.assert_allclose(mu, km.cluster_centers_, atol=1e-12)
    first = np.argmin(((X[:, None, :] - mu0[None]) ** 2).sum(-1), axis=1)
    assert np.array_equal(a, first)
    assert n.tolist() == np.bincount(first, minlength=6).tolist()


def test_subset_refinement_leaves_other_tokens_and_centroids_alone():
    rng = np.random.default_rng(92)
    X = rng.standard_normal((200, 4))
    mu = rng.standard_normal((9, 4)) * 2
    a0 = rng.integers(0, 9, 200)
    S = rng.choice(200, 30, replace=False)
    a, mu2, n = O.subset_refinement(X, a0, mu, S)
    rest = np.setdiff1d(np.arange(200), S)
    assert np.array_equal(a[rest], a0[rest])
    # brute force: nearest of all centroids with explicit loops, ties low
    for t in S:
        best, bd = 0, math.inf
        for c in range(9):
            dd = sum((X[t, k] - mu[c, k]) ** 2 for k in range(4))
            if dd < bd:
                best, bd = c, dd
        assert a[t] == best
    moved = S[a[S] != a0[S]]
    touched = set(a0[moved]) | set(a[moved])
    for c in range(9):
        if c in touched and n[c] > 0:
            np.testing.assert_allclose(mu2[c], X[a == c].mean(axis=0), atol=1e-13)
        else:
            assert np.array_equal(mu2[c], mu[c])
    assert n.sum() == 200
    # an empty subset changes nothing
    a3, mu3, _ = O.subset_refinement(X, a0, mu, [])
    assert np.array_equal(a3, a0) and np.array_equal(mu3, mu)


def test_subset_refinement_pin_catches_a_stale_or_local_update(monkeypatch):
    g = _load("hva_subset_refine.json")
    X = np.array(g["X"])
    # a planted mistake: centroids updated from the anchor-step means by the
    # moved tokens only (the stale-sum transfer) instead of their members
    real = O.subset_refinement

    def transfer(X_, assign, mu, subset):
        a, _, n = real(X_, assign, mu, subset)
        mu = np.asarray(mu, float).copy()
        old = np.bincount(np.asarray(assign), minlength=len(mu))
        sums = old[:, None] * mu
        for t in subset:
            sums[assign[t]] -= X_[t]
            sums[a[t]] += X_[t]
        ok = n > 0
        mu[ok] = sums[ok] / n[ok, None]
        return a, mu, n
    monkeypatch.setattr(O, "subset_refinement", transfer)
    with pytest.raises(AssertionError):
        test_golden_subset_refinement()

