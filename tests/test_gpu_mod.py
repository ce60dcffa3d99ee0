"""GPU parity of selection on 128-token blocks (MOD-DiT block-wise attention,
emitted on 64-token tiles) and of MOD-DiT's structural patterns (parallel
diagonals, vertical columns, block-diagonal = window of radius 0) against
the fp64 oracle: pooled means and scores element by element, every list
(ties exempt as in the other selection tests, read at the selection block),
and attention over the emitted tiles against the oracle's attention at the
128-token block."""

import math
import sys

import numpy as np
import pytest
import torch

from oracle import bsa_oracle as O
from synth import CONFIGS, VideoSpec, config_spec, gen_qkv, mod_pattern_mask
import parity as PT

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import block_sparse_attention_pool_amd as bsa
else:  # collected on CPU, skipped by the marker
    bsa = None

DEV = "cuda:0"


def say(*a):
    print("[gpu-mod]", *a, file=sys.stderr, flush=True)


def gpu_rows64(rp, ci, nnz, B, H, N):
    nB = O.n_blocks(N, 64)
    rows = bsa.csr_rows(rp, ci, nnz)
    return {(b, h): rows[(b * H + h) * nB:(b * H + h + 1) * nB]
            for b in range(B) for h in range(H)}


def collapse128(rows64, N):
    """The 128-block rows behind 64-tile rows, checking that the tile rows
    are exactly their expansion (both 64-blocks of a kept 128-block, the
    same list for the two query halves)."""
    rows128 = [sorted({j // 2 for j in rows64[2 * I]}) for I in range(O.n_blocks(N, 128))]
    assert O.expand_rows(rows128, N, 128, 64) == rows64
    return rows128


def oracle_rows(Q, K, b, h, block, mode, **kw):
    N, d = Q.shape[2], Q.shape[3]
    S = None
    if mode != "static":
        q, k = PT.head64(Q, b, h), PT.head64(K, b, h)
        S = O.pooled_scores(O.pool_means(q, block), O.pool_means(k, block), 1 / math.sqrt(d))
    return S, O.select_rows(S, N, block, mode, **kw)


def forced(N, block, force_diag=False, static=None, patterns=None):
    nB = O.n_blocks(N, block)
    out = []
    for i in range(nB):
        f = {i} if force_diag else set()
        if static is not None:
            f |= O.window_anchor_set(N, block, i, **static)
        if patterns is not None:
            f |= O.pattern_set(nB, i, patterns.get("diagonals", ()), patterns.get("columns", ()))
        out.append(f)
    return out


def run_select(spec, block, mode, **kw):
    Q, K, V = gen_qkv(spec)
    Qd, Kd = (x.to(DEV) for x in (Q, K))
    sc = bsa.bsa_score_blocks(Qd, Kd, block=block, scores=(mode != "static"))
    rp, ci, nnz = bsa.bsa_select_blocks(sc["scores"], Qd, block=block, mode=mode, **kw)
    torch.cuda.synchronize()
    return Q, K, V, sc, gpu_rows64(rp, ci, nnz, *Q.shape[:3])


def check_lists(Q, K, got, block, mode, **kw):
    B, H, N, _ = Q.shape
    F = forced(N, block, kw.get("force_diag", False), kw.get("static"), kw.get("patterns"))
    exempt = 0
    for b in range(B):
        for h in range(H):
            g = got[(b, h)] if block == 64 else collapse128(got[(b, h)], N)
            S, rows = oracle_rows(Q, K, b, h, block, mode, **kw)
            if mode == "topk":
                exempt += PT.compare_topk_rows(g, rows, S, kw["k"], F)
            elif mode == "topp":
                exempt += PT.compare_topp_rows(g, rows, S, O.block_sizes(N, block), kw["p"],
                                               kw["k_min"], kw["k_cap"], F)
            else:
                assert g == rows, f"b{b} h{h}"
    return exempt


SMALL = [
    # (grid, H, d, key): 128-token tails of 55, 39, 0 (N = 1024) and 65 tokens
    ((3, 7, 9), 3, 128, 131),
    ((5, 15, 21), 2, 128, 132),
    ((4, 16, 16), 2, 64, 133),
    ((1, 1, 65), 1, 64, 134),
]


@pytest.mark.parametrize("grid,H,d,key", SMALL)
def test_pool_and_scores_block128(grid, H, d, key):
    spec = VideoSpec(1, H, d, grid, key)
    say("pool/score 128", grid, H, d)
    Q, K, _ = gen_qkv(spec)
    Qd, Kd = (x.to(DEV) for x in (Q, K))
    sc = bsa.bsa_score_blocks(Qd, Kd, block=128, micro=16)
    torch.cuda.synchronize()
    nB = O.n_blocks(spec.N, 128)
    assert sc["scores"].shape == (1, H, nB, nB)
    for h in range(H):
        q, k = PT.head64(Q, 0, h), PT.head64(K, 0, h)
        Qb, Kb = O.pool_means(q, 128), O.pool_means(k, 128)
        np.testing.assert_allclose(sc["qpool"][0, h].double().cpu().numpy(), Qb, atol=2e-6)
        np.testing.assert_allclose(sc["kpool"][0, h].double().cpu().numpy(), Kb, atol=2e-6)
        np.testing.assert_allclose(sc["scores"][0, h].double().cpu().numpy(),
                                   O.pooled_scores(Qb, Kb, 1 / math.sqrt(d)), atol=1e-5)
        np.testing.assert_allclose(sc["qpool16"][0, h].double().cpu().numpy(),
                                   O.pool_means(q, 16), atol=2e-6)
        np.testing.assert_allclose(sc["kpool16"][0, h].double().cpu().numpy(),
                                   O.pool_means(k, 16), atol=2e-6)


@pytest.mark.parametrize("grid,H,d,key", SMALL)
@pytest.mark.parametrize("k,diag", [(1, True), (2, False), (0, True), (99, False)])
def test_topk_select_block128(grid, H, d, key, k, diag):
    spec = VideoSpec(1, H, d, grid, key)
    say("topk 128", grid, k, diag)
    Q, K, _, _, got = run_select(spec, 128, "topk", k=k, force_diag=diag)
    check_lists(Q, K, got, 128, "topk", k=k, force_diag=diag)


@pytest.mark.parametrize("grid,H,d,key", SMALL[:3])
@pytest.mark.parametrize("p,kmin,kcap", [(0.9, 1, 1000), (0.5, 2, 3)])
def test_topp_select_block128(grid, H, d, key, p, kmin, kcap):
    spec = VideoSpec(1, H, d, grid, key)
    say("topp 128", grid, p)
    Q, K, _, _, got = run_select(spec, 128, "topp", p=p, k_min=kmin, k_cap=kcap)
    check_lists(Q, K, got, 128, "topp", p=p, k_min=kmin, k_cap=kcap)


PATTERNS = [
    dict(diagonals=[-3, 0, 2, 500, -500], columns=[0]),
    dict(diagonals=[1, -1], columns=[]),
    dict(diagonals=[], columns=[2, 1]),
]


@pytest.mark.parametrize("block", [64, 128])
@pytest.mark.parametrize("pat", range(len(PATTERNS)))
@pytest.mark.parametrize("r,na", [(0, 0), (1, 2)])
def test_static_window_with_patterns(block, pat, r, na):
    spec = VideoSpec(1, 2, 64, (6, 5, 13), 135)
    say("static + patterns", block, pat, r, na)
    st = dict(frame_tokens=spec.frame_tokens, window_frames=r, n_anchors=na, anchor_offset=5)
    pats = PATTERNS[pat]
    Q, K, _, _, got = run_select(spec, block, "static", static=st, patterns=pats)
    check_lists(Q, K, got, block, "static", static=st, patterns=pats)


@pytest.mark.parametrize("block", [64, 128])
def test_topk_with_patterns(block):
    spec = VideoSpec(1, 3, 128, (8, 6, 11), 136)
    say("topk + patterns", block)
    pats = dict(diagonals=[-2, 3], columns=[1])
    Q, K, _, _, got = run_select(spec, block, "topk", k=2, patterns=pats)
    check_lists(Q, K, got, block, "topk", k=2, patterns=pats)


def test_patterns_only_no_window():
    # STATIC mode with patterns alone: only the diagonals and columns
    spec = VideoSpec(1, 1, 64, (2, 8, 16), 137)
    pats = dict(diagonals=[0, -1], columns=[3])
    Q, K, _, _, got = run_select(spec, 64, "static", patterns=pats)
    nB = O.n_blocks(spec.N, 64)
    for i, row in enumerate(got[(0, 0)]):
        assert row == sorted(O.pattern_set(nB, i, [0, -1], [3]))


@pytest.mark.parametrize("grid,H,d,key", SMALL)
def test_attention_on_block128_rows(grid, H, d, key):
    spec = VideoSpec(1, H, d, grid, key)
    say("attention 128", grid, H, d)
    Q, K, V = gen_qkv(spec)
    N = spec.N
    rows128 = {}
    for h in range(H):
        _, rows128[h] = oracle_rows(Q, K, 0, h, 128, "topk", k=1,
                                    patterns=dict(diagonals=[2], columns=[]))
    if O.n_blocks(N, 128) > 1:
        rows128[0][1] = []   # an empty 128-row: two empty 64-rows
    allrows = [r for h in range(H) for r in O.expand_rows(rows128[h], N, 128, 64)]
    rp, ci = PT.rows_to_csr(allrows)
    Qd, Kd, Vd = (x.to(DEV) for x in (Q, K, V))
    Og, Lg = bsa.bsa_sparse_attn_fwd(Qd, Kd, Vd, rp.to(DEV), ci.to(DEV))
    torch.cuda.synchronize()
    for h in range(H):
        Oref, Lref = O.block_sparse_attention(PT.head64(Q, 0, h), PT.head64(K, 0, h),
                                              PT.head64(V, 0, h), rows128[h], 128,
                                              1 / math.sqrt(d))
        PT.compare_o_lse(Og[0, h], Lg[0, h], Oref, Lref, f"h{h}")


# ------------------------------------------------- full-size layers

def test_workload_block128_topk():
    """The 32K-token layer with 128-token blocks at 25% density: every list
    of every head, attention on sampled query blocks."""
    cfg = 1
    c = CONFIGS[cfg]
    spec = config_spec(cfg)
    Q, K, V = gen_qkv(spec)
    B, H, N, d = Q.shape
    nB = O.n_blocks(N, 128)
    k = bsa.budget_blocks(c["density"], nB)
    say(f"block-128 top-k on {c['name']}: k={k} of {nB}")
    Qd, Kd, Vd = (x.to(DEV) for x in (Q, K, V))
    sc = bsa.bsa_score_blocks(Qd, Kd, block=128)
    rp, ci, nnz = bsa.bsa_select_blocks(sc["scores"], Qd, block=128, mode="topk", k=k)
    torch.cuda.synchronize()
    got = gpu_rows64(rp, ci, nnz, B, H, N)
    exempt = check_lists(Q, K, got, 128, "topk", k=k)
    say(f"lists match, {exempt} tie-exempt rows")
    assert exempt <= max(2, B * H * nB // 1000)
    Og, Lg = bsa.bsa_sparse_attn_fwd(Qd, Kd, Vd, rp, ci)
    torch.cuda.synchronize()
    rng = np.random.default_rng(300)
    for h in (0, H - 1):
        q, kk, v = PT.head64(Q, 0, h), PT.head64(K, 0, h), PT.head64(V, 0, h)
        rows128 = collapse128(got[(0, h)], N)
        for I in sorted(set(rng.choice(nB, 3, replace=False).tolist()) | {nB - 1}):
            qi = O.block_tokens(N, 128, I)
            keys = np.concatenate([O.block_tokens(N, 128, J) for J in rows128[I]])
            Oref, Lref = O.attend(q[qi], kk[keys], v[keys], 1 / math.sqrt(d))
            PT.compare_o_lse(Og[0, h, qi[0]:qi[-1] + 1], Lg[0, h, qi[0]:qi[-1] + 1], Oref, Lref,
                             f"h{h} blk128 {I}")


@pytest.mark.parametrize("cfg,block", [(1, 128), (4, 128), (4, 64)])
def test_workload_mod_pattern_mask(cfg, block):
    """The MOD-style structural mask (intra-frame block-diagonal, temporal
    diagonals at 1 and 2 frames, 4 columns) on full-size layers: every list
    equals the oracle's; attention on sampled blocks of one head."""
    spec = config_spec(cfg)
    Q, K, V = gen_qkv(spec, heads=[0])
    B, H, N, d = Q.shape
    m = mod_pattern_mask(spec, block)
    say(f"MOD mask on {CONFIGS[cfg]['name']}, block {block}: {m['patterns']}")
    Qd, Kd, Vd = (x.to(DEV) for x in (Q, K, V))
    rp, ci, nnz = bsa.bsa_select_blocks(None, Qd, block=block, mode="static", **m)
    torch.cuda.synchronize()
    got = gpu_rows64(rp, ci, nnz, B, H, N)
    _, rows = oracle_rows(Q, K, 0, 0, block, "static", **m)
    g = got[(0, 0)] if block == 64 else collapse128(got[(0, 0)], N)
    assert g == rows
    nBs = O.n_blocks(N, block)
    say(f"density {O.density([rows], nBs):.4f}")
    Og, Lg = bsa.bsa_sparse_attn_fwd(Qd, Kd, Vd, rp, ci)
    torch.cuda.synchronize()
    q, kk, v = PT.head64(Q, 0, 0), PT.head64(K, 0, 0), PT.head64(V, 0, 0)
    rng = np.random.default_rng(301 + cfg)
    for I in sorted(set(rng.choice(nBs, 3, replace=False).tolist()) | {nBs - 1}):
        qi = O.block_tokens(N, block, I)
        keys = np.concatenate([O.block_tokens(N, block, J) for J in rows[I]])
        Oref, Lref = O.attend(q[qi], kk[keys], v[keys], 1 / math.sqrt(d))
        PT.compare_o_lse(Og[0, 0, qi[0]:qi[-1] + 1], Lg[0, 0, qi[0]:qi[-1] + 1], Oref, Lref,
                         f"blk {I}")
