"""GPU parity of the 3D local-window clustering (bsa_local_window_cluster)
against the fp64 oracle (HyperVAttention Algorithm 2).

Assignments are integer decisions taken on float32 distances; the oracle
takes them in float64.  A token whose oracle margin (second-nearest minus
nearest squared distance in its window) is below BAND may resolve either
way: it is exempt, and so are the centroids and counts of the clusters it
joins on either side.  The float32 distance error is about 1e-4 at these
sizes (d <= 128, squared distances of a few hundred), so BAND = 1e-3 leaves a
tenfold margin.  All other assignments and counts must be identical and
centroids agree to CENT_TOL (float32 means of up to a few thousand bf16
values).  Every case asserts that no exemption happened before the last
iteration (an earlier one would change everything after it)."""

import sys

import numpy as np
import pytest
import torch

from oracle import bsa_oracle as O
from synth import VideoSpec, config_spec, gen_qkv

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import block_sparse_attention_pool_amd as bsa
else:  # collected on CPU, skipped by the marker
    bsa = None

DEV = "cuda:0"
BAND = 1e-3
CENT_TOL = 1e-4


def say(*a):
    print("[gpu-cluster]", *a, file=sys.stderr, flush=True)


def initial_centroids(x, thw, cell, window):
    T, H, W = thw
    K, _ = O.cluster_grid(thw, cell, window)
    return np.stack([x[(min(ut * cell[0] + cell[0] // 2, T - 1) * H
                        + min(uh * cell[1] + cell[1] // 2, H - 1)) * W
                       + min(uw * cell[2] + cell[2] // 2, W - 1)]
                     for ut in range(K[0]) for uh in range(K[1]) for uw in range(K[2])])


def compare_head(x, thw, cell, window, iters, a_gpu, mu_gpu, c_gpu, what):
    # margins of every iteration's assignment, on the centroids it used
    mu_prev = initial_centroids(x, thw, cell, window)
    for it in range(1, iters + 1):
        margins = O.assignment_margins(x, thw, cell, window, mu_prev)
        if it < iters:
            assert margins.min() >= BAND, f"{what}: near-tie at iteration {it}; pick other inputs"
            _, mu_prev, _ = O.local_window_clustering(x, thw, cell, window, it)
    a, mu, c = O.local_window_clustering(x, thw, cell, window, iters)
    diff = np.nonzero(a != a_gpu)[0]
    assert np.all(margins[diff] < BAND), f"{what}: {len(diff)} assignments differ outside the tie band"
    touched = set(a[diff].tolist()) | set(a_gpu[diff].tolist())
    keep = np.array([u not in touched for u in range(len(c))])
    np.testing.assert_array_equal(c[keep], c_gpu[keep], err_msg=what)
    np.testing.assert_allclose(mu_gpu[keep], mu[keep], atol=CENT_TOL, rtol=0, err_msg=what)
    assert c_gpu.sum() == x.shape[0]
    return len(diff)


CASES = [
    # (grid, H, d, key, cell, window, iters)
    ((3, 7, 9), 1, 128, 151, (1, 3, 3), (2, 2, 2), 3),
    ((4, 16, 16), 2, 64, 152, (2, 4, 4), (2, 3, 3), 3),
    ((5, 15, 21), 1, 128, 153, (2, 5, 5), (3, 3, 3), 2),   # ragged cells on two axes
    ((6, 10, 13), 1, 64, 154, (3, 4, 4), (2, 2, 3), 4),
    ((2, 9, 50), 1, 128, 155, (1, 3, 7), (2, 3, 5), 2),    # window clipped on t
]


@pytest.mark.parametrize("grid,H,d,key,cell,window,iters", CASES)
def test_cluster_small(grid, H, d, key, cell, window, iters):
    spec = VideoSpec(1, H, d, grid, key)
    say("cluster", grid, cell, window, iters)
    Q, K, _ = gen_qkv(spec)
    for name, X in (("Q", Q), ("K", K)):
        a, mu, c = bsa.bsa_local_window_cluster(X.to(DEV), grid, cell, window, iters)
        torch.cuda.synchronize()
        for h in range(H):
            n = compare_head(X[0, h].double().numpy(), grid, cell, window, iters,
                             a[0, h].cpu().numpy(), mu[0, h].double().cpu().numpy(),
                             c[0, h].cpu().numpy(), f"{name} h{h}")
            say(f"   {name} h{h}: {n} tie-exempt tokens")


def test_cluster_strided_and_deterministic():
    spec = VideoSpec(2, 2, 128, (3, 8, 10), 156)
    Q, _, _ = gen_qkv(spec)
    Qs = Q.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)  # [B, N, H, d] storage
    cell, window = (1, 2, 3), (2, 3, 3)
    r1 = bsa.bsa_local_window_cluster(Qs, (3, 8, 10), cell, window, 3)
    r2 = bsa.bsa_local_window_cluster(Q.to(DEV), (3, 8, 10), cell, window, 3)
    torch.cuda.synchronize()
    for x, y in zip(r1, r2):
        assert torch.equal(x, y)
    for b in range(2):
        for h in range(2):
            compare_head(Q[b, h].double().numpy(), (3, 8, 10), cell, window, 3,
                         r1[0][b, h].cpu().numpy(), r1[1][b, h].double().cpu().numpy(),
                         r1[2][b, h].cpu().numpy(), f"b{b} h{h}")


@pytest.mark.parametrize("which,cell", [("Q", (11, 5, 5)), ("K", (11, 3, 3))])
def test_cluster_hunyuanvideo_layer(which, cell):
    """The 118,800-token HunyuanVideo layer with the page's grids (432 query,
    1215 key cells) and (3, 8, 8) windows; one head, one iteration."""
    spec = config_spec(3)
    Q, K, _ = gen_qkv(spec, heads=[0])
    X = Q if which == "Q" else K
    thw = spec.grid
    a, mu, c = bsa.bsa_local_window_cluster(X.to(DEV), thw, cell, (3, 8, 8), 1)
    torch.cuda.synchronize()
    say(f"HunyuanVideo {which}: {mu.shape[2]} cells; oracle running")
    n = compare_head(X[0, 0].double().numpy(), thw, cell, (3, 8, 8), 1, a[0, 0].cpu().numpy(),
                     mu[0, 0].double().cpu().numpy(), c[0, 0].cpu().numpy(), which)
    say(f"   {n} tie-exempt tokens of {spec.N}")


@pytest.mark.parametrize("grid,H,d,key,cell,window,iters", CASES[:3] + [
    ((33, 45, 80), 1, 128, 3, (11, 5, 5), (3, 8, 8), 1)])
def test_cluster_permutation(grid, H, d, key, cell, window, iters):
    """HVA Eq. 1 on the GPU's clustering: tokens in (cluster, index) order and
    the cluster offsets, identical to the oracle's stable sort of its own
    assignment (the assignments agree exactly on these inputs)."""
    spec = VideoSpec(1, H, d, grid, key)
    Q, _, _ = gen_qkv(spec, heads=[0])
    Qd = Q.to(DEV)
    a, mu, c = bsa.bsa_local_window_cluster(Qd, grid, cell, window, iters)
    perm, off = bsa.bsa_cluster_permute(a, c, Qd, grid, cell, window)
    torch.cuda.synchronize()
    x = Q[0, 0].double().numpy()
    ao, _, co = O.local_window_clustering(x, grid, cell, window, iters)
    assert np.array_equal(ao, a[0, 0].cpu().numpy()), "assignments differ: the case is not exact"
    po, offo = O.cluster_permutation(ao, len(co))
    np.testing.assert_array_equal(perm[0, 0].cpu().numpy(), po)
    np.testing.assert_array_equal(off[0, 0].cpu().numpy(), offo)


def _select_case(mu_q, mu_k, sizes, p, k_min, k_cap, what):
    """GPU cluster top-p on float32 centroids against the oracle on the same
    float32 values; lists compared with the top-p tie rules."""
    import parity as PT
    d = mu_q.shape[1]
    t = lambda x, dt: torch.from_numpy(np.ascontiguousarray(x)).to(dt).to(DEV)[None, None]
    rp, ci, nnz = bsa.bsa_cluster_select(t(mu_q, torch.float32), t(mu_k, torch.float32),
                                         t(sizes, torch.int32), p=p, k_min=k_min, k_cap=k_cap)
    torch.cuda.synchronize()
    got = bsa.csr_rows(rp, ci, nnz)
    q32 = mu_q.astype(np.float32).astype(np.float64)
    k32 = mu_k.astype(np.float32).astype(np.float64)
    rows = O.cluster_topp_rows(q32, k32, sizes, 1 / np.sqrt(d), p, k_min, k_cap)
    S = O.pooled_scores(q32, k32, 1 / np.sqrt(d))
    exempt = PT.compare_topp_rows(got, rows, S, np.asarray(sizes, np.float64), p, k_min, k_cap)
    say(f"   {what}: {sum(len(r) for r in rows)} entries, {exempt} tie-exempt rows")
    return exempt


@pytest.mark.parametrize("grid,H,d,key,cell,window,iters", CASES[:4])
@pytest.mark.parametrize("p,kmin_frac,cap_frac", [(0.9, 0.15, 1.0), (0.5, 0.0, 0.2)])
def test_cluster_select(grid, H, d, key, cell, window, iters, p, kmin_frac, cap_frac):
    spec = VideoSpec(1, H, d, grid, key)
    Q, K, _ = gen_qkv(spec, heads=[0])
    _, mu_q, _ = O.local_window_clustering(Q[0, 0].double().numpy(), grid, cell, window, iters)
    _, mu_k, c_k = O.local_window_clustering(K[0, 0].double().numpy(), grid,
                                             (cell[0], max(1, cell[1] - 1), cell[2]), window, iters)
    Nk = len(c_k)
    k_min = int(np.ceil(kmin_frac * Nk))
    k_cap = max(k_min, int(np.floor(cap_frac * Nk)))
    _select_case(mu_q, mu_k, c_k, p, k_min, k_cap, f"{grid} p={p}")


def test_cluster_select_hunyuanvideo_sizes():
    """The page's HunyuanVideo setting: 432 query and 1215 key clusters,
    top-p 0.9, Min-kc 0.15 (183 key clusters at least); seeded centroids and
    sizes summing to 118,800 tokens (some key clusters empty)."""
    rng = np.random.default_rng(310)
    mu_q = rng.standard_normal((432, 128)) * 0.7
    mu_k = rng.standard_normal((1215, 128)) * 0.7
    sizes = rng.multinomial(118800 - 1215 * 40, np.ones(1215) / 1215) + 40
    sizes[::97] = 0
    exempt = _select_case(mu_q, mu_k, sizes, 0.9, 183, 1215, "HunyuanVideo clusters")
    assert exempt <= 2


# ------------------------------------------------- attention over clusters

def _cluster_attn_case(Q, K, V, aq, ak, Nq, Nk, rows, out_dtype=torch.float32, sample=None,
                       groups=None, strided=False):
    """GPU Eq. 4 on oracle-made clusterings, lists (and merged groups)
    against the oracle; the executed tile pairs against Eq. 8 at a 16-token
    key grain."""
    import math
    import parity as PT
    N, d = Q.shape[2], Q.shape[3]
    pq, oq = O.cluster_permutation(aq, Nq)
    pk, ok = O.cluster_permutation(ak, Nk)
    rp, ci = PT.rows_to_csr(rows)
    t = lambda x: torch.from_numpy(np.asarray(x, dtype=np.int32)).to(DEV)
    gof = None
    if groups is not None:
        name = np.zeros(Nq, dtype=np.int32)
        for S in groups:
            name[S] = min(S)
        gof = t(name)[None, None]
    else:
        groups = [[i] for i in range(Nq)]
    if strided:  # [B, N, H, d] storage: Q, K, V and O through their strides
        Qd, Kd, Vd = (X.transpose(1, 2).contiguous().to(DEV).transpose(1, 2) for X in (Q, K, V))
    else:
        Qd, Kd, Vd = (X.to(DEV) for X in (Q, K, V))
    Og, Lg, pairs = bsa.bsa_cluster_attn_fwd(
        Qd, Kd, Vd, t(pq)[None, None], t(oq)[None, None], t(pk)[None, None],
        t(ok)[None, None], rp.to(DEV), ci.to(DEV), gof, out_dtype=out_dtype)
    torch.cuda.synchronize()
    rows = O.group_rows(groups, rows)
    assert int(pairs.item()) == O.packed_tile_pairs(oq, ok, groups, rows, 64, 16)
    q, k, v = (X[0, 0].double().numpy() for X in (Q, K, V))
    scale = 1 / math.sqrt(d)
    if sample is None:
        Oref, Lref = O.cluster_block_attention(q, k, v, pq, oq, pk, ok, rows, scale)
        PT.compare_o_lse(Og[0, 0], Lg[0, 0], Oref, Lref, "cluster attention",
                         bf16=out_dtype == torch.bfloat16)
    else:
        for i in sample:
            qi = pq[oq[i]:oq[i + 1]]
            if len(qi) == 0:
                continue
            keys = np.concatenate([pk[ok[j]:ok[j + 1]] for j in rows[i]] or [np.zeros(0, int)])
            Oref, Lref = O.attend(q[qi], k[keys], v[keys], scale)
            idx = torch.from_numpy(qi.astype(np.int64))
            PT.compare_o_lse(Og[0, 0][idx.to(DEV)], Lg[0, 0][idx.to(DEV)], Oref, Lref,
                             f"query cluster {i}")
    return int(pairs.item())


@pytest.mark.parametrize("grid,d,key,cq,ck,p", [((3, 7, 9), 128, 161, (1, 3, 3), (1, 2, 3), 0.9),
                                               ((4, 16, 16), 64, 162, (2, 4, 4), (2, 2, 4), 0.5),
                                               ((5, 15, 21), 128, 163, (2, 5, 5), (1, 5, 5), 0.7)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_cluster_attention_small(grid, d, key, cq, ck, p, out_dtype):
    import math
    spec = VideoSpec(1, 1, d, grid, key)
    Q, K, V = gen_qkv(spec)
    x, y = Q[0, 0].double().numpy(), K[0, 0].double().numpy()
    aq, mq, cnt_q = O.local_window_clustering(x, grid, cq, (2, 2, 2), 2)
    ak, mk, cnt_k = O.local_window_clustering(y, grid, ck, (2, 2, 2), 2)
    rows = O.cluster_topp_rows(mq, mk, cnt_k, 1 / math.sqrt(d), p, 1, len(cnt_k))
    rows[0] = []                                   # a query cluster with an empty row
    say("cluster attention", grid, len(cnt_q), "x", len(cnt_k), "clusters,",
        int((cnt_q == 0).sum()), "empty query clusters")
    _cluster_attn_case(Q, K, V, aq, ak, len(cnt_q), len(cnt_k), rows, out_dtype)


def test_cluster_pipeline_end_to_end():
    """GPU clustering, permutation, cluster top-p and Eq. 4 chained; the
    integer decisions equal the oracle's here, so the outputs must too."""
    import math
    import parity as PT
    grid, d, cq, ck, win = (4, 12, 16), 128, (2, 4, 4), (2, 3, 4), (2, 3, 3)
    spec = VideoSpec(1, 1, d, grid, 164)
    Q, K, V = gen_qkv(spec)
    Qd, Kd, Vd = (X.to(DEV) for X in (Q, K, V))
    aq, mq, cnt_q = bsa.bsa_local_window_cluster(Qd, grid, cq, win, 2)
    ak, mk, cnt_k = bsa.bsa_local_window_cluster(Kd, grid, ck, win, 2)
    pq, oq = bsa.bsa_cluster_permute(aq, cnt_q, Qd, grid, cq, win)
    pk, ok = bsa.bsa_cluster_permute(ak, cnt_k, Kd, grid, ck, win)
    Nk = cnt_k.shape[2]
    rp, ci, nnz = bsa.bsa_cluster_select(mq, mk, cnt_k, p=0.9, k_min=2, k_cap=Nk)
    Og, Lg, pairs = bsa.bsa_cluster_attn_fwd(Qd, Kd, Vd, pq, oq, pk, ok, rp, ci)
    torch.cuda.synchronize()
    x, y = Q[0, 0].double().numpy(), K[0, 0].double().numpy()
    aq_o, mq_o, cq_o = O.local_window_clustering(x, grid, cq, win, 2)
    ak_o, mk_o, ck_o = O.local_window_clustering(y, grid, ck, win, 2)
    assert np.array_equal(aq_o, aq[0, 0].cpu().numpy())
    assert np.array_equal(ak_o, ak[0, 0].cpu().numpy())
    rows = O.cluster_topp_rows(mq_o, mk_o, ck_o, 1 / math.sqrt(d), 0.9, 2, Nk)
    assert bsa.csr_rows(rp, ci, nnz) == rows, "cluster lists differ (a tie): pick other inputs"
    pq_o, oq_o = O.cluster_permutation(aq_o, len(cq_o))
    pk_o, ok_o = O.cluster_permutation(ak_o, len(ck_o))
    Oref, Lref = O.cluster_block_attention(x, y, V[0, 0].double().numpy(), pq_o, oq_o, pk_o,
                                           ok_o, rows, 1 / math.sqrt(d))
    PT.compare_o_lse(Og[0, 0], Lg[0, 0], Oref, Lref, "pipeline")
    assert int(pairs.item()) == O.packed_tile_pairs(oq_o, ok_o, [[i] for i in range(len(cq_o))],
                                                    rows, 64, 16)


def test_cluster_attention_hunyuanvideo_shape():
    """118,800 tokens in 432 query and 1215 key clusters (the page's counts;
    here each token's cluster is its grid cell), seeded cluster lists at
    about 15% of the key clusters; sampled query clusters against the
    oracle."""
    spec = config_spec(3)
    Q, K, V = gen_qkv(spec, heads=[0])
    T, H, W = spec.grid
    t, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    cell = lambda k: ((t // k[0]) * -(-H // k[1]) + y // k[1]) * -(-W // k[2]) + x // k[2]
    aq = cell((11, 5, 5)).reshape(-1)
    ak = cell((11, 3, 3)).reshape(-1)
    rng = np.random.default_rng(320)
    rows = [sorted(rng.choice(1215, size=int(rng.integers(120, 240)), replace=False).tolist())
            for _ in range(432)]
    pairs = _cluster_attn_case(Q, K, V, aq, ak, 432, 1215, rows,
                               sample=sorted(rng.choice(432, 6, replace=False).tolist()) + [431])
    say(f"HunyuanVideo shape: {pairs} tile pairs")


# ------------------------------------------------------- merging (Algorithm 1)

def _merge_case(sizes_q, sizes_k, rows, sides, N, tau_q=64, tau_k=64, grain=16):
    """GPU merging against the oracle's Algorithm 1: integer work, so the
    group of every cluster must be identical."""
    import parity as PT
    t = lambda x: torch.from_numpy(np.asarray(x, dtype=np.int32)).to(DEV)
    oq = np.concatenate([[0], np.cumsum(sizes_q)])
    ok = np.concatenate([[0], np.cumsum(sizes_k)])
    rp, ci = PT.rows_to_csr(rows)
    sd = torch.from_numpy(np.ascontiguousarray(sides)).to(DEV)
    gof = bsa.bsa_cluster_merge(t(oq)[None, None], t(ok)[None, None], rp.to(DEV), ci.to(DEV), sd,
                                N=N, tau_q=tau_q, tau_k=tau_k, grain=grain)
    torch.cuda.synchronize()
    grp, groups = O.agglomerative_merge(list(sizes_q), rows, list(sizes_k),
                                        np.asarray(sides)[0, 0].tolist(), tau_q, tau_k, grain)
    np.testing.assert_array_equal(gof[0, 0].cpu().numpy(), grp)
    return groups


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("tau_q,tau_k,grain", [(64, 64, 16), (64, 64, 1), (128, 96, 1)])
def test_cluster_merge_random(seed, tau_q, tau_k, grain):
    from synth import merge_sides
    rng = np.random.default_rng(500 + seed)
    Nq, Nk = int(rng.integers(2, 80)), int(rng.integers(1, 150))
    N = int(rng.integers(max(Nq, Nk), 20000))
    sq = rng.multinomial(N, np.ones(Nq) / Nq)
    sk = rng.multinomial(N, np.ones(Nk) / Nk)
    rows = [sorted(rng.choice(Nk, int(rng.integers(0, Nk + 1)), replace=False).tolist())
            for _ in range(Nq)]
    sides = merge_sides(600 + seed, 1, 1, 3, Nq)
    say(f"merge Nq={Nq} Nk={Nk} N={N} tau=({tau_q},{tau_k}) grain={grain}")
    groups = _merge_case(sq, sk, rows, sides, N, tau_q, tau_k, grain)
    say(f"   {Nq} clusters -> {len(groups)} groups")


def test_cluster_merge_hunyuanvideo_sizes():
    """The page's HunyuanVideo setting: 432 query and 1215 key clusters (the
    cells of the 118,800-token lattice), rows from cluster top-p 0.9 with
    Min-kc 0.15 (183 key clusters) on the cells' mean vectors of the first
    head, three rounds (the page's R = 3)."""
    import math
    from synth import merge_sides
    spec = config_spec(3)
    Q, K, _ = gen_qkv(spec, heads=[0])
    T, H, W = spec.grid
    t, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    cell = lambda k: ((t // k[0]) * -(-H // k[1]) + y // k[1]) * -(-W // k[2]) + x // k[2]
    aq, ak = cell((11, 5, 5)).reshape(-1), cell((11, 3, 3)).reshape(-1)
    sq, sk = np.bincount(aq, minlength=432), np.bincount(ak, minlength=1215)
    xq, xk = Q[0, 0].double().numpy(), K[0, 0].double().numpy()
    mq = np.stack([np.bincount(aq, weights=xq[:, c], minlength=432) for c in range(128)], 1)
    mk = np.stack([np.bincount(ak, weights=xk[:, c], minlength=1215) for c in range(128)], 1)
    rows = O.cluster_topp_rows(mq / sq[:, None], mk / sk[:, None], sk, 1 / math.sqrt(128), 0.9,
                               183, 1215)
    groups = _merge_case(sq, sk, rows, merge_sides(511, 1, 1, 3, 432), spec.N)
    before = O.partition_cost([[i] for i in range(432)], sq, rows, sk, 64, 64, 16)
    after = O.partition_cost(groups, sq, rows, sk, 64, 64, 16)
    say(f"   HunyuanVideo: {len(groups)} groups, cost {before} -> {after}")
    assert len(groups) < 432 and after < before


@pytest.mark.parametrize("out_dtype,strided", [(torch.float32, False), (torch.bfloat16, False),
                                               (torch.float32, True)])
def test_cluster_attention_merged_groups(out_dtype, strided):
    """Eq. 4 over merged groups (each member attends over the union of the
    group's rows) on an oracle-made clustering, oracle-merged."""
    import math
    from synth import merge_sides
    grid, d = (4, 16, 20), 128
    spec = VideoSpec(1, 1, d, grid, 171)
    Q, K, V = gen_qkv(spec)
    x, y = Q[0, 0].double().numpy(), K[0, 0].double().numpy()
    aq, mq, cnt_q = O.local_window_clustering(x, grid, (2, 4, 4), (2, 2, 2), 2)
    ak, mk, cnt_k = O.local_window_clustering(y, grid, (1, 4, 4), (2, 2, 2), 2)
    rows = O.cluster_topp_rows(mq, mk, cnt_k, 1 / math.sqrt(d), 0.8, 3, len(cnt_k))
    sides = merge_sides(172, 1, 1, 3, len(cnt_q))[0, 0].tolist()
    _, groups = O.agglomerative_merge(cnt_q.tolist(), rows, cnt_k.tolist(), sides, 64, 64, 16)
    assert any(len(S) > 1 for S in groups), "no merge happened: pick other inputs"
    say("merged attention", len(cnt_q), "clusters ->", len(groups), "groups")
    _cluster_attn_case(Q, K, V, aq, ak, len(cnt_q), len(cnt_k), rows, out_dtype, groups=groups,
                       strided=strided)


def test_cluster_pipeline_with_merging():
    """GPU clustering, permutation, cluster top-p, merging and Eq. 4 over the
    groups, chained, against the oracle's chain (decisions equal here)."""
    import math
    import parity as PT
    from synth import merge_sides
    grid, d, cq, ck, win = (4, 12, 16), 128, (2, 3, 4), (2, 3, 2), (2, 3, 3)
    spec = VideoSpec(1, 1, d, grid, 173)
    Q, K, V = gen_qkv(spec)
    Qd, Kd, Vd = (X.to(DEV) for X in (Q, K, V))
    aq, mq, cnt_q = bsa.bsa_local_window_cluster(Qd, grid, cq, win, 2)
    ak, mk, cnt_k = bsa.bsa_local_window_cluster(Kd, grid, ck, win, 2)
    pq, oq = bsa.bsa_cluster_permute(aq, cnt_q, Qd, grid, cq, win)
    pk, ok = bsa.bsa_cluster_permute(ak, cnt_k, Kd, grid, ck, win)
    Nq, Nk = cnt_q.shape[2], cnt_k.shape[2]
    rp, ci, nnz = bsa.bsa_cluster_select(mq, mk, cnt_k, p=0.85, k_min=2, k_cap=Nk)
    sides = torch.from_numpy(merge_sides(174, 1, 1, 3, Nq)).to(DEV)
    gof = bsa.bsa_cluster_merge(oq, ok, rp, ci, sides, N=spec.N)
    Og, Lg, pairs = bsa.bsa_cluster_attn_fwd(Qd, Kd, Vd, pq, oq, pk, ok, rp, ci, gof)
    torch.cuda.synchronize()
    x, y = Q[0, 0].double().numpy(), K[0, 0].double().numpy()
    aq_o, mq_o, cq_o = O.local_window_clustering(x, grid, cq, win, 2)
    ak_o, mk_o, ck_o = O.local_window_clustering(y, grid, ck, win, 2)
    assert np.array_equal(aq_o, aq[0, 0].cpu().numpy())
    assert np.array_equal(ak_o, ak[0, 0].cpu().numpy())
    rows = O.cluster_topp_rows(mq_o, mk_o, ck_o, 1 / math.sqrt(d), 0.85, 2, Nk)
    assert bsa.csr_rows(rp, ci, nnz) == rows, "cluster lists differ (a tie): pick other inputs"
    grp, groups = O.agglomerative_merge(cq_o.tolist(), rows, ck_o.tolist(),
                                        sides[0, 0].cpu().numpy().tolist(), 64, 64, 16)
    np.testing.assert_array_equal(gof[0, 0].cpu().numpy(), grp)
    say("pipeline with merging:", Nq, "clusters ->", len(groups), "groups")
    pq_o, oq_o = O.cluster_permutation(aq_o, len(cq_o))
    pk_o, ok_o = O.cluster_permutation(ak_o, len(ck_o))
    grows = O.group_rows(groups, rows)
    Oref, Lref = O.cluster_block_attention(x, y, V[0, 0].double().numpy(), pq_o, oq_o, pk_o,
                                           ok_o, grows, 1 / math.sqrt(d))
    PT.compare_o_lse(Og[0, 0], Lg[0, 0], Oref, Lref, "pipeline with merging")
    assert int(pairs.item()) == O.packed_tile_pairs(oq_o, ok_o, groups, grows, 64, 16)


# ------------------------------------------------------------ Lowe's ratio

# The two distances of a ratio are float32 sums of d <= 128 squared
# differences: a relative error of about d * 2^-24 ~ 1e-5 on each squared
# distance, about 1e-5 on rho in [0, 1] (a second-nearest centroid picked
# among candidates within float32 rounding of each other moves d_2 by less).
# 1e-4 leaves a tenfold margin.
RHO_TOL = 1e-4


def _lowe_case(X, thw, cell, window, iters, frac):
    """GPU ratios against the oracle's on the GPU's own float32 centroids
    (so the clustering's decisions do not enter), and the subset against the
    oracle's with the ratios within 2 RHO_TOL of the cut exempt."""
    Xd = X.to(DEV)
    _, mu, _ = bsa.bsa_local_window_cluster(Xd, thw, cell, window, iters)
    rho, sub = bsa.bsa_lowe_ratio_subset(Xd, mu, thw, cell, window, frac)
    torch.cuda.synchronize()
    B, H, N, _ = X.shape
    n = bsa.budget_blocks(frac, N)
    assert sub.shape[2] == n
    for h in range(H):
        ro = O.lowe_ratios(X[0, h].double().numpy(), thw, cell, window,
                           mu[0, h].double().cpu().numpy())
        rg = rho[0, h].double().cpu().numpy()
        err = np.abs(rg - ro).max()
        assert err <= RHO_TOL, f"head {h}: max |d rho| {err}"
        want = O.lowe_subset(ro, n)
        got = sub[0, h].cpu().numpy()
        assert np.all(np.diff(got) > 0), "subset not ascending"
        if n:
            cut = np.sort(ro)[::-1][n - 1]
            diff = set(got.tolist()) ^ set(want.tolist())
            assert all(abs(ro[i] - cut) <= 2 * RHO_TOL for i in diff), "subset differs off the tie band"
        say(f"   head {h}: max |d rho| {err:.2e}, subset {n} of {N}")


@pytest.mark.parametrize("grid,H,d,key,cell,window,iters", CASES)
def test_lowe_ratio_small(grid, H, d, key, cell, window, iters):
    spec = VideoSpec(1, H, d, grid, key)
    Q, _, _ = gen_qkv(spec)
    say("lowe", grid, cell, window)
    _lowe_case(Q, grid, cell, window, iters, 0.15)


def test_lowe_ratio_edges():
    """A window of one cell (every ratio 0, the subset the lowest indices),
    an empty and a full subset."""
    spec = VideoSpec(1, 1, 64, (2, 6, 8), 181)
    Q, _, _ = gen_qkv(spec)
    Qd = Q.to(DEV)
    thw, cell = (2, 6, 8), (1, 3, 4)
    _, mu, _ = bsa.bsa_local_window_cluster(Qd, thw, cell, (1, 1, 1), 2)
    rho, sub = bsa.bsa_lowe_ratio_subset(Qd, mu, thw, cell, (1, 1, 1), n_sub=10)
    torch.cuda.synchronize()
    assert bool((rho == 0).all()) and sub[0, 0].tolist() == list(range(10))
    _, mu, _ = bsa.bsa_local_window_cluster(Qd, thw, cell, (2, 2, 2), 2)
    rho0, sub0 = bsa.bsa_lowe_ratio_subset(Qd, mu, thw, cell, (2, 2, 2), n_sub=0)
    rho1, sub1 = bsa.bsa_lowe_ratio_subset(Qd, mu, thw, cell, (2, 2, 2), n_sub=96)
    torch.cuda.synchronize()
    assert sub0.shape[2] == 0 and sub1[0, 0].tolist() == list(range(96))
    assert torch.equal(rho0, rho1) and bool(((rho0 >= 0) & (rho0 <= 1)).all())


def test_lowe_ratio_hunyuanvideo_layer():
    """The 118,800-token HunyuanVideo lattice with the page's key grid (1215
    cells), window (3, 8, 8), the page's top 15% (17,820 tokens)."""
    spec = config_spec(3)
    _, K, _ = gen_qkv(spec, heads=[0])
    say("lowe on the HunyuanVideo key grid")
    _lowe_case(K[:, :1], spec.grid, (11, 3, 3), (3, 8, 8), 2, 0.15)


# ------------------------------------------------ fallback paths of the kernels

def test_cluster_cells_beyond_the_bucket_tables():
    """Cells of 2,560 tokens exceed the per-cell LDS table of the bucketed
    update and permutation: the box-scan kernels run instead; clustering and
    permutation against the oracle."""
    grid, cell, window = (2, 40, 96), (2, 40, 32), (1, 1, 2)
    spec = VideoSpec(1, 1, 64, grid, 191)
    Q, _, _ = gen_qkv(spec)
    Qd = Q.to(DEV)
    a, mu, c = bsa.bsa_local_window_cluster(Qd, grid, cell, window, 2)
    perm, off = bsa.bsa_cluster_permute(a, c, Qd, grid, cell, window)
    torch.cuda.synchronize()
    x = Q[0, 0].double().numpy()
    compare_head(x, grid, cell, window, 2, a[0, 0].cpu().numpy(), mu[0, 0].double().cpu().numpy(),
                 c[0, 0].cpu().numpy(), "large cells")
    po, offo = O.cluster_permutation(a[0, 0].cpu().numpy(), c.shape[2])
    np.testing.assert_array_equal(perm[0, 0].cpu().numpy(), po)
    np.testing.assert_array_equal(off[0, 0].cpu().numpy(), offo)


def test_cluster_window_beyond_the_assignment_table():
    """A window of 1,056 cells (more than the 1,024 the prefetching
    assignment tabulates, and more than the bucketed update's slot table):
    the plain matrix-core assignment and the box-scan update run instead;
    clustering and permutation against the oracle."""
    grid, cell, window = (1, 66, 64), (1, 2, 2), (1, 33, 32)
    spec = VideoSpec(1, 1, 64, grid, 193)
    Q, _, _ = gen_qkv(spec)
    Qd = Q.to(DEV)
    a, mu, c = bsa.bsa_local_window_cluster(Qd, grid, cell, window, 2)
    perm, off = bsa.bsa_cluster_permute(a, c, Qd, grid, cell, window)
    torch.cuda.synchronize()
    assert c.shape[2] == 33 * 32
    x = Q[0, 0].double().numpy()
    compare_head(x, grid, cell, window, 2, a[0, 0].cpu().numpy(), mu[0, 0].double().cpu().numpy(),
                 c[0, 0].cpu().numpy(), "window of 1056 cells")
    po, offo = O.cluster_permutation(a[0, 0].cpu().numpy(), c.shape[2])
    np.testing.assert_array_equal(perm[0, 0].cpu().numpy(), po)
    np.testing.assert_array_equal(off[0, 0].cpu().numpy(), offo)


def test_lowe_ratio_window_beyond_the_assignment_table():
    """Lowe's ratios over a window of 1,056 cells: the float32-FMA ratio pass
    runs instead of the matrix-core one; ratios and subset against the
    oracle."""
    grid, cell, window = (1, 66, 64), (1, 2, 2), (1, 33, 32)
    spec = VideoSpec(1, 1, 64, grid, 194)
    Q, _, _ = gen_qkv(spec)
    say("lowe, window of 1056 cells")
    _lowe_case(Q, grid, cell, window, 2, 0.15)


def test_cluster_permutation_of_a_cluster_beyond_lds():
    """Identical tokens: every distance ties and each token takes the lowest
    index of its window, so centroid 0 collects all 4,096 tokens of the 2 x 2
    cells of 1,024 -- more members than the bucketed permutation holds in
    LDS; the box scan places that cluster.  Both sides agree with the
    oracle."""
    grid, cell, window = (1, 64, 64), (1, 32, 32), (1, 3, 3)
    X = torch.full((1, 1, 64 * 64, 64), 0.5, dtype=torch.bfloat16)
    Xd = X.to(DEV)
    a, mu, c = bsa.bsa_local_window_cluster(Xd, grid, cell, window, 2)
    perm, off = bsa.bsa_cluster_permute(a, c, Xd, grid, cell, window)
    torch.cuda.synchronize()
    ao, _, co = O.local_window_clustering(X[0, 0].double().numpy(), grid, cell, window, 2)
    assert np.array_equal(ao, a[0, 0].cpu().numpy()) and co[0] == 4096
    po, offo = O.cluster_permutation(ao, len(co))
    np.testing.assert_array_equal(perm[0, 0].cpu().numpy(), po)
    np.testing.assert_array_equal(off[0, 0].cpu().numpy(), offo)


def test_cluster_pipeline_multi_head():
    """Two batches x two heads through the whole GPU chain (clustering,
    permutation, cluster top-p, merging, attention over the groups): every
    (b, h) against the oracle's chain on its own head, so that per-head
    offsets of every kernel are exercised."""
    import math
    import parity as PT
    from synth import merge_sides
    grid, d, cq, ck, win = (4, 12, 16), 64, (2, 3, 4), (2, 3, 2), (2, 3, 3)
    spec = VideoSpec(2, 2, d, grid, 175)
    Q, K, V = gen_qkv(spec)
    Qd, Kd, Vd = (X.to(DEV) for X in (Q, K, V))
    aq, mq, cnt_q = bsa.bsa_local_window_cluster(Qd, grid, cq, win, 2)
    ak, mk, cnt_k = bsa.bsa_local_window_cluster(Kd, grid, ck, win, 2)
    pq, oq = bsa.bsa_cluster_permute(aq, cnt_q, Qd, grid, cq, win)
    pk, ok = bsa.bsa_cluster_permute(ak, cnt_k, Kd, grid, ck, win)
    Nq, Nk = cnt_q.shape[2], cnt_k.shape[2]
    rp, ci, nnz = bsa.bsa_cluster_select(mq, mk, cnt_k, p=0.85, k_min=2, k_cap=Nk)
    sides_np = merge_sides(176, 2, 2, 3, Nq)
    gof = bsa.bsa_cluster_merge(oq, ok, rp, ci, torch.from_numpy(sides_np).to(DEV), N=spec.N)
    Og, Lg, pairs = bsa.bsa_cluster_attn_fwd(Qd, Kd, Vd, pq, oq, pk, ok, rp, ci, gof)
    torch.cuda.synchronize()
    rows_gpu = bsa.csr_rows(rp, ci, nnz)
    total_pairs = 0
    for b in range(2):
        for h in range(2):
            z = b * 2 + h
            x, y = Q[b, h].double().numpy(), K[b, h].double().numpy()
            aq_o, mq_o, cq_o = O.local_window_clustering(x, grid, cq, win, 2)
            ak_o, mk_o, ck_o = O.local_window_clustering(y, grid, ck, win, 2)
            assert np.array_equal(aq_o, aq[b, h].cpu().numpy()), f"b{b} h{h} query clusters"
            assert np.array_equal(ak_o, ak[b, h].cpu().numpy()), f"b{b} h{h} key clusters"
            rows = O.cluster_topp_rows(mq_o, mk_o, ck_o, 1 / math.sqrt(d), 0.85, 2, Nk)
            assert rows_gpu[z * Nq:(z + 1) * Nq] == rows, f"b{b} h{h}: cluster lists differ"
            grp, groups = O.agglomerative_merge(cq_o.tolist(), rows, ck_o.tolist(),
                                                sides_np[b, h].tolist(), 64, 64, 16)
            np.testing.assert_array_equal(gof[b, h].cpu().numpy(), grp)
            pq_o, oq_o = O.cluster_permutation(aq_o, len(cq_o))
            pk_o, ok_o = O.cluster_permutation(ak_o, len(ck_o))
            np.testing.assert_array_equal(pq[b, h].cpu().numpy(), pq_o)
            grows = O.group_rows(groups, rows)
            Oref, Lref = O.cluster_block_attention(x, y, V[b, h].double().numpy(), pq_o, oq_o,
                                                   pk_o, ok_o, grows, 1 / math.sqrt(d))
            PT.compare_o_lse(Og[b, h], Lg[b, h], Oref, Lref, f"b{b} h{h}")
            total_pairs += O.packed_tile_pairs(oq_o, ok_o, groups, grows, 64, 16)
            say(f"   b{b} h{h}: {Nq} clusters -> {len(groups)} groups")
    assert int(pairs.item()) == total_pairs


def test_cluster_merge_and_attention_at_the_cluster_limit():
    """4096 query and 4096 key clusters (the per-head maximum) over 65,536
    tokens with random assignments and rows: merging checked by what
    Algorithm 1 guarantees (a partition named by lowest members whose Eq. 9
    cost is not above the singletons'), attention over the GPU's groups
    against the oracle on sampled query clusters, executed pairs against
    Eq. 8."""
    import parity as PT
    from synth import merge_sides
    rng = np.random.default_rng(777)
    N, Nq, Nk, d = 65536, 4096, 4096, 64
    spec = VideoSpec(1, 1, d, (1, 64, 1024), 178)
    Q, K, V = gen_qkv(spec)
    aq = rng.integers(0, Nq, N)
    ak = rng.integers(0, Nk, N)
    rows = [sorted(rng.choice(Nk, int(rng.integers(1, 40)), replace=False).tolist())
            for _ in range(Nq)]
    pq, oq = O.cluster_permutation(aq, Nq)
    pk, ok = O.cluster_permutation(ak, Nk)
    t = lambda x: torch.from_numpy(np.asarray(x, dtype=np.int32)).to(DEV)[None, None]
    rp, ci = PT.rows_to_csr(rows)
    rp, ci = rp.to(DEV), ci.to(DEV)
    sides = torch.from_numpy(merge_sides(179, 1, 1, 3, Nq)).to(DEV)
    gof = bsa.bsa_cluster_merge(t(oq), t(ok), rp, ci, sides, N=N)
    Og, Lg, pairs = bsa.bsa_cluster_attn_fwd(Q.to(DEV), K.to(DEV), V.to(DEV), t(pq), t(oq), t(pk),
                                             t(ok), rp, ci, gof)
    torch.cuda.synchronize()
    g = gof[0, 0].cpu().numpy()
    groups = {}
    for i, name in enumerate(g.tolist()):
        groups.setdefault(name, []).append(i)
    assert all(name == min(S) for name, S in groups.items())
    groups = [groups[k] for k in sorted(groups)]
    sq, sk = np.diff(oq), np.diff(ok)
    before = O.partition_cost([[i] for i in range(Nq)], sq, rows, sk, 64, 64, 16)
    after = O.partition_cost(groups, sq, rows, sk, 64, 64, 16)
    say(f"cluster limit: {Nq} clusters -> {len(groups)} groups, cost {before} -> {after}")
    assert after <= before
    grows = O.group_rows(groups, rows)
    assert int(pairs.item()) == O.packed_tile_pairs(oq, ok, groups, grows, 64, 16)
    q, k, v = (X[0, 0].double().numpy() for X in (Q, K, V))
    for i in sorted(rng.choice(Nq, 6, replace=False).tolist()) + [Nq - 1]:
        qi = pq[oq[i]:oq[i + 1]]
        if len(qi) == 0:
            continue
        keys = np.concatenate([pk[ok[j]:ok[j + 1]] for j in grows[i]])
        Oref, Lref = O.attend(q[qi], k[keys], v[keys], 1 / np.sqrt(d))
        idx = torch.from_numpy(qi.astype(np.int64)).to(DEV)
        PT.compare_o_lse(Og[0, 0][idx], Lg[0, 0][idx], Oref, Lref, f"query cluster {i}")


# ------------------------------------------- subset refinement (HVA 4.2)

def _refine_case(X0, X1, thw, cell, window, iters, frac, what):
    """Anchor step on X0 (clustering and Lowe subset on the GPU), refinement
    with X1 on the GPU against the oracle's refinement of the same state.
    A subset token whose oracle margin over all centroids is below BAND is
    exempt together with the centroids it touches."""
    X0d, X1d = X0.to(DEV), X1.to(DEV)
    a0, mu0, c0 = bsa.bsa_local_window_cluster(X0d, thw, cell, window, iters)
    _, sub = bsa.bsa_lowe_ratio_subset(X0d, mu0, thw, cell, window, frac)
    a1, mu1, c1 = bsa.bsa_subset_refine(X1d, sub, a0.clone(), mu0.clone(), c0.clone())
    torch.cuda.synchronize()
    B, H, N, _ = X0.shape
    moved_tot = 0
    for h in range(H):
        x = X1[0, h].double().numpy()
        a_in = a0[0, h].cpu().numpy()
        mu_in = mu0[0, h].double().cpu().numpy()
        S = sub[0, h].cpu().numpy()
        a, mu, c = O.subset_refinement(x, a_in, mu_in, S)
        ag, mug, cg = a1[0, h].cpu().numpy(), mu1[0, h].double().cpu().numpy(), c1[0, h].cpu().numpy()
        # margins over every centroid for the subset tokens
        d2 = ((x[S][:, None, :] - mu_in[None]) ** 2).sum(-1)
        d2.sort(axis=1)
        margin = d2[:, 1] - d2[:, 0] if d2.shape[1] > 1 else np.full(len(S), np.inf)
        diff = np.nonzero(a != ag)[0]
        assert np.all(np.isin(diff, S)), f"{what} h{h}: a token outside the subset changed"
        sub_pos = {int(t): k for k, t in enumerate(S)}
        assert all(margin[sub_pos[int(t)]] < BAND for t in diff), \
            f"{what} h{h}: {len(diff)} refined assignments differ outside the tie band"
        touched = set(a[diff].tolist()) | set(ag[diff].tolist()) | set(a_in[diff].tolist())
        keep = np.array([u not in touched for u in range(len(c))])
        np.testing.assert_array_equal(c[keep], cg[keep], err_msg=what)
        np.testing.assert_allclose(mug[keep], mu[keep], atol=CENT_TOL, rtol=0, err_msg=what)
        assert cg.sum() == N
        moved = int((a[S] != a_in[S]).sum())
        moved_tot += moved
        say(f"   {what} h{h}: subset {len(S)}, moved {moved}, {len(diff)} near-tie differences")
    return moved_tot


REFINE_CASES = [
    # (grid, H, d, key, cell, window, iters, perturbation)
    ((3, 7, 9), 2, 128, 251, (1, 3, 3), (2, 2, 2), 2, 0.5),
    ((4, 16, 16), 1, 64, 252, (2, 4, 4), (2, 3, 3), 3, 0.8),
    ((2, 9, 50), 1, 128, 253, (1, 3, 7), (2, 3, 5), 2, 0.5),
]


@pytest.mark.parametrize("grid,H,d,key,cell,window,iters,pert", REFINE_CASES)
def test_subset_refine_small(grid, H, d, key, cell, window, iters, pert):
    spec = VideoSpec(1, H, d, grid, key)
    Q, _, _ = gen_qkv(spec)
    g = torch.Generator().manual_seed(key)
    # a later denoising step: the same tokens, perturbed
    Q1 = (Q.float() + pert * torch.randn(Q.shape, generator=g)).to(torch.bfloat16)
    say("subset refine", grid, H, d)
    moved = _refine_case(Q, Q1, grid, cell, window, iters, 0.15, f"{grid}")
    assert moved > 0, "the perturbation should move some subset tokens"


def test_subset_refine_empty_and_full_subsets():
    spec = VideoSpec(1, 1, 64, (3, 8, 8), 254)
    Q, _, _ = gen_qkv(spec)
    Qd = Q.to(DEV)
    thw, cell, window = (3, 8, 8), (1, 4, 4), (2, 2, 2)
    a0, mu0, c0 = bsa.bsa_local_window_cluster(Qd, thw, cell, window, 2)
    empty = torch.zeros((1, 1, 0), dtype=torch.int32, device=DEV)
    a1, mu1, c1 = bsa.bsa_subset_refine(Qd, empty, a0.clone(), mu0.clone(), c0.clone())
    torch.cuda.synchronize()
    assert torch.equal(a1, a0) and torch.equal(mu1, mu0) and torch.equal(c1, c0)
    # every token in the subset, centroids the members' means: one Lloyd step
    full = torch.arange(spec.N, dtype=torch.int32, device=DEV).view(1, 1, -1)
    Q1 = (Q.float() + 0.7 * torch.randn(Q.shape, generator=torch.Generator().manual_seed(3))).to(
        torch.bfloat16)
    _refine_case(Q, Q1, thw, cell, window, 2, 1.0, "full subset")


def test_subset_refine_hunyuanvideo_key_grid():
    """The 118,800-token HunyuanVideo lattice with the page's key grid (1215
    cells), window (3, 8, 8), 2 iterations at the anchor step, the page's top
    15% (17,820 tokens) refined against all 1215 centroids at a perturbed
    later step."""
    spec = config_spec(3)
    _, K, _ = gen_qkv(spec, heads=[0])
    K = K[:, :1]
    K1 = (K.float() + 0.3 * torch.randn(K.shape, generator=torch.Generator().manual_seed(31))).to(
        torch.bfloat16)
    say("subset refine on the HunyuanVideo key grid")
    _refine_case(K, K1, spec.grid, (11, 3, 3), (3, 8, 8), 2, 0.15, "hunyuanvideo")
