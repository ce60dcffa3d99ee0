"""GPU parity of the pooled rectification of omitted blocks
(bsa_pooled_rectify) against the fp64 oracle, with the attention tolerances
(O max <= 1e-2, mean <= 1e-3, LSE <= 1e-3): small ragged shapes, both head
dims, float32 and bf16 outputs, strided layouts, rows that keep nothing and
rows that keep everything; the exact case (keys equal within every block:
rectified attention is full attention); the 32K-token layer at full size on
sampled query blocks.  The same with the gain-aware gate, whose (query,
block) decisions within a relative 1e-5 of the threshold are exempt: queries
with such a pair are left out of the element-wise comparison."""

import math
import sys

import numpy as np
import pytest
import torch

from oracle import bsa_oracle as O
from synth import CONFIGS, VideoSpec, config_spec, gen_qkv
import parity as PT

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import block_sparse_attention_pool_amd as bsa
else:  # collected on CPU, skipped by the marker
    bsa = None

DEV = "cuda:0"


def say(*a):
    print("[gpu-rectify]", *a, file=sys.stderr, flush=True)


def oracle_rows(Q, K, b, h, k, diag):
    N, d = Q.shape[2], Q.shape[3]
    q, kk = PT.head64(Q, b, h), PT.head64(K, b, h)
    S = O.pooled_scores(O.pool_means(q, 64), O.pool_means(kk, 64), 1 / math.sqrt(d))
    return O.select_rows(S, N, 64, "topk", k=k, force_diag=diag)


def run_case(Q, K, V, rows, out_dtype=torch.float32, strided=False):
    B, H, N, d = Q.shape
    if strided:
        Qd, Kd, Vd = [x.transpose(1, 2).contiguous().to(DEV).transpose(1, 2) for x in (Q, K, V)]
    else:
        Qd, Kd, Vd = (x.to(DEV) for x in (Q, K, V))
    rp, ci = PT.rows_to_csr([r for b in range(B) for h in range(H) for r in rows[(b, h)]])
    rp, ci = rp.to(DEV), ci.to(DEV)
    O_ = torch.empty_strided(Qd.shape, Qd.stride(), dtype=out_dtype, device=DEV)
    Og, Lg = bsa.bsa_sparse_attn_fwd(Qd, Kd, Vd, rp, ci, out=O_)
    L_sparse = Lg.clone()
    bsa.bsa_pooled_rectify(Qd, Kd, Vd, rp, ci, Og, Lg)
    torch.cuda.synchronize()
    return Og, Lg, L_sparse


SMALL = [
    ((3, 7, 9), 3, 128, 141),
    ((5, 15, 21), 2, 128, 142),
    ((4, 16, 16), 2, 64, 143),
    ((1, 1, 65), 1, 64, 144),
    ((2, 9, 50), 1, 128, 145),     # 900 tokens: 15 blocks, one partial 16-block step
]


@pytest.mark.parametrize("grid,H,d,key", SMALL)
@pytest.mark.parametrize("out_dtype,strided", [(torch.float32, False), (torch.bfloat16, True)])
def test_rectify_small(grid, H, d, key, out_dtype, strided):
    spec = VideoSpec(1, H, d, grid, key)
    say("rectify", grid, H, d, out_dtype, strided)
    Q, K, V = gen_qkv(spec)
    N = spec.N
    nB = O.n_blocks(N, 64)
    rows = {}
    for h in range(H):
        rows[(0, h)] = oracle_rows(Q, K, 0, h, 1, True)
        if nB > 2:
            rows[(0, h)][1] = []                      # keeps nothing: pooled keys only
            rows[(0, h)][nB - 1] = list(range(nB))    # keeps everything: unchanged
    Og, Lg, Ls = run_case(Q, K, V, rows, out_dtype, strided)
    for h in range(H):
        q, k, v = PT.head64(Q, 0, h), PT.head64(K, 0, h), PT.head64(V, 0, h)
        Oref, Lref = O.pooled_rectified_attention(q, k, v, rows[(0, h)], 64, 1 / math.sqrt(d))
        # a bf16 O is rounded by the sparse kernel's store and again by the
        # rectified store: two half-ulp roundings
        e = PT.compare_o_lse(Og[0, h], Lg[0, h], Oref, Lref, f"h{h}",
                             bf16=out_dtype == torch.bfloat16, roundings=2)
        say("   max/mean |dO|", e)
        if nB > 2:
            # a row that keeps every block is left exactly as it was
            t = O.block_tokens(N, 64, nB - 1)
            assert torch.equal(Lg[0, h, t[0]:t[-1] + 1], Ls[0, h, t[0]:t[-1] + 1])
    # the pooled part only adds mass
    assert bool((Lg >= Ls - 1e-6).all())


@pytest.mark.parametrize("d", [64, 128])
def test_rectify_exact_for_blockwise_constant_keys(d):
    spec = VideoSpec(1, 2, d, (3, 10, 13), 146)     # 390 tokens, ragged tail of 6
    Q, K, V = gen_qkv(spec)
    N = spec.N
    for j in range(O.n_blocks(N, 64)):
        t = torch.from_numpy(O.block_tokens(N, 64, j))
        K[:, :, t] = K[:, :, t[:1]]
    say("rectify exact case", d)
    rows = {(0, h): [[i] for i in range(O.n_blocks(N, 64))] for h in range(2)}
    Og, Lg, _ = run_case(Q, K, V, rows)
    for h in range(2):
        q, k, v = PT.head64(Q, 0, h), PT.head64(K, 0, h), PT.head64(V, 0, h)
        Oref, Lref = O.dense_attention(q, k, v, 1 / math.sqrt(d))
        PT.compare_o_lse(Og[0, h], Lg[0, h], Oref, Lref, f"h{h} vs full attention")


def test_rectify_workload_sampled():
    cfg = 1
    c = CONFIGS[cfg]
    spec = config_spec(cfg)
    Q, K, V = gen_qkv(spec)
    B, H, N, d = Q.shape
    nB = O.n_blocks(N, 64)
    k = bsa.budget_blocks(c["density"], nB)
    heads = [0, H - 1]
    say(f"rectify on {c['name']}: oracle lists of heads {heads}")
    rows = {(0, h): (oracle_rows(Q, K, 0, h, k, False) if h in heads else [[] for _ in range(nB)])
            for h in range(H)}
    Og, Lg, Ls = run_case(Q, K, V, rows)
    assert torch.isfinite(Lg).all() and bool((Lg >= Ls - 1e-6).all())
    rng = np.random.default_rng(400)
    scale = 1 / math.sqrt(d)
    for h in heads:
        q, kk, v = PT.head64(Q, 0, h), PT.head64(K, 0, h), PT.head64(V, 0, h)
        sampled = sorted(set(rng.choice(nB, 4, replace=False).tolist()) | {nB - 1})
        # the oracle's pooled part on the sampled rows only (a row that keeps
        # every block has no pooled part and costs nothing)
        rows_s = [rows[(0, h)][i] if i in sampled else list(range(nB)) for i in range(nB)]
        Op, Lp = O.pooled_omitted_attention(q, kk, v, rows_s, 64, scale)
        for i in sampled:
            qi = O.block_tokens(N, 64, i)
            keys = np.concatenate([O.block_tokens(N, 64, j) for j in rows[(0, h)][i]])
            Os, Lsr = O.attend(q[qi], kk[keys], v[keys], scale)
            Oref, Lref = O.lse_merge(Os, Lsr, Op[qi], Lp[qi])
            PT.compare_o_lse(Og[0, h, qi[0]:qi[-1] + 1], Lg[0, h, qi[0]:qi[-1] + 1], Oref, Lref,
                             f"h{h} blk{i}")


# ------------------------------------------------- the gain-aware gate

GATE_BAND = 1e-5  # relative: gate values this close to 2 ln 2 may go either way in float32


def _gated_case(Q, K, V, rows, out_dtype=torch.float32):
    B, H, N, d = Q.shape
    Qd, Kd, Vd = (x.to(DEV) for x in (Q, K, V))
    rp, ci = PT.rows_to_csr([r for b in range(B) for h in range(H) for r in rows[(b, h)]])
    rp, ci = rp.to(DEV), ci.to(DEV)
    O_ = torch.empty(Qd.shape, dtype=out_dtype, device=DEV)
    Og, Lg = bsa.bsa_sparse_attn_fwd(Qd, Kd, Vd, rp, ci, out=O_)
    Ls = Lg.clone()
    Os = Og.clone()
    bsa.bsa_pooled_rectify(Qd, Kd, Vd, rp, ci, Og, Lg, gain_gate=True)
    torch.cuda.synchronize()
    return Og, Lg, Os, Ls


def _check_gated_head(Og, Lg, q, k, v, rows, scale, what, bf16=False):
    """Compares the queries none of whose omitted blocks sits within
    GATE_BAND of the threshold; returns (compared, ambiguous, passed pairs,
    refused pairs)."""
    N = q.shape[0]
    nB = O.n_blocks(N, 64)
    sig2 = scale * scale * (q * q).sum(axis=1)[:, None] * O.block_key_spread(k, 64)[None, :]
    amb = np.abs(sig2 / O.GATE_SIGMA2 - 1.0) < GATE_BAND
    om = np.ones((N, nB), dtype=bool)
    for i, sel in enumerate(rows):
        t = O.block_tokens(N, 64, i)
        om[np.ix_(t, np.asarray(sel, dtype=np.int64))] = False
    bad = (amb & om).any(axis=1)
    Oref, Lref = O.pooled_rectified_attention(q, k, v, rows, 64, scale, gate=True)
    keep = ~bad
    kt = torch.from_numpy(keep)
    PT.compare_o_lse(Og.cpu()[kt], Lg.cpu()[kt], Oref[keep], Lref[keep], what, bf16=bf16,
                     roundings=2)
    G = sig2 < O.GATE_SIGMA2
    return int(keep.sum()), int(bad.sum()), int((G & om).sum()), int((~G & om).sum())


@pytest.mark.parametrize("grid,H,d,key,qscale", [((3, 7, 9), 2, 128, 151, 0.7),
                                                 ((4, 16, 16), 2, 64, 152, 0.8),
                                                 ((2, 9, 50), 1, 128, 153, 0.6),
                                                 ((1, 1, 65), 1, 64, 154, 1.0)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_rectify_gated_small(grid, H, d, key, qscale, out_dtype):
    """Queries scaled so that the gate passes some (query, block) pairs and
    refuses others; rows that keep nothing and rows that keep everything."""
    spec = VideoSpec(1, H, d, grid, key)
    say("rectify gated", grid, H, d, qscale, out_dtype)
    Q, K, V = gen_qkv(spec)
    Q = (Q.float() * qscale).to(torch.bfloat16)
    N = spec.N
    nB = O.n_blocks(N, 64)
    rows = {}
    for h in range(H):
        rows[(0, h)] = oracle_rows(Q, K, 0, h, 1, True)
        if nB > 2:
            rows[(0, h)][1] = []
            rows[(0, h)][nB - 1] = list(range(nB))
    Og, Lg, Os, Ls = _gated_case(Q, K, V, rows, out_dtype)
    scale = 1 / math.sqrt(d)
    tot_pass = tot_fail = 0
    for h in range(H):
        q, k, v = PT.head64(Q, 0, h), PT.head64(K, 0, h), PT.head64(V, 0, h)
        n, amb, npass, nfail = _check_gated_head(Og[0, h], Lg[0, h], q, k, v, rows[(0, h)], scale,
                                                 f"h{h}", bf16=out_dtype == torch.bfloat16)
        say(f"   h{h}: {n} queries compared, {amb} near the threshold; pairs passed {npass}, "
            f"refused {nfail}")
        tot_pass += npass
        tot_fail += nfail
        if nB > 2:
            t = O.block_tokens(N, 64, nB - 1)
            assert torch.equal(Lg[0, h, t[0]:t[-1] + 1], Ls[0, h, t[0]:t[-1] + 1])
    assert bool((Lg >= Ls - 1e-6).all())
    if N > 64:
        assert tot_pass > 0 and tot_fail > 0, "the gate should both pass and refuse here"


def test_rectify_gated_refusing_everything_keeps_the_sparse_result():
    """Queries so large that every pair fails the test: the result is the
    sparse result, bit for bit."""
    spec = VideoSpec(1, 2, 128, (3, 10, 13), 155)
    Q, K, V = gen_qkv(spec)
    Q = (Q.float() * 8.0).to(torch.bfloat16)
    nB = O.n_blocks(spec.N, 64)
    rows = {(0, h): [[i] for i in range(nB)] for h in range(2)}
    Og, Lg, Os, Ls = _gated_case(Q, K, V, rows)
    q, k = PT.head64(Q, 0, 0), PT.head64(K, 0, 0)
    assert not O.rectify_gate(q, k, 64, 1 / math.sqrt(128)).any()
    assert torch.equal(Og, Os) and torch.equal(Lg, Ls)


def test_rectify_gated_workload_sampled():
    """The 32K-token layer with its own (unscaled) queries: the gate on
    sampled query blocks of two heads against the oracle."""
    cfg = 1
    c = CONFIGS[cfg]
    spec = config_spec(cfg)
    Q, K, V = gen_qkv(spec)
    B, H, N, d = Q.shape
    nB = O.n_blocks(N, 64)
    kk_ = bsa.budget_blocks(c["density"], nB)
    heads = [0, H - 1]
    say(f"gated rectify on {c['name']}")
    rows = {(0, h): (oracle_rows(Q, K, 0, h, kk_, False) if h in heads else [[] for _ in range(nB)])
            for h in range(H)}
    Og, Lg, _, Ls = _gated_case(Q, K, V, rows)
    # (heads with empty rows may have every block refused: LSE -inf, O 0)
    assert not torch.isnan(Og).any() and bool((Lg >= Ls - 1e-6).all())
    rng = np.random.default_rng(401)
    scale = 1 / math.sqrt(d)
    for h in heads:
        q, kk, v = PT.head64(Q, 0, h), PT.head64(K, 0, h), PT.head64(V, 0, h)
        sampled = sorted(set(rng.choice(nB, 4, replace=False).tolist()) | {nB - 1})
        # the oracle's gated pooled part on the sampled rows only (rows that
        # keep every block have none), the sparse part per sampled block
        rows_s = [rows[(0, h)][i] if i in sampled else list(range(nB)) for i in range(nB)]
        Op, Lp = O.pooled_omitted_attention(q, kk, v, rows_s, 64, scale, gate=True)
        spread = O.block_key_spread(kk, 64)
        n_cmp = n_pairs = n_pass = 0
        for i in sampled:
            qi = O.block_tokens(N, 64, i)
            keys = np.concatenate([O.block_tokens(N, 64, j) for j in rows[(0, h)][i]])
            Os, Lsr = O.attend(q[qi], kk[keys], v[keys], scale)
            Oref, Lref = O.lse_merge(Os, Lsr, Op[qi], Lp[qi])
            om = np.ones(nB, dtype=bool)
            om[rows[(0, h)][i]] = False
            sig2 = scale * scale * (q[qi] * q[qi]).sum(axis=1)[:, None] * spread[None, om]
            amb = (np.abs(sig2 / O.GATE_SIGMA2 - 1.0) < GATE_BAND).any(axis=1)
            keep = torch.from_numpy(~amb)
            PT.compare_o_lse(Og[0, h, qi[0]:qi[-1] + 1].cpu()[keep],
                             Lg[0, h, qi[0]:qi[-1] + 1].cpu()[keep], Oref[~amb], Lref[~amb],
                             f"h{h} blk{i}")
            n_cmp += int((~amb).sum())
            n_pairs += sig2.size
            n_pass += int((sig2 < O.GATE_SIGMA2).sum())
        say(f"   h{h}: {n_cmp} queries compared; the gate passes {n_pass} of {n_pairs} pairs")
