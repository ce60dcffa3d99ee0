"""GPU parity: every stage of the HIP path against the fp64 oracle on the same
seeded bf16 inputs.  Small shapes (several tiles, ragged tails, both head
dims, strided layouts, empty rows) are checked element by element; the
five workloads at full size are checked on every block list (every macro
row of every head; every micro row of two micro heads) and on sampled
attention rows."""

import math
import sys

import numpy as np
import pytest
import torch

from oracle import bsa_oracle as O
from synth import CONFIGS, VideoSpec, config_spec, gen_qkv, micro_heads, rotation_offset
import parity as PT

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import block_sparse_attention_pool_amd as bsa
else:  # collected on CPU, skipped by the marker
    bsa = None

DEV = "cuda:0"


def say(*a):
    print("[gpu-parity]", *a, file=sys.stderr, flush=True)


def to_dev(*ts):
    return [t.to(DEV) for t in ts]


def oracle_rows_all(Q, K, spec, mode, *, k=0, p=0.9, k_min=1, k_cap=None, force_diag=False,
                    static=None, heads=None):
    """Oracle scores and lists for the given heads of batch 0..B-1."""
    B, H, N, d = Q.shape
    scale = 1.0 / math.sqrt(d)
    out = {}
    for b in range(B):
        for h in (range(H) if heads is None else heads):
            if mode == "static":
                S = None
            else:
                _, _, S = PT.oracle_scores(Q, K, b, h, 64, scale)
            rows = O.select_rows(S, N, 64, mode, k=k, p=p, k_min=k_min, k_cap=k_cap,
                                 force_diag=force_diag, static=static)
            out[(b, h)] = (S, rows)
    return out


def forced_rows(N, force_diag, static):
    nB = O.n_blocks(N, 64)
    rows = []
    for i in range(nB):
        f = set()
        if force_diag:
            f.add(i)
        if static is not None:
            f |= O.window_anchor_set(N, 64, i, **static)
        rows.append(f)
    return rows


def gpu_rows_by_head(row_ptr, col_idx, nnz, B, H, nB):
    rows = bsa.csr_rows(row_ptr, col_idx, nnz)
    return {(b, h): rows[(b * H + h) * nB:(b * H + h + 1) * nB] for b in range(B) for h in range(H)}


# ------------------------------------------------------------- small shapes

SMALL = [
    # (grid, H, d, key) -- ragged tails of 61, 39, 0 and 1 tokens
    ((3, 7, 9), 3, 128, 101),
    ((5, 15, 21), 2, 128, 102),
    ((4, 16, 16), 2, 64, 103),
    ((1, 1, 65), 1, 64, 104),
]


@pytest.mark.parametrize("grid,H,d,key", SMALL)
def test_pool_and_scores(grid, H, d, key):
    spec = VideoSpec(1, H, d, grid, key)
    say("pool/score", grid, H, d)
    Q, K, _ = gen_qkv(spec)
    Qd, Kd = to_dev(Q, K)
    sc = bsa.bsa_score_blocks(Qd, Kd, micro=16)
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(d)
    for h in range(H):
        q, k = PT.head64(Q, 0, h), PT.head64(K, 0, h)
        Qb, Kb, S = PT.oracle_scores(Q, K, 0, h, 64, scale)
        np.testing.assert_allclose(sc["qpool"][0, h].double().cpu().numpy(), Qb, atol=2e-6)
        np.testing.assert_allclose(sc["kpool"][0, h].double().cpu().numpy(), Kb, atol=2e-6)
        np.testing.assert_allclose(sc["scores"][0, h].double().cpu().numpy(), S, atol=1e-5)
        np.testing.assert_allclose(sc["qpool16"][0, h].double().cpu().numpy(),
                                   O.pool_means(q, 16), atol=2e-6)
        np.testing.assert_allclose(sc["kpool16"][0, h].double().cpu().numpy(),
                                   O.pool_means(k, 16), atol=2e-6)


def test_scores_strided_token_major_layout():
    # [B, N, H, d] storage viewed as [B, H, N, d]
    spec = VideoSpec(2, 3, 128, (3, 10, 13), 105)
    say("pool/score strided")
    Q, K, _ = gen_qkv(spec)
    Qs = Q.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
    Ks = K.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
    sc = bsa.bsa_score_blocks(Qs, Ks)
    torch.cuda.synchronize()
    for b in range(2):
        for h in range(3):
            _, _, S = PT.oracle_scores(Q, K, b, h, 64, 1 / math.sqrt(128))
            np.testing.assert_allclose(sc["scores"][b, h].double().cpu().numpy(), S, atol=1e-5)


def _select_case(spec, mode, **kw):
    Q, K, V = gen_qkv(spec)
    Qd, Kd = to_dev(Q, K)
    B, H, N, d = Q.shape
    nB = O.n_blocks(N, 64)
    sc = bsa.bsa_score_blocks(Qd, Kd, scores=(mode != "static"))
    rp, ci, nnz = bsa.bsa_select_blocks(sc["scores"], Qd, mode=mode, **kw)
    torch.cuda.synchronize()
    got = gpu_rows_by_head(rp, ci, nnz, B, H, nB)
    ora = oracle_rows_all(Q, K, spec, mode, **kw)
    return Q, K, V, got, ora


@pytest.mark.parametrize("grid,H,d,key", SMALL)
@pytest.mark.parametrize("k,diag", [(1, True), (2, False), (0, True), (99, False)])
def test_topk_select(grid, H, d, key, k, diag):
    spec = VideoSpec(1, H, d, grid, key)
    say("topk", grid, k, diag)
    N = spec.N
    _, _, _, got, ora = _select_case(spec, "topk", k=k, force_diag=diag)
    F = forced_rows(N, diag, None)
    for bh, (S, rows) in ora.items():
        PT.compare_topk_rows(got[bh], rows, S, k, F)


@pytest.mark.parametrize("grid,H,d,key", SMALL[:3])
@pytest.mark.parametrize("p,kmin,kcap", [(0.9, 1, 1000), (0.5, 2, 3), (0.99, 1, 1)])
def test_topp_select(grid, H, d, key, p, kmin, kcap):
    spec = VideoSpec(1, H, d, grid, key)
    say("topp", grid, p, kmin, kcap)
    _, _, _, got, ora = _select_case(spec, "topp", p=p, k_min=kmin, k_cap=kcap)
    sizes = O.block_sizes(spec.N, 64)
    for bh, (S, rows) in ora.items():
        PT.compare_topp_rows(got[bh], rows, S, sizes, p, kmin, kcap)


@pytest.mark.parametrize("grid,r,na,off", [((6, 5, 13), 1, 4, 7), ((9, 4, 9), 0, 3, -2),
                                           ((6, 5, 13), 2, 0, 0)])
def test_static_select(grid, r, na, off):
    spec = VideoSpec(1, 2, 64, grid, 106)
    say("static", grid, r, na, off)
    st = dict(frame_tokens=spec.frame_tokens, window_frames=r, n_anchors=na, anchor_offset=off)
    _, _, _, got, ora = _select_case(spec, "static", static=st)
    for bh, (_, rows) in ora.items():
        assert got[bh] == rows


@pytest.mark.parametrize("mode,kw", [("topk", dict(k=3)), ("topk", dict(k=2, force_diag=True)),
                                     ("topp", dict(p=0.8, k_min=1, k_cap=6))])
def test_select_two_batches(mode, kw):
    """B = 2: rows of both batches (plain top-k takes the direct CSR path,
    the others the counted one)."""
    spec = VideoSpec(2, 2, 64, (3, 9, 21), 119)
    say("select two batches", mode, kw)
    _, _, _, got, ora = _select_case(spec, mode, **kw)
    assert len(ora) == 4
    for bh, (S, rows) in ora.items():
        if mode == "topk":
            PT.compare_topk_rows(got[bh], rows, S, kw["k"],
                                 forced_rows(spec.N, kw.get("force_diag", False), None))
        else:
            PT.compare_topp_rows(got[bh], rows, S, O.block_sizes(spec.N, 64), kw["p"],
                                 kw["k_min"], kw["k_cap"])


# Rows of 300 to 4096 key blocks: the one-wave-per-row selection with a
# partial last bitmask word (300 = 9 words + 12 bits) and with 8, 12, 16,
# 20, 24, 28, 32, 40, 48, 56 and 64 keys per lane.
@pytest.mark.parametrize("grid,k,diag", [((3, 10, 640), 75, False), ((3, 10, 640), 400, True),
                                         ((7, 40, 160), 175, True), ((5, 50, 300), 293, False),
                                         ((5, 50, 512), 500, True), ((5, 64, 512), 384, False),
                                         ((7, 64, 512), 540, True), ((6, 50, 300), 300, False),
                                         ((6, 64, 480), 700, True), ((8, 64, 512), 1000, False),
                                         ((4, 40, 380), 250, True)])
def test_topk_select_long_rows(grid, k, diag):
    spec = VideoSpec(1, 1, 64, grid, 108)
    say("topk long rows", grid, k, diag)
    _, _, _, got, ora = _select_case(spec, "topk", k=k, force_diag=diag)
    F = forced_rows(spec.N, diag, None)
    for bh, (S, rows) in ora.items():
        PT.compare_topk_rows(got[bh], rows, S, k, F)


@pytest.mark.parametrize("grid,p,kmin,kcap", [((7, 40, 160), 0.9, 1, 140), ((5, 50, 512), 0.9, 1, 400),
                                               ((5, 50, 512), 0.5, 3, 2000), ((3, 10, 640), 0.99, 1, 60),
                                               ((6, 50, 350), 0.9, 1, 330), ((5, 50, 300), 0.8, 2, 240),
                                               ((8, 64, 512), 0.9, 1, 820)])
def test_topp_select_long_rows(grid, p, kmin, kcap):
    spec = VideoSpec(1, 1, 64, grid, 110)
    say("topp long rows", grid, p, kmin, kcap)
    _, _, _, got, ora = _select_case(spec, "topp", p=p, k_min=kmin, k_cap=kcap)
    sizes = O.block_sizes(spec.N, 64)
    for bh, (S, rows) in ora.items():
        PT.compare_topp_rows(got[bh], rows, S, sizes, p, kmin, kcap)


@pytest.mark.parametrize("grid,r,na,off", [((7, 40, 160), 1, 5, 3), ((5, 50, 512), 0, 7, -4)])
def test_static_select_long_rows(grid, r, na, off):
    spec = VideoSpec(1, 1, 64, grid, 109)
    say("static long rows", grid, r, na, off)
    st = dict(frame_tokens=spec.frame_tokens, window_frames=r, n_anchors=na, anchor_offset=off)
    _, _, _, got, ora = _select_case(spec, "static", static=st)
    for bh, (_, rows) in ora.items():
        assert got[bh] == rows


def test_topk_plus_static_union():
    spec = VideoSpec(1, 2, 128, (8, 6, 11), 107)
    say("topk + static")
    st = dict(frame_tokens=spec.frame_tokens, window_frames=1, n_anchors=2, anchor_offset=3)
    _, _, _, got, ora = _select_case(spec, "topk", k=2, force_diag=True, static=st)
    F = forced_rows(spec.N, True, st)
    for bh, (S, rows) in ora.items():
        PT.compare_topk_rows(got[bh], rows, S, 2, F)


def _attn_case(spec, rows_of_head, out_dtype=torch.float32, strided=False):
    Q, K, V = gen_qkv(spec)
    B, H, N, d = Q.shape
    if strided:
        Qd, Kd, Vd = [x.transpose(1, 2).contiguous().to(DEV).transpose(1, 2) for x in (Q, K, V)]
    else:
        Qd, Kd, Vd = to_dev(Q, K, V)
    allrows = [r for b in range(B) for h in range(H) for r in rows_of_head(b, h)]
    rp, ci = PT.rows_to_csr(allrows)
    Og, Lg = bsa.bsa_sparse_attn_fwd(Qd, Kd, Vd, rp.to(DEV), ci.to(DEV), out_dtype=out_dtype)
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(d)
    for b in range(B):
        for h in range(H):
            Oref, Lref = O.block_sparse_attention(PT.head64(Q, b, h), PT.head64(K, b, h),
                                                  PT.head64(V, b, h), rows_of_head(b, h), 64,
                                                  scale)
            e = PT.compare_o_lse(Og[b, h], Lg[b, h], Oref, Lref, f"b{b}h{h}",
                                 bf16=out_dtype == torch.bfloat16)
            say("   max/mean |dO|", e)


@pytest.mark.parametrize("grid,H,d,key", SMALL)
def test_sparse_attention_random_rows(grid, H, d, key):
    spec = VideoSpec(1, H, d, grid, key)
    say("sparse attn", grid, H, d)
    nB = O.n_blocks(spec.N, 64)
    rng = np.random.default_rng(key)
    table = {}

    def rows_of(b, h):
        if (b, h) not in table:
            rows = []
            for i in range(nB):
                n = int(rng.integers(0, nB + 1))
                rows.append(sorted(rng.choice(nB, size=n, replace=False).tolist()))
            table[(b, h)] = rows
        return table[(b, h)]

    _attn_case(spec, rows_of)


def test_staged_v_equals_inline_staging():
    """bsa_attn_stage_v on its own stream, then the attention with V=None,
    gives the bits of the attention that stages V itself (strided V too)."""
    spec = VideoSpec(2, 3, 128, (3, 9, 21), 109)
    Q, K, V = (x.to(DEV) for x in gen_qkv(spec))
    Vs = V.transpose(1, 2).contiguous().transpose(1, 2)  # [B, N, H, d] storage
    nB = O.n_blocks(spec.N, 64)
    rows = [sorted({i, (i * 7) % nB, 0}) for i in range(nB)]
    rp, ci = PT.rows_to_csr([r for _ in range(spec.B * spec.H) for r in rows])
    rp, ci = rp.to(DEV), ci.to(DEV)
    O1, L1 = bsa.bsa_sparse_attn_fwd(Q, K, V, rp, ci)
    ws = bsa.attn_workspace(Q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bsa.bsa_attn_stage_v(Vs, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    O2, L2 = bsa.bsa_sparse_attn_fwd(Q, K, None, rp, ci, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(L1, L2)


def test_sparse_attention_bf16_out_strided_and_empty_rows():
    spec = VideoSpec(2, 2, 128, (4, 9, 11), 108)
    say("sparse attn bf16/strided/empty")
    nB = O.n_blocks(spec.N, 64)

    def rows_of(b, h):
        return [[] if i % 3 == 0 else sorted({i, (i + b + h) % nB, 0}) for i in range(nB)]

    _attn_case(spec, rows_of, out_dtype=torch.bfloat16, strided=True)
    _attn_case(spec, rows_of, out_dtype=torch.float32, strided=True)


@pytest.mark.parametrize("grid,H,d,key", SMALL)
def test_dense_attention(grid, H, d, key):
    spec = VideoSpec(1, H, d, grid, key)
    say("dense attn", grid, H, d)
    Q, K, V = gen_qkv(spec)
    Og, Lg = bsa.bsa_dense_attn_fwd(*to_dev(Q, K, V))
    torch.cuda.synchronize()
    for h in range(H):
        Oref, Lref = O.dense_attention(PT.head64(Q, 0, h), PT.head64(K, 0, h),
                                       PT.head64(V, 0, h), 1 / math.sqrt(d))
        PT.compare_o_lse(Og[0, h], Lg[0, h], Oref, Lref, f"h{h}")


def _micro_oracle(Q, K, spec, rows, m, heads):
    B, H, N, d = Q.shape
    scale = 1 / math.sqrt(d)
    out = {}
    for h in heads:
        q, k = PT.head64(Q, 0, h), PT.head64(K, 0, h)
        Qt, Kt = O.pool_means(q, 16), O.pool_means(k, 16)
        out[h] = (Qt, Kt, [O.micro_select_row(Qt, Kt, rows[h][i], i, N, 64, 16, scale, m)
                           for i in range(len(rows[h]))])
    return out


def compare_micro_rows(got_rows, ora_rows, Qt, Kt, macro_rows, N, scale, m, blocks=None):
    """Rows given in query-block order, or for the query blocks ``blocks``."""
    exempt = 0
    for i, (g, o) in enumerate(zip(got_rows, ora_rows)):
        if g == o:
            continue
        blk = i if blocks is None else blocks[i]
        cand = O.micro_candidates(Qt, Kt, macro_rows[i], blk, N, 64, 16, scale)
        cand.sort(key=lambda t: (-t[0], t[1]))
        thr = cand[min(m, len(cand)) - 1][0]
        sig = {c: s for s, c in cand}
        bad = [c for c in set(g) ^ set(o) if abs(sig.get(c, math.inf) - thr) > PT.TIE_BAND]
        assert not bad, f"micro row {i}: {g} vs {o}"
        # order must still be (sub-tile, key tile)
        assert g == sorted(g, key=lambda c: (c % 4, c // 4))
        exempt += 1
    return exempt


@pytest.mark.parametrize("grid,H,d,key,m", [((3, 7, 9), 2, 128, 111, 5), ((4, 16, 16), 2, 64, 112, 8),
                                            ((2, 8, 13), 3, 128, 113, 1000)])
def test_micro_select_attention_and_merge(grid, H, d, key, m):
    spec = VideoSpec(1, H, d, grid, key, spikes=True)
    say("micro", grid, H, d, m)
    Q, K, V = gen_qkv(spec)
    Qd, Kd, Vd = to_dev(Q, K, V)
    N = spec.N
    nB = O.n_blocks(N, 64)
    scale = 1 / math.sqrt(d)
    heads = [0, H - 1] if H > 1 else [0]
    mask = [h in heads for h in range(H)]
    # macro lists from the oracle (inputs to both sides)
    ora = oracle_rows_all(Q, K, spec, "topk", k=1, force_diag=True)
    rows = {h: ora[(0, h)][1] for h in range(H)}
    rp, ci = PT.rows_to_csr([r for h in range(H) for r in rows[h]])
    rp, ci = rp.to(DEV), ci.to(DEV)
    sc = bsa.bsa_score_blocks(Qd, Kd, scores=False, micro=16)
    mrp, mci, mnnz = bsa.bsa_select_blocks(
        None, Qd, mode="micro",
        micro=dict(m=m, scale=scale, head_mask=mask, macro=(rp, ci),
                   qpool16=sc["qpool16"], kpool16=sc["kpool16"]))
    torch.cuda.synchronize()
    got = gpu_rows_by_head(mrp, mci, mnnz, 1, H, nB)
    mo = _micro_oracle(Q, K, spec, rows, m, heads)
    for h in range(H):
        if h not in heads:
            assert all(len(r) == 0 for r in got[(0, h)])
            continue
        Qt, Kt, mrows = mo[h]
        compare_micro_rows(got[(0, h)], mrows, Qt, Kt, rows[h], N, scale, m)
    # micro attention on the oracle's micro lists
    allm = [mo[h][2][i] if h in heads else [] for h in range(H) for i in range(nB)]
    mrp_o, mci_o = PT.rows_to_csr(allm)
    Om = torch.full(Q.shape, 7.0, dtype=torch.float32, device=DEV)
    Lm = torch.full(Q.shape[:3], 7.0, dtype=torch.float32, device=DEV)
    bsa.bsa_micro_residual_fwd(Qd, Kd, Vd, mrp_o.to(DEV), mci_o.to(DEV), head_mask=mask,
                               out=Om, lse=Lm)
    Ob, Lb = bsa.bsa_sparse_attn_fwd(Qd, Kd, Vd, rp, ci)
    torch.cuda.synchronize()
    refs = {}
    for h in range(H):
        if h not in heads:
            assert torch.all(Om[0, h] == 7.0) and torch.all(Lm[0, h] == 7.0)
            continue
        q, k, v = PT.head64(Q, 0, h), PT.head64(K, 0, h), PT.head64(V, 0, h)
        Ou, Lu = O.micro_attention(q, k, v, mo[h][2], 64, 16, scale)
        PT.compare_o_lse(Om[0, h], Lm[0, h], Ou, Lu, f"micro h{h}")
        Oa, La = O.block_sparse_attention(q, k, v, rows[h], 64, scale)
        refs[h] = O.lse_merge(Oa, La, Ou, Lu)
    # merge, in place into the macro result
    bsa.bsa_lse_merge(Ob, Lb, Om, Lm, head_mask=mask, out=Ob, lse_out=Lb)
    torch.cuda.synchronize()
    for h in heads:
        PT.compare_o_lse(Ob[0, h], Lb[0, h], refs[h][0], refs[h][1], f"merged h{h}")


def test_micro_two_batches_head_subset():
    """Micro selection, residual and merge with B = 2 and a head subset: the
    (batch, micro head) slots of the tile-score product and of the lists
    against the oracle, every row of both batches."""
    spec = VideoSpec(2, 3, 64, (3, 8, 13), 118, spikes=True)
    say("micro two batches", spec.grid)
    Q, K, V = gen_qkv(spec)
    Qd, Kd, Vd = to_dev(Q, K, V)
    B, H, N, d = Q.shape
    nB = O.n_blocks(N, 64)
    scale = 1 / math.sqrt(d)
    m = 12
    heads = [0, 2]
    mask = [h in heads for h in range(H)]
    ora = oracle_rows_all(Q, K, spec, "topk", k=2, force_diag=True)
    rp, ci = PT.rows_to_csr([ora[(b, h)][1][i] for b in range(B) for h in range(H)
                             for i in range(nB)])
    rp, ci = rp.to(DEV), ci.to(DEV)
    sc = bsa.bsa_score_blocks(Qd, Kd, scores=False, micro=16)
    mrp, mci, mnnz = bsa.bsa_select_blocks(
        None, Qd, mode="micro",
        micro=dict(m=m, scale=scale, head_mask=mask, macro=(rp, ci),
                   qpool16=sc["qpool16"], kpool16=sc["kpool16"]))
    torch.cuda.synchronize()
    got = gpu_rows_by_head(mrp, mci, mnnz, B, H, nB)
    mo = {}
    for b in range(B):
        for h in range(H):
            if h not in heads:
                assert all(len(r) == 0 for r in got[(b, h)])
                continue
            q, k = PT.head64(Q, b, h), PT.head64(K, b, h)
            Qt, Kt = O.pool_means(q, 16), O.pool_means(k, 16)
            rows = ora[(b, h)][1]
            mo[(b, h)] = [O.micro_select_row(Qt, Kt, rows[i], i, N, 64, 16, scale, m)
                          for i in range(nB)]
            compare_micro_rows(got[(b, h)], mo[(b, h)], Qt, Kt, rows, N, scale, m)
    # the residual on the oracle's lists, then the merge into the macro result
    allm = [mo[(b, h)][i] if h in heads else [] for b in range(B) for h in range(H)
            for i in range(nB)]
    mrp_o, mci_o = PT.rows_to_csr(allm)
    Om, Lm = bsa.bsa_micro_residual_fwd(Qd, Kd, Vd, mrp_o.to(DEV), mci_o.to(DEV), head_mask=mask)
    Ob, Lb = bsa.bsa_sparse_attn_fwd(Qd, Kd, Vd, rp, ci)
    bsa.bsa_lse_merge(Ob, Lb, Om, Lm, head_mask=mask, out=Ob, lse_out=Lb)
    torch.cuda.synchronize()
    for b in range(B):
        for h in heads:
            q, k, v = PT.head64(Q, b, h), PT.head64(K, b, h), PT.head64(V, b, h)
            Ou, Lu = O.micro_attention(q, k, v, mo[(b, h)], 64, 16, scale)
            PT.compare_o_lse(Om[b, h], Lm[b, h], Ou, Lu, f"micro b{b} h{h}")
            Oa, La = O.block_sparse_attention(q, k, v, ora[(b, h)][1], 64, scale)
            Or, Lr = O.lse_merge(Oa, La, Ou, Lu)
            PT.compare_o_lse(Ob[b, h], Lb[b, h], Or, Lr, f"merged b{b} h{h}")


def test_micro_select_rows_of_more_than_32768_candidates():
    """Query blocks over more than 8192 16-token key tiles (the selection
    kernel that holds 64 candidates per thread), ragged in both tile sizes:
    sampled rows, the first and the last, against the oracle."""
    spec = VideoSpec(1, 1, 64, (7, 73, 258), 114, spikes=True)
    say("micro long rows", spec.grid)
    Q, K, _ = gen_qkv(spec)
    Qd, Kd = to_dev(Q, K)
    N = spec.N
    nB, nT = O.n_blocks(N, 64), O.n_blocks(N, 16)
    assert 4 * nT > 32768 and N % 64 and N % 16
    scale = 1 / math.sqrt(spec.d)
    m = 300
    rows = oracle_rows_all(Q, K, spec, "topk", k=bsa.budget_blocks(0.1, nB))[(0, 0)][1]
    rp, ci = PT.rows_to_csr(rows)
    sc = bsa.bsa_score_blocks(Qd, Kd, scores=False, micro=16)
    mrp, mci, mnnz = bsa.bsa_select_blocks(
        None, Qd, mode="micro",
        micro=dict(m=m, scale=scale, head_mask=[True], macro=(rp.to(DEV), ci.to(DEV)),
                   qpool16=sc["qpool16"], kpool16=sc["kpool16"]))
    torch.cuda.synchronize()
    got = gpu_rows_by_head(mrp, mci, mnnz, 1, 1, nB)[(0, 0)]
    q, k = PT.head64(Q, 0, 0), PT.head64(K, 0, 0)
    Qt, Kt = O.pool_means(q, 16), O.pool_means(k, 16)
    rng = np.random.default_rng(114)
    blocks = sorted(set(rng.choice(nB, size=24, replace=False).tolist()) | {0, nB - 1})
    ora = [O.micro_select_row(Qt, Kt, rows[i], i, N, 64, 16, scale, m) for i in blocks]
    assert all(len(got[i]) == m for i in blocks)
    exempt = compare_micro_rows([got[i] for i in blocks], ora, Qt, Kt, [rows[i] for i in blocks],
                                N, scale, m, blocks=blocks)
    assert exempt <= 1


def test_merge_kernel_on_oracle_inputs():
    rng = np.random.default_rng(5)
    B, H, N, d = 1, 2, 300, 128
    O1 = rng.standard_normal((B, H, N, d))
    O2 = rng.standard_normal((B, H, N, d))
    L1 = rng.standard_normal((B, H, N)) * 3
    L2 = rng.standard_normal((B, H, N)) * 3
    L1[0, 0, :10] = -np.inf
    L2[0, 0, 5:15] = -np.inf
    O1[np.isneginf(L1)] = 0
    O2[np.isneginf(L2)] = 0
    t = lambda x: torch.from_numpy(x).float().to(DEV)
    Og, Lg = bsa.bsa_lse_merge(t(O1), t(L1), t(O2), t(L2))
    torch.cuda.synchronize()
    for h in range(H):
        Oref, Lref = O.lse_merge(O1[0, h].astype(np.float32).astype(np.float64),
                                 L1[0, h].astype(np.float32).astype(np.float64),
                                 O2[0, h].astype(np.float32).astype(np.float64),
                                 L2[0, h].astype(np.float32).astype(np.float64))
        np.testing.assert_allclose(Og[0, h].double().cpu().numpy(), Oref, atol=1e-5)
        Lgh = Lg[0, h].double().cpu().numpy()
        assert np.array_equal(np.isneginf(Lgh), np.isneginf(Lref))
        fin = ~np.isneginf(Lref)
        np.testing.assert_allclose(Lgh[fin], Lref[fin], atol=1e-5)


# ----------------------------------------------------- the five workloads

def _budgets(cfg, nB):
    c = CONFIGS[cfg]
    if c["mode"] == "topk":
        return dict(k=bsa.budget_blocks(c["density"], nB), force_diag=c.get("force_diag", False))
    if c["mode"] == "topp":
        return dict(p=c["p"], k_min=1, k_cap=bsa.cap_blocks(c["cap_density"], nB))
    return {}


@pytest.fixture(scope="module", params=[0, 1, 2, 3, 4])
def workload(request):
    cfg = request.param
    spec = config_spec(cfg)
    say(f"workload {cfg} {CONFIGS[cfg]['name']}: generating")
    Q, K, V = gen_qkv(spec)
    Qd, Kd, Vd = to_dev(Q, K, V)
    yield cfg, spec, (Q, K, V), (Qd, Kd, Vd)
    del Qd, Kd, Vd
    torch.cuda.empty_cache()


def test_workload_lists_and_attention(workload):
    cfg, spec, (Q, K, V), (Qd, Kd, Vd) = workload
    c = CONFIGS[cfg]
    B, H, N, d = Q.shape
    nB = O.n_blocks(N, 64)
    scale = 1 / math.sqrt(d)
    mode = c["mode"]
    kw = _budgets(cfg, nB)
    static = None
    if mode == "static":
        static = dict(frame_tokens=spec.frame_tokens, window_frames=c["window_frames"],
                      n_anchors=c["n_anchors"], anchor_offset=rotation_offset(cfg, 0, nB))
        kw["static"] = static
    say(f"workload {cfg}: GPU score/select", kw if mode != "static" else static)
    sc = bsa.bsa_score_blocks(Qd, Kd, scores=(mode != "static"))
    rp, ci, nnz = bsa.bsa_select_blocks(sc["scores"], Qd, mode=mode, **kw)
    torch.cuda.synchronize()
    got = gpu_rows_by_head(rp, ci, nnz, B, H, nB)
    say(f"workload {cfg}: oracle selection over {H} heads")
    ora = oracle_rows_all(Q, K, spec, mode, **kw)
    F = forced_rows(N, kw.get("force_diag", False), static)
    exempt = 0
    for bh, (S, rows) in ora.items():
        if mode == "topk":
            exempt += PT.compare_topk_rows(got[bh], rows, S, kw["k"], F)
        elif mode == "topp":
            exempt += PT.compare_topp_rows(got[bh], rows, S, O.block_sizes(N, 64), kw["p"],
                                           kw["k_min"], kw["k_cap"])
        else:
            assert got[bh] == rows
    say(f"workload {cfg}: lists match, {exempt} tie-exempt rows of {B * H * nB}")
    assert exempt <= max(2, B * H * nB // 1000)
    if mode != "static":
        for h in (0, H - 1):
            # float32 pooling and dot products: about 1e-7 relative
            np.testing.assert_allclose(sc["scores"][0, h].double().cpu().numpy(), ora[(0, h)][0],
                                       atol=1e-5, rtol=2e-6)
    # attention on the oracle's lists, sampled query blocks of two heads
    allrows = [ora[(b, h)][1][i] for b in range(B) for h in range(H) for i in range(nB)]
    orp, oci = PT.rows_to_csr(allrows)
    say(f"workload {cfg}: GPU sparse attention, nnz={int(orp[-1])}")
    Og, Lg = bsa.bsa_sparse_attn_fwd(Qd, Kd, Vd, orp.to(DEV), oci.to(DEV))
    torch.cuda.synchronize()
    rng = np.random.default_rng(cfg)
    blocks = sorted(set(rng.choice(nB, size=min(nB, 6), replace=False).tolist()) | {nB - 1, 0})
    for h in sorted({0, H // 2, H - 1}):
        q, k, v = PT.head64(Q, 0, h), PT.head64(K, 0, h), PT.head64(V, 0, h)
        rows = ora[(0, h)][1]
        for i in blocks:
            qi = O.block_tokens(N, 64, i)
            keys = np.concatenate([O.block_tokens(N, 64, j) for j in rows[i]])
            Oref, Lref = O.attend(q[qi], k[keys], v[keys], scale)
            PT.compare_o_lse(Og[0, h, qi[0]:qi[-1] + 1], Lg[0, h, qi[0]:qi[-1] + 1], Oref, Lref,
                             f"cfg{cfg} h{h} blk{i}")
    # properties over every row: finite LSE, O a convex combination of V
    assert torch.isfinite(Lg).all()
    vmin = Vd.float().amin(dim=2, keepdim=True)
    vmax = Vd.float().amax(dim=2, keepdim=True)
    assert bool(((Og >= vmin - 1e-3) & (Og <= vmax + 1e-3)).all())
    # the full pipeline: GPU lists into GPU attention; rows whose lists agree
    # with the oracle's must give bit-identical results
    Og2, Lg2 = bsa.bsa_sparse_attn_fwd(Qd, Kd, Vd, rp, ci)
    torch.cuda.synchronize()
    agree = torch.zeros(B, H, N, dtype=torch.bool)
    for (b, h), (S, rows) in ora.items():
        for i in range(nB):
            if got[(b, h)][i] == rows[i]:
                agree[b, h, 64 * i:min(64 * i + 64, N)] = True
    agree = agree.to(DEV)
    assert torch.equal(Lg[agree], Lg2[agree])
    assert torch.equal(Og[agree], Og2[agree])


def test_workload_dense_sampled(workload):
    cfg, spec, (Q, K, V), (Qd, Kd, Vd) = workload
    B, H, N, d = Q.shape
    say(f"workload {cfg}: dense attention (the speedup baseline) on sampled query blocks")
    Og, Lg = bsa.bsa_dense_attn_fwd(Qd, Kd, Vd)
    torch.cuda.synchronize()
    for h in sorted({0, H - 1}):
        q, k, v = PT.head64(Q, 0, h), PT.head64(K, 0, h), PT.head64(V, 0, h)
        for t0 in (0, N // 2, N - 64):
            Oref, Lref = O.attend(q[t0:t0 + 64], k, v, 1 / math.sqrt(d))
            PT.compare_o_lse(Og[0, h, t0:t0 + 64], Lg[0, h, t0:t0 + 64], Oref, Lref,
                             f"dense cfg{cfg} h{h} t{t0}")


def test_workload_micro(workload):
    cfg, spec, (Q, K, V), (Qd, Kd, Vd) = workload
    c = CONFIGS[cfg]
    if "micro_head_frac" not in c:
        pytest.skip("no micro residual in this workload")
    B, H, N, d = Q.shape
    nB = O.n_blocks(N, 64)
    scale = 1 / math.sqrt(d)
    heads = micro_heads(cfg)
    m = c["micro_m"] if "micro_m" in c else int(round(c["micro_density"] * 64 * N / 256))
    mask = [h in heads for h in range(H)]
    kw = _budgets(cfg, nB)
    say(f"workload {cfg}: micro on heads {heads}, m={m}")
    ora = oracle_rows_all(Q, K, spec, "topk", **kw)
    allrows = [ora[(0, h)][1][i] for h in range(H) for i in range(nB)]
    orp, oci = PT.rows_to_csr(allrows)
    orp, oci = orp.to(DEV), oci.to(DEV)
    sc = bsa.bsa_score_blocks(Qd, Kd, scores=False, micro=16)
    mrp, mci, mnnz = bsa.bsa_select_blocks(
        None, Qd, mode="micro",
        micro=dict(m=m, scale=scale, head_mask=mask, macro=(orp, oci),
                   qpool16=sc["qpool16"], kpool16=sc["kpool16"]))
    torch.cuda.synchronize()
    got = gpu_rows_by_head(mrp, mci, mnnz, 1, H, nB)
    rng = np.random.default_rng(100 + cfg)
    hs = [heads[0], heads[-1]]
    blocks = sorted(set(rng.choice(nB, size=min(nB, 4), replace=False).tolist()) | {nB - 1})
    sampled = {}
    for h in hs:
        # every row of the head: the oracle's lists of all query blocks
        q, k = PT.head64(Q, 0, h), PT.head64(K, 0, h)
        Qt, Kt = O.pool_means(q, 16), O.pool_means(k, 16)
        rows = ora[(0, h)][1]
        say(f"workload {cfg}: oracle micro lists of every row of head {h}")
        mo_all = O.micro_select_rows(Qt, Kt, rows, N, 64, 16, scale, m)
        exempt = compare_micro_rows(got[(0, h)], mo_all, Qt, Kt, rows, N, scale, m)
        say(f"workload {cfg}: head {h}: {nB} micro rows match, {exempt} tie-exempt")
        assert exempt <= max(2, nB // 100)
        for i in blocks:
            sampled[(h, i)] = mo_all[i]
    for h in range(H):
        if h not in heads:
            assert all(len(r) == 0 for r in got[(0, h)])
        else:
            # every query block has far more than m candidates in these workloads
            assert all(len(r) == m for r in got[(0, h)])
    # micro attention + merge on the oracle lists for the sampled blocks
    allm = [sampled.get((h, i), []) for h in range(H) for i in range(nB)]
    mrp_o, mci_o = PT.rows_to_csr(allm)
    Om, Lm = bsa.bsa_micro_residual_fwd(Qd, Kd, Vd, mrp_o.to(DEV), mci_o.to(DEV), head_mask=mask)
    Ob, Lb = bsa.bsa_sparse_attn_fwd(Qd, Kd, Vd, orp, oci)
    bsa.bsa_lse_merge(Ob, Lb, Om, Lm, head_mask=mask, out=Ob, lse_out=Lb)
    torch.cuda.synchronize()
    for (h, i), mo in sampled.items():
        q, k, v = PT.head64(Q, 0, h), PT.head64(K, 0, h), PT.head64(V, 0, h)
        qi = O.block_tokens(N, 64, i)
        rows = ora[(0, h)][1]
        keys = np.concatenate([O.block_tokens(N, 64, j) for j in rows[i]])
        Oa, La = O.attend(q[qi], k[keys], v[keys], scale)
        Ou = np.zeros_like(Oa)
        Lu = np.full(len(qi), -np.inf)
        for a in range(4):
            sub = [t for t in range(len(qi)) if t // 16 == a]
            if not sub:
                continue
            tiles = [cc // 4 for cc in mo if cc % 4 == a]
            if tiles:
                kk = np.concatenate([O.block_tokens(N, 16, t) for t in tiles])
                Ou[sub], Lu[sub] = O.attend(q[qi[sub]], k[kk], v[kk], scale)
        PT.compare_o_lse(Om[0, h, qi[0]:qi[-1] + 1], Lm[0, h, qi[0]:qi[-1] + 1], Ou, Lu,
                         f"cfg{cfg} micro h{h} blk{i}")
        Of, Lf = O.lse_merge(Oa, La, Ou, Lu)
        PT.compare_o_lse(Ob[0, h, qi[0]:qi[-1] + 1], Lb[0, h, qi[0]:qi[-1] + 1], Of, Lf,
                         f"cfg{cfg} merged h{h} blk{i}")
