"""GPU parity of the omission-risk reduction (bsa_omission_risk) against the
fp64 oracle.

* The kernel alone, on seeded LSE arrays (small ragged shapes and the five
  workload shapes at full size): per-row shares are float32 expm1 forms of
  exactly the same float32 inputs the oracle upcasts, sums are float64, so
  the three per-head numbers agree to KERNEL_TOL.
* End to end, on LSEs the library computes (sparse, dense, micro + merge):
  the oracle sums the full-attention softmax mass outside each support key
  by key.  A row's share moves by at most e^(Ls - Lf) (|dLs| + |dLf|) when
  the two LSEs carry errors dLs, dLf, so the LSE tolerance of the attention
  parity tests (1e-3 each) bounds every per-row share, its mean and its
  maximum by E2E_TOL = 2e-3.
"""

import math
import sys

import numpy as np
import pytest
import torch

from oracle import bsa_oracle as O
from synth import CONFIGS, VideoSpec, config_spec, gen_qkv, micro_heads
import parity as PT

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import block_sparse_attention_pool_amd as bsa
else:  # collected on CPU, skipped by the marker
    bsa = None

DEV = "cuda:0"
KERNEL_TOL = 1e-6
E2E_TOL = 2 * PT.LSE_MAX


def say(*a):
    print("[gpu-risk]", *a, file=sys.stderr, flush=True)


def seeded_lse(seed, B, H, N, repaired=True):
    """Float32 LSE triples with the structure of real ones: a full-attention
    LSE, a sparse LSE keeping a share of its mass (mostly large, sometimes
    tiny), a repaired LSE recovering part of the rest, plus rows with an
    empty support, rows with nothing omitted and rows with no keys at all."""
    rng = np.random.default_rng(seed)
    shp = (B, H, N)
    Lf = rng.normal(8.0, 2.0, shp)
    kept = rng.beta(5.0, 1.0, shp)
    rec = rng.random(shp) * (1.0 - kept)
    Ls = Lf + np.log(kept)
    Lr = Lf + np.log(kept + rec)
    flat = lambda a: a.reshape(-1)
    n = B * H * N
    pick = lambda frac: rng.choice(n, size=max(1, int(frac * n)), replace=False)
    e = pick(0.01)                      # empty sparse support
    flat(Ls)[e] = -np.inf
    flat(Lr)[e] = flat(Lf)[e] + np.log(flat(rec)[e] + 1e-3)
    z = pick(0.01)                      # support holds every key
    flat(Ls)[z] = flat(Lf)[z]
    flat(Lr)[z] = flat(Lf)[z]
    t = pick(0.01)                      # almost nothing omitted
    flat(Ls)[t] = flat(Lf)[t] + np.log1p(-1e-6)
    flat(Lr)[t] = flat(Ls)[t]
    if n > 3:
        x = pick(0.002)                 # no keys at all
        flat(Lf)[x] = -np.inf
        flat(Ls)[x] = -np.inf
        flat(Lr)[x] = -np.inf
    f32 = lambda a: a.astype(np.float32)
    return f32(Ls), f32(Lf), (f32(Lr) if repaired else None)


def oracle_risk(Ls, Lf, Lr):
    B, H, _ = Ls.shape
    out = np.zeros((B, H, 3))
    for b in range(B):
        for h in range(H):
            w, g = O.risk_from_lse(Ls[b, h].astype(np.float64), Lf[b, h].astype(np.float64),
                                   None if Lr is None else Lr[b, h].astype(np.float64))
            out[b, h] = O.head_risk(w, g)
    return out


KERNEL_SHAPES = [
    (1, 1, 1), (1, 1, 2048), (1, 2, 2049), (2, 3, 5000), (3, 5, 333),
    # the five workloads' [B, H, N]
    (1, 2, 1024), (1, 12, 32760), (1, 40, 75600), (1, 24, 118800), (1, 12, 196560),
]


@pytest.mark.parametrize("shape", KERNEL_SHAPES)
@pytest.mark.parametrize("repaired", [True, False])
def test_risk_kernel_on_seeded_lse(shape, repaired):
    B, H, N = shape
    say("risk kernel", shape, "repaired" if repaired else "no repair")
    Ls, Lf, Lr = seeded_lse(sum(shape) + repaired, B, H, N, repaired)
    t = lambda a: None if a is None else torch.from_numpy(a).to(DEV)
    got = bsa.bsa_omission_risk(t(Ls), t(Lf), t(Lr))
    torch.cuda.synchronize()
    ref = oracle_risk(Ls, Lf, Lr)
    np.testing.assert_allclose(got.cpu().numpy(), ref, atol=KERNEL_TOL, rtol=0)
    if not repaired:
        assert torch.all(got[..., 2] == 0)


def test_risk_kernel_is_deterministic_and_writes_only_its_output():
    Ls, Lf, Lr = seeded_lse(77, 1, 24, 118800)
    t = lambda a: torch.from_numpy(a).to(DEV)
    buf = torch.full((24 * 3 + 64,), 5.0, dtype=torch.float64, device=DEV)
    r1 = bsa.bsa_omission_risk(t(Ls), t(Lf), t(Lr), out=buf[:72].view(1, 24, 3))
    r2 = bsa.bsa_omission_risk(t(Ls), t(Lf), t(Lr))
    torch.cuda.synchronize()
    assert torch.equal(r1, r2)
    assert torch.all(buf[72:] == 5.0)


# ------------------------------------------------------------ end to end

SMALL = [((3, 7, 9), 2, 128, 121), ((4, 16, 16), 3, 64, 122), ((2, 8, 13), 2, 128, 123)]


@pytest.mark.parametrize("grid,H,d,key", SMALL)
def test_risk_end_to_end_small(grid, H, d, key):
    spec = VideoSpec(1, H, d, grid, key, spikes=True)
    say("risk end to end", grid, H, d)
    Q, K, V = gen_qkv(spec)
    Qd, Kd, Vd = (x.to(DEV) for x in (Q, K, V))
    N = spec.N
    nB = O.n_blocks(N, 64)
    scale = 1 / math.sqrt(d)
    rows, mrows = {}, {}
    for h in range(H):
        q, k = PT.head64(Q, 0, h), PT.head64(K, 0, h)
        S = O.pooled_scores(O.pool_means(q, 64), O.pool_means(k, 64), scale)
        rows[h] = O.select_rows(S, N, 64, "topk", k=1, force_diag=True)
        rows[h][0] = []   # one query block with nothing kept
        Qt, Kt = O.pool_means(q, 16), O.pool_means(k, 16)
        mrows[h] = [O.micro_select_row(Qt, Kt, rows[h][i], i, N, 64, 16, scale, 6)
                    for i in range(nB)]
    rp, ci = PT.rows_to_csr([r for h in range(H) for r in rows[h]])
    mrp, mci = PT.rows_to_csr([r for h in range(H) for r in mrows[h]])
    ws = bsa.attn_workspace(Qd)
    _, Ls = bsa.bsa_sparse_attn_fwd(Qd, Kd, Vd, rp.to(DEV), ci.to(DEV), workspace=ws)
    _, Lf = bsa.bsa_dense_attn_fwd(Qd, Kd, None, workspace=ws)
    Ob = torch.zeros(Q.shape, dtype=torch.float32, device=DEV)
    Om, Lm = bsa.bsa_micro_residual_fwd(Qd, Kd, None, mrp.to(DEV), mci.to(DEV), workspace=ws)
    _, Lr = bsa.bsa_lse_merge(Ob, Ls, Om, Lm)
    got = bsa.bsa_omission_risk(Ls, Lf, Lr)
    torch.cuda.synchronize()
    for h in range(H):
        q, k = PT.head64(Q, 0, h), PT.head64(K, 0, h)
        w = O.omitted_mass(q, k, rows[h], 64, scale)
        g = O.micro_mass(q, k, mrows[h], 64, 16, scale)
        ref = O.head_risk(w, g)
        np.testing.assert_allclose(got[0, h].cpu().numpy(), ref, atol=E2E_TOL, rtol=0,
                                   err_msg=f"head {h}")
        # block 0 keeps nothing: its rows omit everything
        assert abs(ref[1] - 1.0) < 1e-12 and abs(float(got[0, h, 1]) - 1.0) <= E2E_TOL


@pytest.mark.parametrize("cfg", [1, 3])
def test_risk_workload_sampled(cfg):
    """Full-size workloads: sparse and dense LSEs of the library on two heads;
    the risk kernel on the LSEs of sampled query blocks, gathered into a
    contiguous [1, 1, n] array, against the oracle's key-by-key mass."""
    c = CONFIGS[cfg]
    spec = config_spec(cfg)
    say(f"risk workload {cfg} {c['name']}: generating")
    Q, K, V = gen_qkv(spec)
    Qd, Kd, Vd = (x.to(DEV) for x in (Q, K, V))
    B, H, N, d = Q.shape
    nB = O.n_blocks(N, 64)
    scale = 1 / math.sqrt(d)
    kk = bsa.budget_blocks(c["density"], nB)
    heads = micro_heads(cfg)[:2] if cfg == 3 else [0, H - 1]
    rng = np.random.default_rng(200 + cfg)
    blocks = sorted(set(rng.choice(nB, size=4, replace=False).tolist()) | {nB - 1})
    m = int(round(c["micro_density"] * 64 * N / 256)) if cfg == 3 else 0
    rows, mrows = {}, {}
    for h in heads:
        q, k = PT.head64(Q, 0, h), PT.head64(K, 0, h)
        S = O.pooled_scores(O.pool_means(q, 64), O.pool_means(k, 64), scale)
        rows[h] = O.select_rows(S, N, 64, "topk", k=kk)
        if cfg == 3:
            Qt, Kt = O.pool_means(q, 16), O.pool_means(k, 16)
            mrows[h] = [O.micro_select_row(Qt, Kt, rows[h][i], i, N, 64, 16, scale, m)
                        if i in blocks else [] for i in range(nB)]
    allrows = [rows[h][i] if h in rows else [] for h in range(H) for i in range(nB)]
    rp, ci = PT.rows_to_csr(allrows)
    ws = bsa.attn_workspace(Qd)
    say(f"risk workload {cfg}: sparse, dense" + (", micro" if cfg == 3 else ""))
    _, Ls = bsa.bsa_sparse_attn_fwd(Qd, Kd, Vd, rp.to(DEV), ci.to(DEV), workspace=ws)
    _, Lf = bsa.bsa_dense_attn_fwd(Qd, Kd, None, workspace=ws)
    Lr = None
    if cfg == 3:
        mask = [h in heads for h in range(H)]
        allm = [mrows[h][i] if h in mrows else [] for h in range(H) for i in range(nB)]
        mrp, mci = PT.rows_to_csr(allm)
        Om, Lm = bsa.bsa_micro_residual_fwd(Qd, Kd, None, mrp.to(DEV), mci.to(DEV),
                                            head_mask=mask, workspace=ws)
        Ob = torch.zeros(Q.shape, dtype=torch.float32, device=DEV)
        _, Lr = bsa.bsa_lse_merge(Ob, Ls, Om, Lm, head_mask=mask, out=Ob, lse_out=Ls.clone())
    torch.cuda.synchronize()
    for h in heads:
        q, k = PT.head64(Q, 0, h), PT.head64(K, 0, h)
        tok = np.concatenate([O.block_tokens(N, 64, i) for i in blocks])
        w = np.concatenate([
            O.softmax_mass_outside(q[O.block_tokens(N, 64, i)], k,
                                   np.concatenate([O.block_tokens(N, 64, j) for j in rows[h][i]]),
                                   scale) for i in blocks])
        g = O.micro_mass(q, k, mrows[h], 64, 16, scale)[tok] if cfg == 3 else np.zeros_like(w)
        ref = O.head_risk(w, g)
        idx = torch.from_numpy(tok).to(DEV)
        sub = lambda L: None if L is None else L[0, h, idx].contiguous().view(1, 1, -1)
        got = bsa.bsa_omission_risk(sub(Ls), sub(Lf), sub(Lr))
        torch.cuda.synchronize()
        say(f"risk workload {cfg} h{h}: oracle {ref}, got {got[0, 0].tolist()}")
        np.testing.assert_allclose(got[0, 0].cpu().numpy(), ref, atol=E2E_TOL, rtol=0,
                                   err_msg=f"cfg{cfg} head {h}")
