"""The hot path captured in a HIP graph: scoring, selection, block-sparse
attention and the micro residual with its merge, replayed several times with
eager work between the replays, must give the eager calls' bits every time
(no library call records a memset or a host synchronisation)."""

import sys

import pytest
import torch

from synth import VideoSpec, gen_qkv

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import block_sparse_attention_pool_amd as bsa
else:  # collected on CPU, skipped by the marker
    bsa = None

DEV = "cuda:0"


def say(*a):
    print("[gpu-graph]", *a, file=sys.stderr, flush=True)


def _step(Q, K, V, ws, O, L, Om, Lm, mask, k):
    sc = bsa.bsa_score_blocks(Q, K, scores=True, micro=16)
    rp, ci, nnz = bsa.bsa_select_blocks(sc["scores"], Q, mode="topk", k=k)
    bsa.bsa_sparse_attn_fwd(Q, K, V, rp, ci, out=O, lse=L, workspace=ws)
    mrp, mci, _ = bsa.bsa_select_blocks(
        None, Q, mode="micro",
        micro=dict(m=8, scale=Q.shape[3] ** -0.5, head_mask=mask, macro=(rp, ci),
                   qpool16=sc["qpool16"], kpool16=sc["kpool16"]))
    bsa.bsa_micro_residual_fwd(Q, K, None, mrp, mci, head_mask=mask, out=Om, lse=Lm,
                               workspace=ws)
    bsa.bsa_lse_merge(O, L, Om, Lm, head_mask=mask, out=O, lse_out=L)
    return nnz


@pytest.mark.parametrize("grid,H,d", [((3, 10, 13), 2, 128), ((4, 16, 16), 3, 64)])
def test_graph_replay_equals_eager(grid, H, d):
    spec = VideoSpec(1, H, d, grid, 201)
    Q, K, V = (x.to(DEV) for x in gen_qkv(spec))
    nB = bsa.n_blocks(spec.N)
    k = max(1, nB // 4)
    mask = [h % 2 == 0 for h in range(H)]
    ws = bsa.attn_workspace(Q)
    O = torch.empty(Q.shape, dtype=torch.float32, device=DEV)
    L = torch.empty(Q.shape[:3], dtype=torch.float32, device=DEV)
    Om, Lm = torch.empty_like(O), torch.empty_like(L)
    _step(Q, K, V, ws, O, L, Om, Lm, mask, k)
    torch.cuda.synchronize()
    ref = (O.clone(), L.clone())
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        _step(Q, K, V, ws, O, L, Om, Lm, mask, k)
    for rep in range(4):
        O.fill_(float(rep))
        L.zero_()
        ws.zero_()  # the replay must stage V^T again
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(O, ref[0]) and torch.equal(L, ref[1]), f"replay {rep}"
    say(f"{grid} H={H} d={d}: 4 replays equal to the eager step")
