"""The no-allocation selection entry point (bsa_select_blocks_noalloc),
called through the C ABI, against bsa_select_blocks with a workspace: the
same CSR bit for bit, on two calls in a row (the second on a smaller input,
over the scratch the first one left), for top-k with the diagonal, top-p,
the static window with anchors and micro tiles."""

import math
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
    print("[gpu-noalloc]", *a, file=sys.stderr, flush=True)


def _both(scores, Q, **kw):
    rp1, ci1, nnz1 = bsa.bsa_select_blocks(scores, Q, **kw)
    # outputs pre-filled with garbage: every entry read back must be written
    rp2 = torch.full_like(rp1, -7)
    ci2 = torch.full_like(ci1, -7)
    nnz2 = torch.full_like(nnz1, -7)
    bsa.bsa_select_blocks_noalloc(scores, Q, row_ptr=rp2, col_idx=ci2, nnz=nnz2, **kw)
    torch.cuda.synchronize()
    n = int(nnz1.item())
    assert int(nnz2.item()) == n
    assert torch.equal(rp1, rp2)
    assert torch.equal(ci1[:n], ci2[:n])
    return n


def _layer(grid, H, d, key, spikes=False):
    spec = VideoSpec(1, H, d, grid, key, spikes=spikes)
    Q, K, _ = gen_qkv(spec)
    return spec, Q.to(DEV), K.to(DEV)


def test_noalloc_select_equals_workspace_select_twice_smaller_second():
    # first call: 2 x 30 x 64 tokens (30 frames of 64), 12 heads -> 900
    # blocks per row, 10,800 rows; second: 4 x 16 x 16, 2 heads
    spec, Q, K = _layer((30, 30, 64), 12, 128, 201)
    nB = -(-spec.N // 64)
    say("noalloc: large top-k", spec.N, nB)
    sc = bsa.bsa_score_blocks(Q, K)
    n1 = _both(sc["scores"], Q, mode="topk", k=225, force_diag=True)
    assert n1 > 0
    spec2, Q2, K2 = _layer((4, 16, 16), 2, 64, 202)
    say("noalloc: small top-p after it")
    sc2 = bsa.bsa_score_blocks(Q2, K2)
    _both(sc2["scores"], Q2, mode="topp", p=0.9, k_min=1, k_cap=12)
    _both(sc2["scores"], Q2, mode="topk", k=4, force_diag=True)


def test_noalloc_static_and_micro():
    spec, Q, K = _layer((6, 10, 32), 3, 64, 203)
    nB = -(-spec.N // 64)
    say("noalloc: static window + anchors")
    st = dict(frame_tokens=spec.frame_tokens, window_frames=1, n_anchors=4, anchor_offset=5)
    _both(None, Q, mode="static", static=st)
    say("noalloc: micro tiles")
    sc = bsa.bsa_score_blocks(Q, K, micro=16)
    rp, ci, _ = bsa.bsa_select_blocks(sc["scores"], Q, mode="topk", k=3, force_diag=True)
    micro = dict(m=12, scale=1 / math.sqrt(64), macro=(rp, ci), qpool16=sc["qpool16"],
                 kpool16=sc["kpool16"], head_mask=[True, False, True])
    _both(None, Q, mode="micro", micro=micro)
    # and a macro call after the micro one (different scratch layout)
    _both(sc["scores"], Q, mode="topk", k=7)


def test_noalloc_refuses_a_selection_beyond_its_scratch():
    # micro tile scores of 8 heads of 65,536 tokens: 8 * 4096^2 * 4 bytes
    Q = torch.empty((1, 8, 65536, 64), dtype=torch.bfloat16, device=DEV)
    f = torch.empty(1, dtype=torch.float32, device=DEV)
    rp = torch.empty(8 * 1024 + 1, dtype=torch.int32, device=DEV)
    micro = dict(m=4, scale=0.125, macro=(rp, rp), qpool16=f, kpool16=f)
    with pytest.raises(bsa.BsaError, match="scratch"):
        bsa.bsa_select_blocks_noalloc(None, Q, row_ptr=rp, col_idx=rp, nnz=f, mode="micro",
                                      micro=micro)
