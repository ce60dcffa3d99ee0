"""CSR validation on the GPU (bsa_check_csr) and the attention workspace's
status word (bsa_attn_take_status).  The checker reads only the arrays it is
given, within their sizes, so it runs on planted bad lists; the attention
calls themselves run on valid lists only, where the status word must stay
clear."""

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
    print("[gpu-csr]", *a, file=sys.stderr, flush=True)


def _counts(rows, n_cols, cap_cut=None, ptr_edit=None):
    rp, ci = PT.rows_to_csr(rows)
    if ptr_edit is not None:
        ptr_edit(rp)
    if cap_cut is not None:
        ci = ci[:cap_cut].clone()
    c = bsa.bsa_check_csr(rp.to(DEV), ci.to(DEV), n_cols)
    torch.cuda.synchronize()
    return c.cpu().tolist()


def test_check_csr_counts_each_fault():
    say("check_csr on planted faults")
    good = [[0, 3, 5], [], [1], list(range(8)), [7]]
    assert _counts(good, 8) == [0, 0, 0]
    assert _counts([[0, 9], [1, 2, 30], [4]], 8) == [0, 2, 0]          # two out of range
    assert _counts([[0, 9], [1, -2, 3], [4]], 8) == [0, 2, 1]          # -2 also breaks the order
    assert _counts([[5, 1], [2, 2], [4, 6]], 8) == [0, 0, 2]           # unsorted, duplicate
    assert _counts(good, 8, cap_cut=10) == [2, 0, 0]                   # rows 3 and 4 end past the cap

    def back(rp):
        rp[2] = 1   # row 1 ends before it starts; row 2 then reads 3, 5, 1 (not ascending)
    assert _counts(good, 8, ptr_edit=back) == [1, 0, 1]
    # many rows (several workgroups) with one fault per 97 rows
    rng = np.random.default_rng(3)
    rows = [sorted(rng.choice(300, size=int(rng.integers(0, 40)), replace=False).tolist())
            for _ in range(1000)]
    n_bad = 0
    for r in range(0, 1000, 97):
        if rows[r]:
            rows[r][-1] = 300 + r
            n_bad += 1
    assert _counts(rows, 300) == [0, n_bad, 0]


def test_selected_lists_pass_the_check_and_attention_keeps_the_status_clear():
    spec = VideoSpec(1, 3, 128, (4, 12, 20), 191)   # 960 tokens, 15 blocks
    Q, K, V = (x.to(DEV) for x in gen_qkv(spec))
    B, H, N, d = Q.shape
    nB, nT = O.n_blocks(N, 64), O.n_blocks(N, 16)
    say("selection -> check -> attention status")
    sc = bsa.bsa_score_blocks(Q, K, micro=16)
    rp, ci, nnz = bsa.bsa_select_blocks(sc["scores"], Q, mode="topk", k=3, force_diag=True)
    torch.cuda.synchronize()
    n = int(nnz.item())
    assert bsa.bsa_check_csr(rp, ci[:n], nB).cpu().tolist() == [0, 0, 0]
    mrp, mci, mnnz = bsa.bsa_select_blocks(
        None, Q, mode="micro",
        micro=dict(m=10, scale=1 / math.sqrt(d), macro=(rp, ci), qpool16=sc["qpool16"],
                   kpool16=sc["kpool16"]))
    torch.cuda.synchronize()
    mn = int(mnnz.item())
    # micro codes 4 beta + a lie in [0, 4 nT); their order is (a, beta), so
    # only the range count applies
    assert bsa.bsa_check_csr(mrp, mci[:mn], 4 * nT).cpu().tolist()[:2] == [0, 0]
    ws = bsa.attn_workspace(Q)
    Om, Lm = bsa.bsa_sparse_attn_fwd(Q, K, V, rp, ci, workspace=ws)
    Ou, Lu = bsa.bsa_micro_residual_fwd(Q, K, None, mrp, mci, workspace=ws)
    st = bsa.bsa_attn_take_status(ws, Q)
    torch.cuda.synchronize()
    assert st.item() == 0
    assert torch.isfinite(Lm).all()
