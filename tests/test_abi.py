"""The C-ABI library: it loads, exports every entry point include/bsa.h
declares, and its host-side validation rejects bad arguments before any
GPU work (these calls return before touching the HIP runtime)."""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _ensure_built():
    lib = os.path.join(ROOT, "block_sparse_attention_pool_amd", "_lib", "libbsa.so")
    if not os.path.exists(lib):
        import importlib.util
        path = os.path.join(ROOT, "block_sparse_attention_pool_amd", "build.py")
        spec = importlib.util.spec_from_file_location("bsa_build", path)
        b = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(b)
        b.build()
    return lib


LIB = _ensure_built()
import block_sparse_attention_pool_amd as bsa  # noqa: E402


def header_functions():
    src = open(os.path.join(ROOT, "include", "bsa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bsa_\w+)\s*\(", src)))


def test_header_declares_the_hot_path():
    fns = header_functions()
    for name in ("bsa_score_blocks", "bsa_select_blocks", "bsa_sparse_attn_fwd",
                 "bsa_micro_residual_fwd", "bsa_lse_merge", "bsa_dense_attn_fwd"):
        assert name in fns


def test_every_declared_symbol_is_exported():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (bsa_\w+)$", out, flags=re.M))
    missing = [f for f in header_functions() if f not in exported]
    assert not missing, missing
    assert set(bsa.EXPORTED) == set(header_functions())


def test_version():
    assert "gfx950" in bsa.bsa_version()


def _shape(B=1, H=2, N=1000, d=128, sb=None, sh=None, sn=None):
    sn = d if sn is None else sn
    sh = N * sn if sh is None else sh
    sb = H * sh if sb is None else sb
    return bsa._Shape(B, H, N, d, sb, sh, sn)


def test_workspace_sizes():
    s = _shape(B=1, H=2, N=1000, d=128)
    npad = 16 * 64
    # the fp16 V^T copy, then the micro residual's sub-tile ordering: signatures
    # and order (2 heads x 16 blocks x 4 sub-tiles), bin counts and offsets
    # (2 heads x 64 bins, + 1), a total
    a256 = lambda x: -(-x // 256) * 256
    vt = 2 * 128 * npad * 2
    # ... and the status word in the last 256 bytes
    order = 2 * a256(128 * 4) + a256(128 * 4) + a256(129 * 4) + 256 + 256
    assert bsa._lib.bsa_attn_workspace_bytes(ctypes.byref(s)) == vt + order
    sp, _ = bsa.make_select_params("topk", k=4, nB=16)
    rows, W = 2 * 16, 1
    ws = bsa._lib.bsa_select_workspace_bytes(ctypes.byref(s), 64, ctypes.byref(sp))
    assert ws == 256 + 256 and rows * W * 4 <= 256
    assert bsa._lib.bsa_select_max_nnz(ctypes.byref(s), 64, ctypes.byref(sp)) == rows * 4
    sp.force_diag = 1
    assert bsa._lib.bsa_select_max_nnz(ctypes.byref(s), 64, ctypes.byref(sp)) == rows * 5


@pytest.mark.parametrize("kw,status,msg", [
    (dict(d=96), 2, "head dim"),
    (dict(N=0), 1, "must all be >= 1"),
    (dict(sn=132), 1, "multiples of 8"),
    (dict(sn=100), 1, "inconsistent"),
    (dict(H=300), 2, "exceeds"),
])
def test_shape_validation(kw, status, msg):
    s = _shape(**kw)
    buf = ctypes.c_void_p(4096)
    st = bsa._lib.bsa_score_blocks(buf, buf, ctypes.byref(s), 64, 0.1, buf, buf, None, 0,
                                   None, None, None)
    assert st == status
    assert msg in bsa.bsa_last_error()


def test_null_and_misaligned_pointers():
    s = _shape()
    good = ctypes.c_void_p(4096)
    st = bsa._lib.bsa_score_blocks(None, good, ctypes.byref(s), 64, 0.1, good, good, None, 0,
                                   None, None, None)
    assert st == 1 and "Q is NULL" in bsa.bsa_last_error()
    bad = ctypes.c_void_p(4098)
    st = bsa._lib.bsa_score_blocks(good, bad, ctypes.byref(s), 64, 0.1, good, good, None, 0,
                                   None, None, None)
    assert st == 1 and "aligned" in bsa.bsa_last_error()
    st = bsa._lib.bsa_score_blocks(good, good, ctypes.byref(s), 32, 0.1, good, good, None, 0,
                                   None, None, None)
    assert st == 2 and "block" in bsa.bsa_last_error()


def test_attention_rejects_small_workspace_and_bad_dtype():
    s = _shape()
    p = ctypes.c_void_p(4096)
    need = bsa._lib.bsa_attn_workspace_bytes(ctypes.byref(s))
    st = bsa._lib.bsa_sparse_attn_fwd(p, p, p, ctypes.byref(s), 64, 0.1, p, p, p, 0, p, p,
                                      need - 1, None)
    assert st == 3 and "workspace" in bsa.bsa_last_error()
    st = bsa._lib.bsa_dense_attn_fwd(p, p, p, ctypes.byref(s), 0.1, p, 7, p, p, need, None)
    assert st == 1 and "o_dtype" in bsa.bsa_last_error()


def test_select_rejects_bad_params():
    s = _shape()
    p = ctypes.c_void_p(4096)
    sp, _ = bsa.make_select_params("topp", p=1.5, nB=16)
    ws = bsa._lib.bsa_select_workspace_bytes(ctypes.byref(s), 64, ctypes.byref(sp))
    st = bsa._lib.bsa_select_blocks(p, ctypes.byref(s), 64, ctypes.byref(sp), p, p, 100, p, p,
                                    ws, None)
    assert st == 1 and "p=" in bsa.bsa_last_error()
    sp, _ = bsa.make_select_params("topk", k=4, nB=16)
    st = bsa._lib.bsa_select_blocks(p, ctypes.byref(s), 64, ctypes.byref(sp), p, p, 100, p, p,
                                    1, None)
    assert st == 3
    sp.mode = 9
    assert bsa._lib.bsa_select_workspace_bytes(ctypes.byref(s), 64, ctypes.byref(sp)) == -1
    assert "mode" in bsa.bsa_last_error()
    # scored selection over more than 4096 blocks is refused up front
    big = _shape(N=4097 * 64)
    sp.mode = 0
    assert bsa._lib.bsa_select_workspace_bytes(ctypes.byref(big), 64, ctypes.byref(sp)) == -1
    sp.mode = 2
    assert bsa._lib.bsa_select_workspace_bytes(ctypes.byref(big), 64, ctypes.byref(sp)) == -1


def test_budget_resolution():
    assert bsa.budget_blocks(0.25, 512) == 128
    assert bsa.budget_blocks(0.25, 16) == 4
    assert bsa.budget_blocks(0.15, 1857) == 279
    assert bsa.cap_blocks(0.20, 1182) == 236
    assert bsa.budget_blocks(0.1, 30) == 3


def test_omission_risk_validation_and_workspace():
    s = _shape(B=2, H=3, N=5000)
    chunks = -(-5000 // 2048)
    need = bsa._lib.bsa_omission_risk_workspace_bytes(ctypes.byref(s))
    assert need == -(-(2 * 3 * chunks * 24) // 256) * 256
    p = ctypes.c_void_p(4096)
    st = bsa._lib.bsa_omission_risk(p, p, None, ctypes.byref(s), p, p, need - 1, None)
    assert st == 3 and "workspace" in bsa.bsa_last_error()
    st = bsa._lib.bsa_omission_risk(None, p, None, ctypes.byref(s), p, p, need, None)
    assert st == 1 and "lse_sparse is NULL" in bsa.bsa_last_error()
    st = bsa._lib.bsa_omission_risk(p, p, ctypes.c_void_p(4098), ctypes.byref(s), p, p, need,
                                    None)
    assert st == 1 and "lse_repaired" in bsa.bsa_last_error()
    st = bsa._lib.bsa_omission_risk(p, p, None, ctypes.byref(s), ctypes.c_void_p(4100), p, need,
                                    None)
    assert st == 1 and "risk" in bsa.bsa_last_error()
    # only B, H, N are read: any d is accepted; too many heads is refused
    assert bsa._lib.bsa_omission_risk_workspace_bytes(ctypes.byref(_shape(d=96))) > 0
    assert bsa._lib.bsa_omission_risk_workspace_bytes(ctypes.byref(_shape(B=300, H=256))) == -1
    assert "65535" in bsa.bsa_last_error()
    assert bsa._lib.bsa_omission_risk_workspace_bytes(ctypes.byref(_shape(N=0))) == -1


def test_heads_at_risk_matches_the_oracle_rule():
    import numpy as np
    from oracle import bsa_oracle as O
    rng = np.random.default_rng(5)
    for H in (1, 7, 24, 40):
        risk = np.round(rng.random(H), 1)   # coarse values: many ties
        for n in (0, 1, H // 3, H, H + 2):
            assert bsa.heads_at_risk(risk, n) == O.heads_at_risk(risk, n)


def test_block128_selection_workspace_and_bounds():
    s = _shape(B=1, H=2, N=1000)          # 8 blocks of 128, 16 of 64
    sp, _ = bsa.make_select_params("topk", k=3, nB=8)
    ws = bsa._lib.bsa_select_workspace_bytes(ctypes.byref(s), 128, ctypes.byref(sp))
    # 128-block bitmasks + counts, then the 64-tile bitmasks + counts
    assert ws == 4 * 256
    # each kept 128-block is two tiles: 3 blocks -> at most 6 of 16 tiles per row
    assert bsa._lib.bsa_select_max_nnz(ctypes.byref(s), 128, ctypes.byref(sp)) == 2 * 16 * 6
    assert bsa._lib.bsa_select_workspace_bytes(ctypes.byref(s), 96, ctypes.byref(sp)) == -1
    assert "block=96" in bsa.bsa_last_error()
    sm, _ = bsa.make_select_params("micro", micro=dict(
        m=4, scale=0.1, macro=(_FakeT(4096), _FakeT(4096)), qpool16=_FakeT(4096),
        kpool16=_FakeT(4096)))
    assert bsa._lib.bsa_select_workspace_bytes(ctypes.byref(s), 128, ctypes.byref(sm)) == -1
    assert "MICRO" in bsa.bsa_last_error()


class _FakeT:
    """Stands in for a device tensor where only an address is read."""
    def __init__(self, addr):
        self.addr = addr

    def data_ptr(self):
        return self.addr


def test_pattern_validation():
    s = _shape(B=1, H=1, N=1000)          # 16 blocks of 64
    sp, keep = bsa.make_select_params("static", patterns=dict(diagonals=[-2, 40], columns=[15]))
    assert bsa._lib.bsa_select_workspace_bytes(ctypes.byref(s), 64, ctypes.byref(sp)) > 0
    # patterns add one block each per row to the bound (static mode without
    # a window keeps only the forced set)
    assert bsa._lib.bsa_select_max_nnz(ctypes.byref(s), 64, ctypes.byref(sp)) == 16 * 3
    sp, keep = bsa.make_select_params("static", patterns=dict(columns=[16]))
    assert bsa._lib.bsa_select_workspace_bytes(ctypes.byref(s), 64, ctypes.byref(sp)) == -1
    assert "column 16" in bsa.bsa_last_error()
    sp, keep = bsa.make_select_params("topk", k=1, patterns=dict(diagonals=list(range(65))))
    assert bsa._lib.bsa_select_workspace_bytes(ctypes.byref(s), 64, ctypes.byref(sp)) == -1
    assert "n_diagonals=65" in bsa.bsa_last_error()
    sp, keep = bsa.make_select_params("topk", k=1)
    sp.n_columns = 2                       # count without a list
    assert bsa._lib.bsa_select_workspace_bytes(ctypes.byref(s), 64, ctypes.byref(sp)) == -1
    assert "NULL" in bsa.bsa_last_error()


def test_pooled_rectify_validation_and_workspace():
    s = _shape(B=1, H=2, N=1000)          # 16 blocks, padded to 16
    need = bsa._lib.bsa_pooled_rectify_workspace_bytes(ctypes.byref(s))
    f32 = -(-(2 * 16 * 128 * 4) // 256) * 256
    h16 = -(-(2 * 16 * 128 * 2) // 256) * 256
    spread = -(-(2 * 16 * 4) // 256) * 256  # key spread per block (gain-aware gate)
    assert need == 2 * f32 + 3 * h16 + spread
    p = ctypes.c_void_p(4096)
    st = bsa._lib.bsa_pooled_rectify(p, p, p, ctypes.byref(s), 64, 0.1, 0, p, p, p, 0, p, p,
                                     need - 1, None)
    assert st == 3 and "workspace" in bsa.bsa_last_error()
    st = bsa._lib.bsa_pooled_rectify(p, p, p, ctypes.byref(s), 64, 0.1, 2, p, p, p, 0, p, p,
                                     need, None)
    assert st == 1 and "gain_gate" in bsa.bsa_last_error()
    st = bsa._lib.bsa_pooled_rectify(p, p, p, ctypes.byref(s), 64, 0.0, 1, p, p, p, 0, p, p,
                                     need, None)
    assert st == 1 and "scale" in bsa.bsa_last_error()
    st = bsa._lib.bsa_pooled_rectify(p, p, None, ctypes.byref(s), 64, 0.1, 0, p, p, p, 0, p, p,
                                     need, None)
    assert st == 1 and "V is NULL" in bsa.bsa_last_error()
    st = bsa._lib.bsa_pooled_rectify(p, p, p, ctypes.byref(s), 128, 0.1, 0, p, p, p, 0, p, p,
                                     need, None)
    assert st == 2 and "block" in bsa.bsa_last_error()
    st = bsa._lib.bsa_pooled_rectify(p, p, p, ctypes.byref(s), 64, 0.1, 0, p, p, p, 5, p, p,
                                     need, None)
    assert st == 1 and "o_dtype" in bsa.bsa_last_error()
    big = _shape(N=4097 * 64)
    assert bsa._lib.bsa_pooled_rectify_workspace_bytes(ctypes.byref(big)) == -1


def test_cluster_validation():
    s = _shape(B=1, H=2, N=3 * 8 * 10)
    cp = bsa._ClusterParams(3, 8, 10, 1, 3, 4, 2, 2, 2, 1)
    assert bsa._lib.bsa_cluster_cells(ctypes.byref(s), ctypes.byref(cp)) == 3 * 3 * 3
    # norms (2 heads x 27 cells), three bf16 parts of every centroid, the
    # update buckets (12 tokens per cell) and their slot starts (8 + 1)
    al = lambda n: -(-n // 256) * 256
    assert bsa._lib.bsa_cluster_workspace_bytes(ctypes.byref(s), ctypes.byref(cp)) == \
        al(2 * 27 * 4) + al(2 * 27 * 3 * 128 * 2) + al(2 * 27 * 12 * 4) + al(2 * 27 * 9 * 4)
    bad = bsa._ClusterParams(3, 8, 11, 1, 3, 4, 2, 2, 2, 1)   # 264 != 240 tokens
    assert bsa._lib.bsa_cluster_cells(ctypes.byref(s), ctypes.byref(bad)) == -1
    assert "lattice" in bsa.bsa_last_error()
    cp.iters = 0
    assert bsa._lib.bsa_cluster_cells(ctypes.byref(s), ctypes.byref(cp)) == -1
    cp.iters, cp.kw = 1, 0
    assert bsa._lib.bsa_cluster_cells(ctypes.byref(s), ctypes.byref(cp)) == -1
    cp.kw = 4
    p = ctypes.c_void_p(4096)
    st = bsa._lib.bsa_local_window_cluster(p, ctypes.byref(s), ctypes.byref(cp), p, p, p, p, 255,
                                           None)
    assert st == 3 and "workspace" in bsa.bsa_last_error()
    st = bsa._lib.bsa_local_window_cluster(None, ctypes.byref(s), ctypes.byref(cp), p, p, p, p,
                                           256, None)
    assert st == 1 and "X is NULL" in bsa.bsa_last_error()


def _align(n):
    return -(-n // 256) * 256


def test_cluster_attention_and_merge_validation_and_workspace():
    L = bsa._lib
    s = _shape(B=1, H=2, N=1000, d=128)
    Nq, Nk = 12, 30
    nTP = max(-(-1000 // 64) + Nq, -(-(-(-1000 // 16) + Nk + 1) // 4))
    NP, W = 64 * nTP, 1
    cap = 2 * Nq * (-(-1000 // 16) + Nk + 1 + 3)
    want = sum(_align(x) for x in (
        2 * (Nq + 1) * 4, 2 * Nq * 4, 2 * (Nk + 1) * 4, 2 * nTP * 4, 2 * NP * 4, 2 * Nq * W * 4,
        2 * Nq * 4, (2 * Nq + 1) * 4, 8, 8, 2 * NP * 128 * 2, 2 * NP * 128 * 2, cap * 4))
    assert L.bsa_cluster_attn_workspace_bytes(ctypes.byref(s), Nq, Nk, 0) == want
    assert L.bsa_cluster_attn_workspace_bytes(ctypes.byref(s), 4097, Nk, 0) == -1
    assert "4096" in bsa.bsa_last_error()
    assert L.bsa_cluster_attn_workspace_bytes(ctypes.byref(s), Nq, 0, 0) == -1
    p = ctypes.c_void_p(4096)
    st = L.bsa_cluster_attn_fwd(p, p, p, ctypes.byref(s), 0.1, Nq, Nk, p, p, p, p, p, p, None, p,
                                0, p, None, p, 255, None)
    assert st == 3 and "workspace" in bsa.bsa_last_error()
    st = L.bsa_cluster_attn_fwd(p, p, p, ctypes.byref(s), 0.1, Nq, Nk, p, p, p, p, p, None, None,
                                p, 0, p, None, p, want, None)
    assert st == 1 and "ccol" in bsa.bsa_last_error()
    st = L.bsa_cluster_attn_fwd(p, p, p, ctypes.byref(s), 0.1, Nq, Nk, p, p, p, p, p, p,
                                ctypes.c_void_p(4098), p, 0, p, None, p, want, None)
    assert st == 1 and "group_of" in bsa.bsa_last_error()
    # merging: slot counts up to ceil(1000 / 16) = 63 need 6 bit planes
    mw = sum(_align(x) for x in (2 * Nq * 4, 2 * Nq * 4, 2 * Nq * 4, 2 * Nq * 4, 2 * 2 * 4,
                                 2 * Nq * 4, 2 * Nq * 8, 2 * Nq * 4, 2 * Nq * W * 4, 2 * 6 * W * 4,
                                 2 * 4))
    assert L.bsa_cluster_merge_workspace_bytes(1, 2, 1000, Nq, Nk, 16) == mw
    assert L.bsa_cluster_merge_workspace_bytes(1, 2, 1000, Nq, Nk, 0) == -1
    assert L.bsa_cluster_merge_workspace_bytes(1, 2, 1000, Nq, 5000, 16) == -1
    st = L.bsa_cluster_merge(p, p, p, p, 1, 2, 1000, Nq, Nk, None, 3, 64, 64, 16, p, p, mw, None)
    assert st == 1 and "sides" in bsa.bsa_last_error()
    st = L.bsa_cluster_merge(p, p, p, p, 1, 2, 1000, Nq, Nk, p, 65, 64, 64, 16, p, p, mw, None)
    assert st == 1 and "rounds" in bsa.bsa_last_error()
    st = L.bsa_cluster_merge(p, p, p, p, 1, 2, 1000, Nq, Nk, p, 3, 0, 64, 16, p, p, mw, None)
    assert st == 1 and "tau" in bsa.bsa_last_error()
    st = L.bsa_cluster_merge(p, p, p, p, 1, 2, 1000, Nq, Nk, p, 3, 64, 64, 16, p, p, mw - 1, None)
    assert st == 3 and "workspace" in bsa.bsa_last_error()


def test_lowe_ratio_validation():
    L = bsa._lib
    s = _shape(B=1, H=2, N=3 * 8 * 10)
    cp = bsa._ClusterParams(3, 8, 10, 1, 3, 4, 2, 2, 2, 1)
    p = ctypes.c_void_p(4096)
    st = L.bsa_lowe_ratio_subset(p, ctypes.byref(s), ctypes.byref(cp), p, 241, p, p, p, 256, None)
    assert st == 1 and "n_sub" in bsa.bsa_last_error()
    st = L.bsa_lowe_ratio_subset(p, ctypes.byref(s), ctypes.byref(cp), p, -1, p, p, p, 256, None)
    assert st == 1 and "n_sub" in bsa.bsa_last_error()
    st = L.bsa_lowe_ratio_subset(p, ctypes.byref(s), ctypes.byref(cp), p, 36, p, None, p, 256,
                                 None)
    assert st == 1 and "subset is NULL" in bsa.bsa_last_error()
    st = L.bsa_lowe_ratio_subset(p, ctypes.byref(s), ctypes.byref(cp), p, 36, p, p, p, 255, None)
    assert st == 3 and "workspace" in bsa.bsa_last_error()
    st = L.bsa_lowe_ratio_subset(p, ctypes.byref(s), ctypes.byref(cp), None, 36, p, p, p, 256,
                                 None)
    assert st == 1 and "centroids is NULL" in bsa.bsa_last_error()


def test_stage_v_validation():
    L = bsa._lib
    s = _shape(B=1, H=2, N=1000, d=128)
    need = L.bsa_attn_workspace_bytes(ctypes.byref(s))
    p = ctypes.c_void_p(4096)
    assert L.bsa_attn_stage_v(p, ctypes.byref(s), p, need - 1, None) == 3
    assert "workspace" in bsa.bsa_last_error()
    assert L.bsa_attn_stage_v(None, ctypes.byref(s), p, need, None) == 1
    assert "V is NULL" in bsa.bsa_last_error()
    assert L.bsa_attn_stage_v(ctypes.c_void_p(4098), ctypes.byref(s), p, need, None) == 1
    bad = _shape(B=1, H=2, N=1000, d=96)
    assert L.bsa_attn_stage_v(p, ctypes.byref(bad), p, need, None) == 2


# ------------------------------------------------------------ CSR validation

def _csr(rows):
    import numpy as np
    rp = np.zeros(len(rows) + 1, np.int32)
    rp[1:] = np.cumsum([len(r) for r in rows])
    ci = np.array([j for r in rows for j in r] or [0], np.int32)
    return rp, ci


def test_validate_csr_host_accepts_valid_lists():
    import numpy as np
    rp, ci = _csr([[0, 3, 5], [], [1], [0, 1, 2, 3, 4, 5, 6, 7]])
    assert bsa.bsa_validate_csr_host(rp, ci, 8) == -1
    # an empty CSR (no rows) and rows with no entries at all
    assert bsa.bsa_validate_csr_host(np.zeros(1, np.int32), np.zeros(1, np.int32), 8) == -1
    assert bsa.bsa_validate_csr_host(np.zeros(4, np.int32), np.zeros(1, np.int32), 8) == -1


@pytest.mark.parametrize("case,row,msg", [
    ("col_high", 1, "outside"), ("col_negative", 0, "outside"), ("unsorted", 2, "ascending"),
    ("duplicate", 2, "ascending"), ("ptr_back", 1, "out of order"), ("ptr_past_cap", 2, "col_cap"),
    ("ptr0", 0, "row_ptr[0]"),
])
def test_validate_csr_host_names_the_first_bad_row(case, row, msg):
    import numpy as np
    rows = [[0, 3], [1, 2], [4, 6], [7]]
    if case == "col_high":
        rows[1] = [1, 8]
    elif case == "col_negative":
        rows[0] = [-1, 3]
    elif case == "unsorted":
        rows[2] = [6, 4]
    elif case == "duplicate":
        rows[2] = [4, 4]
    rp, ci = _csr(rows)
    if case == "ptr_back":
        rp[2] = 1                # row 1 ends before it starts
    elif case == "ptr_past_cap":
        ci = ci[:5]              # row 2 ends at 6, past the 5 entries there are
    elif case == "ptr0":
        rp = rp + 1
        ci = np.concatenate([[0], ci]).astype(np.int32)
    with pytest.raises(bsa.BsaError) as e:
        bsa.bsa_validate_csr_host(rp, ci, 8)
    assert f"row {row}:" in str(e.value) and msg in str(e.value)


def test_validate_csr_host_matches_a_plain_rule_on_random_lists():
    import numpy as np
    rng = np.random.default_rng(11)
    for trial in range(200):
        n_rows, n_cols = int(rng.integers(1, 9)), int(rng.integers(1, 12))
        rows = [sorted(rng.choice(n_cols, size=int(rng.integers(0, n_cols + 1)), replace=False).tolist())
                for _ in range(n_rows)]
        if trial % 3 == 1 and any(rows):
            r = next(i for i, x in enumerate(rows) if x)
            rows[r][-1] = n_cols + int(rng.integers(0, 3))       # out of range
        elif trial % 3 == 2 and any(len(x) > 1 for x in rows):
            r = next(i for i, x in enumerate(rows) if len(x) > 1)
            rows[r][0], rows[r][1] = rows[r][1], rows[r][0]      # unsorted
        ok = all(all(0 <= j < n_cols for j in x) and all(a < b for a, b in zip(x, x[1:]))
                 for x in rows)
        rp, ci = _csr(rows)
        if ok:
            assert bsa.bsa_validate_csr_host(rp, ci, n_cols) == -1
        else:
            with pytest.raises(bsa.BsaError):
                bsa.bsa_validate_csr_host(rp, ci, n_cols)


def test_check_csr_and_take_status_validate_before_any_launch():
    s = _shape(B=1, H=2, N=1000)
    p = ctypes.c_void_p(4096)
    assert bsa._lib.bsa_check_csr(p, -1, p, 10, 16, p, None) == 1
    assert bsa._lib.bsa_check_csr(p, 4, p, -1, 16, p, None) == 1
    assert bsa._lib.bsa_check_csr(None, 4, p, 10, 16, p, None) == 1
    need = bsa._lib.bsa_attn_workspace_bytes(ctypes.byref(s))
    assert bsa._lib.bsa_attn_take_status(p, need - 1, ctypes.byref(s), p, None) == 3
    assert bsa._lib.bsa_attn_take_status(p, need, ctypes.byref(s), None, None) == 1


def test_heads_at_risk_rejects_nan_and_bad_sizes():
    import numpy as np
    with pytest.raises(bsa.BsaError):
        bsa.heads_at_risk(np.array([0.1, float("nan")]), 1)
    assert bsa._lib.bsa_heads_at_risk(None, 3, 1, None) == 1



def test_noalloc_select_refuses_oversized_work_before_any_hip_call():
    # micro tile scores of 8 heads of 65,536 tokens need 512 MiB > 32 MiB;
    # the refusal comes from the size check, before any HIP call (no GPU here)
    assert bsa._lib.bsa_select_scratch_limit() == 32 << 20
    s = _shape(B=1, H=8, N=65536, d=64)
    sp, keep = bsa.make_select_params("micro", micro=dict(
        m=4, scale=0.125, macro=(_AddrOnly(), _AddrOnly()), qpool16=_AddrOnly(), kpool16=_AddrOnly()))
    p = ctypes.c_void_p(4096)
    st = bsa._lib.bsa_select_blocks_noalloc(None, ctypes.byref(s), 64, ctypes.byref(sp), p, p, 10,
                                            p, None)
    assert st == 3 and "scratch" in bsa.bsa_last_error()


class _AddrOnly:
    """Stands in for a device tensor in the parameter struct (only its
    address is stored)."""
    shape = (1, 8, 1, 1)

    def data_ptr(self):
        return 4096
