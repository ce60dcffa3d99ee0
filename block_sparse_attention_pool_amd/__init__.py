"""Python binding of the gfx950 block-sparse attention library (libbsa.so).

Argument marshalling only: every function below allocates its outputs with
torch (device memory and streams are all torch is used for), passes raw
pointers and sizes to the C entry point of the same name declared in
``include/bsa.h``, and raises on a non-zero status.  All computation runs in
the HIP kernels of the library.  The library must have been built
(``python block_sparse_attention_pool_amd/build.py``); importing this module
fails loudly when it is missing.

Tensors Q, K, V are bf16 ``[B, H, N, d]`` on the GPU with the last dimension
contiguous (any strides otherwise, shared by Q, K, V and the outputs).
"""

from __future__ import annotations

import ctypes
import math
import os
from fractions import Fraction

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libbsa.so")

BSA_OK = 0
BSA_F32, BSA_BF16 = 0, 1
SELECT_MODES = {"topk": 0, "topp": 1, "static": 2, "micro": 3}
BLOCK = 64
MICRO = 16


class BsaError(RuntimeError):
    pass


class _Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("d", ctypes.c_int32), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("stride_n", ctypes.c_int64)]


class _SelectParams(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("k", ctypes.c_int32), ("p", ctypes.c_float),
                ("k_min", ctypes.c_int32), ("k_cap", ctypes.c_int32),
                ("force_diag", ctypes.c_int32), ("use_static", ctypes.c_int32),
                ("frame_tokens", ctypes.c_int32), ("window_frames", ctypes.c_int32),
                ("n_anchors", ctypes.c_int32), ("anchor_offset", ctypes.c_int32),
                ("micro", ctypes.c_int32), ("micro_m", ctypes.c_int32),
                ("scale", ctypes.c_float), ("head_mask", ctypes.c_void_p),
                ("macro_row_ptr", ctypes.c_void_p), ("macro_col_idx", ctypes.c_void_p),
                ("qpool16", ctypes.c_void_p), ("kpool16", ctypes.c_void_p),
                ("n_diagonals", ctypes.c_int32), ("diagonals", ctypes.c_void_p),
                ("n_columns", ctypes.c_int32), ("columns", ctypes.c_void_p)]


class _ClusterParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("T", "Hg", "W", "kt", "kh", "kw", "wt", "wh", "ww",
                                              "iters")]


def _load(path: str = _LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with "
            "`python block_sparse_attention_pool_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    P, I32, I64, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    SP = ctypes.POINTER(_Shape)
    PP = ctypes.POINTER(_SelectParams)
    CP = ctypes.POINTER(_ClusterParams)
    sig = {
        "bsa_version": ([], ctypes.c_char_p),
        "bsa_last_error": ([], ctypes.c_char_p),
        "bsa_score_blocks": ([P, P, SP, I32, F32, P, P, P, I32, P, P, P], I32),
        "bsa_select_workspace_bytes": ([SP, I32, PP], I64),
        "bsa_select_max_nnz": ([SP, I32, PP], I64),
        "bsa_select_blocks": ([P, SP, I32, PP, P, P, I64, P, P, I64, P], I32),
        "bsa_attn_workspace_bytes": ([SP], I64),
        "bsa_sparse_attn_fwd": ([P, P, P, SP, I32, F32, P, P, P, I32, P, P, I64, P], I32),
        "bsa_dense_attn_fwd": ([P, P, P, SP, F32, P, I32, P, P, I64, P], I32),
        "bsa_micro_residual_fwd": ([P, P, P, SP, I32, I32, F32, P, P, P, P, I32, P, P, I64, P],
                                   I32),
        "bsa_lse_merge": ([P, P, P, P, SP, I32, P, P, P, P], I32),
        "bsa_omission_risk_workspace_bytes": ([SP], I64),
        "bsa_pooled_rectify_workspace_bytes": ([SP], I64),
        "bsa_cluster_cells": ([SP, CP], I64),
        "bsa_cluster_workspace_bytes": ([SP, CP], I64),
        "bsa_local_window_cluster": ([P, SP, CP, P, P, P, P, I64, P], I32),
        "bsa_cluster_permute_workspace_bytes": ([SP, CP], I64),
        "bsa_cluster_permute": ([P, P, SP, CP, P, P, P, I64, P], I32),
        "bsa_cluster_select_workspace_bytes": ([I32, I32, I32, I32], I64),
        "bsa_cluster_attn_workspace_bytes": ([SP, I32, I32, I32], I64),
        "bsa_cluster_attn_fwd": ([P, P, P, SP, F32, I32, I32, P, P, P, P, P, P, P, P, I32, P, P, P,
                                  I64, P], I32),
        "bsa_cluster_merge_workspace_bytes": ([I32, I32, I32, I32, I32, I32], I64),
        "bsa_lowe_ratio_subset": ([P, SP, CP, P, I32, P, P, P, I64, P], I32),
        "bsa_attn_stage_v": ([P, SP, P, I64, P], I32),
        "bsa_cluster_merge": ([P, P, P, P, I32, I32, I32, I32, I32, P, I32, I32, I32, I32, P, P,
                               I64, P], I32),
        "bsa_cluster_select": ([P, P, P, I32, I32, I32, I32, I32, F32, F32, I32, I32, P, P, I64,
                                P, P, I64, P], I32),
        "bsa_pooled_rectify": ([P, P, P, SP, I32, F32, I32, P, P, P, I32, P, P, I64, P], I32),
        "bsa_omission_risk": ([P, P, P, SP, P, P, I64, P], I32),
        "bsa_heads_at_risk": ([P, I32, I32, P], I32),
        "bsa_subset_refine_workspace_bytes": ([SP, I32], I64),
        "bsa_subset_refine": ([P, SP, I32, P, I32, P, P, P, P, I64, P], I32),
        "bsa_select_blocks_noalloc": ([P, SP, I32, PP, P, P, I64, P, P], I32),
        "bsa_select_scratch_limit": ([], I64),
        "bsa_attn_take_status": ([P, I64, SP, P, P], I32),
        "bsa_check_csr": ([P, I64, P, I64, I32, P, P], I32),
        "bsa_validate_csr_host": ([P, I64, P, I64, I32, P], I32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()
EXPORTED = ("bsa_version", "bsa_last_error", "bsa_score_blocks", "bsa_select_workspace_bytes",
            "bsa_select_max_nnz", "bsa_select_blocks", "bsa_attn_workspace_bytes",
            "bsa_sparse_attn_fwd", "bsa_dense_attn_fwd", "bsa_micro_residual_fwd",
            "bsa_lse_merge", "bsa_omission_risk_workspace_bytes", "bsa_omission_risk",
            "bsa_pooled_rectify_workspace_bytes", "bsa_pooled_rectify", "bsa_cluster_cells",
            "bsa_cluster_workspace_bytes", "bsa_local_window_cluster",
            "bsa_cluster_permute_workspace_bytes", "bsa_cluster_permute",
            "bsa_cluster_select_workspace_bytes", "bsa_cluster_select",
            "bsa_cluster_attn_workspace_bytes", "bsa_cluster_attn_fwd",
            "bsa_cluster_merge_workspace_bytes", "bsa_cluster_merge", "bsa_lowe_ratio_subset",
            "bsa_attn_stage_v", "bsa_heads_at_risk", "bsa_attn_take_status", "bsa_check_csr",
            "bsa_validate_csr_host", "bsa_select_blocks_noalloc", "bsa_select_scratch_limit",
            "bsa_subset_refine_workspace_bytes", "bsa_subset_refine")


def library_path() -> str:
    return _LIB_PATH


def bsa_version() -> str:
    return _lib.bsa_version().decode()


def bsa_last_error() -> str:
    return _lib.bsa_last_error().decode()


def _check(status: int, what: str):
    if status != BSA_OK:
        raise BsaError(f"{what} failed (status {status}): {bsa_last_error()}")


# ----------------------------------------------------------------- marshalling

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def shape_of(Q: torch.Tensor) -> _Shape:
    """bsa_shape of a [B, H, N, d] tensor (element strides, d contiguous)."""
    if Q.dim() != 4:
        raise ValueError("expected a [B, H, N, d] tensor")
    B, H, N, d = Q.shape
    if Q.stride(3) != 1:
        raise ValueError("the last dimension must be contiguous")
    return _Shape(B, H, N, d, Q.stride(0), Q.stride(1), Q.stride(2))


def _same_layout(*ts):
    ts = [t for t in ts if t is not None]
    ref = ts[0]
    for t in ts[1:]:
        if t.shape != ref.shape or t.stride() != ref.stride():
            raise ValueError("Q, K, V (and outputs) must share shape and strides")
        if t.dtype != torch.bfloat16 or ref.dtype != torch.bfloat16:
            raise ValueError("Q, K, V must be bfloat16")


def _out_like(Q, dtype):
    return torch.empty_strided(Q.shape, Q.stride(), dtype=dtype, device=Q.device)


def _odt(dtype):
    if dtype == torch.float32:
        return BSA_F32
    if dtype == torch.bfloat16:
        return BSA_BF16
    raise ValueError("output dtype must be float32 or bfloat16")


def n_blocks(N: int, b: int = BLOCK) -> int:
    return -(-N // b)


def budget_blocks(density: float, nB: int) -> int:
    """Blocks kept for a density budget: ceil(density * nB), exact in
    decimal so that 0.25 * 512 is 128 and not 128.00000000000003."""
    return math.ceil(Fraction(str(density)) * nB)


def cap_blocks(density: float, nB: int) -> int:
    """Largest row length under a density cap: floor(density * nB)."""
    return math.floor(Fraction(str(density)) * nB)


def _head_mask(head_mask, H):
    if head_mask is None:
        return None, None
    arr = (ctypes.c_uint8 * H)(*[1 if h else 0 for h in head_mask])
    return arr, ctypes.cast(arr, ctypes.c_void_p)


# ---------------------------------------------------------------- entry points

def bsa_score_blocks(Q, K, *, block: int = BLOCK, scale: float | None = None,
                     scores: bool = True, micro: int = 0, stream=None):
    """Pooled means and pooled block scores.  Returns a dict with qpool,
    kpool [B,H,nB,d], scores [B,H,nB,nB] (or None) and, when micro=16,
    qpool16, kpool16 [B,H,nT,d]; all float32."""
    _same_layout(Q, K)
    shp = shape_of(Q)
    B, H, N, d = Q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    nB, nT = n_blocks(N, block), n_blocks(N, MICRO)
    f32 = dict(dtype=torch.float32, device=Q.device)
    out = dict(qpool=torch.empty((B, H, nB, d), **f32), kpool=torch.empty((B, H, nB, d), **f32),
               scores=torch.empty((B, H, nB, nB), **f32) if scores else None,
               qpool16=torch.empty((B, H, nT, d), **f32) if micro else None,
               kpool16=torch.empty((B, H, nT, d), **f32) if micro else None)
    st = _lib.bsa_score_blocks(_ptr(Q), _ptr(K), ctypes.byref(shp), block, scale,
                               _ptr(out["qpool"]), _ptr(out["kpool"]), _ptr(out["scores"]),
                               micro, _ptr(out["qpool16"]), _ptr(out["kpool16"]),
                               _stream(stream, Q.device))
    _check(st, "bsa_score_blocks")
    return out


def make_select_params(mode: str = "topk", *, k: int = 0, p: float = 0.9, k_min: int = 1,
                       k_cap: int | None = None, force_diag: bool = False,
                       static: dict | None = None, micro: dict | None = None,
                       patterns: dict | None = None, nB: int | None = None):
    """bsa_select_params for the arguments of bsa_select_blocks, plus the
    host arrays it points to (keep them alive for the call)."""
    sp = _SelectParams()
    sp.mode = SELECT_MODES[mode]
    sp.k = k
    sp.p = p
    sp.k_min = k_min
    sp.k_cap = (nB if nB is not None else 1 << 30) if k_cap is None else k_cap
    sp.force_diag = 1 if force_diag else 0
    if static is not None:
        sp.use_static = 1
        sp.frame_tokens = static["frame_tokens"]
        sp.window_frames = static["window_frames"]
        sp.n_anchors = static.get("n_anchors", 0)
        sp.anchor_offset = static.get("anchor_offset", 0)
    keep = []
    if patterns is not None:
        for field, cnt in (("diagonals", "n_diagonals"), ("columns", "n_columns")):
            vals = [int(v) for v in patterns.get(field, ())]
            arr = (ctypes.c_int32 * max(1, len(vals)))(*vals)
            keep.append(arr)
            setattr(sp, cnt, len(vals))
            setattr(sp, field, ctypes.cast(arr, ctypes.c_void_p).value)
    if micro is not None:
        sp.micro = micro.get("micro", MICRO)
        sp.micro_m = micro["m"]
        sp.scale = micro["scale"]
        row_ptr, col_idx = micro["macro"]
        sp.macro_row_ptr = row_ptr.data_ptr()
        sp.macro_col_idx = col_idx.data_ptr()
        sp.qpool16 = micro["qpool16"].data_ptr()
        sp.kpool16 = micro["kpool16"].data_ptr()
        if micro.get("head_mask") is not None:
            H = micro["qpool16"].shape[1]
            arr, ptr = _head_mask(micro["head_mask"], H)
            keep.append(arr)
            sp.head_mask = ptr.value
    return sp, keep


def bsa_select_blocks(scores, Q_like, *, block: int = BLOCK, mode: str = "topk", k: int = 0,
                      p: float = 0.9, k_min: int = 1, k_cap: int | None = None,
                      force_diag: bool = False, static: dict | None = None,
                      micro: dict | None = None, patterns: dict | None = None, stream=None):
    """CSR block lists.  ``Q_like`` supplies the shape ([B,H,N,d] tensor).
    ``block`` is the selection block (64 or 128; scores, k and the forced
    set count in it); the lists are always emitted on 64-token tiles.
    ``patterns`` = {"diagonals": offsets, "columns": key blocks} adds MOD-DiT
    structural patterns.  Returns (row_ptr int32 [B*H*ceil(N/64)+1], col_idx
    int32 [capacity], nnz int64 device scalar); the first nnz entries of
    col_idx are valid."""
    shp = shape_of(Q_like)
    nB = n_blocks(shp.N, block)
    sp, keep = make_select_params(mode, k=k, p=p, k_min=k_min, k_cap=k_cap,
                                  force_diag=force_diag, static=static, micro=micro,
                                  patterns=patterns, nB=nB)
    ws_bytes = _lib.bsa_select_workspace_bytes(ctypes.byref(shp), block, ctypes.byref(sp))
    if ws_bytes < 0:
        raise BsaError(f"bsa_select_workspace_bytes: {bsa_last_error()}")
    cap = _lib.bsa_select_max_nnz(ctypes.byref(shp), block, ctypes.byref(sp))
    dev = Q_like.device
    rows = shp.B * shp.H * n_blocks(shp.N, BLOCK)
    row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    nnz = torch.empty(1, dtype=torch.int64, device=dev)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    st = _lib.bsa_select_blocks(_ptr(scores), ctypes.byref(shp), block, ctypes.byref(sp),
                                _ptr(row_ptr), _ptr(col_idx), cap, _ptr(nnz), _ptr(ws),
                                ws.numel(), _stream(stream, dev))
    _check(st, "bsa_select_blocks")
    del keep
    return row_ptr, col_idx, nnz


def bsa_select_blocks_noalloc(scores, Q_like, *, row_ptr, col_idx, nnz, block: int = BLOCK,
                              mode: str = "topk", k: int = 0, p: float = 0.9, k_min: int = 1,
                              k_cap: int | None = None, force_diag: bool = False,
                              static: dict | None = None, micro: dict | None = None,
                              patterns: dict | None = None, stream=None):
    """bsa_select_blocks into caller-given outputs (row_ptr int32
    [B*H*ceil(N/64)+1], col_idx int32 [capacity], nnz int64 [1]) with the
    library's static scratch: nothing is allocated here or in the library.
    Returns (row_ptr, col_idx, nnz)."""
    shp = shape_of(Q_like)
    nB = n_blocks(shp.N, block)
    sp, keep = make_select_params(mode, k=k, p=p, k_min=k_min, k_cap=k_cap,
                                  force_diag=force_diag, static=static, micro=micro,
                                  patterns=patterns, nB=nB)
    st = _lib.bsa_select_blocks_noalloc(_ptr(scores), ctypes.byref(shp), block, ctypes.byref(sp),
                                        _ptr(row_ptr), _ptr(col_idx), col_idx.numel(), _ptr(nnz),
                                        _stream(stream, Q_like.device))
    _check(st, "bsa_select_blocks_noalloc")
    del keep
    return row_ptr, col_idx, nnz


def attn_workspace(Q) -> torch.Tensor:
    """The attention calls' workspace, its status word (last 256 bytes)
    zeroed."""
    shp = shape_of(Q)
    n = _lib.bsa_attn_workspace_bytes(ctypes.byref(shp))
    if n < 0:
        raise BsaError(f"bsa_attn_workspace_bytes: {bsa_last_error()}")
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=Q.device)
    ws[-256:].zero_()
    return ws


def bsa_attn_take_status(workspace, Q_like, *, stream=None) -> torch.Tensor:
    """The attention workspace's status word (device int32 [1]), cleared in
    the workspace.  Bit 1: an out-of-range column or tile index was skipped
    since the last clear."""
    shp = shape_of(Q_like)
    out = torch.empty(1, dtype=torch.int32, device=workspace.device)
    st = _lib.bsa_attn_take_status(_ptr(workspace), workspace.numel(), ctypes.byref(shp),
                                   _ptr(out), _stream(stream, workspace.device))
    _check(st, "bsa_attn_take_status")
    return out


def bsa_check_csr(row_ptr, col_idx, n_cols: int, *, stream=None) -> torch.Tensor:
    """Checks a device CSR (int32 row_ptr [rows + 1], int32 col_idx [cap]).
    Returns device int32 [3]: rows with bad pointers, entries outside
    [0, n_cols), entries not strictly ascending."""
    counts = torch.empty(3, dtype=torch.int32, device=row_ptr.device)
    st = _lib.bsa_check_csr(_ptr(row_ptr), row_ptr.numel() - 1, _ptr(col_idx), col_idx.numel(),
                            n_cols, _ptr(counts), _stream(stream, row_ptr.device))
    _check(st, "bsa_check_csr")
    return counts


def bsa_validate_csr_host(row_ptr, col_idx, n_cols: int) -> int:
    """Validates a host CSR (int32 numpy arrays or CPU tensors).  Returns -1
    when valid, else raises BsaError naming the first bad row."""
    import numpy as np
    rp = np.ascontiguousarray(np.asarray(row_ptr), dtype=np.int32)
    ci = np.ascontiguousarray(np.asarray(col_idx), dtype=np.int32)
    bad = ctypes.c_int64(-1)
    st = _lib.bsa_validate_csr_host(rp.ctypes.data_as(ctypes.c_void_p), rp.size - 1,
                                    ci.ctypes.data_as(ctypes.c_void_p), ci.size, n_cols,
                                    ctypes.byref(bad))
    if st != BSA_OK:
        raise BsaError(f"bsa_validate_csr_host: row {bad.value}: {bsa_last_error()}")
    return bad.value


def bsa_sparse_attn_fwd(Q, K, V, row_ptr, col_idx, *, block: int = BLOCK,
                        scale: float | None = None, out_dtype=torch.float32, out=None,
                        lse=None, workspace=None, stream=None):
    """Block-sparse attention forward.  Returns (O [B,H,N,d] out_dtype,
    LSE float32 [B,H,N]).  V=None reuses the fp16 V^T already in
    ``workspace`` from an earlier call on the same V."""
    _same_layout(Q, K, V)
    shp = shape_of(Q)
    scale = 1.0 / math.sqrt(shp.d) if scale is None else scale
    O = _out_like(Q, out_dtype) if out is None else out
    L = torch.empty(Q.shape[:3], dtype=torch.float32, device=Q.device) if lse is None else lse
    ws = attn_workspace(Q) if workspace is None else workspace
    st = _lib.bsa_sparse_attn_fwd(_ptr(Q), _ptr(K), _ptr(V), ctypes.byref(shp), block, scale,
                                  _ptr(row_ptr), _ptr(col_idx), _ptr(O), _odt(O.dtype), _ptr(L),
                                  _ptr(ws), ws.numel(), _stream(stream, Q.device))
    _check(st, "bsa_sparse_attn_fwd")
    return O, L


def bsa_attn_stage_v(V, *, workspace, stream=None):
    """Stage the fp16 V^T of V [B,H,N,d] bf16 into an attention workspace, on
    its own (the attention calls then take V=None)."""
    shp = shape_of(V)
    st = _lib.bsa_attn_stage_v(_ptr(V), ctypes.byref(shp), _ptr(workspace), workspace.numel(),
                               _stream(stream, V.device))
    _check(st, "bsa_attn_stage_v")
    return workspace


def bsa_dense_attn_fwd(Q, K, V, *, scale: float | None = None, out_dtype=torch.float32,
                       out=None, lse=None, workspace=None, stream=None):
    """Full attention with the same engine.  Returns (O, LSE)."""
    _same_layout(Q, K, V)
    shp = shape_of(Q)
    scale = 1.0 / math.sqrt(shp.d) if scale is None else scale
    O = _out_like(Q, out_dtype) if out is None else out
    L = torch.empty(Q.shape[:3], dtype=torch.float32, device=Q.device) if lse is None else lse
    ws = attn_workspace(Q) if workspace is None else workspace
    st = _lib.bsa_dense_attn_fwd(_ptr(Q), _ptr(K), _ptr(V), ctypes.byref(shp), scale, _ptr(O),
                                 _odt(O.dtype), _ptr(L), _ptr(ws), ws.numel(),
                                 _stream(stream, Q.device))
    _check(st, "bsa_dense_attn_fwd")
    return O, L


def bsa_micro_residual_fwd(Q, K, V, mrow_ptr, midx, *, head_mask=None, block: int = BLOCK,
                           micro: int = MICRO, scale: float | None = None,
                           out_dtype=torch.float32, out=None, lse=None, workspace=None,
                           stream=None):
    """Micro-tile residual attention.  Heads outside ``head_mask`` are left
    untouched in ``out``/``lse`` (fresh outputs hold garbage there)."""
    _same_layout(Q, K, V)
    shp = shape_of(Q)
    scale = 1.0 / math.sqrt(shp.d) if scale is None else scale
    O = _out_like(Q, out_dtype) if out is None else out
    L = torch.empty(Q.shape[:3], dtype=torch.float32, device=Q.device) if lse is None else lse
    ws = attn_workspace(Q) if workspace is None else workspace
    arr, hm = _head_mask(head_mask, shp.H)
    st = _lib.bsa_micro_residual_fwd(_ptr(Q), _ptr(K), _ptr(V), ctypes.byref(shp), block, micro,
                                     scale, _ptr(mrow_ptr), _ptr(midx), hm, _ptr(O),
                                     _odt(O.dtype), _ptr(L), _ptr(ws), ws.numel(),
                                     _stream(stream, Q.device))
    _check(st, "bsa_micro_residual_fwd")
    return O, L


def bsa_lse_merge(O1, L1, O2, L2, *, head_mask=None, out=None, lse_out=None, stream=None):
    """Exact LSE merge of two partial results.  out/lse_out may be O1/L1."""
    if O1.dtype != O2.dtype or O1.shape != O2.shape or O1.stride() != O2.stride():
        raise ValueError("O1 and O2 must share dtype, shape and strides")
    shp = shape_of(O1)
    O = _out_like(O1, O1.dtype) if out is None else out
    L = torch.empty_like(L1) if lse_out is None else lse_out
    arr, hm = _head_mask(head_mask, shp.H)
    st = _lib.bsa_lse_merge(_ptr(O1), _ptr(L1), _ptr(O2), _ptr(L2), ctypes.byref(shp),
                            _odt(O1.dtype), hm, _ptr(O), _ptr(L), _stream(stream, O1.device))
    _check(st, "bsa_lse_merge")
    return O, L


def rectify_workspace(Q) -> torch.Tensor:
    shp = shape_of(Q)
    n = _lib.bsa_pooled_rectify_workspace_bytes(ctypes.byref(shp))
    if n < 0:
        raise BsaError(f"bsa_pooled_rectify_workspace_bytes: {bsa_last_error()}")
    return torch.empty(max(n, 256), dtype=torch.uint8, device=Q.device)


def bsa_pooled_rectify(Q, K, V, row_ptr, col_idx, O, LSE, *, block: int = BLOCK,
                       scale: float | None = None, gain_gate: bool = False, workspace=None,
                       stream=None):
    """Adds the pooled estimate of every row's omitted key blocks to the
    sparse result (O, LSE) of the same CSR, in place; with ``gain_gate``
    only the (query, block) pairs whose estimate passes the gain-aware test.
    Returns (O, LSE)."""
    _same_layout(Q, K, V)
    shp = shape_of(Q)
    if O.shape != Q.shape or O.stride() != Q.stride():
        raise ValueError("O must share shape and strides with Q")
    scale = 1.0 / math.sqrt(shp.d) if scale is None else scale
    ws = rectify_workspace(Q) if workspace is None else workspace
    st = _lib.bsa_pooled_rectify(_ptr(Q), _ptr(K), _ptr(V), ctypes.byref(shp), block, scale,
                                 1 if gain_gate else 0, _ptr(row_ptr), _ptr(col_idx), _ptr(O),
                                 _odt(O.dtype), _ptr(LSE), _ptr(ws), ws.numel(),
                                 _stream(stream, Q.device))
    _check(st, "bsa_pooled_rectify")
    return O, LSE


def bsa_local_window_cluster(X, thw, cell, window, iters: int = 1, *, stream=None):
    """3D local-window clustering of a [B, H, N, d] bf16 tensor over the
    token lattice thw = (T, Hg, W).  Returns (assign int32 [B, H, N],
    centroids float32 [B, H, cells, d], counts int32 [B, H, cells])."""
    if X.dtype != torch.bfloat16:
        raise ValueError("X must be bfloat16")
    shp = shape_of(X)
    cp = _ClusterParams(*thw, *cell, *window, iters)
    cells = _lib.bsa_cluster_cells(ctypes.byref(shp), ctypes.byref(cp))
    if cells < 0:
        raise BsaError(f"bsa_cluster_cells: {bsa_last_error()}")
    nws = _lib.bsa_cluster_workspace_bytes(ctypes.byref(shp), ctypes.byref(cp))
    B, H, N, d = X.shape
    dev = X.device
    assign = torch.empty((B, H, N), dtype=torch.int32, device=dev)
    mu = torch.empty((B, H, cells, d), dtype=torch.float32, device=dev)
    counts = torch.empty((B, H, cells), dtype=torch.int32, device=dev)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)
    st = _lib.bsa_local_window_cluster(_ptr(X), ctypes.byref(shp), ctypes.byref(cp), _ptr(assign),
                                       _ptr(mu), _ptr(counts), _ptr(ws), ws.numel(),
                                       _stream(stream, dev))
    _check(st, "bsa_local_window_cluster")
    return assign, mu, counts


def bsa_lowe_ratio_subset(X, centroids, thw, cell, window, frac: float = 0.15, *,
                          n_sub: int | None = None, stream=None):
    """Lowe's ratio (HVA Eq. 6) of every token of X [B, H, N, d] bf16 over its
    window's centroids, and the ceil(frac * N) tokens of largest ratio per
    head (or ``n_sub`` of them).  Returns (rho float32 [B, H, N], subset
    int32 [B, H, n_sub] ascending)."""
    if X.dtype != torch.bfloat16:
        raise ValueError("X must be bfloat16")
    shp = shape_of(X)
    cp = _ClusterParams(*thw, *cell, *window, 1)
    B, H, N, d = X.shape
    if n_sub is None:
        n_sub = budget_blocks(frac, N)
    nws = _lib.bsa_cluster_workspace_bytes(ctypes.byref(shp), ctypes.byref(cp))
    if nws < 0:
        raise BsaError(f"bsa_cluster_workspace_bytes: {bsa_last_error()}")
    dev = X.device
    rho = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    subset = torch.empty((B, H, max(n_sub, 1)), dtype=torch.int32, device=dev)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)
    mu = centroids.contiguous()
    if mu.dtype != torch.float32 or tuple(mu.shape[:2]) != (B, H) or mu.shape[3] != d:
        raise ValueError("centroids must be float32 [B, H, cells, d]")
    st = _lib.bsa_lowe_ratio_subset(_ptr(X), ctypes.byref(shp), ctypes.byref(cp),
                                    _ptr(mu), n_sub, _ptr(rho), _ptr(subset),
                                    _ptr(ws), ws.numel(), _stream(stream, dev))
    _check(st, "bsa_lowe_ratio_subset")
    return rho, subset[..., :n_sub]


def bsa_cluster_permute(assign, counts, X_like, thw, cell, window, *, stream=None):
    """Tokens in cluster order (HVA Eq. 1) from bsa_local_window_cluster's
    assign [B, H, N] and counts [B, H, cells].  Returns (perm int32
    [B, H, N], offsets int32 [B, H, cells + 1])."""
    shp = shape_of(X_like)
    cp = _ClusterParams(*thw, *cell, *window, 1)
    B, H, N, _ = X_like.shape
    cells = counts.shape[2]
    nws = _lib.bsa_cluster_permute_workspace_bytes(ctypes.byref(shp), ctypes.byref(cp))
    if nws < 0:
        raise BsaError(f"bsa_cluster_permute_workspace_bytes: {bsa_last_error()}")
    dev = assign.device
    perm = torch.empty((B, H, N), dtype=torch.int32, device=dev)
    offsets = torch.empty((B, H, cells + 1), dtype=torch.int32, device=dev)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)
    st = _lib.bsa_cluster_permute(_ptr(assign), _ptr(counts), ctypes.byref(shp), ctypes.byref(cp),
                                  _ptr(perm), _ptr(offsets), _ptr(ws), ws.numel(),
                                  _stream(stream, dev))
    _check(st, "bsa_cluster_permute")
    return perm, offsets


def bsa_cluster_select(mu_q, mu_k, size_k, *, p: float = 0.9, k_min: int = 1,
                       k_cap: int | None = None, scale: float | None = None, stream=None):
    """Key clusters of every query cluster (HVA Eq. 2-3).  mu_q [B, H, Nq, d],
    mu_k [B, H, Nk, d] float32, size_k [B, H, Nk] int32.  Returns (row_ptr
    int32 [B*H*Nq+1], col_idx int32, nnz int64 device scalar)."""
    B, H, Nq, d = mu_q.shape
    Nk = mu_k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    k_cap = Nk if k_cap is None else k_cap
    nws = _lib.bsa_cluster_select_workspace_bytes(B, H, Nq, Nk)
    if nws < 0:
        raise BsaError("bsa_cluster_select_workspace_bytes: invalid sizes")
    dev = mu_q.device
    rows = B * H * Nq
    cap = rows * min(Nk, max(k_cap, 1))
    row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    nnz = torch.empty(1, dtype=torch.int64, device=dev)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)
    st = _lib.bsa_cluster_select(_ptr(mu_q), _ptr(mu_k), _ptr(size_k), B, H, Nq, Nk, d, scale, p,
                                 k_min, k_cap, _ptr(row_ptr), _ptr(col_idx), cap, _ptr(nnz),
                                 _ptr(ws), ws.numel(), _stream(stream, dev))
    _check(st, "bsa_cluster_select")
    return row_ptr, col_idx, nnz


def bsa_cluster_merge(off_q, off_k, crow_ptr, ccol, sides, *, N: int, tau_q: int = 64,
                      tau_k: int = 64, grain: int = 16, stream=None):
    """Merging of query clusters by tiled cost (HVA Algorithm 1).  off_q
    [B,H,Nq+1], off_k [B,H,Nk+1] int32 cluster offsets; the cluster CSR of
    bsa_cluster_select; sides uint8 [B,H,rounds,Nq] (the bipartition of every
    round).  Returns group_of int32 [B,H,Nq] (each cluster's group named by
    its lowest member)."""
    B, H = off_q.shape[0], off_q.shape[1]
    Nq, Nk = off_q.shape[2] - 1, off_k.shape[2] - 1
    if sides.dtype != torch.uint8 or sides.dim() != 4 or tuple(sides.shape[:2]) != (B, H) \
            or sides.shape[3] != Nq or not sides.is_contiguous():
        raise ValueError("sides must be contiguous uint8 [B, H, rounds, Nq]")
    rounds = sides.shape[2]
    nws = _lib.bsa_cluster_merge_workspace_bytes(B, H, N, Nq, Nk, grain)
    if nws < 0:
        raise BsaError(f"bsa_cluster_merge_workspace_bytes: {bsa_last_error()}")
    dev = off_q.device
    group_of = torch.empty((B, H, Nq), dtype=torch.int32, device=dev)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)
    st = _lib.bsa_cluster_merge(_ptr(off_q), _ptr(off_k), _ptr(crow_ptr), _ptr(ccol), B, H, N, Nq,
                                Nk, _ptr(sides), rounds, tau_q, tau_k, grain, _ptr(group_of),
                                _ptr(ws), ws.numel(), _stream(stream, dev))
    _check(st, "bsa_cluster_merge")
    return group_of


def bsa_cluster_attn_fwd(Q, K, V, perm_q, off_q, perm_k, off_k, crow_ptr, ccol, group_of=None, *,
                         scale: float | None = None, out_dtype=torch.float32, stream=None):
    """Attention over cluster-induced blocks (HVA Eq. 4), each query cluster
    over the union of its group's rows when ``group_of`` [B,H,Nq] is given.
    Returns (O [B,H,N,d] out_dtype, LSE float32 [B,H,N], executed tile pairs
    int64 device scalar)."""
    _same_layout(Q, K, V)
    shp = shape_of(Q)
    Nq, Nk = off_q.shape[2] - 1, off_k.shape[2] - 1
    scale = 1.0 / math.sqrt(shp.d) if scale is None else scale
    odt = _odt(out_dtype)
    nws = _lib.bsa_cluster_attn_workspace_bytes(ctypes.byref(shp), Nq, Nk, odt)
    if nws < 0:
        raise BsaError(f"bsa_cluster_attn_workspace_bytes: {bsa_last_error()}")
    dev = Q.device
    O = _out_like(Q, out_dtype)
    L = torch.empty(Q.shape[:3], dtype=torch.float32, device=dev)
    pairs = torch.empty(1, dtype=torch.int64, device=dev)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)
    st = _lib.bsa_cluster_attn_fwd(_ptr(Q), _ptr(K), _ptr(V), ctypes.byref(shp), scale, Nq, Nk,
                                   _ptr(perm_q), _ptr(off_q), _ptr(perm_k), _ptr(off_k),
                                   _ptr(crow_ptr), _ptr(ccol), _ptr(group_of), _ptr(O), odt, _ptr(L),
                                   _ptr(pairs),
                                   _ptr(ws), ws.numel(), _stream(stream, dev))
    _check(st, "bsa_cluster_attn_fwd")
    return O, L, pairs


def bsa_subset_refine(X, subset, assign, centroids, counts, *, stream=None):
    """HVA intermediate-step update: the subset tokens (int32 [B, H, n_sub])
    reassigned against every centroid, the centroids they left or joined
    moved to their members' means.  assign [B, H, N] int32, centroids
    [B, H, cells, d] float32 and counts [B, H, cells] int32 are updated in
    place and returned."""
    if X.dtype != torch.bfloat16:
        raise ValueError("X must be bfloat16")
    shp = shape_of(X)
    cells = centroids.shape[2]
    for t, dt in ((subset, torch.int32), (assign, torch.int32), (centroids, torch.float32),
                  (counts, torch.int32)):
        if t.dtype != dt or not t.is_contiguous():
            raise ValueError("subset, assign, counts int32 and centroids float32, contiguous")
    n = _lib.bsa_subset_refine_workspace_bytes(ctypes.byref(shp), cells)
    if n < 0:
        raise BsaError(f"bsa_subset_refine_workspace_bytes: {bsa_last_error()}")
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=X.device)
    st = _lib.bsa_subset_refine(_ptr(X), ctypes.byref(shp), cells, _ptr(subset), subset.shape[2],
                                _ptr(assign), _ptr(centroids), _ptr(counts), _ptr(ws), ws.numel(),
                                _stream(stream, X.device))
    _check(st, "bsa_subset_refine")
    return assign, centroids, counts


def bsa_omission_risk(lse_sparse, lse_full, lse_repaired=None, *, out=None, stream=None):
    """Per-head omission risk from the LSE of a sparse pass, of full
    attention and (optionally) of the repaired pass.  Returns float64
    [B, H, 3] on the device: mean omitted share, largest omitted share and
    mean recovered share over the N rows of each head."""
    for t in (lse_sparse, lse_full, lse_repaired):
        if t is not None and (t.dtype != torch.float32 or t.dim() != 3 or not t.is_contiguous()
                              or t.shape != lse_sparse.shape):
            raise ValueError("LSE arrays must be contiguous float32 [B, H, N] of one shape")
    B, H, N = lse_sparse.shape
    shp = _Shape(B, H, N, 0, 0, 0, 0)
    n = _lib.bsa_omission_risk_workspace_bytes(ctypes.byref(shp))
    if n < 0:
        raise BsaError(f"bsa_omission_risk_workspace_bytes: {bsa_last_error()}")
    dev = lse_sparse.device
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
    risk = torch.empty((B, H, 3), dtype=torch.float64, device=dev) if out is None else out
    st = _lib.bsa_omission_risk(_ptr(lse_sparse), _ptr(lse_full), _ptr(lse_repaired),
                                ctypes.byref(shp), _ptr(risk), _ptr(ws), ws.numel(),
                                _stream(stream, dev))
    _check(st, "bsa_omission_risk")
    return risk


def heads_at_risk(mean_omitted, n: int) -> list[int]:
    """Offline calibration (bsa_heads_at_risk): the ``n`` heads with the
    largest mean omitted share (equal values go to the lower head index), in
    ascending order -- the head set handed to the Micro residual."""
    vals = [float(v) for v in mean_omitted]
    H = len(vals)
    arr = (ctypes.c_double * max(H, 1))(*vals)
    mask = (ctypes.c_uint8 * max(H, 1))()
    st = _lib.bsa_heads_at_risk(ctypes.cast(arr, ctypes.c_void_p), H, n,
                                ctypes.cast(mask, ctypes.c_void_p))
    _check(st, "bsa_heads_at_risk")
    return [h for h in range(H) if mask[h]]


def csr_rows(row_ptr: torch.Tensor, col_idx: torch.Tensor, nnz: torch.Tensor):
    """Host copy of a CSR as a list of lists (for inspection and tests)."""
    rp = row_ptr.cpu().tolist()
    n = int(nnz.item())
    ci = col_idx[:n].cpu().tolist()
    return [ci[rp[r]:rp[r + 1]] for r in range(len(rp) - 1)]
