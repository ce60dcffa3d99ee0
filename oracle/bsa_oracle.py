"""Plain fp64 CPU oracle for training-free block-sparse video-DiT attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import or
call anything here.  The HIP library never uses it and shares no code with it.

Everything is float64 numpy on ONE head at a time: ``X`` arrays are ``[N, d]``
for the N valid tokens of one (batch, head) pair, flattened t-major
(token n = (t * H_grid + y) * W_grid + x).  Inputs arrive as bf16 and are
upcast exactly; nothing is blocked, fused or reordered beyond what the
definitions below state.

Sources (pages as titled):
  [HVA]   "HyperVAttention: Efficient Sparse Attention with Spatio-Temporal
          Clustering for Video Diffusion", section 2 (Preliminaries), Eq. 2-4,
          section 4.1 (3D local-window clustering, Eq. 5), section 4.2
          (Lowe's ratio, Eq. 6), section 4.3
          (hardware cost, Eq. 7-10, Algorithm 1), Appendix A.1 (Top-p,
          Min-kc, R = 3 rounds) and A.2 (Algorithm 2).
  [RSA]   "Rectified SpaAttn: Revisiting Attention Sparsity for Efficient Video
          Generation", abstract: pooled query-key interactions.
  [HyMoR] "HyMoR-Attn: Granularity-Matched Repair of Omitted Attention Support
          for Video Diffusion", abstract: Macro backbone, Micro residual over
          omitted blocks, exact LSE merging.
  [LVSA]  "Long Video Sparse Attention" abstract (page titled "FreqFormer ..."):
          structured window pattern plus rotating global anchors.
  [MOD]   "Mixture of Distributions Matters: Dynamic Sparse Attention for
          Efficient Video Diffusion Transformers", Pattern Mixtures (the
          parallel-diagonal, vertical and block-diagonal bases), Metrics
          (density = computed B x B blocks / total) and Block-wise Attention
          Computation (block size 128).

Readings where the pages are silent:
  * the ragged tail block holds only valid tokens; pooling averages over them
    and attention never sees a padded key;
  * top-k keeps ``k`` blocks ordered by (score descending, index ascending);
  * top-p is inclusive ("at least p"), then clamped to [k_min, k_cap];
  * forced blocks (diagonal, static window/anchors) are a union added after
    top-k/top-p and are not counted in the budget;
  * the micro rule is the 16-token pooled score restricted to omitted blocks,
    top-m per 64-row query block (parity unpinned against the pages: HyMoR
    gives no formula; it is pinned only against its own definition);
  * LSE is the natural log of the softmax normaliser with the scale inside;
    an empty support yields LSE = -inf and O = 0;
  * [MOD]'s parallel-diagonal offsets delta_k = k - n + 1 are read with
    k = 0 .. 2n-2, i.e. all 2n-1 diagonals -(n-1) .. n-1 of the n x n block
    map (the page's 1-based k would start at 2-n and end off the map);
  * a 128-token block selection is executed on 64-token tiles: every kept
    128 x 128 pair is its 2 x 2 tiles, the token support unchanged;
  * the omission risk of a query token is the share of its full softmax mass
    outside its sparse support (HyMoR names the risk, not its formula);
  * [HVA] local-window clustering: argmin ties go to the lower centroid
    index; the last iteration's assignment and the final centroids are
    returned;
  * RSA's pooled rectification is read as attention over the pooled keys of
    the omitted blocks (log-size bias), LSE-merged with the sparse result;
    its gain-aware gate keeps block j for query q when the estimate's
    pooling error under a normal isotropic key spread stays below its gain,
    scale^2 |q|^2 v_j < 2 ln 2 (v_j the block's per-coordinate key
    variance);
  * [HVA] Eq. 6 (Lowe's ratio) is taken over each token's local window,
    the candidates of its assignment, against the centroids given;
  * [HVA] section 4.2's intermediate-step update: the subset tokens are
    reassigned against every centroid, then the centroids any of them left
    or joined become the means of their members (current embeddings); the
    others keep their anchor-step positions;
  * [HVA] Algorithm 1: the random bipartition is an input (a side bit per
    round for every group, read at the group's lowest member); side-0 groups
    choose, ties go to lower indices; a merged group is named by its lowest
    member.
"""

from __future__ import annotations

import math

import numpy as np

NEG_INF = -math.inf


# ----------------------------------------------------------------------------
# Blocks and pooling
# ----------------------------------------------------------------------------

def n_blocks(N: int, b: int) -> int:
    """Number of b-token blocks covering N tokens (the last one may be ragged)."""
    return -(-N // b)


def block_tokens(N: int, b: int, j: int) -> np.ndarray:
    """Indices of the valid tokens of block j: {b*j, ..., min(b*j+b, N) - 1}."""
    return np.arange(b * j, min(b * j + b, N))


def block_sizes(N: int, b: int) -> np.ndarray:
    """Valid token count of every block (the cluster sizes s_j of [HVA] Eq. 2)."""
    return np.array([len(block_tokens(N, b, j)) for j in range(n_blocks(N, b))],
                    dtype=np.float64)


def pool_means(X: np.ndarray, b: int) -> np.ndarray:
    """Per-block mean of the token vectors.

    [RSA] pools queries and keys over blocks; [HVA] section 2 defines a
    centroid as the mean of its members.  Only valid tokens count.
    """
    X = np.asarray(X, dtype=np.float64)
    N = X.shape[0]
    return np.stack([X[block_tokens(N, b, j)].mean(axis=0)
                     for j in range(n_blocks(N, b))])


def pooled_scores(Qbar: np.ndarray, Kbar: np.ndarray, scale: float) -> np.ndarray:
    """Centroid-level logits S_ij = <mu_i^q, mu_j^k> * scale ([HVA] Eq. 2, left)."""
    return scale * (np.asarray(Qbar, np.float64) @ np.asarray(Kbar, np.float64).T)


# ----------------------------------------------------------------------------
# Selection
# ----------------------------------------------------------------------------

def rank_desc(values: np.ndarray) -> np.ndarray:
    """Indices ordered by value descending, ties by index ascending."""
    values = np.asarray(values, dtype=np.float64)
    idx = np.arange(values.shape[0])
    return np.lexsort((idx, -values))


def topk_set(score_row: np.ndarray, k: int) -> set[int]:
    """The k key blocks with the highest pooled score (density budget of
    [MOD] / Top-K selection); ties go to the lower block index."""
    order = rank_desc(score_row)
    return set(int(j) for j in order[:max(0, k)])


def size_weighted_softmax(score_row: np.ndarray, sizes: np.ndarray) -> np.ndarray:
    """P'_ij = s_j exp(S_ij) / sum_o s_o exp(S_io)  ([HVA] Eq. 2, right)."""
    s = np.asarray(score_row, dtype=np.float64)
    w = np.asarray(sizes, dtype=np.float64) * np.exp(s - s.max())
    return w / w.sum()


def topp_length(P: np.ndarray, p: float) -> int:
    """Size of TopP(P; p): the smallest prefix, in descending order of P, whose
    cumulative probability is at least p ([HVA] Eq. 3)."""
    order = rank_desc(P)
    c = np.cumsum(P[order])
    hit = np.nonzero(c >= p)[0]
    return int(hit[0]) + 1 if hit.size else int(P.shape[0])


def topp_set(score_row: np.ndarray, sizes: np.ndarray, p: float,
             k_min: int = 1, k_cap: int | None = None) -> set[int]:
    """Top-p over the size-weighted centroid softmax, clamped to
    [k_min, k_cap] blocks ([HVA] Eq. 2-3; Min-kc of Appendix A.1 as a floor,
    the density cap as a ceiling)."""
    P = size_weighted_softmax(score_row, sizes)
    n = P.shape[0]
    L = topp_length(P, p)
    L = max(L, k_min)
    if k_cap is not None:
        L = min(L, k_cap)
    L = min(L, n)
    order = rank_desc(P)
    return set(int(j) for j in order[:L])


def block_frame_span(N: int, b: int, frame_tokens: int, j: int) -> tuple[int, int]:
    """Lowest and highest latent frame index touched by block j (t-major
    layout: token n lies in frame n // frame_tokens)."""
    toks = block_tokens(N, b, j)
    return int(toks[0]) // frame_tokens, int(toks[-1]) // frame_tokens


def window_anchor_set(N: int, b: int, i: int, frame_tokens: int,
                      window_frames: int, n_anchors: int,
                      anchor_offset: int) -> set[int]:
    """Static block mask of [LVSA]: a temporal window plus rotating global
    anchors.

    Window: key block j is kept for query block i when some token of j lies
    within ``window_frames`` latent frames of some token of i.
    Anchors: ``n_anchors`` key blocks evenly strided over the sequence,
    rotated by ``anchor_offset`` (the rotation the caller draws per call).
    """
    nB = n_blocks(N, b)
    lo_i, hi_i = block_frame_span(N, b, frame_tokens, i)
    out = set()
    for j in range(nB):
        lo_j, hi_j = block_frame_span(N, b, frame_tokens, j)
        if lo_j <= hi_i + window_frames and hi_j >= lo_i - window_frames:
            out.add(j)
    if n_anchors > 0:
        stride = nB // n_anchors
        for a in range(n_anchors):
            out.add((anchor_offset + a * stride) % nB)
    return out


def pattern_set(nB: int, i: int, diagonals=(), columns=()) -> set[int]:
    """Key blocks of query block i under a chosen set of [MOD] structural
    patterns (Pattern Mixtures): a parallel-diagonal pattern of offset delta
    marks block (i, i + delta) of the n x n block map (inter-frame temporal
    continuity); a vertical pattern marks one key column j for every query
    block (global anchors / sinks).  The mask of several patterns is their
    union; offsets that fall off the map mark nothing."""
    out = set()
    for delta in diagonals:
        j = i + int(delta)
        if 0 <= j < nB:
            out.add(j)
    for j in columns:
        if not 0 <= int(j) < nB:
            raise ValueError(f"column {j} outside [0, {nB})")
        out.add(int(j))
    return out


def expand_rows(rows: list[list[int]], N: int, b_from: int, b_to: int) -> list[list[int]]:
    """Rows over b_from-token blocks re-expressed over b_to-token blocks
    (b_from a multiple of b_to): query block i' takes the row of its
    enclosing block i' // r (r = b_from / b_to) and every key block J becomes
    the valid blocks r J .. r J + r - 1.  The token support of every query is
    unchanged."""
    r = b_from // b_to
    assert r * b_to == b_from
    n_to = n_blocks(N, b_to)
    out = []
    for i2 in range(n_to):
        src = rows[i2 // r]
        out.append(sorted(r * J + e for J in src for e in range(r) if r * J + e < n_to))
    return out


def select_rows(scores: np.ndarray | None, N: int, b: int, mode: str, *,
                k: int = 0, p: float = 0.9, k_min: int = 1,
                k_cap: int | None = None, force_diag: bool = False,
                static: dict | None = None,
                patterns: dict | None = None) -> list[list[int]]:
    """Per query block, the ascending list of selected key blocks for one head.

    ``mode`` is "topk", "topp" or "static".  The forced set (the diagonal,
    the [LVSA] window+anchors ``static`` mask and the [MOD] ``patterns``
    {"diagonals": offsets, "columns": key blocks}) is a union on top of the
    scored selection.  ``b`` is the block of the selection (64 or 128 in the
    library; the [MOD] block-wise attention uses 128).
    """
    nB = n_blocks(N, b)
    sizes = block_sizes(N, b)
    rows = []
    for i in range(nB):
        if mode == "topk":
            sel = topk_set(scores[i], k)
        elif mode == "topp":
            sel = topp_set(scores[i], sizes, p, k_min, k_cap)
        elif mode == "static":
            sel = set()
        else:
            raise ValueError(mode)
        if force_diag:
            sel.add(i)
        if static is not None:
            sel |= window_anchor_set(N, b, i, **static)
        if patterns is not None:
            sel |= pattern_set(nB, i, patterns.get("diagonals", ()),
                               patterns.get("columns", ()))
        rows.append(sorted(sel))
    return rows


def density(rows_per_head: list[list[list[int]]], nB: int) -> float:
    """Computed B x B blocks over all blocks ([MOD] Metrics)."""
    tot = sum(len(r) for rows in rows_per_head for r in rows)
    return tot / (len(rows_per_head) * nB * nB)


# ----------------------------------------------------------------------------
# Attention over a support
# ----------------------------------------------------------------------------

def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Scaled dot-product attention of queries q [m,d] over keys K,V [n,d].

    Returns (O [m,d], LSE [m]) with LSE_t = ln sum_tau exp(scale q_t . k_tau).
    An empty key set gives O = 0 and LSE = -inf.
    """
    q = np.asarray(q, np.float64)
    m, d = q.shape
    if K.shape[0] == 0:
        return np.zeros((m, V.shape[1])), np.full(m, NEG_INF)
    z = scale * (q @ np.asarray(K, np.float64).T)
    mx = z.max(axis=1, keepdims=True)
    e = np.exp(z - mx)
    s = e.sum(axis=1)
    lse = mx[:, 0] + np.log(s)
    O = (e @ np.asarray(V, np.float64)) / s[:, None]
    return O, lse


def block_sparse_attention(Q, K, V, rows: list[list[int]], b: int, scale: float):
    """O_i = Attn(Q_i, {K_j, V_j}_{j in A_i}) for every query block i
    ([HVA] Eq. 4 with the identity permutation; the [HyMoR] Macro backbone).

    Restricting each query block to the tokens of its selected key blocks is
    the same as dense softmax(scale Q K^T + M) V with M in {0, -inf}.
    """
    Q = np.asarray(Q, np.float64)
    N, d = Q.shape
    O = np.zeros((N, V.shape[1]))
    L = np.full(N, NEG_INF)
    for i, sel in enumerate(rows):
        qi = block_tokens(N, b, i)
        keys = (np.concatenate([block_tokens(N, b, j) for j in sel])
                if len(sel) else np.zeros(0, dtype=np.int64))
        O[qi], L[qi] = attend(Q[qi], K[keys], V[keys], scale)
    return O, L


def dense_attention(Q, K, V, scale: float):
    """Full attention over all N keys (the dense baseline)."""
    return attend(Q, K, V, scale)


# ----------------------------------------------------------------------------
# Micro residual ([HyMoR]) and the exact LSE merge
# ----------------------------------------------------------------------------

def micro_candidates(Qt: np.ndarray, Kt: np.ndarray, macro_row: list[int], i: int,
                     N: int, b: int, u: int, scale: float):
    """All micro candidates of query block i: pairs (a, beta) where a indexes
    the u-token query sub-tiles of block i and beta a u-token key tile whose
    enclosing b-block was omitted by the macro selection.  Score
    sigma = scale <Qt_{(b/u) i + a}, Kt_beta> on u-token pooled means.

    Returns a list of (sigma, code) with code = (b/u) * beta + a.
    """
    r = b // u
    nT = n_blocks(N, u)
    omitted = np.ones(n_blocks(N, b), dtype=bool)
    omitted[list(macro_row)] = False
    out = []
    for a in range(r):
        qa = r * i + a
        if qa >= nT:
            continue
        for beta in range(nT):
            if not omitted[beta // r]:
                continue
            sigma = scale * float(Qt[qa] @ Kt[beta])
            out.append((sigma, r * beta + a))
    return out


def micro_select_row(Qt, Kt, macro_row, i, N, b, u, scale, m):
    """Online peak-preserving Micro selection for one query block: the top-m
    candidates by (sigma descending, code ascending), returned as codes sorted
    by (sub-tile a, key tile beta)."""
    cand = micro_candidates(Qt, Kt, macro_row, i, N, b, u, scale)
    cand.sort(key=lambda t: (-t[0], t[1]))
    r = b // u
    kept = [c for _, c in cand[:max(0, m)]]
    kept.sort(key=lambda c: (c % r, c // r))
    return kept


def micro_select_rows(Qt, Kt, macro_rows: list[list[int]], N: int, b: int, u: int,
                      scale: float, m: int) -> list[list[int]]:
    """``micro_select_row`` for every query block of a head at once: the
    scores of all (query sub-tile, key tile) pairs are one matrix product
    sigma = scale Qt Kt^T, then each block keeps its top-m candidates by
    (sigma descending, code ascending), emitted in (a, beta) order."""
    r = b // u
    nT = n_blocks(N, u)
    nB = n_blocks(N, b)
    sig = scale * (np.asarray(Qt, np.float64) @ np.asarray(Kt, np.float64).T)
    beta = np.arange(nT)
    out = []
    for i in range(nB):
        omitted = np.ones(nB, dtype=bool)
        omitted[list(macro_rows[i])] = False
        bs = beta[omitted[beta // r]]
        sg, cd = [], []
        for a in range(r):
            qa = r * i + a
            if qa < nT:
                sg.append(sig[qa, bs])
                cd.append(r * bs + a)
        if not sg or m <= 0:
            out.append([])
            continue
        sg, cd = np.concatenate(sg), np.concatenate(cd)
        kept = cd[np.lexsort((cd, -sg))[:m]]
        out.append(sorted(kept.tolist(), key=lambda c: (c % r, c // r)))
    return out


def micro_attention(Q, K, V, micro_rows: list[list[int]], b: int, u: int,
                    scale: float):
    """Micro residual: each u-row query sub-tile attends over the union of its
    selected u-key tiles.  Sub-tiles with no tile get O = 0, LSE = -inf."""
    Q = np.asarray(Q, np.float64)
    N, d = Q.shape
    r = b // u
    O = np.zeros((N, V.shape[1]))
    L = np.full(N, NEG_INF)
    for i, codes in enumerate(micro_rows):
        for a in range(r):
            qa = r * i + a
            if qa * u >= N:
                continue
            qi = block_tokens(N, u, qa)
            tiles = [c // r for c in codes if c % r == a]
            keys = (np.concatenate([block_tokens(N, u, t) for t in tiles])
                    if tiles else np.zeros(0, dtype=np.int64))
            O[qi], L[qi] = attend(Q[qi], K[keys], V[keys], scale)
    return O, L


def lse_merge(O1, L1, O2, L2):
    """Exact merge of two partial softmax results over disjoint supports
    ([HyMoR] exact LSE merging):
        L = ln(e^L1 + e^L2),  O = e^(L1 - L) O1 + e^(L2 - L) O2.
    Both empty (L1 = L2 = -inf) gives O = 0, L = -inf."""
    O1 = np.asarray(O1, np.float64)
    O2 = np.asarray(O2, np.float64)
    L1 = np.asarray(L1, np.float64)
    L2 = np.asarray(L2, np.float64)
    L = np.logaddexp(L1, L2)
    both_empty = np.isneginf(L)
    Ls = np.where(both_empty, 0.0, L)
    w1 = np.where(np.isneginf(L1), 0.0, np.exp(L1 - Ls))
    w2 = np.where(np.isneginf(L2), 0.0, np.exp(L2 - Ls))
    O = w1[:, None] * O1 + w2[:, None] * O2
    O[both_empty] = 0.0
    return O, L


# ----------------------------------------------------------------------------
# Pooled rectification of omitted blocks ([RSA] reading)
#
# [RSA] rectifies sparse attention with pooled query-key interactions: the
# kept (critical) blocks are over-weighted and the omitted (non-critical)
# ones lose their weight entirely.  It gives no formulas.  Reading used
# here: every omitted key block j contributes its pooled estimate -- the
# block's softmax normaliser n_j exp(scale q . Kbar_j) and its value sum
# n_j exp(scale q . Kbar_j) Vbar_j (exact when the block's keys are all
# equal) -- and the estimate is combined with the sparse result by the
# exact LSE merge, which also lowers the kept blocks' weights to their share
# of the larger normaliser.
#
# Gain-Aware Pooling Rectification ([RSA] abstract: the recovered gain must
# exceed the pooling error it brings in) -- reading: for query q and omitted
# block j the gain is the recovered mass w_hat = n_j exp(scale q . Kbar_j).
# The block's true mass is w = w_hat * mean_tau exp(x_tau) with
# x_tau = scale q . (k_tau - Kbar_j), a zero-mean spread; when the keys
# scatter normally and isotropically about their mean with per-coordinate
# variance v_j, x is normal with variance sigma^2 = scale^2 |q|^2 v_j and
# mean_tau exp(x_tau) = exp(sigma^2 / 2), so the pooling error of the
# estimate is w - w_hat = w_hat (exp(sigma^2 / 2) - 1).  The block is
# rectified when gain > error, i.e. exp(sigma^2 / 2) < 2, i.e.
#     scale^2 |q|^2 v_j < 2 ln 2,
# with v_j = sum_tau |k_tau - Kbar_j|^2 / (n_j d) measured over the block's
# valid keys.  The gate is per (query, block); the threshold has no free
# parameter.
# ----------------------------------------------------------------------------

GATE_SIGMA2 = 2.0 * math.log(2.0)


def block_key_spread(K, b: int) -> np.ndarray:
    """v_j: mean squared deviation of block j's valid keys from their mean,
    per coordinate, (1 / (n_j d)) sum_tau |k_tau - Kbar_j|^2."""
    K = np.asarray(K, np.float64)
    N, d = K.shape
    Kb = pool_means(K, b)
    return np.array([((K[block_tokens(N, b, j)] - Kb[j]) ** 2).sum() / (len(block_tokens(N, b, j)) * d)
                     for j in range(n_blocks(N, b))])


def rectify_gate(Q, K, b: int, scale: float) -> np.ndarray:
    """[N, nB] booleans: True where query t's pooled estimate of block j
    passes the gain-aware test scale^2 |q_t|^2 v_j < 2 ln 2."""
    Q = np.asarray(Q, np.float64)
    qn2 = (Q * Q).sum(axis=1)
    v = block_key_spread(K, b)
    return (scale * scale) * qn2[:, None] * v[None, :] < GATE_SIGMA2


def pooled_omitted_attention(Q, K, V, rows: list[list[int]], b: int, scale: float,
                             gate: bool = False):
    """For every valid query token t of block i, attention over the pooled
    keys of the blocks NOT in row i, each with log-size bias ln n_j:
        z_j = scale q_t . Kbar_j + ln n_j,
        LSE_t = ln sum_j e^{z_j},  O_t = sum_j e^{z_j - LSE_t} Vbar_j.
    With ``gate``, block j counts for token t only where ``rectify_gate``
    passes.  A token with no block left gets O = 0, LSE = -inf."""
    Q = np.asarray(Q, np.float64)
    N = Q.shape[0]
    nB = n_blocks(N, b)
    Kb, Vb = pool_means(K, b), pool_means(V, b)
    logn = np.log(block_sizes(N, b))
    G = rectify_gate(Q, K, b, scale) if gate else np.ones((N, nB), dtype=bool)
    O = np.zeros((N, Vb.shape[1]))
    L = np.full(N, NEG_INF)
    for i, sel in enumerate(rows):
        om = np.ones(nB, dtype=bool)
        om[list(sel)] = False
        qi = block_tokens(N, b, i)
        use = om[None, :] & G[qi]
        live = use.any(axis=1)
        if not live.any():
            continue
        z = np.where(use, scale * (Q[qi] @ Kb.T) + logn[None, :], NEG_INF)[live]
        mx = z.max(axis=1, keepdims=True)
        e = np.exp(z - mx)
        ssum = e.sum(axis=1)
        L[qi[live]] = mx[:, 0] + np.log(ssum)
        O[qi[live]] = (e @ Vb) / ssum[:, None]
    return O, L


def pooled_rectified_attention(Q, K, V, rows: list[list[int]], b: int, scale: float,
                               gate: bool = False):
    """Sparse attention over the kept blocks, rectified by the pooled
    estimate of the omitted ones (those passing the gain-aware test with
    ``gate``) through the exact LSE merge."""
    Os, Ls = block_sparse_attention(Q, K, V, rows, b, scale)
    Op, Lp = pooled_omitted_attention(Q, K, V, rows, b, scale, gate=gate)
    return lse_merge(Os, Ls, Op, Lp)


# ----------------------------------------------------------------------------
# Omission risk ([HyMoR] offline risk calibration of layers and heads)
#
# Reading: the page states that the risk of omitting valuable support is
# stable per layer and head and is calibrated offline, but gives no formula.
# The risk of a query token here is the share of its full softmax mass that
# falls on keys outside its sparse support; a repair (the Micro residual)
# brings back the mass of the keys it adds.  A head's risk is the mean over
# its valid tokens.
# ----------------------------------------------------------------------------

def softmax_mass_outside(q: np.ndarray, K: np.ndarray, keys: np.ndarray,
                         scale: float) -> np.ndarray:
    """For queries q [m,d] attending over ALL keys K [N,d], the softmax mass
    on the keys NOT in the index set ``keys``:
        w_t = sum_{tau not in keys} exp(z_t,tau) / sum_tau exp(z_t,tau),
    z = scale q K^T (the full-attention distribution of each query)."""
    z = scale * (np.asarray(q, np.float64) @ np.asarray(K, np.float64).T)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    outside = np.ones(K.shape[0], dtype=bool)
    outside[np.asarray(keys, dtype=np.int64)] = False
    return p[:, outside].sum(axis=1)


def omitted_mass(Q, K, rows: list[list[int]], b: int, scale: float) -> np.ndarray:
    """Per valid query token t of block i: the full-attention softmax mass of
    t outside the tokens of the key blocks in row i (1 for an empty row)."""
    Q = np.asarray(Q, np.float64)
    N = Q.shape[0]
    w = np.zeros(N)
    for i, sel in enumerate(rows):
        qi = block_tokens(N, b, i)
        keys = (np.concatenate([block_tokens(N, b, j) for j in sel])
                if len(sel) else np.zeros(0, dtype=np.int64))
        w[qi] = softmax_mass_outside(Q[qi], K, keys, scale)
    return w


def micro_mass(Q, K, micro_rows: list[list[int]], b: int, u: int,
               scale: float) -> np.ndarray:
    """Per valid query token t of sub-tile a of block i: the full-attention
    softmax mass of t on the union of the u-key tiles of its micro entries
    (a, beta) -- the mass the Micro residual adds to the Macro support."""
    Q = np.asarray(Q, np.float64)
    N = Q.shape[0]
    r = b // u
    g = np.zeros(N)
    for i, codes in enumerate(micro_rows):
        for a in range(r):
            qa = r * i + a
            if qa * u >= N:
                continue
            qi = block_tokens(N, u, qa)
            tiles = [c // r for c in codes if c % r == a]
            if not tiles:
                continue
            keys = np.concatenate([block_tokens(N, u, t) for t in tiles])
            g[qi] = 1.0 - softmax_mass_outside(Q[qi], K, keys, scale)
    return g


def risk_from_lse(L_sparse, L_full, L_repaired=None):
    """Per-row omitted and recovered mass from log-sum-exps alone.  Since
    e^L is the softmax normaliser over a support, the omitted share of a row
    is 1 - e^(L_sparse - L_full) and the share a disjoint repair adds is
    e^(L_repaired - L_full) - e^(L_sparse - L_full).  Rows whose full LSE is
    -inf (no keys at all) count as 0 for both.  Returns (w, g); g is zeros
    when no repaired LSE is given."""
    Ls = np.asarray(L_sparse, np.float64)
    Lf = np.asarray(L_full, np.float64)
    empty = np.isneginf(Lf)
    Lf_safe = np.where(empty, 0.0, Lf)
    kept = np.where(np.isneginf(Ls), 0.0, np.exp(Ls - Lf_safe))
    w = np.where(empty, 0.0, 1.0 - kept)
    if L_repaired is None:
        return w, np.zeros_like(w)
    Lr = np.asarray(L_repaired, np.float64)
    rep = np.where(np.isneginf(Lr), 0.0, np.exp(Lr - Lf_safe))
    g = np.where(empty, 0.0, rep - kept)
    return w, g


def head_risk(w: np.ndarray, g: np.ndarray) -> tuple[float, float, float]:
    """(mean omitted mass, largest omitted mass, mean recovered mass) over the
    valid tokens of one head."""
    w = np.asarray(w, np.float64)
    g = np.asarray(g, np.float64)
    if w.size == 0:
        return 0.0, 0.0, 0.0
    return float(w.mean()), float(w.max()), float(g.mean())


def heads_at_risk(mean_omitted: np.ndarray, n: int) -> list[int]:
    """The n heads of largest mean omitted mass (ties to the lower index),
    ascending: the heads an offline calibration hands the Micro residual."""
    order = sorted(range(len(mean_omitted)), key=lambda h: (-float(mean_omitted[h]), h))
    return sorted(order[:max(0, n)])


# ----------------------------------------------------------------------------
# 3D local-window clustering ([HVA] section 4.1, Eq. 5, Appendix A.2 Alg. 2)
#
# Tokens are a T x H x W lattice (t-major).  A fixed grid of cells of size
# (kt, kh, kw) gives one centroid per cell, initialised at the cell's centre
# token (clamped to the lattice).  Each iteration assigns every token to the
# nearest centroid among the cells of a (wt, wh, ww) window around its own
# cell (the window clipped to the grid), then moves every centroid to the
# mean of its tokens (a centroid with none keeps its position).  Readings:
# ties go to the lower centroid index (cells numbered t-major); the returned
# assignment is that of the last iteration, the centroids those after the
# last update.
# ----------------------------------------------------------------------------

def cluster_grid(thw, cell, window):
    """Cells per axis K = ceil(dim / k) and the window clipped to the grid."""
    K = tuple(-(-thw[a] // cell[a]) for a in range(3))
    w = tuple(min(window[a], K[a]) for a in range(3))
    return K, w


def window_start(g: int, w: int, K: int) -> int:
    """First cell of the window around cell g on one axis: g - floor(w/2),
    clipped to [0, K - w]."""
    return min(max(g - w // 2, 0), K - w)


def window_candidates(thw, cell, window) -> np.ndarray:
    """[HVA] Eq. 5's candidate set N(g(l)) for every token l: the centroids
    of the (wt, wh, ww) window of cells around the token's own cell g(l),
    the window clipped to the grid.  Returns [N, wt*wh*ww] centroid ids in
    ascending order (cells numbered t-major)."""
    T, H, W = thw
    K, w = cluster_grid(thw, cell, window)
    t, h, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    g = [ax.reshape(-1) // cell[a] for a, ax in enumerate((t, h, x))]   # token's cell per axis
    st = [np.array([window_start(int(v), w[a], K[a]) for v in range(K[a])])[g[a]]
          for a in range(3)]                                           # window start per axis
    ot, oh, ow = np.meshgrid(np.arange(w[0]), np.arange(w[1]), np.arange(w[2]), indexing="ij")
    ct = st[0][:, None] + ot.reshape(-1)[None, :]
    ch = st[1][:, None] + oh.reshape(-1)[None, :]
    cw = st[2][:, None] + ow.reshape(-1)[None, :]
    return (ct * K[1] + ch) * K[2] + cw


def nearest_centroid(X, mu, cand) -> np.ndarray:
    """[HVA] Eq. 5: every token's nearest centroid (squared Euclidean
    distance) among its candidates; equal distances go to the lower
    centroid index (candidates are listed ascending, the first minimum
    wins)."""
    best_d = np.full(X.shape[0], np.inf)
    best = np.zeros(X.shape[0], dtype=np.int64)
    for s in range(cand.shape[1]):
        c = cand[:, s]
        dist = ((X - mu[c]) ** 2).sum(axis=1)
        better = dist < best_d
        best_d = np.where(better, dist, best_d)
        best = np.where(better, c, best)
    return best


def member_means(X, a, mu):
    """[HVA] section 4.1: every centroid moves to the mean of the tokens
    assigned to it; a centroid with no token keeps its position.  Returns
    (centroids, counts)."""
    n = mu.shape[0]
    counts = np.bincount(a, minlength=n)
    sums = np.zeros_like(mu)
    np.add.at(sums, a, X)
    out = mu.copy()
    moved = counts > 0
    out[moved] = sums[moved] / counts[moved, None]
    return out, counts


def local_window_clustering(X, thw, cell, window, iters: int):
    """[HVA] section 4.1 (Eq. 5) and Appendix A.2: 3D local-window
    clustering.  A fixed grid of (kt, kh, kw) cells gives one centroid per
    cell, started at the cell's centre token (clamped to the lattice); each
    iteration assigns every token to its nearest centroid within the window
    of cells around its own cell (``nearest_centroid`` over
    ``window_candidates``), then moves the centroids to their members' means.
    Returns (assignment [N] int, centroids [Nc, d], counts [Nc]) after the
    last iteration."""
    X = np.asarray(X, np.float64)
    T, H, W = thw
    N, d = X.shape
    assert N == T * H * W and iters >= 1
    K, _ = cluster_grid(thw, cell, window)
    centre = [np.minimum(np.arange(K[a]) * cell[a] + cell[a] // 2, thw[a] - 1) for a in range(3)]
    ut, uh, uw = np.meshgrid(*centre, indexing="ij")
    mu = X[((ut * H + uh) * W + uw).reshape(-1)].copy()
    cand = window_candidates(thw, cell, window)
    for _ in range(iters):
        a = nearest_centroid(X, mu, cand)
        mu, counts = member_means(X, a, mu)
    return a, mu, counts


def cluster_permutation(assign, n_clusters: int):
    """[HVA] Eq. 1: the permutation that places the tokens of each cluster
    contiguously -- tokens ordered by (cluster, original index), a stable
    sort -- and the start offset of every cluster (n_clusters + 1 entries)."""
    a = np.asarray(assign, dtype=np.int64)
    perm = np.argsort(a, kind="stable")
    offsets = np.zeros(n_clusters + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(np.bincount(a, minlength=n_clusters))
    return perm, offsets


def cluster_topp_rows(mu_q, mu_k, sizes_k, scale: float, p: float, k_min: int = 1,
                      k_cap: int | None = None) -> list[list[int]]:
    """[HVA] Eq. 2-3 on clusters: for every query cluster i, the key clusters
    of TopP(P'_i; p), P'_ij = s_j exp(S_ij) / sum_o s_o exp(S_io) with
    S_ij = scale <mu_i^q, mu_j^k> and s_j the key cluster sizes, clamped to
    [k_min, k_cap] (Min-kc of Appendix A.1 as the floor), ascending."""
    S = pooled_scores(mu_q, mu_k, scale)
    sizes = np.asarray(sizes_k, np.float64)
    return [sorted(topp_set(S[i], sizes, p, k_min, k_cap)) for i in range(S.shape[0])]


def cluster_block_attention(Q, K, V, perm_q, off_q, perm_k, off_k, rows, scale: float):
    """[HVA] Eq. 4: every query of query cluster i attends over the tokens of
    the key clusters in row i (clusters as produced by cluster_permutation;
    the result is written back in the original token order, O = Pi_q^-1 O').
    Queries of a cluster with an empty row get O = 0, LSE = -inf."""
    Q = np.asarray(Q, np.float64)
    N = Q.shape[0]
    O = np.zeros((N, np.asarray(V).shape[1]))
    L = np.full(N, NEG_INF)
    for i, sel in enumerate(rows):
        qi = np.asarray(perm_q[off_q[i]:off_q[i + 1]], dtype=np.int64)
        if qi.size == 0:
            continue
        keys = (np.concatenate([perm_k[off_k[j]:off_k[j + 1]] for j in sel]).astype(np.int64)
                if len(sel) else np.zeros(0, dtype=np.int64))
        O[qi], L[qi] = attend(Q[qi], K[keys], V[keys], scale)
    return O, L


def cluster_tile_pairs(off_q, off_k, rows, tile: int = 64) -> int:
    """Work of executing Eq. 4 on tiles with every cluster padded to whole
    tiles: sum over query clusters of ceil(s_i / tile) times the tiles of its
    selected key clusters, sum of ceil(s_j / tile)."""
    sq = np.diff(np.asarray(off_q))
    sk = np.diff(np.asarray(off_k))
    tq = -(-sq // tile)
    tk = -(-sk // tile)
    return int(sum(int(tq[i]) * int(sum(int(tk[j]) for j in sel)) for i, sel in enumerate(rows)))


def lowe_ratios(X, thw, cell, window, mu) -> np.ndarray:
    """[HVA] Eq. 6: rho = d_1 / d_2 per token, d_1 its Euclidean distance to
    the nearest centroid and d_2 to the nearest other one, both over the
    centroids of its local window (the candidates its assignment uses).
    A token with one candidate has rho = 0; d_1 = d_2 = 0 gives rho = 1."""
    X = np.asarray(X, np.float64)
    mu = np.asarray(mu, np.float64)
    T, H, W = thw
    K, w = cluster_grid(thw, cell, window)
    Kt, Kh, Kw = K
    rho = np.zeros(X.shape[0])
    for t in range(T):
        for h in range(H):
            for x in range(W):
                g = (t // cell[0], h // cell[1], x // cell[2])
                st = [window_start(g[i], w[i], K[i]) for i in range(3)]
                cand = [(vt * Kh + vh) * Kw + vw for vt in range(st[0], st[0] + w[0])
                        for vh in range(st[1], st[1] + w[1]) for vw in range(st[2], st[2] + w[2])]
                n = (t * H + h) * W + x
                dist = np.sort(np.sqrt(((X[n] - mu[cand]) ** 2).sum(axis=1)))
                if len(dist) < 2:
                    rho[n] = 0.0
                elif dist[1] == 0.0:
                    rho[n] = 1.0
                else:
                    rho[n] = dist[0] / dist[1]
    return rho


def lowe_subset(rho, n: int) -> np.ndarray:
    """[HVA] section 4.2: the n tokens with the largest Lowe's ratio (the
    most ambiguous assignments; equal ratios go to the lower index), in
    ascending token order."""
    return np.sort(rank_desc(np.asarray(rho, np.float64))[:max(0, n)])


def subset_refinement(X, assign, mu, subset):
    """[HVA] section 4.2, the intermediate-step update of the hybrid
    clustering: only the cached subset of tokens (the largest Lowe's
    ratios of the anchor step) is revisited.  Each subset token is reassigned
    by a standard k-means step against the whole current centroid set (its
    squared Euclidean distance to every centroid; equal distances to the
    lower index), not only its local window.  Then the corresponding
    centroids -- every centroid a subset token left or joined -- move to the
    mean of their members under the new assignment, with the current token
    embeddings X; a centroid left without members keeps its position, every
    other centroid is untouched.  Returns (assignment [N], centroids [Nc, d],
    members per centroid [Nc]).  ``subset`` holds distinct token indices."""
    X = np.asarray(X, np.float64)
    a = np.asarray(assign, dtype=np.int64).copy()
    mu = np.asarray(mu, np.float64).copy()
    S = np.asarray(subset, dtype=np.int64)
    old = a[S]
    new = np.array([int(np.argmin(((mu - X[t]) ** 2).sum(axis=1))) for t in S], dtype=np.int64)
    a[S] = new
    moved = new != old
    touched = np.union1d(old[moved], new[moved])
    counts = np.bincount(a, minlength=mu.shape[0])
    for c in touched:
        members = np.nonzero(a == c)[0]
        if members.size:
            mu[c] = X[members].mean(axis=0)
    return a, mu, counts


def merge_cost(sq: int, chi, sizes_k, tau_q: int = 64, tau_k: int = 64, g: int = 1) -> int:
    """[HVA] Eq. 7-8: the CTA-aligned work of one query group,
    tau_q ceil(s^q / tau_q) * tau_k ceil(sum_j chi_j s_j^k / tau_k), with the
    selected key clusters packed one after another.  ``g`` is the packing
    grain of a key cluster: with g > 1 each cluster occupies g ceil(s_j / g)
    key slots (g = 1 is the page's form)."""
    sk = np.asarray(sizes_k, dtype=np.int64)
    slots = g * (-(-sk // g))
    keys = int(slots[np.asarray(chi, dtype=bool)].sum())
    return (tau_q * (-(-int(sq) // tau_q))) * (tau_k * (-(-keys // tau_k)))


def partition_cost(groups: list[list[int]], sizes_q, rows, sizes_k,
                   tau_q: int = 64, tau_k: int = 64, g: int = 1) -> int:
    """[HVA] Eq. 9: the total of Eq. 8 over a partition of the query
    clusters; a group's key set is the union of its members' rows."""
    total = 0
    for S in groups:
        chi = np.zeros(len(sizes_k), dtype=bool)
        for i in S:
            chi[list(rows[i])] = True
        total += merge_cost(sum(int(sizes_q[i]) for i in S), chi, sizes_k, tau_q, tau_k, g)
    return total


def agglomerative_merge(sizes_q, rows, sizes_k, sides, tau_q: int = 64, tau_k: int = 64,
                        g: int = 1):
    """[HVA] Algorithm 1 (parallel agglomerative merging), Eq. 8 and 10.

    Starts from singleton groups.  In round r every active group is put on
    one side of the bipartition by ``sides[r][rep]`` (0 or 1), where ``rep``
    is the group's lowest query-cluster index; the random draw is the
    caller's.  Every group A on side 0 finds the group B on side 1 that
    minimises the merge gain dC(A, B) = C(A u B) - C(A) - C(B) (Eq. 10; ties
    to the lower B).  Among the groups A choosing the same B with a negative
    gain, the one with the smallest gain is kept (ties to the lower A).  The
    kept pairs are disjoint and all merge at the end of the round.

    Returns (group id of every query cluster = its group's lowest member,
    list of groups, each ascending, ordered by their lowest member)."""
    nq = len(sizes_q)
    nk = len(sizes_k)
    grp = list(range(nq))
    members = {i: [i] for i in range(nq)}
    chi = {}
    for i in range(nq):
        c = np.zeros(nk, dtype=bool)
        c[list(rows[i])] = True
        chi[i] = c
    sq = {i: int(sizes_q[i]) for i in range(nq)}

    for r in range(len(sides)):
        active = sorted(members)
        side_a = [A for A in active if sides[r][A] == 0]
        side_b = [B for B in active if sides[r][B] == 1]
        if not side_a or not side_b:
            continue
        choice = {}
        for A in side_a:
            best = None
            for B in side_b:
                gain = merge_gain(sq[A], chi[A], sq[B], chi[B], sizes_k, tau_q, tau_k, g)
                if best is None or gain < best[0]:
                    best = (gain, B)
            choice[A] = best
        accepted = disjoint_merges(choice)
        for B, (gain, A) in accepted.items():
            lo, hi = min(A, B), max(A, B)
            members[lo] = sorted(members[lo] + members.pop(hi))
            chi[lo] = chi[lo] | chi.pop(hi)
            sq[lo] = sq[lo] + sq.pop(hi)
            for i in members[lo]:
                grp[i] = lo
    groups = [members[k] for k in sorted(members)]
    return np.asarray(grp, dtype=np.int64), groups


def merge_gain(sq_a: int, chi_a, sq_b: int, chi_b, sizes_k, tau_q: int = 64,
               tau_k: int = 64, g: int = 1) -> int:
    """[HVA] Eq. 10: dC(A, B) = C(A u B) - C(A) - C(B); the union adds the
    query sizes and ORs the key-cluster masks (Eq. 8)."""
    union = np.asarray(chi_a, bool) | np.asarray(chi_b, bool)
    return (merge_cost(sq_a + sq_b, union, sizes_k, tau_q, tau_k, g)
            - merge_cost(sq_a, chi_a, sizes_k, tau_q, tau_k, g)
            - merge_cost(sq_b, chi_b, sizes_k, tau_q, tau_k, g))


def disjoint_merges(choice: dict) -> dict:
    """[HVA] Algorithm 1, the accepted set: from every chooser A's best
    (gain, B), keep the pairs with a negative gain and, for each target B,
    only the chooser of smallest gain (ties to the lower A).  Returns
    {B: (gain, A)}."""
    accepted = {}
    for A in sorted(choice):
        gain, B = choice[A]
        if gain >= 0:
            continue
        if B not in accepted or gain < accepted[B][0]:
            accepted[B] = (gain, A)
    return accepted


def group_rows(groups: list[list[int]], rows) -> list[list[int]]:
    """[HVA] Eq. 8: every member of a merged group attends over the union of
    the group's rows (chi_j(S) = max over members of m_ij)."""
    out = [None] * sum(len(S) for S in groups)
    for S in groups:
        u = sorted(set().union(*[set(rows[i]) for i in S]))
        for i in S:
            out[i] = u
    return out


def packed_tile_pairs(off_q, off_k, groups: list[list[int]], rows, tile: int = 64,
                      g: int = 16) -> int:
    """Work of Eq. 4 on tiles when every query group fills whole query tiles
    and its key clusters are packed one after another at a grain of g
    tokens: sum over groups of ceil(s^q(S) / tile) * ceil(sum g ceil(s_j/g) / tile)
    -- Eq. 8 divided by tile^2."""
    sq = np.diff(np.asarray(off_q))
    sk = np.diff(np.asarray(off_k))
    return partition_cost(groups, sq, rows, sk, tile, tile, g) // (tile * tile)


def assignment_margins(X, thw, cell, window, mu):
    """Per token, the gap between its second-nearest and nearest squared
    distance over its window's centroids (a tie has gap 0)."""
    X = np.asarray(X, np.float64)
    T, H, W = thw
    K, w = cluster_grid(thw, cell, window)
    Kt, Kh, Kw = K
    out = np.zeros(X.shape[0])
    for t in range(T):
        for h in range(H):
            for x in range(W):
                g = (t // cell[0], h // cell[1], x // cell[2])
                st = [window_start(g[i], w[i], K[i]) for i in range(3)]
                cand = [(vt * Kh + vh) * Kw + vw for vt in range(st[0], st[0] + w[0])
                        for vh in range(st[1], st[1] + w[1]) for vw in range(st[2], st[2] + w[2])]
                dd = np.sort(((X[(t * H + h) * W + x] - mu[cand]) ** 2).sum(axis=1))
                out[(t * H + h) * W + x] = dd[1] - dd[0] if len(dd) > 1 else np.inf
    return out


# ----------------------------------------------------------------------------
# Work accounting
# ----------------------------------------------------------------------------

def executed_flops(d: int, b: int, nnz_macro: int, u: int = 16,
                   nnz_micro: int = 0) -> int:
    """Tile-level work of the two attention passes: 4 d b^2 flops per selected
    (query block, key block) pair and 4 d u^2 per micro tile (QK^T and PV,
    two flops per multiply-add), tails counted as full tiles."""
    return 4 * d * (b * b * nnz_macro + u * u * nnz_micro)


def dense_flops(B: int, H: int, N: int, d: int) -> int:
    """4 B H N^2 d flops of full attention over the valid tokens."""
    return 4 * B * H * N * N * d
