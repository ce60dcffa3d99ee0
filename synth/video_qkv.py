"""Seeded, structured bf16 Q/K/V shaped like video-DiT attention inputs.

Tokens come from a latent grid T x Hg x Wg flattened t-major,
n = (t * Hg + y) * Wg + x.  Each of Q, K, V is

    X = N(0, 1) + 0.5 * phi(t, y, x) @ W_h^T

drawn in float32 and rounded to bf16 (round-to-nearest-even).  phi holds 12
smooth positional features (3 axes x 4 frequencies): for axis length L and
coordinate c, feature k is sin(w_k c) for even k and cos(w_k c) for odd k with
w_k = (k + 1) pi / (2 L), so each axis spans at most one period.  W_h is a
d x 12 standard normal matrix drawn per head and shared by Q, K and V, which
gives q.k a spatio-temporal locality term (nearby tokens attend to each other
more strongly, the structure video-DiT attention maps show).

Optional "spikes": every 16-token query tile and key tile gets a code in
0..49; a tile adds alpha * u_code to its tokens, with u_0..u_49 orthonormal,
so that 2% of (query tile, key tile) pairs share a code and gain about
+4 sigma of the base logit distribution.  That plants fine-grained high-value
interactions inside blocks whose 64-token pooled score stays low.

Random streams: numpy PCG64 seeded by SeedSequence(0xB5A, spawn_key=(cfg,
stream, index)); stream 0 = W, 1/2/3 = Q/K/V noise, 4 = spike codes and
directions, 5 = micro-head subset, 6 = anchor rotation offsets, 7 = sample of
pairs for the logit spread, 8 = the bipartition bits of cluster merging.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

ENTROPY = 0xB5A
N_CODES = 50


@dataclasses.dataclass(frozen=True)
class VideoSpec:
    """Shape of one attention layer's input and the seed key that draws it."""

    B: int
    H: int
    d: int
    grid: tuple[int, int, int]  # (T, Hg, Wg) latent frames x height x width
    key: int                     # seed key (the spawn_key's first entry)
    spikes: bool = False

    @property
    def N(self) -> int:
        T, Hg, Wg = self.grid
        return T * Hg * Wg

    @property
    def frame_tokens(self) -> int:
        return self.grid[1] * self.grid[2]


# The five workloads: a tiny reference layer, then layers shaped like
# Wan-2.1-1.3B 480p, Wan-2.1-14B 720p, HunyuanVideo 720p and a 6x long-horizon
# Wan-1.3B layer.  Selection parameters: top-k density, top-p threshold with a
# density cap, micro budget (16x16 tiles per 64-row query block) on a head
# subset, and the static window + rotating anchors mask.
CONFIGS = {
    0: dict(name="tiny-ref-1024", spec=VideoSpec(1, 2, 64, (4, 16, 16), 0),
            mode="topk", density=0.25, force_diag=True, micro_m=8,
            micro_head_frac=1.0),
    1: dict(name="wan2.1-1.3b-480p", spec=VideoSpec(1, 12, 128, (21, 30, 52), 1),
            mode="topk", density=0.25),
    2: dict(name="wan2.1-14b-720p", spec=VideoSpec(1, 40, 128, (21, 45, 80), 2),
            mode="topp", p=0.9, cap_density=0.20),
    3: dict(name="hunyuanvideo-720p", spec=VideoSpec(1, 24, 128, (33, 45, 80), 3,
                                                     spikes=True),
            mode="topk", density=0.15, micro_density=0.02,
            micro_head_frac=0.3),
    4: dict(name="wan-1.3b-6x-horizon", spec=VideoSpec(1, 12, 128, (126, 30, 52), 4),
            mode="static", window_frames=1, n_anchors=4),
}


def config_spec(cfg: int) -> VideoSpec:
    return CONFIGS[cfg]["spec"]


def _rng(key: int, stream: int, index: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=ENTROPY, spawn_key=(key, stream, index))
    return np.random.Generator(np.random.PCG64(ss))


def _positional_features(grid: tuple[int, int, int]) -> np.ndarray:
    """[N, 12] float64 smooth features of (t, y, x), t-major token order."""
    feats = []
    axes = []
    for axis, L in enumerate(grid):
        c = np.arange(L, dtype=np.float64)
        cols = []
        for k in range(4):
            w = (k + 1) * math.pi / (2.0 * L)
            cols.append(np.sin(w * c) if k % 2 == 0 else np.cos(w * c))
        axes.append(np.stack(cols, axis=1))  # [L, 4]
    T, Hg, Wg = grid
    ft = np.repeat(axes[0], Hg * Wg, axis=0)
    fy = np.tile(np.repeat(axes[1], Wg, axis=0), (T, 1))
    fx = np.tile(axes[2], (T * Hg, 1))
    feats = np.concatenate([ft, fy, fx], axis=1)
    return feats


def _spike_plan(spec: VideoSpec):
    """Tile codes for queries and keys and the orthonormal code directions."""
    nT = -(-spec.N // 16)
    r = _rng(spec.key, 4, 0)
    qcode = r.integers(0, N_CODES, size=nT)
    kcode = r.integers(0, N_CODES, size=nT)
    g = r.standard_normal((spec.d, N_CODES))
    u, _ = np.linalg.qr(g)  # d x 50, orthonormal columns
    return qcode, kcode, u.T.astype(np.float32)  # [50, d]


def _head(spec: VideoSpec, h: int, pos: np.ndarray, spike):
    d, N = spec.d, spec.N
    W = _rng(spec.key, 0, h).standard_normal((d, 12))
    base = (0.5 * (pos @ W.T)).astype(np.float32)  # [N, d]
    out = []
    for stream in (1, 2, 3):
        x = _rng(spec.key, stream, h).standard_normal((spec.B, N, d),
                                                      dtype=np.float32)
        x += base[None]
        out.append(x)
    if spike is not None:
        qcode, kcode, u = spike
        # logit spread of the base tensors on a seeded sample of token pairs
        r7 = _rng(spec.key, 7, h)
        ti = r7.integers(0, N, size=4096)
        tj = r7.integers(0, N, size=4096)
        scale = 1.0 / math.sqrt(d)
        z = scale * np.einsum("nd,nd->n", out[0][0, ti].astype(np.float64),
                              out[1][0, tj].astype(np.float64))
        sigma = float(z.std())
        alpha = math.sqrt(4.0 * sigma / scale)
        tok_tile = np.arange(N) // 16
        out[0] += (alpha * u[qcode[tok_tile]])[None]
        out[1] += (alpha * u[kcode[tok_tile]])[None]
    return out


def gen_qkv(spec: VideoSpec, heads: list[int] | None = None):
    """Q, K, V as contiguous bf16 CPU tensors [B, H', N, d] for the listed heads
    (all heads by default).  Deterministic in (spec.key, head)."""
    heads = list(range(spec.H)) if heads is None else list(heads)
    pos = _positional_features(spec.grid)
    spike = _spike_plan(spec) if spec.spikes else None
    Hn = len(heads)
    Q = torch.empty((spec.B, Hn, spec.N, spec.d), dtype=torch.bfloat16)
    K = torch.empty_like(Q)
    V = torch.empty_like(Q)
    for slot, h in enumerate(heads):
        q, k, v = _head(spec, h, pos, spike)
        Q[:, slot] = torch.from_numpy(q).to(torch.bfloat16)
        K[:, slot] = torch.from_numpy(k).to(torch.bfloat16)
        V[:, slot] = torch.from_numpy(v).to(torch.bfloat16)
    return Q, K, V


def micro_heads(cfg: int) -> list[int]:
    """Seeded subset of heads that carry the micro residual."""
    c = CONFIGS[cfg]
    spec = c["spec"]
    frac = c.get("micro_head_frac", 0.0)
    n = int(round(frac * spec.H))
    if n >= spec.H:
        return list(range(spec.H))
    r = _rng(spec.key, 5, 0)
    return sorted(int(h) for h in r.choice(spec.H, size=n, replace=False))


def rotation_offset(cfg: int, call: int, n_blocks: int) -> int:
    """Anchor rotation offset for call number ``call`` (drawn fresh per call)."""
    return int(_rng(CONFIGS[cfg]["spec"].key, 6, call).integers(0, n_blocks))


def merge_sides(key: int, B: int, H: int, rounds: int, n: int) -> np.ndarray:
    """The random bipartition bits of cluster merging: uint8 [B, H, rounds, n]
    (0 or 1 per round and query cluster), drawn from stream 8."""
    return _rng(key, 8, 0).integers(0, 2, size=(B, H, rounds, n), dtype=np.uint8)


def spike_codes(spec: VideoSpec):
    """(query tile codes, key tile codes) of a spiked spec, for recall checks."""
    q, k, _ = _spike_plan(spec)
    return q, k


def mod_pattern_mask(spec: VideoSpec, block: int, frames=(1, 2), n_columns: int = 4) -> dict:
    """A fixed MOD-DiT-style structural mask for a layer of this shape, as
    selection arguments: the intra-frame block-diagonal (window of radius 0),
    parallel diagonals at the block offsets of tokens ``frames`` latent
    frames apart in either direction (the nearest offset below and above
    dt * frame_tokens / block), and ``n_columns`` vertical key columns (the
    first block, a sink, plus evenly strided blocks).  MOD chooses its
    patterns from intensities fitted to a model's dense attention maps;
    with no model, this set stands in for that choice."""
    nB = -(-spec.N // block)
    diags = set()
    for dt in frames:
        lo = (dt * spec.frame_tokens) // block
        for off in (lo, lo + 1):
            diags.update((off, -off))
    cols = sorted({(c * nB) // n_columns for c in range(n_columns)})
    return dict(static=dict(frame_tokens=spec.frame_tokens, window_frames=0,
                            n_anchors=0, anchor_offset=0),
                patterns=dict(diagonals=sorted(diags), columns=cols))
