#!/usr/bin/env python
"""Benchmark of the block-sparse video-DiT attention hot path on one MI355X.

One step = pooled scoring (bsa_score_blocks) + block selection
(bsa_select_blocks) + block-sparse attention (bsa_sparse_attn_fwd) and its
fp16 V^T staging (bsa_attn_stage_v, on a second stream beside the
selection; ``--serial`` keeps one stream), plus micro-tile selection, residual
and LSE merge where the workload has them.  On small (launch-bound) layers
the timed steps replay the step captured as a HIP graph, checked bit for bit
against the eager step first (``--no-graph`` launches eagerly, ``--graph``
replays large layers too).  The default workload is one layer shaped like
Wan-2.1-1.3B at 480p: B=1, H=12, d=128, 21x30x52 = 32760 tokens, 64-token
blocks, top-k at 25% density (k = 128 of 512 key blocks).  ``--config N``
selects another of the five workloads (0 tiny reference, 1 the default,
2 Wan-2.1-14B 720p top-p, 3 HunyuanVideo 720p top-k + micro residual,
4 long-horizon static window).  Inputs are the seeded synthetic generator's
bf16 Q/K/V, resident in HBM before timing starts.

Prints ONE JSON line.  `value` is the executed attention TFLOP of a step
(64x64 block pairs plus 16x16 micro tiles) divided by the whole step time.
Kernel-level figures (the attention kernel alone, measured with HIP events on
the stream it runs on), the speedup over the library's dense flash attention,
per-stage times and bandwidths, the roofline entry of the dominant kernel and
(default workload) the fp64 CPU oracle timed on a bounded sample of the same
workload are reported beside it.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-sparse attn executed TFLOP/s, % bf16 MFMA peak, speedup vs dense"
PEAK_TFLOPS = 2500.0   # MI355X dense bf16/fp16 matrix peak
HBM_GBS = 8000.0       # MI355X HBM3E
N_ROTATIONS = 3        # static workload: anchor offsets cycled over the steps
# Local-window clustering cells (Q, K) per workload: the page's settings for
# the 720p Wan and HunyuanVideo layers; the Wan setting for the others.
CLUSTER_CELLS = {2: ((7, 6, 6), (6, 4, 4)), 3: ((11, 5, 5), (11, 3, 3))}
CLUSTER_WINDOW = (3, 8, 8)
CLUSTER_ITERS = 3
HVA_MIN_KC = {2: 0.18, 3: 0.15}   # the page's Min-kc per layer (Wan 720p, HunyuanVideo)
HVA_ROUNDS = 3                     # rounds of cluster merging (the page's R)
FLUSH_BYTES = 512 << 20  # larger than L2 (8 x 4 MB) plus the 256 MB Infinity Cache


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="time budget of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stage-reps", type=int, default=10)
    ap.add_argument("--config", type=int, default=1, choices=range(5),
                    help="workload: 0 tiny, 1 wan2.1-1.3b-480p (default), 2 wan2.1-14b-720p, "
                         "3 hunyuanvideo-720p, 4 long-horizon static window")
    ap.add_argument("--window-frames", type=int, default=None,
                    help="static window radius in frames (workload 4; default: the literal 1)")
    ap.add_argument("--block", type=int, default=64, choices=(64, 128),
                    help="selection block in tokens (128: MOD-DiT's block-wise size; the "
                         "attention still runs 64-token tiles)")
    ap.add_argument("--mod-mask", action="store_true",
                    help="replace the workload's selection by a fixed MOD-DiT-style structural "
                         "mask: intra-frame block-diagonal, temporal diagonals at 1 and 2 "
                         "frames, 4 vertical columns")
    ap.add_argument("--rectify", action="store_true",
                    help="add the pooled rectification of omitted blocks to the step and "
                         "report its cost and its effect on the error against dense attention")
    ap.add_argument("--gain-gate", action="store_true",
                    help="with --rectify: the step's rectification applies the gain-aware gate "
                         "(both variants are reported either way)")
    ap.add_argument("--no-per-workload", action="store_true",
                    help="skip the summary lines of the other four workloads (run by default "
                         "with the default workload)")
    ap.add_argument("--cluster", action="store_true",
                    help="also time the 3D local-window clustering of Q and K (all heads) with "
                         "the page's grids and (3, 8, 8) windows, 3 iterations")
    ap.add_argument("--hva", action="store_true",
                    help="also run the cluster-induced block pipeline (local-window clustering, "
                         "permutation, cluster top-p 0.9 with the page's Min-kc, attention over "
                         "the clusters) and report its stages")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch every step's kernels eagerly (small layers replay a HIP graph)")
    ap.add_argument("--graph", action="store_true",
                    help="replay the step as a HIP graph on large layers too")
    ap.add_argument("--serial", action="store_true",
                    help="run every stage of a step on one stream (no overlap)")
    ap.add_argument("--torch-sdpa", action="store_true",
                    help="also time torch's scaled_dot_product_attention on the same Q, K, V "
                         "(flash backend only; reported for context)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="first run a plain 256 MiB device copy (reads 256 MiB, writes "
                         "256 MiB) three times, to scale hardware byte counters")
    return ap.parse_args()


def events_ms(fn, reps, stream):
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(reps):
        start.record(stream)
        fn()
        end.record(stream)
        end.synchronize()
        times.append(start.elapsed_time(end))
    times.sort()
    return times[len(times) // 2], times


def cpu_oracle_sample(Q, K, V, rows_by_head, budget_s):
    """Time the fp64 oracle on whole query blocks of the same workload
    (pooling + scores + top-k of the row, then attention over its support)
    until the time budget is used; returns executed TFLOP/s and the sample."""
    import numpy as np
    from oracle import bsa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    B, H, N, d = Q.shape
    nB = O.n_blocks(N, 64)
    k = rows_by_head["k"]
    scale = 1.0 / math.sqrt(d)
    rng = np.random.default_rng(0)
    done_blocks, flops = 0, 0
    t0 = time.perf_counter()
    h = 0
    while time.perf_counter() - t0 < budget_s:
        q = Q[0, h].double().numpy()
        kk = K[0, h].double().numpy()
        v = V[0, h].double().numpy()
        Qb, Kb = O.pool_means(q, 64), O.pool_means(kk, 64)
        for i in rng.choice(nB, size=8, replace=False):
            S_i = O.pooled_scores(Qb[i:i + 1], Kb, scale)[0]
            sel = sorted(O.topk_set(S_i, k))
            qi = O.block_tokens(N, 64, int(i))
            keys = np.concatenate([O.block_tokens(N, 64, j) for j in sel])
            O.attend(q[qi], kk[keys], v[keys], scale)
            done_blocks += 1
            flops += O.executed_flops(d, 64, len(sel))
            if time.perf_counter() - t0 >= budget_s:
                break
        h = (h + 1) % H
    el = time.perf_counter() - t0
    return dict(value=flops / el / 1e12, unit="TFLOP/s", cores=int(threads), kind="oracle",
                sample=f"{done_blocks} query blocks (pool+score+top-k+fp64 attention over "
                       f"{k} key blocks each) of the same layer, {el:.1f} s")


def traffic_entry(kernel_src):
    """HBM bytes per launch of the attention kernel from the committed
    rocprofv3 counter summary, or None when the kernel's sources (the files
    in ``kernel_src``, hashed in order) changed since."""
    path = os.path.join(ROOT, "profiles", "attn_fwd_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    h = hashlib.sha256()
    for f in kernel_src:
        h.update(open(f, "rb").read())
    sha = h.hexdigest()
    if rec.get("kernel_src_sha256") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def build_workload(cfg, args, torch, bsa, keep_host=False):
    """Inputs of workload ``cfg`` resident on the GPU, its selection and the
    step (eager, or replayed as a HIP graph on small layers after a bit-for-
    bit check against the eager step).  Returns a namespace."""
    from types import SimpleNamespace
    from synth import (CONFIGS, config_spec, gen_qkv, micro_heads, mod_pattern_mask,
                       rotation_offset)

    c = CONFIGS[cfg]
    spec = config_spec(cfg)
    Qc, Kc, Vc = gen_qkv(spec)
    dev = torch.device("cuda:0")
    Q, K, V = (x.to(dev) for x in (Qc, Kc, Vc))
    if not keep_host:
        del Qc, Kc, Vc
        Qc = Kc = Vc = None
    B, H, N, d = Q.shape
    blk = args.block
    nB = bsa.n_blocks(N, blk)      # selection blocks
    scale = 1.0 / math.sqrt(d)
    stream = torch.cuda.current_stream(dev)
    mode = "static" if args.mod_mask else c["mode"]

    # selection parameters of the workload
    sel = {}
    if args.mod_mask:
        sel = mod_pattern_mask(spec, blk)
        sel_desc = (f"MOD-style mask: intra-frame + diagonals {sel['patterns']['diagonals']} + "
                    f"columns {sel['patterns']['columns']}")
    elif mode == "topk":
        k = bsa.budget_blocks(c["density"], nB)
        sel = dict(k=k, force_diag=c.get("force_diag", False))
        sel_desc = f"top-k {c['density']:.0%} (k={k} of {nB})" + (" + diagonal" if sel["force_diag"] else "")
    elif mode == "topp":
        cap = bsa.cap_blocks(c["cap_density"], nB)
        sel = dict(p=c["p"], k_min=1, k_cap=cap)
        sel_desc = f"top-p {c['p']} size-weighted, cap {c['cap_density']:.0%} ({cap} of {nB})"
    else:
        wf = c["window_frames"] if args.window_frames is None else args.window_frames
        sel = dict(static=dict(frame_tokens=spec.frame_tokens, window_frames=wf,
                               n_anchors=c["n_anchors"], anchor_offset=rotation_offset(cfg, 0, nB)))
        sel_desc = (f"static window +-{wf} frames + {c['n_anchors']} anchors rotating over "
                    f"{N_ROTATIONS} offsets")
    if blk != 64:
        sel_desc += f"; {blk}-token selection blocks on 64-token tiles"
    micro = None
    if "micro_head_frac" in c or "micro_m" in c:
        heads = micro_heads(cfg)
        m = c["micro_m"] if "micro_m" in c else int(round(c["micro_density"] * 64 * N / 256))
        micro = dict(m=m, mask=[h in heads for h in range(H)], heads=heads)
        sel_desc += f"; micro m={m} on {len(heads)} of {H} heads"

    ws = bsa.attn_workspace(Q)
    ws_rect = bsa.rectify_workspace(Q) if args.rectify else None
    O_buf = torch.empty(Q.shape, dtype=torch.float32, device=dev)
    L_buf = torch.empty(Q.shape[:3], dtype=torch.float32, device=dev)
    Om_buf = Lm_buf = None
    if micro is not None:
        Om_buf = torch.empty_like(O_buf)
        Lm_buf = torch.empty_like(L_buf)

    def score():
        return bsa.bsa_score_blocks(Q, K, block=blk, scores=(mode != "static"),
                                    micro=16 if micro else 0)

    offsets = [rotation_offset(cfg, call, nB) for call in range(N_ROTATIONS)]

    def select(sc, call=0):
        if mode == "static" and not args.mod_mask:
            # the anchors rotate: each call draws its own offset
            sel["static"]["anchor_offset"] = offsets[call % N_ROTATIONS]
        return bsa.bsa_select_blocks(sc["scores"], Q, block=blk, mode=mode, **sel)

    def micro_select(sc, rp, ci):
        return bsa.bsa_select_blocks(
            None, Q, mode="micro",
            micro=dict(m=micro["m"], scale=scale, head_mask=micro["mask"], macro=(rp, ci),
                       qpool16=sc["qpool16"], kpool16=sc["kpool16"]))

    aux = torch.cuda.Stream(device=dev)  # default priority
    # Small layers are launch-bound: one stream, the step replayed as a HIP
    # graph.  Large layers: eager launches with the V staging on a side
    # stream (replaying them as graphs measured no gain).
    small = B * H * N * d < (1 << 24)
    two_streams = not args.serial and not small
    use_graph = (small or args.graph) and not args.no_graph

    def step(call=0, overlap=two_streams):
        # The V^T staging runs on a second stream beside the selection, after
        # the scoring: pooling and staging both stream their tensors from
        # HBM, so running them together only shares the bandwidth, while the
        # selection leaves it free (running the micro branch beside the macro
        # attention as well measured no gain: both fill the chip).
        # fork from and join to the stream the step is issued on (the capture
        # stream while a graph is recorded)
        cur = torch.cuda.current_stream(dev)
        # the static window needs no scores: the selection runs on the mask alone
        sc = score() if (mode != "static" or micro) else {"scores": None}
        if overlap:
            aux.wait_stream(cur)
            with torch.cuda.stream(aux):
                bsa.bsa_attn_stage_v(V, workspace=ws)
        rp, ci, nnz = select(sc, call)
        if overlap:
            cur.wait_stream(aux)
        bsa.bsa_sparse_attn_fwd(Q, K, None if overlap else V, rp, ci, out=O_buf, lse=L_buf,
                                workspace=ws)
        if args.rectify:
            bsa.bsa_pooled_rectify(Q, K, V, rp, ci, O_buf, L_buf, gain_gate=args.gain_gate,
                                   workspace=ws_rect)
        mnnz = None
        if micro is not None:
            mrp, mci, mnnz = micro_select(sc, rp, ci)
            bsa.bsa_micro_residual_fwd(Q, K, None, mrp, mci, head_mask=micro["mask"],
                                       out=Om_buf, lse=Lm_buf, workspace=ws)
            bsa.bsa_lse_merge(O_buf, L_buf, Om_buf, Lm_buf, head_mask=micro["mask"],
                              out=O_buf, lse_out=L_buf)
        return sc, rp, ci, nnz, mnnz

    # the two-stream step must give the one-stream step's bits
    step(0, overlap=False)
    ref = (O_buf.clone(), L_buf.clone())
    step(0, overlap=True)
    torch.cuda.synchronize()
    if not (torch.equal(ref[0], O_buf) and torch.equal(ref[1], L_buf)):
        raise RuntimeError("two-stream step differs from the one-stream step")
    del ref

    for w in range(args.warmup):
        step(w)
    torch.cuda.synchronize()

    # The step as a HIP graph (one per anchor rotation): its kernels replay
    # without launch gaps.  Every graph is replayed three times, with eager
    # work between the replays, and must give its eager step's bits.
    run = step
    graphs = []
    if use_graph:
        variants = N_ROTATIONS if (mode == "static" and not args.mod_mask) else 1
        refs = []
        for r in range(variants):
            step(r, overlap=False)
            torch.cuda.synchronize()
            refs.append((O_buf.clone(), L_buf.clone()))
        capture = torch.cuda.Stream(device=dev)
        for r in range(variants):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=capture):
                # the side stream forks from and joins the capture stream
                outs = step(r, overlap=two_streams)
            graphs.append((g, outs))
        for _ in range(3):
            for r, (g, _outs) in enumerate(graphs):
                # clear what a replay must rewrite: outputs and the staged V^T
                O_buf.zero_()
                L_buf.zero_()
                ws.zero_()
                g.replay()
                torch.cuda.synchronize()
                if not (torch.equal(O_buf, refs[r][0]) and torch.equal(L_buf, refs[r][1])):
                    raise RuntimeError("graph replay differs from the eager step")
        del refs

        def run(call):
            g, outs = graphs[call % len(graphs)]
            g.replay()
            return outs

        for w in range(args.warmup):
            run(w)
        torch.cuda.synchronize()

    return SimpleNamespace(**{k: v for k, v in locals().items() if k not in ("torch", "bsa")})


def time_steps(W, steps, torch):
    """Times `steps` steps of a built workload (synchronised on both sides);
    returns (seconds per step, mean macro entries, mean micro entries, the
    last step's outputs)."""
    nnz_all, mnnz_all = [], []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_i in range(steps):
        last = W.run(s_i)
        nnz_all.append(last[3])
        if last[4] is not None:
            mnnz_all.append(last[4])
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / steps
    nnz_mean = sum(int(x.item()) for x in nnz_all) / len(nnz_all)
    mnnz_mean = sum(int(x.item()) for x in mnnz_all) / len(mnnz_all) if mnnz_all else 0.0
    return step_s, nnz_mean, mnnz_mean, last


def workload_summary(cfg, args, torch, bsa):
    """One line of figures for a workload other than the headline one: step
    time over a few steps, the attention kernel alone (HIP events on its
    stream), the dense kernel of the same library, and the micro stages where
    the workload has them."""
    W = build_workload(cfg, args, torch, bsa)
    steps = 20 if cfg == 0 else 5
    step_s, nnz_mean, mnnz_mean, (sc, rp, ci, nnz, mnnz) = time_steps(W, steps, torch)
    B, H, N, d = W.B, W.H, W.N, W.d
    nnz_v = int(nnz.item())
    macro_flops = 4 * d * 64 * 64 * nnz_v
    dense_flops = 4 * B * H * N * N * d
    exec_flops = 4 * d * (64 * 64 * nnz_mean + 16 * 16 * mnnz_mean)
    reps = 3 if cfg != 0 else 10
    attn_ms, _ = events_ms(
        lambda: bsa.bsa_sparse_attn_fwd(W.Q, W.K, None, rp, ci, out=W.O_buf, lse=W.L_buf,
                                        workspace=W.ws), reps, W.stream)
    dense_ms, _ = events_ms(
        lambda: bsa.bsa_dense_attn_fwd(W.Q, W.K, None, out=W.O_buf, lse=W.L_buf,
                                       workspace=W.ws), 2 if cfg != 0 else 10, W.stream)
    attn_tflops = macro_flops / (attn_ms * 1e-3) / 1e12
    res = {"workload": W.c["name"], "B": B, "H": H, "N": N, "d": d, "selection": W.sel_desc,
           "density": round(nnz_mean / (B * H * bsa.n_blocks(N) ** 2), 4),
           "steps": steps, "step_graph": bool(W.graphs),
           "ms_per_step": round(step_s * 1e3, 4),
           "value_tflops": round(exec_flops / step_s / 1e12, 2),
           "attn_kernel_ms": round(attn_ms, 4),
           "attn_kernel_tflops": round(attn_tflops, 2),
           "pct_mfma_peak": round(100 * attn_tflops / PEAK_TFLOPS, 2),
           "dense_kernel_ms": round(dense_ms, 4),
           "dense_kernel_tflops": round(dense_flops / (dense_ms * 1e-3) / 1e12, 2),
           "speedup_vs_dense": round(dense_ms / attn_ms, 3),
           "pipeline_speedup_vs_dense": round(dense_ms / (step_s * 1e3), 3)}
    if W.micro is not None:
        mrp, mci, mn = W.micro_select(sc, rp, ci)
        msel_ms, _ = events_ms(lambda: W.micro_select(sc, rp, ci), reps, W.stream)
        mattn_ms, _ = events_ms(
            lambda: bsa.bsa_micro_residual_fwd(W.Q, W.K, None, mrp, mci,
                                               head_mask=W.micro["mask"], out=W.Om_buf,
                                               lse=W.Lm_buf, workspace=W.ws), reps, W.stream)
        merge_ms, _ = events_ms(
            lambda: bsa.bsa_lse_merge(W.O_buf, W.L_buf, W.Om_buf, W.Lm_buf,
                                      head_mask=W.micro["mask"], out=W.O_buf, lse_out=W.L_buf),
            reps, W.stream)
        mnv = int(mn.item())
        res["micro"] = {"m": W.micro["m"], "heads": list(W.micro["heads"]),
                        "tiles": mnv, "micro_select_ms": round(msel_ms, 4),
                        "micro_residual_ms": round(mattn_ms, 4),
                        "micro_residual_tflops": round(4 * d * 256 * mnv / (mattn_ms * 1e-3)
                                                       / 1e12, 2),
                        "lse_merge_ms": round(merge_ms, 4)}
    del W
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU only; the path shards "
                                   "by (batch, head) with no exchange between GPUs, and no "
                                   "multi-GPU run is implemented"}))
        sys.exit(2)

    import torch
    import block_sparse_attention_pool_amd as bsa
    from synth import merge_sides

    if args.calibration_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    cfg = args.config
    W = build_workload(cfg, args, torch, bsa, keep_host=True)
    c, spec = W.c, W.spec
    Qc, Kc, Vc = W.Qc, W.Kc, W.Vc
    Q, K, V = W.Q, W.K, W.V
    B, H, N, d = W.B, W.H, W.N, W.d
    blk, nB, scale, stream, mode = W.blk, W.nB, W.scale, W.stream, W.mode
    sel, sel_desc, micro = W.sel, W.sel_desc, W.micro
    ws, ws_rect = W.ws, W.ws_rect
    O_buf, L_buf, Om_buf, Lm_buf = W.O_buf, W.L_buf, W.Om_buf, W.Lm_buf
    score, select, micro_select = W.score, W.select, W.micro_select
    graphs, two_streams = W.graphs, W.two_streams
    dev = torch.device("cuda:0")

    # executed work of the timed steps (rows differ per call when the anchors rotate)
    step_s, nnz_mean, mnnz_mean, (sc, rp, ci, nnz, mnnz) = time_steps(W, args.steps, torch)
    exec_flops = 4 * d * (64 * 64 * nnz_mean + 16 * 16 * mnnz_mean)
    # kernel-level figures below use the lists of the last step
    nnz_v = int(nnz.item())
    mnnz_v = int(mnnz.item()) if mnnz is not None else 0
    macro_flops = 4 * d * 64 * 64 * nnz_v
    dense_flops = 4 * B * H * N * N * d

    # Kernel-level: the attention kernel alone (V^T already staged: V=None).
    reps = args.stage_reps
    attn_ms, _ = events_ms(
        lambda: bsa.bsa_sparse_attn_fwd(Q, K, None, rp, ci, out=O_buf, lse=L_buf, workspace=ws),
        reps, stream)
    # Cold caches: a 512 MB write between reps evicts L2 and the Infinity Cache.
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    cold = []
    for _ in range(max(3, reps // 2)):
        flush.zero_()
        ms, _ = events_ms(
            lambda: bsa.bsa_sparse_attn_fwd(Q, K, None, rp, ci, out=O_buf, lse=L_buf, workspace=ws),
            1, stream)
        cold.append(ms)
    cold.sort()
    attn_cold_ms = cold[len(cold) // 2]
    del flush
    L_sparse = L_buf.clone()
    dense_ms, _ = events_ms(
        lambda: bsa.bsa_dense_attn_fwd(Q, K, None, out=O_buf, lse=L_buf, workspace=ws),
        max(3, reps // 2) if dense_flops < 2e13 else 3, stream)
    L_full = L_buf.clone()
    sdpa_out = None
    if args.torch_sdpa:
        # torch's fused attention on the same tensors, forced onto its flash
        # backend (it raises rather than falling back to the unfused path)
        from torch.nn.attention import SDPBackend, sdpa_kernel
        try:
            with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
                sdpa_ms, _ = events_ms(
                    lambda: torch.nn.functional.scaled_dot_product_attention(Q, K, V), 3, stream)
            sdpa_out = {"backend": "flash", "ms": round(sdpa_ms, 4),
                        "tflops": round(dense_flops / (sdpa_ms * 1e-3) / 1e12, 2),
                        "dense_kernel_speedup": round(sdpa_ms / dense_ms, 3)}
        except RuntimeError as ex:
            sdpa_out = {"backend": "flash", "unavailable": str(ex)[:200]}
    score_ms, _ = events_ms(score, reps, stream) if mode != "static" else (0.0, None)
    select_ms, _ = events_ms(lambda: select(sc), reps, stream)
    attn_v_ms, _ = events_ms(
        lambda: bsa.bsa_sparse_attn_fwd(Q, K, V, rp, ci, out=O_buf, lse=L_buf, workspace=ws),
        reps, stream)
    stages = {"score_blocks": round(score_ms, 4), "select_blocks": round(select_ms, 4),
              "sparse_attn_fwd_with_v_staging": round(attn_v_ms, 4),
              "attn_kernel": round(attn_ms, 4)}
    gbs = {}
    if mode != "static":
        # pooling reads Q and K and writes the means; the score kernel writes nB^2 scores
        gbs["score_blocks"] = round((4 * B * H * N * d + 8 * B * H * nB * d
                                     + 4 * B * H * nB * nB) / (score_ms * 1e-3) / 1e9, 1)
        gbs["select_blocks"] = round((4 * B * H * nB * nB + 4 * nnz_v)
                                     / (select_ms * 1e-3) / 1e9, 1)
    if micro is not None:
        mrp, mci, _ = micro_select(sc, rp, ci)
        msel_ms, _ = events_ms(lambda: micro_select(sc, rp, ci), reps, stream)
        mattn_ms, _ = events_ms(
            lambda: bsa.bsa_micro_residual_fwd(Q, K, None, mrp, mci, head_mask=micro["mask"],
                                               out=Om_buf, lse=Lm_buf, workspace=ws),
            reps, stream)
        merge_ms, _ = events_ms(
            lambda: bsa.bsa_lse_merge(O_buf, L_buf, Om_buf, Lm_buf, head_mask=micro["mask"],
                                      out=O_buf, lse_out=L_buf), reps, stream)
        stages.update({"micro_select": round(msel_ms, 4), "micro_residual_fwd": round(mattn_ms, 4),
                       "lse_merge": round(merge_ms, 4)})
        rows_m = B * len(micro["heads"]) * N
        gbs["lse_merge"] = round(rows_m * (3 * d * 4 + 12) / (merge_ms * 1e-3) / 1e9, 1)
        stages["micro_tflops"] = round(4 * d * 256 * mnnz_v / (mattn_ms * 1e-3) / 1e12, 2)

    # Offline head calibration: omitted softmax share per head (sparse vs full
    # attention) and, with the micro residual, the share it brings back.
    L_rep = None
    if micro is not None:
        L_rep = L_sparse.clone()
        bsa.bsa_lse_merge(O_buf, L_sparse, Om_buf, Lm_buf, head_mask=micro["mask"],
                          out=O_buf, lse_out=L_rep)
    risk = bsa.bsa_omission_risk(L_sparse, L_full, L_rep)
    risk_ms, _ = events_ms(lambda: bsa.bsa_omission_risk(L_sparse, L_full, L_rep, out=risk),
                           reps, stream)
    risk_h = risk[0].cpu()
    mean_w = [round(float(x), 5) for x in risk_h[:, 0]]
    risk_out = {"kernel_ms": round(risk_ms, 4),
                "gbs": round(B * H * N * (12 if L_rep is not None else 8)
                             / (risk_ms * 1e-3) / 1e9, 1),
                "mean_omitted_share_per_head": mean_w,
                "max_omitted_share": round(float(risk_h[:, 1].max()), 5)}
    if micro is not None:
        mh = micro["heads"]
        omitted = sum(float(risk_h[h, 0]) for h in mh)
        risk_out["micro_recovered_share"] = round(
            sum(float(risk_h[h, 2]) for h in mh) / omitted, 5) if omitted > 0 else None
        risk_out["heads_at_risk"] = bsa.heads_at_risk(mean_w, len(mh))
        risk_out["micro_heads"] = list(mh)

    rect_out = None
    if args.rectify:
        # its cost, and mean |O - O_dense| over the whole layer before and after
        Os = torch.empty_like(O_buf)
        Ls = torch.empty_like(L_buf)
        bsa.bsa_sparse_attn_fwd(Q, K, None, rp, ci, out=Os, lse=Ls, workspace=ws)
        Or, Lr = Os.clone(), Ls.clone()
        bsa.bsa_pooled_rectify(Q, K, V, rp, ci, Or, Lr, workspace=ws_rect)
        Od = torch.empty_like(O_buf)
        Ld = torch.empty_like(L_buf)
        bsa.bsa_dense_attn_fwd(Q, K, None, out=Od, lse=Ld, workspace=ws)

        def rect_once(gate):
            Or.copy_(Os)
            Lr.copy_(Ls)
            bsa.bsa_pooled_rectify(Q, K, V, rp, ci, Or, Lr, gain_gate=gate, workspace=ws_rect)

        copy_ms, _ = events_ms(lambda: (Or.copy_(Os), Lr.copy_(Ls)), reps, stream)
        omitted_pairs = B * H * bsa.n_blocks(N) ** 2 - nnz_v
        rect_out = {"gain_gate_in_step": bool(args.gain_gate),
                    "mean_abs_err_vs_dense_sparse": float((Os - Od).abs().mean()),
                    "mean_abs_lse_err_vs_dense_sparse": float((Ls - Ld).abs().mean())}
        for gate in (False, True):
            rect_ms, _ = events_ms(lambda: rect_once(gate), reps, stream)
            rect_ms = max(rect_ms - copy_ms, 1e-6)
            rect_once(gate)
            key = "gated" if gate else "ungated"
            rect_out[key] = {
                "kernel_ms": round(rect_ms, 4),
                "tflops": round(4 * d * 64 * omitted_pairs / (rect_ms * 1e-3) / 1e12, 2),
                "mean_abs_err_vs_dense_rectified": float((Or - Od).abs().mean()),
                "mean_abs_lse_err_vs_dense_rectified": float((Lr - Ld).abs().mean())}
        # share of (query, omitted block) pairs the gate keeps, on two heads'
        # rows: |q|^2 v_j < 2 ln 2 / scale^2 with v_j the block's key spread
        kept = total = 0
        rows_all = bsa.csr_rows(rp, ci, nnz)
        nB64 = bsa.n_blocks(N)
        for h in (0, H - 1):
            Kh = K[0, h].float()
            nfull = nB64 * 64
            Kp = torch.zeros((nfull, d), device=dev)
            Kp[:N] = Kh
            cnt = torch.full((nB64,), 64.0, device=dev)
            cnt[-1] = N - 64 * (nB64 - 1)
            mean = Kp.view(nB64, 64, d).sum(1) / cnt[:, None]
            valid = (torch.arange(nfull, device=dev) < N).float().view(nB64, 64, 1)
            spread = (((Kp.view(nB64, 64, d) - mean[:, None]) ** 2) * valid).sum((1, 2)) / (cnt * d)
            qn2 = (Q[0, h].float() ** 2).sum(1)
            G = qn2[:, None] * spread[None, :] < 2 * math.log(2) / (scale * scale)
            for i in range(nB64):
                om = torch.ones(nB64, dtype=torch.bool, device=dev)
                om[rows_all[h * nB64 + i]] = False
                g = G[64 * i:min(64 * i + 64, N)][:, om]
                kept += int(g.sum())
                total += g.numel()
        rect_out["gate_pass_share_two_heads"] = round(kept / max(total, 1), 4)
        del Os, Or, Od

    cluster_out = None
    if args.cluster:
        cq, ck = CLUSTER_CELLS.get(cfg, CLUSTER_CELLS[2])
        thw = spec.grid
        res = {}
        flops = 0
        for name, X, cell in (("Q", Q, cq), ("K", K, ck)):
            a_, mu_, c_ = bsa.bsa_local_window_cluster(X, thw, cell, CLUSTER_WINDOW, CLUSTER_ITERS)
            ms, _ = events_ms(lambda: bsa.bsa_local_window_cluster(X, thw, cell, CLUSTER_WINDOW,
                                                                     CLUSTER_ITERS), reps, stream)
            Kc = [-(-thw[i] // cell[i]) for i in range(3)]
            wv = 1
            for i in range(3):
                wv *= min(CLUSTER_WINDOW[i], Kc[i])
            # assignment work: one d-long dot product per (token, window centroid)
            flops += 2 * d * N * wv * B * H * CLUSTER_ITERS
            res[name] = {"cells": int(mu_.shape[2]), "cell": list(cell), "ms": round(ms, 4)}
        # HVA section 4.2 on the keys' clustering: Lowe's ratio and its 15%
        # subset, then one intermediate-step refinement of that subset (the
        # subset reassigned against every centroid, the touched centroids
        # re-averaged), each call timed alone from the same clustering
        lowe_ms, _ = events_ms(lambda: bsa.bsa_lowe_ratio_subset(K, mu_, thw, ck, CLUSTER_WINDOW,
                                                                 0.15), reps, stream)
        _, sub = bsa.bsa_lowe_ratio_subset(K, mu_, thw, ck, CLUSTER_WINDOW, 0.15)
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        rt = []
        moved = 0
        for _ in range(reps):
            a2, m2, c2 = a_.clone(), mu_.clone(), c_.clone()
            ev0.record(stream)
            bsa.bsa_subset_refine(K, sub, a2, m2, c2)
            ev1.record(stream)
            ev1.synchronize()
            rt.append(ev0.elapsed_time(ev1))
            moved = int((a2 != a_).sum())
        rt.sort()
        res["K_subset"] = {"n_sub_per_head": int(sub.shape[2]),
                           "lowe_ratio_subset_ms": round(lowe_ms, 4),
                           "subset_refine_ms": round(rt[len(rt) // 2], 4),
                           "tokens_reassigned": moved}
        tot = res["Q"]["ms"] + res["K"]["ms"]
        # the assignment runs three bf16 matrix products per dot product (the
        # centroid's hi, mid and lo parts); rates over the whole call (updates
        # included)
        eff = flops / (tot * 1e-3) / 1e12
        cluster_out = {"iters": CLUSTER_ITERS, "window": list(CLUSTER_WINDOW), **res,
                       "ms_total": round(tot, 4),
                       "assign_tflops_effective": round(eff, 2),
                       "mfma_tflops_executed": round(3 * eff, 2),
                       "frac_bf16_mfma_peak": round(3 * eff / PEAK_TFLOPS, 4)}

    hva_out = None
    if args.hva:
        cq, ck = CLUSTER_CELLS.get(cfg, CLUSTER_CELLS[2])
        thw, win, it = spec.grid, CLUSTER_WINDOW, CLUSTER_ITERS
        min_kc = HVA_MIN_KC.get(cfg, 0.18)
        st = {}

        def clus():
            return (bsa.bsa_local_window_cluster(Q, thw, cq, win, it),
                    bsa.bsa_local_window_cluster(K, thw, ck, win, it))

        (aq, mq, nq), (ak, mk, nk) = clus()
        Nq, Nk = nq.shape[2], nk.shape[2]
        k_min = math.ceil(min_kc * Nk)

        def perm():
            return (bsa.bsa_cluster_permute(aq, nq, Q, thw, cq, win),
                    bsa.bsa_cluster_permute(ak, nk, K, thw, ck, win))

        (pq, oq), (pk, ok) = perm()

        def csel():
            return bsa.bsa_cluster_select(mq, mk, nk, p=0.9, k_min=k_min, k_cap=Nk)

        crp, cci, cnnz = csel()

        sides = torch.from_numpy(merge_sides(spec.key, B, H, HVA_ROUNDS, Nq)).to(dev)

        def cmerge():
            return bsa.bsa_cluster_merge(oq, ok, crp, cci, sides, N=N)

        gof = cmerge()

        def cattn():
            return bsa.bsa_cluster_attn_fwd(Q, K, V, pq, oq, pk, ok, crp, cci)

        def cattn_merged():
            return bsa.bsa_cluster_attn_fwd(Q, K, V, pq, oq, pk, ok, crp, cci, gof)

        _, _, pairs = cattn()
        _, _, pairs_m = cattn_merged()
        r3 = max(3, reps // 3)
        st["cluster_qk"], _ = events_ms(clus, r3, stream)
        st["permute_qk"], _ = events_ms(perm, r3, stream)
        st["cluster_select"], _ = events_ms(csel, r3, stream)
        st["cluster_merge"], _ = events_ms(cmerge, r3, stream)
        st["cluster_attn_merged"], _ = events_ms(cattn_merged, r3, stream)
        attn_unmerged_ms, _ = events_ms(cattn, r3, stream)
        torch.cuda.synchronize()
        pairs_v, pairs_mv = int(pairs.item()), int(pairs_m.item())
        groups = int(sum(len(set(g.tolist())) for g in gof.reshape(B * H, Nq).cpu()))
        # token-level density of the cluster mask before and after merging:
        # sum over query clusters of s_i times the tokens of its (group's) key clusters
        sq = (oq[..., 1:] - oq[..., :-1]).double().reshape(B * H, Nq).cpu().numpy()
        sk = (ok[..., 1:] - ok[..., :-1]).double().reshape(B * H, Nk).cpu().numpy()
        rows_c = bsa.csr_rows(crp, cci, cnnz)
        gl = gof.reshape(B * H, Nq).cpu().numpy()
        tok_pairs = tok_pairs_m = 0.0
        for z in range(B * H):
            union = {}
            for i in range(Nq):
                union.setdefault(gl[z][i], set()).update(rows_c[z * Nq + i])
            for i in range(Nq):
                tok_pairs += sq[z][i] * sk[z][rows_c[z * Nq + i]].sum()
                tok_pairs_m += sq[z][i] * sk[z][sorted(union[gl[z][i]])].sum()
        hva_flops = 4 * d * 64 * 64 * pairs_mv
        total = sum(st.values())
        full = B * H * N * N
        hva_out = {"q_cells": Nq, "k_cells": Nk, "p": 0.9, "min_kc": min_kc, "k_min": k_min,
                   "merge_rounds": HVA_ROUNDS, "groups": groups,
                   "stages_ms": {k: round(v, 4) for k, v in st.items()},
                   "tile_pairs": pairs_mv, "tile_pairs_unmerged": pairs_v,
                   "token_density": round(tok_pairs_m / full, 4),
                   "token_density_unmerged": round(tok_pairs / full, 4),
                   "tile_density": round(pairs_mv / (B * H * bsa.n_blocks(N) ** 2), 4),
                   "tile_density_unmerged": round(pairs_v / (B * H * bsa.n_blocks(N) ** 2), 4),
                   "cluster_attn_unmerged_ms": round(attn_unmerged_ms, 4),
                   "attn_tflops_executed": round(
                       hva_flops / (st["cluster_attn_merged"] * 1e-3) / 1e12, 2),
                   "speedup_attn_vs_dense": round(dense_ms / st["cluster_attn_merged"], 3),
                   "speedup_pipeline_vs_dense": round(dense_ms / total, 3)}

    attn_tflops = macro_flops / (attn_ms * 1e-3) / 1e12
    csrc = os.path.join(ROOT, "block_sparse_attention_pool_amd", "csrc")
    kernel_src = [os.path.join(csrc, "attn.hip"), os.path.join(csrc, "attn_util.h")]
    # the committed counters were taken on the default workload and selection
    traffic = (traffic_entry(kernel_src)
               if (cfg == 1 and blk == 64 and not args.mod_mask and not args.rectify) else None)
    out = {
        "metric": METRIC,
        "value": round(exec_flops / step_s / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded structured video Q/K/V)",
        "config": {"workload": c["name"] + ("+mod-mask" if args.mod_mask else ""),
                   "B": B, "H": H, "N": N, "d": d, "block": blk,
                   "selection": sel_desc,
                   "density": round(nnz_mean / (B * H * bsa.n_blocks(N) ** 2), 4)},
        "step_streams": 2 if two_streams else 1,
        "step_graph": bool(graphs),
        "attn_kernel_ms": round(attn_ms, 4),
        "attn_kernel_tflops": round(attn_tflops, 2),
        "attn_kernel_ms_cold_cache": round(attn_cold_ms, 4),
        "attn_kernel_tflops_cold_cache": round(macro_flops / (attn_cold_ms * 1e-3) / 1e12, 2),
        "pct_mfma_peak": round(100 * attn_tflops / PEAK_TFLOPS, 2),
        "dense_equiv_tflops": round(dense_flops / (attn_ms * 1e-3) / 1e12, 2),
        "dense_kernel_ms": round(dense_ms, 4),
        "dense_kernel_tflops": round(dense_flops / (dense_ms * 1e-3) / 1e12, 2),
        "speedup_vs_dense": round(dense_ms / attn_ms, 3),
        "pipeline_speedup_vs_dense": round(dense_ms / (step_s * 1e3), 3),
        **({"torch_sdpa": sdpa_out} if sdpa_out is not None else {}),
        "stages_ms": stages,
        "stage_gbs": gbs,
        "omission_risk": risk_out,
        **({"pooled_rectify": rect_out} if rect_out is not None else {}),
        **({"local_window_cluster": cluster_out} if cluster_out is not None else {}),
        **({"hva_cluster_pipeline": hva_out} if hva_out is not None else {}),
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_TFLOPS, 4),
                     "traffic": traffic},
    }
    if not args.no_cpu_baseline and cfg == 1 and blk == 64 and not args.mod_mask \
            and not args.rectify:
        rows = {"k": sel["k"]}
        out["cpu_baseline"] = cpu_oracle_sample(Qc, Kc, Vc, rows, args.cpu_seconds)
    headline_only = (args.no_per_workload or cfg != 1 or blk != 64 or args.mod_mask
                     or args.rectify or args.cluster or args.hva or args.window_frames is not None)
    if not headline_only:
        # the other four workloads, one summary each (their inputs generated
        # once, a few steps each); the headline workload's buffers are freed first
        del W, Q, K, V, O_buf, L_buf, Om_buf, Lm_buf, ws
        torch.cuda.empty_cache()
        per = {}
        for other in (0, 2, 3, 4):
            print(f"[bench] per-workload summary of workload {other}", file=sys.stderr, flush=True)
            per[str(other)] = workload_summary(other, args, torch, bsa)
        out["per_workload"] = per
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
