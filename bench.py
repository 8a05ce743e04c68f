#!/usr/bin/env python3
"""Benchmark: one gated tile-sparse attention layer on one MI355X.

A step is one pass of the whole device path over one batch of synthetic
input already resident in HBM:
    g = bf16(x . W_gate^T)                  (vsa_gate_proj)
    tile means, coarse scores, top-k,
    coarse attention                        (vsa_coarse_topk)
    fine block-sparse attention + g*O_coarse (vsa_sparse_attn_fwd)
The tile plan is a pure function of the shape and is built once (cached), as
the method does.

Prints ONE JSON line. `value` is effective TFLOP/s: the kept-pair FLOPs of the
fine pass (4*D per real query-row x real key-row pair, prefix and kept video
tiles only) divided by the layer time; `ms_per_step` is ms per layer.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "ms/layer + effective TFLOP/s (% bf16 MFMA peak) for tile-sparse attn at ~100k tok"
BF16_PEAK_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (vendor figure)
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E (vendor figure)
INT8_PEAK_TOPS = 5033.2     # MI355X dense int8 MFMA (vendor figure)
# INT8 fine pass: per kept pair 2D int8 ops (scores) at the int8 peak and 2D bf16
# flops (P.V) at the bf16 peak, so 4D operations take 2D/INT8 + 2D/BF16 at best.
MIXED_PEAK_TOPS = 2.0 / (1.0 / INT8_PEAK_TOPS + 1.0 / BF16_PEAK_TFLOPS)
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X fp32 matrix (vendor figure)
# fp32 FMA on the vector ALUs without packed (two-wide) instructions, which the library is
# compiled without: 256 CUs x 4 SIMDs x 16 lanes x 2 FLOP x 2.4 GHz.
FP32_VALU_FMA_PEAK_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12


def effective_fine_flops(plan, keep_idx: np.ndarray, heads: int, head_dim: int,
                         ref: bool = False) -> float:
    """4*D * sum over heads and query tiles of rows_i * (real key rows it attends).
    Default mode: keep_idx [H][n_v][k], prefix tiles are sinks and prefix queries
    dense. Reference-sparsity mode: keep_idx [H][n_t][k_ref + k_gen], every list
    explicit."""
    bl = plan.block_len.astype(np.int64)
    if ref:
        kept = bl[keep_idx].sum(-1) if keep_idx.shape[-1] else np.zeros(keep_idx.shape[:2], np.int64)
        return 4.0 * head_dim * float((bl[None, :] * kept).sum())
    P = plan.P
    all_rows = int(bl.sum())
    prefix_rows = int(bl[:P].sum())
    pairs = heads * prefix_rows * all_rows
    kept = bl[keep_idx].sum(-1) if keep_idx.size else np.zeros((heads, plan.n_v), np.int64)
    pairs += int((bl[P:][None, :] * (prefix_rows + kept)).sum())
    return 4.0 * head_dim * float(pairs)


def hbm_passes(wl, plan, kernels, k, k_ref=None, chunks=1):
    """Achieved HBM bandwidth of the memory-bound passes from their algorithmic bytes:
    gather_pool reads Q, K, V once and writes the tile-ordered K, V and the three tile-mean
    arrays; top-k reads the coarse score rows and writes the keep lists; the merge of a
    split fine pass reads every chunk's partial of every (padded row, head) (D bf16 values
    and the fp32 max and sum), the gate and the O_coarse rows once, and writes the output."""
    H, D, S = wl.heads, wl.head_dim, wl.tokens
    S_pad, n_t, n_v, P = plan.S_pad, plan.n_t, plan.n_v, plan.P
    gather = 3 * S * H * D * 2 + 2 * S_pad * H * D * 2 + 3 * H * n_t * D * 4
    if k_ref is None:
        topk = H * n_v * n_v * 4 + H * n_v * k * 4
    else:
        topk = H * n_t * n_t * 4 + H * n_t * (k + k_ref) * 4
    merge = chunks * S_pad * H * (D * 2 + 8) + 2 * S * H * D * 2 + n_t * H * D * 4
    out = {}
    for name, nbytes in (("gather_pool", gather), ("topk", topk), ("merge", merge if chunks > 1 else 0)):
        if nbytes == 0:
            continue
        if name in kernels:
            gbs = nbytes / (kernels[name]["avg_ms"] * 1e-3) / 1e9
            out[name] = {"algorithmic_bytes": int(nbytes), "gb_s": round(gbs, 1),
                         "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
    return out


def compute_passes(wl, plan, kernels, k_ref=None):
    """Rates of the compute-bound side kernels against the peak of the unit each runs on:
    the gate GEMM (2 * hidden FLOP per output, bf16 MFMA), the coarse scores (2 * D FLOP per
    scored tile pair, fp32 FMA chains on the VALU) and the coarse attention (4 * D FLOP per
    (query tile, key tile) pair, fp32 MFMA)."""
    H, D, S = wl.heads, wl.head_dim, wl.tokens
    n = plan.n_t if k_ref is not None else plan.n_v
    work = {
        "gate_gemm": (2.0 * S * wl.hidden * H * D, BF16_PEAK_TFLOPS, "bf16 MFMA"),
        "video_scores": (2.0 * D * n * n * H, FP32_VALU_FMA_PEAK_TFLOPS, "fp32 VALU FMA"),
        "coarse_attn": (4.0 * D * plan.n_t * plan.n_t * H, FP32_MFMA_PEAK_TFLOPS, "fp32 MFMA"),
    }
    out = {}
    for name, (flops, peak, unit) in work.items():
        if name in kernels and flops > 0:
            tf = flops / (kernels[name]["avg_ms"] * 1e-3) / 1e12
            out[name] = {"algorithmic_tflop": round(flops / 1e12, 4), "tflop_s": round(tf, 2),
                         "peak": round(peak, 1), "unit": unit, "frac": round(tf / peak, 4)}
    return out


def selection_report(att, max_heads: int = 8) -> dict:
    """How non-uniform and how spatially coherent the coarse selection is (the
    default mode's video x video scores and keep lists), on up to max_heads spread
    heads, computed after the timed region:
      score_cv: per query tile, std / mean of its coarse softmax weights
        exp(scale (s_ij - max_j s_ij)) over the video key tiles, averaged over rows
        (0 for a uniform row);
      kept_weight: share of those weights on the kept tiles (k / n_v if uniform);
      adjacent_overlap: |keep(i) and keep(i+1)| / k for consecutive video query
        tiles i, i+1 (w-neighbours except at row ends), averaged; a random choice
        of k of n_v tiles gives k / n_v."""
    plan = att.plan
    n_v, P, k = plan.n_v, plan.P, att.k
    if att.ref or k == 0 or n_v < 2:
        return {}
    H, D = att.heads, att.head_dim
    scale = att.scale if att.scale > 0 else D ** -0.5
    sc = att.workspace_view("scores", torch.float32, (H, n_v, n_v))
    heads = sorted({int(h) for h in np.linspace(0, H - 1, min(H, max_heads)).round()})
    cv, kept, ovl = [], [], []
    for h in heads:
        s = sc[h].double()
        w = torch.exp(scale * (s - s.max(dim=1, keepdim=True).values))
        cv.append((w.std(dim=1) / w.mean(dim=1)).mean().item())
        keep = att.keep_idx[h].long() - P                       # [n_v][k] video tile ids
        kept.append((w.gather(1, keep).sum(1) / w.sum(1)).mean().item())
        mask = torch.zeros((n_v, n_v), dtype=torch.bool, device=s.device)
        mask.scatter_(1, keep, True)
        ovl.append(((mask[:-1] & mask[1:]).sum(1).double() / k).mean().item())
    return {"heads": heads, "score_cv": round(float(np.mean(cv)), 4),
            "kept_weight": round(float(np.mean(kept)), 4), "uniform_kept_weight": round(k / n_v, 4),
            "adjacent_overlap": round(float(np.mean(ovl)), 4), "random_overlap": round(k / n_v, 4)}


def cpu_baseline(wl, q, k, v, x, w, plan, kk, fine_flops, k_ref=None, int8=False):
    """The oracle, as it stands, on a bounded sample of this layer, scaled to one layer;
    when that estimate is at most FULL_CPU_LAYER_S the whole layer (every head and token)
    is run and timed instead. k_ref is not None in the reference-sparsity mode; int8
    times the INT8 fine pass."""
    import oracle
    Qb, Kb, Vb = (workloads.bf16_bits(t) for t in (q, k, v))
    xb, wb = workloads.bf16_bits(x), workloads.bf16_bits(w)
    pl = oracle.plan(wl.prefix_segments, wl.grid, wl.tile)
    scale = wl.head_dim ** -0.5

    def head(h):
        """Head h's coarse stage (pool, scores, top-k, O_coarse) and its fine pass."""
        if k_ref is None:
            hr = oracle.head(Qb, Kb, Vb, h, pl, kk, scale)

            def fine(toks):
                return oracle.fine_tokens(Qb, Kb, Vb, h, pl, hr.keep, kk, scale, toks)
        else:
            hr = oracle.head_ref(Qb, Kb, Vb, h, pl, k_ref, kk, scale)

            def fine(toks):
                return oracle.fine_tokens_lists(Qb, Kb, Vb, h, pl, hr.keep, scale, toks)
        if int8:
            csr = (oracle.key_lists_default(pl, hr.keep) if k_ref is None
                   else oracle.key_lists_explicit(hr.keep))

            def fine(toks):
                return oracle.fine_tokens_i8(Qb, Kb, Vb, h, pl, csr, scale, toks)
        return fine

    t0 = time.perf_counter()
    fine = head(0)
    t_head = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    vid_all = np.arange(pl.S)[pl.untile // pl.B >= pl.P]
    vid = rng.choice(vid_all, size=min(2048, vid_all.size), replace=False)
    pre = rng.choice(np.arange(pl.S)[pl.untile // pl.B < pl.P], size=min(256, wl.prefix_tokens),
                     replace=False) if wl.prefix_tokens else np.zeros(0, np.int64)
    t0 = time.perf_counter()
    fine(vid)
    t_vid = (time.perf_counter() - t0) / len(vid)
    t_pre = 0.0
    if len(pre):
        t0 = time.perf_counter()
        fine(pre)
        t_pre = (time.perf_counter() - t0) / len(pre)
    gt = rng.choice(pl.S, size=min(512, pl.S), replace=False)
    t0 = time.perf_counter()
    oracle.gate_proj(xb, wb, gt)
    t_gate = (time.perf_counter() - t0) / len(gt)
    n_video_tok = pl.S - wl.prefix_tokens
    layer_s = (wl.heads * (t_head + n_video_tok * t_vid + wl.prefix_tokens * t_pre)
               + pl.S * t_gate)
    sample = (f"head 0 of {wl.heads}: tile means, all coarse scores, top-k and O_coarse "
              f"({t_head:.2f} s); fine attention of {len(vid)} video and {len(pre)} prefix "
              f"query tokens; gate projection of {len(gt)} tokens; scaled to all heads "
              f"and tokens of one layer")
    if layer_s <= FULL_CPU_LAYER_S:
        toks = np.arange(pl.S)
        t0 = time.perf_counter()
        for h in range(wl.heads):
            head(h)(toks)
        oracle.gate_proj(xb, wb, toks)
        layer_s = time.perf_counter() - t0
        sample = (f"the whole layer: all {wl.heads} heads (coarse stage and the fine pass of all "
                  f"{pl.S} tokens) and the gate projection of every token")
    threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    return {
        "value": fine_flops / layer_s / 1e12,
        "unit": "TFLOP/s",
        "ms_per_layer": layer_s * 1e3,
        "cores": threads,
        "kind": "oracle",
        "sample": sample,
    }


FULL_CPU_LAYER_S = 20.0  # the oracle runs the whole layer when the sample scales to at most this

TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "fine_attn_pmc_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "tile_sparse_video_amd", "csrc", f)
                  for f in ("fine.hip", "device.h")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _median_ms(fn, reps=5, warm=3):
    for _ in range(warm):
        fn()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    return sorted(times)[len(times) // 2]


def library_gemm_8192(dev) -> dict:
    """hipBLASLt's rate (through torch.matmul) on a bf16 8192^3 GEMM on this machine: median of 5."""
    gen = torch.Generator(device="cpu").manual_seed(7)
    m = 8192
    A = torch.randn(m, m, generator=gen).to(torch.bfloat16).to(dev)
    B = torch.randn(m, m, generator=gen).to(torch.bfloat16).to(dev)
    ms = _median_ms(lambda: torch.matmul(A, B))
    del A, B
    return {"tflop": round(2 * m ** 3 / 1e12, 3), "ms": round(ms, 4), "tflop_s": round(2 * m ** 3 / ms / 1e9, 1)}


def ceilings() -> int:
    """What the box reaches with plain library operations, beside the vendor peaks used for
    the roofline fractions: a 2 GiB device copy (read + write bytes), a read-only sum over 2 GiB,
    and bf16 GEMMs through torch.matmul (hipBLASLt) on 8192^3 and on the H3-shaped gate
    projection (98,432 x 5,376 by 5,376 x 5,376, the weight transposed once beforehand).
    Each figure is the median of 5 timed repetitions after 3 warm-up ones."""
    if not torch.cuda.is_available():
        print("bench.py --ceilings needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    med_ms = _median_ms

    res = {"vendor_peaks": {"hbm_gb_s": HBM_PEAK_GBS, "bf16_mfma_tflop_s": BF16_PEAK_TFLOPS}}
    n = 2 << 30
    a = torch.ones(n // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    ms = med_ms(lambda: b.copy_(a))
    res["copy"] = {"bytes": 2 * n, "ms": round(ms, 4), "gb_s": round(2 * n / ms / 1e6, 1)}
    ms = med_ms(lambda: a.sum())
    res["read_sum"] = {"bytes": n, "ms": round(ms, 4), "gb_s": round(n / ms / 1e6, 1)}
    del a, b
    res["gemm_8192"] = library_gemm_8192(dev)
    gen = torch.Generator(device="cpu").manual_seed(7)
    S, hid, N = 98432, 5376, 5376
    x = torch.randn(S, hid, generator=gen).to(torch.bfloat16).to(dev)
    wt = torch.randn(N, hid, generator=gen).to(torch.bfloat16).to(dev).t().contiguous()
    ms = med_ms(lambda: torch.matmul(x, wt))
    res["gemm_gate_h3"] = {"tflop": round(2 * S * hid * N / 1e12, 3), "ms": round(ms, 4),
                           "tflop_s": round(2 * S * hid * N / ms / 1e9, 1)}
    print(json.dumps(res), flush=True)
    return 0


def recorded_traffic(workload: str):
    """HBM-side bytes per fine pass (fine kernel + merge) and the fine kernel's clock and
    MFMA-busy share, from the committed PMC summary; None when it was taken on another
    workload or on a kernel source that has changed since."""
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1)).get(workload)
    if not rec or rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec


def bench_backward(args, wl, tsv, att, qd, kd, vd, xd, wd, g, out, stream, host_inputs) -> int:
    """Training step of one layer: forward (gate projection, coarse, fine) then the
    backward pass; effective FLOPs = 4 D (forward) + 10 D (backward: S, dP, dV, dK,
    dQ) per kept (query row, key row) pair."""
    gen = torch.Generator().manual_seed(4242)
    dout = torch.randn(wl.tokens, wl.heads, wl.head_dim, generator=gen).to(torch.bfloat16).to(qd.device)
    grads = {}

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        tsv.vsa_gate_proj(xd, wd, g, stream=stream)
        att.coarse(qd, kd, vd, stream=stream)
        att.fine_train(qd, g, out, stream=stream)   # also saves lse and O_fine for the backward
        if ev is not None:
            ev[1].record(stream)
        grads["g"] = att.backward(qd, kd, vd, g, dout, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    print("[bench] warmup (training step)", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    tsv.vsa_timing_enable(True, stream)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tsv.vsa_timing_enable(False, stream)
    kernels = {}
    for name in tsv.TIMED_KERNELS:
        n, ms = tsv.vsa_timing_read(name, stream)
        if n:
            kernels[name] = {"launches": n, "avg_ms": round(ms / n, 4)}
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    layer_ms = float(evs[0][0].elapsed_time(evs[-1][2])) / args.steps
    keep_host = att.keep_idx.cpu().numpy()
    fwd_flops = effective_fine_flops(att.plan, keep_host, wl.heads, wl.head_dim, att.ref)
    bwd_flops = 2.5 * fwd_flops
    dkdv_flops = 2.0 * fwd_flops       # S, dP, dV, dK: 8 D per pair
    dkdv_ms = kernels["bwd_dkdv"]["avg_ms"]
    dkdv_tf = dkdv_flops / (dkdv_ms * 1e-3) / 1e12
    result = {
        "metric": "ms/layer fwd+bwd + effective TFLOP/s (fine: 4D fwd + 10D bwd per kept pair)",
        "value": round((fwd_flops + bwd_flops) / (layer_ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(layer_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.note}", "heads": wl.heads, "head_dim": wl.head_dim,
                   "tokens": wl.tokens, "keep_k": att.k,
                   "reference_sparsity": args.reference_sparsity,
                   "ref_keep_k": att.k_ref if att.ref else None, "mode": "training step",
                   "parallelism": "single GPU"},
        "breakdown_ms": {"forward": round(fwd_ms, 4), "backward": round(bwd_ms, 4)},
        "kernels": kernels,
        "effective_tflop": {"forward": round(fwd_flops / 1e12, 3),
                            "backward": round(bwd_flops / 1e12, 3)},
        "wall_s": round(wall, 3),
        "roofline": {
            "kernel": "dkdv_kernel (vsa_sparse_attn_bwd)", "bound": "mfma",
            "achieved": round(dkdv_tf, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(dkdv_tf / BF16_PEAK_TFLOPS, 4),
            "algorithmic_tflop_per_launch": round(dkdv_flops / 1e12, 4),
            "avg_launch_ms": dkdv_ms, "traffic": None,
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_backward(wl, host_inputs, att, dout, g,
                                                        fwd_flops + bwd_flops)
    print(json.dumps(result), flush=True)
    return 0


def bench_producer(args, wl, tsv, att, xd, stream) -> int:
    """The layer from its input x. Fused: vsa_qkv_gate_proj (q, gate natural; K/V tiled
    with the tile means) + vsa_coarse_topk without the gather + the fine pass. Unfused:
    four vsa_gate_proj calls (q, k, v, gate) + vsa_coarse_topk with its gather + the fine
    pass. Same arithmetic, identical outputs (checked here on the last step)."""
    dev = xd.device
    S, H, D = wl.tokens, wl.heads, wl.head_dim
    w4 = workloads.make_w_qkvg(wl).to(dev)
    w_parts = [w4[i].contiguous() for i in range(4)]
    qp = torch.empty((S, H, D), dtype=torch.bfloat16, device=dev)
    gp = torch.empty((S, H * D), dtype=torch.bfloat16, device=dev)
    out_f = torch.empty_like(qp)
    out_u = torch.empty_like(qp)
    proj = [torch.empty((S, H * D), dtype=torch.bfloat16, device=dev) for _ in range(4)]

    def fused(ev=None):
        if ev is not None:
            ev[0].record(stream)
        att.project(xd, w4, qp, gp, stream=stream)
        att.coarse(None, None, None, stream=stream)
        att.fine(qp, gp, out_f, stream=stream)
        if ev is not None:
            ev[1].record(stream)

    def unfused(ev=None):
        if ev is not None:
            ev[0].record(stream)
        for i in range(4):
            tsv.vsa_gate_proj(xd, w_parts[i], proj[i], stream=stream)
        att.coarse(*(t.view(S, H, D) for t in proj[:3]), stream=stream)
        att.fine(proj[0].view(S, H, D), proj[3], out_u, stream=stream)
        if ev is not None:
            ev[1].record(stream)

    res = {}
    for name, fn in (("fused", fused), ("unfused", unfused)):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        tsv.vsa_timing_enable(True, stream)
        for i in range(args.steps):
            fn(evs[i])
        torch.cuda.synchronize()
        tsv.vsa_timing_enable(False, stream)
        kernels = {}
        for kname in tsv.TIMED_KERNELS:
            n, ms = tsv.vsa_timing_read(kname, stream)
            if n:
                kernels[kname] = {"launches": n, "avg_ms": round(ms / n, 4)}
        res[name] = {"ms_per_layer": round(float(np.mean([e[0].elapsed_time(e[1]) for e in evs])), 4),
                     "kernels": kernels}
    identical = bool(torch.equal(out_f.view(torch.int16), out_u.view(torch.int16)))
    keep_host = att.keep_idx.cpu().numpy()
    fine_flops = effective_fine_flops(att.plan, keep_host, H, D, att.ref)
    proj_flops = 2.0 * S * wl.hidden * 4 * H * D
    layer_ms = res["fused"]["ms_per_layer"]
    qkv_ms = res["fused"]["kernels"]["qkv_proj"]["avg_ms"]
    result = {
        "metric": "ms/layer from the layer input (fused q/k/v/gate producer + coarse + fine)",
        "value": round(layer_ms, 4), "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(layer_ms, 4), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.note}", "heads": H, "head_dim": D,
                   "hidden": wl.hidden, "tokens": S, "keep_k": att.k, "mode": "from x (producer)",
                   "split_chunks": att.split_chunks, "parallelism": "single GPU"},
        "fused": res["fused"], "unfused": res["unfused"],
        "outputs_identical": identical,
        "saved_ms": round(res["unfused"]["ms_per_layer"] - layer_ms, 4),
        "effective_fine_tflop": round(fine_flops / 1e12, 3),
        "projection_tflop": round(proj_flops / 1e12, 3),
        "roofline": {"kernel": "qkv_gemm_kernel (vsa_qkv_gate_proj)", "bound": "mfma",
                     "achieved": round(proj_flops / (qkv_ms * 1e-3) / 1e12, 2),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(proj_flops / (qkv_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                     "algorithmic_tflop_per_launch": round(proj_flops / 1e12, 4),
                     "avg_launch_ms": qkv_ms, "traffic": None},
    }
    print(json.dumps(result), flush=True)
    return 0 if identical else 1


def cpu_baseline_backward(wl, host_inputs, att, dout, g, flops):
    """The oracle's backward on a bounded sample: dq of sampled tokens of head 0
    (each token's own keys plus its tile's coarse row), scaled by 3 (dk and dv
    cost the same per pair) to all tokens and heads."""
    import oracle
    q, k, v, x, w = host_inputs
    Qb, Kb, Vb = (workloads.bf16_bits(t) for t in (q, k, v))
    pl = oracle.plan(wl.prefix_segments, wl.grid, wl.tile)
    scale = wl.head_dim ** -0.5
    if att.ref:
        hr = oracle.head_ref(Qb, Kb, Vb, 0, pl, att.k_ref, att.k, scale)
        csr = oracle.key_lists_explicit(hr.keep)
    else:
        hr = oracle.head(Qb, Kb, Vb, 0, pl, att.k, scale)
        csr = oracle.key_lists_default(pl, hr.keep)
    g_bits = workloads.bf16_bits(g.cpu())
    d_bits = workloads.bf16_bits(dout.cpu())
    toks = np.random.default_rng(0).choice(pl.S, size=min(512, pl.S), replace=False)
    t0 = time.perf_counter()
    oracle.dq_tokens(Qb, Kb, Vb, g_bits, d_bits, 0, pl, csr, scale, toks,
                     means=(hr.qm, hr.km, hr.vm))
    per_tok = (time.perf_counter() - t0) / len(toks)
    layer_s = 3.0 * per_tok * pl.S * wl.heads
    threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    return {"value": flops / layer_s / 1e12, "unit": "TFLOP/s", "ms_per_layer": layer_s * 1e3,
            "cores": threads, "kind": "oracle",
            "sample": f"dq of {len(toks)} tokens of head 0 ({per_tok * 1e3:.2f} ms per token), "
                      f"times 3 for dk and dv, scaled to all tokens and heads (backward only)"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="h3", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--reference-sparsity", type=float, default=None, metavar="S",
                    help="run the reference-sparsity mode: every query tile keeps the top "
                         "(1-S) of the prefix tiles as well as the top video tiles")
    ap.add_argument("--int8", action="store_true",
                    help="run the fine pass with INT8 scores (vsa_sparse_attn_fwd_i8)")
    ap.add_argument("--backward", action="store_true",
                    help="time the layer's training step instead: forward plus the backward "
                         "pass (gradients of q, k, v and the gate)")
    ap.add_argument("--producer", action="store_true",
                    help="run the layer from its input x: one chunked-producer GEMM for q, k, "
                         "v and the gate (vsa_qkv_gate_proj, K/V written in tile order with the "
                         "tile means), the coarse stage without its gather, the fine pass; "
                         "timed beside the same layer with four vsa_gate_proj calls and the "
                         "gather")
    ap.add_argument("--split-chunks", type=int, default=0,
                    help="fine-pass key-list split (0 = the library's automatic choice)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB mebibytes (3 times), to scale "
                         "the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--ceilings", action="store_true",
                    help="only measure what the box reaches with plain library operations (a "
                         "device copy, a read-only reduction, bf16 GEMMs through torch.matmul) "
                         "and print it as one JSON line, beside the vendor peaks the roofline uses")
    args = ap.parse_args()
    if args.ceilings:
        return ceilings()
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)
        return 0
    if args.int8 and args.backward:
        print("--int8 times the forward only; the backward pass is bf16", file=sys.stderr)
        return 2
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the library runs "
              "on one GPU (the layer would shard by head with no exchange)", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2

    import tile_sparse_video_amd as tsv

    wl = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {wl.name} inputs ({wl.tokens} tokens)", file=sys.stderr, flush=True)
    q, k, v = workloads.make_qkv(wl)
    x, w = workloads.make_x(wl), workloads.make_w_gate(wl)
    qd, kd, vd, xd, wd = (t.to(dev) for t in (q, k, v, x, w))
    att = tsv.TileSparseAttention(wl.prefix_segments, wl.grid, wl.tile, wl.heads, wl.head_dim,
                                  sparsity=wl.sparsity, keep_k=wl.keep_k, device=dev,
                                  reference_sparsity=args.reference_sparsity, int8=args.int8,
                                  split_chunks=args.split_chunks)
    g = torch.empty((wl.tokens, wl.heads * wl.head_dim), dtype=torch.bfloat16, device=dev)
    out = torch.empty_like(qd)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        tsv.vsa_gate_proj(xd, wd, g, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        att.coarse(qd, kd, vd, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        att.fine(qd, g, out, stream=stream)
        if ev is not None:
            ev[3].record(stream)

    if args.backward:
        return bench_backward(args, wl, tsv, att, qd, kd, vd, xd, wd, g, out, stream,
                              (q, k, v, x, w))
    if args.producer:
        return bench_producer(args, wl, tsv, att, xd, stream)

    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    tsv.vsa_timing_enable(True, stream)     # per-kernel events on the library's launch stream
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tsv.vsa_timing_enable(False, stream)
    kernels = {}
    for name in tsv.TIMED_KERNELS:
        n, ms = tsv.vsa_timing_read(name, stream)
        if n:
            kernels[name] = {"launches": n, "avg_ms": round(ms / n, 4)}
    parts = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(3)]
                      for i in range(args.steps)])
    layer_ms = float(evs[0][0].elapsed_time(evs[-1][3])) / args.steps
    gate_ms, coarse_ms, fine_ms = (float(x) for x in parts.mean(0))

    keep_host = att.keep_idx.cpu().numpy()
    fine_flops = effective_fine_flops(att.plan, keep_host, wl.heads, wl.head_dim, att.ref)
    tflops = fine_flops / (layer_ms * 1e-3) / 1e12
    fine_kernel_ms = kernels["fine_attn"]["avg_ms"]
    fine_tflops = fine_flops / (fine_kernel_ms * 1e-3) / 1e12
    # The fine pass is the fine kernel plus, when the key lists are split, the merge
    # of the chunk partials: both are vsa_sparse_attn_fwd's work.
    merge_ms = kernels.get("merge", {}).get("avg_ms", 0.0)
    pass_ms = fine_kernel_ms + merge_ms
    pass_tflops = fine_flops / (pass_ms * 1e-3) / 1e12
    traffic = None if (att.ref or args.int8) else recorded_traffic(wl.name)
    peak = MIXED_PEAK_TOPS if args.int8 else BF16_PEAK_TFLOPS
    frac_pairs = att.tile_pair_fraction()

    result = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(layer_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 scores, bf16 P.V" if args.int8 else "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: {wl.note}",
            "int8": args.int8,
            "heads": wl.heads, "head_dim": wl.head_dim, "hidden": wl.hidden,
            "tokens": wl.tokens, "prefix_segments": list(wl.prefix_segments),
            "grid": list(wl.grid), "tile": list(wl.tile), "keep_k": att.k,
            "reference_sparsity": args.reference_sparsity,
            "ref_keep_k": att.k_ref if att.ref else None,
            "split_chunks": att.split_chunks,
            "parallelism": "single GPU",
        },
        "ms_per_layer": round(layer_ms, 4),
        "pct_bf16_peak": round(100 * tflops / BF16_PEAK_TFLOPS, 2),
        "breakdown_ms": {"gate_proj": round(gate_ms, 4), "coarse_topk": round(coarse_ms, 4),
                         "sparse_attn_fwd": round(fine_ms, 4)},
        "kernels": kernels,
        "ms_per_layer_attention_only": round(coarse_ms + fine_ms, 4),
        "tile_pair_fraction": round(frac_pairs, 4),
        "effective_fine_tflop": round(fine_flops / 1e12, 3),
        "hbm_passes": hbm_passes(wl, att.plan, kernels, att.k, att.k_ref if att.ref else None,
                                 att.split_chunks),
        "compute_passes": compute_passes(wl, att.plan, kernels, att.k_ref if att.ref else None),
        "wall_s": round(wall, 3),
        "selection": selection_report(att),
        "roofline": {
            "kernel": ("fine_attn_kernel + merge_kernel, INT8 scores (vsa_sparse_attn_fwd_i8; peak "
                       "mixes the int8 and bf16 MFMA peaks per kept pair)" if args.int8 else
                       "fine_attn_kernel + merge_kernel (the fine pass, vsa_sparse_attn_fwd)"),
            "bound": "mfma",
            "achieved": round(pass_tflops, 2),
            "peak": round(peak, 1),
            "unit": "TOP/s" if args.int8 else "TFLOP/s",
            "frac": round(pass_tflops / peak, 4),
            "algorithmic_tflop_per_launch": round(fine_flops / 1e12, 4),
            "avg_launch_ms": round(pass_ms, 4),
            "fine_kernel_alone": {"avg_launch_ms": fine_kernel_ms, "achieved": round(fine_tflops, 2),
                                  "frac": round(fine_tflops / peak, 4)},
            "split_chunks": att.split_chunks,
            "traffic": None if traffic is None else traffic["bytes_per_launch"],
            "mfma_busy": None if traffic is None else traffic.get("mfma_busy"),
            "clock_ghz": None if traffic is None else traffic.get("clock_ghz"),
            "traffic_detail": traffic,
        },
    }
    if not args.int8:
        # Context beside the vendor peak, measured after the timed region: what the vendor
        # library reaches on a plain bf16 GEMM on this machine, and the fine kernel against it.
        lib = library_gemm_8192(dev)
        lib["what"] = "hipBLASLt bf16 GEMM 8192^3 through torch.matmul, median of 5, after the timed layers"
        lib["fine_kernel_over_it"] = round(fine_tflops / lib["tflop_s"], 4)
        result["roofline"]["library_gemm"] = lib
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle sample)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, q, k, v, x, w, att.plan, att.k, fine_flops,
                                              att.k_ref if att.ref else None, args.int8)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
