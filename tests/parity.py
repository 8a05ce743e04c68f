"""Shared machinery for the GPU-vs-oracle parity tests.

Both sides take the same seeded inputs (workloads); the HIP side runs through
the C ABI via the binding, the oracle side through oracle/. Neither side's
output feeds the other: each computes its own plan, keep-sets and gate.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, List, Optional

import numpy as np
import torch

import oracle
import workloads

# Output tolerance: max-abs 2e-2 and relative L2 1e-2 against the oracle's fp64
# result (the method's stated bar for bf16 outputs).
MAX_ABS = 2e-2
REL_L2 = 1e-2


def bf16_ulp(x) -> np.ndarray:
    """Spacing of bf16 numbers at |x|: 2^(e - 7) for |x| in [2^e, 2^(e + 1)) (8
    significant bits), 2^-133 below the normal range."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(e - 7)


def output_bar(got, ref) -> np.ndarray:
    """Per-element bar for bf16 layer outputs against the oracle's bf16 result:
    max-abs 2e-2, except where one bf16 step of the value is larger (|value| >= 4,
    one step = 2^-5 or more): there the two roundings of nearly equal fp32 and fp64
    results may land one step apart, so one step is the bar."""
    return np.maximum(MAX_ABS, bf16_ulp(ref))


def check_output(got, ref, what: str = "") -> tuple:
    """Asserts the output bar element-wise and rel-L2 <= 1e-2; returns (max-abs, rel-L2)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    mx, rl = float(err.max()) if err.size else 0.0, rel_l2(got, ref)
    bad = err > output_bar(got, ref)
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond the bar, worst "
                           f"{float(err[bad].max())} at |ref| {float(np.abs(ref[bad]).max())}")
    assert rl <= REL_L2, f"{what}: rel-L2 {rl}"
    return mx, rl


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def bits(t: torch.Tensor) -> np.ndarray:
    return workloads.bf16_bits(t.detach().cpu().contiguous())


@dataclass
class Inputs:
    wl: workloads.Workload
    q: torch.Tensor   # bf16 CPU [S][H][D]
    k: torch.Tensor
    v: torch.Tensor
    x: torch.Tensor   # bf16 CPU [S][hidden]
    w: torch.Tensor   # bf16 CPU [H*D][hidden]

    @property
    def qb(self):
        return bits(self.q)

    @property
    def kb(self):
        return bits(self.k)

    @property
    def vb(self):
        return bits(self.v)


def make_inputs(wl: workloads.Workload) -> Inputs:
    q, k, v = workloads.make_qkv(wl)
    return Inputs(wl, q, k, v, workloads.make_x(wl), workloads.make_w_gate(wl))


@dataclass
class GpuRun:
    att: object           # tile_sparse_video_amd.TileSparseAttention
    out: torch.Tensor     # device bf16 [S][H][D]
    g: torch.Tensor       # device bf16 [S][H*D]


def run_gpu(inp: Inputs, gate: Optional[torch.Tensor] = None, dev="cuda",
            split_chunks: int = 0) -> GpuRun:
    import tile_sparse_video_amd as tsv
    wl = inp.wl
    att = tsv.TileSparseAttention(wl.prefix_segments, wl.grid, wl.tile, wl.heads, wl.head_dim,
                                  sparsity=wl.sparsity, keep_k=wl.keep_k, device=dev,
                                  split_chunks=split_chunks)
    qd, kd, vd = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    if gate is None:
        xd, wd = inp.x.to(dev), inp.w.to(dev)
        g = torch.empty((wl.tokens, wl.heads * wl.head_dim), dtype=torch.bfloat16, device=dev)
        tsv.vsa_gate_proj(xd, wd, g)
        del xd, wd
    else:
        g = gate.to(dev)
    out = att(qd, kd, vd, g)
    torch.cuda.synchronize()
    return GpuRun(att, out, g)


@dataclass
class OracleHead:
    hr: oracle.HeadResult
    h: int


def oracle_plan(wl):
    return oracle.plan(wl.prefix_segments, wl.grid, wl.tile)


def oracle_k(wl, pl):
    return oracle.keep_count(pl.n_v, wl.sparsity, wl.keep_k)


def unswizzle_k(frags: np.ndarray, D: int) -> np.ndarray:
    """K fragments of one 64-row block ([D/8][64][8] uint16) -> [64][D]."""
    out = np.empty((64, D), dtype=np.uint16)
    for f in range(D // 8):
        kb, c = divmod(f, D // 16)
        for lane in range(64):
            row = 32 * kb + lane % 32
            d0 = 16 * c + 8 * (lane // 32)
            out[row, d0:d0 + 8] = frags[f, lane]
    return out


def unswizzle_v(frags: np.ndarray, D: int) -> np.ndarray:
    """V fragments of one 64-row block ([D/8][64][8] uint16) -> [64][D]."""
    out = np.empty((64, D), dtype=np.uint16)
    for f in range(D // 8):
        db, c = divmod(f, 4)
        for lane in range(64):
            d = 32 * db + lane % 32
            h4 = 4 * (lane // 32)
            rows = [16 * c + h4 + e for e in range(4)] + [16 * c + 8 + h4 + e for e in range(4)]
            out[rows, d] = frags[f, lane]
    return out


def sample_tokens(pl, n: int, seed: int) -> np.ndarray:
    """Tokens to check one by one: first/last of every prefix tile, edge-tile tokens, random rest."""
    rng = np.random.default_rng(seed)
    picks = set()
    for t in range(pl.n_t):
        rows = pl.row_src[t * pl.B: t * pl.B + pl.block_len[t]]
        if t < pl.P or pl.block_len[t] < pl.B:
            picks.add(int(rows[0]))
            picks.add(int(rows[-1]))
    picks = sorted(picks)
    if len(picks) > n // 2:
        picks = list(rng.choice(picks, size=n // 2, replace=False))
    rest = rng.choice(pl.S, size=max(0, n - len(picks)), replace=False)
    return np.unique(np.concatenate([np.asarray(picks, dtype=np.int64), rest.astype(np.int64)]))


def run_gpu_ref(inp: Inputs, ref_sparsity=None, ref_keep_k=None, gate: Optional[torch.Tensor] = None,
                dev="cuda", split_chunks: int = 0) -> GpuRun:
    """The layer in the reference-sparsity mode (every query tile keeps k_ref
    prefix tiles and k_gen video tiles)."""
    import tile_sparse_video_amd as tsv
    wl = inp.wl
    att = tsv.TileSparseAttention(wl.prefix_segments, wl.grid, wl.tile, wl.heads, wl.head_dim,
                                  sparsity=wl.sparsity, keep_k=wl.keep_k, device=dev,
                                  reference_sparsity=ref_sparsity, ref_keep_k=ref_keep_k,
                                  split_chunks=split_chunks)
    qd, kd, vd = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    if gate is None:
        xd, wd = inp.x.to(dev), inp.w.to(dev)
        g = torch.empty((wl.tokens, wl.heads * wl.head_dim), dtype=torch.bfloat16, device=dev)
        tsv.vsa_gate_proj(xd, wd, g)
        del xd, wd
    else:
        g = gate.to(dev)
    out = att(qd, kd, vd, g)
    torch.cuda.synchronize()
    return GpuRun(att, out, g)
