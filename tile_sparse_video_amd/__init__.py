"""Gated, tile-sparse video attention for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libvsa.so`` (hand-written HIP kernels behind the
C ABI in ``include/vsa.h``). Functions carry the C names; this module only
marshals arguments: every step of the computation runs in the library's
kernels. PyTorch supplies device memory and streams.

There is no fallback: if ``libvsa.so`` is missing, importing this package
raises. Build it with ``python tile_sparse_video_amd/build.py`` (or
``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# VSA_LIBRARY names another build of the same library (the host-sanitizer build
# of build.py --sanitize); by default the in-tree libvsa.so.
LIB_PATH = os.environ.get("VSA_LIBRARY") or os.path.join(_HERE, "libvsa.so")

VSA_OK = 0
VSA_ERR_ARG = -1
VSA_ERR_UNSUPPORTED = -2
VSA_ERR_PLAN = -3
VSA_ERR_DEVICE = -4

EXPORTED = (
    "vsa_status_string", "vsa_last_error", "vsa_plan_tiles", "vsa_plan_validate",
    "vsa_keep_count", "vsa_tile_pair_fraction", "vsa_workspace_layout", "vsa_coarse_topk",
    "vsa_sparse_attn_fwd", "vsa_gate_proj", "vsa_timing_enable",
    "vsa_timing_read", "vsa_ref_keep_count", "vsa_tile_pair_fraction_ref", "vsa_coarse_topk_ref",
    "vsa_sparse_attn_fwd_ref", "vsa_bwd_workspace_layout", "vsa_sparse_attn_bwd",
    "vsa_sparse_attn_fwd_i8", "vsa_layer_fwd_groups", "vsa_sparse_attn_fwd_train",
    "vsa_layer_fwd_static", "vsa_qkv_gate_proj",
)
# Size of the library's static workspace (vsa_layer_fwd_static), as vsa.h defines it.
STATIC_WORKSPACE_BYTES = 64 << 20
TIMED_KERNELS = ("gate_gemm", "gather_pool", "video_scores", "coarse_attn", "topk", "fine_attn",
                 "merge", "bwd_gather", "bwd_prep", "bwd_coarse", "bwd_tlist", "bwd_dq", "bwd_dkdv",
                 "bwd_stats", "quant_k", "qkv_proj")


class VsaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {detail} (status {status})")
        self.status = status


class vsa_plan_info(ctypes.Structure):
    _fields_ = [
        ("grid", ctypes.c_int32 * 3), ("tile", ctypes.c_int32 * 3), ("tile_rows", ctypes.c_int32),
        ("n_prefix_tiles", ctypes.c_int32), ("n_video_tiles", ctypes.c_int32),
        ("n_tiles", ctypes.c_int32), ("rows_real", ctypes.c_int64),
        ("rows_padded", ctypes.c_int64), ("prefix_rows", ctypes.c_int64),
    ]


class vsa_ws_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("k_tiled", "v_tiled", "q_mean", "k_mean", "v_mean", "scores", "k_i8",
                 "k_scale", "part_o", "part_ml", "total_bytes")] + [("split_chunks", ctypes.c_int32)]


class vsa_head_group(ctypes.Structure):
    _fields_ = [
        ("info", ctypes.POINTER(vsa_plan_info)), ("row_src_dev", ctypes.c_void_p),
        ("block_len_dev", ctypes.c_void_p), ("head_first", ctypes.c_int32),
        ("heads", ctypes.c_int32), ("sparsity", ctypes.c_double), ("keep_k", ctypes.c_int64),
        ("ref", ctypes.c_int32), ("int8", ctypes.c_int32), ("ref_sparsity", ctypes.c_double),
        ("ref_keep_k", ctypes.c_int64), ("split_chunks", ctypes.c_int32), ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t), ("keep_idx_dev", ctypes.c_void_p),
        ("o_coarse_dev", ctypes.c_void_p),
    ]


class vsa_bwd_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("vrow", "kcol", "qcol", "docol", "qrow", "dorow", "lse", "dt", "doc", "dqm", "dkm",
                 "dvm", "lsec", "dcc", "tlist", "tcount", "tbits", "part_dq", "part_dkv", "ofine",
                 "total_bytes")] + [("split_chunks", ctypes.c_int32)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run tile_sparse_video_amd/build.py "
                          "(the HIP library is required: there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F32, F64, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                 ctypes.c_double, ctypes.c_size_t)
    info_p = ctypes.POINTER(vsa_plan_info)
    sig = {
        "vsa_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "vsa_last_error": ([], ctypes.c_char_p),
        "vsa_plan_tiles": ([P, I32, I32, I32, I32, I32, I32, I32, info_p, P, P, P], ctypes.c_int),
        "vsa_plan_validate": ([info_p, P, I32, P, P, P], ctypes.c_int),
        "vsa_keep_count": ([info_p, F64, I64, ctypes.POINTER(I32)], ctypes.c_int),
        "vsa_tile_pair_fraction": ([info_p, I32, ctypes.POINTER(F64)], ctypes.c_int),
        "vsa_workspace_layout": ([info_p, I32, I32, I32, ctypes.POINTER(vsa_ws_layout)], ctypes.c_int),
        "vsa_coarse_topk": ([info_p, P, P, I32, I32, F64, I64, F32, P, P, P, P, SZ, P, P, P],
                            ctypes.c_int),
        "vsa_sparse_attn_fwd": ([info_p, P, P, I32, I32, I32, F32, I32, P, P, SZ, P, P, P, P, P],
                                ctypes.c_int),
        "vsa_gate_proj": ([P, P, I64, I32, I32, P, P], ctypes.c_int),
        "vsa_ref_keep_count": ([info_p, F64, I64, ctypes.POINTER(I32)], ctypes.c_int),
        "vsa_tile_pair_fraction_ref": ([info_p, I32, I32, ctypes.POINTER(F64)], ctypes.c_int),
        "vsa_coarse_topk_ref": ([info_p, P, P, I32, I32, F64, I64, F64, I64, F32, P, P, P, P, SZ,
                                 P, P, P], ctypes.c_int),
        "vsa_sparse_attn_fwd_ref": ([info_p, P, P, I32, I32, I32, I32, F32, I32, P, P, SZ, P, P, P,
                                     P, P], ctypes.c_int),
        "vsa_sparse_attn_fwd_i8": ([info_p, P, P, I32, I32, I32, I32, F32, I32, P, P, SZ, P, P, P,
                                    P, P], ctypes.c_int),
        "vsa_layer_fwd_groups": ([ctypes.POINTER(vsa_head_group), I32, I32, I32, F32, P, P, P, P,
                                  P, P], ctypes.c_int),
        "vsa_bwd_workspace_layout": ([info_p, I32, I32, I32, ctypes.POINTER(vsa_bwd_layout)],
                                     ctypes.c_int),
        "vsa_sparse_attn_bwd": ([info_p, P, P, I32, I32, I32, I32, F32, I32, P, P, P, P, P, P, SZ, P,
                                 P, P, SZ, P, P, P, P, I32, P], ctypes.c_int),
        "vsa_sparse_attn_fwd_train": ([info_p, P, P, I32, I32, I32, I32, F32, I32, P, P, SZ, P, P,
                                       P, P, P, SZ, P], ctypes.c_int),
        "vsa_layer_fwd_static": ([info_p, P, P, I32, I32, F64, I64, F32, P, P, P, P, P, P, P, P],
                                 ctypes.c_int),
        "vsa_qkv_gate_proj": ([info_p, P, P, I32, I32, I32, P, P, P, P, P, SZ, P], ctypes.c_int),
        "vsa_timing_enable": ([P, I32], ctypes.c_int),
        "vsa_timing_read": ([P, ctypes.c_char_p, ctypes.POINTER(I32), ctypes.POINTER(F64)],
                            ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()


def _check(status: int, where: str) -> None:
    if status != VSA_OK:
        raise VsaError(status, where, _lib.vsa_last_error().decode() or
                       _lib.vsa_status_string(status).decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# ------------------------------------------------------------------ plan --

@dataclass
class Plan:
    """Host plan (vsa_plan_tiles) plus the arguments it was built from."""
    info: vsa_plan_info
    prefix_segments: tuple
    untile: np.ndarray      # int32 [S]
    row_src: np.ndarray     # int32 [S_pad], -1 = padding
    block_len: np.ndarray   # int32 [n_t]

    @property
    def P(self) -> int:
        return self.info.n_prefix_tiles

    @property
    def n_v(self) -> int:
        return self.info.n_video_tiles

    @property
    def n_t(self) -> int:
        return self.info.n_tiles

    @property
    def B(self) -> int:
        return self.info.tile_rows

    @property
    def S(self) -> int:
        return self.info.rows_real

    @property
    def S_pad(self) -> int:
        return self.info.rows_padded


def _segs(prefix_segments: Sequence[int]) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(list(prefix_segments), dtype=np.int64).reshape(-1))


def vsa_plan_tiles(prefix_segments: Sequence[int], grid: Sequence[int], tile: Sequence[int]) -> Plan:
    segs = _segs(prefix_segments)
    info = vsa_plan_info()
    seg_p = segs.ctypes.data if segs.size else None
    _check(_lib.vsa_plan_tiles(seg_p, segs.size, *map(int, grid), *map(int, tile),
                               ctypes.byref(info), None, None, None), "vsa_plan_tiles")
    untile = np.empty(info.rows_real, dtype=np.int32)
    row_src = np.empty(info.rows_padded, dtype=np.int32)
    block_len = np.empty(info.n_tiles, dtype=np.int32)
    _check(_lib.vsa_plan_tiles(seg_p, segs.size, *map(int, grid), *map(int, tile),
                               ctypes.byref(info), untile.ctypes.data, row_src.ctypes.data,
                               block_len.ctypes.data), "vsa_plan_tiles")
    return Plan(info, tuple(int(s) for s in segs), untile, row_src, block_len)


def vsa_plan_validate(plan: Plan, untile=None, row_src=None, block_len=None) -> None:
    segs = _segs(plan.prefix_segments)
    u = np.ascontiguousarray(plan.untile if untile is None else untile, dtype=np.int32)
    r = np.ascontiguousarray(plan.row_src if row_src is None else row_src, dtype=np.int32)
    b = np.ascontiguousarray(plan.block_len if block_len is None else block_len, dtype=np.int32)
    _check(_lib.vsa_plan_validate(ctypes.byref(plan.info), segs.ctypes.data if segs.size else None,
                                  segs.size, u.ctypes.data, r.ctypes.data, b.ctypes.data),
           "vsa_plan_validate")


def vsa_keep_count(info: vsa_plan_info, sparsity: Optional[float] = None,
                   keep_k: Optional[int] = None) -> int:
    k = ctypes.c_int32(0)
    _check(_lib.vsa_keep_count(ctypes.byref(info), float("nan") if sparsity is None else float(sparsity),
                               -1 if keep_k is None else int(keep_k), ctypes.byref(k)),
           "vsa_keep_count")
    return int(k.value)


def vsa_tile_pair_fraction(info: vsa_plan_info, k: int) -> float:
    f = ctypes.c_double(0)
    _check(_lib.vsa_tile_pair_fraction(ctypes.byref(info), int(k), ctypes.byref(f)),
           "vsa_tile_pair_fraction")
    return float(f.value)


def vsa_ref_keep_count(info: vsa_plan_info, ref_sparsity: Optional[float] = None,
                       ref_keep_k: Optional[int] = None) -> int:
    """Kept prefix (reference) tiles per query tile in the reference-sparsity mode."""
    k = ctypes.c_int32(0)
    _check(_lib.vsa_ref_keep_count(ctypes.byref(info),
                                   float("nan") if ref_sparsity is None else float(ref_sparsity),
                                   -1 if ref_keep_k is None else int(ref_keep_k), ctypes.byref(k)),
           "vsa_ref_keep_count")
    return int(k.value)


def vsa_tile_pair_fraction_ref(info: vsa_plan_info, k_ref: int, k_gen: int) -> float:
    f = ctypes.c_double(0)
    _check(_lib.vsa_tile_pair_fraction_ref(ctypes.byref(info), int(k_ref), int(k_gen),
                                           ctypes.byref(f)), "vsa_tile_pair_fraction_ref")
    return float(f.value)


def vsa_workspace_layout(info: vsa_plan_info, heads: int, head_dim: int,
                         split_chunks: int = 0) -> vsa_ws_layout:
    """Workspace regions for `split_chunks` fine-pass key chunks (0 = automatic)."""
    lay = vsa_ws_layout()
    _check(_lib.vsa_workspace_layout(ctypes.byref(info), int(heads), int(head_dim), int(split_chunks),
                                     ctypes.byref(lay)), "vsa_workspace_layout")
    return lay


# ------------------------------------------------------------ GPU calls --

def _need(t: torch.Tensor, name: str, dtype, shape=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def vsa_coarse_topk(info: vsa_plan_info, row_src_dev: torch.Tensor, block_len_dev: torch.Tensor,
                    heads: int, head_dim: int, q: Optional[torch.Tensor], k: Optional[torch.Tensor],
                    v: Optional[torch.Tensor], workspace: torch.Tensor,
                    keep_idx: Optional[torch.Tensor], o_coarse: torch.Tensor,
                    sparsity: Optional[float] = None, keep_k: Optional[int] = None,
                    scale: float = 0.0, stream=None) -> None:
    """q = k = v = None: the workspace already holds the tiled K/V and the tile means
    (vsa_qkv_gate_proj), and the gather is skipped."""
    S = info.rows_real
    if (q is None) != (k is None) or (q is None) != (v is None):
        raise ValueError("pass q, k and v, or none of them")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if t is not None:
            _need(t, n, torch.bfloat16, (S, heads, head_dim))
    _need(row_src_dev, "row_src", torch.int32, (info.rows_padded,))
    _need(block_len_dev, "block_len", torch.int32, (info.n_tiles,))
    _need(workspace, "workspace", torch.uint8)
    _need(o_coarse, "o_coarse", torch.float32, (heads, info.n_tiles, head_dim))
    if keep_idx is not None:
        _need(keep_idx, "keep_idx", torch.int32)
    _check(_lib.vsa_coarse_topk(ctypes.byref(info), _ptr(row_src_dev), _ptr(block_len_dev), heads,
                                head_dim, float("nan") if sparsity is None else float(sparsity),
                                -1 if keep_k is None else int(keep_k), float(scale), _ptr(q),
                                _ptr(k), _ptr(v), _ptr(workspace), workspace.numel(),
                                _ptr(keep_idx), _ptr(o_coarse), _stream(stream)),
           "vsa_coarse_topk")


def vsa_sparse_attn_fwd(info: vsa_plan_info, row_src_dev: torch.Tensor, block_len_dev: torch.Tensor,
                        heads: int, head_dim: int, k: int, q: torch.Tensor, workspace: torch.Tensor,
                        keep_idx: Optional[torch.Tensor], o_coarse: torch.Tensor, gate: torch.Tensor,
                        out: torch.Tensor, scale: float = 0.0, stream=None,
                        split_chunks: int = 0) -> None:
    S = info.rows_real
    _need(q, "q", torch.bfloat16, (S, heads, head_dim))
    _need(gate, "gate", torch.bfloat16)
    if gate.numel() != S * heads * head_dim:
        raise ValueError("gate must hold [S][heads*head_dim] values")
    _need(out, "out", torch.bfloat16, (S, heads, head_dim))
    _need(row_src_dev, "row_src", torch.int32, (info.rows_padded,))
    _need(block_len_dev, "block_len", torch.int32, (info.n_tiles,))
    _need(workspace, "workspace", torch.uint8)
    _need(o_coarse, "o_coarse", torch.float32, (heads, info.n_tiles, head_dim))
    if keep_idx is not None:
        _need(keep_idx, "keep_idx", torch.int32, (heads, info.n_video_tiles, k))
    _check(_lib.vsa_sparse_attn_fwd(ctypes.byref(info), _ptr(row_src_dev), _ptr(block_len_dev), heads,
                                    head_dim, int(k), float(scale), int(split_chunks), _ptr(q),
                                    _ptr(workspace),
                                    workspace.numel(), _ptr(keep_idx), _ptr(o_coarse), _ptr(gate),
                                    _ptr(out), _stream(stream)),
           "vsa_sparse_attn_fwd")


def vsa_coarse_topk_ref(info: vsa_plan_info, row_src_dev: torch.Tensor,
                        block_len_dev: torch.Tensor, heads: int, head_dim: int, q: torch.Tensor,
                        k: torch.Tensor, v: torch.Tensor, workspace: torch.Tensor,
                        keep_idx: Optional[torch.Tensor], o_coarse: torch.Tensor,
                        sparsity: Optional[float] = None, keep_k: Optional[int] = None,
                        ref_sparsity: Optional[float] = None, ref_keep_k: Optional[int] = None,
                        scale: float = 0.0, stream=None) -> None:
    S = info.rows_real
    if (q is None) != (k is None) or (q is None) != (v is None):
        raise ValueError("pass q, k and v, or none of them")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if t is not None:
            _need(t, n, torch.bfloat16, (S, heads, head_dim))
    _need(row_src_dev, "row_src", torch.int32, (info.rows_padded,))
    _need(block_len_dev, "block_len", torch.int32, (info.n_tiles,))
    _need(workspace, "workspace", torch.uint8)
    _need(o_coarse, "o_coarse", torch.float32, (heads, info.n_tiles, head_dim))
    if keep_idx is not None:
        _need(keep_idx, "keep_idx", torch.int32)
        if keep_idx.dim() != 3 or tuple(keep_idx.shape[:2]) != (heads, info.n_tiles):
            raise ValueError("keep_idx must be [heads][n_tiles][k_ref + k_gen]")
    _check(_lib.vsa_coarse_topk_ref(
        ctypes.byref(info), _ptr(row_src_dev), _ptr(block_len_dev), heads, head_dim,
        float("nan") if sparsity is None else float(sparsity), -1 if keep_k is None else int(keep_k),
        float("nan") if ref_sparsity is None else float(ref_sparsity),
        -1 if ref_keep_k is None else int(ref_keep_k), float(scale), _ptr(q), _ptr(k), _ptr(v),
        _ptr(workspace), workspace.numel(), _ptr(keep_idx), _ptr(o_coarse), _stream(stream)),
        "vsa_coarse_topk_ref")


def vsa_sparse_attn_fwd_ref(info: vsa_plan_info, row_src_dev: torch.Tensor,
                            block_len_dev: torch.Tensor, heads: int, head_dim: int, k_ref: int,
                            k_gen: int, q: torch.Tensor, workspace: torch.Tensor,
                            keep_idx: Optional[torch.Tensor], o_coarse: torch.Tensor,
                            gate: torch.Tensor, out: torch.Tensor, scale: float = 0.0,
                            stream=None, split_chunks: int = 0) -> None:
    S = info.rows_real
    _need(q, "q", torch.bfloat16, (S, heads, head_dim))
    _need(gate, "gate", torch.bfloat16)
    if gate.numel() != S * heads * head_dim:
        raise ValueError("gate must hold [S][heads*head_dim] values")
    _need(out, "out", torch.bfloat16, (S, heads, head_dim))
    _need(row_src_dev, "row_src", torch.int32, (info.rows_padded,))
    _need(block_len_dev, "block_len", torch.int32, (info.n_tiles,))
    _need(workspace, "workspace", torch.uint8)
    _need(o_coarse, "o_coarse", torch.float32, (heads, info.n_tiles, head_dim))
    if keep_idx is not None:
        _need(keep_idx, "keep_idx", torch.int32, (heads, info.n_tiles, k_ref + k_gen))
    _check(_lib.vsa_sparse_attn_fwd_ref(ctypes.byref(info), _ptr(row_src_dev), _ptr(block_len_dev),
                                        heads, head_dim, int(k_ref), int(k_gen), float(scale),
                                        int(split_chunks), _ptr(q), _ptr(workspace),
                                        workspace.numel(), _ptr(keep_idx),
                                        _ptr(o_coarse), _ptr(gate), _ptr(out), _stream(stream)),
           "vsa_sparse_attn_fwd_ref")


def vsa_sparse_attn_fwd_i8(info: vsa_plan_info, row_src_dev: torch.Tensor,
                           block_len_dev: torch.Tensor, heads: int, head_dim: int, k_ref: int,
                           k_gen: int, q: torch.Tensor, workspace: torch.Tensor,
                           keep_idx: Optional[torch.Tensor], o_coarse: torch.Tensor,
                           gate: torch.Tensor, out: torch.Tensor, scale: float = 0.0,
                           stream=None, split_chunks: int = 0) -> None:
    """The fine pass with INT8 scores; k_ref < 0 selects the default mode
    (keep_idx [H][n_v][k_gen]), k_ref >= 0 the reference-sparsity mode."""
    S = info.rows_real
    _need(q, "q", torch.bfloat16, (S, heads, head_dim))
    _need(gate, "gate", torch.bfloat16)
    if gate.numel() != S * heads * head_dim:
        raise ValueError("gate must hold [S][heads*head_dim] values")
    _need(out, "out", torch.bfloat16, (S, heads, head_dim))
    _need(row_src_dev, "row_src", torch.int32, (info.rows_padded,))
    _need(block_len_dev, "block_len", torch.int32, (info.n_tiles,))
    _need(workspace, "workspace", torch.uint8)
    _need(o_coarse, "o_coarse", torch.float32, (heads, info.n_tiles, head_dim))
    if keep_idx is not None:
        shape = ((heads, info.n_video_tiles, k_gen) if k_ref < 0
                 else (heads, info.n_tiles, k_ref + k_gen))
        _need(keep_idx, "keep_idx", torch.int32, shape)
    _check(_lib.vsa_sparse_attn_fwd_i8(ctypes.byref(info), _ptr(row_src_dev), _ptr(block_len_dev),
                                       heads, head_dim, int(k_ref), int(k_gen), float(scale),
                                       int(split_chunks), _ptr(q), _ptr(workspace),
                                       workspace.numel(), _ptr(keep_idx),
                                       _ptr(o_coarse), _ptr(gate), _ptr(out), _stream(stream)),
           "vsa_sparse_attn_fwd_i8")


def vsa_bwd_workspace_layout(info: vsa_plan_info, heads: int, head_dim: int,
                             split_chunks: int = 0) -> vsa_bwd_layout:
    lay = vsa_bwd_layout()
    _check(_lib.vsa_bwd_workspace_layout(ctypes.byref(info), int(heads), int(head_dim),
                                         int(split_chunks), ctypes.byref(lay)),
           "vsa_bwd_workspace_layout")
    return lay


def vsa_sparse_attn_bwd(info: vsa_plan_info, row_src_dev: torch.Tensor, block_len_dev: torch.Tensor,
                        heads: int, head_dim: int, k_ref: int, k_gen: int, q, k, v, gate, dout,
                        workspace: torch.Tensor, keep_idx: Optional[torch.Tensor],
                        o_coarse: torch.Tensor, bwd_workspace: torch.Tensor, dq, dk, dv, dgate,
                        scale: float = 0.0, stream=None, saved_stats: bool = False,
                        split_chunks: int = 0) -> None:
    """Backward pass (k_ref < 0: default mode). Gradients are fp32. saved_stats: the
    bwd_workspace holds what vsa_sparse_attn_fwd_train saved for this forward."""
    S = info.rows_real
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        _need(t, n, torch.bfloat16, (S, heads, head_dim))
    _need(gate, "gate", torch.bfloat16)
    if gate.numel() != S * heads * head_dim:
        raise ValueError("gate must hold [S][heads*head_dim] values")
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _need(t, n, torch.float32, (S, heads, head_dim))
    _need(dgate, "dgate", torch.float32)
    if dgate.numel() != S * heads * head_dim:
        raise ValueError("dgate must hold [S][heads*head_dim] values")
    _need(row_src_dev, "row_src", torch.int32, (info.rows_padded,))
    _need(block_len_dev, "block_len", torch.int32, (info.n_tiles,))
    _need(workspace, "workspace", torch.uint8)
    _need(bwd_workspace, "bwd_workspace", torch.uint8)
    _need(o_coarse, "o_coarse", torch.float32, (heads, info.n_tiles, head_dim))
    if keep_idx is not None:
        _need(keep_idx, "keep_idx", torch.int32)
    _check(_lib.vsa_sparse_attn_bwd(
        ctypes.byref(info), _ptr(row_src_dev), _ptr(block_len_dev), heads, head_dim, int(k_ref),
        int(k_gen), float(scale), int(split_chunks), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(dout),
        _ptr(workspace), workspace.numel(), _ptr(keep_idx), _ptr(o_coarse), _ptr(bwd_workspace),
        bwd_workspace.numel(), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dgate), int(bool(saved_stats)),
        _stream(stream)),
        "vsa_sparse_attn_bwd")


def vsa_sparse_attn_fwd_train(info: vsa_plan_info, row_src_dev: torch.Tensor,
                              block_len_dev: torch.Tensor, heads: int, head_dim: int, k_ref: int,
                              k_gen: int, q: torch.Tensor, workspace: torch.Tensor,
                              keep_idx: Optional[torch.Tensor], o_coarse: torch.Tensor,
                              gate: torch.Tensor, out: torch.Tensor, bwd_workspace: torch.Tensor,
                              scale: float = 0.0, stream=None, split_chunks: int = 0) -> None:
    """The fine pass of a training step (k_ref < 0: default mode): the forward's
    output plus the lse and O_fine the backward needs, saved in bwd_workspace."""
    S = info.rows_real
    _need(q, "q", torch.bfloat16, (S, heads, head_dim))
    _need(gate, "gate", torch.bfloat16)
    if gate.numel() != S * heads * head_dim:
        raise ValueError("gate must hold [S][heads*head_dim] values")
    _need(out, "out", torch.bfloat16, (S, heads, head_dim))
    _need(row_src_dev, "row_src", torch.int32, (info.rows_padded,))
    _need(block_len_dev, "block_len", torch.int32, (info.n_tiles,))
    _need(workspace, "workspace", torch.uint8)
    _need(bwd_workspace, "bwd_workspace", torch.uint8)
    _need(o_coarse, "o_coarse", torch.float32, (heads, info.n_tiles, head_dim))
    if keep_idx is not None:
        shape = ((heads, info.n_video_tiles, k_gen) if k_ref < 0
                 else (heads, info.n_tiles, k_ref + k_gen))
        _need(keep_idx, "keep_idx", torch.int32, shape)
    _check(_lib.vsa_sparse_attn_fwd_train(
        ctypes.byref(info), _ptr(row_src_dev), _ptr(block_len_dev), heads, head_dim, int(k_ref),
        int(k_gen), float(scale), int(split_chunks), _ptr(q), _ptr(workspace), workspace.numel(),
        _ptr(keep_idx),
        _ptr(o_coarse), _ptr(gate), _ptr(out), _ptr(bwd_workspace), bwd_workspace.numel(),
        _stream(stream)), "vsa_sparse_attn_fwd_train")


def vsa_qkv_gate_proj(info: vsa_plan_info, row_src_dev: torch.Tensor, block_len_dev: torch.Tensor,
                      heads: int, head_dim: int, x: torch.Tensor, w_qkvg: torch.Tensor,
                      q: torch.Tensor, gate: torch.Tensor, workspace: torch.Tensor,
                      stream=None) -> None:
    """The chunked producer: q and gate in natural order, tiled K/V and the tile means
    in the workspace, from x and the stacked [W_q; W_k; W_v; W_gate]."""
    S = info.rows_real
    _need(x, "x", torch.bfloat16)
    if x.dim() != 2 or x.shape[0] != S:
        raise ValueError("x must be [S][hidden]")
    hidden = x.shape[1]
    _need(w_qkvg, "w_qkvg", torch.bfloat16)
    if w_qkvg.numel() != 4 * heads * head_dim * hidden:
        raise ValueError("w_qkvg must be [4][heads*head_dim][hidden]")
    _need(q, "q", torch.bfloat16, (S, heads, head_dim))
    _need(gate, "gate", torch.bfloat16)
    if gate.numel() != S * heads * head_dim:
        raise ValueError("gate must hold [S][heads*head_dim] values")
    _need(row_src_dev, "row_src", torch.int32, (info.rows_padded,))
    _need(block_len_dev, "block_len", torch.int32, (info.n_tiles,))
    _need(workspace, "workspace", torch.uint8)
    _check(_lib.vsa_qkv_gate_proj(ctypes.byref(info), _ptr(row_src_dev), _ptr(block_len_dev), heads,
                                  head_dim, int(hidden), _ptr(x), _ptr(w_qkvg), _ptr(q), _ptr(gate),
                                  _ptr(workspace), workspace.numel(), _stream(stream)),
           "vsa_qkv_gate_proj")


def vsa_layer_fwd_static(info: vsa_plan_info, row_src_dev: torch.Tensor, block_len_dev: torch.Tensor,
                         heads: int, head_dim: int, q: torch.Tensor, k: torch.Tensor,
                         v: torch.Tensor, gate: torch.Tensor, keep_idx: Optional[torch.Tensor],
                         o_coarse: torch.Tensor, out: torch.Tensor,
                         sparsity: Optional[float] = None, keep_k: Optional[int] = None,
                         scale: float = 0.0, stream=None) -> None:
    """The whole layer (coarse stage, then the unsplit fine pass) with the library's
    static workspace: no device allocation in the call."""
    S = info.rows_real
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _need(t, n, torch.bfloat16, (S, heads, head_dim))
    _need(gate, "gate", torch.bfloat16)
    if gate.numel() != S * heads * head_dim:
        raise ValueError("gate must hold [S][heads*head_dim] values")
    _need(row_src_dev, "row_src", torch.int32, (info.rows_padded,))
    _need(block_len_dev, "block_len", torch.int32, (info.n_tiles,))
    _need(o_coarse, "o_coarse", torch.float32, (heads, info.n_tiles, head_dim))
    if keep_idx is not None:
        _need(keep_idx, "keep_idx", torch.int32)
        if keep_idx.dim() != 3 or tuple(keep_idx.shape[:2]) != (heads, info.n_video_tiles):
            raise ValueError("keep_idx must be [heads][n_v][k]")
    _check(_lib.vsa_layer_fwd_static(
        ctypes.byref(info), _ptr(row_src_dev), _ptr(block_len_dev), heads, head_dim,
        float("nan") if sparsity is None else float(sparsity), -1 if keep_k is None else int(keep_k),
        float(scale), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(keep_idx), _ptr(o_coarse),
        _ptr(out), _stream(stream)), "vsa_layer_fwd_static")


def vsa_gate_proj(x: torch.Tensor, w_gate: torch.Tensor, g: torch.Tensor, stream=None) -> None:
    _need(x, "x", torch.bfloat16)
    _need(w_gate, "w_gate", torch.bfloat16)
    _need(g, "g", torch.bfloat16)
    rows, hidden = x.shape
    out_f = w_gate.shape[0]
    if w_gate.shape[1] != hidden or tuple(g.shape) != (rows, out_f):
        raise ValueError("shapes: x [rows][hidden], w_gate [out][hidden], g [rows][out]")
    _check(_lib.vsa_gate_proj(_ptr(x), _ptr(w_gate), rows, hidden, out_f, _ptr(g), _stream(stream)),
           "vsa_gate_proj")


def vsa_timing_enable(enable: bool, stream=None) -> None:
    """Start (clearing earlier records) or stop per-kernel timing of the library's
    launches on `stream` (default: torch's current stream)."""
    _check(_lib.vsa_timing_enable(_stream(stream), 1 if enable else 0), "vsa_timing_enable")


def vsa_timing_read(kernel: str, stream=None) -> tuple:
    """(launches, total ms) of `kernel` on `stream` since its timing was last enabled;
    waits for them."""
    n = ctypes.c_int32()
    ms = ctypes.c_double()
    _check(_lib.vsa_timing_read(_stream(stream), kernel.encode(), ctypes.byref(n), ctypes.byref(ms)),
           "vsa_timing_read")
    return n.value, ms.value


# ---------------------------------------------------------- convenience --

_PLAN_CACHE: dict = {}


def cached_plan(prefix_segments, grid, tile) -> Plan:
    """The plan is a pure function of the shape: build and validate it once per shape."""
    key = (tuple(int(s) for s in prefix_segments), tuple(int(g) for g in grid), tuple(int(t) for t in tile))
    pl = _PLAN_CACHE.get(key)
    if pl is None:
        pl = vsa_plan_tiles(*key)
        vsa_plan_validate(pl)
        _PLAN_CACHE[key] = pl
    return pl


class TileSparseAttention:
    """One layer's gated tile-sparse attention with its device-side state.

    Holds the cached plan (copied to the device once), the workspace, and the
    keep-index / coarse-output buffers, so each call only enqueues kernels."""

    def __init__(self, prefix_segments, grid, tile, heads: int, head_dim: int,
                 sparsity: Optional[float] = None, keep_k: Optional[int] = None,
                 scale: float = 0.0, device="cuda", reference_sparsity: Optional[float] = None,
                 ref_keep_k: Optional[int] = None, int8: bool = False, split_chunks: int = 0):
        """reference_sparsity / ref_keep_k (either one) switch to the reference-sparsity
        mode: every query tile keeps k_ref prefix tiles and k video tiles. int8 runs
        the fine pass with INT8 scores (vsa_sparse_attn_fwd_i8). split_chunks: the fine
        pass's key-list split for this layer (0 = automatic)."""
        self.int8 = bool(int8)
        self.plan = cached_plan(prefix_segments, grid, tile)
        info = self.plan.info
        self.heads, self.head_dim, self.scale = int(heads), int(head_dim), float(scale)
        self.sparsity, self.keep_k = sparsity, keep_k
        self.k = vsa_keep_count(info, sparsity, keep_k)
        self.ref = reference_sparsity is not None or ref_keep_k is not None
        self.reference_sparsity, self.ref_keep_k = reference_sparsity, ref_keep_k
        self.k_ref = vsa_ref_keep_count(info, reference_sparsity, ref_keep_k) if self.ref else 0
        self.layout = vsa_workspace_layout(info, heads, head_dim, split_chunks)
        self.split_chunks = int(self.layout.split_chunks)
        dev = torch.device(device)
        self.row_src = torch.from_numpy(self.plan.row_src).to(dev)
        self.block_len = torch.from_numpy(self.plan.block_len).to(dev)
        self.workspace = torch.empty(self.layout.total_bytes, dtype=torch.uint8, device=dev)
        if self.ref:
            shape = (heads, info.n_tiles, self.k_ref + self.k)
        else:
            shape = (heads, info.n_video_tiles, self.k)
        self.keep_idx = torch.empty(shape, dtype=torch.int32, device=dev)
        self.o_coarse = torch.empty((heads, info.n_tiles, head_dim), dtype=torch.float32, device=dev)

    @property
    def list_len(self) -> int:
        return self.keep_idx.shape[2]

    def project(self, x, w_qkvg, q, gate, stream=None) -> None:
        """The chunked producer: q and gate (natural order) plus the tiled K/V and tile
        means in this layer's workspace; follow with coarse(None, None, None)."""
        vsa_qkv_gate_proj(self.plan.info, self.row_src, self.block_len, self.heads, self.head_dim,
                          x, w_qkvg, q, gate, self.workspace, stream=stream)

    def coarse(self, q, k, v, stream=None) -> None:
        """q = k = v = None after project(): the gather is skipped."""
        keep = self.keep_idx if self.list_len > 0 else None
        if self.ref:
            vsa_coarse_topk_ref(self.plan.info, self.row_src, self.block_len, self.heads,
                                self.head_dim, q, k, v, self.workspace, keep, self.o_coarse,
                                sparsity=self.sparsity, keep_k=self.keep_k,
                                ref_sparsity=self.reference_sparsity, ref_keep_k=self.ref_keep_k,
                                scale=self.scale, stream=stream)
        else:
            vsa_coarse_topk(self.plan.info, self.row_src, self.block_len, self.heads,
                            self.head_dim, q, k, v, self.workspace, keep, self.o_coarse,
                            sparsity=self.sparsity, keep_k=self.keep_k, scale=self.scale,
                            stream=stream)

    def fine(self, q, gate, out, stream=None) -> None:
        self._stats_saved = False
        keep = self.keep_idx if self.list_len > 0 else None
        if self.int8:
            vsa_sparse_attn_fwd_i8(self.plan.info, self.row_src, self.block_len, self.heads,
                                   self.head_dim, self.k_ref if self.ref else -1, self.k, q,
                                   self.workspace, keep, self.o_coarse, gate, out,
                                   scale=self.scale, stream=stream, split_chunks=self.split_chunks)
        elif self.ref:
            vsa_sparse_attn_fwd_ref(self.plan.info, self.row_src, self.block_len, self.heads,
                                    self.head_dim, self.k_ref, self.k, q, self.workspace, keep,
                                    self.o_coarse, gate, out, scale=self.scale, stream=stream,
                                    split_chunks=self.split_chunks)
        else:
            vsa_sparse_attn_fwd(self.plan.info, self.row_src, self.block_len, self.heads,
                                self.head_dim, self.k, q, self.workspace, keep, self.o_coarse,
                                gate, out, scale=self.scale, stream=stream,
                                split_chunks=self.split_chunks)

    def _bwd_workspace(self, device):
        if not hasattr(self, "bwd_workspace"):
            lay = vsa_bwd_workspace_layout(self.plan.info, self.heads, self.head_dim,
                                           self.split_chunks)
            self.bwd_layout = lay
            self.bwd_workspace = torch.empty(lay.total_bytes, dtype=torch.uint8, device=device)
        return self.bwd_workspace

    def fine_train(self, q, gate, out, stream=None) -> None:
        """The fine pass of a training step: fine()'s output, plus the lse and O_fine
        saved for the next backward() (bf16 path; not with int8)."""
        if self.int8:
            raise ValueError("the training forward is bf16; this layer runs the INT8 pass")
        keep = self.keep_idx if self.list_len > 0 else None
        vsa_sparse_attn_fwd_train(self.plan.info, self.row_src, self.block_len, self.heads,
                                  self.head_dim, self.k_ref if self.ref else -1, self.k, q,
                                  self.workspace, keep, self.o_coarse, gate, out,
                                  self._bwd_workspace(q.device), scale=self.scale, stream=stream,
                                  split_chunks=self.split_chunks)
        self._stats_saved = True

    def backward(self, q, k, v, gate, dout, stream=None):
        """Gradients (dq, dk, dv, dgate), fp32, of the last forward's layer with its
        keep sets held fixed. Call after coarse() and fine() (or fine_train(), whose
        saved statistics it then uses) on the same inputs."""
        self._bwd_workspace(q.device)
        saved = getattr(self, "_stats_saved", False)
        dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        dk, dv = torch.empty_like(dq), torch.empty_like(dq)
        dgate = torch.empty(gate.shape, dtype=torch.float32, device=q.device)
        keep = self.keep_idx if self.list_len > 0 else None
        vsa_sparse_attn_bwd(self.plan.info, self.row_src, self.block_len, self.heads, self.head_dim,
                            self.k_ref if self.ref else -1, self.k, q, k, v, gate, dout,
                            self.workspace, keep, self.o_coarse, self.bwd_workspace, dq, dk, dv,
                            dgate, scale=self.scale, stream=stream, saved_stats=saved,
                            split_chunks=self.split_chunks)
        return dq, dk, dv, dgate

    def tile_pair_fraction(self) -> float:
        if self.ref:
            return vsa_tile_pair_fraction_ref(self.plan.info, self.k_ref, self.k)
        return vsa_tile_pair_fraction(self.plan.info, self.k)

    def __call__(self, q, k, v, gate, out=None, stream=None) -> torch.Tensor:
        if out is None:
            out = torch.empty_like(q)
        self.coarse(q, k, v, stream)
        self.fine(q, gate, out, stream)
        return out

    def workspace_view(self, name: str, dtype, shape) -> torch.Tensor:
        """A typed view of one workspace region (tests read means and scores)."""
        off = getattr(self.layout, name)
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        return self.workspace[off:off + n].view(dtype).view(*shape)


class HeadGroupAttention:
    """One layer whose heads are split into groups of consecutive heads, each with
    its own tile shape (per-head tile shapes); one vsa_layer_fwd_groups call runs
    every group on the shared q, k, v, gate and out.

    groups: sequence of dicts with keys "tile" and "heads" (required) and optional
    "sparsity", "keep_k", "reference_sparsity", "ref_keep_k", "int8", "split_chunks"; the groups
    take the heads in order."""

    def __init__(self, prefix_segments, grid, groups, head_dim: int, scale: float = 0.0,
                 device="cuda", heads_total: Optional[int] = None):
        """heads_total: heads per token row of the tensors (default: the groups' sum;
        heads beyond the groups are left untouched)."""
        self.head_dim, self.scale = int(head_dim), float(scale)
        self.layers, first = [], 0
        for g in groups:
            att = TileSparseAttention(prefix_segments, grid, g["tile"], g["heads"], head_dim,
                                      sparsity=g.get("sparsity"), keep_k=g.get("keep_k"),
                                      scale=scale, device=device,
                                      reference_sparsity=g.get("reference_sparsity"),
                                      ref_keep_k=g.get("ref_keep_k"), int8=g.get("int8", False),
                                      split_chunks=g.get("split_chunks", 0))
            self.layers.append((first, att))
            first += int(g["heads"])
        self.heads_total = first if heads_total is None else int(heads_total)
        arr = (vsa_head_group * len(self.layers))()
        for i, (h0, att) in enumerate(self.layers):
            e = arr[i]
            e.info = ctypes.pointer(att.plan.info)
            e.row_src_dev, e.block_len_dev = _ptr(att.row_src), _ptr(att.block_len)
            e.head_first, e.heads = h0, att.heads
            e.sparsity = float("nan") if att.sparsity is None else float(att.sparsity)
            e.keep_k = -1 if att.keep_k is None else int(att.keep_k)
            e.ref, e.int8 = int(att.ref), int(att.int8)
            e.ref_sparsity = (float("nan") if att.reference_sparsity is None
                              else float(att.reference_sparsity))
            e.ref_keep_k = -1 if att.ref_keep_k is None else int(att.ref_keep_k)
            e.split_chunks = att.split_chunks
            e.workspace, e.workspace_bytes = _ptr(att.workspace), att.workspace.numel()
            e.keep_idx_dev = _ptr(att.keep_idx) if att.list_len > 0 else None
            e.o_coarse_dev = _ptr(att.o_coarse)
        self.groups = arr

    def __call__(self, q, k, v, gate, out=None, stream=None) -> torch.Tensor:
        S = self.layers[0][1].plan.info.rows_real
        H, D = self.heads_total, self.head_dim
        for t, n in ((q, "q"), (k, "k"), (v, "v")):
            _need(t, n, torch.bfloat16, (S, H, D))
        _need(gate, "gate", torch.bfloat16)
        if gate.numel() != S * H * D:
            raise ValueError("gate must hold [S][heads*head_dim] values")
        if out is None:
            out = torch.empty_like(q)
        _need(out, "out", torch.bfloat16, (S, H, D))
        _check(_lib.vsa_layer_fwd_groups(self.groups, len(self.layers), H, D, self.scale, _ptr(q),
                                         _ptr(k), _ptr(v), _ptr(gate), _ptr(out), _stream(stream)),
               "vsa_layer_fwd_groups")
        return out
