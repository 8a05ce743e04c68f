"""CPU oracle for gated, tile-sparse video attention -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The HIP library never loads it, and it
imports nothing from the library package.

The arithmetic lives in ``oracle.c`` (plain C, gcc, ``-ffp-contract=off``);
this module only marshals numpy arrays into it and strings the steps together
in the order the method runs them. Each C function cites the passage of the
pages it follows; see the header of ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Iterable, Optional, Sequence

import numpy as np
from threadpoolctl import threadpool_limits

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# ORACLE_LIBRARY names another build of oracle.c (the host-sanitizer build of
# build(sanitize=True)); by default the in-tree liboracle.so.
_LIB_PATH = os.environ.get("ORACLE_LIBRARY") or os.path.join(_HERE, "liboracle.so")
_SANITIZED_LIB = os.path.join(_HERE, "liboracle_san.so")
_lib = None

_I32P = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_I64P = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_U16P = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_I8P = np.ctypeslib.ndpointer(dtype=np.int8, flags="C_CONTIGUOUS")
_F32P = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_F64P = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")


def build(sanitize: bool = False) -> str:
    """Compile liboracle.so with gcc (plain C, OpenMP, no FMA contraction).
    sanitize=True: the same source with clang and host AddressSanitizer +
    UndefinedBehaviorSanitizer (the runtime the HIP library's sanitizer build
    uses), into liboracle_san.so."""
    if sanitize:
        out = _SANITIZED_LIB
        cmd = ["/opt/rocm/lib/llvm/bin/clang", "-std=c11", "-O1", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-fPIC", "-shared", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-shared-libsan", _SRC,
               "-o", out + ".tmp", "-lm"]
    else:
        out = os.path.join(_HERE, "liboracle.so")
        cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", _SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.orc_bf16_round.argtypes = [f64]
    lib.orc_bf16_round.restype = ctypes.c_uint16
    lib.orc_bf16_value.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_value.restype = f64
    lib.orc_plan.argtypes = [_I64P, i32, i32, i32, i32, i32, i32, i32, _I64P,
                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.orc_plan.restype = ctypes.c_int
    lib.orc_keep_count.argtypes = [i32, f64, i64, ctypes.POINTER(i32)]
    lib.orc_keep_count.restype = ctypes.c_int
    lib.orc_tile_means.argtypes = [_U16P, i32, i32, i32, _I32P, _I32P, i32, i32, _F32P]
    lib.orc_tile_means.restype = None
    lib.orc_video_scores.argtypes = [_F32P, _F32P, i32, i32, i32, _I32P, i32, _F32P]
    lib.orc_video_scores.restype = None
    lib.orc_all_scores.argtypes = [_F32P, _F32P, i32, i32, _I32P, i32, _F32P]
    lib.orc_all_scores.restype = None
    lib.orc_topk_rows.argtypes = [_F32P, i32, i32, i32, i32, _I32P]
    lib.orc_topk_rows.restype = ctypes.c_int
    lib.orc_coarse_attn.argtypes = [_F32P, _F32P, _F32P, i32, i32, f64, _I32P, i32, _F64P]
    lib.orc_coarse_attn.restype = None
    lib.orc_fine_tokens.argtypes = [_U16P, _U16P, _U16P, i32, i32, i32, _I32P, _I32P, i32, i32,
                                    i32, _I32P, i32, f64, _I64P, i64, _F64P]
    lib.orc_fine_tokens.restype = ctypes.c_int
    lib.orc_fine_tokens_lists.argtypes = [_U16P, _U16P, _U16P, i32, i32, i32, _I32P, _I32P, i32,
                                          i32, _I32P, i32, f64, _I64P, i64, _F64P]
    lib.orc_fine_tokens_lists.restype = ctypes.c_int
    lib.orc_quant_blocks_i8.argtypes = [_U16P, i32, i32, i32, _I32P, i32, i32, _I8P, _F32P]
    lib.orc_quant_blocks_i8.restype = ctypes.c_int
    lib.orc_fine_tokens_i8.argtypes = [_U16P, _U16P, _U16P, i32, i32, i32, _I32P, _I32P, i32, i32,
                                       _I32P, _I32P, f64, _I64P, i64, _F64P]
    lib.orc_fine_tokens_i8.restype = ctypes.c_int
    lib.orc_layer_bwd.argtypes = [_U16P, _U16P, _U16P, _U16P, _U16P, i32, i32, i32, _I32P, _I32P,
                                  _I32P, i32, i32, _I32P, _I32P, _F32P, _F32P, _F32P, f64, _F64P,
                                  _F64P, _F64P, _F64P]
    lib.orc_layer_bwd.restype = ctypes.c_int
    lib.orc_dq_tokens.argtypes = [_U16P, _U16P, _U16P, _U16P, _U16P, i32, i32, i32, _I32P, _I32P,
                                  _I32P, i32, i32, _I32P, _I32P, _F32P, _F32P, _F32P, f64, _I64P,
                                  i64, _F64P]
    lib.orc_dq_tokens.restype = ctypes.c_int
    lib.orc_combine.argtypes = [_F64P, _U16P, _F64P, i64, i32, _U16P]
    lib.orc_combine.restype = None
    lib.orc_gate_proj.argtypes = [_U16P, _U16P, i32, i32, _I64P, i64, _U16P]
    lib.orc_gate_proj.restype = None
    lib.orc_tile_pair_fraction.argtypes = [i32, i32, i32]
    lib.orc_tile_pair_fraction.restype = f64
    _lib = lib
    return lib


class OracleError(ValueError):
    pass


# ----------------------------------------------------------------- helpers --

def bf16_round(values) -> np.ndarray:
    """fp64 values -> bf16 bit patterns (uint16), one round-to-nearest-even."""
    lib = _load()
    v = np.asarray(values, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    flat_in, flat_out = v.reshape(-1), out.reshape(-1)
    for i in range(flat_in.size):
        flat_out[i] = lib.orc_bf16_round(float(flat_in[i]))
    return out


def bf16_value(bits) -> np.ndarray:
    """bf16 bit patterns -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


@dataclass
class Plan:
    S: int
    P: int
    n_v: int
    n_t: int
    B: int
    untile: np.ndarray      # int32 [S]
    row_src: np.ndarray     # int32 [n_t * B], -1 = padding
    block_len: np.ndarray   # int32 [n_t]

    @property
    def S_pad(self) -> int:
        return self.n_t * self.B


def plan(prefix_segments: Sequence[int], grid, tile) -> Plan:
    lib = _load()
    seg = np.ascontiguousarray(np.asarray(list(prefix_segments), dtype=np.int64).reshape(-1))
    if seg.size == 0:
        seg = np.zeros(1, dtype=np.int64)
        n_seg = 0
    else:
        n_seg = seg.size
    sizes = np.zeros(5, dtype=np.int64)
    args = (seg, n_seg, grid[0], grid[1], grid[2], tile[0], tile[1], tile[2], sizes)
    if lib.orc_plan(*args, None, None, None) != 0:
        raise OracleError("invalid plan arguments")
    S, P, n_v, n_t, B = (int(x) for x in sizes)
    untile = np.empty(S, dtype=np.int32)
    row_src = np.empty(n_t * B, dtype=np.int32)
    block_len = np.empty(n_t, dtype=np.int32)
    rc = lib.orc_plan(*args, untile.ctypes.data, row_src.ctypes.data, block_len.ctypes.data)
    assert rc == 0
    return Plan(S, P, n_v, n_t, B, untile, row_src, block_len)


def keep_count(n_v: int, sparsity: Optional[float] = None, keep_k: Optional[int] = None) -> int:
    lib = _load()
    k = ctypes.c_int32(0)
    rc = lib.orc_keep_count(int(n_v), float("nan") if sparsity is None else float(sparsity),
                            -1 if keep_k is None else int(keep_k), ctypes.byref(k))
    if rc != 0:
        raise OracleError("invalid keep-count arguments")
    return int(k.value)


def tile_means(X: np.ndarray, h: int, pl: Plan) -> np.ndarray:
    """X: uint16 bf16 bits [S][H][D] -> fp32 [n_t][D] for head h."""
    lib = _load()
    X = np.ascontiguousarray(X, dtype=np.uint16)
    S, H, D = X.shape
    out = np.empty((pl.n_t, D), dtype=np.float32)
    lib.orc_tile_means(X.reshape(-1), H, D, int(h), pl.row_src, pl.block_len, pl.n_t, pl.B,
                       out.reshape(-1))
    return out


def video_scores(qm: np.ndarray, km: np.ndarray, P: int, n_v: int,
                 rows: Optional[Iterable[int]] = None) -> np.ndarray:
    lib = _load()
    D = qm.shape[1]
    r = np.arange(n_v, dtype=np.int32) if rows is None else np.asarray(list(rows), dtype=np.int32)
    r = np.ascontiguousarray(r)
    out = np.empty((r.size, n_v), dtype=np.float32)
    lib.orc_video_scores(np.ascontiguousarray(qm, dtype=np.float32).reshape(-1),
                         np.ascontiguousarray(km, dtype=np.float32).reshape(-1),
                         int(P), int(n_v), int(D), r, int(r.size), out.reshape(-1))
    return out


def topk_rows(scores: np.ndarray, k: int, P: int) -> np.ndarray:
    lib = _load()
    s = np.ascontiguousarray(scores, dtype=np.float32)
    n_rows, n_v = s.shape
    out = np.empty((n_rows, k), dtype=np.int32)
    if lib.orc_topk_rows(s.reshape(-1), n_rows, n_v, int(k), int(P), out.reshape(-1)) != 0:
        raise OracleError("top-k: non-finite score or k out of range")
    return out


def coarse_attn(qm, km, vm, scale: float, rows: Optional[Iterable[int]] = None) -> np.ndarray:
    lib = _load()
    n_t, D = qm.shape
    r = np.arange(n_t, dtype=np.int32) if rows is None else np.asarray(list(rows), dtype=np.int32)
    r = np.ascontiguousarray(r)
    out = np.empty((r.size, D), dtype=np.float64)
    lib.orc_coarse_attn(np.ascontiguousarray(qm, dtype=np.float32).reshape(-1),
                        np.ascontiguousarray(km, dtype=np.float32).reshape(-1),
                        np.ascontiguousarray(vm, dtype=np.float32).reshape(-1),
                        int(n_t), int(D), float(scale), r, int(r.size), out.reshape(-1))
    return out


def fine_tokens(Q, K, V, h: int, pl: Plan, keep_h: np.ndarray, k: int, scale: float,
                tokens: Iterable[int]) -> np.ndarray:
    """O_fine (fp64 [n_tok][D]) of the given query tokens for head h.

    keep_h: int32 [n_v][k] global ids of the kept video key tiles of head h."""
    lib = _load()
    S, H, D = Q.shape
    toks = np.ascontiguousarray(np.asarray(list(tokens), dtype=np.int64))
    keep_h = np.ascontiguousarray(keep_h, dtype=np.int32).reshape(-1)
    if keep_h.size == 0:
        keep_h = np.zeros(1, dtype=np.int32)
    out = np.empty((toks.size, D), dtype=np.float64)
    rc = lib.orc_fine_tokens(np.ascontiguousarray(Q).reshape(-1), np.ascontiguousarray(K).reshape(-1),
                             np.ascontiguousarray(V).reshape(-1), H, D, int(h), pl.untile,
                             pl.row_src, pl.n_t, pl.B, pl.P, keep_h, int(k), float(scale), toks,
                             int(toks.size), out.reshape(-1))
    if rc != 0:
        raise OracleError("fine attention: a query has an empty key set")
    return out


def combine(o_fine: np.ndarray, g_rows: np.ndarray, o_coarse: np.ndarray) -> np.ndarray:
    lib = _load()
    n, D = o_fine.shape
    out = np.empty((n, D), dtype=np.uint16)
    lib.orc_combine(np.ascontiguousarray(o_fine, dtype=np.float64).reshape(-1),
                    np.ascontiguousarray(g_rows, dtype=np.uint16).reshape(-1),
                    np.ascontiguousarray(o_coarse, dtype=np.float64).reshape(-1), n, D,
                    out.reshape(-1))
    return out


def gate_proj(x: np.ndarray, W: np.ndarray, tokens: Optional[Iterable[int]] = None) -> np.ndarray:
    """g = bf16(x . W^T) for the given token rows: uint16 [n_tok][out_f]."""
    lib = _load()
    S, hidden = x.shape
    out_f = W.shape[0]
    toks = np.arange(S, dtype=np.int64) if tokens is None else np.asarray(list(tokens), dtype=np.int64)
    toks = np.ascontiguousarray(toks)
    out = np.empty((toks.size, out_f), dtype=np.uint16)
    lib.orc_gate_proj(np.ascontiguousarray(x).reshape(-1), np.ascontiguousarray(W).reshape(-1),
                      int(hidden), int(out_f), toks, int(toks.size), out.reshape(-1))
    return out


def tile_pair_fraction(P: int, n_v: int, k: int) -> float:
    return float(_load().orc_tile_pair_fraction(int(P), int(n_v), int(k)))


# ------------------------------------------- reference-sparsity variant --
#
# [Veda] "ComfyUI node" inputs table: reference_sparsity applies the same top-k
# setting to the reference tokens ("0 % = full attention"). Reading: the prefix
# (reference) tiles stop being sinks; every query tile keeps its top-k_ref
# prefix key tiles and its top-k_gen video key tiles by coarse score.

def ref_keep_counts(pl: Plan, ref_sparsity=None, ref_keep_k=None, sparsity=None, keep_k=None):
    """(k_ref over the P prefix tiles, k_gen over the n_v video tiles), same rule as O2."""
    return keep_count(pl.P, ref_sparsity, ref_keep_k), keep_count(pl.n_v, sparsity, keep_k)


def all_scores(qm: np.ndarray, km: np.ndarray, rows: Optional[Iterable[int]] = None) -> np.ndarray:
    """fp32 [n_rows][n_t] FMA-chain scores of the given global query tiles against every tile."""
    lib = _load()
    n_t, D = qm.shape
    r = np.arange(n_t, dtype=np.int32) if rows is None else np.asarray(list(rows), dtype=np.int32)
    r = np.ascontiguousarray(r)
    out = np.empty((r.size, n_t), dtype=np.float32)
    lib.orc_all_scores(np.ascontiguousarray(qm, dtype=np.float32).reshape(-1),
                       np.ascontiguousarray(km, dtype=np.float32).reshape(-1),
                       int(n_t), int(D), r, int(r.size), out.reshape(-1))
    return out


def topk_ref(scores: np.ndarray, P: int, k_ref: int, k_gen: int) -> np.ndarray:
    """Per row: the top k_ref of the prefix columns and the top k_gen of the video
    columns (O5 on each group), as ascending global ids: int32 [n_rows][k_ref + k_gen]."""
    pre = topk_rows(np.ascontiguousarray(scores[:, :P]), k_ref, 0)
    vid = topk_rows(np.ascontiguousarray(scores[:, P:]), k_gen, P)
    return np.concatenate([pre, vid], axis=1)


def fine_tokens_lists(Q, K, V, h: int, pl: Plan, lists_h: np.ndarray, scale: float,
                      tokens: Iterable[int]) -> np.ndarray:
    """O_fine (fp64 [n_tok][D]) of the given tokens of head h with an explicit key
    list per query tile: lists_h int32 [n_t][L] global tile ids."""
    lib = _load()
    S, H, D = Q.shape
    toks = np.ascontiguousarray(np.asarray(list(tokens), dtype=np.int64))
    lists_h = np.ascontiguousarray(lists_h, dtype=np.int32)
    L = int(lists_h.shape[1])
    flat = lists_h.reshape(-1) if lists_h.size else np.zeros(1, dtype=np.int32)
    out = np.empty((toks.size, D), dtype=np.float64)
    rc = lib.orc_fine_tokens_lists(np.ascontiguousarray(Q).reshape(-1),
                                   np.ascontiguousarray(K).reshape(-1),
                                   np.ascontiguousarray(V).reshape(-1), H, D, int(h), pl.untile,
                                   pl.row_src, pl.n_t, pl.B, flat, L, float(scale), toks,
                                   int(toks.size), out.reshape(-1))
    if rc != 0:
        raise OracleError("fine attention: a query has an empty or invalid key list")
    return out


def tile_pair_fraction_ref(n_t: int, k_ref: int, k_gen: int) -> float:
    """Every query tile sees k_ref + k_gen key tiles out of n_t."""
    return (k_ref + k_gen) / n_t


def head_ref(Q, K, V, h: int, pl: Plan, k_ref: int, k_gen: int, scale: float,
             score_rows: Optional[Iterable[int]] = None) -> "HeadResult":
    """Pool, score (all tiles), select per group, coarse-attend one head."""
    qm = tile_means(Q, h, pl)
    km = tile_means(K, h, pl)
    vm = tile_means(V, h, pl)
    rows = (np.arange(pl.n_t, dtype=np.int32) if score_rows is None
            else np.asarray(list(score_rows), dtype=np.int32))
    sc = all_scores(qm, km, rows)
    keep = topk_ref(sc, pl.P, k_ref, k_gen)
    oc = coarse_attn(qm, km, vm, scale)
    return HeadResult(qm, km, vm, sc, rows, keep, oc)


def layer_tokens_ref(Q, K, V, g: np.ndarray, h: int, pl: Plan, hr: "HeadResult", scale: float,
                     tokens: Iterable[int], g_is_rows: bool = False):
    """Reference-sparsity outputs (bf16 bits [n_tok][D]) and O_fine of selected tokens.
    hr must come from head_ref over all n_t query tiles."""
    toks = np.asarray(list(tokens), dtype=np.int64)
    D = Q.shape[2]
    assert hr.keep.shape[0] == pl.n_t, "layer_tokens_ref needs the key lists of all tiles"
    o_fine = fine_tokens_lists(Q, K, V, h, pl, hr.keep, scale, toks)
    tiles = pl.untile[toks] // pl.B
    g_rows = (g if g_is_rows else g[toks])[:, h * D:(h + 1) * D]
    return combine(o_fine, np.ascontiguousarray(g_rows), hr.o_coarse[tiles]), o_fine


# ------------------------------------------------------------ INT8 fine pass --

def quant_blocks_i8(X, h: int, pl: Plan):
    """Symmetric INT8 codes of head h's rows in tiled order, one fp32 scale per
    64-row block: (codes int8 [n_t*B][D], scales fp32 [n_t*B/64])."""
    lib = _load()
    S, H, D = X.shape
    codes = np.zeros((pl.S_pad, D), dtype=np.int8)
    scales = np.zeros(pl.S_pad // 64, dtype=np.float32)
    rc = lib.orc_quant_blocks_i8(np.ascontiguousarray(X).reshape(-1), H, D, int(h), pl.row_src,
                                 pl.n_t, pl.B, codes.reshape(-1), scales)
    if rc != 0:
        raise OracleError("INT8 blocks need B to be a multiple of 64")
    return codes, scales


def fine_tokens_i8(Q, K, V, h: int, pl: Plan, csr, scale: float, tokens) -> np.ndarray:
    """O_fine (fp64 [n_tok][D]) with INT8 scores over CSR key lists (off, ids)."""
    lib = _load()
    S, H, D = Q.shape
    off, ids = csr
    toks = np.ascontiguousarray(np.asarray(list(tokens), dtype=np.int64))
    out = np.empty((toks.size, D), dtype=np.float64)
    rc = lib.orc_fine_tokens_i8(*(np.ascontiguousarray(X).reshape(-1) for X in (Q, K, V)), H, D,
                                int(h), pl.untile, pl.row_src, pl.n_t, pl.B,
                                np.ascontiguousarray(off, dtype=np.int32), ids, float(scale), toks,
                                int(toks.size), out.reshape(-1))
    if rc != 0:
        raise OracleError("INT8 fine attention: an empty or invalid key list")
    return out


# ---------------------------------------------------------------- backward --

def key_lists_default(pl: Plan, keep_h: np.ndarray):
    """CSR key lists (off [n_t+1], ids) of the default mode for one head: prefix query
    tiles see every tile; video query tile P+i sees [0, P) and keep_h[i]."""
    lists = []
    for i in range(pl.n_t):
        if i < pl.P:
            lists.append(np.arange(pl.n_t, dtype=np.int32))
        else:
            lists.append(np.concatenate([np.arange(pl.P, dtype=np.int32),
                                         np.asarray(keep_h[i - pl.P], dtype=np.int32)]))
    return _csr(lists)


def key_lists_explicit(lists_h: np.ndarray):
    """CSR key lists from the reference-sparsity [n_t][L] lists of one head."""
    return _csr([np.asarray(r, dtype=np.int32) for r in lists_h])


def _csr(lists):
    off = np.zeros(len(lists) + 1, dtype=np.int32)
    off[1:] = np.cumsum([len(x) for x in lists])
    ids = np.concatenate(lists).astype(np.int32) if off[-1] else np.zeros(1, np.int32)
    return off, np.ascontiguousarray(ids)


def layer_bwd(Q, K, V, G, dOut, h: int, pl: Plan, csr, scale: float):
    """Gradients of the layer for head h: dict of fp64 [S][D] arrays dq, dk, dv, dg.
    G is the bf16 gate [S][H*D]; dOut is bf16 [S][H][D]; csr = (off, ids) key lists."""
    lib = _load()
    S, H, D = Q.shape
    qm, km, vm = (tile_means(X, h, pl) for X in (Q, K, V))
    off, ids = csr
    outs = {n: np.zeros((S, D), dtype=np.float64) for n in ("dq", "dk", "dv", "dg")}
    rc = lib.orc_layer_bwd(*(np.ascontiguousarray(X).reshape(-1) for X in (Q, K, V, G, dOut)),
                           H, D, int(h), pl.untile, pl.row_src, pl.block_len, pl.n_t, pl.B,
                           np.ascontiguousarray(off), ids, qm.reshape(-1), km.reshape(-1),
                           vm.reshape(-1), float(scale), outs["dq"].reshape(-1),
                           outs["dk"].reshape(-1), outs["dv"].reshape(-1), outs["dg"].reshape(-1))
    if rc != 0:
        raise OracleError("backward: a query has an empty key list")
    return outs


def dq_tokens(Q, K, V, G, dOut, h: int, pl: Plan, csr, scale: float, tokens, means=None):
    """dq (fp64 [n_tok][D]) of the given query tokens of head h, as layer_bwd."""
    lib = _load()
    S, H, D = Q.shape
    qm, km, vm = means if means is not None else (tile_means(X, h, pl) for X in (Q, K, V))
    off, ids = csr
    toks = np.ascontiguousarray(np.asarray(list(tokens), dtype=np.int64))
    out = np.zeros((toks.size, D), dtype=np.float64)
    rc = lib.orc_dq_tokens(*(np.ascontiguousarray(X).reshape(-1) for X in (Q, K, V, G, dOut)),
                           H, D, int(h), pl.untile, pl.row_src, pl.block_len, pl.n_t, pl.B,
                           np.ascontiguousarray(off), ids, np.ascontiguousarray(qm).reshape(-1),
                           np.ascontiguousarray(km).reshape(-1), np.ascontiguousarray(vm).reshape(-1),
                           float(scale), toks, int(toks.size), out.reshape(-1))
    if rc != 0:
        raise OracleError("dq: a query has an empty key list")
    return out


def dkdv_tile(Q, K, V, G, dOut, h: int, pl: Plan, csr, scale: float, tile: int, means=None):
    """dk, dv (fp64 [B][D], tile rows in order, padding rows 0) of the key rows of
    one tile jt = `tile` of head h: the gradient orc_layer_bwd computes, restricted
    to those rows, for element-wise checks at full size.

    A key row u of tile jt receives gradient from the query tokens t whose tile's
    key list holds jt, plus the mean's share of the coarse path:
      dv[u] = dvm_jt / n_jt + sum_t p_tu dout_t,
      dk[u] = dkm_jt / n_jt + sum_t scale p_tu (dout_t . v_u - D_t) q_t,
    with p_tu the softmax of t over all of its keys, D_t = dout_t . O_fine[t], and
    (dkm, dvm)_jt the column jt of the tile-level attention's gradient (every query
    tile i contributes through P_c[i][jt], dO_c[i] = sum_{t in i} dout_t * g_t and
    D_c[i] = dO_c[i] . O_c[i]). Written with fp64 numpy matrix products as steps."""
    S, H, D = Q.shape
    B, n_t = pl.B, pl.n_t
    qm, km, vm = means if means is not None else (tile_means(X, h, pl) for X in (Q, K, V))
    qm, km, vm = (np.asarray(m, dtype=np.float64) for m in (qm, km, vm))
    x = lambda A: bf16_value(np.asarray(A)[:, h, :])                  # noqa: E731  fp64 [S][D]
    q, k, v, go = x(Q), x(K), x(V), x(dOut)
    g = bf16_value(np.asarray(G).reshape(S, H, D)[:, h, :])
    rows = pl.row_src.reshape(n_t, B)
    # coarse path: column jt of the tile attention's gradient
    z = scale * (qm @ km.T)
    pc = np.exp(z - z.max(axis=1, keepdims=True))
    pc /= pc.sum(axis=1, keepdims=True)
    oc = pc @ vm
    doc = np.zeros((n_t, D))
    real = pl.row_src >= 0
    np.add.at(doc, np.nonzero(real)[0] // B, go[pl.row_src[real]] * g[pl.row_src[real]])
    dc = (doc * oc).sum(axis=1)
    dz = pc[:, tile] * (doc @ vm[tile] - dc)
    dkm = scale * (dz @ qm)
    dvm = pc[:, tile] @ doc
    own = rows[tile]
    ok = own >= 0
    n_j = int(pl.block_len[tile])
    dk = np.zeros((B, D))
    dv = np.zeros((B, D))
    dk[ok] = dkm / n_j
    dv[ok] = dvm / n_j
    # fine path: every query tile whose key list holds jt, in ascending order
    off, ids = csr
    vj = v[own[ok]]

    def contribution(i):
        lst = ids[off[i]:off[i + 1]]
        blk = rows[lst]                                   # [tiles][B] key rows, -1 = padding
        keys = blk[blk >= 0]
        of_jt = np.repeat(lst, (blk >= 0).sum(axis=1)) == tile   # key columns of tile jt
        qi = rows[i][rows[i] >= 0]
        zi = scale * (q[qi] @ k[keys].T)
        p = np.exp(zi - zi.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        dt = (go[qi] * (p @ v[keys])).sum(axis=1)
        pj = p[:, of_jt]
        ds = pj * (go[qi] @ vj.T - dt[:, None])
        return scale * (ds.T @ q[qi]), pj.T @ go[qi]

    # the query tiles whose key list holds jt; computed on a thread pool (numpy
    # releases the interpreter lock), added in ascending order
    tiles = [i for i in range(n_t) if tile in ids[off[i]:off[i + 1]]]
    with threadpool_limits(1), ThreadPoolExecutor(len(os.sched_getaffinity(0))) as pool:
        parts = list(pool.map(contribution, tiles))
    for pk, pv in parts:
        dk[ok] += pk
        dv[ok] += pv
    return dk, dv


# ------------------------------------------------------- the layer, in order --

@dataclass
class HeadResult:
    """Everything the oracle computes for one head."""
    qm: np.ndarray          # fp32 [n_t][D] pooled Q
    km: np.ndarray
    vm: np.ndarray
    scores: np.ndarray      # fp32 [len(score_rows)][n_v]
    score_rows: np.ndarray  # video query positions that were scored
    keep: np.ndarray        # int32 [len(score_rows)][k]
    o_coarse: np.ndarray    # fp64 [n_t][D]


def head(Q, K, V, h: int, pl: Plan, k: int, scale: float,
         score_rows: Optional[Iterable[int]] = None) -> HeadResult:
    """Pool, score, select and coarse-attend one head (steps O3-O6)."""
    qm = tile_means(Q, h, pl)
    km = tile_means(K, h, pl)
    vm = tile_means(V, h, pl)
    rows = (np.arange(pl.n_v, dtype=np.int32) if score_rows is None
            else np.asarray(list(score_rows), dtype=np.int32))
    sc = video_scores(qm, km, pl.P, pl.n_v, rows)
    keep = topk_rows(sc, k, pl.P)
    oc = coarse_attn(qm, km, vm, scale)
    return HeadResult(qm, km, vm, sc, rows, keep, oc)


def layer_tokens(Q, K, V, g: np.ndarray, h: int, pl: Plan, hr: HeadResult, k: int, scale: float,
                 tokens: Iterable[int], g_is_rows: bool = False):
    """Outputs (bf16 bits [n_tok][D]) and O_fine (fp64) of selected tokens of head h.

    hr.keep must cover every video query tile (score_rows = all). g is the full
    bf16 gate [S][H*D] or, with g_is_rows, already the [n_tok][H*D] rows."""
    toks = np.asarray(list(tokens), dtype=np.int64)
    D = Q.shape[2]
    assert hr.keep.shape[0] == pl.n_v, "layer_tokens needs the keep lists of all video tiles"
    o_fine = fine_tokens(Q, K, V, h, pl, hr.keep, k, scale, toks)
    tiles = pl.untile[toks] // pl.B
    o_coarse = hr.o_coarse[tiles]
    g_rows = (g if g_is_rows else g[toks])[:, h * D:(h + 1) * D]
    return combine(o_fine, np.ascontiguousarray(g_rows), o_coarse), o_fine
