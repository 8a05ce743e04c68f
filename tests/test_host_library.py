"""libvsa host side, on the CPU: exports, plan parity with the oracle, plan
validation, keep-count, workspace layout, and argument checks of the GPU entry
points (which must fail before any device work, so no GPU is touched)."""
import ctypes
import os
import re

import numpy as np
import pytest

import tile_sparse_video_amd as tsv
import workloads
from tests.test_oracle_plan import _random_geometries

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "vsa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vsa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 11
    lib = ctypes.CDLL(tsv.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in vsa.h but not exported"
    assert set(tsv.EXPORTED) == set(names)


@pytest.mark.parametrize("segs,grid,tile", _random_geometries(30, seed=3))
def test_plan_matches_oracle(orc, segs, grid, tile):
    pl = tsv.vsa_plan_tiles(segs, grid, tile)
    o = orc.plan(segs, grid, tile)
    assert (pl.P, pl.n_v, pl.n_t, pl.B, pl.S, pl.S_pad) == (o.P, o.n_v, o.n_t, o.B, o.S, o.S_pad)
    assert np.array_equal(pl.untile, o.untile)
    assert np.array_equal(pl.row_src, o.row_src)
    assert np.array_equal(pl.block_len, o.block_len)
    tsv.vsa_plan_validate(pl)


@pytest.mark.parametrize("name", sorted(workloads.WORKLOADS))
def test_workload_plans_and_keep_counts(orc, name):
    wl = workloads.WORKLOADS[name]
    pl = tsv.cached_plan(wl.prefix_segments, wl.grid, wl.tile)
    o = orc.plan(wl.prefix_segments, wl.grid, wl.tile)
    assert np.array_equal(pl.row_src, o.row_src) and np.array_equal(pl.block_len, o.block_len)
    assert tsv.vsa_keep_count(pl.info, wl.sparsity, wl.keep_k) == \
        orc.keep_count(o.n_v, wl.sparsity, wl.keep_k)
    k = orc.keep_count(o.n_v, wl.sparsity, wl.keep_k)
    assert tsv.vsa_tile_pair_fraction(pl.info, k) == pytest.approx(
        orc.tile_pair_fraction(o.P, o.n_v, k), rel=1e-15)


def test_keep_count_matches_oracle_grid(orc):
    pl = tsv.vsa_plan_tiles([5], (4, 8, 12), (4, 4, 4))
    for s in np.linspace(-0.5, 1.5, 41):
        assert tsv.vsa_keep_count(pl.info, float(s)) == orc.keep_count(pl.n_v, float(s))
    for k in range(pl.n_v + 1):
        assert tsv.vsa_keep_count(pl.info, keep_k=k) == k
    for bad in (dict(keep_k=pl.n_v + 1), dict(sparsity=float("nan"))):
        with pytest.raises(tsv.VsaError) as e:
            tsv.vsa_keep_count(pl.info, **bad)
        assert e.value.status == tsv.VSA_ERR_ARG


def _expect_plan_error(pl, **arrays):
    with pytest.raises(tsv.VsaError) as e:
        tsv.vsa_plan_validate(pl, **arrays)
    assert e.value.status == tsv.VSA_ERR_PLAN


def test_validate_rejects_corrupted_plans():
    pl = tsv.vsa_plan_tiles([30, 70], (5, 6, 9), (4, 4, 4))
    # non-injective untile map
    u = pl.untile.copy()
    u[3] = u[4]
    _expect_plan_error(pl, untile=u)
    # row_src not the inverse of untile
    r = pl.row_src.copy()
    a, b = pl.untile[0], pl.untile[1]
    r[a], r[b] = r[b], r[a]
    _expect_plan_error(pl, row_src=r)
    # a tile whose real rows are not packed first (swap a real row with padding)
    t = int(np.nonzero(pl.block_len < pl.B)[0][0])
    r = pl.row_src.copy()
    u = pl.untile.copy()
    last = t * pl.B + pl.block_len[t] - 1
    tok = r[last]
    r[last], r[t * pl.B + pl.B - 1] = -1, tok
    u[tok] = t * pl.B + pl.B - 1
    _expect_plan_error(pl, row_src=r, untile=u)
    # a tile mixing the prefix and the video (swap one prefix and one video token)
    r = pl.row_src.copy()
    u = pl.untile.copy()
    pa, va = pl.untile[0], pl.untile[pl.S - 1]
    r[pa], r[va] = r[va], r[pa]
    u[r[pa]], u[r[va]] = pa, va
    _expect_plan_error(pl, row_src=r, untile=u)
    # wrong block_len
    bl = pl.block_len.copy()
    bl[0] -= 1
    _expect_plan_error(pl, block_len=bl)


def test_plan_argument_errors():
    for args in (([4], (0, 4, 4), (4, 4, 4)), ([-1], (4, 4, 4), (4, 4, 4)),
                 ([4], (4, 4, 4), (4, 0, 4))):
        with pytest.raises(tsv.VsaError) as e:
            tsv.vsa_plan_tiles(*args)
        assert e.value.status == tsv.VSA_ERR_ARG
    # padded rows must fit int32 indices
    with pytest.raises(tsv.VsaError) as e:
        tsv.vsa_plan_tiles([], (4096, 4096, 256), (4, 4, 4))
    assert e.value.status == tsv.VSA_ERR_ARG


def test_workspace_layout():
    wl = workloads.WORKLOADS["h3"]
    pl = tsv.cached_plan(wl.prefix_segments, wl.grid, wl.tile)
    lay = tsv.vsa_workspace_layout(pl.info, wl.heads, wl.head_dim)
    H, D, n_t, n_v = wl.heads, wl.head_dim, pl.n_t, pl.n_v
    regions = [("k_tiled", H * pl.S_pad * D * 2), ("v_tiled", H * pl.S_pad * D * 2),
               ("q_mean", H * n_t * D * 4), ("k_mean", H * n_t * D * 4),
               ("v_mean", H * n_t * D * 4), ("scores", H * n_v * n_v * 4)]
    end = 0
    for name, size in regions:
        off = getattr(lay, name)
        assert off % 256 == 0 and off >= end
        end = off + size
    assert lay.part_o >= end and lay.total_bytes >= lay.part_ml
    # a 48 MiB head of 64-row tiles splits its key lists into two phases of 8 chunks:
    # room for 16 chunk partials per 64 query rows
    items = H * n_t
    assert lay.part_ml - lay.part_o >= items * 16 * 64 * D * 2
    assert lay.split_chunks == 16
    # the split is an argument: layouts of different splits coexist, and only the
    # partials (placed last) depend on it
    one = tsv.vsa_workspace_layout(pl.info, H, D, 1)
    eight = tsv.vsa_workspace_layout(pl.info, H, D, 8)
    assert one.split_chunks == 1 and eight.split_chunks == 8
    assert one.total_bytes == one.part_o < eight.total_bytes < lay.total_bytes
    for name in ("k_tiled", "v_tiled", "q_mean", "k_mean", "v_mean", "scores", "k_i8", "k_scale",
                 "part_o"):
        assert getattr(one, name) == getattr(lay, name) == getattr(eight, name)
    assert lay.part_ml - lay.part_o == 2 * (eight.part_ml - eight.part_o)
    assert tsv.vsa_workspace_layout(pl.info, H, D, 0).total_bytes == lay.total_bytes
    for bad in (-1, 65):
        with pytest.raises(tsv.VsaError) as e:
            tsv.vsa_workspace_layout(pl.info, H, D, bad)
        assert e.value.status == tsv.VSA_ERR_ARG


def test_automatic_split_rule():
    """1 chunk up to 16 MiB of K+V per head; 8 beyond; at least 16 (two phases) for 64-row
    tiles beyond 32 MiB; 8 per started 96 MiB beyond that."""
    want = {"tiny": 1, "mid": 1, "page5": 8, "h3": 16, "veda": 8, "long": 16}
    for name, c in want.items():
        wl = workloads.WORKLOADS[name]
        pl = tsv.cached_plan(wl.prefix_segments, wl.grid, wl.tile)
        assert tsv.vsa_workspace_layout(pl.info, wl.heads, wl.head_dim).split_chunks == c, name


def test_workspace_layout_unsupported():
    pl = tsv.vsa_plan_tiles([10], (4, 4, 4), (4, 4, 4))
    with pytest.raises(tsv.VsaError) as e:
        tsv.vsa_workspace_layout(pl.info, 2, 96)
    assert e.value.status == tsv.VSA_ERR_UNSUPPORTED
    small = tsv.vsa_plan_tiles([10], (4, 4, 4), (2, 2, 2))   # 8-row tiles
    with pytest.raises(tsv.VsaError) as e:
        tsv.vsa_workspace_layout(small.info, 2, 64)
    assert e.value.status == tsv.VSA_ERR_UNSUPPORTED


# ---- GPU entry points: argument errors are reported before any device call.
# Pointers below are never dereferenced: every case fails validation first.

FAKE = 0x10000


def _coarse(info, heads=2, head_dim=128, sparsity=float("nan"), keep_k=1, scale=0.0,
            ptrs=(FAKE,) * 5, ws_bytes=1 << 40, keep=FAKE, oc=FAKE):
    lib = tsv._lib
    return lib.vsa_coarse_topk(ctypes.byref(info), ptrs[0], ptrs[1], heads, head_dim, sparsity,
                               keep_k, scale, ptrs[2], ptrs[3], ptrs[4], FAKE * 2, ws_bytes, keep,
                               oc, None)


def _fine(info, heads=2, head_dim=128, k=1, scale=0.0, ws_bytes=1 << 40, keep=FAKE,
          q=FAKE, gate=FAKE, out=FAKE, split=0):
    lib = tsv._lib
    return lib.vsa_sparse_attn_fwd(ctypes.byref(info), FAKE, FAKE, heads, head_dim, k, scale, split,
                                   q, FAKE * 2, ws_bytes, keep, FAKE, gate, out, None)


def test_gpu_entry_points_reject_bad_arguments():
    pl = tsv.vsa_plan_tiles([20, 40], (4, 8, 8), (4, 4, 4))
    info = pl.info
    E = tsv
    cases = [
        (_coarse(info, head_dim=96), E.VSA_ERR_UNSUPPORTED),
        (_coarse(info, heads=0), E.VSA_ERR_ARG),
        (_coarse(info, keep_k=pl.n_v + 1), E.VSA_ERR_ARG),
        (_coarse(info, keep_k=-1), E.VSA_ERR_ARG),                  # NaN sparsity
        (_coarse(info, ptrs=(0, FAKE, FAKE, FAKE, FAKE)), E.VSA_ERR_ARG),
        (_coarse(info, keep=0), E.VSA_ERR_ARG),                     # k > 0 needs keep_idx
        (_coarse(info, ws_bytes=1024), E.VSA_ERR_ARG),
        (_coarse(info, scale=float("inf")), E.VSA_ERR_ARG),
        (_fine(info, head_dim=80), E.VSA_ERR_UNSUPPORTED),
        (_fine(info, k=pl.n_v + 1), E.VSA_ERR_ARG),
        (_fine(info, q=0), E.VSA_ERR_ARG),
        (_fine(info, ws_bytes=1024), E.VSA_ERR_ARG),
        (_fine(info, keep=0), E.VSA_ERR_ARG),
        (_fine(info, split=-1), E.VSA_ERR_ARG),
        (_fine(info, split=65), E.VSA_ERR_ARG),
    ]
    for got, want in cases:
        assert got == want, (got, want, tsv._lib.vsa_last_error())
    # empty key set: no prefix tiles and k = 0
    nopre = tsv.vsa_plan_tiles([], (4, 8, 8), (4, 4, 4))
    assert _fine(nopre.info, k=0, keep=0) == E.VSA_ERR_ARG
    assert b"empty key set" in tsv._lib.vsa_last_error()
    # inconsistent plan info
    bad = tsv.vsa_plan_info.from_buffer_copy(info)
    bad.n_tiles += 1
    assert _fine(bad) == E.VSA_ERR_PLAN
    # gate projection shapes
    lib = tsv._lib
    assert lib.vsa_gate_proj(FAKE, FAKE, 10, 100, 64, FAKE, None) == E.VSA_ERR_UNSUPPORTED
    assert lib.vsa_gate_proj(0, FAKE, 10, 128, 64, FAKE, None) == E.VSA_ERR_ARG
    assert lib.vsa_gate_proj(FAKE, FAKE, -1, 128, 64, FAKE, None) == E.VSA_ERR_ARG


def test_status_strings():
    lib = tsv._lib
    for code in (0, -1, -2, -3, -4):
        assert lib.vsa_status_string(code)
    assert lib.vsa_status_string(7) == b"unknown status"


def test_kernel_timing_host_side():
    lib = tsv._lib
    s0, s1 = 0, 0x1234000   # stream handles as keys only: nothing is enqueued on them
    tsv.vsa_timing_enable(True, stream=s0)
    try:
        for name in tsv.TIMED_KERNELS:
            assert tsv.vsa_timing_read(name, stream=s0) == (0, 0.0)   # nothing launched since enable
        with pytest.raises(tsv.VsaError) as e:
            tsv.vsa_timing_read("not_a_kernel", stream=s0)
        assert e.value.status == tsv.VSA_ERR_ARG
        assert lib.vsa_timing_read(None, b"fine_attn", None, None) == tsv.VSA_ERR_ARG
        # timing is per stream: a stream never enabled reads as empty, and enabling
        # or disabling one stream leaves another's state alone
        assert tsv.vsa_timing_read("fine_attn", stream=s1) == (0, 0.0)
        tsv.vsa_timing_enable(True, stream=s1)
        tsv.vsa_timing_enable(False, stream=s1)
        assert tsv.vsa_timing_read("fine_attn", stream=s0) == (0, 0.0)
    finally:
        tsv.vsa_timing_enable(False, stream=s0)
    # failed launches (argument errors) record nothing
    pl = tsv.vsa_plan_tiles([20, 40], (4, 8, 8), (4, 4, 4))
    tsv.vsa_timing_enable(True, stream=s0)
    try:
        assert _fine(pl.info, head_dim=80) == tsv.VSA_ERR_UNSUPPORTED
        assert tsv.vsa_timing_read("fine_attn", stream=s0) == (0, 0.0)
    finally:
        tsv.vsa_timing_enable(False, stream=s0)


# ---- reference-sparsity mode: host-side checks

def test_ref_keep_count_matches_oracle(orc):
    for name in sorted(workloads.WORKLOADS):
        wl = workloads.WORKLOADS[name]
        pl = tsv.cached_plan(wl.prefix_segments, wl.grid, wl.tile)
        o = orc.plan(wl.prefix_segments, wl.grid, wl.tile)
        for s in (0.0, 0.5, 0.9, 1.0, -0.3):
            k_ref, k_gen = orc.ref_keep_counts(o, s, None, s, None)
            assert tsv.vsa_ref_keep_count(pl.info, s) == k_ref
            assert tsv.vsa_tile_pair_fraction_ref(pl.info, k_ref, k_gen) == pytest.approx(
                orc.tile_pair_fraction_ref(o.n_t, k_ref, k_gen), rel=1e-15)
        assert tsv.vsa_ref_keep_count(pl.info, ref_keep_k=pl.P) == pl.P
        with pytest.raises(tsv.VsaError) as e:
            tsv.vsa_ref_keep_count(pl.info, ref_keep_k=pl.P + 1)
        assert e.value.status == tsv.VSA_ERR_ARG
    with pytest.raises(tsv.VsaError):
        tsv.vsa_ref_keep_count(pl.info, float("nan"))
    with pytest.raises(tsv.VsaError):
        tsv.vsa_tile_pair_fraction_ref(pl.info, pl.P + 1, 0)


def test_workspace_scores_region_holds_all_tile_pairs():
    wl = workloads.WORKLOADS["h3"]
    pl = tsv.cached_plan(wl.prefix_segments, wl.grid, wl.tile)
    lay = tsv.vsa_workspace_layout(pl.info, wl.heads, wl.head_dim)
    assert lay.part_o - lay.scores >= wl.heads * pl.n_t * pl.n_t * 4


def test_ref_entry_points_reject_bad_arguments():
    pl = tsv.vsa_plan_tiles([20, 40], (4, 8, 8), (4, 4, 4))
    info = pl.info
    lib = tsv._lib

    def coarse(heads=2, head_dim=128, sparsity=0.5, keep_k=-1, rs=0.5, rk=-1, keep=FAKE,
               ws_bytes=1 << 40, scale=0.0):
        return lib.vsa_coarse_topk_ref(ctypes.byref(info), FAKE, FAKE, heads, head_dim, sparsity,
                                       keep_k, rs, rk, scale, FAKE, FAKE, FAKE, FAKE * 2, ws_bytes,
                                       keep, FAKE, None)

    def fine(heads=2, head_dim=128, k_ref=1, k_gen=1, keep=FAKE, ws_bytes=1 << 40):
        return lib.vsa_sparse_attn_fwd_ref(ctypes.byref(info), FAKE, FAKE, heads, head_dim, k_ref,
                                           k_gen, 0.0, 0, FAKE, FAKE * 2, ws_bytes, keep, FAKE, FAKE,
                                           FAKE, None)

    E = tsv
    cases = [
        (coarse(head_dim=96), E.VSA_ERR_UNSUPPORTED),
        (coarse(heads=0), E.VSA_ERR_ARG),
        (coarse(rk=pl.P + 1), E.VSA_ERR_ARG),
        (coarse(rs=float("nan")), E.VSA_ERR_ARG),
        (coarse(keep_k=pl.n_v + 1), E.VSA_ERR_ARG),
        (coarse(keep=0), E.VSA_ERR_ARG),
        (coarse(ws_bytes=4096), E.VSA_ERR_ARG),
        (coarse(scale=float("nan")), E.VSA_ERR_ARG),
        (fine(k_ref=0, k_gen=0, keep=0), E.VSA_ERR_ARG),   # empty key set
        (fine(k_ref=pl.P + 1), E.VSA_ERR_ARG),
        (fine(k_gen=pl.n_v + 1), E.VSA_ERR_ARG),
        (fine(keep=0), E.VSA_ERR_ARG),
        (fine(head_dim=80), E.VSA_ERR_UNSUPPORTED),
        (fine(ws_bytes=4096), E.VSA_ERR_ARG),
    ]
    for got, want in cases:
        assert got == want, (got, want, lib.vsa_last_error())
    assert b"empty key set" in (fine(k_ref=0, k_gen=0, keep=0), lib.vsa_last_error())[1]


def test_i8_entry_point_rejects_bad_arguments():
    pl = tsv.vsa_plan_tiles([20, 40], (4, 8, 8), (4, 4, 4))
    info = pl.info
    lib = tsv._lib

    def fine(heads=2, head_dim=128, k_ref=-1, k_gen=1, keep=FAKE, ws_bytes=1 << 40, q=FAKE,
             scale=0.0):
        return lib.vsa_sparse_attn_fwd_i8(ctypes.byref(info), FAKE, FAKE, heads, head_dim, k_ref,
                                          k_gen, scale, 0, q, FAKE * 2, ws_bytes, keep, FAKE,
                                          FAKE, FAKE, None)

    E = tsv
    cases = [
        (fine(head_dim=96), E.VSA_ERR_UNSUPPORTED),
        (fine(heads=0), E.VSA_ERR_ARG),
        (fine(k_gen=pl.n_v + 1), E.VSA_ERR_ARG),
        (fine(k_ref=pl.P + 1), E.VSA_ERR_ARG),                 # ref mode: k_ref beyond P
        (fine(k_ref=0, k_gen=0), E.VSA_ERR_ARG),               # ref mode: empty key set
        (fine(q=0), E.VSA_ERR_ARG),
        (fine(keep=0), E.VSA_ERR_ARG),
        (fine(ws_bytes=1024), E.VSA_ERR_ARG),
        (fine(scale=float("nan")), E.VSA_ERR_ARG),
    ]
    for got, want in cases:
        assert got == want, (got, want, lib.vsa_last_error())
    assert b"vsa_sparse_attn_fwd_i8" in lib.vsa_last_error()
    # the INT8 regions: one byte per K element and one scale per 64-row block
    wl = workloads.WORKLOADS["h3"]
    big = tsv.cached_plan(wl.prefix_segments, wl.grid, wl.tile)
    lay = tsv.vsa_workspace_layout(big.info, wl.heads, wl.head_dim)
    assert lay.k_i8 % 256 == 0 and lay.k_scale % 256 == 0
    assert lay.k_scale - lay.k_i8 >= wl.heads * big.S_pad * wl.head_dim
    assert lay.part_o - lay.k_scale >= wl.heads * big.S_pad // 64 * 4
    assert lay.k_i8 >= lay.scores and lay.part_o >= lay.k_scale


def test_group_entry_point_rejects_bad_arguments():
    """vsa_layer_fwd_groups validates every group before enqueuing anything."""
    lib = tsv._lib
    a = tsv.vsa_plan_tiles([20, 40], (4, 8, 8), (4, 4, 4))
    b = tsv.vsa_plan_tiles([20, 40], (4, 8, 8), (1, 8, 8))
    other = tsv.vsa_plan_tiles([20, 41], (4, 8, 8), (4, 4, 4))   # one token more

    def group(pl, first, heads, keep_k=1, ws=FAKE, ref=0, ref_keep_k=-1, split=0):
        g = tsv.vsa_head_group()
        g.info = ctypes.pointer(pl.info)
        g.row_src_dev = g.block_len_dev = FAKE
        g.head_first, g.heads = first, heads
        g.sparsity, g.keep_k = float("nan"), keep_k
        g.ref, g.int8, g.ref_sparsity, g.ref_keep_k = ref, 0, float("nan"), ref_keep_k
        g.split_chunks = split
        g.workspace, g.workspace_bytes = ws, 1 << 40
        g.keep_idx_dev = g.o_coarse_dev = FAKE
        return g

    def call(groups, heads_total=4, head_dim=128):
        arr = (tsv.vsa_head_group * max(1, len(groups)))(*groups)
        return lib.vsa_layer_fwd_groups(arr, len(groups), heads_total, head_dim, 0.0, FAKE, FAKE,
                                        FAKE, FAKE, FAKE, None)

    E = tsv
    assert call([]) == E.VSA_ERR_ARG
    assert call([group(a, 0, 2), group(b, 1, 2)]) == E.VSA_ERR_ARG        # head 1 twice
    assert b"more than one group" in lib.vsa_last_error()
    assert call([group(a, 0, 2), group(b, 2, 3)]) == E.VSA_ERR_ARG        # beyond heads_total
    assert call([group(a, -1, 2)]) == E.VSA_ERR_ARG
    assert call([group(a, 0, 2), group(other, 2, 2)]) == E.VSA_ERR_ARG    # token counts differ
    assert b"tokens" in lib.vsa_last_error()
    assert call([group(a, 0, 2), group(b, 2, 2, keep_k=10 ** 6)]) == E.VSA_ERR_ARG
    assert b"group 1" in lib.vsa_last_error()
    assert call([group(a, 0, 2, ref=1, ref_keep_k=a.P + 1)]) == E.VSA_ERR_ARG
    # pointers and workspaces are checked up front too (null workspace in group 1)
    assert call([group(a, 0, 2), group(b, 2, 2, ws=0)]) == E.VSA_ERR_ARG
    assert b"group 1" in lib.vsa_last_error()
    assert call([group(a, 0, 2), group(b, 2, 2, ws=FAKE + 8)]) == E.VSA_ERR_ARG   # misaligned
    assert call([group(a, 0, 2)], head_dim=96) == E.VSA_ERR_UNSUPPORTED
    assert call([group(a, 0, 2), group(b, 2, 2, split=65)]) == E.VSA_ERR_ARG   # bad split
    assert b"group 1" in lib.vsa_last_error()


def test_heads_beyond_4gib_are_rejected():
    """A head's tile-ordered K is addressed through one 32-bit buffer resource."""
    info = tsv.vsa_plan_info()
    info.grid[:] = (256, 256, 256)
    info.tile[:] = (4, 4, 4)
    info.tile_rows, info.n_prefix_tiles = 64, 0
    info.n_video_tiles = info.n_tiles = 64 * 64 * 64
    info.rows_real = info.rows_padded = 256 ** 3      # 2^24 rows x 128 x 2 B = 4 GiB
    info.prefix_rows = 0
    lib = tsv._lib
    rc = lib.vsa_sparse_attn_fwd(ctypes.byref(info), FAKE, FAKE, 1, 128, 1, 0.0, 0, FAKE, FAKE * 2,
                                 1 << 50, FAKE, FAKE, FAKE, FAKE, None)
    assert rc == tsv.VSA_ERR_UNSUPPORTED, lib.vsa_last_error()
    assert b"4 GiB" in lib.vsa_last_error()
    rc = lib.vsa_sparse_attn_bwd(ctypes.byref(info), FAKE, FAKE, 1, 128, -1, 1, 0.0, 0, FAKE, FAKE,
                                 FAKE, FAKE, FAKE, FAKE * 2, 1 << 50, FAKE, FAKE, FAKE * 2, 1 << 50,
                                 FAKE, FAKE, FAKE, FAKE, 0, None)
    assert rc == tsv.VSA_ERR_UNSUPPORTED, lib.vsa_last_error()
    # head_dim 64 halves the bytes: the same plan passes this check (and fails later on the
    # fake workspace size, still before any device work)
    rc = lib.vsa_sparse_attn_fwd(ctypes.byref(info), FAKE, FAKE, 1, 64, 1, 0.0, 0, FAKE, FAKE * 2,
                                 1024, FAKE, FAKE, FAKE, FAKE, None)
    assert rc == tsv.VSA_ERR_ARG and b"workspace" in lib.vsa_last_error()


def test_training_forward_rejects_bad_arguments():
    pl = tsv.vsa_plan_tiles([20, 40], (4, 8, 8), (4, 4, 4))
    info = pl.info
    lib = tsv._lib

    def call(bw=FAKE * 4, bw_bytes=1 << 40, heads=2, head_dim=128, k_gen=1):
        return lib.vsa_sparse_attn_fwd_train(ctypes.byref(info), FAKE, FAKE, heads, head_dim, -1,
                                             k_gen, 0.0, 0, FAKE, FAKE * 2, 1 << 40, FAKE, FAKE,
                                             FAKE, FAKE, bw, bw_bytes, None)

    E = tsv
    assert call(bw=0) == E.VSA_ERR_ARG
    assert call(bw_bytes=1024) == E.VSA_ERR_ARG
    assert b"backward workspace" in lib.vsa_last_error()
    assert call(bw=FAKE * 4 + 8) == E.VSA_ERR_ARG                  # misaligned
    assert call(head_dim=96) == E.VSA_ERR_UNSUPPORTED
    assert call(k_gen=pl.n_v + 1) == E.VSA_ERR_ARG                 # checked by the forward body
    assert b"vsa_sparse_attn_fwd_train" in lib.vsa_last_error()
    # the O_fine region exists only for heads that split their key lists
    wl = workloads.WORKLOADS["h3"]
    big = tsv.cached_plan(wl.prefix_segments, wl.grid, wl.tile)
    lay = tsv.vsa_bwd_workspace_layout(big.info, wl.heads, wl.head_dim)
    assert lay.total_bytes - lay.ofine >= wl.heads * big.S_pad * wl.head_dim * 4
    small = tsv.vsa_bwd_workspace_layout(info, 2, 128)
    assert small.total_bytes == small.ofine


def test_bwd_layout_transposed_list_regions():
    """The backward workspace holds the transposed key lists ([H][n_t][n_t] int32),
    their counts, and the bit matrix they are built from ([H][n_t][ceil(n_t / 32)]
    words), as disjoint 256-byte-aligned regions in that order."""
    import tile_sparse_video_amd as tsv
    for name in ("tiny", "h3", "page5"):
        wl = workloads.WORKLOADS[name]
        pl = tsv.cached_plan(wl.prefix_segments, wl.grid, wl.tile)
        n_t = pl.info.n_tiles
        lay = tsv.vsa_bwd_workspace_layout(pl.info, wl.heads, wl.head_dim)
        words = (n_t + 31) // 32
        assert lay.tcount - lay.tlist >= wl.heads * n_t * n_t * 4
        assert lay.tbits - lay.tcount >= wl.heads * n_t * 4
        assert lay.part_dq - lay.tbits >= wl.heads * n_t * words * 4
        assert lay.part_dq - lay.tbits < wl.heads * n_t * words * 4 + 256
        for off in (lay.tlist, lay.tcount, lay.tbits, lay.part_dq):
            assert off % 256 == 0


def test_static_entry_point_rejects_before_device_work():
    """vsa_layer_fwd_static: arguments and the static workspace's size are checked
    before anything touches a device."""
    lib = tsv._lib
    wl = workloads.WORKLOADS["h3"]
    big = tsv.cached_plan(wl.prefix_segments, wl.grid, wl.tile)
    small = tsv.vsa_plan_tiles([20, 40], (4, 8, 8), (4, 4, 4))

    def call(info, heads=2, head_dim=128, keep_k=1, gate=FAKE, keep=FAKE, scale=0.0):
        return lib.vsa_layer_fwd_static(ctypes.byref(info), FAKE, FAKE, heads, head_dim,
                                        float("nan"), keep_k, scale, FAKE, FAKE, FAKE, gate, keep,
                                        FAKE, FAKE, None)

    assert call(big.info, heads=wl.heads, keep_k=378) == tsv.VSA_ERR_ARG
    assert b"static one holds" in lib.vsa_last_error()
    need = tsv.vsa_workspace_layout(big.info, wl.heads, wl.head_dim, 1).total_bytes
    assert need > tsv.STATIC_WORKSPACE_BYTES
    mid = workloads.WORKLOADS["mid"]
    mp = tsv.cached_plan(mid.prefix_segments, mid.grid, mid.tile)
    assert tsv.vsa_workspace_layout(mp.info, mid.heads, mid.head_dim, 1).total_bytes \
        <= tsv.STATIC_WORKSPACE_BYTES
    assert call(small.info, head_dim=96) == tsv.VSA_ERR_UNSUPPORTED
    assert call(small.info, gate=0) == tsv.VSA_ERR_ARG
    assert call(small.info, keep=0) == tsv.VSA_ERR_ARG
    assert call(small.info, keep_k=small.n_v + 1) == tsv.VSA_ERR_ARG
    assert call(small.info, scale=float("inf")) == tsv.VSA_ERR_ARG
    nopre = tsv.vsa_plan_tiles([], (4, 8, 8), (4, 4, 4))
    assert call(nopre.info, keep_k=0, keep=0) == tsv.VSA_ERR_ARG
    assert b"empty key set" in lib.vsa_last_error()


def test_producer_rejects_before_device_work():
    """vsa_qkv_gate_proj validates shapes, pointers and the workspace up front."""
    pl = tsv.vsa_plan_tiles([5, 70, 1], (5, 6, 9), (4, 4, 4))
    lib = tsv._lib

    def call(heads=3, head_dim=128, hidden=128, ws_bytes=1 << 40, x=FAKE, ws=FAKE * 2):
        return lib.vsa_qkv_gate_proj(ctypes.byref(pl.info), FAKE, FAKE, heads, head_dim, hidden, x,
                                     FAKE, FAKE, FAKE, ws, ws_bytes, None)

    assert call(head_dim=96) == tsv.VSA_ERR_UNSUPPORTED
    assert call(hidden=100) == tsv.VSA_ERR_UNSUPPORTED
    assert call(heads=1, head_dim=64) == tsv.VSA_ERR_UNSUPPORTED     # H*D = 64
    assert call(heads=0) == tsv.VSA_ERR_ARG
    assert call(x=0) == tsv.VSA_ERR_ARG
    assert call(ws_bytes=1024) == tsv.VSA_ERR_ARG
    assert call(ws=FAKE * 2 + 8) == tsv.VSA_ERR_ARG                   # misaligned
    lay = tsv.vsa_workspace_layout(pl.info, 3, 128, 1)
    assert call(ws_bytes=lay.part_o - 1) == tsv.VSA_ERR_ARG
    assert b"workspace" in lib.vsa_last_error()
