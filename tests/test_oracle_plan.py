"""Pins for the oracle's tile plan and keep-count (CPU only).

The plan is pinned by the worked example the SnackOnAI analysis prints (see
tests/golden/page5_geometry.json), by the tile counts stated with each layer
workload, and by an independent closed form of every token's padded row.
"""
import json
import os

import numpy as np
import pytest

from workloads import WORKLOADS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page5_geometry.json")


def expected_rows(prefix_segments, grid, tile):
    """Each token's padded row from its coordinates alone (closed form).

    Prefix token at offset o of segment m: tile (tiles before m) + o // B, row o % B.
    Video token (t, y, x): tile (t//tt, y//th, x//tw) in t-major tile order after
    the prefix; inside a tile the real tokens form a box of extent
    (min(tt, T-t0), min(th, Hg-h0), min(tw, Wg-w0)) visited lexicographically.
    """
    tt, th, tw = tile
    B = tt * th * tw
    T, Hg, Wg = grid
    rows = []
    tiles_before = 0
    for L in prefix_segments:
        o = np.arange(L)
        rows.append((tiles_before + o // B) * B + o % B)
        tiles_before += -(-L // B)
    P = tiles_before
    nH, nW = -(-Hg // th), -(-Wg // tw)
    t, y, x = np.meshgrid(np.arange(T), np.arange(Hg), np.arange(Wg), indexing="ij")
    t, y, x = t.reshape(-1), y.reshape(-1), x.reshape(-1)
    bt, by, bx = t // tt, y // th, x // tw
    tile_id = P + (bt * nH + by) * nW + bx
    eh = np.minimum(th, Hg - by * th)
    ew = np.minimum(tw, Wg - bx * tw)
    rank = (t - bt * tt) * eh * ew + (y - by * th) * ew + (x - bx * tw)
    rows.append(tile_id * B + rank)
    return np.concatenate(rows).astype(np.int64), P


def test_page5_worked_example(orc):
    g = json.load(open(GOLDEN))
    pl = orc.plan(g["prefix_segments"], g["grid"], g["tile"])
    assert pl.B == g["tile_rows"]
    assert pl.S == g["rows_real"]
    assert pl.S - sum(g["prefix_segments"]) == g["video_tokens"]
    assert pl.P == g["n_prefix_tiles"]
    assert pl.n_v == g["n_video_tiles"]
    assert pl.n_t == g["n_tiles"]
    assert pl.S_pad == g["rows_padded"]
    assert round(100 * (pl.S_pad / pl.S - 1)) == g["padding_overhead_rounded_pct"]
    k75 = orc.keep_count(pl.n_v, sparsity=0.75)
    assert k75 == g["keep_k_at_sparsity_0.75"]
    assert round(100 * orc.tile_pair_fraction(pl.P, pl.n_v, k75), 1) == \
        g["pair_fraction_at_0.75_rounded_pct_1dp"]
    k90 = orc.keep_count(pl.n_v, sparsity=0.90)
    assert round(100 * orc.tile_pair_fraction(pl.P, pl.n_v, k90), 1) == \
        g["pair_fraction_at_0.90_rounded_pct_1dp"]
    # partial edge tiles: 37 = 9*4 + 1 frames, 42 = 10*4 + 2 columns
    video_bl = set(pl.block_len[pl.P:].tolist())
    assert video_bl == {64, 32, 16, 8}


@pytest.mark.parametrize("name,P,n_v,k", [
    ("tiny", 2, 4, 2), ("mid", 22, 64, 16), ("h3", 26, 1512, 378),
    ("veda", 13, 1008, 101), ("long", 26, 5544, 277)])
def test_workload_tile_counts(orc, name, P, n_v, k):
    """Tile counts and keep-counts stated with each layer workload."""
    wl = WORKLOADS[name]
    pl = orc.plan(wl.prefix_segments, wl.grid, wl.tile)
    assert (pl.P, pl.n_v) == (P, n_v)
    assert orc.keep_count(pl.n_v, wl.sparsity, wl.keep_k) == k
    assert pl.S == wl.tokens


def _random_geometries(n, seed=0):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        tile = tuple(int(v) for v in rng.choice([1, 2, 3, 4, 8], size=3))
        grid = tuple(int(v) for v in rng.integers(1, 13, size=3))
        segs = tuple(int(v) for v in rng.integers(0, 150, size=int(rng.integers(0, 5))))
        out.append((segs, grid, tile))
    out.append(((0, 5, 0, 64), (3, 5, 7), (4, 4, 4)))
    out.append(((), (4, 8, 8), (4, 4, 4)))
    return out


@pytest.mark.parametrize("segs,grid,tile", _random_geometries(40))
def test_plan_matches_closed_form(orc, segs, grid, tile):
    pl = orc.plan(segs, grid, tile)
    exp, P = expected_rows(segs, grid, tile)
    assert pl.P == P
    assert np.array_equal(pl.untile.astype(np.int64), exp)
    # row_src is the inverse map; every other row is padding
    inv = np.full(pl.S_pad, -1, dtype=np.int64)
    inv[exp] = np.arange(pl.S)
    assert np.array_equal(pl.row_src.astype(np.int64), inv)


@pytest.mark.parametrize("segs,grid,tile", _random_geometries(25, seed=1))
def test_plan_invariants(orc, segs, grid, tile):
    pl = orc.plan(segs, grid, tile)
    # injective untile map (the pages' node refuses a non-injective map)
    assert np.unique(pl.untile).size == pl.S
    assert int(pl.block_len.sum()) == pl.S
    assert (pl.block_len >= 1).all() and (pl.block_len <= pl.B).all()
    # real rows are packed first inside each tile
    rs = pl.row_src.reshape(pl.n_t, pl.B)
    for t in range(pl.n_t):
        n = pl.block_len[t]
        assert (rs[t, :n] >= 0).all() and (rs[t, n:] == -1).all()
    # segment purity: a tile never mixes two prefix segments, or prefix and video
    seg_of = np.concatenate([np.full(L, m) for m, L in enumerate(segs)] +
                            [np.full(pl.S - sum(segs), len(segs))]).astype(np.int64)
    for t in range(pl.n_t):
        toks = rs[t, :pl.block_len[t]]
        assert np.unique(seg_of[toks]).size == 1
        assert (t < pl.P) == (seg_of[toks[0]] < len(segs))


def test_keep_count_rules(orc):
    # keep ratio = clamp(1 - sparsity, 0, 1)
    assert orc.keep_count(100, sparsity=1.5) == 0
    assert orc.keep_count(100, sparsity=-0.5) == 100
    assert orc.keep_count(100, sparsity=0.0) == 100
    # round half up: 0.25 * 10 = 2.5 -> 3 ; integer k is exact
    assert orc.keep_count(10, sparsity=0.75) == 3
    assert orc.keep_count(1008, keep_k=24) == 24
    with pytest.raises(orc.OracleError):
        orc.keep_count(10, keep_k=11)
    with pytest.raises(orc.OracleError):
        orc.keep_count(10, sparsity=float("nan"))


def test_plan_rejects_bad_arguments(orc):
    with pytest.raises(orc.OracleError):
        orc.plan([10], (0, 4, 4), (4, 4, 4))
    with pytest.raises(orc.OracleError):
        orc.plan([-1], (4, 4, 4), (4, 4, 4))
