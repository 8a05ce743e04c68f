"""Pins for the oracle's reference-sparsity variant (CPU only).

[Veda] "ComfyUI node" inputs table: reference_sparsity applies the same top-k
setting to the reference tokens, and 0 % means full attention. Reading: every
query tile keeps its top-k_ref prefix (reference) key tiles and its top-k_gen
video key tiles. Checked against: torch SDPA (fp64) with a token mask built
from tile coordinates, dense SDPA at zero sparsity, brute-force sorts per key
group, the fp64 dot within the fp32 FMA-chain error bound, and the page's
keep-count rule applied to the prefix tiles.
"""
import numpy as np
import pytest

from tests.test_oracle_numerics import brute_topk, rand_bf16, sdpa64, U32
from tests.test_oracle_plan import expected_rows


def list_mask(segs, grid, tile, lists):
    """Query x key token mask: query token in tile i sees key tokens whose tile
    is in lists[i]; tile membership from coordinates, not from the plan."""
    rows, P = expected_rows(segs, grid, tile)
    B = tile[0] * tile[1] * tile[2]
    tile_of = rows // B
    n_t = int(tile_of.max()) + 1 if tile_of.size else 0
    allowed_tiles = np.zeros((n_t, n_t), dtype=bool)
    for i in range(n_t):
        allowed_tiles[i, lists[i]] = True
    return allowed_tiles[tile_of[:, None], tile_of[None, :]]


def test_ref_keep_counts_follow_the_page_rule(orc):
    pl = orc.plan((512, 512, 512, 128), (24, 48, 84), (4, 4, 4))
    assert pl.P == 26
    assert orc.ref_keep_counts(pl, 0.9, None, 0.75, None) == (3, 378)    # round(2.6) = 3
    assert orc.ref_keep_counts(pl, 0.0, None, 0.0, None) == (26, 1512)   # 0 % = full
    assert orc.ref_keep_counts(pl, None, 5, None, 24) == (5, 24)         # integer form
    with pytest.raises(orc.OracleError):
        orc.ref_keep_counts(pl, None, 27, 0.5, None)


def test_all_scores_chain_and_bound(orc):
    rng = np.random.default_rng(11)
    n_t, D = 23, 64
    qm = rng.standard_normal((n_t, D)).astype(np.float32)
    km = rng.standard_normal((n_t, D)).astype(np.float32)
    got = orc.all_scores(qm, km)
    exact = qm.astype(np.float64) @ km.astype(np.float64).T
    bound = 1.01 * D * U32 * (np.abs(qm).astype(np.float64) @ np.abs(km).astype(np.float64).T)
    assert np.all(np.abs(got - exact) <= bound)
    # integer-valued means: every partial sum is exact
    qi = rng.integers(-8, 8, (n_t, D)).astype(np.float32)
    ki = rng.integers(-8, 8, (n_t, D)).astype(np.float32)
    assert np.array_equal(orc.all_scores(qi, ki), (qi.astype(np.int64) @ ki.astype(np.int64).T))
    # the video block agrees with the video-only scorer (same chain, same order)
    P = 5
    assert np.array_equal(got[P:, P:], orc.video_scores(qm, km, P, n_t - P))
    sub = orc.all_scores(qm, km, rows=[3, 17])
    assert np.array_equal(sub, got[[3, 17]])


@pytest.mark.parametrize("P,n_v,k_ref,k_gen", [(2, 4, 1, 2), (26, 300, 3, 75), (5, 40, 5, 0),
                                               (5, 40, 0, 40), (1, 1, 1, 1)])
def test_topk_ref_is_two_brute_force_selections(orc, P, n_v, k_ref, k_gen):
    rng = np.random.default_rng(P * 1000 + n_v)
    s = rng.standard_normal((30, P + n_v)).astype(np.float32)
    s[::4] = np.round(s[::4] * 2) / 2        # planted ties
    got = orc.topk_ref(s, P, k_ref, k_gen)
    want = np.concatenate([brute_topk(s[:, :P], k_ref, 0), brute_topk(s[:, P:], k_gen, P)], axis=1)
    assert np.array_equal(got, want)
    assert got.shape == (30, k_ref + k_gen)
    assert np.all(np.diff(got, axis=1) > 0)  # ascending global ids overall


@pytest.mark.parametrize("segs,grid,tile,k_ref,k_gen", [
    ((20, 40), (4, 8, 8), (4, 4, 4), 1, 2),    # Tiny geometry
    ((5, 70), (5, 6, 9), (4, 4, 4), 1, 3),     # partial tiles everywhere
    ((9, 9, 9), (3, 4, 4), (1, 4, 4), 0, 2),   # no reference keys at all
    ((9,), (3, 4, 4), (1, 4, 4), 1, 0),        # no video keys at all
])
def test_fine_lists_match_masked_sdpa(orc, segs, grid, tile, k_ref, k_gen):
    pl = orc.plan(segs, grid, tile)
    H, D = 2, 32
    Q, K, V = (rand_bf16((pl.S, H, D), s) for s in (17, 18, 19))
    scale = D ** -0.5
    rng = np.random.default_rng(5)
    for h in range(H):
        lists = np.stack([np.concatenate([np.sort(rng.choice(pl.P, size=k_ref, replace=False)),
                                          np.sort(rng.choice(pl.n_v, size=k_gen, replace=False)) + pl.P])
                          for _ in range(pl.n_t)]).astype(np.int32)
        got = orc.fine_tokens_lists(Q, K, V, h, pl, lists, scale, np.arange(pl.S))
        mask = list_mask(segs, grid, tile, lists)
        ref = sdpa64(*(orc.bf16_value(X)[:, h, :] for X in (Q, K, V)), mask=mask, scale=scale)
        assert np.allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_ref_zero_sparsity_is_dense(orc):
    """0 % reference and 0 % generated sparsity: every query sees every key."""
    segs, grid, tile = (30, 17), (4, 8, 8), (4, 4, 4)
    pl = orc.plan(segs, grid, tile)
    H, D = 1, 64
    Q, K, V = (rand_bf16((pl.S, H, D), s) for s in (4, 5, 6))
    k_ref, k_gen = orc.ref_keep_counts(pl, 0.0, None, 0.0, None)
    hr = orc.head_ref(Q, K, V, 0, pl, k_ref, k_gen, D ** -0.5)
    assert np.array_equal(hr.keep, np.tile(np.arange(pl.n_t, dtype=np.int32), (pl.n_t, 1)))
    got = orc.fine_tokens_lists(Q, K, V, 0, pl, hr.keep, D ** -0.5, np.arange(pl.S))
    ref = sdpa64(*(orc.bf16_value(X)[:, 0, :] for X in (Q, K, V)))
    assert np.allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_ref_all_prefix_kept_matches_sink_mode_for_video_queries(orc):
    """k_ref = P turns the prefix back into sinks for video queries: their fine
    output equals the default path's with the same video keep-sets."""
    segs, grid, tile = (20, 40), (4, 8, 8), (4, 4, 4)
    pl = orc.plan(segs, grid, tile)
    H, D = 2, 64
    Q, K, V = (rand_bf16((pl.S, H, D), s) for s in (21, 22, 23))
    k_gen = 2
    for h in range(H):
        hr = orc.head_ref(Q, K, V, h, pl, pl.P, k_gen, D ** -0.5)
        sink = orc.head(Q, K, V, h, pl, k_gen, D ** -0.5)
        assert np.array_equal(hr.keep[pl.P:, pl.P:], sink.keep)
        vid = np.nonzero(pl.untile // pl.B >= pl.P)[0]
        a = orc.fine_tokens_lists(Q, K, V, h, pl, hr.keep, D ** -0.5, vid)
        b = orc.fine_tokens(Q, K, V, h, pl, sink.keep, k_gen, D ** -0.5, vid)
        assert np.allclose(a, b, rtol=1e-13, atol=1e-14)


def test_ref_empty_key_list_is_an_error(orc):
    pl = orc.plan((9,), (4, 4, 4), (4, 4, 4))
    Q = rand_bf16((pl.S, 1, 8), 1)
    with pytest.raises(orc.OracleError):
        orc.fine_tokens_lists(Q, Q, Q, 0, pl, np.zeros((pl.n_t, 0), np.int32), 1.0, [3])


def test_ref_pair_fraction(orc):
    assert orc.tile_pair_fraction_ref(686, 3, 165) == pytest.approx(168 / 686)
    assert orc.tile_pair_fraction_ref(10, 4, 6) == 1.0
