"""Pins for the oracle's arithmetic (CPU only).

Each oracle step is checked against something other than itself: exact
results on exactly representable inputs, rounding-error bounds against fp64,
a library routine (torch's scaled_dot_product_attention, numpy sorts and
matmuls) on cases where the step reduces to it, or brute force.
"""
import math

import numpy as np
import pytest
import torch

import workloads

U32 = 2.0 ** -24  # unit roundoff of fp32


def bits_of(a_f32: np.ndarray) -> np.ndarray:
    """fp32 values that are exact bf16 -> their bf16 bit patterns."""
    a = np.ascontiguousarray(a_f32, dtype=np.float32)
    assert ((a.view(np.uint32) & 0xFFFF) == 0).all()
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def rand_bf16(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    t = (torch.randn(*shape, generator=g) * scale).to(torch.bfloat16)
    return workloads.bf16_bits(t)


def bf16_neighbours(bits):
    b = np.asarray(bits, dtype=np.int64)
    return b - 1, b + 1


# ------------------------------------------------------------- bf16 rounding --

def test_bf16_round_ties_and_specials(orc):
    one = 1.0
    cases = [
        (one, 0x3F80),
        (one + 2 ** -8, 0x3F80),                 # tie -> even (down)
        (one + 2 ** -7 + 2 ** -8, 0x3F82),       # tie -> even (up)
        (one + 2 ** -8 + 2 ** -30, 0x3F81),      # just above the tie
        (-(one + 2 ** -8 + 2 ** -30), 0xBF81),
        (2.0 ** -130, 0x0008),                   # bf16 subnormal, exact
        (2.0 ** -134, 0x0000),                   # half the smallest subnormal: tie -> 0
        (3 * 2.0 ** -134, 0x0002),               # 1.5 * 2^-133 -> tie -> even (2 * 2^-133)
        (3.0e38 * 2, 0x7F80),                    # overflow
        (0.0, 0x0000),
        (-0.0, 0x8000),
    ]
    for x, want in cases:
        assert int(orc.bf16_round(x)) == want, (x, hex(int(orc.bf16_round(x))), hex(want))


def test_bf16_round_matches_torch_on_fp32_values(orc):
    """For fp32-representable inputs one rounding fp64->bf16 equals torch's fp32->bf16 RNE."""
    g = torch.Generator().manual_seed(3)
    x = torch.randn(4000, generator=g) * torch.exp(torch.randn(4000, generator=g) * 8)
    ours = orc.bf16_round(x.double().numpy())
    ref = workloads.bf16_bits(x.to(torch.bfloat16))
    assert np.array_equal(ours, ref)


# ------------------------------------------------------------------ pooling --

def _tiny_plan(orc, segs=(20, 40), grid=(4, 8, 8), tile=(4, 4, 4)):
    return orc.plan(segs, grid, tile)


def test_tile_means_error_bound(orc):
    pl = _tiny_plan(orc, segs=(37, 5), grid=(5, 6, 7))
    H, D = 3, 16
    X = rand_bf16((pl.S, H, D), 11)
    Xv = orc.bf16_value(X)
    for h in range(H):
        m = orc.tile_means(X, h, pl)
        for t in range(pl.n_t):
            toks = pl.row_src[t * pl.B: t * pl.B + pl.block_len[t]]
            vals = Xv[toks, h, :]
            exact = vals.sum(0) / len(toks)
            n = len(toks)
            bound = (n * U32 / (1 - n * U32)) * np.abs(vals).sum(0) / n + U32 * np.abs(exact) + 1e-45
            assert (np.abs(m[t].astype(np.float64) - exact) <= bound).all()


def test_tile_means_exact_cases(orc):
    pl = _tiny_plan(orc, segs=(1, 64, 3), grid=(4, 4, 4))
    H, D = 1, 8
    rng = np.random.default_rng(5)
    # small integers: every partial sum is exact, so the mean is the correctly
    # rounded quotient of two integers
    vals = rng.integers(-8, 9, size=(pl.S, H, D)).astype(np.float32)
    m = orc.tile_means(bits_of(vals), 0, pl)
    for t in range(pl.n_t):
        toks = pl.row_src[t * pl.B: t * pl.B + pl.block_len[t]]
        s = vals[toks, 0, :].astype(np.float64).sum(0)
        assert np.array_equal(m[t], (s / len(toks)).astype(np.float32))
    # a constant tile averages to the constant; a one-row tile to its row
    const = np.full((pl.S, H, D), 0.3125, dtype=np.float32)
    assert (orc.tile_means(bits_of(const), 0, pl) == np.float32(0.3125)).all()
    assert pl.block_len[0] == 1
    assert np.array_equal(m[0], vals[pl.row_src[0], 0, :])


def test_tile_means_sequential_order(orc):
    """Ascending-row fp32 summation, not pairwise or reversed: 2^24 + 1 + 1 ... cases."""
    pl = orc.plan([3], (1, 1, 1), (1, 1, 4))  # one prefix tile of 3 rows (B = 4), one video token
    assert pl.S == 4
    # rows: 2^24, 1, 1 -> ((2^24 + 1) + 1) = 2^24 in ascending fp32 order
    # (reversed order would give 2^24 + 2); the video token is its own tile
    vals = np.array([2.0 ** 24, 1.0, 1.0, 5.0], dtype=np.float32).reshape(4, 1, 1)
    m = orc.tile_means(bits_of(vals), 0, pl)
    assert m[0, 0] == np.float32(2.0 ** 24 / 3)
    assert m[1, 0] == np.float32(5.0)


# ------------------------------------------------------------------- scores --

def test_scores_fma_chain_ascending(orc):
    """acc = fma(q_d, k_d, acc) over ascending d from +0.

    With a = 1 + 2^-12: q = [1, a], k = [-(1 + 2^-11), a]. Ascending fused:
    -(1+2^-11) then a*a - (1+2^-11) = 2^-24 exactly. Unfused or descending
    evaluation gives 0."""
    a = np.float32(1 + 2 ** -12)
    qm = np.array([[1.0, a]], dtype=np.float32)
    km = np.array([[-(1 + 2 ** -11), a]], dtype=np.float32)
    s = orc.video_scores(qm, km, P=0, n_v=1)
    assert s[0, 0] == np.float32(2.0 ** -24)


def test_scores_error_bound_and_exact(orc):
    rng = np.random.default_rng(9)
    n_t, P, D = 40, 5, 64
    qm = rng.standard_normal((n_t, D)).astype(np.float32)
    km = rng.standard_normal((n_t, D)).astype(np.float32)
    s = orc.video_scores(qm, km, P, n_t - P)
    q64, k64 = qm[P:].astype(np.float64), km[P:].astype(np.float64)
    exact = q64 @ k64.T
    bound = (D * U32 / (1 - D * U32)) * (np.abs(q64) @ np.abs(k64).T)
    assert (np.abs(s - exact) <= bound).all()
    # integer inputs: exact
    qi = rng.integers(-5, 6, size=(n_t, D)).astype(np.float32)
    ki = rng.integers(-5, 6, size=(n_t, D)).astype(np.float32)
    si = orc.video_scores(qi, ki, P, n_t - P, rows=[0, 3, 7])
    ex = qi[P:][[0, 3, 7]].astype(np.int64) @ ki[P:].astype(np.int64).T
    assert np.array_equal(si, ex.astype(np.float32))


# -------------------------------------------------------------------- top-k --

def brute_topk(scores, k, P):
    out = []
    for row in scores:
        j = np.arange(row.size)
        order = np.lexsort((j, -row.astype(np.float64)))  # score desc, index asc
        out.append(np.sort(order[:k]) + P)
    return np.array(out, dtype=np.int32).reshape(len(scores), k)


@pytest.mark.parametrize("n_v,k", [(1, 1), (7, 3), (64, 16), (300, 75), (300, 300), (50, 0)])
def test_topk_matches_full_sort(orc, n_v, k):
    rng = np.random.default_rng(n_v * 31 + k)
    s = rng.standard_normal((20, n_v)).astype(np.float32)
    # plant ties: quantise some rows heavily so many scores are equal
    s[::3] = np.round(s[::3] * 2) / 2
    got = orc.topk_rows(s, k, P=11)
    assert np.array_equal(got, brute_topk(s, k, 11))


def test_topk_tie_lowest_index_and_signed_zero(orc):
    s = np.array([[0.0, 1.0, -0.0, 1.0, 0.0, -1.0]], dtype=np.float32)
    assert orc.topk_rows(s, 2, 0).tolist() == [[1, 3]]
    # three-way tie among +0, -0, +0 for one slot: the lowest index wins
    assert orc.topk_rows(s, 3, 0).tolist() == [[0, 1, 3]]
    s2 = np.array([[-0.0, 0.0, -1.0]], dtype=np.float32)
    assert orc.topk_rows(s2, 1, 0).tolist() == [[0]]


def test_topk_invariants_and_errors(orc):
    rng = np.random.default_rng(2)
    s = rng.standard_normal((50, 128)).astype(np.float32)
    k = 32
    keep = orc.topk_rows(s, k, P=3)
    for r in range(50):
        kept = keep[r] - 3
        assert np.all(np.diff(kept) > 0)
        dropped = np.setdiff1d(np.arange(128), kept)
        assert s[r, kept].min() >= s[r, dropped].max()
    assert np.array_equal(orc.topk_rows(s, 128, P=0), np.tile(np.arange(128), (50, 1)))
    bad = s.copy()
    bad[4, 9] = np.nan
    with pytest.raises(orc.OracleError):
        orc.topk_rows(bad, k, 0)


# --------------------------------------------------------- coarse attention --

def sdpa64(q, k, v, mask=None, scale=None):
    """torch's scaled_dot_product_attention in fp64 on [n, D] inputs."""
    q, k, v = (torch.from_numpy(np.asarray(a, dtype=np.float64))[None, None] for a in (q, k, v))
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m,
                                                            scale=scale)[0, 0].numpy()


def test_coarse_is_dense_token_attention_for_unit_tiles(orc):
    """1x1x1 tiles: each tile is one token, so the tile-level attention is dense
    token attention (with the prefix as ordinary tokens)."""
    pl = orc.plan([3, 2], (2, 3, 4), (1, 1, 1))
    H, D = 2, 16
    Q, K, V = (rand_bf16((pl.S, H, D), s) for s in (1, 2, 3))
    scale = D ** -0.5
    for h in range(H):
        qm, km, vm = (orc.tile_means(X, h, pl) for X in (Q, K, V))
        got = orc.coarse_attn(qm, km, vm, scale)
        tok = pl.row_src  # B = 1: tile i holds token row_src[i]
        ref = sdpa64(*(orc.bf16_value(X)[tok, h, :] for X in (Q, K, V)), scale=scale)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_coarse_uniform_and_dominant(orc):
    rng = np.random.default_rng(4)
    n_t, D = 12, 8
    qm = rng.standard_normal((n_t, D)).astype(np.float32)
    vm = rng.standard_normal((n_t, D)).astype(np.float32)
    km_equal = np.tile(rng.standard_normal((1, D)).astype(np.float32), (n_t, 1))
    got = orc.coarse_attn(qm, km_equal, vm, 0.3)
    assert np.allclose(got, vm.astype(np.float64).mean(0)[None, :], rtol=1e-13, atol=1e-15)
    km = np.zeros((n_t, D), dtype=np.float32)
    km[5] = qm[2] * 1000          # tile 5 dominates the softmax of query tile 2
    got = orc.coarse_attn(qm, km, vm, 1.0, rows=[2])
    assert np.allclose(got[0], vm[5], rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------- fine attention --

def token_tile_mask(pl, P_segs, grid, tile, keep_h):
    """Query x key token mask from the tile rules, with tile membership taken
    from coordinates (not from the plan arrays)."""
    from tests.test_oracle_plan import expected_rows
    rows, P = expected_rows(P_segs, grid, tile)
    B = tile[0] * tile[1] * tile[2]
    tile_of = rows // B
    qt, kt = tile_of[:, None], tile_of[None, :]
    allowed = (qt < P) | (kt < P)
    if keep_h.size:
        kept = np.zeros((pl.n_t, pl.n_t), dtype=bool)
        for i in range(pl.n_v):
            kept[P + i, keep_h[i]] = True
        allowed |= kept[qt, kt]
    return allowed


@pytest.mark.parametrize("segs,grid,tile,k", [
    ((20, 40), (4, 8, 8), (4, 4, 4), 2),      # Tiny geometry
    ((5, 70), (5, 6, 9), (4, 4, 4), 3),       # partial tiles everywhere
    ((), (4, 4, 8), (2, 2, 2), 4),            # no prefix
    ((9,), (3, 4, 4), (1, 4, 4), 0),          # k = 0: video queries see only the prefix
])
def test_fine_matches_masked_sdpa(orc, segs, grid, tile, k):
    pl = orc.plan(segs, grid, tile)
    H, D = 2, 32
    Q, K, V = (rand_bf16((pl.S, H, D), s) for s in (7, 8, 9))
    scale = D ** -0.5
    rng = np.random.default_rng(1)
    for h in range(H):
        keep = np.sort(np.stack([rng.choice(pl.n_v, size=k, replace=False)
                                 for _ in range(pl.n_v)]), axis=1).astype(np.int32) + pl.P
        toks = np.arange(pl.S)
        got = orc.fine_tokens(Q, K, V, h, pl, keep, k, scale, toks)
        mask = token_tile_mask(pl, segs, grid, tile, keep)
        ref = sdpa64(*(orc.bf16_value(X)[:, h, :] for X in (Q, K, V)), mask=mask, scale=scale)
        assert np.allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_fine_sparsity_zero_is_dense(orc):
    """Keeping every video tile (k = n_v) gives dense softmax attention."""
    pl = orc.plan((30, 17), (4, 8, 8), (4, 4, 4))
    H, D = 1, 64
    Q, K, V = (rand_bf16((pl.S, H, D), s) for s in (4, 5, 6))
    k = orc.keep_count(pl.n_v, sparsity=0.0)
    keep = np.tile(np.arange(pl.P, pl.n_t, dtype=np.int32), (pl.n_v, 1))
    got = orc.fine_tokens(Q, K, V, 0, pl, keep, k, D ** -0.5, np.arange(pl.S))
    ref = sdpa64(*(orc.bf16_value(X)[:, 0, :] for X in (Q, K, V)))
    assert np.allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_fine_empty_key_set_is_an_error(orc):
    pl = orc.plan((), (4, 4, 4), (4, 4, 4))
    Q = rand_bf16((pl.S, 1, 8), 1)
    with pytest.raises(orc.OracleError):
        orc.fine_tokens(Q, Q, Q, 0, pl, np.zeros((1, 0), np.int32), 0, 1.0, [3])


# ------------------------------------------------------- combine and gate --

def test_combine_gate_zero_and_one(orc):
    rng = np.random.default_rng(8)
    of = rng.standard_normal((10, 16)) * 0.01
    oc = rng.standard_normal((10, 16)) * 0.003
    zero = np.zeros((10, 16), dtype=np.uint16)
    one = np.full((10, 16), 0x3F80, dtype=np.uint16)
    assert np.array_equal(orc.combine(of, zero, oc), orc.bf16_round(of))
    assert np.array_equal(orc.combine(of, one, oc), orc.bf16_round(of + oc))
    g = rand_bf16((10, 16), 3)
    ref = orc.bf16_round(of + orc.bf16_value(g) * oc)
    assert np.array_equal(orc.combine(of, g, oc), ref)


def test_gate_proj_is_correctly_rounded_matmul(orc):
    x = rand_bf16((37, 96), 21)
    W = rand_bf16((48, 96), 22, scale=0.02)
    g = orc.gate_proj(x, W)
    exact = orc.bf16_value(x) @ orc.bf16_value(W).T          # numpy fp64 matmul
    got = orc.bf16_value(g)
    lo, hi = bf16_neighbours(g)
    # got is a nearest bf16 of the exact product: no neighbour is strictly closer
    err = np.abs(got - exact)
    assert (err <= np.abs(orc.bf16_value(lo.astype(np.uint16)) - exact) * (1 + 1e-12)).all()
    assert (err <= np.abs(orc.bf16_value(hi.astype(np.uint16)) - exact) * (1 + 1e-12)).all()
    sub = orc.gate_proj(x, W, tokens=[5, 0, 36])
    assert np.array_equal(sub, g[[5, 0, 36]])


def test_bf16_step_of_the_output_bar():
    """The output bar's bf16 step: 2^(e-7) on [2^e, 2^(e+1)); the bar is 2e-2 up to
    |value| < 4 and one step (2^-5, 2^-4, ...) from 4 on."""
    from tests import parity
    vals = np.array([1.0, 1.99, 2.0, 3.999, 4.0, -5.0, 8.0, 0.0, 1e-40])
    want = np.array([2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0 ** -6, 2.0 ** -5, 2.0 ** -5, 2.0 ** -4,
                     2.0 ** -133, 2.0 ** -133])
    assert np.array_equal(parity.bf16_ulp(vals), want)
    bar = parity.output_bar(vals, vals)
    assert np.array_equal(bar, np.maximum(2e-2, want))
    # consecutive bf16 numbers differ by exactly the step
    for v in (1.0, 3.0, 4.0, 6.5, 100.0):
        b = int(np.float32(v).view(np.uint32) >> 16)
        nxt = np.uint32((b + 1) << 16).view(np.float32)
        assert float(nxt) - v == parity.bf16_ulp(v)
