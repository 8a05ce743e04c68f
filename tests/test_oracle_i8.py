"""Pins for the oracle's INT8 fine pass (CPU only).

[Veda] "How Veda works" and its performance table: the tile-skip kernel does
its attention arithmetic in INT8; the pages give no scheme. Reading: symmetric
INT8 codes for Q and K, one fp32 scale per 64-row block of the tiled layout,
round half to even, only the score product uses the codes. Checked against:
integer-valued blocks (the codes are the values), round-half-even ties, the
round-to-nearest error bound, power-of-two scaling invariance, and torch's
fp64 attention on inputs whose quantisation is exact (block scales that are
distinct powers of two, so a scale taken from the wrong block shows), plus the
worst-case bound on the output change that the quantisation error allows.
"""
import numpy as np
import pytest
import torch

import workloads
from tests.test_oracle_numerics import rand_bf16, sdpa64, token_tile_mask


def f32_to_bf16_bits(a):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return workloads.bf16_bits(t)


def block_rows(pl, b):
    """Tokens of the real rows of 64-row block b of the tiled layout."""
    r = pl.row_src[64 * b: 64 * b + 64]
    return r[r >= 0]


def exact_blocks(pl, H, D, seed, exps):
    """Integer values times 2^e_b per 64-row block b, each block holding +-127 * 2^e_b:
    the INT8 codes are the integers and the scales are exactly 2^e_b."""
    rng = np.random.default_rng(seed)
    X = np.zeros((pl.S, H, D), dtype=np.float32)
    n_blocks = pl.S_pad // 64
    for b in range(n_blocks):
        toks = block_rows(pl, b)
        if toks.size == 0:
            continue
        e = exps[b % len(exps)]
        vals = rng.integers(-127, 128, (toks.size, H, D)).astype(np.float32)
        vals[0, :, 0] = 127.0 * (1 if b % 2 else -1)
        vals = np.clip(vals, -127, 127)
        X[toks] = vals * np.float32(2.0 ** e)
    return f32_to_bf16_bits(X), X


def test_quant_integer_blocks_are_exact(orc):
    pl = orc.plan((30,), (4, 8, 8), (4, 8, 4))   # B = 128: two blocks per tile
    H, D = 2, 32
    exps = [0, -3, 2, -1, 1]
    bits, X = exact_blocks(pl, H, D, 3, exps)
    for h in range(H):
        codes, scales = orc.quant_blocks_i8(bits, h, pl)
        for b in range(pl.S_pad // 64):
            toks = block_rows(pl, b)
            rows = 64 * b + np.nonzero(pl.row_src[64 * b: 64 * b + 64] >= 0)[0]
            if toks.size == 0:
                assert scales[b] == 0.0 and not codes[64 * b: 64 * b + 64].any()
                continue
            e = exps[b % len(exps)]
            assert scales[b] == np.float32(2.0 ** e)
            assert np.array_equal(codes[rows].astype(np.float32) * np.float32(2.0 ** e), X[toks, h])
            pad = 64 * b + np.nonzero(pl.row_src[64 * b: 64 * b + 64] < 0)[0]
            assert not codes[pad].any()


def test_quant_ties_round_half_to_even(orc):
    pl = orc.plan((), (1, 8, 8), (1, 8, 8))      # one tile of 64 rows
    D = 8
    X = np.zeros((pl.S, 1, D), dtype=np.float32)
    X[0, 0, :] = [127.0, 2.5, 3.5, -2.5, -0.5, 126.5, 0.5, -1.5]
    codes, scales = orc.quant_blocks_i8(f32_to_bf16_bits(X), 0, pl)
    assert scales[0] == np.float32(1.0)
    r0 = int(pl.untile[0])
    assert codes[r0].tolist() == [127, 2, 4, -2, 0, 126, 0, -2]


def test_quant_bound_extremes_and_zero_block(orc):
    pl = orc.plan((40,), (4, 8, 8), (4, 4, 4))
    H, D = 1, 64
    rng = np.random.default_rng(5)
    X = rng.standard_normal((pl.S, H, D)).astype(np.float32)
    # blocks of very different magnitude, and one all-zero block
    for b in range(pl.S_pad // 64):
        X[block_rows(pl, b)] *= np.float32(10.0 ** (b % 5 - 2))
    X[block_rows(pl, 1)] = 0.0
    bits = f32_to_bf16_bits(X)
    xv = orc.bf16_value(bits)[:, 0, :]
    codes, scales = orc.quant_blocks_i8(bits, 0, pl)
    assert np.abs(codes.astype(np.int32)).max() <= 127
    for b in range(pl.S_pad // 64):
        toks = block_rows(pl, b)
        rows = 64 * b + np.nonzero(pl.row_src[64 * b: 64 * b + 64] >= 0)[0]
        a = np.abs(xv[toks]).max() if toks.size else 0.0
        if a == 0.0:
            assert scales[b] == 0.0 and not codes[64 * b: 64 * b + 64].any()
            continue
        assert scales[b] == np.float32(np.float32(a) / np.float32(127.0))
        assert np.abs(codes[rows]).max() == 127          # the largest element maps to +-127
        # Round to nearest gives half a step; x * (127/a), 127/a and a/127 are each
        # rounded to fp32 once, which adds at most 3 units of roundoff of |x|.
        err = np.abs(xv[toks] - codes[rows].astype(np.float64) * np.float64(scales[b]))
        assert np.all(err <= 0.5 * np.float64(scales[b]) + 3.01 * 2.0 ** -24 * np.abs(xv[toks]))
        assert err.max() > 0.4 * scales[b]               # and the half step is reached


def test_quant_power_of_two_invariance(orc):
    pl = orc.plan((12,), (4, 4, 8), (4, 4, 4))
    X = rand_bf16((pl.S, 1, 32), 9)
    c1, s1 = orc.quant_blocks_i8(X, 0, pl)
    X8 = f32_to_bf16_bits(orc.bf16_value(X).astype(np.float32) * np.float32(8.0))
    c2, s2 = orc.quant_blocks_i8(X8, 0, pl)
    assert np.array_equal(c1, c2)
    assert np.array_equal(s2, s1 * np.float32(8.0))


@pytest.mark.parametrize("segs,grid,tile,k", [
    ((20, 40), (4, 8, 8), (4, 4, 4), 2),
    ((5, 70), (5, 6, 9), (4, 4, 4), 3),       # partial tiles everywhere
    ((30,), (4, 8, 8), (4, 8, 4), 2),         # B = 128: two blocks per tile
])
def test_fine_i8_is_exact_attention_when_quantisation_is(orc, segs, grid, tile, k):
    pl = orc.plan(segs, grid, tile)
    H, D = 2, 32
    Qb, _ = exact_blocks(pl, H, D, 11, [0, -2, 1, -1])
    Kb, _ = exact_blocks(pl, H, D, 12, [-1, 2, 0, -3, 1])
    Vb = rand_bf16((pl.S, H, D), 13)
    scale = D ** -0.5 / 256.0   # keeps the integer-valued scores in a sane range
    rng = np.random.default_rng(2)
    for h in range(H):
        keep = np.sort(np.stack([rng.choice(pl.n_v, size=k, replace=False)
                                 for _ in range(pl.n_v)]), axis=1).astype(np.int32) + pl.P
        toks = np.arange(pl.S)
        got = orc.fine_tokens_i8(Qb, Kb, Vb, h, pl, orc.key_lists_default(pl, keep), scale, toks)
        mask = token_tile_mask(pl, segs, grid, tile, keep)
        ref = sdpa64(*(orc.bf16_value(X)[:, h, :] for X in (Qb, Kb, Vb)), mask=mask, scale=scale)
        assert np.allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_fine_i8_within_the_quantisation_bound(orc):
    """|dz| <= scale * sum_d(|q_d| dk + dq |k_d| + dq dk) with dq = sq/2, dk = sk/2 per
    element; then every softmax weight moves by a factor within e^(+-2 eps) and the
    output by at most (e^(2 eps) - 1) max|v|."""
    segs, grid, tile = (20, 40), (4, 8, 8), (4, 4, 4)
    pl = orc.plan(segs, grid, tile)
    H, D = 1, 64
    rng = np.random.default_rng(4)
    Qf = rng.standard_normal((pl.S, H, D)).astype(np.float32)
    for b in range(pl.S_pad // 64):
        Qf[block_rows(pl, b)] *= np.float32(2.0 ** (b % 3 - 1))
    Q, K, V = f32_to_bf16_bits(Qf), rand_bf16((pl.S, H, D), 21), rand_bf16((pl.S, H, D), 22)
    scale = D ** -0.5
    keep = np.sort(np.stack([rng.choice(pl.n_v, size=3, replace=False)
                             for _ in range(pl.n_v)]), axis=1).astype(np.int32) + pl.P
    toks = np.arange(pl.S)
    got = orc.fine_tokens_i8(Q, K, V, 0, pl, orc.key_lists_default(pl, keep), scale, toks)
    exact = orc.fine_tokens(Q, K, V, 0, pl, keep, 3, scale, toks)
    _, sq = orc.quant_blocks_i8(Q, 0, pl)
    _, sk = orc.quant_blocks_i8(K, 0, pl)
    qv, kv, vv = (orc.bf16_value(X)[:, 0, :] for X in (Q, K, V))
    mask = token_tile_mask(pl, segs, grid, tile, keep)
    tq = pl.untile // 64                                # block of each token
    dq = 0.5 * sq[tq].astype(np.float64)[:, None]
    dk = 0.5 * sk[tq].astype(np.float64)[None, :]
    aq = np.abs(qv).sum(1)[:, None]
    ak = np.abs(kv).sum(1)[None, :]
    dz = scale * (aq * dk + dq * ak + D * dq * dk)
    eps = np.where(mask, dz, 0.0).max(1)
    bound = np.expm1(2 * eps)[:, None] * np.abs(vv).max()
    diff = np.abs(got - exact)
    assert np.all(diff <= bound + 1e-12)
    assert diff.max() > 0   # the quantisation does change the result


def test_fine_i8_bad_lists(orc):
    pl = orc.plan((), (4, 4, 4), (4, 4, 4))
    Q = rand_bf16((pl.S, 1, 8), 1)
    with pytest.raises(orc.OracleError):
        orc.fine_tokens_i8(Q, Q, Q, 0, pl, (np.zeros(2, np.int32), np.zeros(1, np.int32)), 1.0, [3])
    with pytest.raises(orc.OracleError):
        orc.fine_tokens_i8(Q, Q, Q, 0, pl, (np.array([0, 1], np.int32), np.array([5], np.int32)), 1.0, [3])
