"""Pins for the oracle's layer backward (CPU only).

The layer's gradient, with the keep sets held fixed, against: torch autograd
(fp64) through an independent dense formulation of the same forward (a token
mask from tile coordinates, tile means with torch, the gated combine), and
exact identities that hold at any size (softmax rows sum to one, so the value
gradients add up to the output gradients and the key gradients to zero).
"""
import numpy as np
import pytest
import torch

import workloads
from tests.test_oracle_numerics import rand_bf16
from tests.test_oracle_plan import expected_rows


def torch_layer_grads(orc, pl, segs, grid, tile, Q, K, V, G, dO, h, lists, scale):
    """Autograd of sum(out * dO) for head h; lists[i] = key tiles of query tile i."""
    rows, P = expected_rows(segs, grid, tile)          # token -> padded row, from coordinates
    B = tile[0] * tile[1] * tile[2]
    tile_of = torch.from_numpy(rows // B)
    n_t = pl.n_t
    H, D = Q.shape[1], Q.shape[2]
    f = lambda X: torch.from_numpy(orc.bf16_value(X)[:, h, :]).requires_grad_(True)  # noqa: E731
    q, k, v = f(Q), f(K), f(V)
    g = torch.from_numpy(orc.bf16_value(G).reshape(-1, H, D)[:, h, :]).requires_grad_(True)
    allowed = torch.zeros((n_t, n_t), dtype=torch.bool)
    for i in range(n_t):
        allowed[i, torch.as_tensor(np.asarray(lists[i], dtype=np.int64))] = True
    mask = allowed[tile_of[:, None], tile_of[None, :]]
    z = (q @ k.T) * scale
    z = z.masked_fill(~mask, float("-inf"))
    o_fine = torch.softmax(z, dim=1) @ v
    onehot = torch.nn.functional.one_hot(tile_of, n_t).double()       # [S][n_t]
    cnt = onehot.sum(0)
    qm, km, vm = ((onehot.T @ x) / cnt[:, None] for x in (q, k, v))
    o_c = torch.softmax((qm @ km.T) * scale, dim=1) @ vm
    out = o_fine + g * o_c[tile_of]
    loss = (out * torch.from_numpy(orc.bf16_value(dO)[:, h, :])).sum()
    loss.backward()
    return {"dq": q.grad.numpy(), "dk": k.grad.numpy(), "dv": v.grad.numpy(), "dg": g.grad.numpy()}


CASES = [
    ((20, 40), (4, 8, 8), (4, 4, 4), "default", 2),   # Tiny geometry
    ((5, 70), (5, 6, 9), (4, 4, 4), "default", 3),    # partial tiles everywhere
    ((9, 9, 9), (3, 4, 4), (1, 4, 4), "ref", (1, 2)),  # reference sparsity, 16-row tiles
    ((), (4, 4, 8), (2, 2, 2), "default", 4),         # no prefix
]


@pytest.mark.parametrize("segs,grid,tile,mode,kk", CASES)
def test_backward_matches_torch_autograd(orc, segs, grid, tile, mode, kk):
    pl = orc.plan(segs, grid, tile)
    H, D = 2, 32
    Q, K, V = (rand_bf16((pl.S, H, D), s) for s in (31, 32, 33))
    G = rand_bf16((pl.S, H * D), 34, scale=0.5)
    dO = rand_bf16((pl.S, H, D), 35)
    scale = D ** -0.5
    rng = np.random.default_rng(7)
    for h in range(H):
        if mode == "default":
            keep = np.sort(np.stack([rng.choice(pl.n_v, size=kk, replace=False)
                                     for _ in range(pl.n_v)]), axis=1).astype(np.int32) + pl.P
            csr = orc.key_lists_default(pl, keep)
        else:
            k_ref, k_gen = kk
            lists = np.stack([np.concatenate([np.sort(rng.choice(pl.P, k_ref, replace=False)),
                                              np.sort(rng.choice(pl.n_v, k_gen, replace=False)) + pl.P])
                              for _ in range(pl.n_t)]).astype(np.int32)
            csr = orc.key_lists_explicit(lists)
        off, ids = csr
        lists_py = [ids[off[i]:off[i + 1]] for i in range(pl.n_t)]
        got = orc.layer_bwd(Q, K, V, G, dO, h, pl, csr, scale)
        want = torch_layer_grads(orc, pl, segs, grid, tile, Q, K, V, G, dO, h, lists_py, scale)
        for name in ("dq", "dk", "dv", "dg"):
            # the oracle's tile means are the fp32 canonical ones, torch's are fp64
            assert np.allclose(got[name], want[name], rtol=1e-5, atol=1e-6), name


def test_backward_sum_identities(orc):
    """sum_u dv_u = sum_t dout_t * (1 + g_t) and sum_u dk_u = 0 (rows of both
    softmaxes sum to one; the mean's derivative spreads a tile's gradient over
    its rows)."""
    segs, grid, tile = (5, 70, 1), (5, 6, 9), (4, 4, 4)
    pl = orc.plan(segs, grid, tile)
    H, D = 1, 64
    Q, K, V = (rand_bf16((pl.S, H, D), s) for s in (41, 42, 43))
    G = rand_bf16((pl.S, H * D), 44)
    dO = rand_bf16((pl.S, H, D), 45)
    hr = orc.head(Q, K, V, 0, pl, 3, D ** -0.5)
    got = orc.layer_bwd(Q, K, V, G, dO, 0, pl, orc.key_lists_default(pl, hr.keep), D ** -0.5)
    go, g = orc.bf16_value(dO)[:, 0, :], orc.bf16_value(G)
    assert np.allclose(got["dv"].sum(0), (go * (1.0 + g)).sum(0), rtol=1e-10, atol=1e-9)
    assert np.allclose(got["dk"].sum(0), 0.0, atol=1e-9)


def test_backward_zero_and_gate_cases(orc):
    pl = orc.plan((20, 40), (4, 8, 8), (4, 4, 4))
    H, D = 1, 32
    Q, K, V = (rand_bf16((pl.S, H, D), s) for s in (51, 52, 53))
    G = rand_bf16((pl.S, H * D), 54)
    hr = orc.head(Q, K, V, 0, pl, 2, D ** -0.5)
    csr = orc.key_lists_default(pl, hr.keep)
    zero = np.zeros((pl.S, H, D), dtype=np.uint16)
    got = orc.layer_bwd(Q, K, V, G, zero, 0, pl, csr, D ** -0.5)
    for name in ("dq", "dk", "dv", "dg"):
        assert not got[name].any()
    # g = 0: the coarse path carries no gradient; dg = dout * O_coarse[tile]
    dO = rand_bf16((pl.S, H, D), 55)
    g0 = orc.layer_bwd(Q, K, V, np.zeros_like(G), dO, 0, pl, csr, D ** -0.5)
    oc = hr.o_coarse[pl.untile // pl.B]
    assert np.allclose(g0["dg"], orc.bf16_value(dO)[:, 0, :] * oc, rtol=1e-12, atol=1e-14)
    assert np.allclose(g0["dv"].sum(0), orc.bf16_value(dO)[:, 0, :].sum(0), rtol=1e-10, atol=1e-9)


def test_dq_tokens_matches_full_backward(orc):
    segs, grid, tile = (5, 70), (5, 6, 9), (4, 4, 4)
    pl = orc.plan(segs, grid, tile)
    H, D = 2, 32
    Q, K, V = (rand_bf16((pl.S, H, D), s) for s in (61, 62, 63))
    G = rand_bf16((pl.S, H * D), 64)
    dO = rand_bf16((pl.S, H, D), 65)
    for h in range(H):
        hr = orc.head(Q, K, V, h, pl, 3, D ** -0.5)
        csr = orc.key_lists_default(pl, hr.keep)
        full = orc.layer_bwd(Q, K, V, G, dO, h, pl, csr, D ** -0.5)
        toks = np.array([0, 3, 11, pl.S - 1, pl.S // 2])
        got = orc.dq_tokens(Q, K, V, G, dO, h, pl, csr, D ** -0.5, toks)
        assert np.allclose(got, full["dq"][toks], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("segs,grid,tile,mode,kk", CASES)
def test_dkdv_tile_matches_torch_autograd(orc, segs, grid, tile, mode, kk):
    """dk and dv of one key tile at a time (the full-size check's oracle) against
    torch autograd of the dense formulation, for every tile of the plan; padding
    rows come back zero."""
    pl = orc.plan(segs, grid, tile)
    H, D = 2, 32
    Q, K, V = (rand_bf16((pl.S, H, D), s) for s in (71, 72, 73))
    G = rand_bf16((pl.S, H * D), 74, scale=0.5)
    dO = rand_bf16((pl.S, H, D), 75)
    scale = D ** -0.5
    rng = np.random.default_rng(9)
    h = 1
    if mode == "default":
        keep = np.sort(np.stack([rng.choice(pl.n_v, size=kk, replace=False)
                                 for _ in range(pl.n_v)]), axis=1).astype(np.int32) + pl.P
        csr = orc.key_lists_default(pl, keep)
    else:
        k_ref, k_gen = kk
        lists = np.stack([np.concatenate([np.sort(rng.choice(pl.P, k_ref, replace=False)),
                                          np.sort(rng.choice(pl.n_v, k_gen, replace=False)) + pl.P])
                          for _ in range(pl.n_t)]).astype(np.int32)
        csr = orc.key_lists_explicit(lists)
    off, ids = csr
    lists_py = [ids[off[i]:off[i + 1]] for i in range(pl.n_t)]
    want = torch_layer_grads(orc, pl, segs, grid, tile, Q, K, V, G, dO, h, lists_py, scale)
    for j in range(pl.n_t):
        dk, dv = orc.dkdv_tile(Q, K, V, G, dO, h, pl, csr, scale, j)
        rows = pl.row_src[j * pl.B:(j + 1) * pl.B]
        real = rows >= 0
        assert not dk[~real].any() and not dv[~real].any()
        assert np.allclose(dk[real], want["dk"][rows[real]], rtol=1e-5, atol=1e-6), j
        assert np.allclose(dv[real], want["dv"][rows[real]], rtol=1e-5, atol=1e-6), j


def test_dkdv_tile_matches_full_backward(orc):
    """The same gradient as the whole-layer oracle, tile by tile, to fp64 rounding."""
    segs, grid, tile = (5, 70), (5, 6, 9), (4, 4, 4)
    pl = orc.plan(segs, grid, tile)
    H, D = 2, 32
    Q, K, V = (rand_bf16((pl.S, H, D), s) for s in (81, 82, 83))
    G = rand_bf16((pl.S, H * D), 84)
    dO = rand_bf16((pl.S, H, D), 85)
    for h in range(H):
        hr = orc.head(Q, K, V, h, pl, 3, D ** -0.5)
        csr = orc.key_lists_default(pl, hr.keep)
        full = orc.layer_bwd(Q, K, V, G, dO, h, pl, csr, D ** -0.5)
        for j in range(pl.n_t):
            dk, dv = orc.dkdv_tile(Q, K, V, G, dO, h, pl, csr, D ** -0.5, j,
                                   means=(hr.qm, hr.km, hr.vm))
            rows = pl.row_src[j * pl.B:(j + 1) * pl.B]
            real = rows >= 0
            assert np.allclose(dk[real], full["dk"][rows[real]], rtol=1e-11, atol=1e-13), (h, j)
            assert np.allclose(dv[real], full["dv"][rows[real]], rtol=1e-11, atol=1e-13), (h, j)
