"""The benchmark's effective FLOPs, the numerator of its headline rate, against a
count by brute force: for every head and query tile, the key tiles the fine pass
attends (all tiles for a prefix query tile; the prefix tiles and the tile's kept
video tiles otherwise; an explicit list per tile in the reference-sparsity mode),
then 4 D FLOP (Q.K^T and P.V, a multiply and an add each) per (real query row,
real key row) pair. The keep lists come from the oracle on the seeded inputs."""
import numpy as np
import pytest

import bench
import oracle
import workloads
from tests import parity
from tests.test_gpu_parity import CUSTOM


def _brute_force(pl, lists_per_head, head_dim):
    rows = [int(x) for x in pl.block_len]
    pairs = 0
    for lists in lists_per_head:
        for i, keys in enumerate(lists):
            pairs += rows[i] * sum(rows[int(j)] for j in keys)
    return 4.0 * head_dim * pairs


def _default_lists(pl, keep_h):
    prefix = list(range(pl.P))
    return [list(range(pl.n_t)) if i < pl.P else prefix + [int(j) for j in keep_h[i - pl.P]]
            for i in range(pl.n_t)]


@pytest.mark.parametrize("name", ["ragged64", "ragged128", "no_prefix", "k0", "dense", "d64", "one_tile"])
def test_effective_flops_default_mode(name):
    wl = CUSTOM[name]
    inp = parity.make_inputs(wl)
    pl = parity.oracle_plan(wl)
    k = parity.oracle_k(wl, pl)
    scale = wl.head_dim ** -0.5
    keep = np.stack([oracle.head(inp.qb, inp.kb, inp.vb, h, pl, k, scale).keep for h in range(wl.heads)])
    assert keep.shape == (wl.heads, pl.n_v, k)
    want = _brute_force(pl, [_default_lists(pl, keep[h]) for h in range(wl.heads)], wl.head_dim)
    got = bench.effective_fine_flops(pl, keep, wl.heads, wl.head_dim, ref=False)
    assert got == want, (got, want)


@pytest.mark.parametrize("name,ref_sparsity", [("ragged64", 0.5), ("ragged128", 0.0), ("no_prefix", 0.9)])
def test_effective_flops_reference_sparsity(name, ref_sparsity):
    wl = CUSTOM[name]
    inp = parity.make_inputs(wl)
    pl = parity.oracle_plan(wl)
    k_ref, k_gen = oracle.ref_keep_counts(pl, ref_sparsity, None, wl.sparsity, wl.keep_k)
    lists = []
    for h in range(wl.heads):
        qm = oracle.tile_means(inp.qb, h, pl)
        km = oracle.tile_means(inp.kb, h, pl)
        lists.append(oracle.topk_ref(oracle.all_scores(qm, km), pl.P, k_ref, k_gen))
    lists = np.stack(lists)
    assert lists.shape == (wl.heads, pl.n_t, k_ref + k_gen)
    want = _brute_force(pl, lists, wl.head_dim)
    got = bench.effective_fine_flops(pl, lists, wl.heads, wl.head_dim, ref=True)
    assert got == want, (got, want)


def test_effective_flops_dense_limit():
    """With every video tile kept, the count is the dense layer's 4 D S^2 per head."""
    wl = CUSTOM["dense"]
    pl = parity.oracle_plan(wl)
    keep = np.tile(np.arange(pl.P, pl.n_t, dtype=np.int32), (wl.heads, pl.n_v, 1))
    got = bench.effective_fine_flops(pl, keep, wl.heads, wl.head_dim, ref=False)
    assert got == 4.0 * wl.head_dim * wl.heads * float(pl.S) ** 2
