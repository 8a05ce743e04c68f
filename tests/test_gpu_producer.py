"""The chunked producer (vsa_qkv_gate_proj) through the C ABI (needs an MI355X).

One GEMM with the layer input's rows taken in tile order writes q and the gate
in natural order and K/V straight into the tile-order fragments with the tile
means. Checked against the existing path, which projects with vsa_gate_proj
(the same k loop, so the same bf16 value for every output) and tiles and pools
in vsa_coarse_topk's gather: projections, tiled K/V, means, keep-sets, O_coarse
and the layer output identical bit for bit. Against the oracle: the projections
within the gate projection's bar (fp32 accumulation vs the correctly rounded
fp64 product), and the means equal to the oracle's pooling (its plan, its
canonical sum) of the projected values, bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import parity
from tests.conftest import gpu_available
from tests.test_gpu_parity import CUSTOM, _u32, assert_gate_close

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a gfx950 GPU")]


def stacked_weights(wl, seed):
    """[W_q; W_k; W_v; W_gate], each [H*D][hidden] ~ N(0, 1/hidden), bf16."""
    gen = torch.Generator().manual_seed(seed)
    HD = wl.heads * wl.head_dim
    w = torch.randn(4, HD, wl.hidden, generator=gen) * wl.hidden ** -0.5
    return w.to(torch.bfloat16)


def run_both(wl, seed=21):
    import tile_sparse_video_amd as tsv
    dev = "cuda"
    x = workloads.make_x(wl).to(dev)
    w = stacked_weights(wl, seed).to(dev)
    S, H, D = wl.tokens, wl.heads, wl.head_dim
    mk = lambda: tsv.TileSparseAttention(wl.prefix_segments, wl.grid, wl.tile, H, D,  # noqa: E731
                                         sparsity=wl.sparsity, keep_k=wl.keep_k, device=dev)
    # the producer path
    prod = mk()
    qp = torch.empty((S, H, D), dtype=torch.bfloat16, device=dev)
    gp = torch.empty((S, H * D), dtype=torch.bfloat16, device=dev)
    prod.project(x, w, qp, gp)
    prod.coarse(None, None, None)
    out_p = torch.empty_like(qp)
    prod.fine(qp, gp, out_p)
    # the existing path: four projections, then the coarse stage's gather
    proj = []
    for i in range(4):
        t = torch.empty((S, H * D), dtype=torch.bfloat16, device=dev)
        tsv.vsa_gate_proj(x, w[i].contiguous(), t)
        proj.append(t)
    ref = mk()
    q_r, k_r, v_r = (t.view(S, H, D) for t in proj[:3])
    ref.coarse(q_r, k_r, v_r)
    out_r = torch.empty_like(qp)
    ref.fine(q_r, proj[3], out_r)
    torch.cuda.synchronize()
    return x, w, prod, ref, (qp, gp, out_p), (proj, out_r)


def same_bits(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


def check_against_existing(wl, prod, ref, got, want):
    (qp, gp, out_p), (proj, out_r) = got, want
    S, H, D = wl.tokens, wl.heads, wl.head_dim
    assert same_bits(qp.view(S, H * D), proj[0]), "q"
    assert same_bits(gp, proj[3]), "gate"
    lay = prod.layout
    for name in ("k_tiled", "v_tiled", "q_mean", "k_mean", "v_mean"):
        a = getattr(lay, name)
        n = {"k_tiled": lay.v_tiled - lay.k_tiled, "v_tiled": lay.q_mean - lay.v_tiled}.get(
            name, H * prod.plan.n_t * D * 4)
        assert torch.equal(prod.workspace[a:a + n], ref.workspace[a:a + n]), name
    assert torch.equal(prod.keep_idx, ref.keep_idx), "keep-sets"
    assert same_bits(prod.o_coarse, ref.o_coarse), "O_coarse"
    assert same_bits(out_p, out_r), "layer output"


def check_against_oracle(wl, x, w, prod, proj, tokens, heads):
    """Projections within the gate projection's bar; means = the oracle's pooling of
    the projected values, bit for bit."""
    S, H, D = wl.tokens, wl.heads, wl.head_dim
    pl = parity.oracle_plan(wl)
    xb = parity.bits(x.cpu())
    for i in range(4):
        wb = parity.bits(w[i].cpu())
        want = oracle.gate_proj(xb, wb, tokens)
        assert_gate_close(parity.bits(proj[i].cpu())[tokens], want, xb[tokens], wb)
    means = [prod.workspace_view(n, torch.float32, (H, pl.n_t, D)).cpu().numpy()
             for n in ("q_mean", "k_mean", "v_mean")]
    for i in range(3):
        X = parity.bits(proj[i].cpu()).reshape(S, H, D)
        for h in heads:
            assert np.array_equal(_u32(means[i][h]), _u32(oracle.tile_means(X, h, pl))), (i, h)


@pytest.mark.parametrize("name", ["ragged64", "ragged128", "d64", "d64_b128", "no_prefix", "one_tile"])
def test_producer_small(name):
    wl = CUSTOM[name]
    if (wl.heads * wl.head_dim) % 128:
        pytest.skip("H*D must be a multiple of 128")
    print(f"[gpu] producer {name}", flush=True)
    x, w, prod, ref, got, want = run_both(wl)
    check_against_existing(wl, prod, ref, got, want)
    check_against_oracle(wl, x, w, prod, want[0], np.arange(wl.tokens), range(wl.heads))


@pytest.mark.parametrize("name", ["mid", "page5"])
def test_producer_workloads(name):
    wl = workloads.WORKLOADS[name]
    print(f"[gpu] producer {name}", flush=True)
    x, w, prod, ref, got, want = run_both(wl)
    check_against_existing(wl, prod, ref, got, want)
    pl = parity.oracle_plan(wl)
    check_against_oracle(wl, x, w, prod, want[0], parity.sample_tokens(pl, 200, 4), range(wl.heads))


@pytest.mark.timeout(900)
def test_producer_full_size_h3():
    """The H3-shaped layer (98,432 tokens, hidden 5,376, 4 x 5,376 outputs): everything
    identical to the existing path on the device; oracle checks on sampled rows and
    on 4 heads' means."""
    wl = workloads.WORKLOADS["h3"]
    print("[gpu] producer h3", flush=True)
    x, w, prod, ref, got, want = run_both(wl)
    check_against_existing(wl, prod, ref, got, want)
    pl = parity.oracle_plan(wl)
    check_against_oracle(wl, x, w, prod, want[0], parity.sample_tokens(pl, 24, 6), [0, 13, 27, 41])

