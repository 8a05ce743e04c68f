"""Per-head tile shapes: vsa_layer_fwd_groups vs the CPU oracle, through the C ABI.

[Veda] "How Veda works": tile shapes are chosen per layer and per head. Reading:
a layer's heads are split into groups of consecutive heads, each with its own
tile plan; every head's output is the single-plan layer's output for that head
and its group's plan. The oracle runs each head with its own group's plan (the
same per-head functions the single-plan parity tests use); keep lists are
bit-exact, outputs within max-abs 2e-2 and relative L2 1e-2.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import parity
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a gfx950 GPU")]


def run_groups(inp, groups):
    import tile_sparse_video_amd as tsv
    wl = inp.wl
    lay = tsv.HeadGroupAttention(wl.prefix_segments, wl.grid, groups, wl.head_dim)
    qd, kd, vd = (t.cuda() for t in (inp.q, inp.k, inp.v))
    g = torch.empty((wl.tokens, wl.heads * wl.head_dim), dtype=torch.bfloat16, device="cuda")
    tsv.vsa_gate_proj(inp.x.cuda(), inp.w.cuda(), g)
    out = lay(qd, kd, vd, g)
    torch.cuda.synchronize()
    return lay, out, g


def check_groups(inp, lay, out, groups, tokens, heads_per_group=None):
    wl = inp.wl
    D = wl.head_dim
    scale = D ** -0.5
    Qb, Kb, Vb = inp.qb, inp.kb, inp.vb
    toks = np.asarray(tokens, dtype=np.int64)
    g_or = oracle.gate_proj(parity.bits(inp.x), parity.bits(inp.w), toks)
    out_gpu = out[torch.from_numpy(toks).cuda()].cpu()
    worst = []
    for (h0, att), grp in zip(lay.layers, groups):
        pl = oracle.plan(wl.prefix_segments, wl.grid, grp["tile"])
        assert np.array_equal(att.plan.row_src, pl.row_src)
        tiles = pl.untile[toks] // pl.B
        keep_gpu = att.keep_idx.cpu().numpy()
        ref_mode = grp.get("reference_sparsity") is not None or grp.get("ref_keep_k") is not None
        hs = range(grp["heads"]) if heads_per_group is None else heads_per_group(grp["heads"])
        for hl in hs:
            h = h0 + hl
            if ref_mode:
                k_ref, k = oracle.ref_keep_counts(pl, grp.get("reference_sparsity"),
                                                  grp.get("ref_keep_k"), grp.get("sparsity"),
                                                  grp.get("keep_k"))
                hr = oracle.head_ref(Qb, Kb, Vb, h, pl, k_ref, k, scale)
                csr = oracle.key_lists_explicit(hr.keep)
            else:
                k = oracle.keep_count(pl.n_v, grp.get("sparsity"), grp.get("keep_k"))
                hr = oracle.head(Qb, Kb, Vb, h, pl, k, scale)
                csr = oracle.key_lists_default(pl, hr.keep)
            assert np.array_equal(keep_gpu[hl], hr.keep), f"keep lists, head {h}"
            if grp.get("int8"):
                o_fine = oracle.fine_tokens_i8(Qb, Kb, Vb, h, pl, csr, scale, toks)
            elif ref_mode:
                o_fine = oracle.fine_tokens_lists(Qb, Kb, Vb, h, pl, hr.keep, scale, toks)
            else:
                o_fine = oracle.fine_tokens(Qb, Kb, Vb, h, pl, hr.keep, k, scale, toks)
            g_rows = np.ascontiguousarray(g_or[:, h * D:(h + 1) * D])
            ref = oracle.bf16_value(oracle.combine(o_fine, g_rows, hr.o_coarse[tiles]))
            got = out_gpu[:, h, :].float().numpy().astype(np.float64)
            mx, rl = float(np.abs(got - ref).max()), parity.rel_l2(got, ref)
            worst.append((mx, rl))
            parity.check_output(got, ref, f"head {h}")
    print(f"[{wl.name} groups] worst max-abs {max(w[0] for w in worst):.3e} "
          f"rel-L2 {max(w[1] for w in worst):.3e}", flush=True)


SMALL_WL = workloads.custom("groups", seed=21, heads=5, head_dim=128, hidden=128,
                            prefix_segments=(20, 45), grid=(5, 8, 12), tile=(4, 4, 4))
SMALL_GROUPS = [
    {"tile": (4, 4, 4), "heads": 2, "keep_k": 3},                 # cubes
    {"tile": (1, 8, 8), "heads": 1, "sparsity": 0.5},             # one frame: spatial
    {"tile": (16, 2, 2), "heads": 1, "keep_k": 2},                # across frames: temporal
    {"tile": (4, 8, 4), "heads": 1, "keep_k": 1},                 # 128-row tiles
]


def test_groups_small_every_token():
    print("[gpu] groups small", flush=True)
    inp = parity.make_inputs(SMALL_WL)
    lay, out, _ = run_groups(inp, SMALL_GROUPS)
    check_groups(inp, lay, out, SMALL_GROUPS, np.arange(SMALL_WL.tokens))


def test_groups_mixed_modes_every_token():
    """Reference sparsity and the INT8 fine pass inside groups."""
    groups = [
        {"tile": (1, 8, 8), "heads": 2, "sparsity": 0.5, "reference_sparsity": 0.5},
        {"tile": (4, 4, 4), "heads": 2, "keep_k": 2, "int8": True},
        {"tile": (16, 2, 2), "heads": 1, "keep_k": 2, "ref_keep_k": 1, "int8": True},
    ]
    print("[gpu] groups mixed modes", flush=True)
    inp = parity.make_inputs(SMALL_WL)
    lay, out, _ = run_groups(inp, groups)
    check_groups(inp, lay, out, groups, np.arange(SMALL_WL.tokens))


def test_one_group_is_the_single_plan_layer():
    """A single group over every head runs the same kernels as TileSparseAttention:
    bit-identical output."""
    wl = SMALL_WL
    print("[gpu] groups: one group vs single plan", flush=True)
    inp = parity.make_inputs(wl)
    groups = [{"tile": (4, 4, 4), "heads": wl.heads, "keep_k": 3}]
    lay, out, g = run_groups(inp, groups)
    wl1 = dataclasses.replace(wl, keep_k=3)
    single = parity.run_gpu(parity.Inputs(wl1, inp.q, inp.k, inp.v, inp.x, inp.w), gate=g.cpu())
    assert torch.equal(out.view(torch.int16), single.out.view(torch.int16))


def test_uncovered_heads_are_untouched():
    import tile_sparse_video_amd as tsv
    wl = SMALL_WL
    print("[gpu] groups: uncovered heads", flush=True)
    inp = parity.make_inputs(wl)
    groups = [{"tile": (4, 4, 4), "heads": 2, "keep_k": 3}]
    # the layer has 5 heads; the group covers heads 0 and 1 only
    lay = tsv.HeadGroupAttention(wl.prefix_segments, wl.grid, groups, wl.head_dim,
                                 heads_total=wl.heads)
    qd, kd, vd = (t.cuda() for t in (inp.q, inp.k, inp.v))
    g = torch.zeros((wl.tokens, wl.heads * wl.head_dim), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(qd, 7.0)
    lay(qd, kd, vd, g, out)
    torch.cuda.synchronize()
    assert bool((out[:, 2:] == 7.0).all())
    assert not bool((out[:, :2] == 7.0).any())


def test_groups_full_size_veda_geometry():
    """The Veda-style layer with its heads split between 128-row cubes, frame tiles
    and time tiles; sampled tokens, two heads per group."""
    wl = workloads.WORKLOADS["veda"]
    groups = [
        {"tile": (4, 8, 4), "heads": 14, "keep_k": 101},
        {"tile": (1, 8, 16), "heads": 14, "sparsity": 0.9},
        {"tile": (16, 2, 4), "heads": 14, "sparsity": 0.9},
    ]
    print("[gpu] groups full size veda: generating inputs", flush=True)
    inp = parity.make_inputs(wl)
    print("[gpu] groups full size veda: running the HIP path", flush=True)
    lay, out, _ = run_groups(inp, groups)
    pl = oracle.plan(wl.prefix_segments, wl.grid, wl.tile)
    toks = parity.sample_tokens(pl, 24, 5)
    print("[gpu] groups full size veda: oracle", flush=True)
    check_groups(inp, lay, out, groups, toks, heads_per_group=lambda n: [0, n - 1])
