"""Reference-sparsity mode: HIP path vs the CPU oracle, through the C ABI.

[Veda] "ComfyUI node" inputs table: reference_sparsity applies the same top-k
setting to the reference tokens. Reading: every query tile (prefix or video)
keeps its k_ref best prefix tiles and its k_gen best video tiles.

Bit-exact: k_ref, tile means, all-pairs coarse scores, the per-group keep
lists. Within tolerance: O_coarse and the layer output (max-abs 2e-2, relative
L2 1e-2 against the oracle's bf16 result).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import parity
from tests.conftest import gpu_available
from tests.test_gpu_parity import CUSTOM, _u32

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a gfx950 GPU")]


def check_layer_ref(inp, run, heads, tokens, ref_sparsity=None, ref_keep_k=None, score_rows=None):
    wl, att = inp.wl, run.att
    pl = parity.oracle_plan(wl)
    k_ref, k_gen = oracle.ref_keep_counts(pl, ref_sparsity, ref_keep_k, wl.sparsity, wl.keep_k)
    assert (att.k_ref, att.k) == (k_ref, k_gen)
    H, D, n_t = wl.heads, wl.head_dim, pl.n_t
    scale = D ** -0.5
    qm = att.workspace_view("q_mean", torch.float32, (H, n_t, D))
    sc = att.workspace_view("scores", torch.float32, (H, n_t, n_t))
    keep = att.keep_idx.cpu().numpy()
    assert keep.shape == (H, n_t, k_ref + k_gen)
    oc = att.o_coarse.cpu().numpy()
    Qb, Kb, Vb = inp.qb, inp.kb, inp.vb
    toks = np.asarray(tokens, dtype=np.int64)
    g_or = oracle.gate_proj(parity.bits(inp.x), parity.bits(inp.w), toks)
    out_gpu = run.out[torch.from_numpy(toks).cuda()].cpu()
    worst = []
    for h in heads:
        hr = oracle.head_ref(Qb, Kb, Vb, h, pl, k_ref, k_gen, scale, score_rows)
        assert np.array_equal(_u32(qm[h].cpu().numpy()), _u32(hr.qm)), f"q means, head {h}"
        rows = hr.score_rows
        assert np.array_equal(_u32(sc[h].cpu().numpy()[rows]), _u32(hr.scores)), f"scores, head {h}"
        assert np.array_equal(keep[h][rows], hr.keep), f"keep lists, head {h}"
        assert parity.rel_l2(oc[h], hr.o_coarse) < 1e-4, f"O_coarse, head {h}"
        if score_rows is not None:
            hr = oracle.head_ref(Qb, Kb, Vb, h, pl, k_ref, k_gen, scale)
        ref_bits, _ = oracle.layer_tokens_ref(Qb, Kb, Vb, g_or, h, pl, hr, scale, toks,
                                              g_is_rows=True)
        ref = oracle.bf16_value(ref_bits)
        got = out_gpu[:, h, :].float().numpy().astype(np.float64)
        mx, rl = float(np.abs(got - ref).max()), parity.rel_l2(got, ref)
        worst.append((mx, rl))
        parity.check_output(got, ref, f"head {h}")
    print(f"[{wl.name} ref] worst max-abs {max(w[0] for w in worst):.3e} "
          f"rel-L2 {max(w[1] for w in worst):.3e}", flush=True)


# (case, ref_sparsity, ref_keep_k): both key groups sparse, reference keys only,
# video keys only, everything kept (dense), no prefix at all.
SMALL = [
    ("ragged64", None, 1),     # P = 3: keep 1 reference tile
    ("ragged128", 0.5, None),
    ("d64", None, 1),
    ("d64_b128", 0.0, None),   # all reference tiles kept
    ("k0", None, 1),           # k_gen = 0: reference keys only
    ("no_prefix", 0.9, None),  # P = 0: video keys only
    ("dense", 0.0, None),      # 0 % everywhere: dense attention
    ("one_tile", None, 0),     # k_ref = 0, one video tile
]


@pytest.mark.parametrize("chunks", [0, 8])
@pytest.mark.parametrize("name,rs,rk", SMALL)
def test_ref_small_every_token(name, rs, rk, chunks):
    import tile_sparse_video_amd as tsv
    wl = CUSTOM[name]
    print(f"[gpu] ref {name} rs={rs} rk={rk} chunks={chunks}", flush=True)
    inp = parity.make_inputs(wl)
    run = parity.run_gpu_ref(inp, rs, rk, split_chunks=chunks)
    check_layer_ref(inp, run, range(wl.heads), np.arange(wl.tokens), rs, rk)


def test_ref_tiny_and_mid():
    for name, rs in (("tiny", 0.5), ("mid", 0.75)):
        wl = workloads.WORKLOADS[name]
        print(f"[gpu] ref {name}", flush=True)
        inp = parity.make_inputs(wl)
        run = parity.run_gpu_ref(inp, rs)
        pl = parity.oracle_plan(wl)
        toks = np.arange(wl.tokens) if name == "tiny" else parity.sample_tokens(pl, 400, 9)
        check_layer_ref(inp, run, range(wl.heads), toks, rs)


def test_ref_page5_geometry():
    wl = workloads.WORKLOADS["page5"]
    print("[gpu] ref page5", flush=True)
    inp = parity.make_inputs(wl)
    run = parity.run_gpu_ref(inp, 0.9)
    pl = parity.oracle_plan(wl)
    check_layer_ref(inp, run, range(wl.heads), parity.sample_tokens(pl, 500, 4), 0.9)


def test_ref_all_prefix_kept_matches_default_path_for_video_tokens():
    """k_ref = P: video query tokens get the default path's output."""
    wl = CUSTOM["ragged64"]
    print("[gpu] ref k_ref = P vs default", flush=True)
    inp = parity.make_inputs(wl)
    a = parity.run_gpu(inp)
    pl = parity.oracle_plan(wl)
    b = parity.run_gpu_ref(inp, None, pl.P)
    vid = torch.from_numpy(np.nonzero(pl.untile // pl.B >= pl.P)[0]).cuda()
    keep_ref = b.att.keep_idx.cpu().numpy()[:, pl.P:, pl.P:]
    assert np.array_equal(keep_ref, a.att.keep_idx.cpu().numpy())
    # same keys, same per-key arithmetic order: identical bits
    assert torch.equal(a.out[vid].view(torch.int16), b.out[vid].view(torch.int16))


@pytest.mark.parametrize("name,rs", [("veda", 0.9), ("h3", 0.75)])
def test_ref_full_size_sampled(name, rs):
    wl = workloads.WORKLOADS[name]
    print(f"[gpu] ref full size {name}: generating inputs", flush=True)
    inp = parity.make_inputs(wl)
    print(f"[gpu] ref full size {name}: running the HIP path", flush=True)
    run = parity.run_gpu_ref(inp, rs)
    pl = parity.oracle_plan(wl)
    heads = sorted({0, wl.heads - 1})
    toks = parity.sample_tokens(pl, 48, 8)
    rows = np.unique(np.concatenate([np.arange(pl.P), pl.untile[toks] // pl.B,
                                     np.random.default_rng(3).choice(pl.n_t, 64, replace=False)]))
    print(f"[gpu] ref full size {name}: oracle on heads {heads}, {len(toks)} tokens", flush=True)
    check_layer_ref(inp, run, heads, toks, rs, score_rows=rows)
    del run
    torch.cuda.empty_cache()
